"""fp64 CPU oracle for the DSA hot path (indexer -> top-k -> sparse attention).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does, and
this package imports nothing from it.  The arithmetic lives in ``dsa_oracle.c``
(plain C, double precision, sequential sums); this module only builds that file
with gcc and marshals numpy arrays into it.

The method it follows is the one the pages describe: "DeepSeek-V3.2-Exp
稀疏注意力机制(DSA)技术深度解析" (sheratonhq.com) section 1 -- a light indexer
scores every history token with few heads, index_head_dim 128, ReLU and FP8;
a top-k selector keeps the k best; the main attention runs over that subset --
and "DeepSeek-V4 百万 token 上下文的工程实现" (blog.hotdry.top), section
"从 O(N²) 到 O(N・k)", which names the same two stages.  The readings taken where
the pages are silent are listed at the top of ``dsa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, E4M3 = 0, 1, 2
_DTYPE_CODES = {"f32": F32, "bf16": BF16, "e4m3": E4M3}

_lib = None


def build(force: bool = True) -> str:
    """Compile dsa_oracle.c into liboracle.so with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, dbl, vp, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
    lib.ora_num_threads.restype = ctypes.c_int
    lib.ora_num_threads.argtypes = []
    lib.ora_set_num_threads.restype = None
    lib.ora_set_num_threads.argtypes = [ctypes.c_int]
    lib.ora_e4m3_value.restype = dbl
    lib.ora_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.ora_bf16_value.restype = dbl
    lib.ora_bf16_value.argtypes = [ctypes.c_uint16]
    lib.ora_index_scores.restype = None
    lib.ora_index_scores.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.ora_topk.restype = None
    lib.ora_topk.argtypes = [i64, i64, vp, vp, i64, vp, vp]
    lib.ora_select_backbone.restype = None
    lib.ora_select_backbone.argtypes = [i64, i64, vp, vp, i64, i64, i64, vp, vp]
    lib.ora_sparse_attn.restype = None
    lib.ora_sparse_attn.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, i32,
                                    vp, vp, vp, vp, vp, dbl, vp, i64, vp, vp, vp]
    lib.ora_dense_causal_attn.restype = None
    lib.ora_dense_causal_attn.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, i32,
                                          vp, vp, vp, vp, vp, dbl, vp, vp, vp]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _stored(a, dtype: str):
    """Return a C-contiguous numpy array of the stored bits for `dtype`."""
    want = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}[dtype]
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"oracle expects {want} storage for {dtype}, got {a.dtype}")
    return a


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _positions(pos, n_q, n_k):
    if pos is None:
        pos = np.arange(n_q, dtype=np.int64) + (n_k - n_q)
    return np.ascontiguousarray(pos, dtype=np.int64)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().ora_num_threads())


def set_num_threads(n: int) -> None:
    """Sets the OpenMP threads of the oracle's parallel loops (n >= 1)."""
    _load().ora_set_num_threads(int(n))


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 code (1 sign, 4 exponent bits bias 7, 3 mantissa)."""
    return _load().ora_e4m3_value(int(code))


def bf16_value(bits: int) -> float:
    return _load().ora_bf16_value(int(bits))


def index_scores(iq, ik, iw, dtype: str, iq_scale=None, ik_scale=None, pos=None):
    """I[t,s] = sum_h w[t,h]*ReLU(q_I[t,h].k_I[s]) for s <= pos[t], else -inf.

    iq [n_q,H,D], ik [n_k,D] in stored form (float32 / uint16 bf16 bits / uint8
    e4m3 codes), per-token fp32 scales for e4m3, iw [n_q,H] fp32.  Returns fp64
    [n_q,n_k].  One sequence per call.
    """
    iq = _stored(iq, dtype)
    ik = _stored(ik, dtype)
    n_q, H, D = iq.shape
    n_k = ik.shape[0]
    assert ik.shape == (n_k, D)
    iw = _f32(iw)
    assert iw.shape == (n_q, H)
    iq_scale, ik_scale = _f32(iq_scale), _f32(ik_scale)
    pos = _positions(pos, n_q, n_k)
    out = np.empty((n_q, n_k), dtype=np.float64)
    _load().ora_index_scores(n_q, n_k, H, D, _DTYPE_CODES[dtype], _ptr(iq), _ptr(iq_scale),
                             _ptr(ik), _ptr(ik_scale), _ptr(iw), _ptr(pos), _ptr(out))
    return out


def topk(scores, k: int, pos=None):
    """Keep m=min(k,pos+1) best keys per row, lower index first among equals.

    Returns (idx [n_q,k] int32 ascending then -1, kth [n_q] fp64 = m-th score).
    """
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    n_q, n_k = scores.shape
    pos = _positions(pos, n_q, n_k)
    idx = np.empty((n_q, k), dtype=np.int32)
    kth = np.empty(n_q, dtype=np.float64)
    _load().ora_topk(n_q, n_k, _ptr(scores), _ptr(pos), k, _ptr(idx), _ptr(kth))
    return idx, kth


def select_backbone(scores, k: int, sinks: int, window: int, pos=None):
    """Top-k over the keys outside a forced set, united with that set.

    The forced set of a row is its first `sinks` keys and its last `window`
    visible keys; the m=min(k, #rest) best of the rest are added.  Returns
    (idx [n_q, k+sinks+window] int32 ascending then -1, kth [n_q] fp64 = the
    m-th best score of the rest, NaN if none).
    """
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    n_q, n_k = scores.shape
    pos = _positions(pos, n_q, n_k)
    idx = np.empty((n_q, k + sinks + window), dtype=np.int32)
    kth = np.empty(n_q, dtype=np.float64)
    _load().ora_select_backbone(n_q, n_k, _ptr(scores), _ptr(pos), k, sinks, window, _ptr(idx), _ptr(kth))
    return idx, kth


def _kv_scales(kv_dtype, k_scale, v_scale, n_k, Hkv, latent):
    if kv_dtype != "e4m3":
        return None, None
    ks = np.ascontiguousarray(k_scale, dtype=np.float32).reshape(n_k, Hkv)
    vs = None if latent else np.ascontiguousarray(v_scale, dtype=np.float32).reshape(n_k, Hkv)
    return ks, vs


def sparse_attn(q, k, v, idx, dtype: str, scale: float, pos=None, latent_dv: int | None = None,
                kv_dtype: str | None = None, k_scale=None, v_scale=None):
    """Softmax attention of each query over its selected key rows only.

    q [n_q,Hq,dqk] (dtype), k [n_k,Hkv,dqk], v [n_k,Hkv,dv] (kv_dtype, default
    dtype; or v None with latent_dv: the value is then the first latent_dv
    entries of the key row), idx [n_q,kk].  An "e4m3" cache carries one fp32
    scale per (token, kv head) row: k_scale, v_scale [n_k,Hkv].
    Returns (out [n_q,Hq,dv] fp64, lse [n_q,Hq] fp64).
    """
    kv_dtype = kv_dtype or dtype
    q = _stored(q, dtype)
    k = _stored(k, kv_dtype)
    n_q, Hq, dqk = q.shape
    n_k, Hkv, _ = k.shape
    latent = v is None
    if latent:
        dv = int(latent_dv)
        assert Hkv == 1 and dv <= dqk
    else:
        v = _stored(v, kv_dtype)
        dv = v.shape[2]
    ks, vs = _kv_scales(kv_dtype, k_scale, v_scale, n_k, Hkv, latent)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    kk = idx.shape[1]
    pos = _positions(pos, n_q, n_k)
    out = np.empty((n_q, Hq, dv), dtype=np.float64)
    lse = np.empty((n_q, Hq), dtype=np.float64)
    _load().ora_sparse_attn(n_q, n_k, Hq, Hkv, dqk, dv, int(latent), _DTYPE_CODES[dtype],
                            _DTYPE_CODES[kv_dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(ks), _ptr(vs),
                            float(scale), _ptr(idx), kk, _ptr(pos), _ptr(out), _ptr(lse))
    return out, lse


def dense_causal_attn(q, k, v, dtype: str, scale: float, pos=None, latent_dv: int | None = None,
                      kv_dtype: str | None = None, k_scale=None, v_scale=None):
    """Textbook dense causal attention over keys s <= pos[t] (a pin for sparse_attn)."""
    kv_dtype = kv_dtype or dtype
    q = _stored(q, dtype)
    k = _stored(k, kv_dtype)
    n_q, Hq, dqk = q.shape
    n_k, Hkv, _ = k.shape
    latent = v is None
    if latent:
        dv = int(latent_dv)
    else:
        v = _stored(v, kv_dtype)
        dv = v.shape[2]
    ks, vs = _kv_scales(kv_dtype, k_scale, v_scale, n_k, Hkv, latent)
    pos = _positions(pos, n_q, n_k)
    out = np.empty((n_q, Hq, dv), dtype=np.float64)
    lse = np.empty((n_q, Hq), dtype=np.float64)
    _load().ora_dense_causal_attn(n_q, n_k, Hq, Hkv, dqk, dv, int(latent), _DTYPE_CODES[dtype],
                                  _DTYPE_CODES[kv_dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(ks), _ptr(vs),
                                  float(scale), _ptr(pos), _ptr(out), _ptr(lse))
    return out, lse


def dsa_forward(inp: dict, rows=None):
    """The whole path for one input set (see dsa_inputs) on selected query rows.

    `inp` holds numpy arrays in stored form for every sequence b:
      iq [B,n_q,H,D], iq_scale [B,n_q]|None, ik [B,n_k,D], ik_scale [B,n_k]|None,
      iw [B,n_q,H], q [B,n_q,Hq,dqk], k [B,n_k,Hkv,dqk], v [B,n_k,Hkv,dv]|None,
      for an FP8 cache (kv_dtype "e4m3") k_scale / v_scale [B,n_k,Hkv],
    plus scalars idx_dtype, attn_dtype, kv_dtype, top_k, scale, latent_dv, pos [B,n_q].
    `rows` is a list of (b, t) pairs (default: all).  Returns a dict of per-row
    results keyed by (b, t): scores, idx, kth, out, lse.
    """
    B, n_q = inp["iq"].shape[:2]
    n_k = inp["ik"].shape[1]
    if rows is None:
        rows = [(b, t) for b in range(B) for t in range(n_q)]
    by_seq: dict[int, list[int]] = {}
    for b, t in rows:
        by_seq.setdefault(b, []).append(t)
    res = {}
    for b, ts in by_seq.items():
        ts = np.asarray(ts, dtype=np.int64)
        pos = np.asarray(inp["pos"][b], dtype=np.int64)[ts]
        iqs = None if inp.get("iq_scale") is None else inp["iq_scale"][b][ts]
        iks = None if inp.get("ik_scale") is None else inp["ik_scale"][b]
        sc = index_scores(inp["iq"][b][ts], inp["ik"][b], inp["iw"][b][ts], inp["idx_dtype"],
                          iqs, iks, pos)
        sinks, window = int(inp.get("sinks", 0)), int(inp.get("window", 0))
        if sinks or window:
            idx, kth = select_backbone(sc, inp["top_k"], sinks, window, pos)
        else:
            idx, kth = topk(sc, inp["top_k"], pos)
        v = None if inp.get("v") is None else inp["v"][b]
        kvs = {}
        if inp.get("kv_dtype", inp["attn_dtype"]) == "e4m3":
            kvs = dict(kv_dtype="e4m3", k_scale=inp["k_scale"][b],
                       v_scale=None if inp.get("v_scale") is None else inp["v_scale"][b])
        out, lse = sparse_attn(inp["q"][b][ts], inp["k"][b], v, idx, inp["attn_dtype"],
                               inp["scale"], pos, inp.get("latent_dv"), **kvs)
        for j, t in enumerate(ts.tolist()):
            res[(b, t)] = dict(scores=sc[j], idx=idx[j], kth=kth[j], out=out[j], lse=lse[j])
    return res


def compress_select(importance, window: int, keep_old: int):
    """Positions a sequence keeps under importance compression (ascending, int64).

    "DeepSeek-V4 百万 token 上下文的工程实现" (blog.hotdry.top), section
    "滑动窗口 KV Cache 与混合策略": recent tokens keep their full K/V, older ones
    are cut down by an importance score.  Read as: the last min(window, n)
    tokens are kept; of the n_old tokens before them, the min(keep_old, n_old)
    of highest importance, the lower position first among equal importance
    (-0.0 equal to +0.0).  Parity pinned by a hand-worked example, a brute
    force over every subset of tiny inputs, and the pages' 45-55 % cut at 1M
    tokens with an 8K window.
    """
    imp = np.asarray(importance, dtype=np.float64).ravel()
    n = imp.size
    w = min(window, n)
    n_old = n - w
    keep = min(keep_old, n_old)
    # one sort of the old tokens: primary key importance descending (negation
    # maps -0.0 and +0.0 to equal keys), secondary key position ascending
    order = np.lexsort((np.arange(n_old), -imp[:n_old]))
    kept_old = np.sort(order[:keep])
    return np.concatenate([kept_old, np.arange(n_old, n)]).astype(np.int64)

