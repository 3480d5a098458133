"""Python binding of libdsa, the gfx950 DeepSeek Sparse Attention hot path.

Argument marshalling only: every step of the path (indexer scores, top-k
selection, sparse attention) runs in the HIP kernels behind the C ABI in
``include/dsa.h``.  PyTorch supplies device memory and the current stream.  If
``libdsa.so`` has not been built the first call raises; there is no fallback.

The entry points mirror the C ABI: ``index_scores``, ``topk``, ``sparse_attn``,
``prefill`` and ``decode``, plus ``workspace_bytes``.  Build the problem once
with :func:`make_problem` (it checks shapes, dtypes and devices and keeps the
tensors alive) and pass it to any of them.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_DEVICE = 0, -1, -2, -3, -4
F32, BF16, FP8_E4M3 = 0, 1, 2
OP_INDEX_SCORES, OP_TOPK, OP_SPARSE_ATTN, OP_PREFILL, OP_DECODE, OP_DENSE_ATTN, OP_COMPRESS_KV = 0, 1, 2, 3, 4, 5, 6
ATTN_AUTO, ATTN_GATHER, ATTN_MASKED = 0, 1, 2
ABI_VERSION = 4

_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}

EXPORTED = ("dsa_abi_version", "dsa_workspace_bytes", "dsa_index_scores", "dsa_topk",
            "dsa_sparse_attn", "dsa_prefill", "dsa_decode", "dsa_decode_noalloc", "dsa_dense_attn",
            "dsa_phase_timing", "dsa_phase_times", "dsa_status_str", "dsa_last_error",
            "dsa_compress_kept", "dsa_compress_kv")
NOALLOC_SCRATCH_BYTES = 64 << 20
# dsa_phase_t, in order
PHASES = ("prep", "index", "topk", "attn")


class Problem(ctypes.Structure):
    """Mirror of dsa_problem_t (all pointers are device addresses)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
        ("q_pos", ctypes.c_void_p),
        ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32), ("idx_dtype", ctypes.c_int32),
        ("iq", ctypes.c_void_p), ("iq_scale", ctypes.c_void_p),
        ("ik", ctypes.c_void_p), ("ik_scale", ctypes.c_void_p), ("iw", ctypes.c_void_p),
        ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32), ("kv_latent", ctypes.c_int32), ("attn_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("top_k", ctypes.c_int32),
        ("attn_mode", ctypes.c_int32),
        ("sink_tokens", ctypes.c_int32), ("local_window", ctypes.c_int32),
    ]


class DSAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_str(status)} ({detail})" if detail else status_str(status))
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libdsa.so (raises if it is missing: build it with long_context_sparse_relu_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m long_context_sparse_relu_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Problem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.dsa_abi_version.restype = ctypes.c_int
    lib.dsa_abi_version.argtypes = []
    lib.dsa_workspace_bytes.restype = sz
    lib.dsa_workspace_bytes.argtypes = [ctypes.c_int, P]
    lib.dsa_index_scores.restype = ctypes.c_int
    lib.dsa_index_scores.argtypes = [P, vp, vp]
    lib.dsa_topk.restype = ctypes.c_int
    lib.dsa_topk.argtypes = [P, vp, vp, vp, sz, vp]
    lib.dsa_sparse_attn.restype = ctypes.c_int
    lib.dsa_sparse_attn.argtypes = [P, vp, vp, vp, vp, sz, vp]
    lib.dsa_prefill.restype = ctypes.c_int
    lib.dsa_prefill.argtypes = [P, vp, vp, vp, vp, sz, vp]
    lib.dsa_decode.restype = ctypes.c_int
    lib.dsa_decode.argtypes = [P, vp, vp, vp, vp, sz, vp]
    lib.dsa_decode_noalloc.restype = ctypes.c_int
    lib.dsa_decode_noalloc.argtypes = [P, vp, vp, vp, vp]
    lib.dsa_dense_attn.restype = ctypes.c_int
    lib.dsa_dense_attn.argtypes = [P, vp, vp, vp, sz, vp]
    lib.dsa_phase_timing.restype = ctypes.c_int
    lib.dsa_compress_kept.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.dsa_compress_kept.restype = ctypes.c_int32
    lib.dsa_compress_kv.argtypes = [P, vp, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(KVCompressed), vp, sz, vp]
    lib.dsa_compress_kv.restype = ctypes.c_int
    lib.dsa_phase_timing.argtypes = [ctypes.c_int]
    lib.dsa_phase_times.restype = ctypes.c_int
    lib.dsa_phase_times.argtypes = [ctypes.POINTER(ctypes.c_float)]
    lib.dsa_status_str.restype = ctypes.c_char_p
    lib.dsa_status_str.argtypes = [ctypes.c_int]
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    if lib.dsa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libdsa ABI {lib.dsa_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().dsa_status_str(status).decode()


def last_error() -> str:
    return load_library().dsa_last_error().decode()


def _check(status: int):
    if status != OK:
        raise DSAError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class DSAProblem:
    """A dsa_problem_t plus the tensors it points into (kept alive here)."""

    def __init__(self, struct: Problem, tensors: dict, device):
        self.struct = struct
        self.tensors = tensors
        self.device = device

    @property
    def rows(self) -> int:
        return self.struct.batch * self.struct.n_q

    @property
    def sel_width(self) -> int:
        """Entries of a selection row: top_k + sink_tokens + local_window."""
        s = self.struct
        return s.top_k + s.sink_tokens + s.local_window

    def ref(self):
        return ctypes.byref(self.struct)


def _contig(name, t, device, dtypes=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


def fp8_kv_record_bytes(heads: int, dim: int) -> int:
    """Bytes of one token's record in an FP8 k or v cache (DSA_FP8_KV_RECORD_BYTES)."""
    return (heads * dim + 4 * heads + 15) // 16 * 16


def make_problem(*, iq, ik, iw, top_k, q=None, k=None, v=None, iq_scale=None, ik_scale=None,
                 q_pos=None, softmax_scale=None, latent_dv=None, kv_heads=None, d_v=None,
                 attn_mode: int = ATTN_AUTO, sink_tokens: int = 0, local_window: int = 0) -> DSAProblem:
    """Describe one batch: see include/dsa.h for the layouts.

    iq [B,n_q,H,128], ik [B,n_k,128] (fp32 | bf16 | float8_e4m3fn, same dtype),
    iq_scale [B,n_q] / ik_scale [B,n_k] fp32 for FP8, iw [B,n_q,H] fp32,
    q [B,n_q,Hq,dqk], k [B,n_k,Hkv,dqk], v [B,n_k,Hkv,dv] or None with
    latent_dv (then the value is k[..., :latent_dv] and Hkv must be 1),
    q_pos [B,n_q] int32 or None.  k and v have q's dtype, or are an FP8 cache
    (q bf16): uint8 token records [B,n_k,fp8_kv_record_bytes(Hkv, dqk)] for k
    and [B,n_k,fp8_kv_record_bytes(Hkv, dv)] for v (codes, then the scales),
    with kv_heads = Hkv and, unless latent, d_v given.  attn_mode: ATTN_AUTO,
    ATTN_GATHER or ATTN_MASKED.  sink_tokens / local_window: the backbone's
    forced keys (the first sink_tokens and last local_window visible keys),
    kept besides the top_k best between them.
    """
    device = iq.device
    idt = (torch.float32, torch.bfloat16, torch.float8_e4m3fn)
    iq = _contig("iq", iq, device, idt)
    ik = _contig("ik", ik, device, (iq.dtype,))
    iw = _contig("iw", iw, device, (torch.float32,))
    iq_scale = _contig("iq_scale", iq_scale, device, (torch.float32,))
    ik_scale = _contig("ik_scale", ik_scale, device, (torch.float32,))
    q_pos = _contig("q_pos", q_pos, device, (torch.int32,))
    if iq.dim() != 4 or ik.dim() != 3 or iw.dim() != 3:
        raise ValueError("iq must be [B,n_q,H,D], ik [B,n_k,D], iw [B,n_q,H]")
    B, n_q, H, D = iq.shape
    n_k = ik.shape[1]
    if ik.shape != (B, n_k, D) or iw.shape != (B, n_q, H):
        raise ValueError(f"shape mismatch: iq {tuple(iq.shape)}, ik {tuple(ik.shape)}, iw {tuple(iw.shape)}")
    if iq.dtype == torch.float8_e4m3fn:
        if iq_scale is None or ik_scale is None:
            raise ValueError("FP8 indexer inputs need iq_scale and ik_scale")
        if iq_scale.shape != (B, n_q) or ik_scale.shape != (B, n_k):
            raise ValueError("iq_scale must be [B,n_q] and ik_scale [B,n_k]")
    if q_pos is not None and q_pos.shape != (B, n_q):
        raise ValueError("q_pos must be [B,n_q]")
    p = Problem()
    p.batch, p.n_q, p.n_k = B, n_q, n_k
    p.q_pos = None if q_pos is None else q_pos.data_ptr()
    p.idx_heads, p.idx_dim, p.idx_dtype = H, D, _DTYPE_CODE[iq.dtype]
    p.iq, p.ik, p.iw = iq.data_ptr(), ik.data_ptr(), iw.data_ptr()
    p.iq_scale = None if iq_scale is None else iq_scale.data_ptr()
    p.ik_scale = None if ik_scale is None else ik_scale.data_ptr()
    p.top_k = int(top_k)
    p.attn_mode = int(attn_mode)
    p.sink_tokens, p.local_window = int(sink_tokens), int(local_window)
    tensors = dict(iq=iq, ik=ik, iw=iw, iq_scale=iq_scale, ik_scale=ik_scale, q_pos=q_pos)
    if q is not None:
        adt = (torch.float32, torch.bfloat16)
        q = _contig("q", q, device, adt)
        if q.dim() != 4 or q.shape[:2] != (B, n_q):
            raise ValueError(f"q must be [B,n_q,Hq,dqk], got {tuple(q.shape)}")
        Hq, dqk = q.shape[2], q.shape[3]
        fp8 = k is not None and k.dtype == torch.uint8
        if fp8:
            if q.dtype != torch.bfloat16:
                raise TypeError("an FP8 KV cache goes with bf16 q")
            if kv_heads is None:
                raise ValueError("an FP8 KV cache (uint8 token records) needs kv_heads")
            Hkv = int(kv_heads)
            k = _contig("k", k, device, (torch.uint8,))
            if k.shape != (B, n_k, fp8_kv_record_bytes(Hkv, dqk)):
                raise ValueError(f"k records must be [B,n_k,{fp8_kv_record_bytes(Hkv, dqk)}], got {tuple(k.shape)}")
        else:
            k = _contig("k", k, device, (q.dtype,))
            if k.dim() != 4 or k.shape[:2] != (B, n_k) or k.shape[3] != dqk:
                raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}")
            Hkv = k.shape[2]
        v = _contig("v", v, device, (k.dtype,))
        if v is None:
            if latent_dv is None:
                raise ValueError("v is None: pass latent_dv for latent key/value rows")
            dv, latent = int(latent_dv), 1
        elif fp8:
            if d_v is None:
                raise ValueError("FP8 value records need d_v")
            dv, latent = int(d_v), 0
            if v.shape != (B, n_k, fp8_kv_record_bytes(Hkv, dv)):
                raise ValueError(f"v records must be [B,n_k,{fp8_kv_record_bytes(Hkv, dv)}], got {tuple(v.shape)}")
        else:
            if v.dim() != 4 or v.shape[:3] != (B, n_k, Hkv):
                raise ValueError(f"v must be [B,n_k,Hkv,dv], got {tuple(v.shape)}")
            dv, latent = v.shape[3], 0
        p.q_heads, p.kv_heads, p.d_qk, p.d_v, p.kv_latent = Hq, Hkv, dqk, dv, latent
        p.attn_dtype = _DTYPE_CODE[q.dtype]
        p.kv_dtype = FP8_E4M3 if fp8 else _DTYPE_CODE[k.dtype]
        p.q, p.k = q.data_ptr(), k.data_ptr()
        p.v = None if v is None else v.data_ptr()
        p.k_scale = None
        p.v_scale = None
        p.softmax_scale = float(softmax_scale) if softmax_scale is not None else 1.0 / math.sqrt(dqk)
        tensors.update(q=q, k=k, v=v)
    return DSAProblem(p, tensors, device)


def workspace_bytes(op: int, prob: DSAProblem) -> int:
    n = load_library().dsa_workspace_bytes(op, prob.ref())
    if n == ctypes.c_size_t(-1).value:
        raise DSAError(E_INVALID, last_error())
    return int(n)


def _workspace(op, prob, workspace):
    need = workspace_bytes(op, prob)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=prob.device)
    return workspace


def index_scores(prob: DSAProblem, scores=None, stream=None):
    """scores [B,n_q,n_k] fp32 (I past pos(t) is -inf)."""
    s = prob.struct
    if scores is None:
        scores = torch.empty((s.batch, s.n_q, s.n_k), dtype=torch.float32, device=prob.device)
    _check(load_library().dsa_index_scores(prob.ref(), _ptr(scores), _stream(stream)))
    return scores


def topk(prob: DSAProblem, scores, idx=None, workspace=None, stream=None):
    """idx [B,n_q,sel_width] int32: kept positions ascending, then -1."""
    s = prob.struct
    if idx is None:
        idx = torch.empty((s.batch, s.n_q, prob.sel_width), dtype=torch.int32, device=prob.device)
    ws = _workspace(OP_TOPK, prob, workspace)
    _check(load_library().dsa_topk(prob.ref(), _ptr(scores), _ptr(idx), _ptr(ws), ws.numel(),
                                   _stream(stream)))
    return idx


def _out_tensors(prob, out, lse):
    s = prob.struct
    dt = {F32: torch.float32, BF16: torch.bfloat16}[s.attn_dtype]
    if out is None:
        out = torch.empty((s.batch, s.n_q, s.q_heads, s.d_v), dtype=dt, device=prob.device)
    if lse is None:
        lse = torch.empty((s.batch, s.n_q, s.q_heads), dtype=torch.float32, device=prob.device)
    return out, lse


def sparse_attn(prob: DSAProblem, idx, out=None, lse=None, workspace=None, stream=None):
    """(out [B,n_q,Hq,dv], lse [B,n_q,Hq]) of attention over the rows in idx."""
    out, lse = _out_tensors(prob, out, lse)
    ws = _workspace(OP_SPARSE_ATTN, prob, workspace)
    _check(load_library().dsa_sparse_attn(prob.ref(), _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                          _stream(stream)))
    return out, lse


def _fused(fn, op, prob, out, lse, idx_out, workspace, stream):
    out, lse = _out_tensors(prob, out, lse)
    ws = _workspace(op, prob, workspace)
    _check(fn(prob.ref(), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse, idx_out


def prefill(prob: DSAProblem, out=None, lse=None, idx_out=None, workspace=None, stream=None):
    return _fused(load_library().dsa_prefill, OP_PREFILL, prob, out, lse, idx_out, workspace, stream)


def decode(prob: DSAProblem, out=None, lse=None, idx_out=None, workspace=None, stream=None):
    return _fused(load_library().dsa_decode, OP_DECODE, prob, out, lse, idx_out, workspace, stream)


def decode_noalloc(prob: DSAProblem, out=None, lse=None, idx_out=None, stream=None):
    """dsa_decode on the library's static per-GPU scratch (no workspace).  Calls
    on one GPU must not overlap; out/lse are allocated here only when not given."""
    out, lse = _out_tensors(prob, out, lse)
    _check(load_library().dsa_decode_noalloc(prob.ref(), _ptr(out), _ptr(lse), _ptr(idx_out), _stream(stream)))
    return out, lse, idx_out


def dense_attn(prob: DSAProblem, out=None, lse=None, workspace=None, stream=None):
    """(out, lse) of dense causal attention: every query over all its visible keys."""
    out, lse = _out_tensors(prob, out, lse)
    ws = _workspace(OP_DENSE_ATTN, prob, workspace)
    _check(load_library().dsa_dense_attn(prob.ref(), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                         _stream(stream)))
    return out, lse


class KVCompressed(ctypes.Structure):
    """dsa_kv_compressed_t: output pointers of dsa_compress_kv."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("ik", ctypes.c_void_p),
                ("ik_scale", ctypes.c_void_p), ("pos", ctypes.c_void_p)]


def compress_kept(n_k: int, window: int, keep_old: int) -> int:
    """Tokens per sequence that dsa_compress_kv keeps."""
    return int(load_library().dsa_compress_kept(n_k, window, keep_old))


def compress_kv(prob: DSAProblem, importance, window: int, keep_old: int, out=None, workspace=None, stream=None):
    """Importance compression of the cache `prob` points at (see dsa_compress_kv).

    Returns a dict of the compressed cache: k, v (None when latent), ik and
    ik_scale (None when the problem has none) with n_k replaced by n_keep, and
    pos [B, n_keep] int32, the kept tokens' original positions.
    """
    s = prob.struct
    t = prob.tensors
    importance = _contig("importance", importance, prob.device, (torch.float32,))
    n_keep = compress_kept(s.n_k, window, keep_old)

    def like(x):
        return None if x is None else torch.empty((x.shape[0], n_keep, *x.shape[2:]), dtype=x.dtype,
                                                  device=prob.device)
    if out is None:
        out = dict(k=like(t.get("k")), v=like(t.get("v")), ik=like(t.get("ik")), ik_scale=like(t.get("ik_scale")),
                   pos=torch.empty((s.batch, n_keep), dtype=torch.int32, device=prob.device))
    o = KVCompressed(*(None if out.get(n) is None else out[n].data_ptr()
                       for n in ("k", "v", "ik", "ik_scale", "pos")))
    ws = _workspace(OP_COMPRESS_KV, prob, workspace)
    _check(load_library().dsa_compress_kv(prob.ref(), _ptr(importance), int(window), int(keep_old),
                                          ctypes.byref(o), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def phase_timing(enable: bool):
    """Turn the fused entry points' phase timer on or off (see dsa_phase_timing)."""
    _check(load_library().dsa_phase_timing(1 if enable else 0))


def phase_times() -> dict:
    """GPU microseconds per phase of the latest timed fused call (waits for it)."""
    buf = (ctypes.c_float * len(PHASES))()
    _check(load_library().dsa_phase_times(buf))
    return {name: float(buf[i]) for i, name in enumerate(PHASES)}
