"""Seeded synthetic inputs for the DSA hot path.

This module serves both sides -- the HIP library's tests/benchmark and the fp64
oracle -- and therefore holds none of the method's arithmetic: it only draws
random tensors, plants needle keys, scales outlier tokens and stores values in
the formats the path consumes (fp32, bf16, OCP FP8 E4M3 codes with one fp32
scale per token row).

Workloads (all Gaussian; q_I, k_I ~ N(0,1)/sqrt(128), indexer head weights
w ~ N(0,1)/2, main q/k/v ~ N(0,1), softmax scale 1/sqrt(d_qk)):

  tiny_prefill_f32  1 sequence, L=512, indexer 4x128 fp32, k=64, attention
                    8 heads x 64 fp32 MHA, 16 planted needles, seed 0
  prefill_bf16_8k   1 sequence, L=8192, indexer 16x128 bf16, k=2048,
                    attention 16x128 bf16 MHA, 64 planted needles
  prefill_fp8_32k   1 sequence, L=32768, indexer 16x128 E4M3 + per-token
                    scale, k=2048, attention 32x128 bf16 MHA, 0.1% of tokens
                    scaled x8 before quantisation
  decode_128k       64 sequences x 1 query over 131072 cached tokens, indexer
                    16x128 E4M3 cache, k=2048, bf16 KV with 32 query heads
                    over 4 KV heads (GQA), d=128, seeded per sequence
  decode_1m         8 sequences x 1 query over 1048576 tokens, indexer 16x128
                    E4M3, k=512, one shared latent bf16 row of width 576 per
                    token (value = first 512 entries), 128 query heads,
                    256 planted needles per sequence
  prefill_fp8_128k  prefill_fp8_32k's shapes at L=131072 (128K context, k=2048,
                    about 1.6% of the longest prefix)
  decode_128k_fp8kv decode_128k with the main KV cache stored as E4M3 codes
                    and one fp32 scale per (token, kv head) row
  decode_128k_backbone  decode_128k with 4 sink tokens and a 4096-key local
                    window kept besides the top-k (sinks / window fields)
  decode_1m_window  decode_1m with an 8192-key local window

Any spec may set kv_dtype="e4m3" (with attn_dtype "bf16"): the main k and v
are drawn as above and stored as E4M3 codes with one fp32 scale (amax/448) per
(token, kv head) row, in k_scale / v_scale [B,n_k,Hkv] (latent rows: k_scale
only), and packed as the library takes them, token records of codes then
scales (k_rec / v_rec; kv_args gives a problem's k / v arguments either way).

A needle is an indexer key made a noisy copy of one query's strongest head:
for a random key position s and a query t >= s, h = argmax_h w[t,h] (the query
is redrawn if no weight is positive) and k_I[s] = q_I[t,h] + 0.1*N(0,1)/sqrt(128).
"""
from __future__ import annotations

import math

import numpy as np
import torch

E4M3_MAX = 448.0  # largest finite OCP E4M3 value (1.75 * 2^8)

CONFIGS: dict[str, dict] = {
    "tiny_prefill_f32": dict(B=1, n_q=512, n_k=512, idx_heads=4, idx_dim=128, idx_dtype="f32",
                             top_k=64, q_heads=8, kv_heads=8, d_qk=64, d_v=64, latent=False,
                             attn_dtype="f32", needles=16, outlier_frac=0.0, w_bf16=False),
    "prefill_bf16_8k": dict(B=1, n_q=8192, n_k=8192, idx_heads=16, idx_dim=128, idx_dtype="bf16",
                            top_k=2048, q_heads=16, kv_heads=16, d_qk=128, d_v=128, latent=False,
                            attn_dtype="bf16", needles=64, outlier_frac=0.0, w_bf16=True),
    "prefill_fp8_32k": dict(B=1, n_q=32768, n_k=32768, idx_heads=16, idx_dim=128,
                            idx_dtype="e4m3", top_k=2048, q_heads=32, kv_heads=32, d_qk=128,
                            d_v=128, latent=False, attn_dtype="bf16", needles=0,
                            outlier_frac=0.001, w_bf16=False),
    "decode_128k": dict(B=64, n_q=1, n_k=131072, idx_heads=16, idx_dim=128, idx_dtype="e4m3",
                        top_k=2048, q_heads=32, kv_heads=4, d_qk=128, d_v=128, latent=False,
                        attn_dtype="bf16", needles=0, outlier_frac=0.0, w_bf16=False),
    "decode_1m": dict(B=8, n_q=1, n_k=1048576, idx_heads=16, idx_dim=128, idx_dtype="e4m3",
                      top_k=512, q_heads=128, kv_heads=1, d_qk=576, d_v=512, latent=True,
                      attn_dtype="bf16", needles=256, outlier_frac=0.0, w_bf16=False),
}
CONFIGS["prefill_fp8_128k"] = dict(CONFIGS["prefill_fp8_32k"], n_q=131072, n_k=131072)
CONFIGS["decode_128k_fp8kv"] = dict(CONFIGS["decode_128k"], kv_dtype="e4m3")
CONFIGS["decode_128k_backbone"] = dict(CONFIGS["decode_128k"], sinks=4, window=4096)
CONFIGS["decode_1m_window"] = dict(CONFIGS["decode_1m"], window=8192)

_TORCH_STORE = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}
_TENSOR_IDS = {"iq": 1, "ik": 2, "iw": 3, "q": 4, "k": 5, "v": 6, "needle": 7, "outlier": 8,
               "importance": 9}


def spec(name: str, **overrides) -> dict:
    s = dict(CONFIGS[name])
    s.update(overrides)
    s["name"] = name
    return s


def custom_spec(**fields) -> dict:
    """A spec with explicit fields (used for small and edge-case shapes)."""
    base = dict(B=1, n_q=8, n_k=8, idx_heads=4, idx_dim=128, idx_dtype="f32", top_k=4,
                q_heads=2, kv_heads=2, d_qk=64, d_v=64, latent=False, attn_dtype="f32",
                needles=0, outlier_frac=0.0, w_bf16=False, name="custom")
    base.update(fields)
    return base


def _gen(device, seed: int, tensor: str, b: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + _TENSOR_IDS[tensor] * 10_007 + int(b))
    return g


def _randn(shape, g, device):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def quantize_e4m3_per_row(x: torch.Tensor):
    """Store fp32 rows as E4M3 codes with one fp32 scale per row (amax/448).

    `x` is [..., n]; the scale is shared by the last dimension.  Values are
    rounded to nearest-even by torch's cast after clamping to +-448.  Returns
    (codes float8_e4m3fn [..., n], scale float32 [...]).
    """
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn), scale.to(torch.float32)


def pack_fp8_kv_records(codes: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """An FP8 cache's token records: codes [B,n_k,Hkv,d] float8_e4m3fn and
    scales [B,n_k,Hkv] fp32 -> uint8 [B,n_k,rec], each token's Hkv*d code
    bytes, then its Hkv fp32 scales (little-endian), then zeros up to a
    multiple of 16 bytes (the layout the library's header defines)."""
    B, n_k, Hkv, d = codes.shape
    rec = (Hkv * d + 4 * Hkv + 15) // 16 * 16
    out = torch.zeros((B, n_k, rec), dtype=torch.uint8, device=codes.device)
    out[:, :, :Hkv * d] = codes.contiguous().view(torch.uint8).reshape(B, n_k, Hkv * d)
    out[:, :, Hkv * d:Hkv * d + 4 * Hkv] = scale.contiguous().view(torch.uint8).reshape(B, n_k, 4 * Hkv)
    return out


def kv_args(inp: dict) -> dict:
    """The main k / v arguments of a problem over `inp`: the tensors as drawn,
    or an FP8 cache's token records with kv_heads and d_v."""
    if inp["kv_dtype"] != "e4m3":
        return dict(k=inp["k"], v=inp["v"], latent_dv=inp["latent_dv"])
    return dict(k=inp["k_rec"], v=inp["v_rec"], latent_dv=inp["latent_dv"], kv_heads=inp["kv_heads"],
                d_v=None if inp["v"] is None else inp["d_v"])


def make_inputs(s: dict, device="cpu", seed: int = 0) -> dict:
    """Draw one input set for spec `s` on `device`.

    Returns a dict of tensors in stored form:
      iq [B,n_q,H,D], iq_scale [B,n_q] (E4M3 only), ik [B,n_k,D], ik_scale [B,n_k],
      iw [B,n_q,H] fp32, q [B,n_q,Hq,dqk], k [B,n_k,Hkv,dqk], v [B,n_k,Hkv,dv] or
      None (latent), k_scale / v_scale [B,n_k,Hkv] (E4M3 cache only, else None),
      and for an E4M3 cache k_rec / v_rec, the same as token records
      (pack_fp8_kv_records; v_rec None when latent),
      pos [B,n_q] int32 (last visible key: n_k-n_q+t),
    and the scalars of the spec plus `scale` = 1/sqrt(d_qk).
    """
    B, n_q, n_k = s["B"], s["n_q"], s["n_k"]
    H, D = s["idx_heads"], s["idx_dim"]
    Hq, Hkv, dqk, dv = s["q_heads"], s["kv_heads"], s["d_qk"], s["d_v"]
    idt, adt = s["idx_dtype"], s["attn_dtype"]
    kvt = s.get("kv_dtype") or adt
    if kvt != adt:
        assert kvt == "e4m3" and adt == "bf16", "an FP8 cache goes with bf16 queries"
    latent = bool(s["latent"])
    if latent:
        assert Hkv == 1 and dv <= dqk
    out = {k: v for k, v in s.items()}
    out["kv_dtype"] = kvt
    out["scale"] = 1.0 / math.sqrt(dqk)
    out["latent_dv"] = dv if latent else None
    pos = (torch.arange(n_q, dtype=torch.int32) + (n_k - n_q)).expand(B, n_q).contiguous()
    out["pos"] = pos.to(device)

    iq_l, iqs_l, ik_l, iks_l, iw_l, q_l, k_l, v_l, ks_l, vs_l = ([] for _ in range(10))
    needle_pairs = []
    for b in range(B):
        iq = _randn((n_q, H, D), _gen(device, seed, "iq", b), device) / math.sqrt(D)
        ik = _randn((n_k, D), _gen(device, seed, "ik", b), device) / math.sqrt(D)
        iw = _randn((n_q, H), _gen(device, seed, "iw", b), device) / 2.0
        if s.get("w_bf16"):
            iw = iw.to(torch.bfloat16).to(torch.float32)
        if s.get("needles", 0):
            for key, query in _plant_needles(iq, ik, iw, int(s["needles"]), n_k - n_q,
                                             _gen("cpu", seed, "needle", b)):
                needle_pairs.append((b, key, query))
        if s.get("outlier_frac", 0.0) > 0:
            _scale_outliers(iq, ik, float(s["outlier_frac"]), n_k - n_q,
                            _gen("cpu", seed, "outlier", b))
        if idt == "e4m3":
            c, sc = quantize_e4m3_per_row(iq.reshape(n_q, H * D))
            iq_l.append(c.reshape(n_q, H, D)); iqs_l.append(sc)
            c, sc = quantize_e4m3_per_row(ik)
            ik_l.append(c); iks_l.append(sc)
        else:
            iq_l.append(iq.to(_TORCH_STORE[idt])); ik_l.append(ik.to(_TORCH_STORE[idt]))
        iw_l.append(iw)
        q_l.append(_randn((n_q, Hq, dqk), _gen(device, seed, "q", b), device).to(_TORCH_STORE[adt]))
        kb = _randn((n_k, Hkv, dqk), _gen(device, seed, "k", b), device)
        vb = None if latent else _randn((n_k, Hkv, dv), _gen(device, seed, "v", b), device)
        if kvt == "e4m3":
            c, sc = quantize_e4m3_per_row(kb)
            k_l.append(c); ks_l.append(sc)
            if vb is not None:
                c, sc = quantize_e4m3_per_row(vb)
                v_l.append(c); vs_l.append(sc)
        else:
            k_l.append(kb.to(_TORCH_STORE[kvt]))
            if vb is not None:
                v_l.append(vb.to(_TORCH_STORE[kvt]))
    out["iq"] = torch.stack(iq_l)
    out["ik"] = torch.stack(ik_l)
    out["iq_scale"] = torch.stack(iqs_l) if idt == "e4m3" else None
    out["ik_scale"] = torch.stack(iks_l) if idt == "e4m3" else None
    out["iw"] = torch.stack(iw_l)
    out["q"] = torch.stack(q_l)
    out["k"] = torch.stack(k_l)
    out["v"] = torch.stack(v_l) if not latent else None
    out["k_scale"] = torch.stack(ks_l) if ks_l else None
    out["v_scale"] = torch.stack(vs_l) if vs_l else None
    if kvt == "e4m3":
        out["k_rec"] = pack_fp8_kv_records(out["k"], out["k_scale"])
        out["v_rec"] = None if latent else pack_fp8_kv_records(out["v"], out["v_scale"])
    out["needle_pairs"] = needle_pairs
    return out


def _plant_needles(iq, ik, iw, count, offset, g):
    """Make `count` distinct indexer keys noisy copies of some query's best head.

    Returns the (key position, source query row) pairs that were planted.
    """
    n_q, H, D = iq.shape
    n_k = ik.shape[0]
    count = min(count, n_k)
    keys = torch.randperm(n_k, generator=g)[:count].tolist()
    dev = ik.device
    w_host = iw.detach().to("cpu")
    planted = []
    for s in keys:
        # queries that can see key s: t with offset + t >= s
        t_lo = max(0, s - offset)
        if t_lo >= n_q:
            continue
        for _ in range(64):
            t = int(torch.randint(t_lo, n_q, (1,), generator=g))
            h = int(torch.argmax(w_host[t]))
            if float(w_host[t, h]) > 0:
                break
        else:
            continue
        noise = torch.randn(D, generator=g).to(dev) * (0.1 / math.sqrt(D))
        ik[s] = iq[t, h] + noise
        planted.append((s, t))
    return planted


def _scale_outliers(iq, ik, frac, offset, g):
    """Multiply the indexer q and k rows of round(frac*n_k) tokens by 8."""
    n_q = iq.shape[0]
    n_k = ik.shape[0]
    count = int(round(frac * n_k))
    toks = torch.randperm(n_k, generator=g)[:count].tolist()
    for s in toks:
        ik[s] *= 8.0
        t = s - offset
        if 0 <= t < n_q:
            iq[t] *= 8.0


def stored_numpy(t):
    """Host numpy copy of a stored tensor: float32, bf16 bits as uint16, E4M3 codes as uint8."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy()
    raise TypeError(f"unexpected stored dtype {t.dtype}")


def oracle_view(inp: dict, seqs=None) -> dict:
    """Numpy copies (stored form) of the sequences `seqs` (default: all) for the oracle."""
    B = inp["iq"].shape[0]
    seqs = list(range(B)) if seqs is None else list(seqs)
    sel = torch.tensor(seqs, dtype=torch.long)
    res = {k: v for k, v in inp.items()
           if not isinstance(v, torch.Tensor) and v is not None and k != "needle_pairs"}
    res["needle_pairs"] = [(seqs.index(b), s, t) for (b, s, t) in inp.get("needle_pairs", [])
                           if b in seqs]
    res["latent_dv"] = inp.get("latent_dv")
    for name in ("iq", "iq_scale", "ik", "ik_scale", "iw", "q", "k", "v", "k_scale", "v_scale", "pos"):
        t = inp.get(name)
        if t is None:
            res[name] = None
            continue
        res[name] = stored_numpy(t.index_select(0, sel.to(t.device)))
    res["seq_ids"] = seqs
    return res


def importance_scores(B: int, n_k: int, kind: str = "normal", device="cpu", seed: int = 0) -> torch.Tensor:
    """Per-token importance [B, n_k] fp32 for cache compression.

    kind "normal": standard normal draws; "ties": integers in [-3, 3] with every
    zero's sign drawn at random (many equal values, -0.0 beside +0.0); "const":
    all zeros, half of them -0.0 (every token ties).
    """
    rows = []
    for b in range(B):
        g = _gen("cpu", seed, "importance", b)
        if kind == "normal":
            x = torch.randn(n_k, generator=g, dtype=torch.float32)
        elif kind == "ties":
            x = torch.randint(-3, 4, (n_k,), generator=g).to(torch.float32)
            neg = torch.randint(0, 2, (n_k,), generator=g).bool() & (x == 0)
            x = torch.where(neg, torch.full_like(x, -0.0), x)
        elif kind == "const":
            x = torch.zeros(n_k, dtype=torch.float32)
            x[1::2] = -0.0
        else:
            raise ValueError(f"unknown importance kind {kind!r}")
        rows.append(x)
    return torch.stack(rows).to(device)

