"""GPU parity of dsa_compress_kv (importance compression of the cache).

The kept positions are compared bit for bit with oracle.compress_select on the
same importance (an integer result decided by comparisons of the same fp32
values), every copied row bit for bit with the input row at that position, and
a decode over a compressed cache with the oracle's decode over the same
compressed tensors.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import long_context_sparse_relu_amd as dsa
import oracle
from dsa_inputs import custom_spec, importance_scores, kv_args, make_inputs, oracle_view, spec

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)

_GQA = dict(n_q=1, idx_heads=16, idx_dtype="e4m3", top_k=256, q_heads=8, kv_heads=2, d_qk=128, d_v=128,
            attn_dtype="bf16")
_LATENT = dict(n_q=1, idx_heads=16, idx_dtype="e4m3", top_k=128, q_heads=16, kv_heads=1, d_qk=576, d_v=512,
               latent=True, attn_dtype="bf16")

# (case, spec fields, window, keep_old, importance kind); the sizes span several
# 4096-token chunks and 16384-token histogram blocks with ragged tails
CASES = [
    ("gqa_normal", dict(_GQA, B=2, n_k=40000), 3000, 15000, "normal"),
    ("gqa_ties", dict(_GQA, B=3, n_k=20001), 1000, 7000, "ties"),
    ("all_tied", dict(_GQA, B=1, n_k=9000), 500, 4000, "const"),
    ("fp8_kv", dict(_GQA, B=2, n_k=12345, kv_dtype="e4m3"), 100, 5000, "normal"),
    ("latent_ties", dict(_LATENT, B=2, n_k=10000), 2048, 3000, "ties"),
    ("f32_small", dict(B=2, n_q=8, n_k=300), 50, 100, "ties"),
    ("bf16_idx", dict(_GQA, B=1, n_k=5000, idx_dtype="bf16"), 64, 999, "normal"),
    ("keep_none", dict(_GQA, B=2, n_k=5000), 64, 0, "normal"),
    ("keep_every_old", dict(_GQA, B=2, n_k=5000), 64, 10 ** 6, "normal"),
    ("window_covers_all", dict(_GQA, B=1, n_k=3000), 4096, 10, "normal"),
    ("no_window", dict(_GQA, B=2, n_k=7000), 0, 1234, "ties"),
    ("one_token", dict(_GQA, B=1, n_k=1), 0, 1, "normal"),
]


def _problem(inp):
    return dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=inp["top_k"], q=inp["q"],
                            iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"], softmax_scale=inp["scale"],
                            **kv_args(inp))


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _check_compressed(inp, imp, window, keep_old, res):
    B = imp.shape[0]
    kv = kv_args(inp)
    n_keep = dsa.compress_kept(imp.shape[1], window, keep_old)
    assert res["pos"].shape == (B, n_keep)
    imp_h = imp.cpu().numpy()
    for b in range(B):
        want = oracle.compress_select(imp_h[b], window, keep_old)
        got = res["pos"][b].cpu().numpy()
        assert np.array_equal(got, want), f"sequence {b}: kept positions differ"
        sel = torch.as_tensor(want, dtype=torch.long, device=DEV)
        for name, src in (("k", kv["k"]), ("v", kv["v"]), ("ik", inp["ik"]), ("ik_scale", inp["ik_scale"])):
            if src is None:
                assert res[name] is None
                continue
            assert torch.equal(_bits(res[name][b]), _bits(src[b].index_select(0, sel))), f"{name} rows of {b}"


@pytest.mark.parametrize("case,fields,window,keep_old,kind", CASES, ids=[c[0] for c in CASES])
def test_compress_matches_oracle(case, fields, window, keep_old, kind):
    inp = make_inputs(custom_spec(name=case, **fields), device=DEV, seed=3)
    imp = importance_scores(fields["B"], fields["n_k"], kind, device=DEV, seed=5)
    prob = _problem(inp)
    res = dsa.compress_kv(prob, imp, window, keep_old)
    torch.cuda.synchronize()
    _check_compressed(inp, imp, window, keep_old, res)


def test_compress_twice_reuses_workspace():
    # a second call on the same workspace with another cut: nothing of the first survives
    fields = dict(_GQA, B=2, n_k=30000)
    inp = make_inputs(custom_spec(name="twice", **fields), device=DEV, seed=4)
    prob = _problem(inp)
    ws = torch.empty(dsa.workspace_bytes(dsa.OP_COMPRESS_KV, prob), dtype=torch.uint8, device=DEV)
    for kind, window, keep in (("normal", 2000, 20000), ("ties", 100, 3000)):
        imp = importance_scores(2, 30000, kind, device=DEV, seed=6)
        res = dsa.compress_kv(prob, imp, window, keep, workspace=ws)
        torch.cuda.synchronize()
        _check_compressed(inp, imp, window, keep, res)


def test_decode_over_compressed_cache_matches_oracle():
    fields = dict(_GQA, B=2, n_k=20000, top_k=512)
    inp = make_inputs(custom_spec(name="dec_after_compress", **fields), device=DEV, seed=7)
    imp = importance_scores(2, 20000, "normal", device=DEV, seed=8)
    res = dsa.compress_kv(_problem(inp), imp, 4096, 6000)
    n_keep = res["pos"].shape[1]
    small = dict(inp)
    small.update(n_k=n_keep, k=res["k"], v=res["v"], ik=res["ik"], ik_scale=res["ik_scale"],
                 pos=torch.full((2, 1), n_keep - 1, dtype=torch.int32, device=DEV))
    prob = _problem(small)
    idx = torch.empty((2, 1, small["top_k"]), dtype=torch.int32, device=DEV)
    out, lse, _ = dsa.decode(prob, idx_out=idx)
    torch.cuda.synchronize()
    ref = oracle.dsa_forward(oracle_view(small))
    for (b, t), r in ref.items():
        g = idx[b, t].cpu().numpy()
        assert np.array_equal(np.sort(g[g >= 0]), np.sort(r["idx"][r["idx"] >= 0])), f"selection of {b}"
        err = float(np.abs(out[b, t].float().cpu().numpy() - r["out"]).max())
        assert err <= 2e-2, f"attention error {err} at sequence {b}"
        assert np.allclose(lse[b, t].cpu().numpy(), r["lse"], atol=2e-3)


def test_compress_full_size_1m_latent_cache():
    # the benchmarked cut: 8 sequences of 1M tokens (576-wide latent rows, FP8
    # indexer keys), an 8K window and half of the older tokens
    s = spec("decode_1m")
    inp = make_inputs(s, device=DEV, seed=0)
    n = s["n_k"]
    imp = importance_scores(s["B"], n, "normal", device=DEV, seed=0)
    res = dsa.compress_kv(_problem(inp), imp, 8192, (n - 8192) // 2)
    torch.cuda.synchronize()
    _check_compressed(inp, imp, 8192, (n - 8192) // 2, res)
