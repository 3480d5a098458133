"""dsa_decode_noalloc: the fused decode on the library's static per-GPU scratch
(no workspace argument, nothing allocated), called through the C ABI and
compared with dsa_decode on a caller-allocated workspace.

Two calls in a row on the same GPU, the second on a smaller problem (and with
the selection kept in the scratch), so whatever the first call left in the
shared array must not leak into the second.  The same kernels run in both
entry points, so selections, outputs and lse must be identical.
"""
from __future__ import annotations

import ctypes

import pytest
import torch

import long_context_sparse_relu_amd as dsa
from dsa_inputs import custom_spec, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _compare(fields, seed, keep_idx):
    inp = make_inputs(custom_spec(name="noalloc", **fields), device=DEV, seed=seed)
    prob = dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=inp["top_k"], q=inp["q"],
                            k=inp["k"], v=inp["v"], iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"],
                            softmax_scale=inp["scale"], latent_dv=inp["latent_dv"])
    B, k = fields["B"], fields["top_k"]
    ref_idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    ref_out, ref_lse, _ = dsa.decode(prob, idx_out=ref_idx)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    idx = torch.full_like(ref_idx, -7) if keep_idx else None
    lib = dsa.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.dsa_decode_noalloc(prob.ref(), _ptr(out), _ptr(lse), _ptr(idx), stream)
    assert st == dsa.OK, dsa.last_error()
    torch.cuda.synchronize()
    if keep_idx:
        assert torch.equal(idx, ref_idx), "selections differ"
    assert torch.equal(out, ref_out), "outputs differ"
    assert torch.equal(lse, ref_lse), "lse differs"


def test_noalloc_decode_matches_decode_on_two_calls():
    # long rows: the sampled top-k (candidate lists, bound, recompute row in the scratch)
    _compare(dict(B=8, n_q=1, n_k=131072, idx_heads=16, idx_dtype="e4m3", top_k=2048, q_heads=32,
                  kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16"), seed=1, keep_idx=True)
    # smaller: fewer, shorter rows; the selection lives in the scratch too
    _compare(dict(B=3, n_q=1, n_k=20000, idx_heads=16, idx_dtype="e4m3", top_k=256, q_heads=8,
                  kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16"), seed=2, keep_idx=False)
