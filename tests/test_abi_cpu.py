"""CPU checks of the C ABI: the library loads, exports what include/dsa.h
declares, its struct layout matches the binding, and host-side validation
rejects bad calls before anything reaches a device (no kernel is launched in
these tests: every call here fails validation first)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import long_context_sparse_relu_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        pytest.fail("libdsa.so is not built (python -m long_context_sparse_relu_amd.build)")
    return dsa.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_header_declarations_are_exported(lib):
    names = _declared()
    assert set(names) == set(dsa.EXPORTED)
    for n in names:
        assert hasattr(lib, n), f"{n} missing from libdsa.so"
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (dsa_\w+)", out))
    assert exported == set(names)


def test_abi_version_and_status_strings(lib):
    assert lib.dsa_abi_version() == dsa.ABI_VERSION
    for st in (dsa.OK, dsa.E_INVALID, dsa.E_UNSUPPORTED, dsa.E_WORKSPACE, dsa.E_DEVICE):
        assert dsa.status_str(st).startswith("DSA_")
    assert "unknown" in dsa.status_str(42)


def test_struct_layout_matches_header(tmp_path):
    fields = [f[0] for f in dsa.Problem._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'    printf("%s %zu\\n", "{f}", offsetof(dsa_problem_t, {f}));' for f in fields)
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"dsa.h\"\nint main(void){\n"
                   + body + '\n    printf("sizeof %zu\\n", sizeof(dsa_problem_t));\n    return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(dsa.Problem, f).offset, f
    assert int(got["sizeof"]) == ctypes.sizeof(dsa.Problem)


def test_fp8_kv_record_layout(tmp_path):
    """The header's record size macro, the binding's and the input packer agree:
    each token's codes, then its per-head fp32 scales, then zeros to 16 bytes."""
    import torch
    from dsa_inputs import pack_fp8_kv_records
    cases = [(4, 128), (1, 576), (1, 512), (2, 64), (3, 128), (8, 128)]
    src = tmp_path / "rec.c"
    body = "\n".join(f'    printf("%d\\n", DSA_FP8_KV_RECORD_BYTES({h}, {d}));' for h, d in cases)
    src.write_text("#include <stdio.h>\n#include \"dsa.h\"\nint main(void){\n" + body + "\n    return 0;\n}\n")
    exe = tmp_path / "rec"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    for (h, d), n in zip(cases, got):
        assert n == dsa.fp8_kv_record_bytes(h, d)
        assert n % 16 == 0 and h * d + 4 * h <= n < h * d + 4 * h + 16
    g = torch.Generator().manual_seed(5)
    codes = (torch.randn((2, 3, 3, 8), generator=g) * 4).to(torch.float8_e4m3fn)
    scale = torch.rand((2, 3, 3), generator=g) + 0.5
    rec = pack_fp8_kv_records(codes, scale)
    assert rec.shape == (2, 3, dsa.fp8_kv_record_bytes(3, 8)) and rec.dtype == torch.uint8
    for b in range(2):
        for s in range(3):
            r = rec[b, s]
            assert torch.equal(r[:24], codes[b, s].reshape(-1).view(torch.uint8))
            assert torch.equal(r[24:36].view(torch.float32), scale[b, s])
            assert torch.all(r[36:] == 0)


def _problem(**over):
    p = dsa.Problem()
    p.batch, p.n_q, p.n_k = 2, 1, 4096
    p.idx_heads, p.idx_dim, p.idx_dtype = 16, 128, dsa.FP8_E4M3
    fake = 0x7F0000000000  # never dereferenced: every call below fails validation first
    p.iq = p.ik = p.iw = p.iq_scale = p.ik_scale = fake
    p.q_heads, p.kv_heads, p.d_qk, p.d_v, p.kv_latent = 32, 4, 128, 128, 0
    p.attn_dtype = p.kv_dtype = dsa.BF16
    p.q = p.k = p.v = fake
    p.softmax_scale = 0.088
    p.top_k = 2048
    for k, v in over.items():
        setattr(p, k, v)
    return p


FAKE = ctypes.c_void_p(0x7F0000000000)


@pytest.mark.parametrize("over,status", [
    (dict(batch=0), dsa.E_INVALID),
    (dict(n_q=0), dsa.E_INVALID),
    (dict(n_q=5000), dsa.E_INVALID),
    (dict(n_k=(1 << 24) + 1, n_q=1), dsa.E_UNSUPPORTED),
    (dict(idx_dim=64), dsa.E_UNSUPPORTED),
    (dict(idx_heads=65), dsa.E_UNSUPPORTED),
    (dict(idx_dtype=7), dsa.E_INVALID),
    (dict(iq_scale=None), dsa.E_INVALID),
    (dict(iw=None), dsa.E_INVALID),
    (dict(top_k=0), dsa.E_UNSUPPORTED),
    (dict(top_k=8193), dsa.E_UNSUPPORTED),
    (dict(kv_heads=5), dsa.E_INVALID),
    (dict(v=None), dsa.E_INVALID),
    (dict(kv_latent=1), dsa.E_INVALID),             # latent needs kv_heads == 1
    (dict(d_qk=1024), dsa.E_UNSUPPORTED),
    (dict(attn_dtype=dsa.FP8_E4M3), dsa.E_UNSUPPORTED),
    (dict(kv_dtype=dsa.F32), dsa.E_INVALID),         # neither attn_dtype nor FP8
    (dict(kv_dtype=dsa.FP8_E4M3, k_scale=0x7F0000000000), dsa.E_INVALID),   # scales live in the records
    (dict(kv_dtype=dsa.FP8_E4M3, v_scale=0x7F0000000000), dsa.E_INVALID),
    (dict(kv_dtype=dsa.FP8_E4M3, attn_dtype=dsa.F32), dsa.E_UNSUPPORTED),   # FP8 cache needs bf16 q
    (dict(attn_mode=3), dsa.E_INVALID),
    (dict(sink_tokens=-1), dsa.E_INVALID),
    (dict(local_window=-5), dsa.E_INVALID),
    (dict(top_k=8192, local_window=8193), dsa.E_UNSUPPORTED),          # selection row over 16384 entries
    (dict(attn_mode=dsa.ATTN_MASKED, q_heads=4, kv_heads=1, kv_latent=1, d_qk=576, d_v=512, v=None),
     dsa.E_UNSUPPORTED),                                                     # masked: d128 only
    (dict(softmax_scale=0.0), dsa.E_INVALID),
    (dict(softmax_scale=float("inf")), dsa.E_INVALID),
    (dict(n_q=2), dsa.E_INVALID),                   # decode takes one query row
])
def test_decode_validation(lib, over, status):
    p = _problem(**over)
    st = lib.dsa_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == status, dsa.last_error()
    assert dsa.last_error()


def test_dense_attn_validation(lib):
    p = _problem(n_q=64, n_k=4096)
    need = lib.dsa_workspace_bytes(dsa.OP_DENSE_ATTN, ctypes.byref(p))
    assert 0 < need < ctypes.c_size_t(-1).value          # 2 rows x 32 heads: the key walk is split
    assert lib.dsa_dense_attn(ctypes.byref(p), None, None, FAKE, need, None) == dsa.E_INVALID   # out missing
    assert lib.dsa_dense_attn(ctypes.byref(p), FAKE, None, FAKE, need - 1, None) == dsa.E_WORKSPACE
    fp32 = _problem(attn_dtype=dsa.F32, kv_dtype=dsa.F32)
    assert lib.dsa_dense_attn(ctypes.byref(fp32), FAKE, None, FAKE, need, None) == dsa.E_UNSUPPORTED
    assert lib.dsa_workspace_bytes(dsa.OP_DENSE_ATTN, ctypes.byref(fp32)) == ctypes.c_size_t(-1).value
    d64 = _problem(d_qk=64, d_v=64)
    assert lib.dsa_dense_attn(ctypes.byref(d64), FAKE, None, FAKE, need, None) == dsa.E_UNSUPPORTED
    assert "dense" in dsa.last_error()
    # the masked kernels address a sequence's K and V with 32-bit offsets:
    # n_k * kv_heads * 256 B must stay below 2 GiB (here exactly 2 GiB)
    huge = _problem(n_q=64, n_k=1 << 20, kv_heads=8, q_heads=8)
    assert lib.dsa_workspace_bytes(dsa.OP_DENSE_ATTN, ctypes.byref(huge)) == ctypes.c_size_t(-1).value
    assert lib.dsa_dense_attn(ctypes.byref(huge), FAKE, None, FAKE, 1 << 40, None) == dsa.E_UNSUPPORTED
    assert "2 GiB" in dsa.last_error()
    masked = _problem(n_q=64, n_k=1 << 18, kv_heads=32, q_heads=32, attn_mode=dsa.ATTN_MASKED)
    assert lib.dsa_sparse_attn(ctypes.byref(masked), FAKE, FAKE, None, FAKE, 1 << 40, None) == dsa.E_UNSUPPORTED
    assert "2 GiB" in dsa.last_error()
    fits = _problem(n_q=64, n_k=(1 << 20) - 64, kv_heads=8, q_heads=8)
    assert lib.dsa_workspace_bytes(dsa.OP_DENSE_ATTN, ctypes.byref(fits)) != ctypes.c_size_t(-1).value


def test_null_problem_and_outputs(lib):
    assert lib.dsa_index_scores(None, FAKE, None) == dsa.E_INVALID
    p = _problem()
    assert lib.dsa_index_scores(ctypes.byref(p), None, None) == dsa.E_INVALID
    assert lib.dsa_topk(ctypes.byref(p), None, FAKE, FAKE, 1 << 40, None) == dsa.E_INVALID
    assert lib.dsa_sparse_attn(ctypes.byref(p), None, FAKE, None, None, 0, None) == dsa.E_INVALID
    assert lib.dsa_prefill(ctypes.byref(p), None, None, None, FAKE, 1 << 40, None) == dsa.E_INVALID


def test_workspace_sizes_and_shortfall(lib):
    p = _problem()
    need_topk = lib.dsa_workspace_bytes(dsa.OP_TOPK, ctypes.byref(p))
    need_dec = lib.dsa_workspace_bytes(dsa.OP_DECODE, ctypes.byref(p))
    assert 0 < need_topk < need_dec
    assert lib.dsa_workspace_bytes(dsa.OP_INDEX_SCORES, ctypes.byref(p)) == 0
    assert lib.dsa_workspace_bytes(99, ctypes.byref(p)) == ctypes.c_size_t(-1).value
    assert lib.dsa_topk(ctypes.byref(p), FAKE, FAKE, FAKE, need_topk - 1, None) == dsa.E_WORKSPACE
    assert lib.dsa_topk(ctypes.byref(p), FAKE, FAKE, None, need_topk, None) == dsa.E_WORKSPACE
    # idx_out NULL: the workspace must also hold the selection, which is what need_dec counts
    assert lib.dsa_decode(ctypes.byref(p), FAKE, FAKE, None, FAKE, need_dec - 1, None) == dsa.E_WORKSPACE
    assert "workspace" in dsa.last_error()
    bad = _problem(n_q=3)
    assert lib.dsa_workspace_bytes(dsa.OP_DECODE, ctypes.byref(bad)) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("op", [dsa.OP_PREFILL, dsa.OP_DECODE])
@pytest.mark.parametrize("over", [dict(q_heads=0), dict(kv_heads=0), dict(kv_heads=5), dict(idx_heads=0),
                                  dict(idx_dim=64), dict(iw=None), dict(attn_dtype=7), dict(q=None)])
def test_fused_workspace_query_validates_like_the_entry_points(lib, op, over):
    """dsa_workspace_bytes for the fused ops runs the entry points' checks:
    a problem the call would reject sizes to SIZE_MAX (never a crash, e.g. a
    division by a zero head count while laying out the workspace)."""
    p = _problem(**over)
    assert lib.dsa_workspace_bytes(op, ctypes.byref(p)) == ctypes.c_size_t(-1).value
    assert dsa.last_error()


def test_noalloc_decode_rejects_problems_beyond_its_scratch(lib):
    """dsa_decode_noalloc validates like dsa_decode and refuses, before any
    device call, a problem whose scratch need exceeds the static array."""
    assert lib.dsa_decode_noalloc(ctypes.byref(_problem(n_q=2)), FAKE, FAKE, FAKE, None) == dsa.E_INVALID
    assert lib.dsa_decode_noalloc(ctypes.byref(_problem()), None, FAKE, FAKE, None) == dsa.E_INVALID
    big = _problem(batch=64, n_k=1 << 20)
    need = lib.dsa_workspace_bytes(dsa.OP_DECODE, ctypes.byref(big))
    assert need > dsa.NOALLOC_SCRATCH_BYTES
    assert lib.dsa_decode_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, None) == dsa.E_UNSUPPORTED
    assert "scratch" in dsa.last_error()


def test_binding_rejects_missing_library(tmp_path):
    saved = dsa._lib
    dsa._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            dsa.load_library(str(tmp_path / "nope.so"))
    finally:
        dsa._lib = saved


def test_phase_timer_without_a_timed_call(lib):
    """The timer's host side: nothing timed yet (or timing switched off) is an
    error, as is a NULL output; switching it on and off always succeeds."""
    assert lib.dsa_phase_timing(0) == dsa.OK
    assert lib.dsa_phase_times(None) == dsa.E_INVALID
    buf = (ctypes.c_float * len(dsa.PHASES))()
    assert lib.dsa_phase_times(buf) == dsa.E_INVALID
    assert "no timed" in dsa.last_error()
    assert lib.dsa_phase_timing(1) == dsa.OK
    assert lib.dsa_phase_times(buf) == dsa.E_INVALID
    assert lib.dsa_phase_timing(0) == dsa.OK


def test_compress_kept_counts(lib):
    assert dsa.compress_kept(12, 3, 4) == 7
    assert dsa.compress_kept(12, 20, 4) == 12
    assert dsa.compress_kept(12, 3, 100) == 12
    assert dsa.compress_kept(12, 0, 0) == 0
    assert dsa.compress_kept(1 << 20, 8192, ((1 << 20) - 8192) // 2) == 8192 + ((1 << 20) - 8192) // 2


def test_compress_validation(lib):
    p = _problem()
    need = lib.dsa_workspace_bytes(dsa.OP_COMPRESS_KV, ctypes.byref(p))
    assert 0 < need != ctypes.c_size_t(-1).value
    good = dsa.KVCompressed(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)

    def call(prob=p, imp=FAKE, window=8, keep=16, out=good, ws=FAKE, nbytes=need):
        return lib.dsa_compress_kv(ctypes.byref(prob), imp, window, keep, None if out is None else ctypes.byref(out),
                                   ws, nbytes, None)
    assert call(imp=None) == dsa.E_INVALID
    assert call(out=None) == dsa.E_INVALID
    assert call(window=-1) == dsa.E_INVALID
    assert call(keep=-1) == dsa.E_INVALID
    assert call(nbytes=need - 1) == dsa.E_WORKSPACE
    assert call(ws=None) == dsa.E_WORKSPACE
    assert call(out=dsa.KVCompressed(FAKE.value, None, FAKE.value, FAKE.value, FAKE.value)) == dsa.E_INVALID
    assert call(out=dsa.KVCompressed(FAKE.value, FAKE.value, FAKE.value, None, FAKE.value)) == dsa.E_INVALID
    assert call(out=dsa.KVCompressed(FAKE.value, FAKE.value, None, FAKE.value, FAKE.value)) == dsa.E_INVALID
    assert call(prob=_problem(kv_heads=0)) == dsa.E_INVALID
    assert call(prob=_problem(k=None)) == dsa.E_INVALID
    assert call(prob=_problem(kv_latent=1)) == dsa.E_INVALID          # latent with 4 kv heads
    assert call(prob=_problem(batch=1024, n_k=1 << 24)) == dsa.E_UNSUPPORTED
    assert lib.dsa_workspace_bytes(dsa.OP_COMPRESS_KV, ctypes.byref(_problem(kv_heads=0))) == \
        ctypes.c_size_t(-1).value
    # nothing to keep: valid, and nothing is enqueued (no device needed)
    assert call(window=0, keep=0) == dsa.OK


def test_compress_rejects_rows_not_a_multiple_of_four_bytes(lib):
    p = _problem(d_qk=63, d_v=63, kv_heads=1, q_heads=1)      # bf16 rows of 126 bytes
    need = lib.dsa_workspace_bytes(dsa.OP_COMPRESS_KV, ctypes.byref(p))
    out = dsa.KVCompressed(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    st = lib.dsa_compress_kv(ctypes.byref(p), FAKE, 8, 16, ctypes.byref(out), FAKE, need, None)
    assert st == dsa.E_UNSUPPORTED and "aligned" in dsa.last_error()
