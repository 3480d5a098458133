"""Pins for the fp64 oracle, checked against things other than the oracle itself.

Each test ties one part of the oracle to what the pages or mathematics fix:
format definitions checked against torch's own dtypes, algebraic identities of
the ReLU-weighted score, closed forms, brute force over all subsets, and the
textbook dense attention (torch's SDPA in float64) that sparse attention must
reduce to when k covers the whole prefix.  The method follows
"DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度解析" (sheratonhq.com) section 1.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import custom_spec, make_inputs, oracle_view, spec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- formats --

def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # S.1111.111 only: the format has no infinity
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**16, size=4000, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- indexer --

def _rand_index_problem(rng, n_q=6, n_k=9, H=3, D=16):
    iq = rng.standard_normal((n_q, H, D)).astype(np.float32)
    ik = rng.standard_normal((n_k, D)).astype(np.float32)
    iw = rng.standard_normal((n_q, H)).astype(np.float32)
    return iq, ik, iw


def test_index_scores_relu_identities():
    """ReLU(x) - ReLU(-x) = x and ReLU(x) + ReLU(-x) = |x| give two linear forms.

    I(k) - I(-k) = sum_h w_h (q_h . k)  and  I(k) + I(-k) = sum_h w_h |q_h . k|,
    both computed here with numpy matrix products: a dropped ReLU, a wrong sign,
    a transposed operand or a dropped weight all break one of them.
    """
    rng = np.random.default_rng(2)
    iq, ik, iw = _rand_index_problem(rng)
    n_q, n_k = iq.shape[0], ik.shape[0]
    pos = np.full(n_q, n_k - 1)
    plus = oracle.index_scores(iq, ik, iw, "f32", pos=pos)
    minus = oracle.index_scores(iq, -ik, iw, "f32", pos=pos)
    dots = np.einsum("thd,sd->ths", iq.astype(np.float64), ik.astype(np.float64))
    lin = np.einsum("th,ths->ts", iw.astype(np.float64), dots)
    absf = np.einsum("th,ths->ts", iw.astype(np.float64), np.abs(dots))
    np.testing.assert_allclose(plus - minus, lin, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(plus + minus, absf, rtol=1e-12, atol=1e-12)


def test_index_scores_hand_worked_example():
    with open(os.path.join(GOLDEN, "indexer_worked_example.json")) as f:
        ex = json.load(f)
    iq = np.array(ex["q_I"], dtype=np.float32)[None]          # one query
    ik = np.array(ex["k_I"], dtype=np.float32)
    iw = np.array(ex["w"], dtype=np.float32)[None]
    got = oracle.index_scores(iq, ik, iw, "f32", pos=[len(ik) - 1])[0]
    assert got.tolist() == ex["expected_scores"]
    idx, kth = oracle.topk(got[None], ex["top_k"], pos=[len(ik) - 1])
    assert idx[0].tolist() == ex["expected_topk"]
    assert kth[0] == ex["expected_kth"]


def test_index_scores_closed_form_self_match():
    """H=1, w=1 and k_I[s] = q_I[t] give I[t,s] = |q_I[t]|^2."""
    rng = np.random.default_rng(3)
    D = 128
    q = rng.standard_normal((5, 1, D)).astype(np.float32)
    k = q[:, 0, :].copy()
    w = np.ones((5, 1), dtype=np.float32)
    sc = oracle.index_scores(q, k, w, "f32", pos=np.full(5, 4))
    want = np.sum(q[:, 0, :].astype(np.float64) ** 2, axis=1)
    np.testing.assert_allclose(np.diag(sc), want, rtol=1e-13)


def test_index_scores_causal_mask():
    rng = np.random.default_rng(4)
    iq, ik, iw = _rand_index_problem(rng, n_q=7, n_k=7)
    sc = oracle.index_scores(iq, ik, iw, "f32")  # default pos[t] = t
    assert np.all(np.isneginf(sc[np.triu_indices(7, 1)]))
    assert np.all(np.isfinite(sc[np.tril_indices(7)]))
    ik2 = ik.copy()
    ik2[5:] = rng.standard_normal(ik2[5:].shape)
    sc2 = oracle.index_scores(iq, ik2, iw, "f32")
    assert np.array_equal(sc[:5, :5], sc2[:5, :5])  # future keys change nothing before them


def test_index_scores_head_permutation_and_scaling():
    rng = np.random.default_rng(5)
    iq, ik, iw = _rand_index_problem(rng, H=5)
    pos = np.full(iq.shape[0], ik.shape[0] - 1)
    base = oracle.index_scores(iq, ik, iw, "f32", pos=pos)
    perm = rng.permutation(5)
    permuted = oracle.index_scores(iq[:, perm], ik, iw[:, perm], "f32", pos=pos)
    np.testing.assert_allclose(permuted, base, rtol=1e-12, atol=1e-14)
    scaled = oracle.index_scores(iq, 4.0 * ik, iw, "f32", pos=pos)  # c>0: I scales by c
    np.testing.assert_allclose(scaled, 4.0 * base, rtol=1e-12, atol=1e-14)


def test_index_scores_fp8_scale_factorisation():
    """Positive per-token scales leave ReLU's kink in place: I = sq*sk*I(codes)."""
    rng = np.random.default_rng(6)
    n_q, n_k, H, D = 4, 11, 3, 128
    iq = rng.integers(0, 256, (n_q, H, D), dtype=np.uint8)
    ik = rng.integers(0, 256, (n_k, D), dtype=np.uint8)
    iq[(iq & 0x7F) == 0x7F] = 0x10  # no NaN codes
    ik[(ik & 0x7F) == 0x7F] = 0x10
    iw = rng.standard_normal((n_q, H)).astype(np.float32)
    sq = rng.uniform(0.01, 2.0, n_q).astype(np.float32)
    sk = rng.uniform(0.01, 2.0, n_k).astype(np.float32)
    pos = np.full(n_q, n_k - 1)
    unit = oracle.index_scores(iq, ik, iw, "e4m3", pos=pos)
    scaled = oracle.index_scores(iq, ik, iw, "e4m3", sq, sk, pos=pos)
    want = unit * sq.astype(np.float64)[:, None] * sk.astype(np.float64)[None, :]
    np.testing.assert_allclose(scaled, want, rtol=1e-12, atol=1e-300)


def test_index_scores_bf16_equals_f32_on_bf16_values():
    rng = np.random.default_rng(7)
    iq, ik, iw = _rand_index_problem(rng)
    iq_b = torch.from_numpy(iq).to(torch.bfloat16)
    ik_b = torch.from_numpy(ik).to(torch.bfloat16)
    pos = np.full(iq.shape[0], ik.shape[0] - 1)
    a = oracle.index_scores(iq_b.view(torch.int16).numpy().view(np.uint16),
                            ik_b.view(torch.int16).numpy().view(np.uint16), iw, "bf16", pos=pos)
    b = oracle.index_scores(iq_b.float().numpy(), ik_b.float().numpy(), iw, "f32", pos=pos)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ top-k --

def _brute_topk(scores_row, visible, k):
    """Max-sum subset of size min(k, visible); ties -> lexicographically smallest."""
    m = min(k, visible)
    best, best_sum = None, -math.inf
    for comb in itertools.combinations(range(visible), m):  # lexicographic order
        s = sum(scores_row[i] for i in comb)
        if s > best_sum:
            best, best_sum = comb, s
    return list(best) + [-1] * (k - m)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 11))
    k = int(rng.integers(1, 5))
    scores = rng.integers(-2, 3, size=(L, L)).astype(np.float64)  # many exact ties
    scores[0, 0] = -0.0
    pos = np.arange(L)
    for t in range(L):
        scores[t, t + 1:] = -np.inf
    idx, kth = oracle.topk(scores, k, pos)
    for t in range(L):
        want = _brute_topk(scores[t], t + 1, k)
        assert idx[t].tolist() == want, (t, scores[t], idx[t], want)
        m = min(k, t + 1)
        assert kth[t] == min(scores[t, i] for i in want[:m])


def _brute_backbone(scores_row, visible, k, sinks, window):
    """Forced first `sinks` and last `window` visible keys, plus the max-sum size-m subset of the rest
    (ties -> lexicographically smallest), ascending, padded with -1 to k + sinks + window."""
    forced = [s for s in range(visible) if s < sinks or s >= visible - window]
    rest = [s for s in range(visible) if s not in forced]
    m = min(k, len(rest))
    best, best_sum = (), -math.inf
    for comb in itertools.combinations(rest, m):          # lexicographic order of positions
        tot = sum(scores_row[i] for i in comb)
        if tot > best_sum:
            best, best_sum = comb, tot
    row = sorted(forced + list(best))
    return row + [-1] * (k + sinks + window - len(row)), best


@pytest.mark.parametrize("seed", range(8))
def test_backbone_selection_brute_force(seed):
    rng = np.random.default_rng(300 + seed)
    L = int(rng.integers(1, 12))
    k, sinks, window = (int(x) for x in rng.integers(0, 4, size=3))
    k = max(k, 1)
    scores = rng.integers(-2, 3, size=(L, L)).astype(np.float64)  # many exact ties
    pos = np.arange(L)
    for t in range(L):
        scores[t, t + 1:] = -np.inf
    idx, kth = oracle.select_backbone(scores, k, sinks, window, pos)
    assert idx.shape == (L, k + sinks + window)
    for t in range(L):
        want, picks = _brute_backbone(scores[t], t + 1, k, sinks, window)
        assert idx[t].tolist() == want, (t, sinks, window, k, scores[t], idx[t], want)
        if picks:
            assert kth[t] == min(scores[t, i] for i in picks)
        else:
            assert math.isnan(kth[t])


def test_backbone_without_forced_keys_is_topk():
    rng = np.random.default_rng(31)
    sc = rng.standard_normal((40, 60))
    pos = rng.integers(-1, 60, size=40)
    a, ka = oracle.select_backbone(sc, 7, 0, 0, pos)
    b, kb = oracle.topk(sc, 7, pos)
    assert np.array_equal(a, b) and np.array_equal(ka, kb, equal_nan=True)


def test_backbone_forced_keys_do_not_use_the_budget():
    """The window holds the highest scores, yet the k picks all come from outside it."""
    n = 50
    sc = np.tile(np.arange(n, dtype=np.float64), (1, 1))        # score = position: recent keys score highest
    idx, _ = oracle.select_backbone(sc, 5, 2, 10, [n - 1])
    row = [s for s in idx[0].tolist() if s >= 0]
    assert row == [0, 1] + list(range(35, 40)) + list(range(40, 50))


def test_backbone_covering_everything_keeps_the_prefix():
    rng = np.random.default_rng(32)
    sc = rng.standard_normal((6, 30))
    pos = np.array([0, 3, 10, 19, 25, 29])
    idx, _ = oracle.select_backbone(sc, 10, 4, 16, pos)            # k + sinks + window = 30 >= every prefix
    for t, p in enumerate(pos):
        assert idx[t].tolist() == list(range(p + 1)) + [-1] * (30 - p - 1)


def test_topk_all_zero_weights_selects_first_positions():
    rng = np.random.default_rng(8)
    iq, ik, iw = _rand_index_problem(rng, n_q=9, n_k=9)
    sc = oracle.index_scores(iq, ik, np.zeros_like(iw), "f32")
    idx, _ = oracle.topk(sc, 4)
    for t in range(9):
        m = min(4, t + 1)
        assert idx[t].tolist() == list(range(m)) + [-1] * (4 - m)


def test_topk_invariants_and_needles_tiny_config():
    inp = make_inputs(spec("tiny_prefill_f32"), device="cpu", seed=0)
    ov = oracle_view(inp)
    pos = ov["pos"][0]
    sc = oracle.index_scores(ov["iq"][0], ov["ik"][0], ov["iw"][0], "f32", pos=pos)
    idx, kth = oracle.topk(sc, ov["top_k"], pos)
    k = ov["top_k"]
    for t in range(sc.shape[0]):
        m = min(k, t + 1)
        row = idx[t]
        assert np.all(row[m:] == -1)
        sel = row[:m]
        assert len(set(sel.tolist())) == m and np.all(sel >= 0) and np.all(sel <= t)
        assert np.all(np.diff(sel) > 0)
        assert np.min(sc[t, sel]) == kth[t]
        rest = np.setdiff1d(np.arange(t + 1), sel)
        if rest.size:
            assert np.max(sc[t, rest]) <= kth[t]
    pairs = ov["needle_pairs"]
    assert len(pairs) == 16
    hits = sum(int(s in set(idx[t].tolist())) for (_, s, t) in pairs)
    assert hits == len(pairs)  # every planted key is kept by the query it copies


# -------------------------------------------------------------- attention --

def _sdpa64(q, k, v, mask, scale):
    """torch float64 SDPA per head; q [T,H,d], k [S,H,d], v [S,H,dv], mask [T,S] bool."""
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2)
    vt = torch.from_numpy(v).permute(1, 0, 2)
    m = torch.from_numpy(mask)[None].expand(qt.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out.permute(1, 0, 2).numpy()


def test_dense_causal_matches_torch_sdpa():
    rng = np.random.default_rng(9)
    L, H, d = 13, 3, 16
    q = rng.standard_normal((L, H, d)).astype(np.float32)
    k = rng.standard_normal((L, H, d)).astype(np.float32)
    v = rng.standard_normal((L, H, d)).astype(np.float32)
    out, lse = oracle.dense_causal_attn(q, k, v, "f32", 0.25)
    mask = np.tril(np.ones((L, L), dtype=bool))
    ref = _sdpa64(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), mask, 0.25)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    z = 0.25 * np.einsum("thd,shd->ths", q.astype(np.float64), k.astype(np.float64))
    z[:, :, :][np.broadcast_to(~mask[:, None, :], z.shape)] = -np.inf
    np.testing.assert_allclose(lse, np.log(np.sum(np.exp(z), axis=2)), rtol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (6, 1)])
def test_sparse_with_full_k_equals_dense(hq, hkv):
    rng = np.random.default_rng(10 + hq)
    L, d = 12, 32
    q = rng.standard_normal((L, hq, d)).astype(np.float32)
    k = rng.standard_normal((L, hkv, d)).astype(np.float32)
    v = rng.standard_normal((L, hkv, d)).astype(np.float32)
    idx = np.tile(np.arange(L, dtype=np.int32), (L, 1))  # everything; future rows skipped
    o_s, l_s = oracle.sparse_attn(q, k, v, idx, "f32", 0.3)
    o_d, l_d = oracle.dense_causal_attn(q, k, v, "f32", 0.3)
    np.testing.assert_allclose(o_s, o_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l_s, l_d, rtol=1e-13)
    grp = hq // hkv
    ref = _sdpa64(q.astype(np.float64), np.repeat(k, grp, 1).astype(np.float64),
                  np.repeat(v, grp, 1).astype(np.float64), np.tril(np.ones((L, L), bool)), 0.3)
    np.testing.assert_allclose(o_s, ref, rtol=1e-10, atol=1e-12)


def test_sparse_attn_closed_forms():
    rng = np.random.default_rng(11)
    n_k, hq, hkv, d = 20, 8, 2, 16
    q = rng.standard_normal((3, hq, d)).astype(np.float32)
    k = rng.standard_normal((n_k, hkv, d)).astype(np.float32)
    consts = np.array([1.5, -2.25], dtype=np.float32)
    v = np.broadcast_to(consts[None, :, None], (n_k, hkv, d)).copy()
    idx = np.array([[0, 5, 7, -1], [3, -1, -1, -1], [19, 2, 11, 4]], dtype=np.int32)
    pos = np.full(3, n_k - 1)
    out, lse = oracle.sparse_attn(q, k, v, idx, "f32", 0.5, pos)
    for h in range(hq):  # constant value rows -> output equals that constant (head grouping)
        np.testing.assert_allclose(out[:, h, :], consts[h // (hq // hkv)], rtol=1e-14)
    # one selected row: output is that row's value, lse is its logit
    v2 = rng.standard_normal((n_k, hkv, d)).astype(np.float32)
    out1, lse1 = oracle.sparse_attn(q, k, v2, idx, "f32", 0.5, pos)
    for h in range(hq):
        g = h // (hq // hkv)
        np.testing.assert_allclose(out1[1, h], v2[3, g], rtol=1e-14)
        assert lse1[1, h] == pytest.approx(0.5 * float(np.dot(q[1, h].astype(np.float64),
                                                              k[3, g].astype(np.float64))), rel=1e-13)
    # zero query -> uniform weights: mean of the selected rows and lse = ln(m)
    outz, lsez = oracle.sparse_attn(np.zeros_like(q), k, v2, idx, "f32", 0.5, pos)
    for t, sel in enumerate([[0, 5, 7], [3], [19, 2, 11, 4]]):
        for h in range(hq):
            g = h // (hq // hkv)
            np.testing.assert_allclose(outz[t, h], v2[sel, g].astype(np.float64).mean(0), rtol=1e-12)
            assert lsez[t, h] == pytest.approx(math.log(len(sel)), rel=1e-14)


def test_sparse_attn_latent_value_is_key_prefix():
    rng = np.random.default_rng(12)
    L, hq, dqk, dv = 10, 4, 24, 16
    q = rng.standard_normal((L, hq, dqk)).astype(np.float32)
    k = rng.standard_normal((L, 1, dqk)).astype(np.float32)
    idx = np.tile(np.arange(L, dtype=np.int32), (L, 1))
    out, _ = oracle.sparse_attn(q, k, None, idx, "f32", 0.2, latent_dv=dv)
    ref = _sdpa64(q.astype(np.float64), np.repeat(k, hq, 1).astype(np.float64),
                  np.repeat(k[:, :, :dv], hq, 1).astype(np.float64),
                  np.tril(np.ones((L, L), bool)), 0.2)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_sparse_attn_skips_invalid_entries():
    rng = np.random.default_rng(13)
    n_k, h, d = 8, 2, 8
    q = rng.standard_normal((2, h, d)).astype(np.float32)
    k = rng.standard_normal((n_k, h, d)).astype(np.float32)
    v = rng.standard_normal((n_k, h, d)).astype(np.float32)
    pos = np.array([3, 7])
    idx = np.array([[-1, 9, 5, 100], [2, -1, 8, 6]], dtype=np.int32)  # row 0: nothing valid
    out, lse = oracle.sparse_attn(q, k, v, idx, "f32", 0.4, pos)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    ref, ref_lse = oracle.sparse_attn(q[1:], k, v, np.array([[2, 6]], np.int32), "f32", 0.4, pos[1:])
    np.testing.assert_array_equal(out[1], ref[0])
    np.testing.assert_array_equal(lse[1], ref_lse[0])


def test_pipeline_matches_brute_force_subset_attention():
    """Whole path on tiny shapes: brute-force subset, then torch SDPA over it."""
    sp = custom_spec(n_q=9, n_k=9, idx_heads=2, idx_dim=16, top_k=3, q_heads=4, kv_heads=2,
                     d_qk=8, d_v=8)
    inp = make_inputs(sp, device="cpu", seed=3)
    ov = oracle_view(inp)
    res = oracle.dsa_forward(ov)
    iq, ik, iw = ov["iq"][0], ov["ik"][0], ov["iw"][0]
    q, k, v = ov["q"][0], ov["k"][0], ov["v"][0]
    dots = np.einsum("thd,sd->ths", iq.astype(np.float64), ik.astype(np.float64))
    full = np.einsum("th,ths->ts", iw.astype(np.float64), np.maximum(dots, 0.0))
    for t in range(9):
        sel = _brute_topk(full[t], t + 1, 3)
        assert res[(0, t)]["idx"].tolist() == sel
        mask = np.zeros((1, 9), bool)
        mask[0, [s for s in sel if s >= 0]] = True
        ref = _sdpa64(q[t:t + 1].astype(np.float64), np.repeat(k, 2, 1).astype(np.float64),
                      np.repeat(v, 2, 1).astype(np.float64), mask, ov["scale"])
        np.testing.assert_allclose(res[(0, t)]["out"], ref[0], rtol=1e-10, atol=1e-12)


# --- FP8 (E4M3) main KV cache: codes times one fp32 scale per (token, kv head) row ---

def _e4m3_codes(rng, shape):
    """Random finite E4M3 codes (NaN codes 0x7F / 0xFF excluded)."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint16)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)


def _e4m3_dequant_torch(codes, scales):
    """torch's own float8_e4m3fn decoder, times the row scales, in float64."""
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    return (vals * torch.from_numpy(scales.astype(np.float64))[..., None]).numpy()


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4)])
def test_fp8_cache_attention_matches_torch_sdpa(hq, hkv):
    """The FP8 cache path against torch's float8 decoder and float64 SDPA over
    the selected rows (a boolean mask per query)."""
    rng = np.random.default_rng(41 + hq)
    n_q, n_k, d = 4, 30, 16
    q = rng.standard_normal((n_q, hq, d)).astype(np.float32)
    kc, vc = _e4m3_codes(rng, (n_k, hkv, d)), _e4m3_codes(rng, (n_k, hkv, d))
    ks = rng.uniform(0.001, 0.01, (n_k, hkv)).astype(np.float32)
    vs = rng.uniform(0.5, 2.0, (n_k, hkv)).astype(np.float32)
    idx = np.stack([rng.choice(n_k, 9, replace=False) for _ in range(n_q)]).astype(np.int32)
    pos = np.full(n_q, n_k - 1)
    out, lse = oracle.sparse_attn(q, kc, vc, idx, "f32", 0.3, pos, kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    kd, vd = _e4m3_dequant_torch(kc, ks), _e4m3_dequant_torch(vc, vs)
    grp = hq // hkv
    mask = np.zeros((n_q, n_k), dtype=bool)
    for t in range(n_q):
        mask[t, idx[t]] = True
    ref = _sdpa64(q.astype(np.float64), np.repeat(kd, grp, 1), np.repeat(vd, grp, 1), mask, 0.3)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    z = 0.3 * np.einsum("thd,shd->ths", q.astype(np.float64), np.repeat(kd, grp, 1))
    z[np.broadcast_to(~mask[:, None, :], z.shape)] = -np.inf
    np.testing.assert_allclose(lse, np.log(np.sum(np.exp(z - z.max(2, keepdims=True)), 2)) + z.max(2),
                               rtol=1e-12)


def test_fp8_cache_scale_invariants():
    """Scaling every V scale by c scales the output by c; scaling every K
    scale by c equals scaling the softmax scale by c; the dense routine
    agrees with the sparse one on the FP8 cache with every key kept."""
    rng = np.random.default_rng(47)
    n_k, hq, hkv, d = 24, 6, 3, 32
    q = rng.standard_normal((n_k, hq, d)).astype(np.float32)
    kc, vc = _e4m3_codes(rng, (n_k, hkv, d)), _e4m3_codes(rng, (n_k, hkv, d))
    ks = rng.uniform(0.002, 0.02, (n_k, hkv)).astype(np.float32)
    vs = rng.uniform(0.25, 4.0, (n_k, hkv)).astype(np.float32)
    idx = np.tile(np.arange(n_k, dtype=np.int32), (n_k, 1))
    kw = dict(kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    o, l = oracle.sparse_attn(q, kc, vc, idx, "f32", 0.2, None, **kw)
    o2, _ = oracle.sparse_attn(q, kc, vc, idx, "f32", 0.2, None, kv_dtype="e4m3", k_scale=ks, v_scale=vs * 2)
    np.testing.assert_allclose(o2, 2 * o, rtol=1e-12, atol=1e-14)
    o3, l3 = oracle.sparse_attn(q, kc, vc, idx, "f32", 0.1, None, kv_dtype="e4m3", k_scale=ks * 2, v_scale=vs)
    np.testing.assert_allclose(o3, o, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(l3, l, rtol=1e-12)
    od, ld = oracle.dense_causal_attn(q, kc, vc, "f32", 0.2, None, **kw)
    np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, ld, rtol=1e-13)


def test_fp8_latent_value_uses_key_scale():
    """A latent FP8 row: the value is the first dv dequantised entries of the
    key row, with the key row's scale."""
    rng = np.random.default_rng(53)
    n_k, hq, dqk, dv = 16, 4, 48, 32
    q = rng.standard_normal((3, hq, dqk)).astype(np.float32)
    kc = _e4m3_codes(rng, (n_k, 1, dqk))
    ks = rng.uniform(0.01, 0.1, (n_k, 1)).astype(np.float32)
    idx = np.array([[1, 4, 9], [0, 2, -1], [15, 7, 3]], dtype=np.int32)
    out, _ = oracle.sparse_attn(q, kc, None, idx, "f32", 0.25, np.full(3, n_k - 1), latent_dv=dv,
                                kv_dtype="e4m3", k_scale=ks)
    kd = _e4m3_dequant_torch(kc, ks)
    for t, sel in enumerate([[1, 4, 9], [0, 2], [15, 7, 3]]):
        for h in range(hq):
            z = 0.25 * kd[sel, 0, :] @ q[t, h].astype(np.float64)
            p = np.exp(z - z.max()); p /= p.sum()
            np.testing.assert_allclose(out[t, h], p @ kd[sel, 0, :dv], rtol=1e-11, atol=1e-13)


# ---- importance compression of the cache ------------------------------------

def _golden_importance(vals):
    return np.array([-0.0 if v == "-0.0" else float(v) for v in vals], dtype=np.float32)


def test_compress_hand_worked_example():
    with open(os.path.join(GOLDEN, "compress_worked_example.json")) as f:
        g = json.load(f)
    imp = _golden_importance(g["importance"])
    assert np.signbit(imp[5]) and imp[5] == 0.0
    for case in g["cases"]:
        got = oracle.compress_select(imp, case["window"], case["keep_old"])
        assert got.tolist() == case["kept"], case


@pytest.mark.parametrize("seed", range(6))
def test_compress_brute_force_over_subsets(seed):
    # the kept old set is the unique subset of its size that no swap improves:
    # every kept token beats every dropped one (higher importance, or equal
    # importance and a lower position)
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    imp = rng.integers(-2, 3, n).astype(np.float32)
    imp[rng.random(n) < 0.3] = -0.0
    for window in range(0, n + 2):
        n_old = max(0, n - window)
        for keep in range(0, n_old + 2):
            m = min(keep, n_old)
            valid = []
            for sub in itertools.combinations(range(n_old), m):
                kept = set(sub)
                if all(imp[s] > imp[d] or (imp[s] == imp[d] and s < d)
                       for s in kept for d in range(n_old) if d not in kept):
                    valid.append(sorted(sub) + list(range(n_old, n)))
            assert len(valid) == 1
            assert oracle.compress_select(imp, window, keep).tolist() == valid[0]


def test_compress_degenerate_cases():
    imp = np.zeros(1000, dtype=np.float32)
    imp[1::2] = -0.0
    # every token ties: the lowest old positions win
    assert oracle.compress_select(imp, 100, 300).tolist() == list(range(300)) + list(range(900, 1000))
    # a strictly increasing importance keeps the newest old tokens
    inc = np.arange(1000, dtype=np.float32)
    assert oracle.compress_select(inc, 10, 5).tolist() == list(range(985, 1000))
    assert oracle.compress_select(inc, 0, 0).tolist() == []
    assert oracle.compress_select(-inf_row(7), 2, 1).tolist() == [0, 5, 6]


def inf_row(n):
    r = np.full(n, np.inf, dtype=np.float32)
    r[0] = -r[0]
    return r


def test_compress_matches_the_pages_memory_cut():
    # the pages: an 8K window plus importance compression cuts the KV cache by
    # 45-55 % at 1M tokens; keeping half of the older tokens lands inside that
    n = 1 << 20
    imp = np.random.default_rng(0).standard_normal(n).astype(np.float32)
    kept = oracle.compress_select(imp, 8192, (n - 8192) // 2)
    cut = 1.0 - kept.size / n
    assert 0.45 <= cut <= 0.55
    assert np.all(np.diff(kept) > 0) and kept[-8192:].tolist() == list(range(n - 8192, n))
    # every kept old token's importance is at least every dropped one's
    old = np.zeros(n - 8192, dtype=bool)
    old[kept[:-8192]] = True
    assert imp[:n - 8192][old].min() >= imp[:n - 8192][~old].max()
