"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every case draws seeded inputs (dsa_inputs), runs the library on cuda:0 and
compares with the oracle on the same inputs: index scores row by row, top-k
sets under the swap rule, attention over the oracle's own index set, and the
fused entry end to end where the sets agree.  Large workloads are checked on
sampled query rows (first, last and seeded random ones); small ones in full.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import long_context_sparse_relu_amd as dsa
import oracle
from dsa_inputs import custom_spec, kv_args, make_inputs, oracle_view, pack_fp8_kv_records, spec
from parity import check_attn, check_backbone_row, check_scores, check_topk_row

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _problem_kwargs(inp):
    return dict(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=inp["top_k"], q=inp["q"],
                iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"], softmax_scale=inp["scale"],
                sink_tokens=inp.get("sinks", 0), local_window=inp.get("window", 0),
                attn_mode=inp.get("attn_mode", dsa.ATTN_AUTO), **kv_args(inp))


def _problem(inp, row_sel=None):
    """dsa problem for the whole batch, or for query rows `row_sel` (via q_pos)."""
    kw = _problem_kwargs(inp)
    if row_sel is not None:
        sel = torch.as_tensor(row_sel, dtype=torch.long, device=DEV)
        for name in ("iq", "iw", "q", "iq_scale"):
            if kw[name] is not None:
                kw[name] = kw[name].index_select(1, sel).contiguous()
        kw["q_pos"] = inp["pos"].index_select(1, sel).contiguous()
    return dsa.make_problem(**kw)


def _sample_rows(n_q, count, seed):
    if n_q <= count:
        return list(range(n_q))
    rng = np.random.default_rng(seed)
    rows = {0, n_q - 1, n_q // 2}
    while len(rows) < count:
        rows.add(int(rng.integers(0, n_q)))
    return sorted(rows)


def _host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def _log_stats(stats):
    """Append a case's observed errors to the JSON-lines file named by
    DSA_PARITY_LOG, if set (the committed parity summary is made from it)."""
    path = os.environ.get("DSA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(stats) + "\n")


def run_case(inp, seqs, rows, fused="prefill", check_e2e=True, unfused=True):
    """GPU run, then per-row oracle comparison on (seqs x rows).

    Checked per sampled row: the index scores (unfused entry point over the
    whole batch, or with unfused=False over a q_pos sub-problem of the
    sampled rows), the top-k set under the swap rule (fused; also the unfused
    set, which must equal the fused one), the attention over the oracle's own
    set (unfused dsa_sparse_attn on a sub-problem), and the fused out and lse
    against the oracle's attention over the fused call's own set on every
    sampled row (and over the oracle's set on the rows where the two agree).
    """
    prob = _problem(inp)
    idx_f = torch.empty((inp["B"], inp["n_q"], prob.sel_width), dtype=torch.int32, device=DEV)
    fn = dsa.prefill if fused == "prefill" else dsa.decode
    if unfused:
        scores = dsa.index_scores(prob)
        idx = dsa.topk(prob, scores)
    out_f, lse_f, _ = fn(prob, idx_out=idx_f)
    torch.cuda.synchronize()
    if unfused:
        assert torch.equal(idx, idx_f), "fused and unfused selections differ"
    ov = oracle_view(inp, seqs)
    k = inp["top_k"]
    adt = inp["attn_dtype"]
    swaps = 0
    stats = dict(case=inp.get("name"), score_err=0.0, attn={}, e2e_own={}, e2e_oracle_set={}, rows=0,
                 e2e_rows=0)
    for j, b in enumerate(seqs):
        pos = ov["pos"][j][rows].astype(np.int64)
        iqs = None if ov["iq_scale"] is None else ov["iq_scale"][j][rows]
        iks = None if ov["ik_scale"] is None else ov["ik_scale"][j]
        ora_sc = oracle.index_scores(ov["iq"][j][rows], ov["ik"][j], ov["iw"][j][rows],
                                     inp["idx_dtype"], iqs, iks, pos)
        sinks, window = inp.get("sinks", 0), inp.get("window", 0)
        if sinks or window:
            ora_idx, kth = oracle.select_backbone(ora_sc, k, sinks, window, pos)
        else:
            ora_idx, kth = oracle.topk(ora_sc, k, pos)
        # the sampled rows as their own problem (explicit positions)
        sub = _problem({**inp, **{n: inp[n][b:b + 1] for n in
                                  ("iq", "iw", "q", "k", "ik", "pos")},
                        "v": None if inp["v"] is None else inp["v"][b:b + 1],
                        **{n: None if inp.get(n) is None else inp[n][b:b + 1]
                           for n in ("iq_scale", "ik_scale", "k_scale", "v_scale", "k_rec", "v_rec")}},
                       row_sel=rows)
        if unfused:
            g_sc = scores[b][rows].cpu().numpy()
        else:
            g_sc = dsa.index_scores(sub)[0].cpu().numpy()
        g_idx = idx_f[b][rows].cpu().numpy()
        same = []
        for r in range(len(rows)):
            stats["score_err"] = max(stats["score_err"], check_scores(g_sc[r], ora_sc[r], pos[r]))
            if sinks or window:
                n = check_backbone_row(g_idx[r], ora_idx[r], ora_sc[r], kth[r], pos[r], k, sinks, window)
            else:
                n = check_topk_row(g_idx[r], ora_idx[r], ora_sc[r], kth[r], pos[r], k)
            swaps += n
            same.append(n == 0)
        # attention over the oracle's index set, through the sub-problem
        o_idx_dev = torch.from_numpy(ora_idx).to(DEV).reshape(1, len(rows), ora_idx.shape[1]).contiguous()
        g_out, g_lse = dsa.sparse_attn(sub, o_idx_dev)
        torch.cuda.synchronize()
        v = None if ov["v"] is None else ov["v"][j]
        kv = {}
        if inp["kv_dtype"] == "e4m3":
            kv = dict(kv_dtype="e4m3", k_scale=ov["k_scale"][j],
                      v_scale=None if ov["v_scale"] is None else ov["v_scale"][j])
        ora_out, ora_lse = oracle.sparse_attn(ov["q"][j][rows], ov["k"][j], v, ora_idx, adt,
                                              inp["scale"], pos, inp["latent_dv"], **kv)
        check_attn(_host(g_out[0]), _host(g_lse[0]), ora_out, ora_lse, adt, stats["attn"])
        if check_e2e:
            # the fused output against the oracle's attention over the fused
            # call's own selection, on every sampled row
            own_out, own_lse = oracle.sparse_attn(ov["q"][j][rows], ov["k"][j], v, g_idx, adt,
                                                  inp["scale"], pos, inp["latent_dv"], **kv)
            fo = _host(out_f[b][rows])
            fl = _host(lse_f[b][rows])
            check_attn(fo, fl, own_out, own_lse, adt, stats["e2e_own"])
            stats["e2e_rows"] += len(rows)
            keep = np.nonzero(same)[0]
            if keep.size:
                check_attn(fo[keep], fl[keep], ora_out[keep], ora_lse[keep], adt, stats["e2e_oracle_set"])
        stats["rows"] += len(rows)
    stats["swaps"] = swaps
    assert stats["rows"] > 0, "no row was compared"
    assert not check_e2e or stats["e2e_rows"] == stats["rows"], "a fused output went unchecked"
    print(f"[parity] {inp.get('name')}: {stats}", flush=True)
    _log_stats(stats)
    return stats, idx_f, out_f


EDGE_CASES = {
    # ragged key count, several 4096-key chunks, fp32 everything
    "ragged_f32": dict(n_q=37, n_k=9000, idx_heads=4, top_k=100, q_heads=4, kv_heads=2, d_qk=64, d_v=64),
    # k larger than any visible prefix: everything kept, then -1 padding
    "k_exceeds_prefix": dict(n_q=20, n_k=20, idx_heads=3, top_k=64, q_heads=2, kv_heads=2, d_qk=64, d_v=64),
    "k_is_one": dict(n_q=33, n_k=300, idx_heads=16, top_k=1, q_heads=8, kv_heads=1, d_qk=128, d_v=128,
                     attn_dtype="bf16", idx_dtype="bf16"),
    "single_head_indexer": dict(n_q=16, n_k=700, idx_heads=1, top_k=50, q_heads=2, kv_heads=1, d_qk=64, d_v=64),
    "many_heads_generic": dict(B=2, n_q=5, n_k=3000, idx_heads=64, top_k=256, q_heads=16, kv_heads=16,
                               d_qk=128, d_v=128, attn_dtype="bf16"),
    "fp8_odd_heads": dict(B=3, n_q=4, n_k=5000, idx_heads=5, idx_dtype="e4m3", top_k=300, q_heads=24,
                          kv_heads=3, d_qk=128, d_v=128, attn_dtype="bf16"),
    # FP8 prefill rows with fewer than 16 indexer heads (the tiled kernel pads them with zeros)
    "fp8_tiled_odd_heads": dict(n_q=150, n_k=3000, idx_heads=5, idx_dtype="e4m3", top_k=300, q_heads=8,
                                kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16"),
    "fp8_gqa_decode_ragged": dict(B=5, n_q=1, n_k=12345, idx_heads=16, idx_dtype="e4m3", top_k=2048,
                                  q_heads=32, kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16"),
    "latent_small": dict(B=2, n_q=1, n_k=4000, idx_heads=16, idx_dtype="e4m3", top_k=512, q_heads=20,
                         kv_heads=1, d_qk=576, d_v=512, latent=True, attn_dtype="bf16"),
    # long ragged rows: the fused decode takes the sampled top-k (n_k >= 16 k)
    "fp8_sampled_ragged": dict(B=3, n_q=1, n_k=50001, idx_heads=16, idx_dtype="e4m3", top_k=1000,
                               q_heads=8, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16"),
    # prefill long enough for the masked dense tiles (GQA, ragged last query block)
    "masked_prefill_gqa": dict(n_q=300, n_k=300, idx_heads=8, idx_dtype="bf16", top_k=64, q_heads=4,
                               kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16"),
    "masked_prefill_prefix": dict(B=2, n_q=130, n_k=1000, idx_heads=4, idx_dtype="bf16", top_k=200,
                                  q_heads=2, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16"),
    "bf16_generic_d64": dict(n_q=50, n_k=2000, idx_heads=8, top_k=128, q_heads=8, kv_heads=2,
                             d_qk=64, d_v=64, attn_dtype="bf16", idx_dtype="bf16"),
    # FP8 (E4M3) main KV cache with per-(token, kv head) scales
    "fp8kv_gqa_decode_ragged": dict(B=5, n_q=1, n_k=12345, idx_heads=16, idx_dtype="e4m3", top_k=2048,
                                    q_heads=32, kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16",
                                    kv_dtype="e4m3"),
    "fp8kv_prefill_mha": dict(n_q=70, n_k=900, idx_heads=8, idx_dtype="bf16", top_k=100, q_heads=4,
                              kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16", kv_dtype="e4m3"),
    "fp8kv_latent": dict(B=2, n_q=1, n_k=4000, idx_heads=16, idx_dtype="e4m3", top_k=512, q_heads=20,
                         kv_heads=1, d_qk=576, d_v=512, latent=True, attn_dtype="bf16", kv_dtype="e4m3"),
    "fp8kv_generic_d64": dict(n_q=20, n_k=1500, idx_heads=4, top_k=77, q_heads=8, kv_heads=2,
                              d_qk=64, d_v=64, attn_dtype="bf16", idx_dtype="bf16", kv_dtype="e4m3"),
    # backbone: forced first sink keys and last window keys, top-k between them
    "backbone_prefill": dict(n_q=300, n_k=2000, idx_heads=8, idx_dtype="bf16", top_k=100, q_heads=8,
                             kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16", sinks=4, window=64),
    "backbone_decode_fp8": dict(B=4, n_q=1, n_k=50000, idx_heads=16, idx_dtype="e4m3", top_k=512, q_heads=32,
                                kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16", sinks=16, window=2048),
    "backbone_window_covers": dict(n_q=20, n_k=40, idx_heads=3, top_k=4, q_heads=2, kv_heads=2, d_qk=64,
                                   d_v=64, sinks=2, window=30),
    "backbone_sinks_only": dict(n_q=37, n_k=9000, idx_heads=4, top_k=100, q_heads=4, kv_heads=2, d_qk=64,
                                d_v=64, sinks=8),
    "backbone_long_rows": dict(n_q=16, n_k=40000, idx_heads=16, idx_dtype="e4m3", top_k=300, q_heads=8,
                               kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16", sinks=3, window=1000),
    # the sampled decode select over the ranked keys only
    "backbone_sampled_small_rest": dict(B=2, n_q=1, n_k=12000, idx_heads=16, idx_dtype="e4m3", top_k=512,
                                        q_heads=8, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16", sinks=4,
                                        window=11700),
    "backbone_sampled_needles": dict(B=3, n_q=1, n_k=60000, idx_heads=16, idx_dtype="e4m3", top_k=256,
                                     q_heads=8, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16", sinks=2,
                                     window=4096, needles=64),
    "backbone_short_prompt": dict(B=2, n_q=200, n_k=200, idx_heads=8, idx_dtype="bf16", top_k=50, q_heads=4,
                                  kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16", sinks=10, window=150),
}


@pytest.mark.parametrize("name", sorted(EDGE_CASES))
def test_edge_case(name):
    fields = dict(EDGE_CASES[name])
    inp = make_inputs(custom_spec(name=name, **fields), device=DEV, seed=5)
    n_q = fields["n_q"]
    fused = "decode" if n_q == 1 else "prefill"
    run_case(inp, list(range(fields.get("B", 1))), list(range(n_q)), fused=fused)


@pytest.mark.parametrize("n_q,n_k,idt", [(3001, 3001, "e4m3"), (301, 9001, "e4m3"), (2003, 6003, "bf16"),
                                         (700, 5000, "e4m3")])
def test_tiled_indexer_work_splits(n_q, n_k, idt):
    """The tiled indexer's split of (query block, key tile) pairs over workgroups:
    a prefill from scratch (the first query blocks see one key tile, so the
    launch falls back from equal runs to pieces), a prefix (equal runs that
    cross block boundaries) and bf16 blocks of 8 rows; rows on both sides of
    block boundaries are checked, scores (-inf past each row's position),
    selections and attention, fused against unfused."""
    sp = custom_spec(name=f"splits_{n_q}_{n_k}_{idt}", n_q=n_q, n_k=n_k, idx_heads=16, idx_dtype=idt, top_k=256,
                     q_heads=8, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=31)
    tq = 128 if idt == "e4m3" else 8                 # rows per query block of the FP8 / bf16 kernels
    nqb = (n_q + tq - 1) // tq
    edges = [r for blk in (1, 2, nqb // 2, nqb - 1) for r in (blk * tq - 1, blk * tq) if 0 <= r < n_q]
    rows = sorted(set([0, 1, n_q - 1] + edges + list(_sample_rows(n_q, 12, 7))))
    run_case(inp, [0], rows, fused="prefill")


def test_all_zero_weights_pick_lowest_positions():
    """All scores tie at 0: the lower position must win, exactly."""
    sp = custom_spec(name="zero_w", B=2, n_q=3, n_k=10000, idx_heads=16, idx_dtype="e4m3", top_k=2048,
                     q_heads=8, kv_heads=1, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=9)
    inp["iw"].zero_()
    prob = _problem(inp)
    idx = dsa.topk(prob, dsa.index_scores(prob)).cpu().numpy()
    for b in range(2):
        for t in range(3):
            assert idx[b, t].tolist() == list(range(2048))


def test_explicit_positions_and_empty_rows():
    sp = custom_spec(name="qpos", B=2, n_q=6, n_k=3000, idx_heads=16, idx_dtype="e4m3", top_k=700,
                     q_heads=4, kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=11)
    q_pos = torch.tensor([[-1, 0, 5, 699, 700, 2999], [1500, -1, 2, 2998, 100, 2000]],
                         dtype=torch.int32, device=DEV)
    inp["pos"] = q_pos
    prob = dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=700, q=inp["q"],
                            k=inp["k"], v=inp["v"], iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"],
                            q_pos=q_pos)
    scores = dsa.index_scores(prob)
    idx = dsa.topk(prob, scores)
    out, lse = dsa.sparse_attn(prob, idx)
    out_f, lse_f, _ = dsa.prefill(prob)
    torch.cuda.synchronize()
    ov = oracle_view(inp)
    for b in range(2):
        pos = ov["pos"][b].astype(np.int64)
        sc = oracle.index_scores(ov["iq"][b], ov["ik"][b], ov["iw"][b], "e4m3",
                                 ov["iq_scale"][b], ov["ik_scale"][b], pos)
        o_idx, kth = oracle.topk(sc, 700, pos)
        g = idx[b].cpu().numpy()
        for t in range(6):
            if pos[t] < 0:
                assert np.all(g[t] == -1)
                assert torch.all(out[b, t] == 0) and torch.all(torch.isneginf(lse[b, t]))
                assert torch.all(out_f[b, t] == 0) and torch.all(torch.isneginf(lse_f[b, t]))
                continue
            check_scores(scores[b, t].cpu().numpy(), sc[t], pos[t])
            check_topk_row(g[t], o_idx[t], sc[t], kth[t], pos[t], 700)


@pytest.mark.parametrize("idt", ["e4m3", "bf16"])
def test_prefill_indexer_explicit_positions(idt):
    """Query blocks of the tiled prefill indexer with a ragged last block and
    per-row positions: empty rows (negative positions) next to long ones, so
    one block mixes rows that see nothing with rows that see every chunk."""
    n_q, n_k = 45, 5000
    sp = custom_spec(name="qpos_tiled", B=2, n_q=n_q, n_k=n_k, idx_heads=16 if idt == "e4m3" else 8,
                     idx_dtype=idt, top_k=300, q_heads=4, kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=23)
    rng = np.random.default_rng(23)
    qp = rng.integers(0, n_k, size=(2, n_q))
    qp[0, [0, 7, 33, 44]] = [-1, -9, -1, n_k - 1]
    qp[1, [1, 32, 40]] = [-3, 0, n_k - 1]
    q_pos = torch.tensor(qp, dtype=torch.int32, device=DEV)
    prob = dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=300, q=inp["q"],
                            k=inp["k"], v=inp["v"], iq_scale=inp.get("iq_scale"),
                            ik_scale=inp.get("ik_scale"), q_pos=q_pos)
    scores = dsa.index_scores(prob)
    idx = dsa.topk(prob, scores)
    idx_f = torch.empty((2, n_q, 300), dtype=torch.int32, device=DEV)
    dsa.prefill(prob, idx_out=idx_f)
    torch.cuda.synchronize()
    inp["pos"] = q_pos
    ov = oracle_view(inp)
    for b in range(2):
        pos = ov["pos"][b].astype(np.int64)
        sc = oracle.index_scores(ov["iq"][b], ov["ik"][b], ov["iw"][b], idt,
                                 ov["iq_scale"][b] if idt == "e4m3" else None,
                                 ov["ik_scale"][b] if idt == "e4m3" else None, pos)
        o_idx, kth = oracle.topk(sc, 300, pos)
        g, gf = idx[b].cpu().numpy(), idx_f[b].cpu().numpy()
        for t in range(n_q):
            check_scores(scores[b, t].cpu().numpy(), sc[t], pos[t])
            check_topk_row(g[t], o_idx[t], sc[t], kth[t], pos[t], 300)
            check_topk_row(gf[t], o_idx[t], sc[t], kth[t], pos[t], 300)


def test_sampled_topk_positions_and_ties():
    """Fused decode in the sampled regime: per-row positions (empty, short and
    long rows) and an all-zero-weight row, whose ties force the recompute path."""
    sp = custom_spec(name="sampled_qpos", B=6, n_q=1, n_k=20000, idx_heads=16, idx_dtype="e4m3",
                     top_k=256, q_heads=8, kv_heads=1, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=17)
    q_pos = torch.tensor([[-1], [0], [255], [256], [5000], [19999]], dtype=torch.int32, device=DEV)
    inp["iw"][5].zero_()                  # every score of row 5 ties at zero
    inp["pos"] = q_pos
    prob = dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=256, q=inp["q"], k=inp["k"],
                            v=inp["v"], iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"], q_pos=q_pos)
    idx = dsa.topk(prob, dsa.index_scores(prob))
    idx_f = torch.empty_like(idx)
    out_f, lse_f, _ = dsa.decode(prob, idx_out=idx_f)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_f), "sampled and full top-k differ"
    got = idx_f.cpu().numpy()
    assert np.all(got[0, 0] == -1)
    assert got[1, 0].tolist() == [0] + [-1] * 255
    assert got[2, 0].tolist() == list(range(256))
    assert got[5, 0].tolist() == list(range(256))        # ties resolve to the lowest positions
    ov = oracle_view(inp)
    for b in (3, 4):
        pos = ov["pos"][b].astype(np.int64)
        sc = oracle.index_scores(ov["iq"][b], ov["ik"][b], ov["iw"][b], "e4m3",
                                 ov["iq_scale"][b], ov["ik_scale"][b], pos)
        o_idx, kth = oracle.topk(sc, 256, pos)
        check_topk_row(got[b, 0], o_idx[0], sc[0], kth[0], pos[0], 256)
    assert torch.all(out_f[0, 0] == 0) and torch.all(torch.isneginf(lse_f[0, 0]))


def test_decode_is_deterministic():
    sp = custom_spec(name="det", B=8, n_q=1, n_k=50000, idx_heads=16, idx_dtype="e4m3", top_k=2048,
                     q_heads=32, kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=13)
    prob = _problem(inp)
    a = dsa.decode(prob, idx_out=torch.empty((8, 1, 2048), dtype=torch.int32, device=DEV))
    b = dsa.decode(prob, idx_out=torch.empty((8, 1, 2048), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(a[2], b[2])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("n_k", [20000, 6000])
@pytest.mark.parametrize("sinks,window", [(0, 0), (3, 500)])
def test_topk_long_rows_many_per_workgroup(sinks, window, n_k):
    """dsa_topk over LDS-resident rows with explicit positions: rows of up to
    20000 keys (over 16K: one row fills most of a compute unit's LDS, so each
    workgroup selects several rows in turn and loads the next while selecting
    the current) and of up to 6000 (the 512-thread select, three rows per
    compute unit).  700 rows, some short enough to keep every key, over
    seeded fp32 scores quantised to 2^-10 so exact ties are common.  The kept
    sets must equal the oracle's exactly (the same scores on both sides; ties
    to the lower position), with and without a backbone."""
    n_q, k = 700, 1000
    sp = custom_spec(name="long_rows", n_q=n_q, n_k=n_k, idx_heads=4, idx_dtype="bf16", top_k=k,
                     q_heads=2, kv_heads=1, d_qk=64, d_v=64, attn_dtype="bf16", sinks=sinks, window=window)
    inp = make_inputs(sp, device=DEV, seed=41)
    g = torch.Generator().manual_seed(41)
    pos = torch.randint(n_k // 2, n_k, (1, n_q), generator=g, dtype=torch.int32)
    pos[0, :40] = torch.randint(0, k + sinks + window, (40,), generator=g, dtype=torch.int32)
    pos[0, -1] = n_k - 1
    scores = torch.round(torch.randn((1, n_q, n_k), generator=g) * 1024.0) / 1024.0
    prob = dsa.make_problem(**_problem_kwargs(inp), q_pos=pos.to(DEV))
    idx = dsa.topk(prob, scores.to(DEV))
    torch.cuda.synchronize()
    sc = scores[0].double().numpy()
    p_np = pos[0].numpy().astype(np.int64)
    if sinks or window:
        o_idx, _ = oracle.select_backbone(sc, k, sinks, window, p_np)
    else:
        o_idx, _ = oracle.topk(sc, k, p_np)
    g_idx = idx[0].cpu().numpy()
    bad = [r for r in range(n_q) if not np.array_equal(g_idx[r], o_idx[r])]
    assert not bad, f"rows {bad[:5]} differ (of {len(bad)})"


@pytest.mark.parametrize("k,window", [(2048, 0), (8192, 0), (2048, 12000)])
def test_topk_sampled_bracket_rows(k, window):
    """dsa_topk over rows of 16K-32K keys, the register-resident select that
    brackets the k-th score from a sample of every eighth key.  Rows cycle
    through: Gaussian scores; rows barely longer than k (the bracket's lower
    end leaves the sample); a few planted needles far above the rest; scores
    rounded to 2^-6 (long runs of exact ties inside the bracket); and 3k/4
    distinct keys above 1000 keys tied exactly at the k-th score, everything
    else far below (the tied block fills one second-level bin, too many to
    rank by comparison).  With a local window most keys are also forced to
    -inf.  Every row must equal the oracle's selection exactly (ties to the
    lower position)."""
    n_q, n_k = 250, 32768
    sp = custom_spec(name="bracket", n_q=n_q, n_k=n_k, idx_heads=4, idx_dtype="bf16", top_k=k,
                     q_heads=2, kv_heads=1, d_qk=64, d_v=64, attn_dtype="bf16", window=window)
    inp = make_inputs(sp, device=DEV, seed=53)
    g = torch.Generator().manual_seed(53)
    pos = torch.randint(16384, n_k, (1, n_q), generator=g, dtype=torch.int32)
    kind = torch.arange(n_q) % 5
    short = (kind == 1)
    pos[0, short] = torch.clamp(k + window + torch.randint(1, 200, (int(short.sum()),), generator=g,
                                                             dtype=torch.int32), max=n_k - 1)
    pos[0, -1] = n_k - 1
    sc = torch.randn((n_q, n_k), generator=g)
    nd = torch.randint(0, n_k, (n_q, 8), generator=g)
    needles = (kind == 2).unsqueeze(1).expand(n_q, 8)
    sc[torch.arange(n_q).unsqueeze(1).expand(n_q, 8)[needles], nd[needles]] = 50.0
    sc[kind == 3] = torch.round(sc[kind == 3] * 64.0) / 64.0
    n_above, n_tie = 3 * k // 4, 1000
    for r in torch.nonzero(kind == 4).flatten().tolist():
        ranked_end = int(pos[0, r]) + 1 - window          # keys past it are the forced window
        sel = torch.randperm(ranked_end, generator=g)[:n_above + n_tie]
        sc[r] = torch.randn(n_k, generator=g) - 6.0
        sc[r, sel[:n_above]] = 1.5 + 0.5 * torch.rand(n_above, generator=g)
        sc[r, sel[n_above:]] = 1.0
    scores = sc.unsqueeze(0).float()
    prob = dsa.make_problem(**_problem_kwargs(inp), q_pos=pos.to(DEV))
    idx = dsa.topk(prob, scores.to(DEV))
    torch.cuda.synchronize()
    s_np = sc.double().numpy()
    p_np = pos[0].numpy().astype(np.int64)
    if window:
        o_idx, _ = oracle.select_backbone(s_np, k, 0, window, p_np)
    else:
        o_idx, _ = oracle.topk(s_np, k, p_np)
    g_idx = idx[0].cpu().numpy()
    bad = [r for r in range(n_q) if not np.array_equal(g_idx[r], o_idx[r])]
    assert not bad, f"rows {bad[:5]} (kinds {[int(kind[r]) for r in bad[:5]]}) differ (of {len(bad)})"


@pytest.mark.parametrize("n_k", [12000, 24000])
def test_topk_lds_rows_with_skewed_scores(n_k):
    """dsa_topk over rows selected in LDS (12000 keys: one row per workgroup;
    24000: the persistent form), each row exact against the oracle.  The
    select bins scores linearly over each row's finite range, so the rows
    cycle through distributions that stress that: Gaussian; one huge outlier
    (every other key in the lowest bin: the order-key radix select takes
    over); a heavy tail; two values with ties across the threshold; and
    -inf scores mixed in."""
    n_q, k = 300, 1000
    sp = custom_spec(name="lds_skew", n_q=n_q, n_k=n_k, idx_heads=4, idx_dtype="bf16", top_k=k,
                     q_heads=2, kv_heads=1, d_qk=64, d_v=64, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=47)
    g = torch.Generator().manual_seed(47)
    pos = torch.randint(n_k // 2, n_k, (1, n_q), generator=g, dtype=torch.int32)
    pos[0, -1] = n_k - 1
    sc = torch.randn((n_q, n_k), generator=g)
    kind = torch.arange(n_q) % 5
    sc[kind == 1, 7] = 1e30
    sc[kind == 2] = torch.exp(3.0 * sc[kind == 2])
    two = torch.where(torch.rand((n_q, n_k), generator=g) < 0.05, 1.0, 0.5)
    sc[kind == 3] = two[kind == 3]
    ninf = torch.rand((n_q, n_k), generator=g) < 0.3
    sc[(kind == 4).unsqueeze(1) & ninf] = -float("inf")
    scores = sc.unsqueeze(0).float()
    prob = dsa.make_problem(**_problem_kwargs(inp), q_pos=pos.to(DEV))
    idx = dsa.topk(prob, scores.to(DEV))
    torch.cuda.synchronize()
    o_idx, _ = oracle.topk(scores[0].double().numpy(), k, pos[0].numpy().astype(np.int64))
    g_idx = idx[0].cpu().numpy()
    bad = [r for r in range(n_q) if not np.array_equal(g_idx[r], o_idx[r])]
    assert not bad, f"rows {bad[:5]} differ (of {len(bad)})"


@pytest.mark.parametrize("case", ["all_tied", "sample_overstates"])
def test_topk_candidate_lists_fall_back_to_the_whole_row(case):
    """dsa_topk over 300 rows of 20000 keys selects through sampled candidate
    lists.  Two rows patterns defeat the sample, and the row must then be
    selected again from its scores: every score equal (every key is a
    candidate, far more than the list holds; the lowest positions win), and
    a row whose sampled runs of 16 keys score 1.0 where only 400 keys do (the
    list ends shorter than k).  The kept sets must equal the oracle's exactly."""
    n_q, n_k, k = 300, 20000, 1000
    sp = custom_spec(name="cand_fallback", n_q=n_q, n_k=n_k, idx_heads=4, idx_dtype="bf16", top_k=k,
                     q_heads=2, kv_heads=1, d_qk=64, d_v=64, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=43)
    pos = torch.full((1, n_q), n_k - 1, dtype=torch.int32)
    if case == "all_tied":
        scores = torch.full((1, n_q, n_k), 0.25)
    else:
        # the sampled keys: runs of 16 from multiples of n_k // 256; 25 runs score 1.0
        scores = torch.full((1, n_q, n_k), 0.5)
        gap = n_k // 256
        for j in range(25):
            scores[0, :, 3 * j * gap:3 * j * gap + 16] = 1.0
    prob = dsa.make_problem(**_problem_kwargs(inp), q_pos=pos.to(DEV))
    idx = dsa.topk(prob, scores.to(DEV))
    torch.cuda.synchronize()
    o_idx, _ = oracle.topk(scores[0].double().numpy(), k, pos[0].numpy().astype(np.int64))
    g_idx = idx[0].cpu().numpy()
    bad = [r for r in range(n_q) if not np.array_equal(g_idx[r], o_idx[r])]
    assert not bad, f"rows {bad[:5]} differ (of {len(bad)})"


def test_workspace_too_small_is_rejected():
    sp = custom_spec(name="ws", B=1, n_q=1, n_k=5000, idx_heads=16, idx_dtype="e4m3", top_k=64,
                     q_heads=4, kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=1)
    prob = _problem(inp)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(dsa.DSAError) as ei:
        dsa.decode(prob, workspace=small)
    assert ei.value.status == dsa.E_WORKSPACE


@pytest.mark.parametrize("n_k,fused", [(40000, "decode"), (9000, "unfused")])
def test_massive_exact_ties_resolve_to_lowest_positions(n_k, fused):
    """5000 key rows are byte copies of the query's strongest indexer head, so
    their scores are bit-identical and lead the row: the k kept positions
    must be exactly 0..k-1 of the copies.  Selecting them takes every radix
    digit down to the last position bits (the long decode rows go through
    the sampled candidate path, the 9000-key rows through the LDS row path)."""
    k = 512
    sp = custom_spec(name="ties", B=2, n_q=1, n_k=n_k, idx_heads=16, idx_dtype="e4m3", top_k=k,
                     q_heads=8, kv_heads=1, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=29)
    for b in range(2):
        h = int(torch.argmax(inp["iw"][b, 0]).item())
        inp["ik"][b, :5000] = inp["iq"][b, 0, h].unsqueeze(0)
        inp["ik_scale"][b, :5000] = inp["iq_scale"][b, 0]
    prob = _problem(inp)
    if fused == "decode":
        idx = torch.empty((2, 1, k), dtype=torch.int32, device=DEV)
        dsa.decode(prob, idx_out=idx)
    else:
        idx = dsa.topk(prob, dsa.index_scores(prob))
    torch.cuda.synchronize()
    ov = oracle_view(inp)
    for b in range(2):
        sc = oracle.index_scores(ov["iq"][b], ov["ik"][b], ov["iw"][b], "e4m3", ov["iq_scale"][b],
                                 ov["ik_scale"][b], None)
        o_idx, _ = oracle.topk(sc, k, None)
        assert o_idx[0].tolist() == list(range(k)), "the copies must lead the row"
        assert idx[b, 0].cpu().tolist() == list(range(k))


def test_phase_timer_records_each_phase():
    """The opt-in phase timer: a sampled decode runs all four phases, the
    timed call's results equal an untimed call's, and switching it off stops
    the recording."""
    sp = custom_spec(name="timer", B=4, n_q=1, n_k=40000, idx_heads=16, idx_dtype="e4m3", top_k=512,
                     q_heads=8, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=3)
    prob = _problem(inp)
    i0 = torch.empty((4, 1, 512), dtype=torch.int32, device=DEV)
    i1 = torch.empty_like(i0)
    o0, l0, _ = dsa.decode(prob, idx_out=i0)
    dsa.phase_timing(True)
    try:
        o1, l1, _ = dsa.decode(prob, idx_out=i1)
        t = dsa.phase_times()
    finally:
        dsa.phase_timing(False)
    assert set(t) == set(dsa.PHASES)
    assert all(v > 0 for v in t.values()), t
    assert torch.equal(i0, i1) and torch.equal(o0, o1) and torch.equal(l0, l1)
    with pytest.raises(dsa.DSAError):
        dsa.phase_times()


def test_tiny_prefill_f32_full():
    inp = make_inputs(spec("tiny_prefill_f32"), device=DEV, seed=0)
    stats, idx, _ = run_case(inp, [0], list(range(512)))
    assert stats["swaps"] == 0
    got = idx[0].cpu().numpy()
    hits = sum(int(s in set(got[t].tolist())) for (_, s, t) in inp["needle_pairs"])
    print(f"[parity] tiny_prefill_f32 needle recall {hits}/{len(inp['needle_pairs'])}")


def test_prefill_bf16_8k_sampled():
    inp = make_inputs(spec("prefill_bf16_8k"), device=DEV, seed=0)
    run_case(inp, [0], _sample_rows(8192, 24, 1))


def test_prefill_fp8_32k_sampled():
    inp = make_inputs(spec("prefill_fp8_32k"), device=DEV, seed=0)
    run_case(inp, [0], _sample_rows(32768, 12, 2))


def test_prefill_fp8_128k_sampled():
    """DSA prefill at 128K context with k = 2048 (about 1.6% of the longest
    prefix), in the launch configuration the benchmark times: the fused call
    over the whole sequence.  Its score blocks hold 512 rows; the first 2048
    rows keep every visible key (selection fill), rows up to 32K keys take the
    LDS row select and longer rows the four-kernel radix select; the
    attention is the masked walk over up to 2048 key tiles with a 2 GiB
    selection bitmap.  Sampled rows: first and last, both sides of score-block
    edges and of the 2048- and 32K-key boundaries, and seeded random rows.
    The unfused scores of those rows come from a q_pos sub-problem (the full
    score matrix would be 64 GiB)."""
    inp = make_inputs(spec("prefill_fp8_128k"), device=DEV, seed=0)
    n = 131072
    rows = sorted(set([0, 1, 2047, 2048, 2049, 2559, 2560, 32767, 32768, 33279, 33280, 65535, 65536,
                       n - 513, n - 512, n - 2, n - 1] + _sample_rows(n, 6, 4)))
    run_case(inp, [0], rows, fused="prefill", unfused=False)


def test_decode_128k_sampled():
    """The benchmarked workload, in the launch configuration the benchmark times."""
    inp = make_inputs(spec("decode_128k"), device=DEV, seed=0)
    run_case(inp, [0, 17, 63], [0], fused="decode")


def test_decode_128k_fp8kv_sampled():
    """The 128K decode workload over an E4M3 main KV cache."""
    inp = make_inputs(spec("decode_128k_fp8kv"), device=DEV, seed=0)
    run_case(inp, [0, 31, 63], [0], fused="decode")


def test_fp8kv_scales_act_per_row():
    """Scaling one kept row's value scale changes out (as the oracle says) and never lse."""
    sp = custom_spec(name="fp8kv_scale", B=1, n_q=1, n_k=3000, idx_heads=16, idx_dtype="e4m3",
                     top_k=256, q_heads=16, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16",
                     kv_dtype="e4m3")
    inp = make_inputs(sp, device=DEV, seed=3)
    prob = _problem(inp)
    idx = dsa.topk(prob, dsa.index_scores(prob))
    out0, lse0 = dsa.sparse_attn(prob, idx)
    torch.cuda.synchronize()
    s = int(idx[0, 0, 5])
    inp2 = dict(inp)
    inp2["v_scale"] = inp["v_scale"].clone()
    inp2["v_scale"][0, s] *= 64.0
    inp2["v_rec"] = pack_fp8_kv_records(inp2["v"], inp2["v_scale"])
    out1, lse1 = dsa.sparse_attn(_problem(inp2), idx)
    torch.cuda.synchronize()
    assert torch.equal(lse0, lse1), "the value scale must not touch the softmax"
    ov = oracle_view(inp2, [0])
    pos = ov["pos"][0].astype(np.int64)
    ora_out, ora_lse = oracle.sparse_attn(ov["q"][0], ov["k"][0], ov["v"][0], idx[0].cpu().numpy(), "bf16",
                                          inp["scale"], pos, None, kv_dtype="e4m3",
                                          k_scale=ov["k_scale"][0], v_scale=ov["v_scale"][0])
    check_attn(_host(out1[0]), _host(lse1[0]), ora_out, ora_lse, "bf16")
    assert (out1.float() - out0.float()).abs().max().item() > 1e-3


def test_decode_1m_sampled():
    inp = make_inputs(spec("decode_1m"), device=DEV, seed=0)
    stats, idx, _ = run_case(inp, [0, 7], [0], fused="decode")
    got = idx.cpu().numpy()
    hits = sum(int(s in set(got[b, 0].tolist())) for (b, s, t) in inp["needle_pairs"])
    assert hits >= 0.95 * len(inp["needle_pairs"]), f"needle recall {hits}/{len(inp['needle_pairs'])}"


@pytest.mark.parametrize("workload,zero_rows", [("decode_128k", [5, 17]), ("decode_1m", [3])])
def test_decode_rows_recomputed_in_full_at_full_size(workload, zero_rows):
    """Rows whose indexer head weights are all zero score 0 at every key: every
    key is a candidate, the row's list overflows and the finish recomputes the
    whole row over several workgroups, then selects the lowest k positions.
    The benchmarked shapes, with the other rows on the candidate path beside
    them; fused, unfused and oracle must agree."""
    inp = make_inputs(spec(workload), device=DEV, seed=0)
    inp["name"] = f"{workload}_zero_weight_rows"
    for b in zero_rows:
        inp["iw"][b].zero_()
    stats, idx, _ = run_case(inp, zero_rows + [0], [0], fused="decode")
    k = inp["top_k"]
    for b in zero_rows:
        assert idx[b, 0].cpu().tolist() == list(range(k))


# --- masked MHA mode, dense causal attention and the dense fallback --------------------------

def _attn_problem(inp, **kw):
    return dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=inp["top_k"], q=inp["q"],
                            k=inp["k"], v=inp["v"], softmax_scale=inp["scale"], **kw)


@pytest.mark.parametrize("B,n_q,n_k,Hq,Hkv", [(2, 150, 400, 8, 2), (1, 300, 300, 4, 4), (3, 1, 2000, 8, 1)])
def test_dense_attn_matches_oracle(B, n_q, n_k, Hq, Hkv):
    """Causal attention over every visible key (ragged query blocks, a cached prefix, decode)."""
    sp = custom_spec(name="dense", B=B, n_q=n_q, n_k=n_k, idx_heads=4, idx_dtype="bf16", top_k=8,
                     q_heads=Hq, kv_heads=Hkv, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=11)
    out, lse = dsa.dense_attn(_attn_problem(inp))
    torch.cuda.synchronize()
    ov = oracle_view(inp)
    for b in range(B):
        o_out, o_lse = oracle.dense_causal_attn(ov["q"][b], ov["k"][b], ov["v"][b], "bf16", inp["scale"],
                                                ov["pos"][b].astype(np.int64))
        check_attn(_host(out[b]), _host(lse[b]), o_out, o_lse, "bf16")


def test_dense_attn_explicit_positions():
    """q_pos rows, including one that sees nothing (out = 0, lse = -inf)."""
    sp = custom_spec(name="dense_pos", B=1, n_q=70, n_k=500, idx_heads=4, idx_dtype="bf16", top_k=8,
                     q_heads=4, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=12)
    g = torch.Generator().manual_seed(3)
    pos = torch.randint(-1, 500, (1, 70), generator=g, dtype=torch.int32)
    pos[0, 5] = -1
    out, lse = dsa.dense_attn(_attn_problem(inp, q_pos=pos.to(DEV)))
    torch.cuda.synchronize()
    ov = oracle_view(inp)
    o_out, o_lse = oracle.dense_causal_attn(ov["q"][0], ov["k"][0], ov["v"][0], "bf16", inp["scale"],
                                            pos[0].numpy().astype(np.int64))
    check_attn(_host(out[0]), _host(lse[0]), o_out, o_lse, "bf16")
    assert torch.isneginf(lse[0, 5]).all() and (out[0, 5] == 0).all()


@pytest.mark.parametrize("n_q,n_k,k", [(200, 700, 100), (64, 3000, 512), (130, 130, 40), (32, 20000, 1024)])
def test_attention_modes_agree(n_q, n_k, k):
    """AUTO, GATHER and MASKED compute the same attention over the same selection."""
    sp = custom_spec(name="modes", B=2, n_q=n_q, n_k=n_k, idx_heads=8, idx_dtype="bf16", top_k=k,
                     q_heads=8, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=13)
    idxs, outs = [], []
    for mode in (dsa.ATTN_AUTO, dsa.ATTN_GATHER, dsa.ATTN_MASKED):
        prob = _attn_problem(inp, attn_mode=mode)
        idx = torch.empty((2, n_q, k), dtype=torch.int32, device=DEV)
        out, lse, _ = dsa.prefill(prob, idx_out=idx)
        torch.cuda.synchronize()
        idxs.append(idx)
        outs.append((out, lse))
    assert torch.equal(idxs[0], idxs[1]) and torch.equal(idxs[0], idxs[2])
    ov = oracle_view(inp)
    for b in range(2):
        pos = ov["pos"][b].astype(np.int64)
        o_out, o_lse = oracle.sparse_attn(ov["q"][b], ov["k"][b], ov["v"][b], idxs[0][b].cpu().numpy(), "bf16",
                                          inp["scale"], pos)
        for out, lse in outs:
            check_attn(_host(out[b]), _host(lse[b]), o_out, o_lse, "bf16")


@pytest.mark.parametrize("mode", ["dense", "masked"])
def test_masked_tiles_ignore_memory_past_the_keys(mode):
    """K and V end inside larger buffers whose tail holds bf16 NaN, and the
    last key tile is partial (1000 keys = 15 tiles + 40).  The masked kernels
    read whole 64-key tiles; rows past n_k must read as zeros (never the
    memory that follows), so the output stays finite and matches the oracle,
    through dsa_dense_attn and through the fused prefill in MASKED mode."""
    n_q, n_k, Hq, Hkv, k = 100, 1000, 4, 2, 200
    sp = custom_spec(name="nan_tail", B=1, n_q=n_q, n_k=n_k, idx_heads=4, idx_dtype="bf16", top_k=k,
                     q_heads=Hq, kv_heads=Hkv, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=21)
    for name in ("k", "v"):
        t = inp[name]
        big = torch.full((t.numel() + 64 * Hkv * 128 * 2,), float("nan"), dtype=torch.bfloat16, device=DEV)
        big[: t.numel()] = t.reshape(-1)
        inp[name] = big[: t.numel()].view(t.shape)
    ov = oracle_view(inp)
    pos = ov["pos"][0].astype(np.int64)
    if mode == "dense":
        out, lse = dsa.dense_attn(_attn_problem(inp))
        torch.cuda.synchronize()
        o_out, o_lse = oracle.dense_causal_attn(ov["q"][0], ov["k"][0], ov["v"][0], "bf16", inp["scale"], pos)
    else:
        idx = torch.empty((1, n_q, k), dtype=torch.int32, device=DEV)
        out, lse, _ = dsa.prefill(_problem({**inp, "attn_mode": dsa.ATTN_MASKED}), idx_out=idx)
        torch.cuda.synchronize()
        o_out, o_lse = oracle.sparse_attn(ov["q"][0], ov["k"][0], ov["v"][0], idx[0].cpu().numpy(), "bf16",
                                          inp["scale"], pos)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    check_attn(_host(out[0]), _host(lse[0]), o_out, o_lse, "bf16")


def test_short_prompt_is_dense_attention():
    """top_k >= every prefix: the selection is 0..t exactly and the output is dense attention."""
    sp = custom_spec(name="short", B=2, n_q=500, n_k=500, idx_heads=16, idx_dtype="e4m3", top_k=512,
                     q_heads=8, kv_heads=2, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=14)
    prob = _problem(inp)
    idx = torch.empty((2, 500, 512), dtype=torch.int32, device=DEV)
    out, lse, _ = dsa.prefill(prob, idx_out=idx)
    d_out, d_lse = dsa.dense_attn(prob)
    torch.cuda.synchronize()
    j = torch.arange(512, device=DEV, dtype=torch.int32)
    t = torch.arange(500, device=DEV, dtype=torch.int32)[:, None]
    want = torch.where(j[None, :] <= t, j[None, :], torch.full_like(j[None, :], -1))
    assert torch.equal(idx, want.expand(2, 500, 512))
    assert torch.equal(out, d_out) and torch.equal(lse, d_lse)
    ov = oracle_view(inp)
    o_out, o_lse = oracle.dense_causal_attn(ov["q"][1], ov["k"][1], ov["v"][1], "bf16", inp["scale"],
                                            ov["pos"][1].astype(np.int64))
    check_attn(_host(out[1]), _host(lse[1]), o_out, o_lse, "bf16")


def test_prefill_first_block_takes_dense_fallback():
    """16K prefill, k = 4096: the first row block (rows t < 4096) skips the indexer and top-k."""
    sp = custom_spec(name="fallback16k", B=1, n_q=16384, n_k=16384, idx_heads=16, idx_dtype="e4m3",
                     top_k=4096, q_heads=4, kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16")
    inp = make_inputs(sp, device=DEV, seed=15)
    rows = [0, 1, 1000, 4095, 4096, 4097, 9000, 16383]
    _, idx, _ = run_case(inp, [0], rows, fused="prefill")
    got = idx[0, 4095].cpu()
    assert torch.equal(got, torch.arange(4096, dtype=torch.int32))
