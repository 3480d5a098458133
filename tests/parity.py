"""Parity rules between the HIP path and the fp64 oracle (test helpers).

Rules (one per output kind):
  * index scores: |gpu - oracle| <= SCORE_ATOL + SCORE_RTOL*|oracle| where the
    oracle is finite, and -inf exactly where the key is in the future;
  * top-k sets: with G the GPU's kept set and O the oracle's, |G| = |O| = m,
    G holds distinct visible positions in ascending order padded with -1, and
    every oracle position the GPU dropped scores within tau = 1e-3*|S_k| of
    every position it kept instead (S_k the oracle's m-th score), so a swap is
    only allowed between keys the fp64 scores cannot tell apart at that
    precision;
  * attention outputs: max-abs error <= 1e-4 for the fp32 path and <= 2e-2 for
    the bf16 / FP8 paths, compared against the oracle over the same index set.
"""
from __future__ import annotations

import numpy as np

SCORE_ATOL = 1e-4
SCORE_RTOL = 1e-4
TAU_REL = 1e-3
OUT_TOL = {"f32": 1e-4, "bf16": 2e-2}
LSE_TOL = {"f32": 1e-4, "bf16": 2e-3}


def check_scores(gpu_row, ora_row, pos):
    gpu_row = np.asarray(gpu_row, dtype=np.float64)
    vis = max(0, min(pos + 1, len(ora_row)))
    assert np.all(np.isneginf(gpu_row[vis:])), "future keys must score -inf"
    a, b = gpu_row[:vis], ora_row[:vis]
    err = np.abs(a - b)
    bad = err > SCORE_ATOL + SCORE_RTOL * np.abs(b)
    assert not bad.any(), f"score mismatch at {np.nonzero(bad)[0][:8]}: gpu {a[bad][:4]} oracle {b[bad][:4]}"
    return float(err.max()) if vis else 0.0


def check_topk_row(gpu_idx, ora_idx, ora_scores, kth, pos, k):
    """Returns the number of allowed swaps in this row (0 when identical)."""
    gpu_idx = np.asarray(gpu_idx)
    vis = max(0, min(pos + 1, len(ora_scores)))
    m = min(k, vis)
    assert np.all(gpu_idx[m:] == -1), f"padding: {gpu_idx[m:][:8]}"
    g = gpu_idx[:m]
    assert np.all(g >= 0) and np.all(g <= pos), "kept positions must be visible"
    assert np.all(np.diff(g) > 0), "kept positions must be distinct and ascending"
    G, O = set(g.tolist()), set(int(x) for x in ora_idx[:m])
    if G == O:
        return 0
    only_o = np.array(sorted(O - G))
    only_g = np.array(sorted(G - O))
    assert len(only_o) == len(only_g)
    tau = TAU_REL * abs(kth)
    gap = ora_scores[only_o].max() - ora_scores[only_g].min()
    assert gap < tau, (f"top-k swap beyond tolerance: dropped {only_o[:4]} ({ora_scores[only_o][:4]}) "
                       f"kept {only_g[:4]} ({ora_scores[only_g][:4]}), tau {tau}")
    return len(only_o)


def attn_errors(gpu_out, gpu_lse, ora_out, ora_lse):
    """Observed errors of an attention result: out max-abs, out max-abs relative
    to max|oracle out| (a diagnostic), and lse max-abs over non-empty rows."""
    gpu_out = np.asarray(gpu_out, dtype=np.float64)
    err = float(np.abs(gpu_out - ora_out).max()) if gpu_out.size else 0.0
    scale = float(np.abs(ora_out).max()) if gpu_out.size else 0.0
    gl = np.asarray(gpu_lse, dtype=np.float64)
    fin = np.isfinite(ora_lse)
    lerr = float(np.abs(gl[fin] - ora_lse[fin]).max()) if fin.any() else 0.0
    return {"out": err, "out_rel": err / scale if scale > 0 else 0.0, "lse": lerr}


def check_attn(gpu_out, gpu_lse, ora_out, ora_lse, dtype, errors=None):
    """Asserts the attention rule; returns the out max-abs error.  With
    `errors` (a dict) the observed errors are also folded into it (max)."""
    e = attn_errors(gpu_out, gpu_lse, ora_out, ora_lse)
    assert e["out"] <= OUT_TOL[dtype], f"attention max-abs error {e['out']} > {OUT_TOL[dtype]}"
    gl = np.asarray(gpu_lse, dtype=np.float64)
    fin = np.isfinite(ora_lse)
    assert np.array_equal(np.isneginf(gl), ~fin), "empty rows must give lse = -inf"
    assert e["lse"] <= LSE_TOL[dtype], f"lse error {e['lse']}"
    if errors is not None:
        for key, v in e.items():
            errors[key] = max(errors.get(key, 0.0), v)
    return e["out"]


def check_backbone_row(gpu_idx, ora_idx, ora_scores, kth, pos, k, sinks, window):
    """A backbone selection row: its forced keys exactly, then the top-k rule on the picks.

    The forced keys are the first `sinks` and last `window` visible ones; the
    picks are the kept keys between them, m = min(k, their count) of them,
    compared with the oracle's under the same swap tolerance as check_topk_row.
    Returns the number of allowed swaps.
    """
    gpu_idx = np.asarray(gpu_idx)
    vis = max(0, min(pos + 1, len(ora_scores)))
    forced = {s for s in range(vis) if s < sinks or s >= vis - window}
    n_rest = vis - len(forced)
    m = min(k, n_rest)
    total = len(forced) + m
    assert np.all(gpu_idx[total:] == -1), f"padding: {gpu_idx[total:][:8]}"
    g = gpu_idx[:total]
    assert np.all(g >= 0) and np.all(g <= pos), "kept positions must be visible"
    assert np.all(np.diff(g) > 0), "kept positions must be distinct and ascending"
    G = set(g.tolist())
    assert forced <= G, f"forced keys missing: {sorted(forced - G)[:8]}"
    O = set(int(x) for x in ora_idx[:total])
    assert forced <= O
    pg, po = G - forced, O - forced
    assert len(pg) == len(po) == m
    if pg == po:
        return 0
    only_o = np.array(sorted(po - pg))
    only_g = np.array(sorted(pg - po))
    tau = TAU_REL * abs(kth)
    gap = ora_scores[only_o].max() - ora_scores[only_g].min()
    assert gap < tau, (f"backbone swap beyond tolerance: dropped {only_o[:4]} kept {only_g[:4]}, tau {tau}")
    return len(only_o)
