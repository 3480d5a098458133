"""Benchmark of the DSA hot path on one MI355X.

One step = one fused decode call (lightning indexer over every cached key,
top-k selection, attention over the selected rows) for the whole batch of the
workload: by default 64 single-token queries over 131072 cached tokens each,
16 FP8 indexer heads of dim 128, k = 2048, bf16 KV cache with 32 query heads
over 4 KV heads of dim 128.  Inputs are seeded synthetic Gaussians already
resident in HBM when the timed region starts.

Prints ONE JSON line (rank 0):
  value         query tokens per second over the K timed steps
  roofline      the dominant kernel (the indexer's FP8 key stream) against HBM
                bandwidth: algorithmic bytes per launch / its mean launch time
                from HIP events on the stream it runs on
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload
  phases_us     mean time of each unfused step (indexer, top-k, attention)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query-tokens/s for indexer+top-k+sparse attn at 128K ctx, k=2048; % of roofline"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
INDEXER_SOURCES = [os.path.join(ROOT, "long_context_sparse_relu_amd", "csrc", f)
                   for f in ("indexer.hip", "dsa_device.h")]


def _source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key):
    """Measured HBM bytes per launch for the kernel, if the counters match its source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != _source_hash(INDEXER_SOURCES):
        return None
    return int(rec["bytes_per_launch"])


def _events_mean_us(fn, reps, stream):
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return 1000.0 * sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / reps


def _cpu_baseline(inp, n_seq):
    import oracle
    from dsa_inputs import oracle_view
    seqs = list(range(min(n_seq, inp["B"])))
    ov = oracle_view(inp, seqs)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    oracle.dsa_forward(ov)
    dt = time.perf_counter() - t0
    return {"value": len(seqs) * inp["n_q"] / dt, "unit": "query-tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{len(seqs)} of {inp['B']} sequences ({inp['n_q']} query x {inp['n_k']} keys each), "
                       f"whole path in fp64: indexer, top-k, attention; {dt:.2f} s")}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_128k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=64, help="sequences the oracle baseline runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--phase-reps", type=int, default=10)
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); a multi-GPU run is not part of "
              "this build", file=sys.stderr)
        return 2

    import torch
    import long_context_sparse_relu_amd as dsa
    from dsa_inputs import spec, make_inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    s = spec(args.workload)
    if s["n_q"] != 1:
        print("bench.py times the decode workloads (n_q == 1)", file=sys.stderr)
        return 2
    print(f"[bench] generating {args.workload} inputs", file=sys.stderr, flush=True)
    inp = make_inputs(s, device=dev, seed=args.seed)
    B, N, k = s["B"], s["n_k"], s["top_k"]
    prob = dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=k, q=inp["q"], k=inp["k"],
                            v=inp["v"], iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"],
                            softmax_scale=inp["scale"], latent_dv=inp["latent_dv"])
    out, lse = dsa._out_tensors(prob, None, None)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.workspace_bytes(dsa.OP_DECODE, prob), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        dsa.decode(prob, out=out, lse=lse, idx_out=idx, workspace=ws, stream=stream)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] timed steps", file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # unfused phases, each its own launch sequence on the same stream
    scores = torch.empty((B, 1, N), dtype=torch.float32, device=dev)
    tws = torch.empty(dsa.workspace_bytes(dsa.OP_TOPK, prob), dtype=torch.uint8, device=dev)
    reps = args.phase_reps
    idx_us = _events_mean_us(lambda: dsa.index_scores(prob, scores, stream), reps, stream)
    topk_us = _events_mean_us(lambda: dsa.topk(prob, scores, idx, tws, stream), reps, stream)
    attn_us = _events_mean_us(lambda: dsa.sparse_attn(prob, idx, out, lse, stream), reps, stream)

    # algorithmic bytes of the indexer launch: every FP8 key row + its scale,
    # plus the queries, scales and head weights
    H, D = s["idx_heads"], s["idx_dim"]
    idx_bytes = B * N * (D + 4) + B * (H * D + 4 + 4 * H)
    row = s["kv_heads"] * (s["d_qk"] + (0 if s["latent"] else s["d_v"])) * 2
    gather_bytes = B * k * row
    achieved = idx_bytes / (idx_us * 1e-6) / 1e9
    traffic = _traffic(f"k_index_fp8_mfma@{args.workload}")
    total_bytes = idx_bytes + gather_bytes
    res = {
        "metric": METRIC,
        "value": B / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-indexer/bf16-attn",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "context": N, "top_k": k,
                   "idx_heads": H, "idx_dim": D, "idx_dtype": s["idx_dtype"],
                   "q_heads": s["q_heads"], "kv_heads": s["kv_heads"], "d_qk": s["d_qk"],
                   "d_v": s["d_v"], "latent": s["latent"], "attn_dtype": s["attn_dtype"]},
        "roofline": {"bound": "hbm", "kernel": "k_index_fp8_mfma", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": idx_bytes, "mean_us": idx_us},
        "step_roofline": {"algorithmic_bytes": total_bytes,
                          "achieved_GBs": total_bytes / (ms_per_step * 1e-3) / 1e9,
                          "frac": total_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "phases_us": {"index_scores": idx_us, "topk": topk_us, "sparse_attn": attn_us,
                      "gather_GBs": gather_bytes / (attn_us * 1e-6) / 1e9},
    }
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = _cpu_baseline(inp, args.cpu_sample)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
