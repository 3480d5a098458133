"""Benchmark of the DSA hot path on one MI355X.

One step = one fused call (lightning indexer over every visible key, top-k
selection, attention over the selected rows) for the whole batch of the
workload: by default decode_128k, 64 single-token queries over 131072 cached
tokens each, 16 FP8 indexer heads of dim 128, k = 2048, bf16 KV cache with 32
query heads over 4 KV heads of dim 128 (dsa_decode).  decode_128k_fp8kv is
the same over an E4M3 main KV cache.  The prefill workloads (--workload
prefill_*) time dsa_prefill over the whole sequence.  Inputs are
seeded synthetic Gaussians already resident in HBM when the timed region
starts.

Prints ONE JSON line (rank 0):
  value         query tokens per second over the K timed steps
  roofline      the dominant kernel of the step, the indexer (decode: its FP8
                key stream against HBM bandwidth; prefill: its contraction
                against the MFMA peak of its dtype): algorithmic bytes or flops
                per launch / its mean duration inside the fused step, from the
                library's phase timer (HIP events on the step's stream)
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload
  attn_roofline the attention phase of the step: gathered K/V bytes against HBM
                bandwidth (decode), or the sparse flops against the bf16 peak
                (prefill)
  fused_phases_us  mean time of each phase of the fused step
  phases_us     mean time of each unfused entry point (indexer, top-k, attention)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query-tokens/s for indexer+top-k+sparse attn at 128K ctx, k=2048; % of roofline"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
INDEXER_SOURCES = [os.path.join(ROOT, "long_context_sparse_relu_amd", "csrc", f)
                   for f in ("indexer.hip", "fp8_index.h", "dsa_device.h", "dsa_kernels.h")]


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


def _events_mean_us(fn, reps, stream, host=None):
    """Mean GPU microseconds of fn (HIP events on `stream` around each call); with
    a dict `host`, host['us'] gets the mean host time of enqueueing one call."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    h = 0.0
    for i in range(reps):
        starts[i].record(stream)
        t = time.perf_counter()
        fn()
        h += time.perf_counter() - t
        ends[i].record(stream)
    torch.cuda.synchronize()
    if host is not None:
        host["us"] = 1e6 * h / reps
    return 1000.0 * sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / reps


def _sweep_mask(dsa, torch, dev, ladder, ks, chunks, chunk_nk, reps):
    """Masked MHA against gather attention, and DSA against dense attention, over L and k.

    Part "prefill": one sequence of L tokens (indexer 16 FP8 heads, attention 32
    bf16 heads of dim 128, MHA), for each k: the fused dsa_prefill step, its
    attention alone in GATHER and in MASKED mode, and dsa_dense_attn.  Part
    "chunk": n_q new queries over a cache of chunk_nk keys, k = ks[-1]: the
    attention in both modes.  Each time is the median of `reps` calls, each
    after a read of 1 GiB (so the gathered rows come from HBM, not a cache).
    Prints one JSON line per point and a summary line.
    """
    from dsa_inputs import custom_spec, kv_args, make_inputs
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def timed(fn, n):
        ts = []
        for _ in range(n + 1):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(1000.0 * e0.elapsed_time(e1))
        ts = sorted(ts[1:])
        return ts[len(ts) // 2]

    def problem(inp, k, mode):
        return dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=k, q=inp["q"],
                                iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"],
                                softmax_scale=inp["scale"], attn_mode=mode, **kv_args(inp))

    def attn_times(inp, k, idx, n, n_gather=None):
        res = {}
        for name, mode in (("gather", dsa.ATTN_GATHER), ("masked", dsa.ATTN_MASKED)):
            prob = problem(inp, k, mode)
            out, lse = dsa._out_tensors(prob, None, None)
            ws = torch.empty(max(1, dsa.workspace_bytes(dsa.OP_SPARSE_ATTN, prob)), dtype=torch.uint8, device=dev)
            reps_ = n_gather if (name == "gather" and n_gather) else n
            res[name] = timed(lambda: dsa.sparse_attn(prob, idx, out, lse, ws, stream), reps_)
        return res

    points = []
    for L in ladder:
        for k in ks:
            sp = custom_spec(name=f"prefill_L{L}", B=1, n_q=L, n_k=L, idx_heads=16, idx_dim=128, idx_dtype="e4m3",
                             top_k=k, q_heads=32, kv_heads=32, d_qk=128, d_v=128, attn_dtype="bf16",
                             outlier_frac=0.001)
            inp = make_inputs(sp, device=dev, seed=0)
            prob = problem(inp, k, dsa.ATTN_AUTO)
            out, lse = dsa._out_tensors(prob, None, None)
            idx = torch.empty((1, L, k), dtype=torch.int32, device=dev)
            ws = torch.empty(dsa.workspace_bytes(dsa.OP_PREFILL, prob), dtype=torch.uint8, device=dev)
            # long prefills: fewer timed calls (a gathered MHA prefill at 128K
            # reads about 4 TB)
            n = reps if L <= 8192 else (max(3, reps // 3) if L <= 32768 else 2)
            dsa_us = timed(lambda: dsa.prefill(prob, out, lse, idx, ws, stream), n)
            dsa.phase_timing(True)
            try:
                dsa.prefill(prob, out, lse, idx, ws, stream)
                phases = dsa.phase_times()
            finally:
                dsa.phase_timing(False)
            dws = torch.empty(max(1, dsa.workspace_bytes(dsa.OP_DENSE_ATTN, prob)), dtype=torch.uint8, device=dev)
            dense_us = timed(lambda: dsa.dense_attn(prob, out, lse, dws, stream), n)
            at = attn_times(inp, k, idx, n, n_gather=1 if L > 32768 else None)
            pt = {"sweep": "mask", "part": "prefill", "L": L, "k": k, "dsa_prefill_us": dsa_us,
                  "dsa_phases_us": phases, "attn_gather_us": at["gather"], "attn_masked_us": at["masked"],
                  "dense_attn_us": dense_us, "dsa_over_dense": dsa_us / dense_us}
            points.append(pt)
            print(json.dumps(pt), flush=True)
            del inp, prob, out, lse, idx, ws, dws
            torch.cuda.empty_cache()
    k = ks[-1]
    for hq, hkv in ((32, 32), (32, 4)):
        for n_q in chunks:
            sp = custom_spec(name=f"chunk{n_q}", B=1, n_q=n_q, n_k=chunk_nk, idx_heads=16, idx_dim=128,
                             idx_dtype="e4m3", top_k=k, q_heads=hq, kv_heads=hkv, d_qk=128, d_v=128,
                             attn_dtype="bf16")
            inp = make_inputs(sp, device=dev, seed=0)
            prob = problem(inp, k, dsa.ATTN_AUTO)
            out, lse = dsa._out_tensors(prob, None, None)
            idx = torch.empty((1, n_q, k), dtype=torch.int32, device=dev)
            ws = torch.empty(dsa.workspace_bytes(dsa.OP_PREFILL, prob), dtype=torch.uint8, device=dev)
            dsa_us = timed(lambda: dsa.prefill(prob, out, lse, idx, ws, stream), reps)
            at = attn_times(inp, k, idx, reps)
            dws = torch.empty(max(1, dsa.workspace_bytes(dsa.OP_DENSE_ATTN, prob)), dtype=torch.uint8, device=dev)
            dense_us = timed(lambda: dsa.dense_attn(prob, out, lse, dws, stream), reps)
            pt = {"sweep": "mask", "part": "chunk", "q_heads": hq, "kv_heads": hkv, "n_q": n_q, "n_k": chunk_nk,
                  "k": k, "dsa_prefill_us": dsa_us, "attn_gather_us": at["gather"], "attn_masked_us": at["masked"],
                  "dense_attn_us": dense_us}
            points.append(pt)
            print(json.dumps(pt), flush=True)
            del inp, prob, idx, out, lse, ws, dws
            torch.cuda.empty_cache()
    summary = {"sweep": "mask", "summary": True}
    for k in ks:
        pre = [p for p in points if p["part"] == "prefill" and p["k"] == k]
        wins = [p["L"] for p in pre if p["dsa_prefill_us"] < p["dense_attn_us"]]
        summary[f"k{k}_smallest_L_where_dsa_beats_dense"] = min(wins) if wins else None
        summary[f"k{k}_masked_faster_at_L"] = [p["L"] for p in pre if p["attn_masked_us"] < p["attn_gather_us"]]
    for hq, hkv in ((32, 32), (32, 4)):
        summary[f"chunk_{hq}x{hkv}_masked_faster_at_n_q"] = [
            p["n_q"] for p in points if p["part"] == "chunk" and p["kv_heads"] == hkv
            and p["attn_masked_us"] < p["attn_gather_us"]]
    print(json.dumps(summary), flush=True)
    return 0


def _sweep_ladder(dsa, torch, dev, lengths, ks, reps):
    """Decode time and bytes against context length L and k (one query per sequence).

    The decode_128k layout (indexer 16 FP8 heads of dim 128, bf16 KV with 32
    query heads over 4 kv heads of dim 128) at L tokens of context, 64
    sequences up to 128K and 8 beyond (memory).  Per point: the fused
    dsa_decode step and its phases, the algorithmic bytes (indexer keys and
    scales once, kept K/V rows once), dsa_dense_attn over every key, and the
    dense ideal (every K/V row read once at 8 TB/s).  Medians of `reps` calls,
    each after a 1 GiB read.  One JSON line per point.
    """
    from dsa_inputs import custom_spec, kv_args, make_inputs
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def timed(fn, n):
        ts = []
        for _ in range(n + 1):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(1000.0 * e0.elapsed_time(e1))
        ts = sorted(ts[1:])
        return ts[len(ts) // 2]

    for L in lengths:
        B = 64 if L <= 131072 else 8
        sp = custom_spec(name=f"decode_L{L}", B=B, n_q=1, n_k=L, idx_heads=16, idx_dim=128, idx_dtype="e4m3",
                         top_k=max(ks), q_heads=32, kv_heads=4, d_qk=128, d_v=128, attn_dtype="bf16")
        print(f"[ladder] inputs L={L} B={B}", file=sys.stderr, flush=True)
        inp = make_inputs(sp, device=dev, seed=0)
        for k in ks:
            prob = dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=k, q=inp["q"],
                                    iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"],
                                    softmax_scale=inp["scale"], **kv_args(inp))
            out, lse = dsa._out_tensors(prob, None, None)
            idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
            ws = torch.empty(dsa.workspace_bytes(dsa.OP_DECODE, prob), dtype=torch.uint8, device=dev)
            step_us = timed(lambda: dsa.decode(prob, out, lse, idx, ws, stream), reps)
            dsa.phase_timing(True)
            try:
                acc = {}
                for _ in range(reps):
                    flush.sum()
                    dsa.decode(prob, out, lse, idx, ws, stream)
                    for n_, v_ in dsa.phase_times().items():
                        acc[n_] = acc.get(n_, 0.0) + v_ / reps
            finally:
                dsa.phase_timing(False)
            idx_bytes = B * L * (128 + 4) + B * (16 * 128 + 4 + 16 * 4)
            gather_bytes = B * min(k, L) * 4 * 128 * 2 * 2
            pt = {"sweep": "ladder", "L": L, "B": B, "k": k, "step_us": step_us,
                  "q_tok_per_s": B / (step_us * 1e-6), "phases_us": acc,
                  "indexer_bytes": idx_bytes, "gather_bytes": gather_bytes,
                  "indexer_GBs": idx_bytes / (acc["index"] * 1e-6) / 1e9,
                  "gather_GBs": gather_bytes / (acc["attn"] * 1e-6) / 1e9,
                  "step_frac_of_hbm": (idx_bytes + gather_bytes) / (step_us * 1e-6) / 8e12}
            if k == ks[0]:
                dws = torch.empty(max(1, dsa.workspace_bytes(dsa.OP_DENSE_ATTN, prob)), dtype=torch.uint8,
                                  device=dev)
                pt["dense_attn_us"] = timed(lambda: dsa.dense_attn(prob, out, lse, dws, stream),
                                            reps if L <= 131072 else 2)
                del dws
            pt["dense_ideal_us"] = B * L * 4 * 128 * 2 * 2 / 8e12 * 1e6
            print(json.dumps(pt), flush=True)
            del prob, out, lse, idx, ws
        del inp
        torch.cuda.empty_cache()
    return 0


def _sweep_compress(dsa, torch, dev, reps):
    """Importance compression of whole caches: one JSON line per cache shape.

    The cut is the pages' operating point: an 8K recent window and half of the
    older tokens kept.  Bytes per call = importance read once (4 B per token)
    + every kept token's rows read and written + its position written; the
    call's time is the median of HIP-event-timed calls on the launch stream,
    each after a 1 GiB read that flushes the caches.
    """
    from dsa_inputs import importance_scores, kv_args, make_inputs, spec
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    # the ceiling a plain device copy reaches (bytes read + written)
    a = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    c = torch.empty_like(a)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        c.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(1e3 * e0.elapsed_time(e1))
    us = float(np.median(times))
    print(json.dumps({"sweep": "compress", "cache": "plain_copy_4GiB", "us": round(us, 1), "bytes": 2 * a.numel(),
                      "tb_s": round(2 * a.numel() / us / 1e6, 3), "frac_hbm": round(2 * a.numel() / us / 8e6, 3)}),
          flush=True)
    del a, c
    for name in ("decode_1m", "decode_128k", "decode_128k_fp8kv"):
        s = spec(name)
        print(f"[bench] compress: generating {name} inputs", file=sys.stderr, flush=True)
        inp = make_inputs(s, device=dev, seed=0)
        B, N, window = s["B"], s["n_k"], 8192
        keep_old = (N - window) // 2
        imp = importance_scores(B, N, "normal", device=dev, seed=0)
        prob = dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=s["top_k"], q=inp["q"],
                                iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"], **kv_args(inp))
        ws = torch.empty(dsa.workspace_bytes(dsa.OP_COMPRESS_KV, prob), dtype=torch.uint8, device=dev)
        res = dsa.compress_kv(prob, imp, window, keep_old, workspace=ws, stream=stream)
        n_keep = res["pos"].shape[1]
        row = sum(t[0, 0].numel() * t.element_size() for t in (res["k"], res["v"], res["ik"], res["ik_scale"])
                  if t is not None)
        times = []
        for _ in range(reps):
            flush.add_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dsa.compress_kv(prob, imp, window, keep_old, out=res, workspace=ws, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(1e3 * e0.elapsed_time(e1))
        us = float(np.median(times))
        nbytes = B * N * 4 + B * n_keep * (2 * row + 4)
        print(json.dumps({"sweep": "compress", "cache": name, "batch": B, "tokens": N, "window": window,
                          "keep_old": keep_old, "kept": n_keep, "cache_cut": round(1 - n_keep / N, 4),
                          "row_bytes": row, "us": round(us, 1), "bytes": nbytes,
                          "tb_s": round(nbytes / us / 1e6, 3), "frac_hbm": round(nbytes / us / 1e6 / 8.0, 3)}),
              flush=True)
        del inp, imp, prob, ws, res
        torch.cuda.empty_cache()
    return 0


def _cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _cpu_baseline(inp, n_seq, n_rows, min_s=10.0):
    """The oracle on n_seq sequences (decode) or n_rows evenly spread query rows
    (prefill), on every host CPU this process may run on."""
    import oracle
    from dsa_inputs import oracle_view
    oracle.set_num_threads(len(os.sched_getaffinity(0)))
    threads = oracle.num_threads()
    if inp["n_q"] == 1:
        seqs = list(range(min(n_seq, inp["B"])))
        ov = oracle_view(inp, seqs)
        rows = None
        what = f"{len(seqs)} of {inp['B']} sequences (1 query x {inp['n_k']} keys each)"
        count = len(seqs)
    else:
        ov = oracle_view(inp, [0])
        n_q = inp["n_q"]
        ts = sorted({int(round(i * (n_q - 1) / max(1, n_rows - 1))) for i in range(n_rows)})
        rows = [(0, t) for t in ts]
        what = f"{len(ts)} of {n_q} query rows of sequence 0, evenly spread (their prefixes average {sum(ts) / len(ts) + 1:.0f} keys)"
        count = len(ts)
    # whole passes until about min_s seconds of CPU work (at most 8), for a stable rate
    reps, total = 0, 0.0
    while reps < 8 and (reps == 0 or total < min_s):
        t0 = time.perf_counter()
        oracle.dsa_forward(ov, rows)
        total += time.perf_counter() - t0
        reps += 1
    return {"value": reps * count / total, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "cpus_available": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
            "sample": f"{what}, whole path in fp64: indexer, top-k, attention; {reps} pass(es), {total:.2f} s"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_128k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=64, help="sequences the oracle baseline runs (decode)")
    ap.add_argument("--cpu-rows", type=int, default=48, help="query rows the oracle baseline runs (prefill)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--zero-weight-rows", type=int, default=0,
                    help="zero the indexer head weights of the first R query rows: every score of such a row ties "
                         "at 0, so a decode row overflows its sampled candidate list and is recomputed in full "
                         "(times that fallback; the workload is then not the benchmark's)")
    ap.add_argument("--phase-reps", type=int, default=10)
    ap.add_argument("--sweep", choices=["mask", "ladder", "compress"], default=None,
                    help="instead of the step benchmark: 'mask' = masked vs gather attention and DSA vs dense "
                         "attention in prefill; 'ladder' = decode time and bytes against context length and k "
                         "(JSON line per point); 'compress' = importance compression of whole caches")
    ap.add_argument("--lengths", default="4096,16384,65536,131072,262144,524288,1048576")
    ap.add_argument("--ladder-ks", default="256,512,2048")
    ap.add_argument("--ladder", default="1024,2048,4096,8192,16384,32768,65536,131072")
    ap.add_argument("--ks", default="512,2048")
    ap.add_argument("--chunks", default="16,64,256,1024,4096")
    ap.add_argument("--chunk-nk", type=int, default=32768)
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        return 2

    import torch
    import long_context_sparse_relu_amd as dsa
    from dsa_inputs import kv_args, make_inputs, spec

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.sweep == "ladder":
        return _sweep_ladder(dsa, torch, dev, [int(x) for x in args.lengths.split(",")],
                             [int(x) for x in args.ladder_ks.split(",")], max(3, args.steps // 4))
    if args.sweep == "compress":
        return _sweep_compress(dsa, torch, dev, max(3, args.steps // 4))
    if args.sweep == "mask":
        return _sweep_mask(dsa, torch, dev, [int(x) for x in args.ladder.split(",")],
                           [int(x) for x in args.ks.split(",")], [int(x) for x in args.chunks.split(",")],
                           args.chunk_nk, max(3, args.steps // 4))
    s = spec(args.workload)
    decode = s["n_q"] == 1
    print(f"[bench] generating {args.workload} inputs", file=sys.stderr, flush=True)
    inp = make_inputs(s, device=dev, seed=args.seed)
    B, N, k, n_q = s["B"], s["n_k"], s["top_k"], s["n_q"]
    if args.zero_weight_rows:
        inp["iw"].view(B * n_q, -1)[:args.zero_weight_rows].zero_()
    prob = dsa.make_problem(iq=inp["iq"], ik=inp["ik"], iw=inp["iw"], top_k=k, q=inp["q"],
                            iq_scale=inp["iq_scale"], ik_scale=inp["ik_scale"], softmax_scale=inp["scale"],
                            sink_tokens=s.get("sinks", 0), local_window=s.get("window", 0), **kv_args(inp))
    out, lse = dsa._out_tensors(prob, None, None)
    idx = torch.empty((B, n_q, prob.sel_width), dtype=torch.int32, device=dev)
    op = dsa.OP_DECODE if decode else dsa.OP_PREFILL
    ws = torch.empty(dsa.workspace_bytes(op, prob), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    fused = dsa.decode if decode else dsa.prefill

    def step():
        fused(prob, out=out, lse=lse, idx_out=idx, workspace=ws, stream=stream)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] timed steps", file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    th = time.perf_counter()
    for _ in range(args.steps):
        step()
    host_step_us = 1e6 * (time.perf_counter() - th) / args.steps   # enqueue time, the GPU runs behind
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # the fused step's phases, from the library's event timer on the step's stream
    reps = args.phase_reps
    dsa.phase_timing(True)
    acc = {name: 0.0 for name in dsa.PHASES}
    try:
        for _ in range(reps):
            step()
            for name, us in dsa.phase_times().items():
                acc[name] += us
    finally:
        dsa.phase_timing(False)
    fused_us = {name: v / reps for name, v in acc.items()}
    idx_us_fused = fused_us["index"]

    # unfused phases, each its own launch sequence on the same stream (only
    # where the full score matrix the unfused indexer writes is at most 8 GiB)
    unfused = B * n_q * N * 4 <= (8 << 30)
    if unfused:
        scores = torch.empty((B, n_q, N), dtype=torch.float32, device=dev)
        tws = torch.empty(dsa.workspace_bytes(dsa.OP_TOPK, prob), dtype=torch.uint8, device=dev)
        aws = torch.empty(max(1, dsa.workspace_bytes(dsa.OP_SPARSE_ATTN, prob)), dtype=torch.uint8, device=dev)
        hi, ht, ha = {}, {}, {}
        idx_us = _events_mean_us(lambda: dsa.index_scores(prob, scores, stream), reps, stream, hi)
        topk_us = _events_mean_us(lambda: dsa.topk(prob, scores, idx, tws, stream), reps, stream, ht)
        attn_us = _events_mean_us(lambda: dsa.sparse_attn(prob, idx, out, lse, aws, stream), reps, stream, ha)
        del scores, tws, aws

    H, D = s["idx_heads"], s["idx_dim"]
    kbytes = {"f32": 4, "bf16": 2, "e4m3": 1}[s["idx_dtype"]]
    kvt = inp["kv_dtype"]
    abytes = {"f32": 4, "bf16": 2, "e4m3": 1}[kvt]
    # bytes of one kept token's K/V rows over all kv heads (an FP8 cache adds a 4-byte scale per row)
    n_rows_kv = 1 if s["latent"] else 2
    row = s["kv_heads"] * ((s["d_qk"] + (0 if s["latent"] else s["d_v"])) * abytes
                           + (4 * n_rows_kv if kvt == "e4m3" else 0))
    # visible keys and kept keys summed over every query row
    pairs = sum(N - n_q + t + 1 for t in range(n_q)) * B
    kept = sum(min(prob.sel_width, N - n_q + t + 1) for t in range(n_q)) * B
    gather_bytes = kept * row
    attn_flops = 2 * kept * s["q_heads"] * (s["d_qk"] + s["d_v"])
    if decode:
        # HBM bound: every key row (+ its scale) streams once, plus queries and head weights
        idx_bytes = B * N * (D * kbytes + (4 if s["idx_dtype"] == "e4m3" else 0)) + B * (H * D * kbytes + 4 + 4 * H)
        achieved = idx_bytes / (idx_us_fused * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": "k_index_fp8_mfma (candidate mode)", "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": _traffic(f"k_index_fp8_mfma@{args.workload}"),
                "algorithmic_bytes": idx_bytes, "mean_us": idx_us_fused}
        # the gather attention against HBM bandwidth: selected K/V bytes / its fused-phase time
        attn_roof = {"bound": "hbm", "kernel": "sparse gather attention", "achieved":
                     gather_bytes / (fused_us["attn"] * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "algorithmic_bytes": gather_bytes, "mean_us": fused_us["attn"]}
        attn_roof["frac"] = attn_roof["achieved"] / HBM_PEAK_GBS
        total_bytes = idx_bytes + gather_bytes
        step_roof = {"algorithmic_bytes": total_bytes,
                     "achieved_GBs": total_bytes / (ms_per_step * 1e-3) / 1e9,
                     "frac": total_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS}
    else:
        # a dense contraction: 2*H*D flops per visible (query, key) pair
        idx_flops = 2 * pairs * H * D
        peak = {"e4m3": 5000.0, "bf16": 2500.0, "f32": 157.3}[s["idx_dtype"]]
        achieved = idx_flops / (idx_us_fused * 1e-6) / 1e12
        kern = ("k_index_generic" if not (s["idx_dtype"] != "f32" and n_q >= 16 and H <= 16)
                else "k_index_fp8_q16" if s["idx_dtype"] == "e4m3" else "k_index_tiled")
        roof = {"bound": "mfma" if s["idx_dtype"] != "f32" else "alu", "kernel": kern, "achieved": achieved,
                "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None,
                "algorithmic_flops": idx_flops, "mean_us": idx_us_fused}
        attn_roof = {"bound": "mfma", "kernel": "sparse attention", "achieved":
                     attn_flops / (fused_us["attn"] * 1e-6) / 1e12, "peak": 2500.0, "unit": "TFLOP/s",
                     "algorithmic_flops": attn_flops, "mean_us": fused_us["attn"]}
        attn_roof["frac"] = attn_roof["achieved"] / 2500.0
        # the masked walk computes whole causal tiles: its executed work is the dense causal product
        attn_roof["dense_equivalent_flops"] = 2 * pairs * s["q_heads"] * (s["d_qk"] + s["d_v"])
        attn_roof["dense_equivalent_frac"] = attn_roof["dense_equivalent_flops"] / (fused_us["attn"] * 1e6) / 2500.0
        step_roof = {"indexer_flops": idx_flops, "attention_flops": attn_flops,
                     "ideal_us_at_peaks": idx_flops / (peak * 1e6) + attn_flops / (2500.0 * 1e6)}
    res = {
        "metric": METRIC,
        "value": B * n_q / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{s['idx_dtype']}-indexer/{s['attn_dtype']}-attn"
                 + (f"/{kvt}-kv" if kvt != s["attn_dtype"] else ""),
        "data": "synthetic",
        "config": {"workload": args.workload + (f"+{args.zero_weight_rows}_zero_weight_rows"
                                                 if args.zero_weight_rows else ""), "batch": B, "n_q": n_q, "context": N, "top_k": k,
                   "idx_heads": H, "idx_dim": D, "idx_dtype": s["idx_dtype"],
                   "q_heads": s["q_heads"], "kv_heads": s["kv_heads"], "d_qk": s["d_qk"],
                   "d_v": s["d_v"], "latent": s["latent"], "attn_dtype": s["attn_dtype"],
                   "kv_dtype": kvt, "sink_tokens": s.get("sinks", 0), "local_window": s.get("window", 0)},
        "roofline": roof,
        "attn_roofline": attn_roof,
        "step_roofline": step_roof,
        "fused_phases_us": fused_us,
        "phases_us": {"index_scores": idx_us, "topk": topk_us, "sparse_attn": attn_us,
                      "gather_GBs": gather_bytes / (attn_us * 1e-6) / 1e9,
                      "attn_TFLOPs": attn_flops / (attn_us * 1e-6) / 1e12} if unfused else None,
        # host time of enqueueing one call (binding + C ABI + launches), against
        # the GPU time above: the fused step is GPU-bound when it is smaller
        "host_enqueue_us": {"fused_step": host_step_us,
                            **({"index_scores": hi["us"], "topk": ht["us"], "sparse_attn": ha["us"]}
                               if unfused else {})},
    }
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = _cpu_baseline(inp, args.cpu_sample, args.cpu_rows)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
