"""Markdown table of the observed parity errors logged by the GPU tests.

Usage: DSA_PARITY_LOG=log.jsonl python -m pytest tests -m gpu ...; then
python tests/parity_summary.py log.jsonl.  One row per run_case call: rows
compared, allowed top-k swaps, score max-abs error, the attention over the
oracle's index set (dsa_sparse_attn) and the fused output against the oracle
over the fused call's own selection, as max-abs, max-abs / max|out| and lse
max-abs.
"""
from __future__ import annotations

import json
import sys


def main(path: str) -> int:
    recs = [json.loads(line) for line in open(path) if line.strip()]
    print("| case | rows | swaps | score max-abs | attn out max-abs | attn rel | attn lse | fused out max-abs "
          "| fused rel | fused lse |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for r in recs:
        a, e = r["attn"], r["e2e_own"]
        print(f"| {r['case']} | {r['rows']} | {r['swaps']} | {r['score_err']:.2e} | {a.get('out', 0):.2e} | "
              f"{a.get('out_rel', 0):.2e} | {a.get('lse', 0):.2e} | {e.get('out', 0):.2e} | {e.get('out_rel', 0):.2e} "
              f"| {e.get('lse', 0):.2e} |")
    worst = {k: max(r["e2e_own"].get(k, 0.0) for r in recs) for k in ("out", "out_rel", "lse")}
    print(f"\n{len(recs)} cases, {sum(r['rows'] for r in recs)} rows compared end to end; worst fused out "
          f"max-abs {worst['out']:.2e} (relative {worst['out_rel']:.2e}), worst lse {worst['lse']:.2e}.")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
