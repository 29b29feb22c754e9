"""Margin rows of the five named workloads, from the CPU oracle alone: batch rows whose outcome a correct rounding
could change (accept test |u - p/q| <= 1e-5, Gumbel top-2 gap <= 1e-5, top-p |M / Z_K - P| <= 1e-6, or a residual
that vanishes in fp64), which the parity tests check against the oracle's alternative resolutions instead of
bit-exactly.  Drafts are drawn with the oracle's own sampler (as in the parity tests).  Prints a markdown table.

    python3 tests/margin_counts.py [--all-offsets]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import parity  # noqa: E402
from rejection_sampling_verify_16_amd import workloads as W  # noqa: E402


def main():
    all_offsets = "--all-offsets" in sys.argv
    o = oracle.get()
    threads = min(os.cpu_count() or 1, 16)
    print("| workload | batch rows x offsets | margin rows | accept | gap | top-p | fallback | sentinel |")
    print("|---|---|---|---|---|---|---|---|")
    for name in ("1", "2", "3", "4a", "4b", "5"):
        w = W.CONFIGS[name]()
        drafts = w.draft_tokens(parity.oracle_sampler(o))
        offs = list(w.offsets) if all_offsets else [w.offsets[0]]
        tot = dict(margin=0, accept=0, gap=0, topp=0, fallback=0, sentinel=0)
        t0 = time.perf_counter()
        for off in offs:
            r = o.spec_verify(w.target, w.draft, drafts, w.temperature, w.top_k, w.top_p, seed=w.seed, offset=off,
                              num_threads=threads)
            live = ~r.sentinel
            m = r.margin_rows(parity.ACCEPT_TOL, parity.GAP_TOL, parity.TOPP_TOL) & live
            tot["margin"] += int(m.sum())
            tot["accept"] += int(((r.accept_margin <= parity.ACCEPT_TOL) & live).sum())
            tot["gap"] += int(((r.gumbel_gap <= parity.GAP_TOL) & live).sum())
            tot["topp"] += int(((r.topp_margin <= parity.TOPP_TOL) & live).sum())
            tot["fallback"] += int((r.fallback & live).sum())
            tot["sentinel"] += int(r.sentinel.sum())
        print(f"| {name}: {w.name} | {w.B} x {len(offs)} | {tot['margin']} | {tot['accept']} | {tot['gap']} | "
              f"{tot['topp']} | {tot['fallback']} | {tot['sentinel']} |", flush=True)
        print(f"  ({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
