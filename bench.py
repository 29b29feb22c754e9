"""Benchmark of libspecverify on one MI355X: verified rows/s and logit bandwidth vs the HBM roofline.

One step = one spec_verify() call over one batch of synthetic inputs already resident in HBM
(default workload: B=64, k=2, V=157184, bf16, mixed temperature / top-k / top-p per row).
Input sets are rotated so that the working set exceeds the 256 MB Infinity Cache.

Prints one JSON line.  Besides the throughput it reports
  roofline:     the statistics kernel (it streams every logit once): algorithmic logit bytes per
                launch / its average duration (HIP events the library records around each of its
                kernels, over a second pass of the same calls), against the 8 TB/s HBM peak;
  cpu_baseline: the CPU oracle timed on this host on a bounded sample of the same workload;
  commit:       the commit step after verify (spec_commit) on a hybrid-model state workload, with its own
                throughput, roofline and CPU baseline (skip with --no-commit, alone with --commit-only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified rows/s + logits HBM GB/s (% peak), B=64 k=2 V=157184 bf16"
HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 1 << 30
_CSRC = os.path.join(ROOT, "rejection_sampling_verify_16_amd", "csrc")
KERNEL_SRC = [os.path.join(_CSRC, f) for f in ("specverify.hip", "sv_common.h")]
COMMIT_SRC = [os.path.join(_CSRC, "commit.hip")]


def kernel_digest(files=None) -> str:
    """Digest of the kernel sources' code (comments and whitespace removed), so that a traffic figure stays
    attached to the code it was measured on."""
    import re
    h = hashlib.sha256()
    for f in files or KERNEL_SRC:
        with open(f) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic_target(config: str):
    """(summary file, kernel name fragment, sources) of the dominant kernel of a workload."""
    if config == "commit":
        return os.path.join(ROOT, "profiles", "traffic_commit.json"), "k_commit", COMMIT_SRC
    return os.path.join(ROOT, "profiles", f"traffic_config{config}.json"), "k1_stats", KERNEL_SRC


def load_traffic(config: str):
    """HBM traffic per launch from the committed PMC summary, if it was taken on this kernel."""
    path, _, files = _traffic_target(config)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_digest") != kernel_digest(files):
        return None
    return t.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="3", help="workload: 1, 2, 3, 4a, 4b, 5 (with --pmc-summary also: commit)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--raw-logprobs", action="store_true",
                    help="time spec_verify_raw (also the raw logprobs of the committed tokens)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-commit", action="store_true", help="skip the commit-step measurement")
    ap.add_argument("--commit-only", action="store_true", help="only the commit-step measurement")
    ap.add_argument("--commit-steps", type=int, default=100)
    ap.add_argument("--no-tree", action="store_true", help="skip the tree-verification measurement")
    ap.add_argument("--tree-only", action="store_true", help="only the tree-verification measurement")
    ap.add_argument("--configs", default="1,2,4a,4b,5",
                    help="other workloads timed after the headline one (comma list; empty: none)")
    ap.add_argument("--configs-only", action="store_true", help="only the other workloads")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times (PMC calibration)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="summarise rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this benchmark and of the copy "
                         "probe into profiles/traffic_config<C>.json (no GPU needed)")
    ap.add_argument("--pmc-report", nargs="+", metavar="DIR",
                    help="print the mean of every counter per kernel (per dispatch) over rocprofv3 --pmc CSV runs "
                         "(no GPU needed)")
    args = ap.parse_args()
    if args.pmc_report:
        pmc_report(args.pmc_report)
        return
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import rejection_sampling_verify_16_amd as sv
    from rejection_sampling_verify_16_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)
        return
    if args.commit_only:
        print(json.dumps({"commit": bench_commit(args, dev)}), flush=True)
        return
    if args.tree_only:
        print(json.dumps({"tree": bench_tree(args, dev)}), flush=True)
        return
    if args.configs_only:
        print(json.dumps({"configs": bench_configs(args, dev)}), flush=True)
        return
    w = W.CONFIGS[args.config]()
    B, k, V = w.B, w.k, w.V
    bf16 = w.dtype == "bf16"
    tgt0, drf0, drafts, T, K, P = verify_inputs(w, dev)

    n_sets = max(2, math.ceil(ROTATE_BYTES / w.logit_bytes))
    sets = [(tgt0, drf0)] + [(tgt0.clone(), drf0.clone()) for _ in range(n_sets - 1)]
    out = sv.alloc_outputs(B, k, dev, raw=args.raw_logprobs)
    ws = sv.make_workspace(B, k, V, sv.SPEC_DTYPE_BF16 if bf16 else sv.SPEC_DTYPE_F32, dev)
    stream = torch.cuda.current_stream(dev)
    offsets = w.offsets

    def step(i, timing=None):
        t_, d_ = sets[i % n_sets]
        sv.spec_verify(t_, d_, drafts, T, K, P, seed=w.seed, offset=offsets[i % len(offsets)], out=out,
                       workspace=ws, stream=stream, raw=args.raw_logprobs, timing=timing)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` calls ----
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / args.steps

    # ---- per-kernel durations: HIP events recorded by the library around each of its kernels,
    # on the stream the kernels run on, over a second pass of the same `steps` calls ----
    kms = kernel_durations(sv, step, args.steps, stream)
    k1_ms = kms[0]
    km_ms = kms[1] if len(kms) > 1 else 0.0
    k5_ms = kms[2] if len(kms) > 2 else 0.0
    logit_bytes = w.logit_bytes
    draft_pos_bytes = w.B * 2 * w.k * w.V * (2 if bf16 else 4)  # rows K5 re-reads (bonus row aside)
    k1_gbps = logit_bytes / (k1_ms * 1e-3) / 1e9
    rows_per_s = B / (ms_per_step * 1e-3)
    traffic = load_traffic(args.config)

    result = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "verified rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "k": k, "V": V, "logit_bytes_per_step": logit_bytes,
                   "raw_logprobs": bool(args.raw_logprobs),
                   "rotating_input_sets": n_sets},
        "logits_GBps": logit_bytes / (ms_per_step * 1e-3) / 1e9,
        "pct_hbm_peak": 100.0 * logit_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "wall_s": wall,
        "roofline": {
            "bound": "hbm",
            "achieved": k1_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": k1_gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel": "k1_stats",
            "kernel_ms_mean": k1_ms,
            "algorithmic_bytes": logit_bytes,
        },
        "kernels": {
            "k1_stats": {"ms_mean": k1_ms, "bytes": logit_bytes, "GBps": k1_gbps},
            # per-row merges of K1's slice partials and the kept thresholds (re-reads only rows whose
            # threshold needs a count over the whole row)
            "k1_rows": {"ms_mean": km_ms},
            # K5 streams the draft-position rows of batch rows it cannot finish from recorded
            # candidates; this is its traffic when every row is streamed (an upper bound)
            "k5_verify": {"ms_mean": k5_ms, "bytes_all_rows_streamed": draft_pos_bytes},
        },
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, drafts.cpu().numpy(), args.cpu_seconds)
    del sets, out, ws
    torch.cuda.empty_cache()
    if args.configs:
        result["configs"] = bench_configs(args, dev)
    if not args.no_tree:
        result["tree"] = bench_tree(args, dev)
    if not args.no_commit:
        result["commit"] = bench_commit(args, dev)
    print(json.dumps(result), flush=True)


def verify_inputs(w, dev):
    """Device inputs of a verify workload: logits, parameters and the drafts drawn from q by the library's
    plain sampler (plus the workload's overrides)."""
    import torch
    import rejection_sampling_verify_16_amd as sv
    bf16 = w.dtype == "bf16"

    def to_dev(a):
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if bf16 else torch.from_numpy(a)
        return t.to(dev)

    tt = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)
    tgt, drf = to_dev(w.target), to_dev(w.draft)
    rows, Tr, Kr, Pr, rb, rp = w.draft_sampling_inputs()
    dtok, _ = sv.spec_sample(drf.reshape(w.B * w.k, w.V), tt(Tr, np.float32), tt(Kr, np.int32), tt(Pr, np.float32),
                             tt(rb, np.int32), tt(rp, np.int32), seed=w.draft_seed, offset=w.draft_offset)
    drafts = dtok.reshape(w.B, w.k).contiguous()
    for b, i, t in w.draft_overrides:
        drafts[b, i] = t
    return tgt, drf, drafts, tt(w.temperature, np.float32), tt(w.top_k, np.int32), tt(w.top_p, np.float32)


def bench_configs(args, dev):
    """The other named workloads, one after another: per-call time over back-to-back calls on rotating input
    sets (inputs resident in HBM), verified rows/s, logit GB/s against the HBM peak, and each kernel's mean
    duration from the library's event hook.  Config 5 runs its 100 offsets (0..99) on the same inputs."""
    import torch
    import rejection_sampling_verify_16_amd as sv
    from rejection_sampling_verify_16_amd import workloads as W
    res = {}
    stream = torch.cuda.current_stream(dev)
    for name in [c for c in args.configs.split(",") if c]:
        w = W.CONFIGS[name]()
        tgt0, drf0, drafts, T, K, P = verify_inputs(w, dev)
        n_sets = max(2, math.ceil(ROTATE_BYTES / w.logit_bytes))
        sets = [(tgt0, drf0)] + [(tgt0.clone(), drf0.clone()) for _ in range(n_sets - 1)]
        out = sv.alloc_outputs(w.B, w.k, dev)
        ws = sv.make_workspace(w.B, w.k, w.V, sv.SPEC_DTYPE_BF16 if w.dtype == "bf16" else sv.SPEC_DTYPE_F32, dev)
        offs = w.offsets
        n = len(offs) if len(offs) > 1 else 200

        def step(i, timing=None):
            t_, d_ = sets[i % n_sets]
            sv.spec_verify(t_, d_, drafts, T, K, P, seed=w.seed, offset=offs[i % len(offs)], out=out, workspace=ws,
                           stream=stream, timing=timing)

        for i in range(10):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        kms = kernel_durations(sv, step, n, stream)
        k1_ms = kms[0]
        km_ms = kms[1] if len(kms) > 1 else 0.0
        k5_ms = kms[2] if len(kms) > 2 else 0.0
        acc = out["accept_len"].float().mean().item()
        gbps = w.logit_bytes / (ms * 1e-3) / 1e9
        k1_gbps = w.logit_bytes / (k1_ms * 1e-3) / 1e9
        res[name] = {
            "workload": w.name, "B": w.B, "k": w.k, "V": w.V, "dtype": w.dtype, "calls": n,
            "us_per_call": ms * 1e3, "verified_rows_per_s": w.B / (ms * 1e-3), "logit_bytes_per_call": w.logit_bytes,
            "logits_GBps": gbps, "pct_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
            "kernels_us": {"k1_stats": k1_ms * 1e3, "k1_rows": km_ms * 1e3, "k5_verify": k5_ms * 1e3},
            "k1_stats_roofline_frac": k1_gbps / HBM_PEAK_GBPS, "mean_accept_len": acc,
        }
        print(f"[bench] config {name}: {ms * 1e3:.1f} us/call", file=sys.stderr, flush=True)
        del sets, out, ws, tgt0, drf0
        torch.cuda.empty_cache()
    return res


def bench_tree(args, dev):
    """Tree verification (spec_tree_verify) on an EAGLE-style 9-node tree per batch row (B=64, V=157184,
    bf16, mixed parameters): verified rows/s, per-kernel durations from the library's event hook, and the
    row-statistics kernel against the HBM roofline with the tree's logit bytes (every node row read once)."""
    import torch
    import rejection_sampling_verify_16_amd as sv
    from rejection_sampling_verify_16_amd import workloads as W
    w = W.tree_eagle9()
    d = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)
    tgt0 = torch.from_numpy(w.target.view(np.int16)).view(torch.bfloat16).to(dev)
    n_sets = max(2, math.ceil(ROTATE_BYTES / w.logit_bytes))
    sets = [tgt0] + [tgt0.clone() for _ in range(n_sets - 1)]
    par, tok = d(w.parent, np.int32), d(w.node_tokens, np.int32)
    T, K, P = d(w.temperature, np.float32), d(w.top_k, np.int32), d(w.top_p, np.float32)
    ws = torch.zeros(sv.tree_workspace_size(w.B, w.N, w.V, sv.SPEC_DTYPE_BF16), dtype=torch.uint8, device=dev)
    out = None
    stream = torch.cuda.current_stream(dev)

    def step(i, timing=None):
        nonlocal out
        out = sv.spec_tree_verify(sets[i % n_sets], par, tok, T, K, P, seed=w.seed, offset=i, out=out, workspace=ws,
                                  stream=stream, timing=timing)

    n = max(50, args.steps // 2)
    for i in range(10):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    k1_ms, km_ms, kt_ms = kernel_durations(sv, step, n, stream)
    gbps = w.logit_bytes / (k1_ms * 1e-3) / 1e9
    acc = out["accept_len"].cpu().numpy()
    res = {
        "metric": "verified rows/s (draft trees)",
        "value": w.B / (ms * 1e-3),
        "unit": "verified rows/s",
        "steps": n,
        "ms_per_step": ms,
        "dtype": "bf16",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "V": w.V, "parents": list(W.EAGLE_TREE_9),
                   "logit_bytes_per_step": w.logit_bytes, "rotating_input_sets": n_sets},
        "mean_accept_len": float(acc.mean()),
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None, "kernel": "k1_stats (tree rows)",
                     "kernel_ms_mean": k1_ms, "algorithmic_bytes": w.logit_bytes},
        "kernels": {"k1_stats": {"ms_mean": k1_ms}, "k1_rows": {"ms_mean": km_ms}, "k_tree": {"ms_mean": kt_ms}},
    }
    if not args.no_cpu_baseline:
        import oracle
        o = oracle.get()
        threads = min(os.cpu_count() or 1, 16)
        calls, t0 = 0, time.perf_counter()
        while True:
            o.tree_verify(w.target, w.parent, w.node_tokens, w.temperature, w.top_k, w.top_p, seed=w.seed,
                          offset=calls, num_threads=threads)
            calls += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 5.0) or calls >= 200:
                break
        res["cpu_baseline"] = {"value": w.B * calls / el, "unit": "verified rows/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{calls} full calls of the tree workload ({w.B} rows each), {el:.1f} s"}
    return res


def bench_commit(args, dev):
    """The commit step after verify on its own workload: one spec_commit call per step, inputs resident in
    HBM; per-launch duration from HIP events around each call on the stream it runs on (one kernel per
    call), against the HBM roofline with the bytes the committed rows move (read + write)."""
    import torch
    import rejection_sampling_verify_16_amd as sv
    from rejection_sampling_verify_16_amd import workloads as W
    w = W.commit_hybrid()
    stream = torch.cuda.current_stream(dev)

    def dev_bytes(a, lead):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.uint8).reshape(*a.shape[:lead], -1)).to(dev)

    tensors = [(dev_bytes(t.verify_state, 3), dev_bytes(t.state_cache, 2)) for t in w.tensors]
    slot = torch.from_numpy(w.state_slot).to(dev)
    acc = torch.from_numpy(w.accept_len).to(dev)
    seq = torch.from_numpy(w.seq_len.copy()).to(dev)
    status = torch.empty(w.B, dtype=torch.int32, device=dev)

    def step():
        sv.spec_commit(tensors, slot, acc, seq_len=seq, status=status, stream=stream)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    n = args.commit_steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    ms_kernel = float(np.mean(per))
    ms_step = e0.elapsed_time(e1) / n
    moved = w.moved_bytes
    gbps = moved / (ms_kernel * 1e-3) / 1e9
    res = {
        "metric": "committed rows/s + state HBM GB/s (% peak)",
        "value": w.B / (ms_step * 1e-3),
        "unit": "committed rows/s",
        "steps": n,
        "ms_per_step": ms_step,
        "config": {"workload": w.name, "B": w.B, "k": w.k, "num_slots": w.num_slots,
                   "tensors": {t.name: {"layers": int(t.verify_state.shape[0]),
                                        "row_bytes": int(t.verify_state[0, 0, 0].nbytes)} for t in w.tensors},
                   "committed_rows": int(((w.accept_len >= 1) & (w.accept_len <= w.k + 1)).sum())},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": load_traffic("commit"), "kernel": "k_commit",
                     "kernel_ms_mean": ms_kernel, "algorithmic_bytes": moved},
    }
    # the same commit by slot numbers: verify would have written each position's state into a scratch slot
    # of a pool holding a committed slot and k+1 scratch slots per row; no state byte moves
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.B * (w.k + 2)).astype(np.int32)
    ss = torch.from_numpy(perm[:w.B].copy()).to(dev)
    ps = torch.from_numpy(perm[w.B:].reshape(w.B, w.k + 1).copy()).to(dev)

    def slot_step():
        sv.spec_commit_slots(ss, ps, acc, w.B * (w.k + 2), seq_len=seq, status=status, stream=stream)

    for _ in range(5):
        slot_step()
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        slot_step()
        b.record(stream)
    torch.cuda.synchronize()
    us_slots = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    res["slot_commit"] = {"kernel": "k_commit_slots", "us_mean": us_slots, "committed_rows_per_s": w.B / (us_slots * 1e-6),
                          "state_bytes_moved": 0,
                          "note": "launch-latency bound: B int32 swaps, no state bytes; same workload and accept lengths"}
    if not args.no_cpu_baseline:
        import oracle
        o = oracle.get()
        host = [(np.ascontiguousarray(t.verify_state).view(np.uint8).reshape(*t.verify_state.shape[:3], -1),
                 np.ascontiguousarray(t.state_cache).view(np.uint8).reshape(*t.state_cache.shape[:2], -1).copy())
                for t in w.tensors]
        seq_h = w.seq_len.copy()
        calls, t0 = 0, time.perf_counter()
        while True:
            o.commit(host, w.state_slot, w.accept_len, seq_h)
            calls += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 5.0) or calls >= 200:
                break
        res["cpu_baseline"] = {"value": w.B * calls / el, "unit": "committed rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"{calls} full commits of the benchmark workload ({w.B} rows each), {el:.1f} s"}
    return res


def _pmc_per_kernel(run_dir, counter):
    """Mean value of one counter per kernel name over the dispatches of a rocprofv3 --pmc CSV run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    vals = {}
    for r in csv.DictReader(open(files[0])):
        if r.get("Counter_Name") != counter:
            continue
        name = r.get("Kernel_Name", "").split("(")[0]
        vals.setdefault(name, []).append(float(r["Counter_Value"]))
    return {k: (float(np.mean(v)), len(v)) for k, v in vals.items()}


def pmc_report(dirs):
    """Markdown table: kernel x counter, mean value per dispatch, over the library's kernels."""
    import csv
    import glob
    vals = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for r in csv.DictReader(open(files[0])):
            name = r.get("Kernel_Name", "").split("(")[0]
            if "sv::" not in name:
                continue
            vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    counters = sorted({c for k in vals.values() for c in k})
    print("| kernel | dispatches | " + " | ".join(counters) + " |")
    print("|---|---|" + "---|" * len(counters))
    for name in sorted(vals):
        n = max(len(v) for v in vals[name].values())
        cells = [f"{np.mean(vals[name][c]):.4g}" if c in vals[name] else "" for c in counters]
        print(f"| {name} | {n} | " + " | ".join(cells) + " |")


def pmc_summary(args):
    """HBM traffic of the statistics kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by
    the ratio of true bytes to the same counter's reading for a plain copy kernel of known size."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.pmc_summary
    copy_bytes = (args.copy_probe_mb or 256) << 20

    def copy_kernel(d):
        # the largest-reading kernel of the copy-probe run is the probe's copy
        return max(d.items(), key=lambda kv: kv[1][0])

    cf_name, (cf_kib, _) = copy_kernel(_pmc_per_kernel(cfetch_dir, "FETCH_SIZE"))
    cw_name, (cw_kib, _) = copy_kernel(_pmc_per_kernel(cwrite_dir, "WRITE_SIZE"))
    f_scale = copy_bytes / (cf_kib * 1024.0)
    w_scale = copy_bytes / (cw_kib * 1024.0)
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")
    path, main_kernel, files = _traffic_target(args.config)
    out = {"config": args.config, "kernel_digest": kernel_digest(files), "copy_probe_bytes": copy_bytes,
           "copy_kernel": cf_name, "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for name, (kib, n) in fetch.items():
        if "sv::" not in name:
            continue
        wk = write.get(name, (0.0, 0))[0]
        out["kernels"][name] = {"fetch_kib_raw": kib, "write_kib_raw": wk, "dispatches": n,
                                "fetch_bytes": kib * 1024.0 * f_scale, "write_bytes": wk * 1024.0 * w_scale}
    k1 = [v for k, v in out["kernels"].items() if main_kernel in k]
    out["kernel"] = main_kernel
    out["bytes_per_launch"] = (k1[0]["fetch_bytes"] + k1[0]["write_bytes"]) if k1 else None
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def kernel_durations(sv, step, n, stream):
    """Mean duration (ms) of each of the library's kernels over n calls, from HIP events that the timed
    entry points record around the launches of each call, on the stream the kernels run on.  step(i, timing)
    makes call i with that KernelTiming.  Returns one mean per kernel the calls launched."""
    import torch
    nk = sv.SPEC_MAX_KERNELS
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nk)] for _ in range(n)]
    for row in evs:  # a first record creates the underlying hipEvent_t
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    used = set()
    for i in range(n):
        t = sv.KernelTiming([e.cuda_event for e in evs[i]])
        step(i, t)
        used.add(t.kernels)
    torch.cuda.synchronize()
    assert len(used) == 1, f"calls launched different kernel counts: {used}"
    nk_used = used.pop()
    per = [[evs[i][2 * j].elapsed_time(evs[i][2 * j + 1]) for i in range(n)] for j in range(nk_used)]
    return tuple(float(np.mean(x)) for x in per)


def cpu_baseline(w, drafts, seconds):
    """The CPU oracle, as it stands, on whole calls of the same workload until ~`seconds` pass."""
    import oracle
    o = oracle.get()
    threads = min(os.cpu_count() or 1, 16)
    calls, t0 = 0, time.perf_counter()
    while True:
        o.spec_verify(w.target, w.draft, drafts, w.temperature, w.top_k, w.top_p, seed=w.seed,
                      offset=w.offsets[calls % len(w.offsets)], num_threads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds or calls >= 1000:
            break
    return {"value": w.B * calls / el, "unit": "verified rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} full calls of the benchmark workload ({w.B} batch rows each), {el:.1f} s"}


if __name__ == "__main__":
    main()
