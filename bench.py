"""Benchmark of libspecverify on one MI355X: verified rows/s and logit bandwidth vs the HBM roofline.

One step = one spec_verify() call over one batch of synthetic inputs already resident in HBM
(default workload: B=64, k=2, V=157184, bf16, mixed temperature / top-k / top-p per row).
Input sets are rotated so that the working set exceeds the 256 MB Infinity Cache.

Prints one JSON line.  Besides the throughput (whole timed region) it reports
  samples:      the timed calls split into --samples equal runs: median / min / max per call;
  roofline:     the statistics kernel (it streams every logit once): algorithmic logit bytes per
                launch / its average duration (HIP events the library records around each of its
                kernels, over a second pass of the same calls), against the 8 TB/s HBM peak;
  read_stream:  a plain read of the same number of bytes (the probe library's 16-byte loads), the
                bandwidth one pass over the logits can reach on this GPU;
  traffic:      HBM bytes per call from the committed PMC summary (when taken on these sources):
                each kernel's and the whole call's, against the algorithmic logit bytes;
  cpu_baseline: the CPU oracle timed on this host on a bounded sample of the same workload, with the
                host's core count, the threads used and a one-thread figure; and the oracle's margin rows
                (outcomes a correct rounding could change, exempt from bit-exact comparison) per workload;
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
KERNEL_SRC = [os.path.join(_CSRC, f) for f in ("specverify.hip", "sv_common.h", "sv_resident.h")]
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


def _traffic_target(config: str, resident: bool = False):
    """(summary file, kernel name, sources) of the dominant kernel of a workload (on the resident path: the
    resident kernel's own summary)."""
    if config == "commit":
        return os.path.join(ROOT, "profiles", "traffic_commit.json"), "k_commit", COMMIT_SRC
    if config == "tree":
        return os.path.join(ROOT, "profiles", "traffic_tree.json"), "k1_stats", KERNEL_SRC
    if resident:
        return os.path.join(ROOT, "profiles", f"traffic_config{config}_resident.json"), "kr_verify", KERNEL_SRC
    return os.path.join(ROOT, "profiles", f"traffic_config{config}.json"), "k1_stats", KERNEL_SRC


KERNELS_STAGED = ("k1_stats", "k1_rows", "k5_verify")
KERNELS_RESIDENT = ("kr_verify",)


def load_traffic(config: str, knames=None):
    """HBM traffic per call from the committed PMC summary, if it was taken on these kernel sources and on
    the kernels the call launches: {"kernel_bytes": the first kernel's, "call_bytes": all of them,
    "per_kernel": {name: bytes}}, or None."""
    path, main, files = _traffic_target(config, resident=bool(knames) and tuple(knames) == KERNELS_RESIDENT)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_digest") != kernel_digest(files):
        return None
    per = {}
    for name, v in t.get("kernels", {}).items():
        short = name.split("<")[0].split("::")[-1]
        per[short] = v["fetch_bytes"] + v["write_bytes"]
    want = list(knames) if knames else [main]
    if any(kn not in per for kn in want):
        return None
    return {"kernel_bytes": per[want[0]], "call_bytes": float(sum(per[kn] for kn in want)),
            "per_kernel": {kn: per[kn] for kn in want}, "file": path}


def _kernel_bytes(tr):
    return tr["kernel_bytes"] if tr else None


def timed_calls(step, n, samples, stream):
    """n calls back to back in one timed region (device events around it), with events between `samples`
    equal runs of them: (total ms, ms per call, host wall seconds, {median / min / max us per call})."""
    import torch
    samples = max(1, min(samples, n))
    bounds = [round(j * n / samples) for j in range(samples + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(samples + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record(stream)
    for j in range(samples):
        for i in range(bounds[j], bounds[j + 1]):
            step(i)
        evs[j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total = evs[0].elapsed_time(evs[-1])
    per = [evs[j].elapsed_time(evs[j + 1]) / (bounds[j + 1] - bounds[j]) * 1e3 for j in range(samples)
           if bounds[j + 1] > bounds[j]]
    return total, total / n, wall, {"runs": len(per), "calls_per_run": n // samples,
                                    "us_per_call_median": float(np.median(per)), "us_per_call_min": float(min(per)),
                                    "us_per_call_max": float(max(per))}


def read_stream_reference(dev, nbytes, runs=8, per_run=10):
    """Bandwidth of a plain 16-byte-load read of nbytes from the probe library, timed the way the verify
    calls are: `runs` runs of `per_run` launches back to back between events, rotating over buffers that
    together exceed the last-level cache; the median run gives the figure.  None if the probe is not built."""
    import ctypes
    import torch
    probe = os.path.join(ROOT, "rejection_sampling_verify_16_amd", "libsvprobe.so")
    if not os.path.exists(probe):
        return None
    L = ctypes.CDLL(probe)
    L.probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    L.probe_read_stream.restype = ctypes.c_int
    nvec = nbytes // 16
    nbuf = max(2, math.ceil(ROTATE_BYTES / max(nbytes, 1)))
    bufs = [torch.empty(nvec * 16, dtype=torch.uint8, device=dev).fill_(j + 1) for j in range(nbuf)]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * 8
    sink = torch.zeros(blocks, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch(i):
        return L.probe_read_stream(ctypes.c_void_p(bufs[i % nbuf].data_ptr()), nvec, ctypes.c_void_p(sink.data_ptr()),
                                   blocks, ctypes.c_void_p(stream.cuda_stream))

    for i in range(2 * nbuf):  # warm-up
        if launch(i) != 0:
            return None
    torch.cuda.synchronize()
    per = []
    i = 0
    for _ in range(runs):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(per_run):
            if launch(i) != 0:
                return None
            i += 1
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / per_run)
    ms = float(np.median(per))
    del bufs
    torch.cuda.empty_cache()
    gbps = nvec * 16 / (ms * 1e-3) / 1e9
    return {"bytes": nvec * 16, "us_median": ms * 1e3, "GBps": gbps, "pct_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
            "kernel": "k_read_stream", "grid": [blocks, 256], "timing": f"{runs} runs of {per_run} back-to-back launches"}


def occupancy_probe(dev, spin_ticks=2000):
    """Most 256-thread workgroups alive at once, per register reservation, from the probe library's spin
    kernel (4 workgroups per CU more than can fit, each waiting spin_ticks of the 100 MHz wall clock).  The
    compiler's own occupancy report says 8 waves per SIMD for all but the 102-SGPR and 69-VGPR variants (7)."""
    import ctypes
    import torch
    probe = os.path.join(ROOT, "rejection_sampling_verify_16_amd", "libsvprobe.so")
    L = ctypes.CDLL(probe)
    L.probe_occupancy.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_ulonglong, ctypes.c_void_p]
    L.probe_occupancy.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * 12
    out = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    names = ["plain", "80 SGPRs", "82 SGPRs", "102 SGPRs", "61 VGPRs", "69 VGPRs"]
    res = {"cus": cus, "workgroups": blocks, "threads": 256}
    for v, name in enumerate(names):
        out.zero_()
        assert L.probe_occupancy(v, ctypes.c_void_p(out.data_ptr()), blocks, spin_ticks, None) == 0
        torch.cuda.synchronize()
        t = out.cpu().numpy().reshape(blocks, 2)
        ev = np.concatenate([np.stack([t[:, 0], np.ones(blocks)], 1), np.stack([t[:, 1], -np.ones(blocks)], 1)])
        ev = ev[np.lexsort((ev[:, 1], ev[:, 0]))]  # ends before starts at equal stamps
        live = int(np.cumsum(ev[:, 1]).max())
        res[name] = {"max_resident": live, "per_cu": live / cus}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="3",
                    help="workload: 1, 2, 3, 4a, 4b, 5 (with --pmc-summary also: commit, tree)")
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
    ap.add_argument("--path", choices=["auto", "staged", "resident"], default="auto",
                    help="the library's path for the verify calls (auto: its own choice)")
    ap.add_argument("--samples", type=int, default=10, help="runs the timed calls are split into (median / min)")
    ap.add_argument("--no-read-stream", action="store_true", help="skip the read-only stream reference")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times (PMC calibration of "
                         "WRITE_SIZE; with --read-probe: a plain read instead, for FETCH_SIZE)")
    ap.add_argument("--occupancy-probe", action="store_true",
                    help="only report how many workgroups the hardware holds at once per register reservation")
    ap.add_argument("--read-probe", action="store_true",
                    help="with --copy-probe-mb: the probe library's read-only stream instead of the copy")
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
    if args.occupancy_probe:
        print(json.dumps({"occupancy": occupancy_probe(dev)}), flush=True)
        return
    if args.copy_probe_mb and args.read_probe:
        n = args.copy_probe_mb << 20
        rs = read_stream_reference(dev, n, runs=2, per_run=5)
        print(json.dumps({"read_probe_bytes": n, "result": rs}), flush=True)
        return
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

    path = {"auto": sv.PATH_AUTO, "staged": sv.PATH_STAGED, "resident": sv.PATH_RESIDENT}[args.path]

    def step(i, timing=None):
        t_, d_ = sets[i % n_sets]
        if timing is None and path != sv.PATH_AUTO:
            timing = sv.KernelTiming(path=path)
        elif timing is not None:
            timing.path = path
        sv.spec_verify(t_, d_, drafts, T, K, P, seed=w.seed, offset=offsets[i % len(offsets)], out=out,
                       workspace=ws, stream=stream, raw=args.raw_logprobs, timing=timing)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` calls, with events between equal runs of them ----
    ms, ms_per_step, wall, samples = timed_calls(step, args.steps, args.samples, stream)

    # ---- per-kernel durations: HIP events recorded by the library around each of its kernels,
    # on the stream the kernels run on, over a second pass of the same `steps` calls ----
    kms = kernel_durations(sv, step, args.steps, stream)
    knames = KERNELS_RESIDENT if len(kms) == 1 else KERNELS_STAGED[:len(kms)]
    logit_bytes = w.logit_bytes
    draft_pos_bytes = w.B * 2 * w.k * w.V * (2 if bf16 else 4)  # rows K5 re-reads (bonus row aside)
    k1_ms = kms[0]  # the kernel that streams every logit once: K1, or the resident kernel
    k1_gbps = logit_bytes / (k1_ms * 1e-3) / 1e9
    rows_per_s = B / (ms_per_step * 1e-3)
    tr = load_traffic(args.config, knames)

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
                   "raw_logprobs": bool(args.raw_logprobs), "path": args.path,
                   "rotating_input_sets": n_sets},
        "samples": samples,
        "logits_GBps": logit_bytes / (ms_per_step * 1e-3) / 1e9,
        "pct_hbm_peak": 100.0 * logit_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "wall_s": wall,
        "roofline": {
            "bound": "hbm",
            "achieved": k1_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": k1_gbps / HBM_PEAK_GBPS,
            "traffic": tr["kernel_bytes"] if tr else None,
            "kernel": knames[0],
            "kernel_ms_mean": k1_ms,
            "algorithmic_bytes": logit_bytes,
        },
        "kernels": {knames[j]: {"ms_mean": kms[j]} for j in range(len(kms))},
    }
    result["kernels"][knames[0]].update({"bytes": logit_bytes, "GBps": k1_gbps})
    if "k5_verify" in result["kernels"]:
        # K5 streams the draft-position rows of batch rows it cannot finish from recorded candidates; this
        # is its traffic when every row is streamed (an upper bound)
        result["kernels"]["k5_verify"]["bytes_all_rows_streamed"] = draft_pos_bytes
    if tr:
        result["traffic"] = {"whole_call_bytes": tr["call_bytes"], "algorithmic_bytes": logit_bytes,
                             "whole_call_ratio": tr["call_bytes"] / logit_bytes, "per_kernel": tr["per_kernel"],
                             "source": os.path.relpath(tr["file"], ROOT)}
    else:
        result["traffic"] = None
    if not args.no_read_stream:
        rs = read_stream_reference(dev, logit_bytes)
        if rs:
            rs["call_pct_of_read_stream"] = 100.0 * result["logits_GBps"] / rs["GBps"]
        result["read_stream"] = rs

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
        _, ms, _, samples = timed_calls(step, n, args.samples, stream)
        kms = kernel_durations(sv, step, n, stream)
        knames = KERNELS_RESIDENT if len(kms) == 1 else KERNELS_STAGED[:len(kms)]
        acc = out["accept_len"].float().mean().item()
        gbps = w.logit_bytes / (ms * 1e-3) / 1e9
        k1_gbps = w.logit_bytes / (kms[0] * 1e-3) / 1e9
        res[name] = {
            "workload": w.name, "B": w.B, "k": w.k, "V": w.V, "dtype": w.dtype, "calls": n,
            "us_per_call": ms * 1e3, "samples": samples, "verified_rows_per_s": w.B / (ms * 1e-3),
            "logit_bytes_per_call": w.logit_bytes, "logits_GBps": gbps, "pct_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
            "kernels_us": {knames[j]: kms[j] * 1e3 for j in range(len(kms))},
            "stream_kernel_roofline_frac": k1_gbps / HBM_PEAK_GBPS, "mean_accept_len": acc,
        }
        tr = load_traffic(name, knames)
        if tr:
            res[name]["traffic"] = {"whole_call_bytes": tr["call_bytes"], "whole_call_ratio": tr["call_bytes"] / w.logit_bytes,
                                    "per_kernel": tr["per_kernel"], "source": os.path.relpath(tr["file"], ROOT)}
        if not args.no_cpu_baseline:
            res[name]["oracle_margin"] = oracle_margins(w, drafts.cpu().numpy())
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
    _, ms, _, samples = timed_calls(step, n, args.samples, stream)
    k1_ms, km_ms, kt_ms = kernel_durations(sv, step, n, stream)
    gbps = w.logit_bytes / (k1_ms * 1e-3) / 1e9
    acc = out["accept_len"].cpu().numpy()
    res = {
        "metric": "verified rows/s (draft trees)",
        "value": w.B / (ms * 1e-3),
        "unit": "verified rows/s",
        "steps": n,
        "ms_per_step": ms,
        "samples": samples,
        "dtype": "bf16",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "V": w.V, "parents": list(W.EAGLE_TREE_9),
                   "logit_bytes_per_step": w.logit_bytes, "rotating_input_sets": n_sets},
        "mean_accept_len": float(acc.mean()),
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None, "kernel": "k1_stats (tree rows)",
                     "kernel_ms_mean": k1_ms, "algorithmic_bytes": w.logit_bytes},
        "kernels": {"k1_stats": {"ms_mean": k1_ms}, "k1_rows": {"ms_mean": km_ms}, "k_tree": {"ms_mean": kt_ms}},
    }
    tr = load_traffic("tree", ("k1_stats", "k1_rows", "k_tree"))
    if tr:
        res["roofline"]["traffic"] = tr["kernel_bytes"]
        res["traffic"] = {"whole_call_bytes": tr["call_bytes"], "algorithmic_bytes": w.logit_bytes,
                          "whole_call_ratio": tr["call_bytes"] / w.logit_bytes, "per_kernel": tr["per_kernel"],
                          "source": os.path.relpath(tr["file"], ROOT)}
    else:
        res["traffic"] = None
    if not args.no_cpu_baseline:
        import oracle
        o = oracle.get()
        threads = min(host_cores(), 16)
        calls, t0 = 0, time.perf_counter()
        while True:
            o.tree_verify(w.target, w.parent, w.node_tokens, w.temperature, w.top_k, w.top_p, seed=w.seed,
                          offset=calls, num_threads=threads)
            calls += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 5.0) or calls >= 200:
                break
        res["cpu_baseline"] = {"value": w.B * calls / el, "unit": "verified rows/s", "cores": threads,
                               "host_cores": host_cores(), "kind": "oracle",
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
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": _kernel_bytes(load_traffic("commit")), "kernel": "k_commit",
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


def _kernel_name(full: str) -> str:
    """A kernel's name without its parameter list (and without an anonymous-namespace prefix)."""
    full = full.replace("(anonymous namespace)::", "")
    return full.split("(")[0]


def _pmc_per_kernel(run_dir, counter):
    """Median value of one counter per kernel name over the dispatches of a rocprofv3 --pmc CSV run (the
    median: a run's first dispatch of a kernel can belong to a different-sized call, such as the drafts'
    own sampling call)."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    vals = {}
    for r in csv.DictReader(open(files[0])):
        if r.get("Counter_Name") != counter:
            continue
        name = _kernel_name(r.get("Kernel_Name", ""))
        vals.setdefault(name, []).append(float(r["Counter_Value"]))
    return {k: (float(np.median(v)), len(v)) for k, v in vals.items()}


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
            name = _kernel_name(r.get("Kernel_Name", ""))
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
    """HBM traffic per kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by the ratio of
    true bytes to the same counter's reading for a plain kernel of known size (the largest-reading kernel of
    each calibration run: a read-only stream for FETCH_SIZE, a copy for WRITE_SIZE, both --copy-probe-mb)."""
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
    path_opt = getattr(args, "path", "auto")
    path, main_kernel, files = _traffic_target(args.config, resident=path_opt == "resident")
    out = {"config": args.config, "path": path_opt, "kernel_digest": kernel_digest(files), "copy_probe_bytes": copy_bytes,
           "copy_kernel": cf_name, "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_scale_kernel": cf_name, "write_scale_kernel": cw_name, "kernels": {}}
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


# Margin tolerances of the parity bar: accept test |u - p/q|, Gumbel top-2 gap, top-p |M / Z_K - P|.
MARGIN_ACCEPT, MARGIN_GAP, MARGIN_TOPP = 1e-5, 1e-5, 1e-6


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def oracle_margins(w, drafts, offsets=None):
    """The CPU oracle's margin rows of a workload (cpu_baseline leg): batch rows whose outcome a correct
    rounding could change (exempt from the bit-exact comparison, checked against the oracle's alternative
    resolutions by the parity tests), and its sentinel rows, over the given offsets (default: the first)."""
    import oracle
    o = oracle.get()
    offs = offsets if offsets is not None else [w.offsets[0]]
    margin = sentinel = 0
    t0 = time.perf_counter()
    for off in offs:
        r = o.spec_verify(w.target, w.draft, drafts, w.temperature, w.top_k, w.top_p, seed=w.seed, offset=off,
                          num_threads=min(host_cores(), 16))
        m = r.margin_rows(MARGIN_ACCEPT, MARGIN_GAP, MARGIN_TOPP) & ~r.sentinel
        margin += int(m.sum())
        sentinel += int(r.sentinel.sum())
    return {"margin_rows": margin, "sentinel_rows": sentinel, "batch_rows": w.B * len(offs), "offsets": len(offs),
            "tolerances": {"accept": MARGIN_ACCEPT, "gumbel_gap": MARGIN_GAP, "top_p": MARGIN_TOPP},
            "seconds": time.perf_counter() - t0}


def cpu_baseline(w, drafts, seconds):
    """The CPU oracle, as it stands, on whole calls of the same workload until ~`seconds` pass (all usable
    host cores, at most 16), a one-thread figure on a bounded sample of its batch rows, and the oracle's
    margin rows of the workload."""
    import oracle
    o = oracle.get()
    cores = host_cores()
    threads = min(cores, 16)
    calls, t0 = 0, time.perf_counter()
    while True:
        o.spec_verify(w.target, w.draft, drafts, w.temperature, w.top_k, w.top_p, seed=w.seed,
                      offset=w.offsets[calls % len(w.offsets)], num_threads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds or calls >= 1000:
            break
    # one thread, on the first few batch rows (the same rows every run)
    nb = min(w.B, 8)
    calls1, t1 = 0, time.perf_counter()
    while True:
        o.spec_verify(w.target[:nb], w.draft[:nb], drafts[:nb], w.temperature[:nb], w.top_k[:nb], w.top_p[:nb],
                      seed=w.seed, offset=w.offsets[0], num_threads=1)
        calls1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= min(seconds, 5.0) or calls1 >= 1000:
            break
    return {"value": w.B * calls / el, "unit": "verified rows/s", "cores": threads, "host_cores": cores,
            "kind": "oracle",
            "sample": f"{calls} full calls of the benchmark workload ({w.B} batch rows each), {el:.1f} s, "
                      f"{threads} threads",
            "one_thread": {"value": nb * calls1 / el1, "unit": "verified rows/s", "cores": 1,
                           "sample": f"{calls1} calls on the first {nb} batch rows, {el1:.1f} s"},
            "margin": oracle_margins(w, drafts)}


if __name__ == "__main__":
    main()
