"""Host logic of bench.py (no GPU): the kernel-source digest that keys the traffic summaries, the PMC traffic
scaling against kernels of known size (per-dispatch medians), the whole-call traffic, the sampled timing helper's
arithmetic and the one-GPU guard."""
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write(path, text):
    with open(path, "w") as f:
        f.write(text)
    return str(path)


def test_kernel_digest_ignores_comments_and_layout(tmp_path):
    a = _write(tmp_path / "a.hip", "int f(int x) {  // doubles\n  return 2 * x; /* twice */\n}\n")
    b = _write(tmp_path / "b.hip", "int f(int x)\n{\n    return 2*x;\n}\n")
    c = _write(tmp_path / "c.hip", "int f(int x) { return 3 * x; }\n")
    assert bench.kernel_digest([a]) == bench.kernel_digest([b])
    assert bench.kernel_digest([a]) != bench.kernel_digest([c])


def _pmc_dir(root, name, counter, rows):
    d = root / name
    d.mkdir()
    lines = ["Kernel_Name,Counter_Name,Counter_Value"]
    for kernel, value in rows:
        lines.append(f'"{kernel}",{counter},{value}')
    _write(d / "run_counter_collection.csv", "\n".join(lines) + "\n")
    return str(d)


def test_pmc_summary_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    k1 = "void sv::k1_stats<sv::BF16, 8, false>(sv::Params)"
    k5 = "void sv::k5_verify<sv::BF16, 2, false>(sv::Params)"
    copy = "__amd_rocclr_copyBuffer"
    mib = 256
    # three dispatches of K1, the first a smaller call (the drafts' own sampling call): the median is taken
    fetch = _pmc_dir(tmp_path, "fetch", "FETCH_SIZE", [(k1, 400.0), (k1, 1000.0), (k1, 1200.0), (k5, 50.0)])
    write = _pmc_dir(tmp_path, "write", "WRITE_SIZE", [(k1, 4.0), (k1, 20.0), (k1, 30.0), (k5, 2.0)])
    # the copy reads half and writes all of the bytes it moves, as the MI355X counters report
    cfetch = _pmc_dir(tmp_path, "cfetch", "FETCH_SIZE", [(copy, mib * 512.0), ("other", 1.0),
                                                          ("(anonymous namespace)::k_other(int)", 2.0)])
    cwrite = _pmc_dir(tmp_path, "cwrite", "WRITE_SIZE", [(copy, mib * 1024.0)])
    out = tmp_path / "traffic.json"
    src = _write(tmp_path / "k.hip", "int k;\n")
    monkeypatch.setattr(bench, "_traffic_target", lambda config, resident=False: (str(out), "k1_stats", [src]))
    args = types.SimpleNamespace(pmc_summary=[fetch, write, cfetch, cwrite], copy_probe_mb=mib, config="3", path="auto")
    bench.pmc_summary(args)
    t = json.load(open(out))
    assert t["copy_kernel"] == copy
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    k = t["kernels"]["void sv::k1_stats<sv::BF16, 8, false>"]
    assert k["dispatches"] == 3
    assert k["fetch_bytes"] == pytest.approx(1000.0 * 1024 * 2.0)
    assert k["write_bytes"] == pytest.approx(20.0 * 1024 * 1.0)
    assert t["bytes_per_launch"] == pytest.approx(1000.0 * 1024 * 2.0 + 20.0 * 1024)
    assert t["kernel_digest"] == bench.kernel_digest([src])
    # the dominant kernel's bytes, and a whole call's over the kernels it launches
    tr = bench.load_traffic("3")
    assert tr["kernel_bytes"] == pytest.approx(t["bytes_per_launch"])
    call = bench.load_traffic("3", ("k1_stats", "k5_verify"))
    assert call["call_bytes"] == pytest.approx(1000.0 * 1024 * 2.0 + 20.0 * 1024 + 50.0 * 1024 * 2.0 + 2.0 * 1024)
    assert bench.load_traffic("3", ("k1_stats", "k1_rows")) is None  # a kernel without counters: no figure
    # a summary taken on other kernel code is not used
    _write(tmp_path / "k.hip", "int k2;\n")
    assert bench.load_traffic("3") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
