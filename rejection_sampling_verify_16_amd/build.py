"""Build libspecverify.so (hipcc, gfx950) in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("specverify.hip", "commit.hip")]
OUT = os.path.join(HERE, "libspecverify.so")
# test and benchmark probes of the device helpers: a library of their own, never linked into the product
PROBE_SRCS = [os.path.join(HERE, "csrc", "probe.hip")]
PROBE_OUT = os.path.join(HERE, "libsvprobe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # no packed-fp32 instructions are generated (they are avoided on this target)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc(srcs, out, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", out + ".tmp", *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    if verbose:
        print(r.stderr)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    """Builds the product library and, separately, the probe library; returns the product's path."""
    _hipcc(PROBE_SRCS, PROBE_OUT, verbose)
    return _hipcc(SRCS, OUT, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
