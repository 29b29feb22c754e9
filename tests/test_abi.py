"""The C-ABI library loads and exports every function include/*.h declares; host-side checks
that return before any GPU call.  CPU only."""
import ctypes
import glob
import os
import re

import pytest

import rejection_sampling_verify_16_amd as sv
from rejection_sampling_verify_16_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sv.LIB_PATH) or os.path.getmtime(sv.LIB_PATH) < os.path.getmtime(hip_build.SRC):
        hip_build.build()
    return sv.lib()


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(spec_\w+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert {"spec_verify", "spec_verify_workspace_size", "spec_verify_status_string", "spec_sample",
            "spec_sample_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared but not exported"


def test_workspace_sizes(L):
    assert sv.workspace_size(64, 2, 157184) > 0
    assert sv.workspace_size(256, 4, 248320) > 0
    assert sv.workspace_size(1, 1, 1024, sv.SPEC_DTYPE_F32) > 0
    assert sv.workspace_size(0, 2, 157184) == 0        # B < 1
    assert sv.workspace_size(4, 0, 157184) == 0        # k < 1
    assert sv.workspace_size(4, 9, 157184) == 0        # k > 8
    assert sv.workspace_size(4, 2, 1001) == 0          # bf16 needs V % 8 == 0
    assert sv.workspace_size(4, 2, 1002, sv.SPEC_DTYPE_F32) == 0
    assert L.spec_sample_workspace_size(16, 4096, 0) > 0


def test_kernel_event_hook_arguments(L):
    """The benchmark hook checks its count, and NULL turns it off."""
    assert L.spec_set_kernel_events(None, 0) == 0
    arr = (ctypes.c_void_p * 3)()
    assert L.spec_set_kernel_events(arr, 3) == 1


def test_status_strings(L):
    for s in range(5):
        assert L.spec_verify_status_string(s)
    assert L.spec_verify_status_string(99) == b"unknown status"


def test_invalid_scalars_rejected_before_launch(L):
    # invalid sizes and offsets are rejected on the host, before any device call
    P = ctypes.c_void_p(16)
    for B, k, V, off in [(0, 2, 1024, 0), (2, 0, 1024, 0), (2, 2, 1000 + 4, 0), (2, 2, 1024, 1 << 32)]:
        st = L.spec_verify(P, P, 0, P, P, P, P, B, k, V, 0, off, P, P, P, P, P, 1 << 30, None)
        assert st == 1
    # null pointers
    st = L.spec_verify(None, P, 0, P, P, P, P, 2, 2, 1024, 0, 0, P, P, P, P, P, 1 << 30, None)
    assert st == 1
    # misaligned logits
    st = L.spec_verify(ctypes.c_void_p(18), P, 0, P, P, P, P, 2, 2, 1024, 0, 0, P, P, P, P, P, 1 << 30, None)
    assert st == 1


def test_raw_variant_rejects_missing_output(L):
    # spec_verify_raw needs its extra output; size checks match spec_verify's, all before any device call
    P = ctypes.c_void_p(16)
    st = L.spec_verify_raw(P, P, 0, P, P, P, P, 2, 2, 1024, 0, 0, P, P, P, None, P, P, 1 << 30, None)
    assert st == 1
    st = L.spec_verify_raw(P, P, 0, P, P, P, P, 0, 2, 1024, 0, 0, P, P, P, P, P, P, 1 << 30, None)
    assert st == 1
