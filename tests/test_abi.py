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
    if not os.path.exists(sv.LIB_PATH) or os.path.getmtime(sv.LIB_PATH) < max(map(os.path.getmtime, hip_build.SRCS)):
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


def test_timed_entry_points_need_their_timing(L):
    """The timed entry points reject a missing spec_timing_t (or one without events) before any device call,
    and there is no process-wide timing state to set."""
    assert not hasattr(L, "spec_set_kernel_events")
    P = ctypes.c_void_p(16)
    st = L.spec_verify_timed(P, P, 0, P, P, P, P, 2, 2, 1024, 0, 0, P, P, P, None, P, P, 1 << 30, None, None)
    assert st == 1
    t = sv.Timing(None, 0, 0, 0)
    st = L.spec_verify_timed(P, P, 0, P, P, P, P, 0, 2, 1024, 0, 0, P, P, P, None, P, P, 1 << 30, None,
                             ctypes.byref(t))   # B = 0: rejected before any device call
    assert st == 1
    st = L.spec_tree_verify_timed(P, 0, P, P, P, P, P, 2, 3, 1024, 0, 0, P, P, P, P, P, 1 << 30, None, None)
    assert st == 1
    with pytest.raises(ValueError):
        sv.KernelTiming([0] * 3)
    # a path other than auto / staged / resident is rejected before anything else
    bad = sv.Timing(None, 0, 7, 0)
    st = L.spec_verify_timed(P, P, 0, P, P, P, P, 2, 2, 1024, 0, 0, P, P, P, None, P, P, 1 << 30, None,
                             ctypes.byref(bad))
    assert st == 1
    with pytest.raises(ValueError):
        sv.KernelTiming(path=3)
    assert (sv.PATH_AUTO, sv.PATH_STAGED, sv.PATH_RESIDENT) == (0, 1, 2)


def test_smallest_vocabulary(L):
    """V needs only whole 16-byte vectors: 8 bf16 or 4 fp32 logits per row."""
    assert sv.workspace_size(2, 1, 8) > 0
    assert sv.workspace_size(2, 1, 4, sv.SPEC_DTYPE_F32) > 0
    assert sv.workspace_size(2, 1, 4) == 0
    assert L.spec_sample_workspace_size(3, 4, 1) > 0


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


def test_commit_rejects_bad_arguments_before_launch(L):
    """spec_commit's host checks: sizes, tensor count, null pointers, overlapping buffers and aliased
    per-row arrays are rejected before any device call (a valid call then fails only for want of a GPU)."""
    def T(vs, cache, rb=64, layers=2):
        return sv.StateTensor(vs, cache, rb, layers)
    P = lambda a: ctypes.c_void_p(a)
    slot, acc, seq, stat = P(0x10000), P(0x20000), P(0x30000), P(0x40000)
    B, k, ns = 4, 2, 8
    ok = (sv.StateTensor * 2)(T(0x1000000, 0x2000000), T(0x3000000, 0x4000000, 36, 1))

    def call(descs=ok, n=2, s=slot, a=acc, q=seq, st=stat, B=B, k=k, ns=ns):
        return L.spec_commit(descs, n, s, a, q, st, B, k, ns, None)

    for kw in [dict(B=0), dict(B=(1 << 20) + 1), dict(k=-1), dict(k=256), dict(ns=0), dict(n=9), dict(n=-1),
               dict(s=None), dict(a=None), dict(q=acc), dict(st=slot), dict(q=stat)]:
        assert call(**kw) == 1, kw
    assert call(descs=None, n=1) == 1
    bad = [T(0, 0x2000000), T(0x1000000, 0), T(0x1000000, 0x2000000, rb=0), T(0x1000000, 0x2000000, layers=0),
           T(0x1000000, 0x1000000 + 64 * 2 * 4 * 3 - 64),   # cache starts inside the verify buffer
           T(0x1000000, 0x2000000, layers=(1 << 31) // 4)]   # layers * B >= 2^31
    for d in bad:
        assert call(descs=(sv.StateTensor * 1)(d), n=1) == 1, (d.verify_state, d.state_cache, d.row_bytes, d.layers)
    two_caches = (sv.StateTensor * 2)(T(0x1000000, 0x2000000), T(0x3000000, 0x2000000 + 64))
    assert call(descs=two_caches) == 1
    cross = (sv.StateTensor * 2)(T(0x1000000, 0x2000000), T(0x3000000, 0x1000000 + 128, 36, 1))
    assert call(descs=cross) == 1
    # valid arguments: only the device check remains, which fails where no GPU is visible (never run with
    # a GPU present: the pointers above are not device memory)
    import torch
    if torch.cuda.device_count() == 0:
        assert call() == 3
        assert call(n=0, descs=None) == 3


def test_commit_slots_rejects_bad_arguments_before_launch(L):
    """spec_commit_slots' host checks: sizes, null pointers, overlapping per-row arrays."""
    P = lambda a: ctypes.c_void_p(a)
    ss, ps, acc, seq, st = P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x50000)
    B, k, ns = 4, 2, 100

    def call(ss=ss, ps=ps, acc=acc, seq=seq, st=st, B=B, k=k, ns=ns):
        return L.spec_commit_slots(ss, ps, acc, seq, st, B, k, ns, None)

    for kw in [dict(B=0), dict(B=(1 << 20) + 1), dict(k=-1), dict(k=256), dict(ns=0), dict(ss=None), dict(ps=None),
               dict(acc=None), dict(ps=P(0x10000 + 8)), dict(seq=P(0x20000 + 4 * 4 * 3 - 4)), dict(st=acc),
               dict(seq=st)]:
        assert call(**kw) == 1, kw
    import torch
    if torch.cuda.device_count() == 0:
        assert call() == 3
        assert call(seq=None, st=None) == 3


def test_tree_verify_sizes_and_rejects(L):
    """Tree workspace sizes and host-side argument checks (no device call)."""
    assert sv.tree_workspace_size(64, 9, 157184) > 0
    assert sv.tree_workspace_size(1, 1, 1024, sv.SPEC_DTYPE_F32) > 0
    assert sv.tree_workspace_size(4, 64, 4096) > 0
    assert sv.tree_workspace_size(4, 65, 4096) == 0      # more than 64 nodes
    assert sv.tree_workspace_size(4, 0, 4096) == 0
    assert sv.tree_workspace_size(1 << 20, 17, 1024) == 0  # B * N > 2^24
    P = ctypes.c_void_p(16)
    ok = (P, 0, P, P, P, P, P, 4, 9, 1024, 0, 0, P, P, P, P, P, 1 << 30, None)
    for i, bad in [(7, 0), (8, 0), (8, 65), (9, 1001), (11, 1 << 32), (0, None), (2, None), (13, None),
                   (0, ctypes.c_void_p(18))]:
        args = list(ok)
        args[i] = bad
        assert L.spec_tree_verify(*args) == 1, (i, bad)
    args = list(ok)
    args[16] = None                                       # no workspace
    assert L.spec_tree_verify(*args) == 2
