"""MI355X-native speculative-decoding verify sampler: Python binding of libspecverify.

The binding only marshals arguments: torch tensors (device memory and streams) are turned
into raw pointers and passed to the C ABI declared in ``include/specverify.h``.  Every step
of the verify method runs in the library's HIP kernels.  If the library has not been built
the calls raise; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

SPEC_DTYPE_BF16 = 0
SPEC_DTYPE_F32 = 1
SPEC_MAX_KERNELS = 3  # kernels one call launches at most (spec_timing_t.kernels says how many it did)
STATUS = {0: "SPEC_OK", 1: "SPEC_ERR_INVALID_ARGUMENT", 2: "SPEC_ERR_WORKSPACE",
          3: "SPEC_ERR_UNSUPPORTED_DEVICE", 4: "SPEC_ERR_LAUNCH"}

SPEC_COMMIT_MAX_TENSORS = 8

_lib = None


class StateTensor(ctypes.Structure):
    """spec_state_tensor_t: one stateful tensor of the commit step, stacked across layers."""
    _fields_ = [("verify_state", ctypes.c_void_p), ("state_cache", ctypes.c_void_p),
                ("row_bytes", ctypes.c_int64), ("layers", ctypes.c_int32)]


PATH_AUTO, PATH_STAGED, PATH_RESIDENT = 0, 1, 2  # SPEC_PATH_*


class Timing(ctypes.Structure):
    """spec_timing_t: per-call kernel timing (events[2j] / events[2j+1] around kernel j)."""
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("kernels", ctypes.c_int32), ("path", ctypes.c_int32),
                ("wait_limit", ctypes.c_uint64)]


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str = "spec_verify"):
        super().__init__(f"{what} failed: {STATUS.get(status, status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        # torch ships its own HIP runtime; loading torch first makes the library bind that same runtime
        # (loaded first, the library would bind the system one and torch would then share it)
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        P, I32, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
        L.spec_verify_workspace_size.argtypes = [I32, I32, I32, ctypes.c_int]
        L.spec_verify_workspace_size.restype = SZ
        L.spec_verify.argtypes = [P, P, ctypes.c_int, P, P, P, P, I32, I32, I32, U64, U64, P, P, P, P, P, SZ, P]
        L.spec_verify_raw.argtypes = [P, P, ctypes.c_int, P, P, P, P, I32, I32, I32, U64, U64, P, P, P, P, P, P,
                                      SZ, P]
        L.spec_verify.restype = ctypes.c_int
        L.spec_verify_raw.restype = ctypes.c_int
        L.spec_sample_workspace_size.argtypes = [I32, I32, ctypes.c_int]
        L.spec_sample_workspace_size.restype = SZ
        L.spec_sample.argtypes = [P, ctypes.c_int, P, P, P, P, P, I32, I32, U64, U64, P, P, P, SZ, P]
        L.spec_sample.restype = ctypes.c_int
        L.spec_verify_status_string.argtypes = [ctypes.c_int]
        L.spec_verify_status_string.restype = ctypes.c_char_p
        L.spec_tree_verify_workspace_size.argtypes = [I32, I32, I32, ctypes.c_int]
        L.spec_tree_verify_workspace_size.restype = SZ
        L.spec_tree_verify.argtypes = [P, ctypes.c_int, P, P, P, P, P, I32, I32, I32, U64, U64, P, P, P, P, P, SZ, P]
        L.spec_tree_verify.restype = ctypes.c_int
        L.spec_commit.argtypes = [ctypes.POINTER(StateTensor), I32, P, P, P, P, I32, I32, I32, P]
        L.spec_commit.restype = ctypes.c_int
        L.spec_commit_slots.argtypes = [P, P, P, P, P, I32, I32, I32, P]
        L.spec_commit_slots.restype = ctypes.c_int
        L.spec_verify_noalloc.argtypes = [P, P, ctypes.c_int, P, P, P, P, I32, I32, I32, U64, U64, P, P, P, P, P]
        L.spec_verify_noalloc.restype = ctypes.c_int
        L.spec_verify_timed.argtypes = [P, P, ctypes.c_int, P, P, P, P, I32, I32, I32, U64, U64, P, P, P, P, P, P,
                                        SZ, P, ctypes.POINTER(Timing)]
        L.spec_verify_timed.restype = ctypes.c_int
        L.spec_tree_verify_timed.argtypes = [P, ctypes.c_int, P, P, P, P, P, I32, I32, I32, U64, U64, P, P, P, P, P,
                                             SZ, P, ctypes.POINTER(Timing)]
        L.spec_tree_verify_timed.restype = ctypes.c_int
        _lib = L
    return _lib


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SPEC_DTYPE_BF16
    if t.dtype == torch.float32:
        return SPEC_DTYPE_F32
    raise TypeError("logits must be torch.bfloat16 or torch.float32")


def workspace_size(B: int, k: int, V: int, dtype: int = SPEC_DTYPE_BF16) -> int:
    return int(lib().spec_verify_workspace_size(B, k, V, dtype))


def make_workspace(B: int, k: int, V: int, dtype: int = SPEC_DTYPE_BF16, device="cuda"):
    """A device workspace for spec_verify (reusable across calls on one stream; it needs no clearing,
    zero-filled here only so that a fresh one holds no stale bytes)."""
    import torch
    n = workspace_size(B, k, V, dtype)
    if n == 0:
        raise ValueError("invalid sizes for spec_verify")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def alloc_outputs(B: int, k: int, device="cuda", raw: bool = False):
    import torch
    out = dict(tokens=torch.empty((B, k + 1), dtype=torch.int32, device=device),
               accept_len=torch.empty((B,), dtype=torch.int32, device=device),
               logprobs=torch.empty((B, k + 1), dtype=torch.float32, device=device),
               alpha=torch.empty((B, k), dtype=torch.float32, device=device))
    if raw:
        out["raw_logprobs"] = torch.empty((B, k + 1), dtype=torch.float32, device=device)
    return out


class KernelTiming:
    """Per-call instrumentation: 2 * SPEC_MAX_KERNELS raw hipEvent_t handles (ints, created with timing
    enabled) or None, the path to take (``path``: PATH_AUTO, PATH_STAGED or PATH_RESIDENT) and a bound on
    the one-launch path's waits (``wait_limit``, 100 MHz ticks; 0 = the library's default).  Passed as
    ``timing=`` to spec_verify / spec_tree_verify, it makes the call go through the timed entry point, which
    records events[2j] / events[2j+1] around kernel j; afterwards ``kernels`` holds how many kernels the call
    launched (1: the resident path)."""

    def __init__(self, events=None, wait_limit: int = 0, path: int = 0):
        if events is not None and len(events) != 2 * SPEC_MAX_KERNELS:
            raise ValueError(f"events: {2 * SPEC_MAX_KERNELS} hipEvent_t handles")
        if path not in (PATH_AUTO, PATH_STAGED, PATH_RESIDENT):
            raise ValueError("path: PATH_AUTO, PATH_STAGED or PATH_RESIDENT")
        self._arr = None if events is None else (ctypes.c_void_p * len(events))(*events)
        self.wait_limit = int(wait_limit)
        self.path = int(path)
        self.kernels = 0

    def _struct(self):
        ev = None if self._arr is None else ctypes.cast(self._arr, ctypes.POINTER(ctypes.c_void_p))
        return Timing(ev, 0, self.path, self.wait_limit)


def spec_verify(target_logits, draft_logits, draft_tokens, temperature, top_k, top_p, seed: int = 0,
                offset: int = 0, out=None, workspace=None, stream=None, raw: bool = False, timing=None):
    """Run the verify step on device tensors; returns a dict of output tensors.

    target_logits [B, k+1, V] and draft_logits [B, k, V] (bf16 or fp32, contiguous, same device),
    draft_tokens int32 [B, k], temperature float32 [B], top_k int32 [B], top_p float32 [B].
    ``out`` (from alloc_outputs) and ``workspace`` (from make_workspace) may be passed in to
    avoid allocations; ``stream`` defaults to torch's current stream.  ``raw=True`` calls
    spec_verify_raw and adds "raw_logprobs" (ln softmax of the unprocessed target logits at each
    committed token).  ``timing`` (a KernelTiming) calls spec_verify_timed instead, which also records
    its events around the call's kernels.
    """
    import torch
    B, k1, V = target_logits.shape
    k = k1 - 1
    dt = _dtype_code(target_logits)
    for t in (target_logits, draft_logits, draft_tokens, temperature, top_k, top_p):
        if not t.is_contiguous():
            raise ValueError("all inputs must be contiguous")
    if out is None:
        out = alloc_outputs(B, k, target_logits.device, raw=raw)
    if raw and "raw_logprobs" not in out:
        raise ValueError("raw=True needs out['raw_logprobs'] (alloc_outputs(..., raw=True))")
    if workspace is None:
        workspace = make_workspace(B, k, V, dt, target_logits.device)
    if stream is None:
        stream = torch.cuda.current_stream(target_logits.device)
    head = (target_logits.data_ptr(), draft_logits.data_ptr(), dt, draft_tokens.data_ptr(), temperature.data_ptr(),
            top_k.data_ptr(), top_p.data_ptr(), B, k, V, int(seed), int(offset), out["tokens"].data_ptr(),
            out["accept_len"].data_ptr(), out["logprobs"].data_ptr())
    tail = (out["alpha"].data_ptr(), workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
    if timing is not None:
        t = timing._struct()
        st = lib().spec_verify_timed(*head, out["raw_logprobs"].data_ptr() if raw else None, *tail, ctypes.byref(t))
        timing.kernels = int(t.kernels)
    elif raw:
        st = lib().spec_verify_raw(*head, out["raw_logprobs"].data_ptr(), *tail)
    else:
        st = lib().spec_verify(*head, *tail)
    if st != 0:
        raise SpecVerifyError(st)
    return out


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, temperature, top_k, top_p, out, seed: int = 0,
                        offset: int = 0, stream=None):
    """spec_verify without a workspace (the library's per-GPU static scratch, see spec_verify_noalloc in the
    C header); ``out`` (from alloc_outputs) is required, so the call allocates nothing."""
    import torch
    B, k1, V = target_logits.shape
    dt = _dtype_code(target_logits)
    for t in (target_logits, draft_logits, draft_tokens, temperature, top_k, top_p):
        if not t.is_contiguous():
            raise ValueError("all inputs must be contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(target_logits.device)
    st = lib().spec_verify_noalloc(target_logits.data_ptr(), draft_logits.data_ptr(), dt, draft_tokens.data_ptr(),
                                   temperature.data_ptr(), top_k.data_ptr(), top_p.data_ptr(), B, k1 - 1, V, int(seed),
                                   int(offset), out["tokens"].data_ptr(), out["accept_len"].data_ptr(),
                                   out["logprobs"].data_ptr(), out["alpha"].data_ptr(),
                                   ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise SpecVerifyError(st, "spec_verify_noalloc")
    return out


def spec_sample(logits, temperature, top_k, top_p, row_b=None, row_pos=None, seed: int = 0, offset: int = 0,
                out=None, workspace=None, stream=None):
    """Plain sampler on device tensors: one token per row of ``logits`` [R, V].

    Returns (tokens int32 [R], logprobs float32 [R]).  ``row_b``/``row_pos`` (int32 [R]) are the
    stream coordinates of each row (default: row index, 0)."""
    import torch
    R, V = logits.shape
    dt = _dtype_code(logits)
    if out is None:
        out = (torch.empty(R, dtype=torch.int32, device=logits.device),
               torch.empty(R, dtype=torch.float32, device=logits.device))
    if workspace is None:
        n = int(lib().spec_sample_workspace_size(R, V, dt))
        if n == 0:
            raise ValueError("invalid sizes for spec_sample")
        workspace = torch.zeros(n, dtype=torch.uint8, device=logits.device)
    if stream is None:
        stream = torch.cuda.current_stream(logits.device)
    st = lib().spec_sample(logits.data_ptr(), dt, temperature.data_ptr(), top_k.data_ptr(), top_p.data_ptr(),
                           row_b.data_ptr() if row_b is not None else None,
                           row_pos.data_ptr() if row_pos is not None else None, R, V, int(seed), int(offset),
                           out[0].data_ptr(), out[1].data_ptr(), workspace.data_ptr(), workspace.numel(),
                           ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise SpecVerifyError(st, "spec_sample")
    return out


def tree_workspace_size(B: int, N: int, V: int, dtype: int = SPEC_DTYPE_BF16) -> int:
    return int(lib().spec_tree_verify_workspace_size(B, N, V, dtype))


def spec_tree_verify(target_logits, parent, node_tokens, temperature, top_k, top_p, seed: int = 0, offset: int = 0,
                     out=None, workspace=None, stream=None, timing=None):
    """Tree verification on device tensors: target_logits [B, N, V] (bf16 or fp32), parent and node_tokens
    int32 [B, N], temperature float32 [B], top_k int32 [B], top_p float32 [B].  Returns a dict with
    tokens [B, N], path [B, N], accept_len [B] (int32) and logprobs [B, N] (float32)."""
    import torch
    B, N, V = target_logits.shape
    dt = _dtype_code(target_logits)
    for t in (target_logits, parent, node_tokens, temperature, top_k, top_p):
        if not t.is_contiguous():
            raise ValueError("all inputs must be contiguous")
    dev = target_logits.device
    if out is None:
        out = dict(tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
                   path=torch.empty((B, N), dtype=torch.int32, device=dev),
                   accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                   logprobs=torch.empty((B, N), dtype=torch.float32, device=dev))
    if workspace is None:
        n = tree_workspace_size(B, N, V, dt)
        if n == 0:
            raise ValueError("invalid sizes for spec_tree_verify")
        workspace = torch.zeros(n, dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    args = (target_logits.data_ptr(), dt, parent.data_ptr(), node_tokens.data_ptr(), temperature.data_ptr(),
            top_k.data_ptr(), top_p.data_ptr(), B, N, V, int(seed), int(offset), out["tokens"].data_ptr(),
            out["path"].data_ptr(), out["accept_len"].data_ptr(), out["logprobs"].data_ptr(), workspace.data_ptr(),
            workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
    if timing is not None:
        t = timing._struct()
        st = lib().spec_tree_verify_timed(*args, ctypes.byref(t))
        timing.kernels = int(t.kernels)
    else:
        st = lib().spec_tree_verify(*args)
    if st != 0:
        raise SpecVerifyError(st, "spec_tree_verify")
    return out


def spec_commit(tensors, state_slot, accept_len, seq_len=None, status=None, stream=None, k=None):
    """Commit step on device tensors.

    ``tensors``: list of (verify_state, state_cache) pairs, verify_state [L, B, k+1, ...] and state_cache
    [L, num_slots, ...] (contiguous, one dtype per pair; copied bit for bit).  state_slot and accept_len
    are int32 [B]; seq_len (int32 [B], updated in place) and status (int32 [B] out) may be None.  For a
    call without tensors, pass ``k``.  The caches of committed rows are updated in place; returns status."""
    import torch
    B = state_slot.shape[0]
    descs = (StateTensor * max(1, len(tensors)))()
    num_slots = None
    for i, (vs, cache) in enumerate(tensors):
        if not (vs.is_contiguous() and cache.is_contiguous()):
            raise ValueError("state tensors must be contiguous")
        if vs.dtype != cache.dtype or vs.shape[3:] != cache.shape[2:] or vs.shape[0] != cache.shape[0] \
                or vs.shape[1] != B:
            raise ValueError("verify_state [L, B, k+1, ...] and state_cache [L, num_slots, ...] do not match")
        if k is None:
            k = vs.shape[2] - 1
        if vs.shape[2] != k + 1 or (num_slots is not None and cache.shape[1] != num_slots):
            raise ValueError("all tensors must share k and num_slots")
        num_slots = cache.shape[1]
        descs[i] = StateTensor(vs.data_ptr(), cache.data_ptr(), vs[0, 0, 0].numel() * vs.element_size(), vs.shape[0])
    if k is None:
        raise ValueError("k is needed when no tensors are given")
    if num_slots is None:
        num_slots = 1 << 30
    for t in (state_slot, accept_len, seq_len, status):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or t.shape != (B,)):
            raise ValueError("state_slot, accept_len, seq_len and status must be contiguous int32 [B]")
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=state_slot.device)
    if stream is None:
        stream = torch.cuda.current_stream(state_slot.device)
    st = lib().spec_commit(descs, len(tensors), state_slot.data_ptr(), accept_len.data_ptr(),
                           seq_len.data_ptr() if seq_len is not None else None, status.data_ptr(), B, k,
                           num_slots, ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise SpecVerifyError(st, "spec_commit")
    return status


def spec_commit_slots(state_slot, pos_slot, accept_len, num_slots: int, seq_len=None, status=None, stream=None):
    """Commit by slot numbers on device tensors: state_slot int32 [B] and pos_slot int32 [B, k+1] are
    updated in place (see spec_commit_slots in the C header); seq_len (int32 [B]) too when given.
    Returns status int32 [B]."""
    import torch
    B, k1 = pos_slot.shape
    for t, shape in ((state_slot, (B,)), (pos_slot, (B, k1)), (accept_len, (B,)), (seq_len, (B,)), (status, (B,))):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or tuple(t.shape) != shape):
            raise ValueError("state_slot, accept_len, seq_len, status: contiguous int32 [B]; pos_slot [B, k+1]")
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=state_slot.device)
    if stream is None:
        stream = torch.cuda.current_stream(state_slot.device)
    st = lib().spec_commit_slots(state_slot.data_ptr(), pos_slot.data_ptr(), accept_len.data_ptr(),
                                 seq_len.data_ptr() if seq_len is not None else None, status.data_ptr(), B, k1 - 1,
                                 int(num_slots), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise SpecVerifyError(st, "spec_commit_slots")
    return status
