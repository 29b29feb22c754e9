"""Plain CPU oracle of the speculative-decoding verify sampler (ctypes binding).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The product path (the GPU
library and its Python binding) never imports, links or calls it, and the two share
no code.

The C++ source (``specverify_oracle.cpp``) computes everything in double precision;
this module only builds it with g++, loads it, and marshals numpy arrays.
Logit arrays are numpy ``uint16`` (raw bf16 bit patterns) or ``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "specverify_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")
MUTANT_DIR = os.path.join(HERE, "_mutants")

DTYPE_BF16 = 0
DTYPE_F32 = 1

_CFLAGS = ["-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", "-ffp-contract=off", "-fno-fast-math"]


def lib_path(mutant: int | None = None) -> str:
    if mutant is None:
        return LIB
    return os.path.join(MUTANT_DIR, f"liboracle_m{mutant}.so")


def build(mutant: int | None = None, force: bool = True) -> str:
    """Compile the oracle (or a negative-control mutant) with g++; returns the .so path."""
    out = lib_path(mutant)
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
        return out
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["g++", *_CFLAGS, "-o", out + ".tmp", SRC]
    if mutant is not None:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(out + ".tmp", out)
    return out


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64
_D = ctypes.c_double


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_P)


@dataclass
class VerifyResult:
    tokens: np.ndarray       # int32 [B, k+1]
    accept_len: np.ndarray   # int32 [B]
    logprobs: np.ndarray     # float64 [B, k+1]
    alpha: np.ndarray        # float64 [B, k]
    accept_margin: np.ndarray  # float64 [B]
    gumbel_gap: np.ndarray     # float64 [B]
    topp_margin: np.ndarray    # float64 [B]
    residual_mass: np.ndarray  # float64 [B]
    fallback: np.ndarray       # bool [B]
    sentinel: np.ndarray       # bool [B]
    n_accepted: np.ndarray     # int32 [B]
    topp_rows: np.ndarray | None = None   # float64 [B, 2k+1, 2]: |M/Z_K - P| at the chosen and next larger value
    accept_pos: np.ndarray | None = None  # float64 [B, k]: |u - p/q| per evaluated accept test (+inf otherwise)

    def margin_rows(self, tol_accept: float = 1e-5, tol_gap: float = 1e-5, tol_topp: float = 1e-5) -> np.ndarray:
        """Rows whose outcome a different (correct) rounding could change: boolean [B]."""
        return ((self.accept_margin <= tol_accept) | (self.gumbel_gap <= tol_gap)
                | (self.topp_margin <= tol_topp) | self.fallback)


@dataclass
class TreeResult:
    tokens: np.ndarray       # int32 [B, N]
    path: np.ndarray         # int32 [B, N]
    accept_len: np.ndarray   # int32 [B]
    logprobs: np.ndarray     # float64 [B, N]
    accept_margin: np.ndarray  # float64 [B]
    gumbel_gap: np.ndarray     # float64 [B]
    topp_margin: np.ndarray    # float64 [B]
    stop_node: np.ndarray      # int32 [B]

    @property
    def sentinel(self) -> np.ndarray:
        return self.accept_len == 0

    def margin_rows(self, tol_accept: float = 1e-5, tol_gap: float = 1e-5, tol_topp: float = 1e-5) -> np.ndarray:
        return (self.accept_margin <= tol_accept) | (self.gumbel_gap <= tol_gap) | (self.topp_margin <= tol_topp)


class Oracle:
    """Loaded oracle library (optionally a negative-control mutant)."""

    def __init__(self, mutant: int | None = None, rebuild: bool = False):
        path = lib_path(mutant)
        if rebuild or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
            build(mutant)
        self.mutant = mutant
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.oracle_philox4x32_10.argtypes = [_P, _P, _P]
        L.oracle_philox4x32_10.restype = None
        L.oracle_accept_uniform.argtypes = [_U64, _U32, _U32, _U32]
        L.oracle_accept_uniform.restype = _D
        L.oracle_gumbel_uniform.argtypes = [_U64, _U32, _U32, _U32, _U32, _U32]
        L.oracle_gumbel_uniform.restype = _D
        L.oracle_row_probs.argtypes = [_P, _I32, _D, _I32, _D, _P, _P]
        L.oracle_row_probs.restype = ctypes.c_int
        L.oracle_spec_verify.argtypes = [_P, _P, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _U64, _U64,
                                         _P, _P, _P, _P, _P, _P, _I32]
        L.oracle_spec_verify.restype = ctypes.c_int
        L.oracle_spec_verify_ex.argtypes = [_P, _P, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _U64, _U64,
                                            _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32]
        L.oracle_spec_verify_ex.restype = ctypes.c_int
        L.oracle_sample.argtypes = [_P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _U64, _U64, _P, _P, _P, _I32]
        L.oracle_sample.restype = ctypes.c_int
        L.oracle_raw_logprobs.argtypes = [_P, _I32, _P, _P, _I32, _I32, _I32, _P, _P, _I32]
        L.oracle_raw_logprobs.restype = ctypes.c_int
        L.oracle_commit.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, ctypes.c_int64]
        L.oracle_commit.restype = ctypes.c_int
        L.oracle_tree_verify.argtypes = [_P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _U64, _U64, _P, _P, _P, _P,
                                         _P, _I32]
        L.oracle_tree_verify.restype = ctypes.c_int
        L.oracle_commit_slots.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32]
        L.oracle_commit_slots.restype = ctypes.c_int

    # -- random streams ---------------------------------------------------------------
    def philox(self, ctr, key) -> np.ndarray:
        c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(4))
        k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
        out = np.zeros(4, dtype=np.uint32)
        self.lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
        return out

    def accept_uniform(self, seed: int, b: int, i: int, offset: int) -> float:
        return self.lib.oracle_accept_uniform(seed, b, i, offset)

    def gumbel_uniform(self, seed: int, tag: int, b: int, j: int, x: int, offset: int) -> float:
        return self.lib.oracle_gumbel_uniform(seed, tag, b, j, x, offset)

    # -- one row's sampler distribution ---------------------------------------------
    def row_probs(self, logits, T: float, K: int = 0, P: float = 1.0):
        l = np.ascontiguousarray(np.asarray(logits, dtype=np.float64))
        V = l.shape[0]
        probs = np.zeros(V, dtype=np.float64)
        info = np.zeros(8, dtype=np.float64)
        rc = self.lib.oracle_row_probs(_ptr(l), V, float(T), int(K), float(P), _ptr(probs), _ptr(info))
        if rc != 0:
            raise ValueError("row has no distribution (all -inf)")
        return probs, dict(m=info[0], argmax=int(info[1]), Z=info[2], kept=int(info[3]), thr=info[4],
                           topp_margin=info[5], topp_at=info[6], topp_prev=info[7])

    # -- the verify step ------------------------------------------------------------------
    def spec_verify(self, target, draft, draft_tokens, temperature, top_k, top_p, seed: int = 0,
                    offset: int = 0, num_threads: int = 0, alt=None, details: bool = False) -> VerifyResult:
        """The verify step.  ``details`` adds the per-decision distances (topp_rows, accept_pos).  ``alt``
        (int32 [B, 4], see oracle_spec_verify_ex) computes only the rows with alt[b, 3] != 0, each with the
        alternative resolutions it names; other rows of the result are zeros."""
        target = np.ascontiguousarray(target)
        draft = np.ascontiguousarray(draft)
        if target.dtype == np.uint16:
            dtype = DTYPE_BF16
        elif target.dtype == np.float32:
            dtype = DTYPE_F32
        else:
            raise TypeError("logits must be uint16 (bf16 bits) or float32")
        if draft.dtype != target.dtype:
            raise TypeError("target and draft logits must share a dtype")
        B, k1, V = target.shape
        k = k1 - 1
        if draft.shape != (B, k, V):
            raise ValueError("draft logits must be [B, k, V]")
        dt = np.ascontiguousarray(np.asarray(draft_tokens, dtype=np.int32).reshape(B, k))
        T = np.ascontiguousarray(np.asarray(temperature, dtype=np.float32).reshape(B))
        K = np.ascontiguousarray(np.asarray(top_k, dtype=np.int32).reshape(B))
        P = np.ascontiguousarray(np.asarray(top_p, dtype=np.float32).reshape(B))
        tokens = np.zeros((B, k + 1), dtype=np.int32)
        acc = np.zeros(B, dtype=np.int32)
        lp = np.zeros((B, k + 1), dtype=np.float64)
        al = np.zeros((B, k), dtype=np.float64)
        diag = np.zeros((B, 4), dtype=np.float64)
        fl = np.zeros(B, dtype=np.int32)
        if alt is None and not details:
            rc = self.lib.oracle_spec_verify(_ptr(target), _ptr(draft), dtype, _ptr(dt), _ptr(T), _ptr(K), _ptr(P),
                                             B, k, V, int(seed), int(offset), _ptr(tokens), _ptr(acc), _ptr(lp),
                                             _ptr(al), _ptr(diag), _ptr(fl), int(num_threads))
            tr = ap = None
        else:
            a = None if alt is None else np.ascontiguousarray(np.asarray(alt, dtype=np.int32).reshape(B, 4))
            tr = np.zeros((B, 2 * k + 1, 2), dtype=np.float64)
            ap = np.zeros((B, k), dtype=np.float64)
            rc = self.lib.oracle_spec_verify_ex(_ptr(target), _ptr(draft), dtype, _ptr(dt), _ptr(T), _ptr(K),
                                                _ptr(P), B, k, V, int(seed), int(offset), _ptr(tokens), _ptr(acc),
                                                _ptr(lp), _ptr(al), _ptr(diag), _ptr(fl), _ptr(a), _ptr(tr), _ptr(ap),
                                                int(num_threads))
        if rc != 0:
            raise ValueError("oracle_spec_verify rejected its scalar arguments")
        return VerifyResult(tokens, acc, lp, al, diag[:, 0].copy(), diag[:, 1].copy(), diag[:, 2].copy(),
                            diag[:, 3].copy(), (fl & 1) != 0, (fl & 2) != 0, (fl >> 8).astype(np.int32), tr, ap)

    # -- tree verification ---------------------------------------------------------------
    def tree_verify(self, target, parent, node_tokens, temperature, top_k, top_p, seed: int = 0, offset: int = 0,
                    num_threads: int = 0) -> TreeResult:
        """Recursive rejection over a draft tree per batch row: target [B, N, V] (uint16 bf16 bits or
        float32), parent and node_tokens int32 [B, N] (entry 0, the root, ignored), parameters [B]."""
        target = np.ascontiguousarray(target)
        if target.dtype == np.uint16:
            dtype = DTYPE_BF16
        elif target.dtype == np.float32:
            dtype = DTYPE_F32
        else:
            raise TypeError("logits must be uint16 (bf16 bits) or float32")
        B, N, V = target.shape
        par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32).reshape(B, N))
        tok = np.ascontiguousarray(np.asarray(node_tokens, dtype=np.int32).reshape(B, N))
        T = np.ascontiguousarray(np.asarray(temperature, dtype=np.float32).reshape(B))
        K = np.ascontiguousarray(np.asarray(top_k, dtype=np.int32).reshape(B))
        P = np.ascontiguousarray(np.asarray(top_p, dtype=np.float32).reshape(B))
        tokens = np.zeros((B, N), dtype=np.int32)
        path = np.zeros((B, N), dtype=np.int32)
        acc = np.zeros(B, dtype=np.int32)
        lp = np.zeros((B, N), dtype=np.float64)
        diag = np.zeros((B, 4), dtype=np.float64)
        rc = self.lib.oracle_tree_verify(_ptr(target), dtype, _ptr(par), _ptr(tok), _ptr(T), _ptr(K), _ptr(P), B, N, V,
                                         int(seed), int(offset), _ptr(tokens), _ptr(path), _ptr(acc), _ptr(lp),
                                         _ptr(diag), int(num_threads))
        if rc != 0:
            raise ValueError("oracle_tree_verify rejected its scalar arguments")
        stop = np.where(acc > 0, diag[:, 3], -1).astype(np.int32)
        return TreeResult(tokens, path, acc, lp, diag[:, 0].copy(), diag[:, 1].copy(), diag[:, 2].copy(), stop)

    # -- raw logprobs of the committed tokens --------------------------------------------
    def raw_logprobs(self, target, tokens, accept_len, temperature=None, num_threads: int = 0) -> np.ndarray:
        """ln softmax of each committed position's unprocessed target logits at its token: float64 [B, k+1]
        (0 after the committed slots, NaN for rows with accept_len 0).  ``temperature`` only feeds a
        negative-control mutant; the definition does not use it."""
        target = np.ascontiguousarray(target)
        if target.dtype == np.uint16:
            dtype = DTYPE_BF16
        elif target.dtype == np.float32:
            dtype = DTYPE_F32
        else:
            raise TypeError("logits must be uint16 (bf16 bits) or float32")
        B, k1, V = target.shape
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(B, k1))
        acc = np.ascontiguousarray(np.asarray(accept_len, dtype=np.int32).reshape(B))
        T = np.ascontiguousarray(np.ones(B, np.float32) if temperature is None
                                 else np.asarray(temperature, dtype=np.float32).reshape(B))
        out = np.zeros((B, k1), dtype=np.float64)
        rc = self.lib.oracle_raw_logprobs(_ptr(target), dtype, _ptr(tok), _ptr(acc), B, k1 - 1, V, _ptr(T),
                                          _ptr(out), int(num_threads))
        if rc != 0:
            raise ValueError("oracle_raw_logprobs rejected its arguments")
        return out

    # -- commit step ----------------------------------------------------------------------
    def commit(self, tensors, state_slot, accept_len, seq_len=None):
        """Commit step over a list of (verify_state, state_cache) numpy pairs, each
        verify_state [L, B, k+1, ...] and state_cache [L, num_slots, ...] of one dtype:
        state_cache[l, state_slot[b]] = verify_state[l, b, accept_len[b] - 1] for rows with
        1 <= accept_len <= k+1 and a slot in range, every layer and every pair.  seq_len (int32 [B],
        may be None) gains accept_len[b] on those rows, once.  The caches and seq_len are updated in
        place; returns status int32 [B] (0 committed, 1 bad accept_len, 2 bad slot)."""
        assert len(tensors) >= 1
        B = int(np.asarray(state_slot).shape[0])
        slot = np.ascontiguousarray(np.asarray(state_slot, dtype=np.int32).reshape(B))
        acc = np.ascontiguousarray(np.asarray(accept_len, dtype=np.int32).reshape(B))
        if seq_len is not None:
            assert seq_len.dtype == np.int32 and seq_len.flags.c_contiguous and seq_len.shape == (B,)
        status = np.zeros(B, dtype=np.int32)
        for idx, (vs, cache) in enumerate(tensors):
            vs = np.ascontiguousarray(vs)
            L, B2, k1 = vs.shape[:3]
            assert B2 == B and cache.flags.c_contiguous and cache.dtype == vs.dtype
            assert cache.shape[0] == L and cache.shape[2:] == vs.shape[3:]
            row_bytes = vs[0, 0, 0].nbytes
            rc = self.lib.oracle_commit(_ptr(vs), _ptr(cache), _ptr(slot), _ptr(acc),
                                        _ptr(seq_len if idx == 0 else None), _ptr(status), L, B, k1 - 1,
                                        int(cache.shape[1]), int(row_bytes))
            if rc != 0:
                raise ValueError("oracle_commit rejected its arguments")
        return status

    def commit_slots(self, state_slot, pos_slot, accept_len, num_slots, seq_len=None):
        """Commit by slot numbers: state_slot int32 [B] and pos_slot int32 [B, k+1] are swapped in place at
        (b, accept_len[b] - 1) for rows with a valid accept length and slots in 0..num_slots-1; seq_len
        (int32 [B], may be None) gains accept_len there.  Returns status int32 [B]."""
        B, k1 = pos_slot.shape
        for a, shape in ((state_slot, (B,)), (pos_slot, (B, k1))):
            assert a.dtype == np.int32 and a.flags.c_contiguous and a.shape == shape
        if seq_len is not None:
            assert seq_len.dtype == np.int32 and seq_len.flags.c_contiguous and seq_len.shape == (B,)
        acc = np.ascontiguousarray(np.asarray(accept_len, dtype=np.int32).reshape(B))
        status = np.zeros(B, dtype=np.int32)
        rc = self.lib.oracle_commit_slots(_ptr(state_slot), _ptr(pos_slot), _ptr(acc), _ptr(seq_len), _ptr(status),
                                          B, k1 - 1, int(num_slots))
        if rc != 0:
            raise ValueError("oracle_commit_slots rejected its arguments")
        return status

    # -- plain sampler ---------------------------------------------------------------------
    def sample(self, logits, temperature, top_k, top_p, row_b, row_pos, seed: int = 0, offset: int = 0,
               num_threads: int = 0):
        """Sample one token per row of ``logits`` [R, V]; returns (tokens, logprobs, gap)."""
        logits = np.ascontiguousarray(logits)
        if logits.dtype == np.uint16:
            dtype = DTYPE_BF16
        elif logits.dtype == np.float32:
            dtype = DTYPE_F32
        else:
            raise TypeError("logits must be uint16 (bf16 bits) or float32")
        R, V = logits.shape
        T = np.ascontiguousarray(np.asarray(temperature, dtype=np.float32).reshape(R))
        K = np.ascontiguousarray(np.asarray(top_k, dtype=np.int32).reshape(R))
        P = np.ascontiguousarray(np.asarray(top_p, dtype=np.float32).reshape(R))
        rb = np.ascontiguousarray(np.asarray(row_b, dtype=np.int32).reshape(R))
        rp = np.ascontiguousarray(np.asarray(row_pos, dtype=np.int32).reshape(R))
        tok = np.zeros(R, dtype=np.int32)
        lp = np.zeros(R, dtype=np.float64)
        gap = np.zeros(R, dtype=np.float64)
        rc = self.lib.oracle_sample(_ptr(logits), dtype, _ptr(T), _ptr(K), _ptr(P), _ptr(rb), _ptr(rp), R, V,
                                    int(seed), int(offset), _ptr(tok), _ptr(lp), _ptr(gap), int(num_threads))
        if rc != 0:
            raise ValueError("oracle_sample rejected its scalar arguments")
        return tok, lp, gap


_default: Oracle | None = None


def get() -> Oracle:
    """The (lazily built and loaded) reference oracle."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
