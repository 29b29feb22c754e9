"""Seeded synthetic inputs for the verify sampler (logits, sampling parameters, ties).

This module holds no arithmetic of the verify method: it draws logits and per-row
parameters with numpy, rounds them to bf16, and injects exact ties.  Draft tokens are
"sampled from q", which needs a sampler; the caller supplies one (``sampler``
argument), so the same recipe serves the tests (which pass the CPU oracle's sampler)
and the benchmark (which passes the GPU library's plain sampler).

Stand-ins: the pages measure on real model logits over public prompt sets; those are
not available here, so every workload is synthetic, shaped like the pages' setting
(vocabulary ~157k, k = 1..4 drafts, temperature 1 or mixed, top-k/top-p as in plain
sampling).  Generator: ``numpy.random.Generator(PCG64(1000 + index))``; logits are drawn
in float32 and rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable

import numpy as np

# sampler(logits[R, V], T[R], K[R], P[R], row_b[R], row_pos[R], seed, offset) -> tokens[R]
Sampler = Callable[..., np.ndarray]


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One verify workload: inputs of spec_verify() except the draft tokens."""
    name: str
    B: int
    k: int
    V: int
    dtype: str                 # "bf16" (uint16 bit patterns) or "f32"
    target: np.ndarray         # [B, k+1, V]
    draft: np.ndarray          # [B, k, V]
    temperature: np.ndarray    # float32 [B]
    top_k: np.ndarray          # int32 [B]
    top_p: np.ndarray          # float32 [B]
    seed: int = 0              # verify seed
    offsets: list = field(default_factory=lambda: [0])
    draft_seed: int = 0        # plain-sampler stream used to draw the drafts
    draft_offset: int = 0
    # (b, i, token) written over the sampled drafts (tie rows that must be rejected)
    draft_overrides: list = field(default_factory=list)
    tie_rows_target: list = field(default_factory=list)   # (b, i) with an injected exact tie
    tie_rows_draft: list = field(default_factory=list)

    @property
    def logit_bytes(self) -> int:
        return self.target.nbytes + self.draft.nbytes

    def draft_sampling_inputs(self):
        """(logits[B*k, V], T, K, P, row_b, row_pos) for drawing the draft tokens from q."""
        B, k = self.B, self.k
        rows = self.draft.reshape(B * k, self.V)
        T = np.repeat(self.temperature, k)
        K = np.repeat(self.top_k, k)
        P = np.repeat(self.top_p, k)
        row_b = np.repeat(np.arange(B, dtype=np.int32), k)
        row_pos = np.tile(np.arange(k, dtype=np.int32), B)
        return rows, T, K, P, row_b, row_pos

    def draft_tokens(self, sampler: Sampler) -> np.ndarray:
        """Draw the drafts from q with ``sampler`` and apply the overrides: int32 [B, k]."""
        rows, T, K, P, rb, rp = self.draft_sampling_inputs()
        tok = np.asarray(sampler(rows, T, K, P, rb, rp, self.draft_seed, self.draft_offset), dtype=np.int32)
        tok = tok.reshape(self.B, self.k).copy()
        for b, i, t in self.draft_overrides:
            tok[b, i] = t
        return tok


def _normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def _inject_tie(row: np.ndarray, rng: np.random.Generator, above: bool):
    """Copy the row maximum to a second index (above or below the first maximum).

    Returns (first_max_index, tie_index) or None when no such index exists."""
    vals = bf16_to_f32(row) if row.dtype == np.uint16 else row
    a = int(np.argmax(vals))
    if above and a + 1 < row.shape[0]:
        j = int(rng.integers(a + 1, row.shape[0]))
    elif (not above) and a > 0:
        j = int(rng.integers(0, a))
    else:
        return None
    row[j] = row[a]
    return a, j


def make(B: int, k: int, V: int, *, dtype: str = "bf16", seed: int = 1000, target_sigma: float = 2.5,
         noise_sigma: float = 0.8, boost: float = 0.0, zipf: float = 0.0, temperature=1.0, top_k=0,
         top_p=1.0, mixed_params: bool = False, tie_fraction: float = 0.0, name: str = "custom",
         offsets=None) -> Workload:
    """General recipe behind the five named workloads.

    target = N(0, target_sigma^2) [+ boost at one uniform index per logit row]
             [- zipf * ln(v + 1) over token ids]; draft = target + N(0, noise_sigma^2),
    drawn per batch row in float32, then rounded to bf16 (or kept float32).
    ``mixed_params`` draws T ~ U[0.6, 1.2], top-k in {0, 50}, top-p in {1.0, 0.95}.
    ``tie_fraction`` injects exact ties into ceil(fraction) of target and draft rows.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    is_bf16 = dtype == "bf16"
    tgt = np.empty((B, k + 1, V), dtype=np.uint16 if is_bf16 else np.float32)
    drf = np.empty((B, k, V), dtype=np.uint16 if is_bf16 else np.float32)
    prior = None
    if zipf:
        prior = (-np.float32(zipf) * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    for b in range(B):
        t = _normal(rng, (k + 1, V), target_sigma)
        if boost:
            idx = rng.integers(0, V, size=k + 1)
            t[np.arange(k + 1), idx] += np.float32(boost)
        if prior is not None:
            t += prior[None, :]
        d = t[:k] + _normal(rng, (k, V), noise_sigma)
        if is_bf16:
            tgt[b] = bf16_rne(t)
            drf[b] = bf16_rne(d)
        else:
            tgt[b] = t
            drf[b] = d
    if mixed_params:
        T = rng.uniform(0.6, 1.2, size=B).astype(np.float32)
        K = np.where(rng.random(B) < 0.5, 0, 50).astype(np.int32)
        P = np.where(rng.random(B) < 0.5, 1.0, 0.95).astype(np.float32)
    else:
        T = np.full(B, temperature, dtype=np.float32)
        K = np.full(B, top_k, dtype=np.int32)
        P = np.full(B, top_p, dtype=np.float32)
    w = Workload(name=name, B=B, k=k, V=V, dtype=dtype, target=tgt, draft=drf, temperature=T, top_k=K, top_p=P,
                 offsets=list(offsets) if offsets is not None else [0])
    if tie_fraction > 0:
        n_t = math.ceil(tie_fraction * B * (k + 1))
        n_d = math.ceil(tie_fraction * B * k)
        t_rows = rng.choice(B * (k + 1), size=n_t, replace=False)
        d_rows = rng.choice(B * k, size=n_d, replace=False)
        with_draft = 0
        for c, r in enumerate(t_rows):
            b, i = divmod(int(r), k + 1)
            res = _inject_tie(tgt[b, i], rng, above=(c % 2 == 1))
            if res is None:
                continue
            w.tie_rows_target.append((b, i))
            a, j = res
            # half of the tied target rows that have a draft get the higher-index tied token as
            # their draft: the lowest index is the argmax, so that draft must be rejected.
            if i < k:
                if with_draft % 2 == 0:
                    w.draft_overrides.append((b, i, max(a, j)))
                with_draft += 1
        for c, r in enumerate(d_rows):
            b, i = divmod(int(r), k)
            if _inject_tie(drf[b, i], rng, above=(c % 2 == 1)) is not None:
                w.tie_rows_draft.append((b, i))
    return w


# ---- the five named workloads ------------------------------------------------------------

def config1() -> Workload:
    """B=1, k=1, V=1024, fp32; target N(0, 3^2), draft = target + N(0, 1); T=1, no truncation."""
    return make(1, 1, 1024, dtype="f32", seed=1001, target_sigma=3.0, noise_sigma=1.0, name="B1_k1_V1024_f32")


def config2() -> Workload:
    """B=16, k=2, V=157184, bf16; N(0, 2.5^2) + 8 at one index per row; noise 0.8; T=1."""
    return make(16, 2, 157184, seed=1002, target_sigma=2.5, noise_sigma=0.8, boost=8.0,
                name="B16_k2_V157184_bf16")


def config3() -> Workload:
    """B=64, k=2, V=157184, bf16; as config 2 with mixed T / top-k / top-p per row."""
    return make(64, 2, 157184, seed=1003, target_sigma=2.5, noise_sigma=0.8, boost=8.0, mixed_params=True,
                name="B64_k2_V157184_bf16_mixed")


def config4(k: int) -> Workload:
    """B=128, k=1 or 2, V=157184, bf16, greedy; noise 0.5; exact ties in 1% of rows."""
    return make(128, k, 157184, seed=1004 + (k - 1) * 100, target_sigma=2.5, noise_sigma=0.5, boost=8.0,
                temperature=0.0, tie_fraction=0.01, name=f"B128_k{k}_V157184_bf16_greedy")


def config5(n_calls: int = 100) -> Workload:
    """B=256, k=4, V=248320, bf16; N(0, 3^2) - 1.1 ln(v+1); noise 1.2; T=1, top-p 0.9; offsets 0..99."""
    return make(256, 4, 248320, seed=1005, target_sigma=3.0, noise_sigma=1.2, zipf=1.1, top_p=0.9,
                offsets=range(n_calls), name="B256_k4_V248320_bf16_topp")


CONFIGS = {"1": config1, "2": config2, "3": config3, "4a": lambda: config4(1), "4b": lambda: config4(2),
           "5": config5}


# ---- commit step ------------------------------------------------------------------------------
#
# The pages give no state sizes, so these are stand-ins shaped like a hybrid linear-attention model's
# stacked caches: per layer a recurrent state of H heads x d_k x d_v fp32 values and a conv window of
# (W - 1) positions x C channels in bf16, one verify-state entry per fed position.  State bytes are
# random (the copy is bit for bit, so their values do not matter); slots are a random injection of the
# batch rows into a larger pool; accept lengths follow a steady per-draft acceptance rate.

@dataclass
class CommitTensor:
    name: str
    verify_state: np.ndarray   # [L, B, k+1, ...]
    state_cache: np.ndarray    # [L, num_slots, ...] (the cache before the commit)


@dataclass
class CommitWorkload:
    name: str
    B: int
    k: int
    num_slots: int
    tensors: list              # of CommitTensor
    state_slot: np.ndarray     # int32 [B]
    accept_len: np.ndarray     # int32 [B]
    seq_len: np.ndarray        # int32 [B] (before the commit)

    @property
    def moved_bytes(self) -> int:
        """Bytes read plus bytes written by a commit of the rows that are committed."""
        ok = (self.accept_len >= 1) & (self.accept_len <= self.k + 1) & (self.state_slot >= 0) & \
             (self.state_slot < self.num_slots)
        per_row = sum(t.verify_state[:, 0, 0].nbytes for t in self.tensors)
        return 2 * int(ok.sum()) * per_row


def _random_bytes(rng: np.random.Generator, shape, dtype) -> np.ndarray:
    """Pseudo-random contents (the bytes of uniform doubles; fast to draw at GB sizes)."""
    n = int(np.prod(shape)) * np.dtype(dtype).itemsize
    return rng.random((n + 7) // 8).view(np.uint8)[:n].view(dtype).reshape(shape)


def accept_lengths(rng: np.random.Generator, B: int, k: int, rate: float) -> np.ndarray:
    """accept_len = 1 + number of leading accepted drafts, each accepted with probability `rate`."""
    acc = np.ones(B, dtype=np.int32)
    alive = np.ones(B, dtype=bool)
    for _ in range(k):
        alive &= rng.random(B) < rate
        acc += alive
    return acc


def make_commit(B: int, k: int, num_slots: int, shapes, *, seed: int, rate: float = 0.75, sentinels: int = 0,
                bad_slots: int = 0, name: str = "commit") -> CommitWorkload:
    """``shapes``: list of (name, layers, per-row state shape, numpy dtype)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    tensors = [CommitTensor(n, _random_bytes(rng, (L, B, k + 1) + tuple(s), dt),
                            _random_bytes(rng, (L, num_slots) + tuple(s), dt)) for n, L, s, dt in shapes]
    slot = rng.permutation(num_slots)[:B].astype(np.int32)
    acc = accept_lengths(rng, B, k, rate)
    if sentinels:
        acc[rng.choice(B, size=sentinels, replace=False)] = 0
    if bad_slots:
        rows = rng.choice(B, size=bad_slots, replace=False)
        slot[rows] = np.where(np.arange(bad_slots) % 2 == 0, num_slots + rows, -1 - rows).astype(np.int32)
    seq = rng.integers(1, 4096, size=B).astype(np.int32)
    return CommitWorkload(name, B, k, num_slots, tensors, slot, acc, seq)


def commit_hybrid(B: int = 64, k: int = 2, layers: int = 12, heads: int = 16, dk: int = 128, dv: int = 128,
                  conv_w: int = 4, conv_c: int = 6144, num_slots: int = 128, seed: int = 2001) -> CommitWorkload:
    """Hybrid linear-attention stand-in: `layers` layers, each with an fp32 recurrent state
    [heads, dk, dv] (1 MiB at the defaults) and a bf16 conv window [conv_w - 1, conv_c] (36 KiB)."""
    shapes = [("recurrent", layers, (heads, dk, dv), np.float32),
              ("conv", layers, (conv_w - 1, conv_c), np.uint16)]
    return make_commit(B, k, num_slots, shapes, seed=seed,
                       name=f"commit_B{B}_k{k}_L{layers}_rec{heads}x{dk}x{dv}f32_conv{conv_w - 1}x{conv_c}bf16")


COMMIT_CONFIGS = {"hybrid": commit_hybrid}


# ---- tree verification --------------------------------------------------------------------------
#
# Draft trees shaped like EAGLE top-k trees: the children of a node are the m most likely tokens of a
# noisy copy of that node's target logits (a stand-in for the draft model), in decreasing order, so
# siblings are distinct and the first child is the draft's favourite.  Target logits per node as in the
# chain workloads.

# parents of a 9-node tree: the root has 4 children, its first child 2, its second 1, and the first
# grandchild 1 (depth 3, 8 draft tokens)
EAGLE_TREE_9 = (0, 0, 0, 0, 0, 1, 1, 2, 5)


@dataclass
class TreeWorkload:
    name: str
    B: int
    N: int
    V: int
    dtype: str
    target: np.ndarray        # [B, N, V] (uint16 bf16 bits or float32)
    parent: np.ndarray        # int32 [B, N]
    node_tokens: np.ndarray   # int32 [B, N]
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    seed: int = 0
    offset: int = 0

    @property
    def logit_bytes(self) -> int:
        return self.target.nbytes


def random_tree(rng: np.random.Generator, N: int, max_children: int = 4) -> np.ndarray:
    """A random recursive tree: node i >= 1 takes a uniformly chosen earlier node with room as its parent."""
    par = np.zeros(N, dtype=np.int32)
    nch = np.zeros(N, dtype=np.int32)
    for i in range(1, N):
        room = np.flatnonzero(nch[:i] < max_children)
        par[i] = int(rng.choice(room))
        nch[par[i]] += 1
    return par


def make_tree(B: int, V: int, parents=EAGLE_TREE_9, *, N: int = 0, dtype: str = "bf16", seed: int = 3000,
              target_sigma: float = 2.5, noise_sigma: float = 0.8, boost: float = 8.0, temperature=1.0, top_k=0,
              top_p=1.0, mixed_params: bool = False, name: str = "tree", offset: int = 0) -> TreeWorkload:
    """``parents`` fixes one topology for every row; ``parents=None`` draws a random tree of N nodes per row."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if parents is not None:
        N = len(parents)
    is_bf16 = dtype == "bf16"
    tgt = np.empty((B, N, V), dtype=np.uint16 if is_bf16 else np.float32)
    par = np.zeros((B, N), dtype=np.int32)
    tok = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        pr = np.asarray(parents, dtype=np.int32) if parents is not None else random_tree(rng, N)
        t = _normal(rng, (N, V), target_sigma)
        if boost:
            t[np.arange(N), rng.integers(0, V, size=N)] += np.float32(boost)
        tgt[b] = bf16_rne(t) if is_bf16 else t
        tv = bf16_to_f32(tgt[b]) if is_bf16 else tgt[b]
        par[b] = pr
        for u in range(N):
            kids = [c for c in range(1, N) if pr[c] == u]
            if kids:
                noisy = tv[u] + _normal(rng, (V,), noise_sigma)
                m = len(kids)
                cand = np.argpartition(-noisy, m - 1)[:m] if m < V else np.arange(V)
                tok[b, kids] = cand[np.argsort(-noisy[cand], kind="stable")]
    if mixed_params:
        T = rng.uniform(0.6, 1.2, size=B).astype(np.float32)
        K = np.where(rng.random(B) < 0.5, 0, 50).astype(np.int32)
        P = np.where(rng.random(B) < 0.5, 1.0, 0.95).astype(np.float32)
    else:
        T = np.full(B, temperature, dtype=np.float32)
        K = np.full(B, top_k, dtype=np.int32)
        P = np.full(B, top_p, dtype=np.float32)
    return TreeWorkload(name, B, N, V, dtype, tgt, par, tok, T, K, P, seed=seed, offset=offset)


def tree_eagle9() -> TreeWorkload:
    """B=64, 9-node EAGLE-style tree (8 drafts, depth 3), V=157184, bf16, mixed T / top-k / top-p; target rows
    N(0, 2.5^2) + 15 at one index, so the top token holds about half the mass at T = 1 (a next-token
    distribution as peaked as a language model's, which is what makes target-only acceptance likely)."""
    return make_tree(64, 157184, EAGLE_TREE_9, seed=3001, boost=15.0, mixed_params=True,
                     name="tree_B64_N9_V157184_bf16_mixed")


TREE_CONFIGS = {"eagle9": tree_eagle9}
