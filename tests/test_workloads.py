"""The seeded input generator: shapes, bf16 rounding, ties, determinism (CPU only)."""
import numpy as np
import torch

from rejection_sampling_verify_16_amd import workloads as W


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 100_000), rng.normal(0, 1e-3, 1000), [0.0, -0.0, 1.0, -2.5, 3.0e38]])
    x = x.astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(W.bf16_rne(x), want)
    np.testing.assert_array_equal(W.bf16_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_shapes_and_determinism():
    a = W.make(4, 2, 4096, seed=5, boost=8.0, mixed_params=True)
    b = W.make(4, 2, 4096, seed=5, boost=8.0, mixed_params=True)
    assert a.target.shape == (4, 3, 4096) and a.draft.shape == (4, 2, 4096)
    assert a.target.dtype == np.uint16
    np.testing.assert_array_equal(a.target, b.target)
    np.testing.assert_array_equal(a.top_p, b.top_p)
    assert set(np.unique(a.top_k)) <= {0, 50} and set(np.unique(a.top_p)) <= {np.float32(1.0), np.float32(0.95)}
    assert np.all((a.temperature >= 0.6) & (a.temperature <= 1.2))


def test_ties_are_exact():
    w = W.make(64, 2, 2048, seed=9, noise_sigma=0.5, boost=8.0, temperature=0.0, tie_fraction=0.05)
    assert w.tie_rows_target and w.tie_rows_draft
    for b, i in w.tie_rows_target:
        v = W.bf16_to_f32(w.target[b, i])
        assert np.sum(v == v.max()) >= 2
    for b, i, t in w.draft_overrides:
        v = W.bf16_to_f32(w.target[b, i])
        assert v[t] == v.max() and t > int(np.argmax(v))


def test_named_configs_small():
    c1 = W.config1()
    assert (c1.B, c1.k, c1.V, c1.dtype) == (1, 1, 1024, "f32") and c1.target.dtype == np.float32
    assert c1.logit_bytes == (2 * 1 + 1) * 1024 * 4


def test_tree_workloads_are_valid_trees():
    """Tree generator: parents earlier than their node, sibling tokens distinct and in range, children in
    decreasing order of the noisy parent row, deterministic per seed; random trees honour the branching cap."""
    w = W.make_tree(6, 4096, None, N=20, seed=11, boost=10.0, mixed_params=True)
    w2 = W.make_tree(6, 4096, None, N=20, seed=11, boost=10.0, mixed_params=True)
    np.testing.assert_array_equal(w.parent, w2.parent)
    np.testing.assert_array_equal(w.node_tokens, w2.node_tokens)
    assert w.target.shape == (6, 20, 4096)
    for b in range(w.B):
        for i in range(1, w.N):
            assert 0 <= w.parent[b, i] < i and 0 <= w.node_tokens[b, i] < w.V
        for u in range(w.N):
            kids = [c for c in range(1, w.N) if w.parent[b, c] == u]
            assert len(kids) <= 4
            toks = w.node_tokens[b, kids]
            assert len(set(toks.tolist())) == len(kids)
    e = W.tree_eagle9()
    assert (e.B, e.N, e.V) == (64, 9, 157184) and list(e.parent[0]) == list(W.EAGLE_TREE_9)
    # the root's first child is the top token of a noisy copy of the root row: usually the row's argmax
    top = np.argmax(W.bf16_to_f32(e.target[:, 0]), axis=1)
    assert np.mean(e.node_tokens[:, 1] == top) > 0.9


def test_commit_workloads():
    """Commit generator: tensor shapes, an injective slot map, accept lengths in range, sentinels and bad slots
    where asked, and the moved-bytes figure."""
    w = W.make_commit(50, 3, 80, [("rec", 2, (4, 8), np.float32), ("conv", 3, (3, 5), np.uint16)], seed=7,
                      sentinels=4, bad_slots=3)
    assert w.tensors[0].verify_state.shape == (2, 50, 4, 4, 8) and w.tensors[0].state_cache.shape == (2, 80, 4, 8)
    assert w.tensors[1].verify_state.dtype == np.uint16
    good = (w.state_slot >= 0) & (w.state_slot < w.num_slots)
    assert (~good).sum() == 3 and len(set(w.state_slot[good].tolist())) == good.sum()
    assert (w.accept_len == 0).sum() == 4 and np.all(w.accept_len <= w.k + 1)
    ok = (w.accept_len >= 1) & good
    assert w.moved_bytes == 2 * int(ok.sum()) * (2 * 4 * 8 * 4 + 3 * 3 * 5 * 2)
    rng = np.random.default_rng(0)
    acc = W.accept_lengths(rng, 200_000, 2, 0.75)
    np.testing.assert_allclose(np.bincount(acc, minlength=4)[1:] / 200_000, [0.25, 0.75 * 0.25, 0.75 ** 2], atol=5e-3)
