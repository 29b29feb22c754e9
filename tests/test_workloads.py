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
