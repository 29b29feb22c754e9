"""The device random stream, checked directly (not only end to end through the verify step):
the product's Philox-4x32-10 on the published known-answer vectors and on random counters against the
oracle's independent implementation, every 23-bit Gumbel code through the race transform against fp64,
and every 24-bit accept code.  Runs the product's own device helpers through the probe library
(libsvprobe.so, built beside the product library but never linked into it)."""
import ctypes
import os

import numpy as np
import pytest

import oracle
import oracle_pins

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "rejection_sampling_verify_16_amd",
                     "libsvprobe.so")

# Bound on the relative error of E2 = -log2 U and of the race key scale 1 / E2 over all 2^23 codes.  A race
# key w / E2 compares in natural-log units as ln w - ln E2, so a relative error e of E2 moves a key by
# about e: with e <= 1e-6 every draw whose top-2 gap exceeds the 1e-5 margin is decided as in fp64.
E2_REL_TOL = 1e-6
KEY_REL_TOL = 1.5e-6


@pytest.fixture(scope="module")
def P():
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} is missing: build first")
    # torch brings its own HIP runtime: initialise it before the probe library binds one of its own
    import torch
    torch.cuda.init()
    L = ctypes.CDLL(PROBE)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    L.probe_philox.argtypes = [vp, vp, vp, i32, vp]
    L.probe_philox_uk.argtypes = [vp, ctypes.c_uint32, ctypes.c_uint32, vp, i32, vp]
    L.probe_race_e2.argtypes = [vp, vp, vp]
    L.probe_u24.argtypes = [vp, vp]
    for f in (L.probe_philox, L.probe_philox_uk, L.probe_race_e2, L.probe_u24):
        f.restype = ctypes.c_int
    return L


def _philox_gpu(P, ctr, key):
    import torch
    c = torch.from_numpy(np.ascontiguousarray(ctr, dtype=np.uint32).view(np.int32)).cuda()
    k = torch.from_numpy(np.ascontiguousarray(key, dtype=np.uint32).view(np.int32)).cuda()
    out = torch.empty_like(c)
    assert P.probe_philox(c.data_ptr(), k.data_ptr(), out.data_ptr(), c.shape[0], None) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def test_philox_kat_on_device(P):
    rows = [[int(t, 16) for t in line.split()] for line in oracle_pins.read_golden_table("philox4x32_10_kat.txt")]
    v = np.array(rows, dtype=np.uint64).astype(np.uint32)
    got = _philox_gpu(P, v[:, 0:4], v[:, 4:6])
    np.testing.assert_array_equal(got, v[:, 6:10])


def test_philox_random_counters_match_oracle(P):
    rng = np.random.default_rng(17)
    n = 4096
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    ctr[:64, 1:] = 0            # small counters, as the streams use them
    got = _philox_gpu(P, ctr, key)
    o = oracle.get()
    want = np.array([o.philox(ctr[i], key[i]) for i in range(n)], dtype=np.uint32)
    np.testing.assert_array_equal(got, want)


def _philox_uk_gpu(P, ctr, key):
    import torch
    c = torch.from_numpy(np.ascontiguousarray(ctr, dtype=np.uint32).view(np.int32)).cuda()
    out = torch.empty_like(c)
    assert P.probe_philox_uk(c.data_ptr(), int(key[0]), int(key[1]), out.data_ptr(), c.shape[0], None) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def test_philox_uniform_key_kat_on_device(P):
    """The verify kernels' form (one key per launch, three-input xors from the third round on)."""
    rows = [[int(t, 16) for t in line.split()] for line in oracle_pins.read_golden_table("philox4x32_10_kat.txt")]
    v = np.array(rows, dtype=np.uint64).astype(np.uint32)
    for r in v:
        got = _philox_uk_gpu(P, r[None, 0:4], r[4:6])
        np.testing.assert_array_equal(got[0], r[6:10])


def test_philox_uniform_key_random_counters_match_oracle(P):
    """Counters shaped like the draws' (x >> 2 per lane; position, row and offset words shared by the
    wave) and fully random ones, under a few keys."""
    rng = np.random.default_rng(23)
    o = oracle.get()
    n = 2048
    for key in ([0, 0], [0xFFFFFFFF, 0xFFFFFFFF], list(rng.integers(0, 2**32, size=2, dtype=np.uint64))):
        key = np.array(key, dtype=np.uint64).astype(np.uint32)
        ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
        ctr[: n // 2, 0] = np.arange(n // 2, dtype=np.uint32)
        ctr[: n // 2, 1:] = ctr[0, 1:]
        got = _philox_uk_gpu(P, ctr, key)
        want = np.array([o.philox(ctr[i], key) for i in range(n)], dtype=np.uint32)
        np.testing.assert_array_equal(got, want)


def test_race_transform_exhaustive(P):
    """All 2^23 uniform codes: E2 = -log2((j + 0.5) 2^-23) and its reciprocal, against fp64."""
    import torch
    n = 1 << 23
    e2 = torch.empty(n, dtype=torch.float32, device="cuda")
    sc = torch.empty(n, dtype=torch.float32, device="cuda")
    assert P.probe_race_e2(e2.data_ptr(), sc.data_ptr(), None) == 0
    torch.cuda.synchronize()
    e2, sc = e2.cpu().numpy().astype(np.float64), sc.cpu().numpy().astype(np.float64)
    U = (np.arange(n, dtype=np.float64) + 0.5) * 2.0 ** -23
    exact = -np.log2(U)
    rel = np.abs(e2 / exact - 1.0)
    krel = np.abs(sc * exact - 1.0)
    worst = int(np.argmax(rel))
    print(f"[rng] E2 max rel err {rel.max():.3g} at code {worst} (U = {U[worst]:.9g}); "
          f"near U -> 1 (last 4096 codes) {rel[-4096:].max():.3g}; key scale max rel err {krel.max():.3g}",
          flush=True)
    assert np.all(e2 > 0)
    assert rel.max() <= E2_REL_TOL
    assert krel.max() <= KEY_REL_TOL


def test_accept_uniform_codes_exact(P):
    """All 2^24 accept codes map exactly to j 2^-24 (so only p/q rounding separates GPU and oracle)."""
    import torch
    n = 1 << 24
    u = torch.empty(n, dtype=torch.float32, device="cuda")
    assert P.probe_u24(u.data_ptr(), None) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u.cpu().numpy().astype(np.float64), np.arange(n, dtype=np.float64) * 2.0 ** -24)
