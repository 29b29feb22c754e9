"""The one-launch resident path (SPEC_PATH_RESIDENT) against the CPU oracle, element by element, with the
same margin accounting as the staged path: the named bf16 workloads that fit one workgroup per compute unit,
ragged and maximal vocabularies, k = 1..4, narrow and wide top-k windows (and their fallback to the exact
whole-row selection), small top-p, greedy rows with ties; and the bounded waits: a call whose waits are cut
to a few clock ticks ends with every batch row either a sentinel row or the oracle's row, and the next call
is correct.  Special values, sentinels, candidate edges and garbage workspaces are covered by the parity
tests run on both paths."""
import numpy as np
import pytest

import oracle
import parity
from rejection_sampling_verify_16_amd import workloads as W
from test_gpu_parity import _check

pytestmark = pytest.mark.gpu

RESIDENT = 2


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("name", ["2", "3"])
def test_named_workload_resident(o, name):
    w = W.CONFIGS[name]()
    _check(o, w, [0, 1], w.name, path=RESIDENT)


CASES = [
    ("ragged_mixed", 8, 2, 50008, dict(boost=8.0, mixed_params=True)),
    ("k1_wide", 12, 1, 61448, dict(temperature=0.8, top_p=0.9)),
    ("k3_narrow_topk", 8, 3, 65536, dict(temperature=0.8, top_k=200)),
    ("k4_topp", 3, 4, 20000, dict(temperature=1.0, top_p=0.5)),
    ("large_topk", 4, 4, 131080, dict(temperature=1.3, top_k=5000)),
    ("topk_257_wide", 6, 2, 30000, dict(temperature=1.0, top_k=257, top_p=0.97)),
    ("tiny_topp", 6, 2, 12008, dict(temperature=0.9, top_p=0.05)),
    ("flat_topk", 4, 2, 30000, dict(target_sigma=0.05, noise_sigma=0.02, temperature=1.0, top_k=100)),
    ("min_V", 3, 1, 8, dict(temperature=1.0)),
    ("k1_T2", 16, 1, 32768, dict(temperature=2.0, top_k=1000, top_p=0.99)),
    ("greedy_ties", 24, 2, 40000, dict(temperature=0.0, tie_fraction=0.2)),
    ("maxV_mixed", 4, 2, 1 << 20, dict(boost=8.0, mixed_params=True)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_resident_cases(o, case):
    name, B, k, V, kw = case
    w = W.make(B, k, V, seed=7000 + B + V, name=name, **kw)
    _check(o, w, [0, 5], name, path=RESIDENT)


def test_bounded_waits_give_up_cleanly(o):
    """Waits cut to 2 ticks of the 100 MHz clock: workgroups that give up turn their batch row into a sentinel
    row (token -1, accept length 0, NaN logprob and alpha) and exit, so the launch always completes; rows
    that were not abandoned are the oracle's.  The same buffers then serve a normal call at parity."""
    import torch
    import rejection_sampling_verify_16_amd as sv
    w = W.make(32, 2, 157184, seed=7100, boost=8.0, mixed_params=True, name="give_up")
    drafts = w.draft_tokens(parity.oracle_sampler(o))
    dev = parity.device_inputs(w, drafts)
    out = sv.alloc_outputs(w.B, w.k)
    ws = sv.make_workspace(w.B, w.k, w.V)
    r, alt = parity.verify_oracle(o, w.target, w.draft, drafts, w.temperature, w.top_k, w.top_p, 3, 2)
    tm = sv.KernelTiming(path=RESIDENT, wait_limit=2)
    print("[resident] give-up call: wait_limit 2 ticks", flush=True)
    g = parity.run_gpu(dev, 3, 2, out=out, workspace=ws, timing=tm)
    assert tm.kernels == 1
    sent = g["accept_len"] == 0
    print(f"[resident] abandoned rows: {int(sent.sum())} of {w.B}", flush=True)
    assert np.all(g["tokens"][sent] == -1) and np.all(np.isnan(g["logprobs"][sent]))
    assert np.all(np.isnan(g["alpha"][sent]))
    print("[resident] normal call on the same buffers", flush=True)
    g2 = parity.run_gpu(dev, 3, 2, out=out, workspace=ws, timing=sv.KernelTiming(path=RESIDENT))
    parity.compare(g2, r, drafts, w.V, label="give_up/after", alt=alt)
    # the rows the first call completed are the oracle's: checked with its abandoned rows taken from the second
    mix = {key: np.where(sent.reshape((-1,) + (1,) * (v.ndim - 1)), g2[key], v) for key, v in g.items()}
    parity.compare(mix, r, drafts, w.V, label="give_up/kept", alt=alt)
    torch.cuda.synchronize()
