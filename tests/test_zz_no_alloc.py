"""spec_verify_noalloc (no workspace argument; the library's static per-GPU scratch) against spec_verify with
its own workspace: bit-identical outputs, and oracle parity, over two calls in a row whose second is smaller;
sizes beyond the scratch are refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle
import parity
from rejection_sampling_verify_16_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_noalloc_matches_spec_verify_two_calls():
    import torch
    import rejection_sampling_verify_16_amd as sv
    o = oracle.get()
    cases = [(W.make(40, 3, 65536, seed=61, boost=8.0, mixed_params=True, name="noalloc_big"), 5, 3),
             (W.make(6, 1, 16384, seed=62, boost=6.0, mixed_params=True, name="noalloc_small"), 2, 8)]
    for w, seed, off in cases:
        print(f"[noalloc] {w.name} B={w.B} k={w.k} V={w.V}", flush=True)
        drafts = w.draft_tokens(parity.oracle_sampler(o))
        dev = parity.device_inputs(w, drafts)
        ref = parity.run_gpu(dev, seed, off)                    # spec_verify, its own workspace
        out = sv.alloc_outputs(w.B, w.k)
        for t in out.values():
            t.fill_(-7)
        sv.spec_verify_noalloc(dev["target"], dev["draft"], dev["drafts"], dev["T"], dev["K"], dev["P"], out,
                               seed=seed, offset=off)
        torch.cuda.synchronize()
        got = {key: t.cpu().numpy() for key, t in out.items()}
        for key in ref:
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{w.name}: {key}")
        r, alt = parity.verify_oracle(o, w.target, w.draft, drafts, w.temperature, w.top_k, w.top_p, seed, off)
        rep = parity.compare(got, r, drafts, w.V, label=f"noalloc/{w.name}", alt=alt)
        print(f"[noalloc] {w.name}: {rep}", flush=True)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    import rejection_sampling_verify_16_amd as sv
    L = sv.lib()
    B, k, V = 4096, 4, 1 << 20
    assert sv.workspace_size(B, k, V) > (128 << 20)
    P = ctypes.c_void_p(256)   # never dereferenced: the size check comes first
    st = L.spec_verify_noalloc(P, P, 0, P, P, P, P, B, k, V, 0, 0, P, P, P, P, None)
    assert st == 2
