"""GPU parity of tree verification (spec_tree_verify): against the CPU oracle on seeded trees, and bit for bit
against the GPU chain verify step on chain-shaped trees with one-hot draft rows."""
import numpy as np
import pytest

import oracle
from parity import ACCEPT_TOL, GAP_TOL, LOGPROB_TOL, TOPP_TOL
from rejection_sampling_verify_16_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def _dev_logits(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


def run_tree_gpu(w, seed, offset, garbage_workspace=False):
    import torch
    import rejection_sampling_verify_16_amd as sv
    d = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to("cuda:0")
    ws = None
    if garbage_workspace:  # the workspace needs no initialisation
        n = sv.tree_workspace_size(w.B, w.N, w.V, sv.SPEC_DTYPE_F32 if w.dtype == "f32" else sv.SPEC_DTYPE_BF16)
        ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = sv.spec_tree_verify(_dev_logits(w.target), d(w.parent, np.int32), d(w.node_tokens, np.int32),
                              d(w.temperature, np.float32), d(w.top_k, np.int32), d(w.top_p, np.float32),
                              seed=seed, offset=offset, workspace=ws)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in out.items()}


def compare_tree(g, r, w, label):
    """Sentinel rows exactly; rows outside the margins bit-exact (tokens, path, accept length) with logprobs
    within the tolerance; margin rows must still be a valid walk of their tree."""
    B, N = w.B, w.N
    sent = r.sentinel
    margin = r.margin_rows(ACCEPT_TOL, GAP_TOL, TOPP_TOL) & ~sent
    strict = ~margin & ~sent
    assert np.all(g["accept_len"][sent] == 0), f"{label}: sentinel accept_len"
    assert np.all(g["tokens"][sent] == -1) and np.all(g["path"][sent] == -1), f"{label}: sentinel tokens/path"
    assert np.all(np.isnan(g["logprobs"][sent])), f"{label}: sentinel logprobs"
    bad = strict & ((g["accept_len"] != r.accept_len) | np.any(g["tokens"] != r.tokens, axis=1)
                    | np.any(g["path"] != r.path, axis=1))
    assert not bad.any(), (f"{label}: {bad.sum()} strict rows differ, first {np.flatnonzero(bad)[:5]}: "
                           f"gpu {g['tokens'][bad][:2]} oracle {r.tokens[bad][:2]}")
    for b in np.flatnonzero(~sent):
        n = g["accept_len"][b] - 1
        assert 0 <= n < N, f"{label}: row {b} accept_len {n + 1}"
        prev = 0
        for i in range(n):
            node = g["path"][b, i]
            assert 1 <= node < N and w.parent[b, node] == prev, f"{label}: row {b} path {g['path'][b]}"
            assert g["tokens"][b, i] == w.node_tokens[b, node]
            prev = node
        assert 0 <= g["tokens"][b, n] < w.V and np.all(g["tokens"][b, n + 1:] == -1)
        assert np.all(g["path"][b, n:] == -1)
        assert np.all(g["logprobs"][b, n + 1:] == 0.0)
        if strict[b]:
            err = np.abs(g["logprobs"][b, :n + 1] - r.logprobs[b, :n + 1]).max()
            assert err <= LOGPROB_TOL, f"{label}: row {b} logprob error {err}"
    return {"rows": B, "margin": int(margin.sum()), "sentinel": int(sent.sum()),
            "mean_accept": float(g["accept_len"][~sent].mean()) if (~sent).any() else 0.0}


def check(o, w, seed=5, offsets=(1,), garbage_workspace=False):
    print(f"tree case {w.name}: B={w.B} N={w.N} V={w.V} {w.dtype}", flush=True)
    reps = []
    for off in offsets:
        g = run_tree_gpu(w, seed, off, garbage_workspace)
        r = o.tree_verify(w.target, w.parent, w.node_tokens, w.temperature, w.top_k, w.top_p, seed=seed, offset=off)
        reps.append(compare_tree(g, r, w, f"{w.name}@{off}"))
    return reps


CASES = {
    # the benchmark tree at full size
    "eagle9": W.tree_eagle9,
    # random trees, 16 nodes, several slices and a ragged vocabulary tail
    "random16_ragged": lambda: W.make_tree(32, 3 * 4096 + 8, None, N=16, seed=3011, boost=10.0, mixed_params=True,
                                           name="random16_ragged"),
    # the most nodes a tree may have, fp32
    "nodes64_f32": lambda: W.make_tree(4, 4096, None, N=64, dtype="f32", seed=3012, boost=12.0, mixed_params=True,
                                       name="nodes64_f32"),
    # a single node: the bonus draw from the root
    "single_node": lambda: W.make_tree(16, 8192, (0,), seed=3013, mixed_params=True, name="single_node"),
    # top-p only, flatter rows (drawn tokens after rejections are common)
    "topp_flat": lambda: W.make_tree(48, 32768, W.EAGLE_TREE_9, seed=3014, boost=6.0, top_p=0.9, temperature=1.1,
                                     name="topp_flat"),
    # top-k only with K below the children count of the root
    "topk3": lambda: W.make_tree(48, 32768, W.EAGLE_TREE_9, seed=3015, boost=9.0, top_k=3, name="topk3"),
    # greedy
    "greedy": lambda: W.make_tree(64, 65536, W.EAGLE_TREE_9, seed=3016, boost=5.0, temperature=0.0, name="greedy"),
    # many trees: 9000 node rows, enough for the statistics kernel's wide slices; a ragged vocabulary tail
    "many_trees_wide": lambda: W.make_tree(1000, 4104, W.EAGLE_TREE_9, seed=3017, boost=9.0, mixed_params=True,
                                           name="many_trees_wide"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_tree_parity(o, case):
    check(o, CASES[case](), offsets=(1, 2))


def test_tree_workspace_needs_no_initialisation(o):
    check(o, CASES["random16_ragged"](), offsets=(3,), garbage_workspace=True)


def test_tree_greedy_ties_and_unusable_rows(o):
    """Greedy rows with exact ties at the argmax (lowest index wins, also when a child holds the higher
    tied index), and rows that must come back as sentinels: bad parent, repeated sibling token, token out
    of range, a NaN in a row the walk never visits, an invalid temperature."""
    w = W.make_tree(12, 8192, W.EAGLE_TREE_9, seed=3017, boost=6.0, temperature=0.0, name="greedy_ties_bad")
    tv = w.target
    for b in range(6):   # tie the root's maximum with a higher index; make that index a child
        a = int(np.argmax(W.bf16_to_f32(tv[b, 0])))
        j = (a + 1 + b) % w.V
        tv[b, 0, j] = tv[b, 0, a]
        w.node_tokens[b, 1] = j if b % 2 == 0 else a
        # the root's other children get tokens away from both tied indices
        w.node_tokens[b, 2:5] = [(a + 100 + 7 * i) % w.V for i in range(3)]
    w.parent[6, 3] = 5                     # parent not earlier
    w.node_tokens[7, 2] = w.node_tokens[7, 1]   # siblings with one token
    w.node_tokens[8, 4] = w.V              # token out of range
    tv[9, 8, 17] = 0x7FC0                  # NaN (bf16) in the deepest row
    w.temperature[10] = -1.0
    rep = check(o, w)
    assert rep[0]["sentinel"] == 5


def test_tree_chain_equals_chain_verify():
    """Chain-shaped trees give the chain verify step's outputs for one-hot draft rows (bf16 mixed, fp32,
    greedy): tokens and accept lengths bit for bit, path = 1..n, and logprobs equal up to the rounding of the
    kept-set normaliser (spec_verify's one-launch path sums it in another order than the tree kernels)."""
    import torch
    import rejection_sampling_verify_16_amd as sv
    for name, B, k, V, dtype, kw in [("bf16_mixed", 64, 2, 157184, "bf16", dict(boost=12.0, mixed_params=True)),
                                     ("f32_k4", 32, 4, 8192, "f32", dict(boost=8.0, mixed_params=True)),
                                     ("greedy", 32, 3, 32768, "bf16", dict(boost=4.0, temperature=0.0))]:
        print(f"chain tree {name}", flush=True)
        w = W.make_tree(B, V, tuple([0] + list(range(k))), dtype=dtype, seed=3020 + k, **kw)
        drafts = w.node_tokens[:, 1:].copy()
        if dtype == "bf16":
            one_hot = np.full((B, k, V), 0xFF80, np.uint16)     # -inf
            for b in range(B):
                one_hot[b, np.arange(k), drafts[b]] = 0          # +0
        else:
            one_hot = np.full((B, k, V), -np.inf, np.float32)
            for b in range(B):
                one_hot[b, np.arange(k), drafts[b]] = 0.0
        d = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to("cuda:0")
        T, K, P = d(w.temperature, np.float32), d(w.top_k, np.int32), d(w.top_p, np.float32)
        c = sv.spec_verify(_dev_logits(w.target), _dev_logits(one_hot), d(drafts, np.int32), T, K, P, seed=9, offset=4)
        t = sv.spec_tree_verify(_dev_logits(w.target), d(w.parent, np.int32), d(w.node_tokens, np.int32), T, K, P,
                                seed=9, offset=4)
        torch.cuda.synchronize()
        c = {k_: v.cpu().numpy() for k_, v in c.items()}
        t = {k_: v.cpu().numpy() for k_, v in t.items()}
        np.testing.assert_array_equal(t["accept_len"], c["accept_len"])
        np.testing.assert_array_equal(t["tokens"], c["tokens"])
        np.testing.assert_allclose(t["logprobs"], c["logprobs"], rtol=0, atol=4e-6)
        for b in range(B):
            n = c["accept_len"][b] - 1
            assert list(t["path"][b]) == list(range(1, n + 1)) + [-1] * (k + 1 - n)
        assert len(set(c["accept_len"].tolist())) > 1


def test_tree_determinism_and_graph_replay():
    """Repeated calls give identical outputs; a captured HIP graph of the call replays them exactly, with
    unrelated eager calls between replays."""
    import torch
    import rejection_sampling_verify_16_amd as sv
    w = W.make_tree(32, 65536, W.EAGLE_TREE_9, seed=3030, boost=12.0, mixed_params=True, name="graph")
    d = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to("cuda:0")
    args = (_dev_logits(w.target), d(w.parent, np.int32), d(w.node_tokens, np.int32), d(w.temperature, np.float32),
            d(w.top_k, np.int32), d(w.top_p, np.float32))
    eager = {k_: v.cpu().numpy() for k_, v in sv.spec_tree_verify(*args, seed=4, offset=7).items()}
    again = {k_: v.cpu().numpy() for k_, v in sv.spec_tree_verify(*args, seed=4, offset=7).items()}
    for key in eager:
        np.testing.assert_array_equal(eager[key], again[key])
    gws = torch.zeros(sv.tree_workspace_size(w.B, w.N, w.V), dtype=torch.uint8, device="cuda:0")
    gout = sv.spec_tree_verify(*args, seed=4, offset=7, workspace=gws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sv.spec_tree_verify(*args, seed=4, offset=7, out=gout, workspace=gws)
    for rep in range(3):
        for key in gout:
            gout[key].fill_(7)
        graph.replay()
        torch.cuda.synchronize()
        for key in eager:
            np.testing.assert_array_equal(gout[key].cpu().numpy(), eager[key], err_msg=f"replay {rep} {key}")
        sv.spec_tree_verify(*args, seed=5, offset=1)   # unrelated eager work between replays
        torch.cuda.synchronize()
