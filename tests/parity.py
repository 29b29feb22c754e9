"""GPU-vs-oracle comparison with margin accounting (used by the ``gpu`` tests and smoke()).

Parity bar: for every batch row outside the margins, tokens and accept_len are bit-exact;
logprobs agree within 2e-4 on committed slots, alpha within 1e-5.  A row is a margin row
when some accept test had |u - p/q| <= 1e-5, the Gumbel top-2 gap at the drawn position was
<= 1e-5, a top-p decision was within TOPP_TOL of the boundary, or the residual fell back to p
(possible only through rounding).  Margin rows are counted and checked for validity only.
Sentinel rows must match exactly.
"""
from __future__ import annotations

import numpy as np

import oracle

LOGPROB_TOL = 2e-4
ALPHA_TOL = 1e-5
ACCEPT_TOL = 1e-5
GAP_TOL = 1e-5
TOPP_TOL = 2e-6   # top-p decision margin (this build's extension; GPU mass sums are good to ~1e-7)


def oracle_sampler(o: oracle.Oracle):
    def sample(rows, T, K, P, rb, rp, seed, offset):
        tok, _, _ = o.sample(rows, T, K, P, rb, rp, seed=seed, offset=offset)
        return tok
    return sample


def device_inputs(w, drafts, device="cuda"):
    import torch
    if w.dtype == "bf16":
        t = torch.from_numpy(w.target.view(np.int16)).view(torch.bfloat16)
        d = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(w.target)
        d = torch.from_numpy(w.draft)
    return dict(target=t.to(device), draft=d.to(device),
                drafts=torch.from_numpy(np.ascontiguousarray(drafts, dtype=np.int32)).to(device),
                T=torch.from_numpy(w.temperature).to(device), K=torch.from_numpy(w.top_k).to(device),
                P=torch.from_numpy(w.top_p).to(device))


def run_gpu(dev, seed, offset, out=None, workspace=None):
    import torch
    import rejection_sampling_verify_16_amd as sv
    res = sv.spec_verify(dev["target"], dev["draft"], dev["drafts"], dev["T"], dev["K"], dev["P"], seed=seed,
                         offset=offset, out=out, workspace=workspace)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in res.items()}


def compare(g: dict, r: oracle.VerifyResult, drafts: np.ndarray, V: int, label: str = "") -> dict:
    """Assert the parity bar; returns counts for reporting."""
    B, k1 = r.tokens.shape
    k = k1 - 1
    sent = r.sentinel
    margin = r.margin_rows(ACCEPT_TOL, GAP_TOL, TOPP_TOL) & ~sent
    strict = ~margin & ~sent

    # sentinel rows: exact
    assert np.all(g["accept_len"][sent] == 0), f"{label}: sentinel accept_len"
    assert np.all(g["tokens"][sent] == -1), f"{label}: sentinel tokens"
    assert np.all(np.isnan(g["logprobs"][sent])) and np.all(np.isnan(g["alpha"][sent])), f"{label}: sentinel NaN"
    gs = g["accept_len"][~sent]
    assert np.all((gs >= 1) & (gs <= k + 1)), f"{label}: GPU marked a valid row invalid or accept_len out of range"

    # strict rows: bit-exact tokens / accept_len
    bad = strict & (np.any(g["tokens"] != r.tokens, axis=1) | (g["accept_len"] != r.accept_len))
    if bad.any():
        idx = np.nonzero(bad)[0][:5]
        detail = [(int(b), g["tokens"][b].tolist(), r.tokens[b].tolist(), float(r.accept_margin[b]),
                   float(r.gumbel_gap[b]), float(r.topp_margin[b])) for b in idx]
        raise AssertionError(f"{label}: {int(bad.sum())} strict rows differ (row, gpu, oracle, acc-margin, gap, "
                             f"topp-margin): {detail}")
    # logprobs on committed slots; padding exact
    slot = np.arange(k + 1)[None, :] < r.accept_len[:, None]
    sel = strict[:, None] & slot
    d = np.abs(g["logprobs"].astype(np.float64) - r.logprobs)
    assert np.all(np.isfinite(g["logprobs"][sel])), f"{label}: non-finite logprob"
    if sel.any():
        worst = float(d[sel].max())
        assert worst <= LOGPROB_TOL, f"{label}: logprob error {worst}"
    pad = strict[:, None] & ~slot
    assert np.all(g["logprobs"][pad] == 0.0) and np.all(g["tokens"][pad] == -1), f"{label}: padding"
    # alpha does not depend on random draws: every valid row outside the top-p margin
    arow = ~sent & ~(r.topp_margin <= TOPP_TOL)
    da = np.abs(g["alpha"].astype(np.float64) - r.alpha)[arow]
    alpha_err = float(da.max()) if da.size else 0.0
    assert alpha_err <= ALPHA_TOL, f"{label}: alpha error {alpha_err}"

    # margin rows: the GPU's own output must still be a well-formed verify result
    for b in np.nonzero(margin)[0]:
        n = int(g["accept_len"][b]) - 1
        assert np.array_equal(g["tokens"][b, :n], drafts[b, :n]), f"{label}: margin row {b} prefix"
        assert 0 <= g["tokens"][b, n] < V, f"{label}: margin row {b} drawn token"
        assert np.all(g["tokens"][b, n + 1:] == -1), f"{label}: margin row {b} padding"
        assert np.all(np.isfinite(g["logprobs"][b, :n + 1])), f"{label}: margin row {b} logprobs"
    return dict(rows=int(B), margin=int(margin.sum()), sentinel=int(sent.sum()),
                logprob_err=float(d[sel].max()) if sel.any() else 0.0, alpha_err=alpha_err,
                mean_accept=float(r.accept_len[~sent].mean()) if (~sent).any() else 0.0)
