"""GPU-vs-oracle comparison with margin accounting (used by the ``gpu`` tests and smoke()).

Parity bar: for every batch row outside the margins, tokens and accept_len are bit-exact;
logprobs agree within 2e-4 on committed slots, alpha within 1e-5.  A row is a margin row when
one of its decisions lies within rounding of its boundary: an evaluated accept test with
|u - p/q| <= 1e-5, a Gumbel top-2 gap <= 1e-5 at the drawn position, or a top-p decision whose
cumulative mass lies within TOPP_TOL of P (this build's extension of the margin rule).  A margin
row is not exempt: the GPU's output must equal, to the same bar, the oracle's output under one
combination of the two resolutions of each such decision (the test taken the other way, the
Gumbel runner-up, the top-p threshold one distinct value lower or higher), which the oracle
computes for exactly that row (``oracle_spec_verify_ex``).  The only rows checked for validity
alone are those whose residual mass vanished in fp64 (the oracle then draws from p_n; possible
only through rounding).  Sentinel rows must match exactly.
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle

LOGPROB_TOL = 2e-4
ALPHA_TOL = 1e-5
ACCEPT_TOL = 1e-5
GAP_TOL = 1e-5
TOPP_TOL = 1e-6   # top-p decision margin (GPU mass sums in fp32 / 2^40 fixed point are good to a few 1e-7)
MAX_DECISIONS = 6  # near-boundary decisions of one row whose combinations are enumerated (2^6 outcomes)


def oracle_sampler(o: oracle.Oracle):
    def sample(rows, T, K, P, rb, rp, seed, offset):
        tok, _, _ = o.sample(rows, T, K, P, rb, rp, seed=seed, offset=offset)
        return tok
    return sample


def verify_oracle(o: oracle.Oracle, target, draft, drafts, T, K, P, seed: int, offset: int):
    """The oracle's verify result with per-decision details, and a function evaluating alternative
    resolutions (an int32 [B, 4] array as oracle.spec_verify's ``alt``) on the same inputs."""
    r = o.spec_verify(target, draft, drafts, T, K, P, seed=seed, offset=offset, details=True)

    def alt(a):
        return o.spec_verify(target, draft, drafts, T, K, P, seed=seed, offset=offset, alt=a, details=True)
    return r, alt


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


def run_gpu(dev, seed, offset, out=None, workspace=None, timing=None):
    """One verify call on device inputs; ``timing`` (a KernelTiming) selects the path and reports the number
    of kernels the call launched."""
    import torch
    import rejection_sampling_verify_16_amd as sv
    res = sv.spec_verify(dev["target"], dev["draft"], dev["drafts"], dev["T"], dev["K"], dev["P"], seed=seed,
                         offset=offset, out=out, workspace=workspace, timing=timing)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in res.items()}


def decisions(r: oracle.VerifyResult, b: int) -> list:
    """The near-boundary decisions of row b: ("down" | "up", logit row), ("flip", position), ("runner", 0)."""
    out = []
    if r.topp_rows is not None:
        for row in range(r.topp_rows.shape[1]):
            if r.topp_rows[b, row, 0] <= TOPP_TOL:
                out.append(("down", row))
            if r.topp_rows[b, row, 1] <= TOPP_TOL:
                out.append(("up", row))
    if r.accept_pos is not None:
        for i in np.flatnonzero(r.accept_pos[b] <= ACCEPT_TOL):
            out.append(("flip", int(i)))
    if r.gumbel_gap[b] <= GAP_TOL:
        out.append(("runner", 0))
    return out


def alt_row(combo) -> np.ndarray | None:
    """The oracle's alt entry of one combination of alternative resolutions (None if inconsistent: one logit
    row moved both down and up)."""
    a = np.zeros(4, np.int32)
    for kind, j in combo:
        if kind == "down":
            a[0] |= 1 << j
        elif kind == "up":
            a[1] |= 1 << j
        elif kind == "flip":
            a[2] |= 1 << j
        else:
            a[2] |= 1 << 16
    if a[0] & a[1]:
        return None
    a[3] = 1
    return a


def _row_ok(g: dict, r: oracle.VerifyResult, b: int, k: int) -> tuple[bool, str]:
    """Row b of the GPU output against row b of an oracle result, to the parity bar."""
    if g["accept_len"][b] != r.accept_len[b] or np.any(g["tokens"][b] != r.tokens[b]):
        return False, f"tokens {g['tokens'][b].tolist()} vs {r.tokens[b].tolist()}"
    n1 = int(r.accept_len[b])
    lp = g["logprobs"][b].astype(np.float64)
    if not np.all(np.isfinite(lp[:n1])):
        return False, "non-finite logprob"
    err = float(np.abs(lp[:n1] - r.logprobs[b, :n1]).max()) if n1 else 0.0
    if err > LOGPROB_TOL:
        return False, f"logprob error {err}"
    if not np.all(lp[n1:] == 0.0):
        return False, "padding logprobs"
    aerr = float(np.abs(g["alpha"][b].astype(np.float64) - r.alpha[b]).max()) if k else 0.0
    if aerr > ALPHA_TOL:
        return False, f"alpha error {aerr}"
    return True, ""


def compare(g: dict, r: oracle.VerifyResult, drafts: np.ndarray, V: int, label: str = "", alt=None) -> dict:
    """Assert the parity bar; returns counts for reporting.  ``r`` and ``alt`` come from verify_oracle()
    (``alt`` may be None only if no row lies in the margin)."""
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
    da = np.abs(g["alpha"].astype(np.float64) - r.alpha)[strict]
    alpha_err = float(da.max()) if da.size else 0.0
    assert alpha_err <= ALPHA_TOL, f"{label}: alpha error {alpha_err}"

    # margin rows: equal to the oracle's output under one combination of the alternative resolutions
    counts = dict(main=0, alternative=0, fallback=0)
    kinds = {}
    todo = []  # (b, [alt rows]) still unmatched
    for b in np.flatnonzero(margin):
        dec = decisions(r, b)
        for kind, _ in dec:
            kinds[kind] = kinds.get(kind, 0) + 1
        if r.fallback[b] and not dec:
            # the residual vanished in fp64 (rounding only): a well-formed result drawn from p_n is all
            # that is fixed
            n = int(g["accept_len"][b]) - 1
            assert np.array_equal(g["tokens"][b, :n], drafts[b, :n]), f"{label}: fallback row {b} prefix"
            assert 0 <= g["tokens"][b, n] < V and np.all(g["tokens"][b, n + 1:] == -1), f"{label}: fallback row {b}"
            counts["fallback"] += 1
            continue
        ok, _ = _row_ok(g, r, b, k)
        if ok:
            counts["main"] += 1
            continue
        assert len(dec) <= MAX_DECISIONS, f"{label}: margin row {b} has {len(dec)} near-boundary decisions"
        combos = [c for n_ in range(1, len(dec) + 1) for c in itertools.combinations(dec, n_)]
        rows = [a for a in (alt_row(c) for c in combos) if a is not None]
        todo.append((int(b), rows))
    if todo:
        assert alt is not None, f"{label}: margin rows need the oracle's alternative resolutions (verify_oracle)"
        pending = {b: rows for b, rows in todo}
        reason = {}
        rnd = 0
        while pending:  # one oracle call per round: each pending row's next combination
            a = np.zeros((B, 4), np.int32)
            for b, rows in pending.items():
                a[b] = rows[rnd]
            ra = alt(a)
            for b in list(pending):
                ok, why = _row_ok(g, ra, b, k)
                if ok:
                    counts["alternative"] += 1
                    del pending[b]
                    continue
                reason.setdefault(b, []).append(why)
                if rnd + 1 >= len(pending[b]):
                    raise AssertionError(f"{label}: margin row {b} matches no resolution of its decisions "
                                         f"{decisions(r, b)}: {reason[b][:4]}")
            rnd += 1
    return dict(rows=int(B), margin=int(margin.sum()), margin_main=counts["main"],
                margin_alternative=counts["alternative"], margin_fallback=counts["fallback"],
                margin_kinds=kinds, sentinel=int(sent.sum()),
                logprob_err=float(d[sel].max()) if sel.any() else 0.0, alpha_err=alpha_err,
                mean_accept=float(r.accept_len[~sent].mean()) if (~sent).any() else 0.0)
