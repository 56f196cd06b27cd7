"""Shared helpers of the GPU parity tests: run the library through its C ABI on device
copies of host inputs, run the oracle on the same host inputs, compare.

Parity rule (from the benchmark spec of the verification step): greedy and tree results are
bit-exact; stochastic results match in tokens, accepted lengths and committed lengths, with
probabilities within 1e-5 absolute, except where a decision's uniform (or, for top-p, the
kept mass) lies within 1e-5 of its boundary (the oracle reports that distance per decision).
Such a sequence is compared up to that decision and not after it; it is counted by the kind
of its first near-boundary decision (acceptance test, top-p cut of a tested row, the final
draw, the top-p cut of the bonus row), and the counts go to the session's parity report.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from draft_verification_03_amd import binding as B

PROB_TOL = 1e-5
MARGIN = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def draft_tokens_oracle(x, seed_draft=9090):
    """The drafter's tokens: d_k drawn from q_k's filtered law (T, top-p of its sequence),
    by the oracle, one gamma = 0 round per draft row keyed (seed_draft, seq_id, L+k)."""
    cu = x["cu_gamma"]
    Bn = len(cu) - 1
    n = int(cu[-1])
    if n == 0:
        return np.zeros(0, np.int32)
    b_of = np.repeat(np.arange(Bn), np.diff(cu))
    k_of = np.arange(n) - cu[b_of]
    T = x["temperature"][b_of]
    P = None if x["top_p"] is None else x["top_p"][b_of]
    K = None if x.get("top_k") is None else x["top_k"][b_of]
    return oracle.draw_tokens(x["draft"][:, :x["stride"]], T, P, seed_draft,
                              x["seq_id"][b_of], x["committed_len"][b_of] + k_of,
                              vocab=x["vocab"], top_k=K)


def run_oracle_chain(x, tokens, seed, override=None, lead=1, nthreads=0):
    return oracle.verify_chain_v(x["target"], x["draft"], x["cu_gamma"], tokens,
                                 x["temperature"], x["top_p"], x["seq_id"],
                                 x["committed_len"], lead_slots=lead, seed=seed,
                                 uniform_override=override, nthreads=nthreads,
                                 vocab=x["vocab"], top_k=x.get("top_k"),
                                 eos_token=x.get("eos_token"), max_emit=x.get("max_emit"))


def run_gpu_chain(x, tokens, seed, override=None, lead=1, probes=True, no_draft=False,
                  workspace=None, noalloc=False):
    cu = x["cu_gamma"]
    Bn = len(cu) - 1
    n_d = int(cu[-1])
    n_t = n_d + Bn
    t = dict(
        target=dev(x["target"]),
        draft=None if (no_draft or x["draft"] is None or x["draft"].shape[0] == 0)
        else dev(x["draft"]),
        cu=dev(cu), tok=dev(tokens if n_d else np.zeros(1, np.int32)),
        temp=dev(x["temperature"]),
        topp=None if x["top_p"] is None else dev(x["top_p"]),
        topk=None if x.get("top_k") is None else dev(x["top_k"]),
        eos=None if x.get("eos_token") is None else dev(x["eos_token"]),
        cap=None if x.get("max_emit") is None else dev(x["max_emit"]),
        nemit=torch.full((Bn,), -7, dtype=torch.int32, device="cuda"),
        sid=dev(x["seq_id"]), L=dev(x["committed_len"]),
        out=torch.full((max(n_t, 1),), -1, dtype=torch.int32, device="cuda"),
        nacc=torch.full((Bn,), -7, dtype=torch.int32, device="cuda"),
        flags=torch.full((Bn,), -7, dtype=torch.int32, device="cuda"),
        pr=torch.full((max(n_d, 1), 3), float("nan"), device="cuda") if probes else None,
        ps=torch.full((Bn, 2), float("nan"), device="cuda") if probes else None,
        ovr=None if override is None else dev(override.astype(np.float32)),
    )
    a = B.chain_args(target_logits=t["target"], draft_logits=t["draft"], cu_gamma=t["cu"],
                     draft_tokens=t["tok"], temperature=t["temp"], top_p=t["topp"],
                     seq_id=t["sid"], committed_len=t["L"], out_tokens=t["out"],
                     num_accepted=t["nacc"], seq_flags=t["flags"], probe_rows=t["pr"],
                     probe_seq=t["ps"], uniform_override=t["ovr"], seed=seed, lead_slots=lead,
                     vocab=x["vocab"], max_gamma=max(int(np.diff(cu).max()) if Bn else 0, 0),
                     total_draft_rows=n_d, row_stride=x["stride"], top_k=t["topk"],
                     eos_token=t["eos"], max_emit=t["cap"], num_emitted=t["nemit"])
    if noalloc:
        B.spec_verify_chain_noalloc(a)
    else:
        B.spec_verify_chain(a, workspace=workspace)
    torch.cuda.synchronize()
    return dict(out_tokens=t["out"].cpu().numpy()[:n_t], num_accepted=t["nacc"].cpu().numpy(),
                num_emitted=t["nemit"].cpu().numpy(),
                committed_len=t["L"].cpu().numpy(), seq_flags=t["flags"].cpu().numpy(),
                probe_rows=None if not probes else t["pr"].cpu().numpy()[:n_d].astype(np.float64),
                probe_seq=None if not probes else t["ps"].cpu().numpy().astype(np.float64))


def _close(a, b, tol):
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | (np.abs(a - b) <= tol)))


class Boundary:
    """Near-boundary sequences of one comparison, by the kind of their first such decision:
    ``acceptance`` (|u - a| < 1e-5 at a tested position), ``topp`` (the top-p cut of a tested
    position's p or q row), ``draw`` (the final residual/bonus draw's CDF step, or R < 1e-5),
    ``draw_topp`` (the bonus row's top-p cut). ``disagreed`` lists those whose GPU result
    differs from the oracle's after that decision (accepted count, emitted count or tokens)."""

    KINDS = ("acceptance", "topp", "draw", "draw_topp")

    def __init__(self):
        for k in self.KINDS:
            setattr(self, k, [])
        self.disagreed = []

    @property
    def before_draw(self):
        """Sequences whose first near-boundary decision precedes the final draw."""
        return self.acceptance + self.topp

    @property
    def at_draw(self):
        return self.draw + self.draw_topp

    def counts(self):
        return {k: len(getattr(self, k)) for k in self.KINDS}

    def __iter__(self):  # (before the draw, at the draw), as two lists
        return iter((self.before_draw, self.at_draw))


def compare_chain(x, o, g, exact=False, probes=True):
    """Asserts parity sequence by sequence and returns the near-boundary sequences
    (:class:`Boundary`).

    A sequence whose first near-boundary decision is the acceptance test or a top-p cut at
    draft position kb is compared up to it: the kb - 1 accepted drafts (both sides accept
    them; nothing before kb is uncertain), their tokens and per-row probabilities, and at kb
    itself the probabilities when only the acceptance test is uncertain (the law is not).
    One whose first near-boundary decision is the final draw is compared up to the draw:
    accepted count, committed length, accepted tokens, per-row probabilities."""
    cu = x["cu_gamma"]
    Bn = len(cu) - 1
    bnd = Boundary()
    tol = 0.0 if exact else PROB_TOL
    for b in range(Bn):
        m_acc, m_all = (np.inf, np.inf) if exact else o["margin"][b]
        n = int(o["num_accepted"][b])
        t0, d0 = int(cu[b]) + b, int(cu[b])
        gb = int(cu[b + 1] - cu[b])
        ctx = f"seq {b}: oracle n={n} flags={o['seq_flags'][b]} gpu n={g['num_accepted'][b]}"
        if m_acc < MARGIN:
            rm = o["row_margin"][d0:d0 + gb]
            near = np.flatnonzero(rm.min(axis=1) < MARGIN)
            assert near.size, ctx  # the sequence margin comes from one of its positions
            kb = int(near[0])  # 0-based: positions 0..kb-1 are certain accepts
            law_ok = rm[kb, 1] >= MARGIN
            (bnd.acceptance if law_ok else bnd.topp).append(b)
            assert g["num_accepted"][b] >= kb, ctx
            assert np.array_equal(g["out_tokens"][t0:t0 + kb], o["out_tokens"][t0:t0 + kb]), ctx
            if probes and g["probe_rows"] is not None:
                m = kb + 1 if law_ok else kb
                assert _close(g["probe_rows"][d0:d0 + m], o["probe_rows"][d0:d0 + m], tol), ctx
            ne = int(o["num_emitted"][b])
            same = (int(g["num_accepted"][b]) == n and int(g["num_emitted"][b]) == ne and
                    np.array_equal(g["out_tokens"][t0:t0 + ne], o["out_tokens"][t0:t0 + ne]))
            if not same:
                bnd.disagreed.append(b)
            continue
        full = m_all >= MARGIN
        if not full:
            dm = o["draw_margin"][b]
            (bnd.draw_topp if dm[0] < MARGIN else bnd.draw).append(b)
        assert g["num_accepted"][b] == n, ctx
        assert g["committed_len"][b] == o["committed_len"][b], ctx
        ign = B.FLAG_TOPP_SLOW | (0 if full else B.FLAG_RESID_FALLBACK)
        assert (g["seq_flags"][b] & ~ign) == (o["seq_flags"][b] & ~ign), ctx
        if o["seq_flags"][b] & (B.FLAG_BAD_TOKEN | B.FLAG_BAD_PARAM):
            continue
        ne = int(o["num_emitted"][b])
        drawn = ne == n + 1  # no early stop inside the accepted drafts
        if full:
            assert g["num_emitted"][b] == ne, ctx
        m = ne if full else n
        assert np.array_equal(g["out_tokens"][t0:t0 + m], o["out_tokens"][t0:t0 + m]), ctx
        if not full and (int(g["num_emitted"][b]) != ne or
                         not np.array_equal(g["out_tokens"][t0:t0 + ne],
                                            o["out_tokens"][t0:t0 + ne])):
            bnd.disagreed.append(b)
        if probes and g["probe_rows"] is not None:
            tested = min(n + 1, gb) if drawn else n
            assert _close(g["probe_rows"][d0:d0 + tested], o["probe_rows"][d0:d0 + tested],
                          tol), ctx
            if full:
                assert _close(g["probe_seq"][b], o["probe_seq"][b], tol), ctx
    return bnd


# Parity report of the session: one entry per comparison, written by conftest at the end of
# the session to the file named by SPECV_PARITY_REPORT (if set).
REPORT = []


def record(label, sequences, kind, counts, **extra):
    entry = dict(label=label, sequences=int(sequences), kind=kind,
                 boundary={k: int(v) for k, v in counts.items()})
    entry.update(extra)
    REPORT.append(entry)
    say(f"[parity] {label}: {sequences} sequences, near-boundary {entry['boundary']}, "
        f"disagreeing {entry.get('disagreed', '-')}")


def expected_boundary(o, frac_slack=5.0):
    """Expected number of draw-boundary sequences if the oracle's margins are right: a
    draw whose chosen token has probability w (in the uniform's units) sits within 1e-5 of
    one of its two boundaries with probability min(1, 2e-5 / w)."""
    w = o["probe_seq"][:, 1]
    w = w[np.isfinite(w) & (w > 0)]
    e = float(np.minimum(1.0, 2 * MARGIN / w).sum())
    return e + frac_slack * np.sqrt(e) + 3


def check_chain(x, seed=1234, override=None, lead=1, tokens=None, exact=False, label="",
                max_acc_boundary_frac=0.02):
    say(f"[chain] {label}: B={len(x['cu_gamma']) - 1} V={x['vocab']} stride={x['stride']} "
        f"draft_rows={int(x['cu_gamma'][-1])} seed={seed}")
    if tokens is None:
        tokens = draft_tokens_oracle(x)
    o = run_oracle_chain(x, tokens, seed, override, lead)
    say(f"[chain] {label}: oracle done; launching GPU")
    g = run_gpu_chain(x, tokens, seed, override, lead)
    bnd = compare_chain(x, o, g, exact=exact)
    Bn = len(x["cu_gamma"]) - 1
    record(label, Bn, "chain greedy" if exact else "chain", bnd.counts(),
           disagreed=len(bnd.disagreed), draft_rows=int(x["cu_gamma"][-1]),
           vocab=int(x["vocab"]))
    # acceptance tests sit within 1e-5 of their boundary with probability ~2e-5 per test
    assert len(bnd.before_draw) <= max(2, max_acc_boundary_frac * Bn)
    if override is None and not exact:
        assert len(bnd.at_draw) <= expected_boundary(o)
    return o, g, bnd
