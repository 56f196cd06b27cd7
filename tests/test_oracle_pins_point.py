"""Pins of the oracle's point-mass draft law (reading R24 of oracle/spec_oracle.c): a drafter
without a law -- the n-gram prompt lookup -- proposes each draft with certainty, so with no
draft rows and T > 0 the draft law q_k is the point mass at d_k ("KV Cache 优化（四）" §4 eq.
a(x) and eq. p'(x) with that q: a = min(1, p(d)), residual = p without d).

Pinned against: the output law integrated over the uniforms (it must be p exactly); the
chain's probes against the oracle's own row laws (already pinned elsewhere) and the residual
and bonus draws against numpy inverse CDFs.
"""
import numpy as np
import pytest

from draft_verification_03_amd import workloads as W

from test_oracle_pins import _threshold


@pytest.mark.parametrize("seed", range(6))
def test_point_mass_output_law_is_p(orc, seed):
    """P(out = v) = P(accept) [v = d] + P(reject) r_v / R = p(d)[v = d] + p_v [v != d] = p_v,
    measured on the oracle's one-position step by bisection over u_acc and u_res."""
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 7))
    p = rng.integers(0, 9, size=V).astype(float)
    p[rng.integers(0, V)] += 1
    p /= p.sum()
    d = int(rng.integers(0, V))
    q = np.zeros(V)
    q[d] = 1.0
    a = _threshold(lambda u: orc.position_step(p, q, d, u, 0.5)[0])
    a = a if orc.position_step(p, q, d, 0.0, 0.5)[0] else 0.0
    assert abs(a - p[d]) < 1e-12  # acceptance probability min(1, p(d)/1)
    out = np.zeros(V)
    out[d] += a
    if p[d] < 1.0:
        tok_at = lambda u: orc.position_step(p, q, d, 1.0, u)[1]  # noqa: E731 (u_acc=1 rejects)
        prev = 0.0
        for x in range(V):
            end = _threshold(lambda u: tok_at(u) <= x)
            if tok_at(0.0) <= x:
                out[x] += (1 - a) * (end - prev)
                prev = end
        assert tok_at(0.0) != d and tok_at(0.999999) != d  # the residual never draws d
    assert np.max(np.abs(out - p)) < 1e-9


@pytest.mark.parametrize("T,P", [(0.8, 1.0), (1.0, 0.9), (0.5, 0.6)])
def test_chain_with_point_mass_drafts(orc, T, P):
    """No draft rows, T > 0: probes read q(d) = 1 and p(d) from the row's law; a forced
    rejection (u_acc = 1) draws the inverse CDF of p without d; full acceptance (u_acc = 0,
    every p(d) > 0) ends with the bonus draw from p_{gamma+1}."""
    rng = np.random.default_rng(int(T * 10 + P * 100))
    V, B, g = 200, 6, 4
    cu = np.arange(0, B * g + 1, g).astype(np.int32)
    tgt = W.bf16_bits(rng.standard_normal((B * (g + 1), V)).astype(np.float32) * 2)
    tgt_f = W.bf16_to_f32(tgt)
    toks = np.array([int(np.argmax(tgt_f[(i // g) * (g + 1) + i % g])) for i in range(B * g)],
                    np.int32)  # the rows' argmax: inside every nucleus
    Ts = np.full(B, T, np.float32)
    Ps = np.full(B, P, np.float32)
    u = rng.random(B * (g + 1)).astype(np.float32)
    for reject in (True, False):
        ovr = np.zeros((B * (g + 1), 2), np.float32)
        ovr[:, 0] = 1.0 if reject else 0.0
        ovr[:, 1] = u
        r = orc.verify_chain_v(tgt, None, cu, toks, Ts, Ps, None, np.zeros(B, np.int32),
                               uniform_override=ovr, vocab=V)
        for b in range(B):
            t0 = cu[b] + b
            if reject:
                assert r["num_accepted"][b] == 0
                p, _ = orc.dist(tgt[t0], float(Ts[b]), float(Ps[b]))
                assert abs(r["probe_rows"][cu[b], 0] - p[toks[cu[b]]]) < 1e-13
                assert r["probe_rows"][cu[b], 1] == 1.0
                res = p.copy()
                res[toks[cu[b]]] = 0.0
                if res.sum() > 0:
                    want = int(np.searchsorted(np.cumsum(res) / res.sum(), u[t0], side="right"))
                else:  # p(d) = 1 (a nucleus of one token): no residual mass, the draw is from p
                    want = int(np.searchsorted(np.cumsum(p), u[t0], side="right"))
                    assert r["seq_flags"][b] & orc.F_RESID_FALLBACK
                assert r["out_tokens"][t0] == want
            else:
                assert r["num_accepted"][b] == g
                p, _ = orc.dist(tgt[t0 + g], float(Ts[b]), float(Ps[b]))
                want = int(np.searchsorted(np.cumsum(p), u[t0 + g], side="right"))
                assert r["out_tokens"][t0 + g] == want
