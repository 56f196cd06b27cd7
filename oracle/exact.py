"""Exact-rational mini-oracle of speculative sampling -- TEST INFRASTRUCTURE.

Works on probability vectors of ``fractions.Fraction`` (no logits, no floating point), so
the pages' worked examples and the losslessness identity can be checked with equality.

Sources: "KV Cache 优化（四）：Speculative Decoding 投机解码" §4 (eq. a(x), eq. p'(x)) and
§5 (bonus token); "10.6 投机解码" (llm_internals) §10.6.1 (the five steps of a round and the
argument that the output law is p), §10.6.2 (tokens per round); the LLM-glossary page
"投机解码", section on exact acceptance (the q = 0 and zero-residual edge cases).
"""
from __future__ import annotations

from fractions import Fraction
from itertools import product


def accept_prob(p, q, x):
    """a(x) = min(1, p(x)/q(x)); where q(x) = 0 the ratio is not needed: 1 if p(x) > 0."""
    if q[x] > 0:
        return min(Fraction(1), Fraction(p[x]) / Fraction(q[x]))
    return Fraction(1) if p[x] > 0 else Fraction(0)


def residual(p, q):
    """norm(max(0, p - q)); when the positive part has no mass, p itself."""
    r = [max(Fraction(0), Fraction(a) - Fraction(b)) for a, b in zip(p, q)]
    R = sum(r)
    if R == 0:
        return [Fraction(a) for a in p]
    return [x / R for x in r]


def acceptance_rate(p, q):
    """Probability that one drafted token (drawn from q) is accepted."""
    return sum(Fraction(q[d]) * accept_prob(p, q, d) for d in range(len(q)))


def output_law(p, q):
    """Law of the token one position emits: the drafted token when accepted, else a draw
    from the residual."""
    V = len(p)
    rej = 1 - acceptance_rate(p, q)
    r = residual(p, q)
    return [Fraction(q[x]) * accept_prob(p, q, x) + rej * r[x] for x in range(V)]


def round_law(p_fn, q_fn, gamma, ctx=()):
    """Exact law of what one round emits, as {emitted tuple: probability}.

    p_fn(prefix) / q_fn(prefix) return the target / draft law of the next token after the
    context extended by ``prefix``. The drafter proposes d_1..d_gamma one by one from q;
    positions are tested left to right; the first rejection emits a residual draw and ends
    the round; a round with every draft accepted adds one token from p_{gamma+1}.
    """
    law = {}
    V = len(p_fn(tuple(ctx)))
    for d in product(range(V), repeat=gamma):
        pd = Fraction(1)
        pre = tuple(ctx)
        for k in range(gamma):
            pd *= Fraction(q_fn(pre)[d[k]])
            pre = pre + (d[k],)
        if pd == 0:
            continue
        reach = pd  # probability of drafting d and accepting d_1..d_k so far
        pre = tuple(ctx)
        for k in range(gamma):
            p, q = p_fn(pre), q_fn(pre)
            a = accept_prob(p, q, d[k])
            rej = reach * (1 - a)
            if rej:
                for y, ry in enumerate(residual(p, q)):
                    if ry:
                        e = tuple(d[:k]) + (y,)
                        law[e] = law.get(e, Fraction(0)) + rej * ry
            reach *= a
            pre = pre + (d[k],)
            if reach == 0:
                break
        if reach:
            for y, py in enumerate(p_fn(pre)):
                if py:
                    e = tuple(d) + (y,)
                    law[e] = law.get(e, Fraction(0)) + reach * Fraction(py)
    return law


def target_law(p_fn, n, ctx=()):
    """Law of n tokens sampled one by one from the target: {tuple: probability}."""
    law = {(): Fraction(1)}
    for _ in range(n):
        nxt = {}
        for s, ps in law.items():
            for y, py in enumerate(p_fn(tuple(ctx) + s)):
                if py:
                    nxt[s + (y,)] = nxt.get(s + (y,), Fraction(0)) + ps * Fraction(py)
        law = nxt
    return law


def stream_law(p_fn, round_lw, n, ctx=()):
    """Law of the first n tokens of the stream a round starts, when tokens after the round's
    last emitted one come from the target itself."""
    out = {}
    for e, pe in round_lw.items():
        if len(e) >= n:
            s = e[:n]
            out[s] = out.get(s, Fraction(0)) + pe
        else:
            for tail, pt in target_law(p_fn, n - len(e), tuple(ctx) + e).items():
                s = e + tail
                out[s] = out.get(s, Fraction(0)) + pe * pt
    return out


def markov_long_run(target, draft, gamma):
    """Long-run accepted drafts per round and rounds per emitted token, exactly, for
    first-order Markov target/draft tables (rows = previous token), by the stationary law of
    the round-start token. Returns (accepted_per_call, calls_per_token)."""
    V = len(target)
    laws = []
    for s in range(V):
        def p_fn(pre, s=s):
            return target[pre[-1] if pre else s]

        def q_fn(pre, s=s):
            return draft[pre[-1] if pre else s]
        laws.append(round_law(p_fn, q_fn, gamma))
    # Transition matrix of the round-start token, and per-state expected lengths.
    M = [[Fraction(0)] * V for _ in range(V)]
    elen = []
    for s in range(V):
        el = Fraction(0)
        for e, pe in laws[s].items():
            M[s][e[-1]] += pe
            el += pe * len(e)
        elen.append(el)
    pi = _stationary(M)
    mean_len = sum(pi[s] * elen[s] for s in range(V))
    return mean_len - 1, 1 / mean_len


def _stationary(M):
    """Solve pi M = pi, sum(pi) = 1 exactly by Gaussian elimination over Fractions."""
    V = len(M)
    A = [[(M[j][i] - (1 if i == j else 0)) for j in range(V)] for i in range(V)]
    A[-1] = [Fraction(1)] * V
    b = [Fraction(0)] * (V - 1) + [Fraction(1)]
    for c in range(V):
        piv = next(r for r in range(c, V) if A[r][c] != 0)
        A[c], A[piv] = A[piv], A[c]
        b[c], b[piv] = b[piv], b[c]
        for r in range(V):
            if r != c and A[r][c] != 0:
                f = A[r][c] / A[c][c]
                A[r] = [x - f * y for x, y in zip(A[r], A[c])]
                b[r] -= f * b[c]
    return [b[i] / A[i][i] for i in range(V)]
