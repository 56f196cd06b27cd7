"""Pins of the exact-rational mini-oracle (oracle/exact.py) against what the pages fix:
the printed worked examples (tests/golden/worked_examples.json) and the losslessness
identity P(output x) = min(p, q) + max(0, p - q) = p, checked by exhaustive enumeration."""
import json
import os
import random
from fractions import Fraction as F

import pytest

from oracle import exact

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def fr(xs):
    return [F(x) for x in xs]


def test_three_token_example():
    g = GOLD["three_token"]
    p, q = fr(g["p"]), fr(g["q"])
    assert [exact.accept_prob(p, q, x) for x in range(3)] == fr(g["acceptance"])
    assert exact.acceptance_rate(p, q) == F(g["acceptance_rate"])
    assert exact.residual(p, q) == fr(g["residual"])
    assert exact.output_law(p, q) == fr(g["output"])


def test_ab_example():
    g = GOLD["a_b"]
    p, q = fr(g["p"]), fr(g["q"])
    assert [exact.accept_prob(p, q, x) for x in range(2)] == fr(g["acceptance"])
    assert [q[x] * exact.accept_prob(p, q, x) for x in range(2)] == fr(g["accepted_mass"])
    assert exact.output_law(p, q) == fr(g["output"])


def _rand_law(rng, V, zeros=True):
    w = [rng.randint(0 if zeros else 1, 9) for _ in range(V)]
    if sum(w) == 0:
        w[rng.randrange(V)] = 1
    s = sum(w)
    return [F(x, s) for x in w]


@pytest.mark.parametrize("seed", range(40))
def test_one_position_law_is_target(seed):
    """Exhaustive: the emitted token's law equals p, and the acceptance rate is 1 - TV."""
    rng = random.Random(seed)
    V = rng.randint(1, 6)
    p, q = _rand_law(rng, V), _rand_law(rng, V)
    assert exact.output_law(p, q) == p
    tv = sum(abs(a - b) for a, b in zip(p, q)) / 2
    assert exact.acceptance_rate(p, q) == 1 - tv


@pytest.mark.parametrize("seed", range(6))
def test_round_stream_is_target_autoregressive(seed):
    """Sequence level, exhaustive for gamma <= 3, V <= 3: the stream a round starts (tokens
    after the round come from the target) has the target's autoregressive law."""
    rng = random.Random(100 + seed)
    V = rng.randint(2, 3)
    gamma = rng.randint(1, 3)
    tp = {}
    tq = {}

    def law(table, pre):
        key = pre[-2:]
        if key not in table:
            table[key] = _rand_law(rng, V, zeros=(seed % 2 == 0))
        return table[key]

    p_fn = lambda pre: law(tp, pre)  # noqa: E731
    q_fn = lambda pre: law(tq, pre)  # noqa: E731
    rl = exact.round_law(p_fn, q_fn, gamma)
    assert sum(rl.values()) == 1
    assert all(1 <= len(e) <= gamma + 1 for e in rl)
    for n in range(1, gamma + 2):
        assert exact.stream_law(p_fn, rl, n) == exact.target_law(p_fn, n)


def test_markov_experiment_long_run():
    """The glossary page's vocab-4 experiment: exact long-run accepted drafts per call and
    target calls per token of its tables, against its printed Monte-Carlo run (3.512 and
    0.222 over ~22,000 calls; the per-call standard deviation is ~1.1, so the printed figure
    sits within 3 standard errors of the exact value)."""
    g = GOLD["markov_experiment"]
    T = [[F(str(x)) for x in r] for r in g["target"]]
    D = [[F(str(x)) for x in r] for r in g["draft"]]
    acc, cpt = exact.markov_long_run(T, D, g["k"])
    se = 1.13 / (g["tokens"] * float(cpt)) ** 0.5
    assert abs(float(acc) - g["printed_accepted_per_call"]) < 3 * se
    assert abs(float(cpt) - g["printed_calls_per_token"]) < 5e-4
    # accepted per call and calls per token are tied by tokens/call = accepted + 1
    assert cpt == 1 / (acc + 1)
