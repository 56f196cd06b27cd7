"""The vocab-4 Markov workload as a speculative stream ("投机解码" glossary page, the runnable
experiment: a first-order Markov target and a perturbed draft table, tokens emitted until a
fixed count, transition frequencies compared with the target table).

A stream is a sequence of verification rounds over one sequence. The caller supplies the two
sides of a round as callbacks, so that one driver serves the oracle and the GPU library:
``propose(last, pos)`` returns the round's draft tokens (a chain from the draft table
starting after ``last``), and ``verify(last, drafts, pos)`` returns the round's emitted tokens
(the accepted drafts, then the correction or bonus token). The stream is cut at ``n_tokens``
(the last round's surplus is dropped, as the experiment does).
"""
from __future__ import annotations

import numpy as np


class StreamStats:
    def __init__(self):
        self.rounds = 0
        self.accepted = 0  # accepted drafts summed over the rounds

    @property
    def accepted_per_round(self):
        return self.accepted / max(self.rounds, 1)


def run_stream(propose, verify, n_tokens: int, start: int = 0):
    """Returns (emitted tokens as int64 array of length n_tokens, StreamStats)."""
    buf = np.empty(n_tokens, np.int64)
    st = StreamStats()
    filled, last = 0, start
    while filled < n_tokens:
        drafts = propose(last, filled)
        emitted = np.asarray(verify(last, drafts, filled), np.int64)
        st.rounds += 1
        st.accepted += len(emitted) - 1
        take = min(len(emitted), n_tokens - filled)
        buf[filled:filled + take] = emitted[:take]
        filled += take
        last = int(buf[filled - 1])
    return buf, st


def transition_freq(tokens, V: int = 4, start: int = 0):
    """Row-normalised counts of (previous, next) pairs over the stream, the first token's
    predecessor being ``start``."""
    t = np.asarray(tokens, np.int64)
    prev = np.concatenate(([start], t[:-1]))
    counts = np.bincount(prev * V + t, minlength=V * V).reshape(V, V).astype(np.float64)
    return counts / counts.sum(axis=1, keepdims=True)


def oracle_proposer(oracle, draft_rows, gamma, seed_draft, vocab=4):
    """Draft chain from the draft table's bf16 rows, drawn by the oracle one token at a time
    (purpose BONUS of a gamma = 0 round keyed (seed_draft, 0, pos + j))."""
    one = np.ones(1, np.float32)
    sid = np.zeros(1, np.uint32)

    def propose(last, pos):
        chain = []
        for j in range(gamma):
            prev = chain[-1] if chain else last
            t = oracle.draw_tokens(draft_rows[prev:prev + 1], one, None, seed_draft, sid,
                                   np.array([pos + j], np.int32), vocab=vocab,
                                   nthreads=1)
            chain.append(int(t[0]))
        return chain

    return propose


def round_rows(target_rows, draft_rows, last, drafts):
    """The round's logits rows: target rows after [last, d_1..d_gamma], draft rows after
    [last, d_1..d_{gamma-1}]."""
    ctx = [last] + list(drafts)
    return target_rows[ctx], draft_rows[ctx[:-1]]
