"""The vocab-4 Markov workload on the GPU (B = 1, gamma = 4, 100,000 emitted tokens), and the
glossary page's own tables ("投机解码", the runnable experiment). The stream is the GPU's:
each round is verified by the library and the stream continues from the library's emitted
tokens; the oracle verifies the same round and must agree (decisions within 1e-5 of their
boundary excepted, counted and reported). The transition frequencies of the GPU's stream
must lie within 0.02 of the target table (the page's pass criterion)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from draft_verification_03_amd import binding as B
from draft_verification_03_amd import workloads as W

from harness import MARGIN, record, say
from markov_stream import oracle_proposer, round_rows, run_stream, transition_freq

pytestmark = pytest.mark.gpu

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


class GpuRound:
    """One sequence's verification round through the C ABI on device buffers that are reused
    round after round; each call is checked against the oracle on the same inputs."""

    def __init__(self, T, D, gamma, seed):
        self.tl, self.dl = W.log_rows_bf16(T), W.log_rows_bf16(D)
        self.gamma, self.seed = gamma, seed
        i32 = dict(dtype=torch.int32, device="cuda")
        self.d_tgt = torch.zeros((gamma + 1, 8), dtype=torch.int16, device="cuda")
        self.d_drf = torch.zeros((gamma, 8), dtype=torch.int16, device="cuda")
        self.d_tok = torch.zeros(gamma, **i32)
        self.d_L = torch.zeros(1, **i32)
        self.d_out = torch.zeros(gamma + 1, **i32)
        self.d_n = torch.zeros(1, **i32)
        self.d_e = torch.zeros(1, **i32)
        self.ws = torch.empty(B.spec_verify_chain_workspace_size(1, gamma, 4),
                              dtype=torch.uint8, device="cuda")
        self.args = B.chain_args(
            target_logits=self.d_tgt, draft_logits=self.d_drf,
            cu_gamma=torch.tensor([0, gamma], **i32), draft_tokens=self.d_tok,
            temperature=torch.ones(1, dtype=torch.float32, device="cuda"),
            committed_len=self.d_L, out_tokens=self.d_out, num_accepted=self.d_n,
            num_emitted=self.d_e, seq_flags=torch.zeros(1, **i32), seed=seed, vocab=4,
            max_gamma=gamma, total_draft_rows=gamma, row_stride=8)
        self.boundary = 0
        self.disagreed = 0

    def __call__(self, last, drafts, pos):
        tgt, drf = round_rows(self.tl, self.dl, last, drafts)
        self.d_tgt.copy_(torch.from_numpy(np.ascontiguousarray(tgt).view(np.int16)))
        self.d_drf.copy_(torch.from_numpy(np.ascontiguousarray(drf).view(np.int16)))
        self.d_tok.copy_(torch.tensor(drafts, dtype=torch.int32))
        self.d_L.fill_(pos)
        B.spec_verify_chain(self.args, workspace=self.ws)
        ne = int(self.d_e.item())
        gpu = self.d_out.cpu().numpy()[:ne]
        o = oracle.verify_chain_v(tgt, drf, np.array([0, self.gamma], np.int32),
                                  np.array(drafts, np.int32), np.ones(1, np.float32), None,
                                  np.zeros(1, np.uint32), np.array([pos], np.int32),
                                  seed=self.seed, vocab=4, nthreads=1)
        n = int(o["num_accepted"][0])
        m_acc, m_all = o["margin"][0]
        if m_all < MARGIN:
            self.boundary += 1
        if m_acc >= MARGIN:  # the accepted count and the pointer are certain
            assert int(self.d_n.item()) == n and int(self.d_L.item()) == pos + 1 + n, pos
            k = n + 1 if m_all >= MARGIN else n
            assert np.array_equal(gpu[:k], o["out_tokens"][:k]), pos
        if not np.array_equal(gpu, o["out_tokens"][:int(o["num_emitted"][0])]):
            self.disagreed += 1  # a boundary round: the stream follows the GPU
        return gpu


def gpu_stream(T, D, n_tokens, gamma=4, seed=303, seed_draft=909):
    rnd = GpuRound(T, D, gamma, seed)
    propose = oracle_proposer(oracle, rnd.dl, gamma, seed_draft)
    toks, st = run_stream(propose, rnd, n_tokens)
    return toks, st, rnd


def test_markov_dirichlet_workload():
    T, D = W.markov_tables()
    say("[markov] Dirichlet(2) tables, 100000 tokens, gamma=4")
    toks, st, rnd = gpu_stream(T, D, 100000)
    f = transition_freq(toks)
    say(f"[markov] rounds={st.rounds} accepted/round={st.accepted_per_round:.4f} "
        f"boundary rounds={rnd.boundary} (GPU and oracle differ in {rnd.disagreed}); "
        f"max |freq - T| = {np.abs(f - T).max():.5f}")
    record("c1 Markov B=1 gamma=4 V=4, 100000 tokens", st.rounds, "markov rounds",
           {"acceptance_or_draw": rnd.boundary}, disagreed=rnd.disagreed,
           max_freq_error=float(np.abs(f - T).max()))
    assert np.abs(f - T).max() < 0.02
    assert rnd.boundary <= 5 and rnd.disagreed <= rnd.boundary


def test_markov_page_tables():
    g = GOLD["markov_experiment"]
    T, D = np.array(g["target"]), np.array(g["draft"])
    say("[markov] glossary page tables, 100000 tokens, k=4")
    toks, st, rnd = gpu_stream(T, D, g["tokens"], gamma=g["k"])
    f = transition_freq(toks)
    say(f"[markov] accepted/round={st.accepted_per_round:.4f} "
        f"rounds/token={st.rounds / g['tokens']:.4f} boundary rounds={rnd.boundary}")
    record("glossary Markov tables, k=4, 100000 tokens", st.rounds, "markov rounds",
           {"acceptance_or_draw": rnd.boundary}, disagreed=rnd.disagreed,
           max_freq_error=float(np.abs(f - T).max()))
    assert np.abs(f - T).max() < g["max_error"]
    assert abs(st.accepted_per_round - g["printed_accepted_per_call"]) < 0.06
    assert rnd.disagreed <= rnd.boundary
