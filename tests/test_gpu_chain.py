"""GPU parity of spec_verify_chain against the fp64 oracle, through the C ABI.

Full-size workloads (the chain configurations at their stated sizes), small cases that
span several 512-logit tiles with a ragged tail, greedy bit-exactness, edge cases, the
uniform-override decision grid on the pages' worked examples, determinism and
independence from batch composition."""
import numpy as np
import pytest
import torch

import oracle
from draft_verification_03_amd import binding as B
from draft_verification_03_amd import workloads as W

from harness import (check_chain, compare_chain, draft_tokens_oracle, run_gpu_chain,
                     run_oracle_chain, say)

pytestmark = pytest.mark.gpu


# ---- full-size workloads --------------------------------------------------------------

def test_c2_full():
    check_chain(W.chain_inputs("c2"), seed=11, label="c2 B=64 gamma=4 V=32000 T=1")


def test_c2_full_greedy_bit_exact():
    check_chain(W.chain_inputs("c2", temperature=0.0), seed=12, exact=True,
                label="c2 greedy")


def test_c3_full():
    o, g, bnd = check_chain(W.chain_inputs("c3"), seed=13,
                            label="c3 B=256 gamma=8 V=128256 T=0.7 top-p 0.9")
    slow = int(((g["seq_flags"] & B.FLAG_TOPP_SLOW) != 0).sum())
    say(f"[chain] c3: sequences with a multi-pass top-p row: {slow}")


@pytest.mark.parametrize("P,K", [(0.9, None), (0.8, 40), (None, None)])
def test_batch_beyond_the_cus(P, K):
    """B=300 > 256 compute units: the resolve runs two 512-thread workgroups per CU. Top-p
    (list draws from the prefetched list heads), top-k, and no filter (row draws)."""
    x = W.chain_inputs("c3", B=300, V=20000, top_p=P)
    if K is not None:
        x["top_k"] = np.where(np.arange(300) % 2 == 0, K, 0).astype(np.int32)
    check_chain(x, seed=16, label=f"B=300 V=20000 top-p {P} top-k {K}")


def test_c5_full():
    check_chain(W.chain_inputs("c5"), seed=15, label="c5 ragged B=1024 V=128256")


# ---- small cases: tiles, ragged tails, mixed modes ----------------------------------------

@pytest.mark.parametrize("V,stride", [(1001, 1008), (4099, 4104), (513, 520), (7, 8), (1, 8)])
def test_ragged_vocab_tail(V, stride):
    x = W.chain_inputs("c2", B=12, V=V, stride=stride, gamma=(0, 6), seed=V)
    check_chain(x, seed=21, label=f"ragged V={V}")


@pytest.mark.parametrize("topp", [0.5, 0.9, 0.99])
def test_top_p_small(topp):
    x = W.chain_inputs("c3", B=16, V=6000, top_p=topp, seed=int(topp * 100))
    check_chain(x, seed=22, label=f"top-p {topp}")


def test_top_p_flat_rows_take_the_exact_search():
    """Flat logits: the nucleus is far wider than the capture window, so the multi-pass
    threshold search runs (flagged) and still matches the oracle."""
    x = W.chain_inputs("c2", B=6, V=3000, gamma=2, temperature=1.0, top_p=0.9, seed=5)
    x["target"][:] = W.bf16_bits(W.bf16_to_f32(x["target"]) * 0.05)
    x["draft"][:] = W.bf16_bits(W.bf16_to_f32(x["draft"]) * 0.05)
    o, g, _ = check_chain(x, seed=23, label="flat top-p")
    assert np.all(g["seq_flags"] & B.FLAG_TOPP_SLOW)


def test_top_p_nuclei_across_list_sizes():
    """Nuclei from tens to hundreds of tokens: plateaus of K boosted ids (+8 over N(0, 0.3^2)),
    K chosen so that the kept lists cross the sizes at which the resolve step switches from
    drawing over the lists to a pass over the row pair."""
    rng = np.random.default_rng(41)
    V, stride, gamma = 12000, 12000, 4
    Ks = [40, 70, 150, 250, 290, 600]
    Bn = len(Ks)
    tgt = np.zeros((Bn * (gamma + 1), stride), np.float32)
    drf = np.zeros((Bn * gamma, stride), np.float32)
    for b, K in enumerate(Ks):
        ids = rng.choice(V, size=K, replace=False)
        for k in range(gamma + 1):
            row = rng.normal(0.0, 0.3, V).astype(np.float32)
            row[ids] += 8.0
            tgt[b * (gamma + 1) + k] = row
            if k < gamma:
                drf[b * gamma + k] = row + rng.normal(0.0, 0.5, V).astype(np.float32)
    x = dict(target=W.bf16_bits(tgt), draft=W.bf16_bits(drf),
             cu_gamma=np.arange(Bn + 1, dtype=np.int32) * gamma,
             temperature=np.ones(Bn, np.float32), top_p=np.full(Bn, 0.9, np.float32),
             seq_id=np.arange(Bn, dtype=np.uint32),
             committed_len=rng.integers(0, 4096, Bn).astype(np.int32), vocab=V, stride=stride)
    sizes = [oracle.dist(x["target"][r, :V], 1.0, 0.9)[1]["nucleus"]
             for r in range(0, Bn * (gamma + 1), gamma + 1)]
    assert min(sizes) < 64 and any(64 < n <= 256 for n in sizes) and max(sizes) > 256, sizes
    for seed in (42, 43, 44):
        check_chain(x, seed=seed, label=f"top-p list sizes {sizes} seed {seed}")


def _window_rows(rng, V, n_top, n_window):
    """Rows with n_top tied logits at 12, n_window logits spread over [5.5, 7] (inside a 7*T
    window at T = 1, but with little mass) and the rest near -6."""
    row = rng.normal(-6.0, 1.0, V).astype(np.float32)
    ids = rng.choice(V, size=n_top + n_window, replace=False)
    row[ids[:n_top]] = 12.0
    row[ids[n_top:]] = rng.uniform(5.5, 7.0, n_window).astype(np.float32)
    return row


def test_top_p_window_beyond_the_candidate_buffer():
    """More than 1024 logits inside the capture window, a nucleus of ten: the list is built by
    the pass over the captured vectors (some of them spilled), not from the bins' candidates,
    and still matches the oracle."""
    rng = np.random.default_rng(77)
    V, gamma, Bn = 20000, 3, 8
    tgt = np.stack([_window_rows(rng, V, 10, 1100) for _ in range(Bn * (gamma + 1))])
    drf = np.stack([tgt[b * (gamma + 1) + k] + rng.normal(0.0, 0.3, V).astype(np.float32)
                    for b in range(Bn) for k in range(gamma)])
    x = dict(target=W.bf16_bits(tgt), draft=W.bf16_bits(drf),
             cu_gamma=np.arange(Bn + 1, dtype=np.int32) * gamma,
             temperature=np.ones(Bn, np.float32), top_p=np.full(Bn, 0.5, np.float32),
             seq_id=np.arange(Bn, dtype=np.uint32),
             committed_len=rng.integers(0, 4096, Bn).astype(np.int32), vocab=V, stride=V)
    row0 = W.bf16_to_f32(x["target"][0])
    assert int((row0 >= row0.max() - 7.0).sum()) > 1024
    assert oracle.dist(x["target"][0], 1.0, 0.5)[1]["nucleus"] == 10
    o, g, _ = check_chain(x, seed=29, label="window beyond the candidate buffer")
    assert not np.any(g["seq_flags"] & B.FLAG_TOPP_SLOW)


@pytest.mark.parametrize("V,topp", [(128256, 0.9), (128256, None), (200000, 0.9),
                                    (200000, None)])
def test_every_draft_accepted_bonus_draw(V, topp):
    """Draft rows equal to target rows: every test accepts (p = q), so every sequence ends
    with the bonus draw from p_{gamma+1}, whose law the resolve step computes itself -- from
    registers up to 16384 vectors per row, by streaming passes beyond."""
    x = W.chain_inputs("c3", B=12, V=V, gamma=(0, 6), top_p=topp, seed=45)
    cu = x["cu_gamma"]
    x["draft"] = x["target"][np.concatenate(
        [np.arange(int(cu[b]) + b, int(cu[b + 1]) + b) for b in range(12)]).astype(int)].copy()
    o, g, _ = check_chain(x, seed=46, label=f"all accepted V={V} top-p={topp}")
    assert np.all(o["num_accepted"] == np.diff(cu))


def test_mixed_temperatures_and_greedy():
    x = W.chain_inputs("c5", B=40, V=5000, seed=3)
    x["temperature"][::3] = 0.0
    x["temperature"][1::7] = 0.05
    check_chain(x, seed=24, label="mixed T incl. greedy")


def test_gamma_zero_and_max_gamma():
    x = W.chain_inputs("c2", B=8, V=2000, gamma=(0, 0), seed=6)
    check_chain(x, seed=25, label="gamma=0 (bonus only)")
    x = W.chain_inputs("c2", B=3, V=600, gamma=64, seed=7, temperature=0.3)
    x["draft"] = x["target"][np.concatenate([np.arange(int(x['cu_gamma'][b]) + b,
                                                      int(x['cu_gamma'][b]) + b + 64)
                                            for b in range(3)])].copy()
    check_chain(x, seed=26, label="gamma=64, draft == target rows")


@pytest.mark.parametrize("lead", [0, 1])
def test_lead_slots(lead):
    x = W.chain_inputs("c2", B=10, V=1500, seed=8)
    check_chain(x, seed=27, lead=lead, label=f"lead_slots={lead}")


def test_adversarial_tokens_and_bad_params():
    """Uniformly random drafts (many rejections, q(d) = 0 under top-p), an out-of-range
    token, a negative temperature and a top-p above 1: device-detected, no progress."""
    x = W.chain_inputs("c3", B=12, V=3000, seed=9)
    tok = W.random_tokens(int(x["cu_gamma"][-1]), 3000, seed=1)
    tok[int(x["cu_gamma"][2])] = 3000 + 5
    x["temperature"][4] = -1.0
    x["top_p"][5] = 1.5
    o, g, _ = check_chain(x, seed=28, tokens=tok, label="adversarial")
    assert g["seq_flags"][2] == B.FLAG_BAD_TOKEN and g["num_accepted"][2] == 0
    assert g["seq_flags"][4] == B.FLAG_BAD_PARAM and g["seq_flags"][5] == B.FLAG_BAD_PARAM
    assert g["committed_len"][4] == x["committed_len"][4]
    assert (o["seq_flags"] & oracle.F_Q_ZERO).any()


def test_zero_residual_falls_back_to_p():
    """Draft row == target row, top-p, draft token outside both nuclei: q(d) = 0 and
    p(d) = 0, so the test rejects and the residual has no mass; the draw uses p itself.
    R = 0 exactly on both sides here (identical rows, identical arithmetic per side), so the
    draw is compared too, with the uniform's own margin for the draw from p."""
    x = W.chain_inputs("c3", B=4, V=2000, gamma=1, seed=10)
    x["draft"][:] = x["target"][x["cu_gamma"][:-1] + np.arange(4)]
    tl = W.bf16_to_f32(x["target"])
    tok = np.array([int(np.argmin(tl[int(x['cu_gamma'][b]) + b])) for b in range(4)], np.int32)
    o = run_oracle_chain(x, tok, 29)
    g = run_gpu_chain(x, tok, 29)
    assert np.all(o["seq_flags"] == (oracle.F_Q_ZERO | oracle.F_RESID_FALLBACK))
    assert np.array_equal(g["seq_flags"] & ~B.FLAG_TOPP_SLOW, o["seq_flags"])
    assert np.all(g["num_accepted"] == 0) and np.all(o["probe_seq"][:, 0] == 0.0)
    for b in range(4):
        u = oracle.uniform(29, b, int(x["committed_len"][b]) + 1, oracle.PURPOSE_RESIDUAL)
        p, info = oracle.dist(x["target"][b * 2, :2000], 0.7, 0.9)
        y, margin = oracle.sample(p, u)
        assert o["out_tokens"][2 * b] == y
        if margin >= 1e-5:
            assert g["out_tokens"][2 * b] == y


# ---- the pages' worked examples through the kernel (uniform override grid) -------------

def _example_rows(p, q, reps):
    """bf16 logits rows ln p, ln q (exact enough: the grid compares against the oracle)."""
    V = len(p)
    tl = np.full((reps * 2, 8), 0xFF80, np.uint16)
    dl = np.full((reps, 8), 0xFF80, np.uint16)
    for r in range(reps):
        tl[2 * r, :V] = W.bf16_bits(np.log(np.array(p, np.float32)))
        tl[2 * r + 1, :V] = W.bf16_bits(np.log(np.array(p, np.float32)))
        dl[r, :V] = W.bf16_bits(np.log(np.array(q, np.float32)))
    return tl, dl


@pytest.mark.parametrize("case", ["three_token", "a_b"])
def test_worked_example_decision_grid(case):
    """Every (draft token, u_acc, u_res) on an n x n grid: the kernel's decisions equal the
    oracle's away from boundaries, and the grid law is close to the printed output law."""
    p, q, want = {"three_token": ([.4, .4, .2], [.6, .3, .1], [.4, .4, .2]),
                  "a_b": ([.6, .4], [.8, .2], [.6, .4])}[case]
    V = len(p)
    n = 24
    reps = V * n * n
    tl, dl = _example_rows(p, q, reps)
    cu = np.arange(reps + 1, dtype=np.int32)
    ovr = np.full((2 * reps, 2), 0.4321, np.float32)  # bonus rows: a draw away from u = 0
    tok = np.zeros(reps, np.int32)
    r = 0
    for d in range(V):
        for i in range(n):
            for j in range(n):
                tok[r] = d
                ovr[2 * r, 0] = (i + 0.5) / n
                ovr[2 * r, 1] = (j + 0.5) / n
                r += 1
    x = dict(target=tl, draft=dl, cu_gamma=cu, temperature=np.ones(reps, np.float32),
             top_p=None, seq_id=np.arange(reps, dtype=np.uint32),
             committed_len=np.zeros(reps, np.int32), vocab=V, stride=8)
    o, g, bnd = check_chain(x, seed=0, override=ovr, tokens=tok, label=f"grid {case}")
    qv = np.array([float(np.exp(W.bf16_to_f32(dl[0, :V]).astype(np.float64)[k]))
                   for k in range(V)])
    qv /= qv.sum()
    law = np.zeros(V)
    for rr in range(reps):
        law[g["out_tokens"][2 * rr]] += qv[tok[rr]] / (n * n)
    assert np.abs(law - np.array(want)).max() < 0.03


# ---- properties --------------------------------------------------------------------------

def test_deterministic_and_batch_independent():
    """Same inputs twice: identical bits. A sequence's result depends on its own rows,
    parameters and seq_id only: reversing the batch order (same seq_ids) permutes the
    outputs."""
    x = W.chain_inputs("c3", B=20, V=4000, gamma=(1, 6), seed=12)
    tok = draft_tokens_oracle(x)
    g1 = run_gpu_chain(x, tok, 77)
    g2 = run_gpu_chain(x, tok, 77)
    for k in g1:
        assert np.array_equal(g1[k], g2[k], equal_nan=True), k
    cu = x["cu_gamma"]
    order = np.arange(19, -1, -1)
    gam = np.diff(cu)[order]
    cu2 = np.concatenate([[0], np.cumsum(gam)]).astype(np.int32)
    tr = np.concatenate([x["target"][cu[b] + b:cu[b + 1] + b + 1] for b in order])
    dr = np.concatenate([x["draft"][cu[b]:cu[b + 1]] for b in order])
    tk = np.concatenate([tok[cu[b]:cu[b + 1]] for b in order])
    y = dict(x, target=tr, draft=dr, cu_gamma=cu2, temperature=x["temperature"][order],
             top_p=x["top_p"][order], seq_id=x["seq_id"][order],
             committed_len=x["committed_len"][order])
    g3 = run_gpu_chain(y, tk, 77)
    for i, b in enumerate(order):
        n = g1["num_accepted"][b]
        assert g3["num_accepted"][i] == n
        assert np.array_equal(g3["out_tokens"][cu2[i] + i:cu2[i] + i + n + 1],
                              g1["out_tokens"][cu[b] + b:cu[b] + b + n + 1])


@pytest.mark.parametrize("name", ["c5", "c3"])
def test_repeated_full_size_calls_give_identical_bits(name):
    """The same full-size call twice gives identical bits in every output: the rows' trips
    are claimed by whichever wave is free, so the row statistics must not depend on which
    wave took which trip."""
    x = W.chain_inputs(name)
    tok = draft_tokens_oracle(x)
    g1 = run_gpu_chain(x, tok, 91)
    g2 = run_gpu_chain(x, tok, 91)
    for k in g1:
        assert np.array_equal(g1[k], g2[k], equal_nan=True), k


def test_replay_after_rollback_is_identical():
    """Uniforms are keyed by absolute position: running the same round again from the same
    committed length reproduces it bit for bit (checkpoint/replay)."""
    x = W.chain_inputs("c2", B=16, V=3000, seed=13)
    tok = draft_tokens_oracle(x)
    g1 = run_gpu_chain(x, tok, 5)
    g2 = run_gpu_chain(x, tok, 5)
    assert np.array_equal(g1["out_tokens"], g2["out_tokens"])
    assert np.array_equal(g1["committed_len"], g2["committed_len"])


def test_tokens_per_round_closed_form_on_gpu():
    """iid acceptance (q one-hot, p = [alpha, 1-alpha]): mean tokens per round matches
    (1 - alpha^(gamma+1)) / (1 - alpha), alpha as the oracle reads it from the bf16 rows
    ("10.6 投机解码" §10.6.2)."""
    alpha, gamma, Bn = 0.8, 4, 20000
    tgt = np.full((Bn * (gamma + 1), 8), 0xFF80, np.uint16)
    tgt[:, 0] = W.bf16_bits(np.float32(0.0))
    tgt[:, 1] = W.bf16_bits(np.float32(np.log((1 - alpha) / alpha)))
    drf = np.full((Bn * gamma, 8), 0xFF80, np.uint16)
    drf[:, 0] = W.bf16_bits(np.float32(0.0))
    L = np.random.default_rng(3).integers(0, 1 << 20, size=Bn).astype(np.int32)
    x = dict(target=tgt, draft=drf, cu_gamma=np.arange(Bn + 1, dtype=np.int32) * gamma,
             temperature=np.ones(Bn, np.float32), top_p=None,
             seq_id=np.arange(Bn, dtype=np.uint32), committed_len=L, vocab=2, stride=8)
    o, g, _ = check_chain(x, seed=31, tokens=np.zeros(Bn * gamma, np.int32),
                          label="iid alpha=0.8")
    a = float(o["probe_rows"][0, 0])
    closed = (1 - a ** (gamma + 1)) / (1 - a)
    em = g["num_accepted"] + 1.0
    assert abs(em.mean() - closed) < 4 * em.std() / np.sqrt(Bn)


def test_workspace_reuse_between_shapes():
    """One workspace serves consecutive calls of different shapes (contents need not be
    initialised)."""
    x1 = W.chain_inputs("c3", B=8, V=5000, seed=14)
    x2 = W.chain_inputs("c2", B=30, V=700, gamma=(0, 5), seed=15)
    ws = torch.full((B.spec_verify_chain_workspace_size(64, 512, 8192),), 0xAB,
                    dtype=torch.uint8, device="cuda")
    for x, s in ((x1, 1), (x2, 2), (x1, 3)):
        tok = draft_tokens_oracle(x)
        o = run_oracle_chain(x, tok, s)
        g = run_gpu_chain(x, tok, s, workspace=ws)
        acc_bnd, _ = compare_chain(x, o, g)
        assert len(acc_bnd) <= 1
