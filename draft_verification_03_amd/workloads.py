"""Seeded synthetic inputs for the verification step.

This module only draws inputs. It holds none of the verification arithmetic (no softmax,
no top-p, no acceptance test, no sampling by a uniform): draft tokens are drawn by whichever
side consumes the inputs -- the oracle in the tests, the GPU library (a gamma = 0 call) in
the benchmark. All randomness is numpy ``default_rng(seed)`` in float32, rounded to bf16
with round-to-nearest-even.

Workloads (shapes follow the pages' verify step: target logits for gamma+1 positions and
draft logits for gamma positions per request, "10.6 投机解码" §10.6.3; the tree follows the
draft tree of "投机推理：小模型搭树，大模型一次验证"):

* ``markov``  -- B=1, gamma=4, vocab 4: first-order Markov target table with Dirichlet(2)
  rows, draft = target + U(-0.05, 0.05), clamped at 1e-6 and renormalised.
* ``c2``      -- B=64, gamma=4, V=32000: target N(0, 2^2), draft = target + N(0, 0.5^2), T=1.
* ``c3``      -- B=256, gamma=8, V=128256: target N(0, 3^2) with floor(V/100) distinct ids
  per row boosted by +8, draft = target + N(0, 1^2), T=0.7, top-p 0.9 on both laws.
* ``c5``      -- B=1024, gamma_b ~ U{1..8}, V=128256: target N(0, 2^2), T_b ~ U[0.5, 1.2],
  draft = target + N(0, sigma_b^2) with sigma_b ~ U[0.3, 1.5], no top-p.
* ``tree``    -- B=128, V=151936, 13-node tree (root + [6], [2,2], [1,1]) with random
  distinct sibling tokens, 5 target rows per sequence of N(0, 2^2) logits, each boosting one
  child's token by +14 with probability 0.7; KV cache 32 layers x 8 KV heads x head_dim 128,
  1024 slots.
* ``tree_draft`` -- the drafting side of the same tree: top_head [1, 2, 2], top_k_spec [[6],
  [2, 2], [1, 1]] ("投机推理" tree configuration section), B=128, V=151936; step s has
  B * top_head[s] draft rows of N(0, 2^2) logits; root tokens uniform, root positions
  L_b ~ U{0..1010}.
* ``ngram``   -- B=256 token histories (prompt + generated text) of U{1024..8192} tokens over
  V=128256, built from segments: with probability 1/2 a fresh span of U{4..32} uniform tokens,
  else a copy of an earlier span of the history, so that trailing n-grams recur (the pages'
  setting for model-free drafts: output that overlaps its input).

Every chain workload has committed lengths L_b ~ U{0..4095} and seq_id = b.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------
# bf16 helpers (bit patterns carried as uint16)
# --------------------------------------------------------------------------------------


def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


# --------------------------------------------------------------------------------------
# Chain workloads
# --------------------------------------------------------------------------------------

CHAIN_CONFIGS = {
    # name: (B, gamma (int, or (lo, hi) per sequence), V, target sigma, boost prob, boost,
    #        draft sigma (float or (lo, hi)), T (float or (lo, hi)), top_p or None)
    "c2": dict(B=64, gamma=4, V=32000, sigma=2.0, boost_p=0.0, boost=0.0, noise=0.5,
               T=1.0, top_p=None),
    "c3": dict(B=256, gamma=8, V=128256, sigma=3.0, boost_p=0.01, boost=8.0, noise=1.0,
               T=0.7, top_p=0.9),
    "c5": dict(B=1024, gamma=(1, 8), V=128256, sigma=2.0, boost_p=0.0, boost=0.0,
               noise=(0.3, 1.5), T=(0.5, 1.2), top_p=None),
}

SEEDS = {"markov": 101, "c2": 202, "c3": 303, "tree": 404, "c5": 505, "tree_draft": 606,
         "ngram": 707}


def _pool_map(fn, n):
    from concurrent.futures import ThreadPoolExecutor
    import os
    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fn, range(n)))


def chain_inputs(name: str, seed: int | None = None, B: int | None = None,
                 V: int | None = None, gamma=None, temperature=None, top_p="cfg",
                 stride: int | None = None, max_len: int = 4096) -> dict:
    """Seeded inputs of one chain workload, optionally resized (B, V, gamma, T, top_p) for
    small parity cases. Returns host arrays:

    target  uint16 [sum(gamma_b+1), stride]   draft uint16 [sum(gamma_b), stride]
    cu_gamma int32 [B+1], temperature float32 [B], top_p float32 [B] or None,
    seq_id uint32 [B], committed_len int32 [B], vocab, stride, gamma (max).

    Per-sequence scalars come from one generator; each sequence's rows come from its own
    child stream of ``SeedSequence(seed)``, so the result does not depend on the number of
    threads that fill it. Boosted logits (c3): floor(V/100) distinct ids per target row,
    shared by the draft row of the same position.
    """
    cfg = dict(CHAIN_CONFIGS[name])
    if B is not None:
        cfg["B"] = B
    if V is not None:
        cfg["V"] = V
    if gamma is not None:
        cfg["gamma"] = gamma
    if temperature is not None:
        cfg["T"] = temperature
    if top_p != "cfg":
        cfg["top_p"] = top_p
    sd = SEEDS[name] if seed is None else seed
    rng = np.random.default_rng(sd)
    Bn, Vn = cfg["B"], cfg["V"]
    st = round_up(Vn, 8) if stride is None else stride
    g = cfg["gamma"]
    if isinstance(g, tuple):
        gam = rng.integers(g[0], g[1] + 1, size=Bn).astype(np.int32)
    else:
        gam = np.full(Bn, g, dtype=np.int32)
    cu = np.zeros(Bn + 1, dtype=np.int32)
    cu[1:] = np.cumsum(gam)
    T = cfg["T"]
    temp = (rng.uniform(T[0], T[1], size=Bn) if isinstance(T, tuple)
            else np.full(Bn, T)).astype(np.float32)
    ns = cfg["noise"]
    noise = (rng.uniform(ns[0], ns[1], size=Bn) if isinstance(ns, tuple)
             else np.full(Bn, ns)).astype(np.float32)
    tp = None if cfg["top_p"] is None else np.full(Bn, cfg["top_p"], dtype=np.float32)
    L = rng.integers(0, max_len, size=Bn).astype(np.int32)
    n_t, n_d = int(cu[-1]) + Bn, int(cu[-1])
    target = np.zeros((n_t, st), dtype=np.uint16)
    draft = np.zeros((n_d, st), dtype=np.uint16)
    kids = np.random.SeedSequence(sd).spawn(Bn)
    n_boost = int(Vn * cfg["boost_p"])

    def fill(b):
        r = np.random.default_rng(kids[b])
        gb = int(gam[b])
        t = r.standard_normal((gb + 1, Vn), dtype=np.float32)
        t *= np.float32(cfg["sigma"])
        for i in range(gb + 1 if n_boost else 0):
            t[i, r.choice(Vn, n_boost, replace=False)] += np.float32(cfg["boost"])
        d = r.standard_normal((gb, Vn), dtype=np.float32)
        d *= noise[b]
        d += t[:gb]
        r0 = int(cu[b]) + b
        target[r0:r0 + gb + 1, :Vn] = bf16_bits(t)
        draft[int(cu[b]):int(cu[b]) + gb, :Vn] = bf16_bits(d)

    _pool_map(fill, Bn)
    return dict(target=target, draft=draft, cu_gamma=cu, temperature=temp, top_p=tp,
                seq_id=np.arange(Bn, dtype=np.uint32), committed_len=L, vocab=Vn,
                stride=st, gamma=int(gam.max()) if Bn else 0, noise=noise)


def random_tokens(n: int, V: int, seed: int) -> np.ndarray:
    """Uniformly random token ids: adversarial draft tokens for edge-case tests."""
    return np.random.default_rng(seed).integers(0, V, size=n).astype(np.int32)


# --------------------------------------------------------------------------------------
# Markov tables (vocab 4)
# --------------------------------------------------------------------------------------


def markov_tables(seed: int | None = None, V: int = 4):
    """Target rows Dirichlet(2); draft = target + U(-0.05, 0.05), clamped at 1e-6 and
    renormalised. float64 [V, V] each (row = previous token)."""
    rng = np.random.default_rng(SEEDS["markov"] if seed is None else seed)
    target = rng.dirichlet(np.full(V, 2.0), size=V)
    draft = target + rng.uniform(-0.05, 0.05, size=(V, V))
    draft = np.maximum(draft, 1e-6)
    draft /= draft.sum(axis=1, keepdims=True)
    return target, draft


def log_rows_bf16(table: np.ndarray, stride: int = 8) -> np.ndarray:
    """Logits rows for a probability table: bf16(ln p), padded to ``stride`` (padding is
    never read; it holds -inf)."""
    V = table.shape[1]
    out = np.full((table.shape[0], stride), 0xFF80, dtype=np.uint16)
    out[:, :V] = bf16_bits(np.log(table).astype(np.float32))
    return out


# --------------------------------------------------------------------------------------
# Tree workload
# --------------------------------------------------------------------------------------

TREE_SPEC = dict(top_k=[[6], [2, 2], [1, 1]], top_head=[1, 2, 2])


def tree_inputs(seed: int | None = None, B: int = 128, V: int = 151936, sigma: float = 2.0,
                hit: float = 0.7, boost: float = 14.0, max_len: int = 1010) -> dict:
    """Synthetic draft trees of the [6], [2,2], [1,1] shape and their target rows.

    Topology per sequence: root 0; nodes 1..6 are its children; nodes 7, 8 are children of
    node 1 and 9, 10 of node 2; two of nodes 7..10, drawn at random, get one child each
    (nodes 11 and 12, in index order). Sibling tokens are distinct uniform ids. Target rows
    exist for the five expanded nodes [root, 1, 2, the two expanded depth-2 nodes]: N(0,
    sigma^2) logits in which, with probability ``hit``, the token of one of the node's
    children gets +``boost`` (drawn uniformly among the children that have rows of their own,
    if any), so that the tree walk can go on through it; otherwise the row's argmax has nothing
    to do with the children. Node 0 is the root token (already emitted; never verified).
    """
    rng = np.random.default_rng(SEEDS["tree"] if seed is None else seed)
    N = 13
    R = 5
    st = round_up(V, 8)
    logits = np.zeros((B, R, st), dtype=np.uint16)
    parent = np.zeros((B, N), dtype=np.int32)
    node_row = np.full((B, N), -1, dtype=np.int32)
    node_token = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        t = rng.standard_normal((R, V), dtype=np.float32) * np.float32(sigma)
        deep = sorted(int(i) for i in rng.choice(np.arange(7, 11), size=2, replace=False))
        par = [-1, 0, 0, 0, 0, 0, 0, 1, 1, 2, 2, deep[0], deep[1]]
        tok = [0] * N
        tok[0] = int(rng.integers(0, V))
        for node in range(N):  # distinct tokens among each node's children
            kids = [c for c in range(1, N) if par[c] == node]
            for c, v in zip(kids, rng.choice(V, size=len(kids), replace=False)):
                tok[c] = int(v)
        rows = {0: 0, 1: 1, 2: 2, deep[0]: 3, deep[1]: 4}
        for node, r in rows.items():
            kids = [c for c in range(1, N) if par[c] == node]
            inner = [c for c in kids if c in rows] or kids
            if rng.random() < hit:
                t[r, tok[inner[int(rng.integers(0, len(inner)))]]] += np.float32(boost)
        logits[b, :, :V] = bf16_bits(t)
        parent[b] = par
        node_token[b] = tok
        for node, r in rows.items():
            node_row[b, node] = r
    L = rng.integers(0, max_len, size=B).astype(np.int32)
    return dict(logits=logits, parent=parent, node_row=node_row, node_token=node_token,
                rows_per_seq=R, num_nodes=N, max_depth=3, vocab=V, stride=st,
                committed_len=L)


TREE_SHAPE = dict(top_head=(1, 2, 2), top_k_spec=((6,), (2, 2), (1, 1)))


def tree_draft_inputs(seed: int | None = None, B: int = 128, V: int = 151936,
                      top_head=TREE_SHAPE["top_head"], top_k_spec=TREE_SHAPE["top_k_spec"],
                      sigma: float = 2.0, quant: float | None = None, stride: int | None = None,
                      max_len: int = 1010) -> dict:
    """Draft rows of one tree-drafting round: for step s, ``B * top_head[s]`` rows of
    N(0, sigma^2) logits (row b * top_head[s] + j follows the j-th node expanded for sequence
    b). ``quant`` rounds the logits to multiples of 1/quant first (many exact ties). Root
    tokens are uniform over the vocabulary, root positions L_b ~ U{0..max_len}."""
    rng = np.random.default_rng(SEEDS["tree_draft"] if seed is None else seed)
    st = round_up(V, 8) if stride is None else stride
    rows = []
    for h in top_head:
        x = rng.standard_normal((B * h, V), dtype=np.float32) * np.float32(sigma)
        if quant:
            x = np.round(x * quant) / np.float32(quant)
        r = np.zeros((B * h, st), dtype=np.uint16)
        r[:, :V] = bf16_bits(x)
        rows.append(r)
    return dict(rows=rows, top_head=tuple(top_head), top_k_spec=tuple(map(tuple, top_k_spec)),
                root_token=rng.integers(0, V, size=B).astype(np.int32),
                pos_base=rng.integers(0, max_len + 1, size=B).astype(np.int32), vocab=V,
                stride=st, batch=B)


def ngram_inputs(seed: int | None = None, B: int = 256, min_len: int = 1024,
                 max_len: int = 8192, V: int = 128256, copy_prob: float = 0.5,
                 span=(4, 32), stride: int | None = None) -> dict:
    """Token histories for the n-gram lookup: segments that are either fresh uniform tokens or
    copies of an earlier span of the same history."""
    rng = np.random.default_rng(SEEDS["ngram"] if seed is None else seed)
    st = round_up(max_len, 8) if stride is None else stride
    tok = np.zeros((B, st), np.int32)
    lens = rng.integers(min_len, max_len + 1, size=B).astype(np.int32)
    for b in range(B):
        h = []
        while len(h) < lens[b]:
            n = int(rng.integers(span[0], span[1] + 1))
            if len(h) > n and rng.random() < copy_prob:
                i = int(rng.integers(0, len(h) - n))
                h.extend(h[i:i + n])
            else:
                h.extend(rng.integers(0, V, size=n).tolist())
        tok[b, :lens[b]] = h[:lens[b]]
    return dict(tokens=tok, hist_len=lens, vocab=V, stride=st, batch=B)


# --------------------------------------------------------------------------------------
# KV cache contents: a fixed hash of the element's coordinates, so expected values after a
# commit are known without copying the cache on the host.
# --------------------------------------------------------------------------------------

KV_SHAPE = dict(num_layers=32, num_kv_heads=8, head_dim=128, slots=1024)


def kv_hash(layer, kv, seq, slot, head, dim):
    """uint16 pattern (as int64) of cache element (layer, K=0/V=1, seq, slot, head, dim).

    Works on Python ints, numpy int64 arrays and torch int64 tensors alike: every product
    is of a value below 2^31 and a constant below 2^32, so nothing overflows int64.
    """
    x = ((((layer * 2 + kv) * 131 + seq) * 4099 + slot) * 16 + head) * 257 + dim
    x = x & 0x7FFFFFFF
    x = (x * 0x9E3779B1 + 0x7F4A7C15) & 0x7FFFFFFF
    x = x ^ (x >> 17)
    x = (x * 0x85EBCA6B) & 0x7FFFFFFF
    x = x ^ (x >> 13)
    return x & 0xFFFF
