"""Writes tree_rank_fp64.json: draft rows of one small tree-drafting round in which the two
candidates for the last expansion have path log-probabilities that are equal once rounded to
binary32 but differ in fp64, the node with the higher index being the more probable.

The expansion rule ("投机推理：小模型搭树，大模型一次验证", tree configuration and draft
steps: the next nodes are chosen by path probability) then picks the higher index, while a
ranking of binary32-rounded values (a tie, broken to the lower index) would pick the other.
Only inputs are stored; the test derives the expected choice itself. The search uses numpy and
scipy alone (seeded): root row R, rows A and B of the root's two most probable children, V=8.
Run from the repository root: python tests/golden/make_tree_rank_fp64.py
"""
import json
import os

import numpy as np
from scipy.special import log_softmax

V = 8
SEED = 12345


def bf16_grid(rng, shape):
    x = rng.uniform(-4, 4, size=shape).astype(np.float32)
    bits = x.view(np.uint32) & np.uint32(0xFFFF0000)  # a bf16 value (truncated float)
    return (bits >> 16).astype(np.uint16), bits.view(np.float32).astype(np.float64)


def search():
    rng = np.random.default_rng(SEED)
    n = 1_000_000
    for _ in range(200):
        (rb, R), (ab, A), (bb, Bm) = (bf16_grid(rng, (n, V)) for _ in range(3))
        idx = np.arange(n)
        oR = np.argsort(-R, axis=1, kind="stable")
        la = log_softmax(R, axis=1)[idx, oR[:, 0]] + \
            log_softmax(A, axis=1)[idx, np.argsort(-A, axis=1, kind="stable")[:, 0]]
        lb = log_softmax(R, axis=1)[idx, oR[:, 1]] + \
            log_softmax(Bm, axis=1)[idx, np.argsort(-Bm, axis=1, kind="stable")[:, 0]]
        hit = (la.astype(np.float32) == lb.astype(np.float32)) & (lb > la)
        if hit.any():
            i = int(np.flatnonzero(hit)[0])
            return rb[i], ab[i], bb[i]
    raise RuntimeError("no case found")


if __name__ == "__main__":
    r, a, b = search()
    out = {
        "source": "投机推理：小模型搭树，大模型一次验证 -- tree configuration and draft steps "
                  "(expansion of the most probable nodes by path probability)",
        "generator": "tests/golden/make_tree_rank_fp64.py (numpy/scipy search, seed %d)" % SEED,
        "vocab": V,
        "top_head": [1, 2, 1],
        "top_k_spec": [[2], [1, 1], [1]],
        "root_row_bf16": [int(v) for v in r],
        "child_rows_bf16": [[int(v) for v in a], [int(v) for v in b]],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tree_rank_fp64.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, ensure_ascii=False)
        f.write("\n")
    print(path)
