"""GPU parity of spec_verify_tree (bit-exact against the oracle) and kv_commit_path
(bit-exact against the oracle on small caches; at full size against the definition on
hash-filled caches), through the C ABI."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from draft_verification_03_amd import binding as B
from draft_verification_03_amd import workloads as W

from harness import dev, record, say

pytestmark = pytest.mark.gpu

TREE = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "tree_worked_example.json")))


def run_gpu_tree(logits, parent, node_row, node_token, R, max_depth, tree_stride, V):
    Bn, N = node_token.shape
    t = dict(l=dev(logits.reshape(-1, logits.shape[-1])), par=dev(parent), row=dev(node_row),
             tok=dev(node_token),
             pn=torch.full((Bn, max_depth), -9, dtype=torch.int32, device="cuda"),
             pl=torch.full((Bn,), -9, dtype=torch.int32, device="cuda"),
             out=torch.full((Bn, max_depth + 1), -1, dtype=torch.int32, device="cuda"),
             ne=torch.full((Bn,), -9, dtype=torch.int32, device="cuda"),
             fl=torch.full((Bn,), -9, dtype=torch.int32, device="cuda"))
    a = B.tree_args(target_logits=t["l"], parent=t["par"], node_row=t["row"],
                    node_token=t["tok"], path_nodes=t["pn"], path_len=t["pl"],
                    out_tokens=t["out"], num_emitted=t["ne"], seq_flags=t["fl"], vocab=V,
                    rows_per_seq=R, max_depth=max_depth, tree_stride=tree_stride,
                    row_stride=logits.shape[-1])
    B.spec_verify_tree(a)
    torch.cuda.synchronize()
    return {k: t[k2].cpu().numpy() for k, k2 in (("path_nodes", "pn"), ("path_len", "pl"),
                                                 ("out_tokens", "out"), ("num_emitted", "ne"),
                                                 ("seq_flags", "fl"))}


def compare_tree(o, g):
    assert np.array_equal(g["path_len"], o["path_len"])
    assert np.array_equal(g["num_emitted"], o["num_emitted"])
    assert np.array_equal(g["seq_flags"], o["seq_flags"])
    assert np.array_equal(g["path_nodes"], o["path_nodes"])
    for b in range(len(o["num_emitted"])):
        n = o["num_emitted"][b]
        assert np.array_equal(g["out_tokens"][b, :n], o["out_tokens"][b, :n]), b


def test_tree_c4_full():
    x = W.tree_inputs()
    say(f"[tree] c4 B=128 V=151936 rows=5 nodes=13")
    o = oracle.verify_tree(x["logits"], x["parent"], x["node_row"], x["node_token"],
                           x["rows_per_seq"], x["max_depth"], x["num_nodes"], vocab=x["vocab"])
    g = run_gpu_tree(x["logits"], x["parent"], x["node_row"], x["node_token"],
                     x["rows_per_seq"], x["max_depth"], x["num_nodes"], x["vocab"])
    compare_tree(o, g)
    say(f"[tree] c4: path length histogram {np.bincount(g['path_len'], minlength=4)}")
    record("c4 tree greedy verify B=128 V=151936, 13 nodes, 5 rows", 128, "tree bit-exact", {},
           path_len_hist=np.bincount(g["path_len"], minlength=4).tolist())
    assert len(set(g["path_len"].tolist())) > 1


def test_tree_worked_example_on_gpu():
    V = TREE["vocab"]
    names = [n["name"] for n in TREE["nodes"]]
    parent = np.array([[n["parent"] for n in TREE["nodes"]]], np.int32)
    tok = np.array([[n["token"] for n in TREE["nodes"]]], np.int32)
    rng = np.random.default_rng(9)
    logits = np.zeros((1, len(TREE["rows"]), V), np.uint16)
    node_row = np.full((1, len(names)), -1, np.int32)
    for i, r in enumerate(TREE["rows"]):
        xr = rng.standard_normal(V).astype(np.float32)
        xr[r["target_top1"]] = 10.0
        logits[0, i] = W.bf16_bits(xr)
        node_row[0, names.index(r["node"])] = i
    say("[tree] worked example")
    g = run_gpu_tree(logits, parent, node_row, tok, len(TREE["rows"]), 3, 0, V)
    assert [names[i] for i in g["path_nodes"][0]] == TREE["expected"]["path_names"]
    assert list(g["out_tokens"][0, :3]) == TREE["expected"]["path_tokens"]
    assert g["num_emitted"][0] == 3 and g["seq_flags"][0] == B.FLAG_NO_ROW


@pytest.mark.parametrize("Bn,V", [(64, 13), (160, 13), (64, 2309), (160, 2309)])
@pytest.mark.parametrize("shared", [False, True])
def test_tree_random_small(shared, Bn, V):
    """Random topologies (duplicate sibling tokens, rows missing on some nodes), ragged V
    (13: matches are frequent; 2309: nine trips of a row, the last partial), per-sequence or
    shared topology; rounded normal logits, so ties (and -0 beside +0) are frequent; 64 and
    160 sequences (1920 and 4800 row workgroups, more than the CUs hold at once)."""
    rng = np.random.default_rng(17 + shared)
    N, R, depth = 40, 30, 6
    stride = (V + 7) // 8 * 8 + 8 * (V > 100)
    par = np.zeros((1 if shared else Bn, N), np.int32)
    row = np.full((1 if shared else Bn, N), -1, np.int32)
    for s in range(par.shape[0]):
        par[s] = [-1] + [int(rng.integers(max(0, i - 6), i)) for i in range(1, N)]
        has = rng.random(N) < 0.7
        has[0] = True
        idx = np.flatnonzero(has)[:R]
        row[s, idx] = np.arange(len(idx))
    tok = rng.integers(0, V, size=(Bn, N)).astype(np.int32)
    logits = np.full((Bn, R, stride), 0xFF80, np.uint16)
    logits[..., :V] = W.bf16_bits(np.round(rng.standard_normal((Bn, R, V)) * 2).astype(np.float32))
    # make half of the children carry their parent's target argmax, so that long paths and
    # duplicate matching siblings occur
    am = W.bf16_to_f32(logits[..., :V]).argmax(-1)
    for b in range(Bn):
        s_ = 0 if shared else b
        for i in range(1, N):
            r = row[s_, par[s_, i]]
            if r >= 0 and rng.random() < 0.5:
                tok[b, i] = am[b, r]
    ts = 0 if shared else N
    say(f"[tree] random small shared={shared} B={Bn} V={V}")
    o = oracle.verify_tree(logits, np.broadcast_to(par, (Bn, N)).copy(),
                           np.broadcast_to(row, (Bn, N)).copy(), tok, R, depth, N, vocab=V)
    g = run_gpu_tree(logits, par, row, tok, R, depth, ts, V)
    compare_tree(o, g)
    assert (g["path_len"] >= 2).any()


@pytest.mark.parametrize("max_depth", [1, 64])
def test_tree_largest_shape(max_depth):
    """The largest tree the call takes: 256 nodes, each with its own row (256 rows per
    sequence), and an 80-node spine whose tokens are the target argmax of their parent, so
    the walk runs into the path capacity. Sequence 0 keeps the whole spine (a full path,
    then the extra token at the last node), sequence 1 breaks it at depth 30, sequence 2
    loses node 50's row (the walk stops there without an extra token), sequence 3 has
    random tokens only."""
    rng = np.random.default_rng(256)
    Bn, N, R, V, spine = 4, 256, 256, 61, 80
    stride = 64
    par = np.zeros((Bn, N), np.int32)
    par[:, 0] = -1
    par[:, 1:spine + 1] = np.arange(spine)
    for b in range(Bn):
        par[b, spine + 1:] = [int(rng.integers(0, i)) for i in range(spine + 1, N)]
    row = np.tile(np.arange(N, dtype=np.int32), (Bn, 1))
    row[2, 50] = -1
    logits = np.full((Bn, R, stride), 0xFF80, np.uint16)
    logits[..., :V] = W.bf16_bits(np.round(rng.standard_normal((Bn, R, V)) * 2).astype(np.float32))
    am = W.bf16_to_f32(logits[..., :V]).argmax(-1)
    tok = rng.integers(0, V, size=(Bn, N)).astype(np.int32)
    for b in range(3):
        tok[b, 1:spine + 1] = am[b, np.arange(spine)]
    tok[1, 30] = (am[1, 29] + 1) % V
    say(f"[tree] largest shape N={N} R={R} max_depth={max_depth}")
    o = oracle.verify_tree(logits, par, row, tok, R, max_depth, N, vocab=V)
    g = run_gpu_tree(logits, par, row, tok, R, max_depth, N, V)
    compare_tree(o, g)
    assert g["path_len"][0] == max_depth and g["num_emitted"][0] == max_depth + 1
    assert np.array_equal(g["path_nodes"][0], np.arange(1, max_depth + 1))
    if max_depth == 64:
        assert g["path_len"][1] >= 29
        assert g["path_len"][2] == 50 and g["num_emitted"][2] == 50
        assert g["seq_flags"][2] == B.FLAG_NO_ROW


@pytest.mark.parametrize("Bn", [2, 130])
def test_tree_bad_topology_flagged(Bn):
    par = np.tile(np.array([[-1, 0, 0, 1]], np.int32), (Bn, 1))
    par[0] = [-1, 0, 2, 1]  # seq 0: parent 2 of node 2
    row = np.tile(np.array([[0, 1, -1, -1]], np.int32), (Bn, 1))
    row[0] = [0, -1, -1, -1]
    if Bn > 2:
        row[2, 3] = 2  # a row index past rows_per_seq
    tok = np.zeros((Bn, 4), np.int32)
    logits = np.zeros((Bn, 2, 8), np.uint16)
    say(f"[tree] bad topology B={Bn}")
    g = run_gpu_tree(logits, par, row, tok, 2, 3, 4, 8)
    assert g["seq_flags"][0] == B.FLAG_BAD_TREE and g["num_emitted"][0] == 0
    assert g["seq_flags"][1] != B.FLAG_BAD_TREE and g["num_emitted"][1] >= 1
    if Bn > 2:
        assert g["seq_flags"][2] == B.FLAG_BAD_TREE and g["num_emitted"][2] == 0
        o = oracle.verify_tree(logits, par, row, tok, 2, 3, 4, vocab=8)
        compare_tree(o, g)


# ---- KV commit ---------------------------------------------------------------------------

def _run_gpu_kv(k_layers, v_layers, paths, plen, L, lead, max_depth, cap=None):
    Bn, S, H, Dh = k_layers[0].shape
    kt = [dev(a) for a in k_layers]
    vt = [dev(a) for a in v_layers]
    Lt = dev(L)
    fl = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    a = B.kv_args(k_cache=kt, v_cache=vt, path_nodes=dev(paths), path_len=dev(plen),
                  committed_len=Lt, seq_flags=fl, num_kv_heads=H, head_dim=Dh,
                  seq_stride=S * H * Dh, slot_stride=H * Dh, head_stride=Dh,
                  slot_capacity=S if cap is None else cap, lead_slots=lead,
                  max_depth=max_depth)
    B.kv_commit_path(a)
    torch.cuda.synchronize()
    return ([t.cpu().numpy().view(np.uint16) for t in kt],
            [t.cpu().numpy().view(np.uint16) for t in vt], Lt.cpu().numpy(), fl.cpu().numpy())


@pytest.mark.parametrize("lead", [1, 0])
def test_kv_commit_small_vs_oracle(lead):
    rng = np.random.default_rng(40 + lead)
    Bn, S, H, Dh, nl, depth = 9, 48, 3, 16, 4, 5
    k = [rng.integers(0, 65536, size=(Bn, S, H, Dh)).astype(np.uint16) for _ in range(nl)]
    v = [rng.integers(0, 65536, size=(Bn, S, H, Dh)).astype(np.uint16) for _ in range(nl)]
    paths = np.full((Bn, depth), -1, np.int32)
    plen = np.zeros(Bn, np.int32)
    cases = [[1, 7, 11], [1, 2, 3, 4, 5], [2, 9], [], [3, 4, 12, 20, 31], [6], [2, 3, 40],
             [1, 5, 9, 13], [50]]  # last two: out of range for some L
    for b, c in enumerate(cases):
        paths[b, :len(c)] = c
        plen[b] = len(c)
    L = np.array([0, 5, 10, 3, 1, 40, 2, 30, 0], np.int32)
    say(f"[kv] small lead={lead}")
    ko, vo = [a.copy() for a in k], [a.copy() for a in v]
    cl_o, fl_o = oracle.kv_commit(ko, vo, paths, plen, L, lead, depth)
    kg, vg, cl_g, fl_g = _run_gpu_kv(k, v, paths, plen, L, lead, depth)
    assert np.array_equal(cl_g, cl_o) and np.array_equal(fl_g, fl_o)
    assert (fl_o & B.FLAG_SLOT_OOB).any()
    for l in range(nl):
        assert np.array_equal(kg[l], ko[l]) and np.array_equal(vg[l], vo[l])


def test_kv_commit_ragged_workgroup_split():
    """3 layers x K,V x 11 heads x 128: 1056 chunks per slot, so a sequence's copy spans two
    workgroups, the second holding 32 chunks; tree paths and a chain rollback."""
    rng = np.random.default_rng(48)
    Bn, S, H, Dh, nl, depth = 5, 24, 11, 128, 3, 3
    k = [rng.integers(0, 65536, size=(Bn, S, H, Dh)).astype(np.uint16) for _ in range(nl)]
    v = [rng.integers(0, 65536, size=(Bn, S, H, Dh)).astype(np.uint16) for _ in range(nl)]
    paths = np.array([[2, 5, 9], [1, 2, 3], [3, 4, -1], [6, -1, -1], [-1, -1, -1]], np.int32)
    plen = np.array([3, 3, 2, 1, 0], np.int32)
    L = np.array([4, 10, 0, 7, 3], np.int32)
    say("[kv] ragged workgroup split")
    ko, vo = [a.copy() for a in k], [a.copy() for a in v]
    cl_o, fl_o = oracle.kv_commit(ko, vo, paths, plen, L, 1, depth)
    kg, vg, cl_g, fl_g = _run_gpu_kv(k, v, paths, plen, L, 1, depth)
    assert np.array_equal(cl_g, cl_o) and np.array_equal(fl_g, fl_o) and not fl_o.any()
    for l in range(nl):
        assert np.array_equal(kg[l], ko[l]) and np.array_equal(vg[l], vo[l])


def test_kv_commit_overlapping_paths_vs_oracle():
    """Paths that are not tree paths: a step's source can be an earlier step's destination
    ([2, 1], [3, 1, 2], ...), inside one group of in-flight steps and across groups (depth 9).
    The commit must equal in-order copying, byte for byte."""
    rng = np.random.default_rng(47)
    Bn, S, H, Dh, nl, depth = 24, 40, 2, 16, 2, 9
    k = [rng.integers(0, 65536, size=(Bn, S, H, Dh)).astype(np.uint16) for _ in range(nl)]
    v = [rng.integers(0, 65536, size=(Bn, S, H, Dh)).astype(np.uint16) for _ in range(nl)]
    paths = np.full((Bn, depth), -1, np.int32)
    plen = np.zeros(Bn, np.int32)
    fixed = [[2, 1], [3, 1, 2], [2, 1, 4, 3, 6, 5, 8, 7, 9], [1, 1, 1, 1, 1, 1],
             [5, 4, 3, 2, 1], [1, 2, 3, 4, 5, 6, 7, 8, 9], [9, 8, 7, 6, 5, 4, 3, 2, 1],
             [2, 3, 4, 5, 6, 7, 8, 9, 1]]
    for b in range(Bn):
        c = fixed[b] if b < len(fixed) else \
            list(rng.integers(1, depth + 3, size=int(rng.integers(1, depth + 1))))
        paths[b, :len(c)] = c
        plen[b] = len(c)
    L = rng.integers(0, S - depth - 4, size=Bn).astype(np.int32)
    say("[kv] overlapping paths")
    ko, vo = [a.copy() for a in k], [a.copy() for a in v]
    cl_o, fl_o = oracle.kv_commit(ko, vo, paths, plen, L, 1, depth)
    kg, vg, cl_g, fl_g = _run_gpu_kv(k, v, paths, plen, L, 1, depth)
    assert np.array_equal(cl_g, cl_o) and np.array_equal(fl_g, fl_o)
    assert not fl_o.any()
    for l in range(nl):
        assert np.array_equal(kg[l], ko[l]) and np.array_equal(vg[l], vo[l])


def test_kv_commit_c4_full_size():
    """32 layers x K,V x [128 seq][1024 slots][8 heads][128] bf16 (17.2 GB), every element a
    hash of its coordinates. After committing the oracle's tree paths, every element of every
    cache equals the hash of its source coordinates (the path's source slot for committed
    slots, its own slot elsewhere), bit for bit; the pointer moved by lead + D."""
    x = W.tree_inputs()
    o = oracle.verify_tree(x["logits"], x["parent"], x["node_row"], x["node_token"],
                           x["rows_per_seq"], x["max_depth"], x["num_nodes"], vocab=x["vocab"])
    NL, H, Dh, S = (W.KV_SHAPE[k] for k in ("num_layers", "num_kv_heads", "head_dim", "slots"))
    Bn = 128
    say(f"[kv] c4 full size: allocating {2 * NL * Bn * S * H * Dh * 2 / 1e9:.1f} GB")
    sl = torch.arange(S, device="cuda", dtype=torch.int64).view(1, S, 1, 1)
    sq = torch.arange(Bn, device="cuda", dtype=torch.int64).view(Bn, 1, 1, 1)
    hh = torch.arange(H, device="cuda", dtype=torch.int64).view(1, 1, H, 1)
    dd = torch.arange(Dh, device="cuda", dtype=torch.int64).view(1, 1, 1, Dh)
    caches = [[None, None] for _ in range(NL)]
    for l in range(NL):
        for kv in range(2):
            h = W.kv_hash(l, kv, sq, sl, hh, dd)
            caches[l][kv] = h.to(torch.int32).to(torch.int16)
            del h
    L = x["committed_len"]
    paths = o["path_nodes"]
    plen = o["path_len"]
    Lt = dev(L)
    fl = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    a = B.kv_args(k_cache=[c[0] for c in caches], v_cache=[c[1] for c in caches],
                  path_nodes=dev(paths), path_len=dev(plen), committed_len=Lt, seq_flags=fl,
                  num_kv_heads=H, head_dim=Dh, seq_stride=S * H * Dh, slot_stride=H * Dh,
                  head_stride=Dh, slot_capacity=S, lead_slots=1, max_depth=x["max_depth"])
    say("[kv] c4 full size: commit")
    B.kv_commit_path(a)
    torch.cuda.synchronize()
    assert np.array_equal(Lt.cpu().numpy(), L + 1 + plen) and int(fl.abs().sum()) == 0
    # expected source slot of every (seq, slot)
    src = np.tile(np.arange(S), (Bn, 1))
    for b in range(Bn):
        for j in range(1, plen[b] + 1):
            src[b, L[b] + j] = L[b] + paths[b, j - 1]
    moved = int((src != np.arange(S)[None]).sum())
    srt = torch.from_numpy(src).cuda().view(Bn, S, 1, 1)
    say(f"[kv] c4 full size: checking all {Bn * S} (seq, slot) rows of the {2 * NL} caches, "
        f"{moved} moved")
    for l in range(NL):
        for kv in range(2):
            got = caches[l][kv].to(torch.int64) & 0xFFFF
            want = W.kv_hash(l, kv, sq, srt, hh, dd)
            assert torch.equal(got, want), (l, kv)
            del got, want
    record("c4 KV commit, 32 layers x K,V x [128][1024][8][128] bf16", Bn, "kv bit-exact",
           {}, rows_checked=Bn * S * 2 * NL, rows_moved=moved * 2 * NL)
    del caches
    torch.cuda.empty_cache()
