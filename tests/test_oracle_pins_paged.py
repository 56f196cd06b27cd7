"""Pins of the oracle's paged KV commit (reading R22 of oracle/spec_oracle.c): "10.6 投机解码"
§10.6.3 -- after a rejection the cache length is cut back and a paged cache releases the blocks
it no longer needs; "KV Cache 优化（四）" §6 -- one committed-length pointer.

Pinned against:
  * the contiguous commit (reading R12, pinned in test_oracle_pins): gathering a paged cache
    through its block table (numpy fancy indexing) gives a contiguous cache, and committing
    either way yields the same gathered bytes and committed lengths;
  * properties of the release: the released blocks are exactly the mapped blocks at or past
    ceil(L' / block_size), appended in (sequence, logical block) order; nothing else changes
    in the table; no block is lost or duplicated; untouched physical blocks keep their bytes;
  * a hand-built chain rollback and rejected inputs.
"""
import numpy as np
import pytest


def _paged_case(rng, B=6, bs=4, max_blocks=8, nb=64, H=2, D=16, nl=2, depth=3, lead=1,
                tree=True):
    """Random block tables over a shuffled pool, committed lengths, and paths."""
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((B, max_blocks), -1, np.int32)
    L = np.zeros(B, np.int32)
    used = 0
    for b in range(B):
        L[b] = rng.integers(0, (max_blocks - 2) * bs - depth - lead)
        top = L[b] + lead + depth  # slots the verify step wrote reach top - 1
        nmap = min(max_blocks, -(-top // bs) + int(rng.integers(0, 2)))  # sometimes one spare
        bt[b, :nmap] = perm[used:used + nmap]
        used += nmap
    free = np.zeros(nb, np.int32)
    free[:nb - used] = perm[used:]
    free_count = nb - used
    k = [rng.integers(0, 65536, size=(nb, bs, H, D)).astype(np.uint16) for _ in range(nl)]
    v = [rng.integers(0, 65536, size=(nb, bs, H, D)).astype(np.uint16) for _ in range(nl)]
    plen = rng.integers(0, depth + 1, size=B).astype(np.int32)
    paths = np.full((B, depth), -1, np.int32)
    for b in range(B):
        if tree:  # a tree path: node j at depth j, index >= j, increasing
            nodes = np.sort(rng.choice(np.arange(1, 3 * depth + 1), size=plen[b], replace=False))
            nodes = np.maximum(nodes, np.arange(1, plen[b] + 1))
        else:
            nodes = np.arange(1, plen[b] + 1)
        paths[b, :plen[b]] = nodes
        # the verify step wrote the tree nodes' slots: make sure those blocks are mapped
        hi = L[b] + lead - 1 + (nodes.max() if plen[b] else 0)
        need = hi // bs + 1
        for lb in range(need):
            if bt[b, lb] < 0:
                bt[b, lb] = free[free_count - 1]
                free_count -= 1
    return dict(k=k, v=v, bt=bt, L=L, paths=paths, plen=plen, free=free,
                free_count=free_count, lead=lead, depth=depth, bs=bs)


def _gather(c, bt, b, bs):
    """Sequence b's logical slots as a contiguous [slots, H, D] array (unmapped -> zeros)."""
    out = np.zeros((bt.shape[1] * bs,) + c.shape[2:], c.dtype)
    for lb, pb in enumerate(bt[b]):
        if pb >= 0:
            out[lb * bs:(lb + 1) * bs] = c[pb]
    return out


@pytest.mark.parametrize("seed,lead,tree", [(1, 1, True), (2, 0, True), (3, 1, False),
                                            (4, 1, True), (5, 0, False)])
def test_paged_equals_contiguous_commit(orc, seed, lead, tree):
    rng = np.random.default_rng(seed)
    x = _paged_case(rng, lead=lead, tree=tree)
    bs, bt0 = x["bs"], x["bt"].copy()
    B = bt0.shape[0]
    # contiguous reference: gather every sequence, commit with the contiguous oracle
    kc = [np.stack([_gather(c, bt0, b, bs) for b in range(B)]) for c in x["k"]]
    vc = [np.stack([_gather(c, bt0, b, bs) for b in range(B)]) for c in x["v"]]
    cl_c, fl_c = orc.kv_commit(kc, vc, x["paths"], x["plen"], x["L"], lead, x["depth"])
    k, v = [c.copy() for c in x["k"]], [c.copy() for c in x["v"]]
    bt = bt0.copy()
    free = x["free"].copy()
    cl, fc, fl = orc.kv_commit_paged(k, v, bt, x["paths"], x["plen"], x["L"], free,
                                     x["free_count"], lead, x["depth"])
    assert np.array_equal(cl, cl_c) and np.array_equal(fl, fl_c)
    for b in range(B):
        upto = cl[b]  # the committed prefix must read the same bytes through either layout
        for c_paged, c_cont in zip(k + v, kc + vc):
            assert np.array_equal(_gather(c_paged, bt0, b, bs)[:upto], c_cont[b][:upto]), b


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_release_set_order_and_conservation(orc, seed):
    rng = np.random.default_rng(seed)
    x = _paged_case(rng, B=8, tree=bool(seed % 2))
    bs, bt0 = x["bs"], x["bt"].copy()
    owner = {int(pb): (b, lb) for b in range(bt0.shape[0]) for lb, pb in enumerate(bt0[b])
             if pb >= 0}
    k, v = [c.copy() for c in x["k"]], [c.copy() for c in x["v"]]
    bt, free = bt0.copy(), x["free"].copy()
    cl, fc, fl = orc.kv_commit_paged(k, v, bt, x["paths"], x["plen"], x["L"], free,
                                     x["free_count"], x["lead"], x["depth"])
    released = list(free[x["free_count"]:fc])
    # exactly the mapped blocks past each sequence's new length, in (sequence, block) order
    want = [(b, lb) for b in range(bt0.shape[0]) for lb in range(bt0.shape[1])
            if bt0[b, lb] >= 0 and fl[b] == 0 and lb * bs >= cl[b] + (-cl[b]) % bs]
    assert [owner[int(p)] for p in released] == want
    # the table: released entries -1, every other entry unchanged
    for b, lb in want:
        assert bt[b, lb] == -1
        bt[b, lb] = bt0[b, lb]
    assert np.array_equal(bt, bt0)
    # no block lost or duplicated
    pool = list(free[:fc]) + [int(p) for p in bt.ravel() if p >= 0 and p not in released]
    assert sorted(pool) == list(range(len(free)))
    # blocks no copy writes keep their bytes
    written = set()
    for b in range(bt0.shape[0]):
        if fl[b]:
            continue
        base = x["L"][b] + x["lead"] - 1
        for j in range(1, x["plen"][b] + 1):
            if x["paths"][b, j - 1] != j:
                written.add(int(bt0[b, (base + j) // bs]))
    for p in range(len(free)):
        if p not in written:
            assert all(np.array_equal(c1[p], c0[p]) for c1, c0 in zip(k + v, x["k"] + x["v"]))


def test_chain_rollback_by_hand(orc):
    """block_size 4, L = 5, lead 1: x at slot 5, drafts at 6..9, so blocks 0..2 are mapped
    (table [7, 3, 9, -1]). One accepted draft: L' = 7, two blocks stay, block 9 is released
    after the two free blocks already listed; no byte moves (identity path)."""
    nb, bs, H, D = 12, 4, 1, 8
    k = [np.arange(nb * bs * H * D, dtype=np.uint16).reshape(nb, bs, H, D)]
    v = [k[0][::-1].copy()]
    bt = np.array([[7, 3, 9, -1]], np.int32)
    free = np.full(nb, -1, np.int32)
    free[:2] = [0, 1]
    k0, v0 = k[0].copy(), v[0].copy()
    cl, fc, fl = orc.kv_commit_paged(k, v, bt, np.array([[1, 2, 3, 4]], np.int32),
                                     np.array([1], np.int32), np.array([5], np.int32), free, 2,
                                     1, 4)
    assert cl[0] == 7 and fc == 3 and list(free[:3]) == [0, 1, 9] and fl[0] == 0
    assert list(bt[0]) == [7, 3, -1, -1]
    assert np.array_equal(k[0], k0) and np.array_equal(v[0], v0)


def test_rejected_inputs_leave_the_sequence_untouched(orc):
    """An unmapped destination block, a new length beyond the table, and a path node < 1 are
    flagged SLOT_OOB; the other sequences commit as usual."""
    nb, bs, H, D = 16, 4, 1, 8
    rng = np.random.default_rng(9)
    k = [rng.integers(0, 65536, size=(nb, bs, H, D)).astype(np.uint16)]
    v = [rng.integers(0, 65536, size=(nb, bs, H, D)).astype(np.uint16)]
    bt = np.array([[0, 1, -1, -1],    # path sources in block 2, unmapped: flagged
                   [2, 3, 4, 5],      # fine
                   [6, 7, 8, 9],      # L' = 14 + 1 + 3 = 18 > 16 slots: flagged
                   [10, 11, -1, -1]], np.int32)
    L = np.array([6, 3, 14, 2], np.int32)
    paths = np.array([[3, 4, 5], [2, 3, 6], [1, 2, 3], [0, 1, 2]], np.int32)
    plen = np.array([3, 3, 3, 2], np.int32)
    free = np.full(nb, -1, np.int32)
    free[:4] = [12, 13, 14, 15]
    bt0 = bt.copy()
    k0, v0 = k[0].copy(), v[0].copy()
    cl, fc, fl = orc.kv_commit_paged(k, v, bt, paths, plen, L, free, 4, 1, 3)
    # seq 0: base 6, path [3, 4, 5] -> src 9, 10, 11 (block 2, unmapped): flagged
    # seq 3: path node 0 is not a node: flagged
    assert list(fl) == [orc.F_SLOT_OOB, 0, orc.F_SLOT_OOB, orc.F_SLOT_OOB]
    assert list(cl) == [6, 3 + 1 + 3, 14, 2]
    assert np.array_equal(bt[[0, 2, 3]], bt0[[0, 2, 3]])
    # seq 1: L' = 7 needs blocks 0, 1; blocks 4 and 5 are released
    assert list(bt[1]) == [2, 3, -1, -1] and fc == 6 and list(free[4:6]) == [4, 5]
    # seq 0, 2, 3's blocks keep their bytes
    for p in [0, 1, 6, 7, 8, 9, 10, 11]:
        assert np.array_equal(k[0][p], k0[p]) and np.array_equal(v[0][p], v0[p])


def test_released_block_ids_must_be_valid(orc):
    """A table entry among the blocks the release would free that is not a valid block id
    (>= num_blocks) makes the sequence SLOT_OOB: nothing moves, its table and length stay;
    a negative entry there is an unmapped block (nothing to release)."""
    nb, bs, H, D = 8, 4, 1, 8
    rng = np.random.default_rng(11)
    k = [rng.integers(0, 65536, size=(nb, bs, H, D)).astype(np.uint16)]
    v = [rng.integers(0, 65536, size=(nb, bs, H, D)).astype(np.uint16)]
    bt = np.array([[0, 1, 99, -1],   # L' = 5: block 2 (id 99) would be released: flagged
                   [2, 3, -1, -5]],  # L' = 5: entries 2, 3 unmapped: nothing released
                  np.int32)
    L = np.array([1, 1], np.int32)
    paths = np.array([[2, 3, 4], [3, 2, 1]], np.int32)
    plen = np.array([3, 3], np.int32)
    free = np.full(nb, -1, np.int32)
    free[:4] = [4, 5, 6, 7]
    bt0, k0 = bt.copy(), k[0].copy()
    cl, fc, fl = orc.kv_commit_paged(k, v, bt, paths, plen, L, free, 4, 1, 3)
    assert list(fl) == [orc.F_SLOT_OOB, 0] and list(cl) == [1, 5] and fc == 4
    assert np.array_equal(bt, bt0)
    for p in (0, 1):  # sequence 0's blocks keep their bytes
        assert np.array_equal(k[0][p], k0[p])
    # sequence 1 (base 1): slot 4 -> slot 2, slot 3 stays, then slot 2 -> slot 4, in order;
    # block id 2 holds slots 0..3 and block id 3 slots 4..7
    assert np.array_equal(k[0][2][2], k0[3][0]) and np.array_equal(k[0][3][0], k0[3][0])


def test_full_free_list_keeps_the_block_in_the_table(orc):
    """A released block that finds the free list at its capacity stays in the table and the
    sequence is flagged FREE_FULL; the length and the copy are done, and blocks that fit are
    released as usual (sequences in order, blocks in logical order)."""
    nb, bs, H, D = 6, 2, 1, 8
    k = [np.arange(nb * bs * H * D, dtype=np.uint16).reshape(nb, bs, H, D)]
    v = [k[0].copy()]
    bt = np.array([[0, 1, 2], [3, 4, 5]], np.int32)
    L = np.array([0, 0], np.int32)
    paths = np.array([[1], [1]], np.int32)
    plen = np.array([1, 1], np.int32)
    free = np.full(3, -1, np.int32)  # capacity 3, one id already listed
    free[0] = 9
    cl, fc, fl = orc.kv_commit_paged(k, v, bt, paths, plen, L, free, 1, 1, 1)
    # L' = 2: each sequence keeps block 0 and would release blocks 1, 2
    assert list(cl) == [2, 2] and fc == 3 and list(free) == [9, 1, 2]
    assert list(fl) == [0, orc.F_FREE_FULL]
    assert list(bt[0]) == [0, -1, -1] and list(bt[1]) == [3, 4, 5]
