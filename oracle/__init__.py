"""fp64 CPU oracle of the speculative-sampling verification step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The product library never imports, links or calls it, and the two
share no code: this package wraps ``spec_oracle.c`` (plain C, fp64), written from the pages,
plus ``exact.py``, an exact-rational version of the one-position rule.

Every function here is argument marshalling around the C oracle; the arithmetic lives in
``spec_oracle.c`` with its citations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB = os.path.join(_HERE, "libspec_oracle.so")

PURPOSE_ACCEPT, PURPOSE_RESIDUAL, PURPOSE_BONUS = 0, 1, 2
F_BAD_TOKEN, F_Q_ZERO, F_RESID_FALLBACK, F_NO_ROW = 1, 2, 4, 8
F_SLOT_OOB, F_BAD_TREE, F_BAD_PARAM, F_EOS, F_LEN_CAP = 16, 32, 128, 256, 512
F_FREE_FULL = 1024


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, IEEE semantics: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int


def _declare(L):
    L.oracle_philox4x32_10.argtypes = [_P, _P, _P]
    L.oracle_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
    L.oracle_uniform.restype = ctypes.c_double
    L.oracle_dist.argtypes = [_P, _I, ctypes.c_double, ctypes.c_double, _I, _P, _P, _P]
    L.oracle_dist.restype = _I
    L.oracle_sample.argtypes = [_P, _I, ctypes.c_double, _P]
    L.oracle_sample.restype = _I
    L.oracle_position_step.argtypes = [_P, _P, _I, _I, ctypes.c_double, ctypes.c_double,
                                       _P, _P, _P, _P]
    L.oracle_position_step.restype = _I
    L.oracle_verify_chain.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _I, ctypes.c_uint64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, _I]
    L.oracle_verify_chain.restype = _I
    L.oracle_verify_tree.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, _I]
    L.oracle_verify_tree.restype = _I
    L.oracle_kv_commit.argtypes = [_I, _I, _I, _I, _P, _P, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, _I, _I, _I, _P, _P, _P, _P]
    L.oracle_kv_commit.restype = _I
    L.oracle_tree_draft.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P,
                                    _P, _P, _P, _I, _P, _I]
    L.oracle_tree_draft.restype = _I
    L.oracle_kv_commit_paged.argtypes = [_I, _I, _I, _I, _P, _P, _I, _I, _I, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int64, _I, _I, _P, _P, _P,
                                         _P, _P, _I, _P, _P]
    L.oracle_kv_commit_paged.restype = _I
    L.oracle_ngram_draft.argtypes = [_I, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P]
    L.oracle_ngram_draft.restype = _I


class _RowInfo(ctypes.Structure):
    _fields_ = [("argmax", ctypes.c_int), ("nucleus", ctypes.c_int), ("m", ctypes.c_double),
                ("tk", ctypes.c_double), ("tstar", ctypes.c_double), ("z", ctypes.c_double),
                ("zs", ctypes.c_double), ("topp_margin", ctypes.c_double)]


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def philox(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed, id_, pos, purpose):
    return lib().oracle_uniform(int(seed), int(id_), int(pos), int(purpose))


def dist(row_bits, T, P=1.0, K=0):
    """Filtered (top-k K, then top-p P), normalised law of one bf16 row. Returns (pi, info
    dict)."""
    row = _c(row_bits, np.uint16)
    V = row.shape[0]
    pi = np.zeros(V, dtype=np.float64)
    scratch = np.zeros(V, dtype=np.float64)
    info = _RowInfo()
    rc = lib().oracle_dist(_ptr(row), V, float(T), float(P), int(K), _ptr(pi), _ptr(scratch),
                           ctypes.addressof(info))
    d = {f: getattr(info, f) for f, _ in _RowInfo._fields_}
    d["rc"] = rc
    return pi, d


def sample(w, u):
    w = _c(w, np.float64)
    m = ctypes.c_double(0.0)
    tok = lib().oracle_sample(_ptr(w), w.shape[0], float(u), ctypes.addressof(m))
    return tok, m.value


def position_step(p, q, d, u_acc, u_res):
    """One verified position on probability vectors: (accepted, token, flags, info[4])."""
    p = _c(p, np.float64)
    q = _c(q, np.float64)
    V = p.shape[0]
    tok = ctypes.c_int(-1)
    flags = ctypes.c_int(0)
    scratch = np.zeros(V, dtype=np.float64)
    info = np.zeros(4, dtype=np.float64)
    acc = lib().oracle_position_step(_ptr(p), _ptr(q), V, int(d), float(u_acc), float(u_res),
                                     ctypes.addressof(tok), ctypes.addressof(flags),
                                     _ptr(scratch), _ptr(info))
    return bool(acc), (None if acc else tok.value), flags.value, info


def verify_chain(target, draft, cu_gamma, draft_tokens, temperature, top_p=None, seq_id=None,
                 committed_len=None, lead_slots=1, seed=0, uniform_override=None, nthreads=0,
                 top_k=None, eos_token=None, max_emit=None):
    """Chain verification of a ragged batch on host arrays.

    target: uint16 [sum(gamma_b+1), row_stride]; draft: uint16 [sum(gamma_b), row_stride] or
    None; vocab is taken as ``target.shape[1]`` unless the arrays carry a ``vocab`` attribute,
    so pass ``vocab=`` through :func:`verify_chain_v` for padded strides.
    """
    return verify_chain_v(target, draft, cu_gamma, draft_tokens, temperature, top_p, seq_id,
                          committed_len, lead_slots, seed, uniform_override, nthreads,
                          vocab=None, top_k=top_k, eos_token=eos_token, max_emit=max_emit)


def verify_chain_v(target, draft, cu_gamma, draft_tokens, temperature, top_p=None,
                   seq_id=None, committed_len=None, lead_slots=1, seed=0,
                   uniform_override=None, nthreads=0, vocab=None, top_k=None, eos_token=None,
                   max_emit=None):
    target = _c(target, np.uint16)
    draft = _c(draft, np.uint16)
    cu = _c(cu_gamma, np.int32)
    B = cu.shape[0] - 1
    n_draft = int(cu[-1])
    n_target = n_draft + B
    stride = target.shape[1]
    V = stride if vocab is None else int(vocab)
    assert target.shape[0] >= n_target
    toks = _c(draft_tokens if draft_tokens is not None else np.zeros(0), np.int32)
    if toks.size == 0:
        toks = np.zeros(max(n_draft, 1), dtype=np.int32)
    temp = _c(temperature, np.float32)
    tp = _c(top_p, np.float32)
    tk = _c(top_k, np.int32)
    eos = _c(eos_token, np.int32)
    cap = _c(max_emit, np.int32)
    sid = _c(seq_id, np.uint32)
    L = _c(committed_len if committed_len is not None else np.zeros(B), np.int32)
    ovr = _c(uniform_override, np.float32)
    out = {
        "out_tokens": np.full(max(n_target, 1), -1, dtype=np.int32),
        "num_accepted": np.zeros(B, dtype=np.int32),
        "num_emitted": np.zeros(B, dtype=np.int32),
        "committed_len": np.zeros(B, dtype=np.int32),
        "seq_flags": np.zeros(B, dtype=np.int32),
        "probe_rows": np.full((max(n_draft, 1), 3), np.nan, dtype=np.float64),
        "probe_seq": np.full((B, 2), np.nan, dtype=np.float64),
        # [B][2]: distance to the nearest decision boundary among (0) the acceptance tests
        # and the top-p cuts of their rows, (1) those and the final draw (and its row's cut)
        "margin": np.full((B, 2), np.inf, dtype=np.float64),
        # [n_draft][2] per tested draft position: |u_acc - a_k|, and the nearer of the top-p
        # cut margins of p_k and q_k (inf where the position was not tested)
        "row_margin": np.full((max(n_draft, 1), 2), np.inf, dtype=np.float64),
        # [B][2] the final draw: the top-p cut margin of the bonus row (inf for a residual
        # draw or none), and the draw's own margin (0 when R < 1e-5; inf without a draw)
        "draw_margin": np.full((B, 2), np.inf, dtype=np.float64),
    }
    rc = lib().oracle_verify_chain(
        B, V, stride, _ptr(target), _ptr(draft), _ptr(cu), _ptr(toks), _ptr(temp), _ptr(tp),
        _ptr(tk), _ptr(eos), _ptr(cap), _ptr(sid), _ptr(L), int(lead_slots), int(seed),
        _ptr(ovr), _ptr(out["out_tokens"]), _ptr(out["num_accepted"]), _ptr(out["num_emitted"]),
        _ptr(out["committed_len"]), _ptr(out["seq_flags"]),
        _ptr(out["probe_rows"]), _ptr(out["probe_seq"]), _ptr(out["margin"]),
        _ptr(out["row_margin"]), _ptr(out["draw_margin"]), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_verify_chain failed")
    out["out_tokens"] = out["out_tokens"][:n_target]
    out["probe_rows"] = out["probe_rows"][:n_draft]
    out["row_margin"] = out["row_margin"][:n_draft]
    return out


def draw_tokens(rows, temperature, top_p, seed, ids, start_pos, vocab=None, nthreads=0,
                top_k=None):
    """One token per row from the row's filtered law: a round with gamma = 0 per row.

    Row i is a one-row sequence with id ``ids[i]`` and committed length ``start_pos[i]``, so
    its uniform is keyed (seed, ids[i], start_pos[i]+1, BONUS). A drafter that samples its
    own tokens this way matches the GPU library called with gamma = 0.
    """
    rows = _c(rows, np.uint16)
    n = rows.shape[0]
    if n == 0:
        return np.zeros(0, dtype=np.int32)
    r = verify_chain_v(rows, None, np.zeros(n + 1, dtype=np.int32), None, temperature, top_p,
                       ids, start_pos, lead_slots=1, seed=seed, nthreads=nthreads, vocab=vocab,
                       top_k=top_k)
    return r["out_tokens"].copy()


def verify_tree(logits, parent, node_row, node_token, rows_per_seq, max_depth, tree_stride,
                vocab=None, nthreads=0):
    logits = _c(logits, np.uint16)
    par = _c(parent, np.int32)
    nrow = _c(node_row, np.int32)
    tok = _c(node_token, np.int32)
    B, num_nodes = tok.shape
    stride = logits.shape[-1]
    V = stride if vocab is None else int(vocab)
    out = {
        "path_nodes": np.full((B, max_depth), -1, dtype=np.int32),
        "path_len": np.zeros(B, dtype=np.int32),
        "out_tokens": np.full((B, max_depth + 1), -1, dtype=np.int32),
        "num_emitted": np.zeros(B, dtype=np.int32),
        "seq_flags": np.zeros(B, dtype=np.int32),
    }
    lib().oracle_verify_tree(B, V, stride, int(rows_per_seq), int(num_nodes), int(max_depth),
                             int(tree_stride), _ptr(logits), _ptr(par), _ptr(nrow), _ptr(tok),
                             _ptr(out["path_nodes"]), _ptr(out["path_len"]),
                             _ptr(out["out_tokens"]), _ptr(out["num_emitted"]),
                             _ptr(out["seq_flags"]), int(nthreads))
    return out


def kv_commit(k_layers, v_layers, path_nodes, path_len, committed_len, lead_slots, max_depth,
              slot_capacity=None):
    """Commit on host caches, in place. k_layers/v_layers: lists of uint16 arrays shaped
    [B, S, H, D] (contiguous). Returns (committed_len, seq_flags)."""
    k0 = k_layers[0]
    B, S, H, D = k0.shape
    nl = len(k_layers)
    kp = (ctypes.c_void_p * nl)(*[a.ctypes.data for a in k_layers])
    vp = (ctypes.c_void_p * nl)(*[a.ctypes.data for a in v_layers])
    pn = _c(path_nodes, np.int32)
    pl = _c(path_len, np.int32)
    cl = np.array(committed_len, dtype=np.int32, copy=True)
    fl = np.zeros(B, dtype=np.int32)
    lib().oracle_kv_commit(B, nl, H, D, kp, vp, S * H * D, H * D, D,
                           int(S if slot_capacity is None else slot_capacity), int(lead_slots),
                           int(max_depth), _ptr(pn), _ptr(pl), _ptr(cl), _ptr(fl))
    return cl, fl


def tree_nodes(top_head, top_k_spec):
    """Number of nodes (root included) of a tree with this configuration."""
    return 1 + sum(sum(k) for k in top_k_spec[:len(top_head)])


def tree_draft(rows_by_step, top_head, top_k_spec, root_token, pos_base=None, tree_stride=None,
               vocab=None, nthreads=0):
    """Builds the draft trees of a batch (reading R20 of spec_oracle.c).

    rows_by_step[s]: uint16 [B * top_head[s], row_stride], row b * top_head[s] + j holding the
    draft logits after the j-th node expanded at step s. top_k_spec[s]: top_head[s] child
    counts. Returns parent, node_token, node_row, node_logp (fp64), position_ids, ancestor
    (uint8 [B, n, n]), expand ([depth, B, max head]) and select_margin ([depth, B]); raises
    ValueError for an invalid configuration.
    """
    depth = len(top_head)
    rows = np.concatenate([_c(r, np.uint16) for r in rows_by_step[:depth]], axis=0)
    rt = _c(root_token, np.int32)
    B = rt.shape[0]
    stride = rows.shape[1]
    V = stride if vocab is None else int(vocab)
    n = tree_nodes(top_head, top_k_spec)
    ts = n if tree_stride is None else int(tree_stride)
    th = np.asarray(top_head, np.int32)
    ks = np.asarray([k for s in range(depth) for k in top_k_spec[s]], np.int32)
    es = int(th.max())
    out = {
        "parent": np.zeros((B, ts), np.int32), "node_token": np.zeros((B, ts), np.int32),
        "node_row": np.zeros((B, ts), np.int32), "node_logp": np.zeros((B, ts), np.float64),
        "position_ids": np.zeros((B, ts), np.int32),
        "ancestor": np.zeros((B, ts, ts), np.uint8),
        "expand": np.full((depth, B, es), -1, np.int32),
        "select_margin": np.zeros((depth, B), np.float64),
    }
    rc = lib().oracle_tree_draft(B, V, stride, depth, _ptr(th), _ptr(ks), _ptr(rows), _ptr(rt),
                                 _ptr(_c(pos_base, np.int32)), ts, _ptr(out["parent"]),
                                 _ptr(out["node_token"]), _ptr(out["node_row"]),
                                 _ptr(out["node_logp"]), _ptr(out["position_ids"]),
                                 _ptr(out["ancestor"]), _ptr(out["expand"]), es,
                                 _ptr(out["select_margin"]), int(nthreads))
    if rc != 0:
        raise ValueError("invalid tree configuration")
    out["num_nodes"] = n
    return out


def kv_commit_paged(k_layers, v_layers, block_table, path_nodes, path_len, committed_len,
                    free_list, free_count, lead_slots, max_depth):
    """Paged commit on host caches, in place (reading R22). k_layers/v_layers: lists of
    uint16 arrays shaped [num_blocks, block_size, H, D] (contiguous). block_table
    [B, max_blocks] and free_list (its length is the free list's capacity) are updated in
    place. Returns
    (committed_len, free_count, seq_flags)."""
    nb, bs, H, D = k_layers[0].shape
    nl = len(k_layers)
    kp = (ctypes.c_void_p * nl)(*[a.ctypes.data for a in k_layers])
    vp = (ctypes.c_void_p * nl)(*[a.ctypes.data for a in v_layers])
    bt = block_table
    assert bt.dtype == np.int32 and bt.flags.c_contiguous
    assert free_list.dtype == np.int32 and free_list.flags.c_contiguous
    B, max_blocks = bt.shape
    pn = _c(path_nodes, np.int32)
    pl = _c(path_len, np.int32)
    cl = np.array(committed_len, dtype=np.int32, copy=True)
    fc = np.array([free_count], dtype=np.int32)
    fl = np.zeros(B, dtype=np.int32)
    lib().oracle_kv_commit_paged(B, nl, H, D, kp, vp, bs, max_blocks, nb, bs * H * D, H * D, D,
                                 int(lead_slots), int(max_depth), _ptr(bt), _ptr(pn), _ptr(pl),
                                 _ptr(cl), _ptr(free_list), int(free_list.size), _ptr(fc),
                                 _ptr(fl))
    return cl, int(fc[0]), fl


def ngram_draft(tokens, hist_len, nmin, nmax, gamma, draft_stride=None):
    """n-gram prompt lookup over token histories [B, stride] (reading R23). Returns drafts
    [B, draft_stride] (-1 padded), num_drafts, match_len and match_pos."""
    t = _c(tokens, np.int32)
    hl = _c(hist_len, np.int32)
    B, stride = t.shape
    ds = int(gamma if draft_stride is None else draft_stride)
    out = {"drafts": np.full((B, ds), -1, np.int32), "num_drafts": np.zeros(B, np.int32),
           "match_len": np.zeros(B, np.int32), "match_pos": np.zeros(B, np.int32),
           "seq_flags": np.zeros(B, np.int32)}
    lib().oracle_ngram_draft(B, stride, _ptr(t), _ptr(hl), int(nmin), int(nmax), int(gamma), ds,
                             _ptr(out["drafts"]), _ptr(out["num_drafts"]),
                             _ptr(out["match_len"]), _ptr(out["match_pos"]),
                             _ptr(out["seq_flags"]))
    return out
