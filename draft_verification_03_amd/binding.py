"""Thin ctypes binding of libspecv.so (include/spec_verify.h).

Argument marshalling only: every step of the verification runs in the library's gfx950
kernels. PyTorch supplies device memory (``tensor.data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``). The library must have been built
(``draft_verification_03_amd.build``); loading fails loudly if it is missing -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

_P = ctypes.c_void_p
_I32 = ctypes.c_int32

SPEC_OK = 0
SPEC_ERR_INVALID_ARG = -1
SPEC_ERR_UNSUPPORTED = -2
SPEC_ERR_HIP = -3
SPEC_ERR_WORKSPACE = -4

FLAG_BAD_TOKEN, FLAG_Q_ZERO, FLAG_RESID_FALLBACK, FLAG_NO_ROW = 1, 2, 4, 8
FLAG_SLOT_OOB, FLAG_BAD_TREE, FLAG_TOPP_SLOW, FLAG_BAD_PARAM = 16, 32, 64, 128
FLAG_EOS, FLAG_LEN_CAP, FLAG_FREE_FULL = 256, 512, 1024


class spec_chain_args(ctypes.Structure):
    _fields_ = [
        ("batch", _I32), ("vocab", _I32), ("row_stride", _I32), ("max_gamma", _I32),
        ("total_draft_rows", _I32), ("lead_slots", _I32), ("seed", ctypes.c_uint64),
        ("target_logits", _P), ("draft_logits", _P), ("cu_gamma", _P), ("draft_tokens", _P),
        ("temperature", _P), ("top_p", _P), ("top_k", _P), ("seq_id", _P),
        ("committed_len", _P), ("out_tokens", _P), ("num_accepted", _P), ("seq_flags", _P),
        ("probe_rows", _P), ("probe_seq", _P), ("uniform_override", _P),
        ("eos_token", _P), ("max_emit", _P), ("num_emitted", _P),
    ]


class spec_tree_args(ctypes.Structure):
    _fields_ = [
        ("batch", _I32), ("vocab", _I32), ("row_stride", _I32), ("num_nodes", _I32),
        ("rows_per_seq", _I32), ("max_depth", _I32), ("tree_stride", _I32),
        ("target_logits", _P), ("parent", _P), ("node_row", _P), ("node_token", _P),
        ("path_nodes", _P), ("path_len", _P), ("out_tokens", _P), ("num_emitted", _P),
        ("seq_flags", _P),
    ]


class spec_tree_draft_args(ctypes.Structure):
    _fields_ = [
        ("batch", _I32), ("vocab", _I32), ("row_stride", _I32), ("depth", _I32),
        ("step", _I32), ("tree_stride", _I32), ("expand_stride", _I32),
        ("top_head", _P), ("top_k_spec", _P), ("draft_logits", _P), ("root_token", _P),
        ("pos_base", _P), ("parent", _P), ("node_token", _P), ("node_row", _P),
        ("node_logp", _P), ("position_ids", _P), ("ancestor_mask", _P), ("expand_nodes", _P),
        ("seq_flags", _P),
    ]


class spec_paged_kv_args(ctypes.Structure):
    _fields_ = [
        ("batch", _I32), ("num_layers", _I32), ("num_kv_heads", _I32), ("head_dim", _I32),
        ("block_size", _I32), ("max_blocks", _I32), ("num_blocks", _I32),
        ("free_capacity", _I32), ("lead_slots", _I32), ("max_depth", _I32),
        ("block_stride", ctypes.c_int64), ("slot_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64), ("k_cache", _P), ("v_cache", _P),
        ("block_table", _P), ("path_nodes", _P), ("path_len", _P), ("committed_len", _P),
        ("free_list", _P), ("free_count", _P), ("seq_flags", _P),
    ]


class spec_ngram_args(ctypes.Structure):
    _fields_ = [
        ("batch", _I32), ("hist_stride", _I32), ("ngram_min", _I32), ("ngram_max", _I32),
        ("num_draft", _I32), ("draft_stride", _I32), ("tokens", _P), ("hist_len", _P),
        ("draft_tokens", _P), ("num_drafts", _P), ("match_len", _P), ("match_pos", _P),
        ("seq_flags", _P),
    ]


class spec_kv_args(ctypes.Structure):
    _fields_ = [
        ("batch", _I32), ("num_layers", _I32), ("num_kv_heads", _I32), ("head_dim", _I32),
        ("seq_stride", ctypes.c_int64), ("slot_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64), ("slot_capacity", _I32), ("lead_slots", _I32),
        ("max_depth", _I32), ("k_cache", _P), ("v_cache", _P), ("path_nodes", _P),
        ("path_len", _P), ("committed_len", _P), ("seq_flags", _P),
    ]


class SpecError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libspecv error {code}: {msg}")
        self.code = code


_lib = None

# Layout revision of the argument structs above; must equal the library's SPEC_ABI_VERSION.
ABI_VERSION = 8


def lib_path() -> str:
    return _build.LIB


def lib():
    """The loaded library. Raises if libspecv.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(f"{_build.LIB} is missing: build it with "
                               "`python -m draft_verification_03_amd.build` (no fallback path)")
        L = ctypes.CDLL(_build.LIB)
        L.spec_abi_version.restype = ctypes.c_int
        L.spec_last_error.restype = ctypes.c_char_p
        L.spec_verify_chain_workspace_size.argtypes = [_I32, _I32, _I32]
        L.spec_verify_chain_workspace_size.restype = ctypes.c_size_t
        L.spec_verify_chain.argtypes = [ctypes.POINTER(spec_chain_args), _P, ctypes.c_size_t, _P]
        L.spec_verify_chain_noalloc.argtypes = [ctypes.POINTER(spec_chain_args), _P]
        L.spec_verify_chain_timed.argtypes = [ctypes.POINTER(spec_chain_args), _P,
                                              ctypes.c_size_t, _P, _P]
        L.spec_verify_chain_timed.restype = _I32
        L.spec_verify_chain_noalloc.restype = _I32
        L.spec_verify_chain.restype = ctypes.c_int
        L.spec_verify_tree_workspace_size.argtypes = [_I32, _I32]
        L.spec_verify_tree_workspace_size.restype = ctypes.c_size_t
        L.spec_verify_tree.argtypes = [ctypes.POINTER(spec_tree_args), _P, ctypes.c_size_t, _P]
        L.spec_verify_tree.restype = ctypes.c_int
        L.kv_commit_path.argtypes = [ctypes.POINTER(spec_kv_args), _P]
        L.kv_commit_path.restype = ctypes.c_int
        L.spec_tree_draft_workspace_size.argtypes = [_I32, _I32, _I32, _P, _P]
        L.spec_tree_draft_workspace_size.restype = ctypes.c_size_t
        L.spec_tree_draft_step.argtypes = [ctypes.POINTER(spec_tree_draft_args), _P,
                                           ctypes.c_size_t, _P]
        L.spec_tree_draft_step.restype = ctypes.c_int
        L.kv_commit_paged.argtypes = [ctypes.POINTER(spec_paged_kv_args), _P]
        L.kv_commit_paged.restype = ctypes.c_int
        L.spec_ngram_draft.argtypes = [ctypes.POINTER(spec_ngram_args), _P]
        L.spec_ngram_draft.restype = ctypes.c_int
        if L.spec_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{_build.LIB} has ABI version {L.spec_abi_version()}, the "
                               f"binding expects {ABI_VERSION}: rebuild the library")
        _lib = L
    return _lib


def spec_abi_version() -> int:
    return lib().spec_abi_version()


def spec_last_error() -> str:
    return lib().spec_last_error().decode()


def spec_verify_chain_workspace_size(batch, total_draft_rows, vocab) -> int:
    return lib().spec_verify_chain_workspace_size(batch, total_draft_rows, vocab)


def spec_verify_tree_workspace_size(batch, rows_per_seq) -> int:
    return lib().spec_verify_tree_workspace_size(batch, rows_per_seq)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _keep(args, *objs):
    """The structs carry raw device addresses: hold the tensors they came from for as long
    as the struct lives, so that a tensor passed inline is not freed (and its memory reused,
    e.g. by the workspace) before the kernels run."""
    held = getattr(args, "_held", [])
    held.extend(o for o in objs if o is not None and not isinstance(o, int))
    args._held = held


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(rc):
    if rc != SPEC_OK:
        raise SpecError(rc, spec_last_error())


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def chain_args(*, target_logits, cu_gamma, temperature, committed_len, out_tokens,
               num_accepted, vocab, max_gamma, total_draft_rows, draft_logits=None,
               draft_tokens=None, top_p=None, seq_id=None, seq_flags=None, probe_rows=None,
               probe_seq=None, uniform_override=None, seed=0, lead_slots=1, row_stride=None,
               top_k=None, eos_token=None, max_emit=None,
               num_emitted=None):
    """Fills a spec_chain_args from tensors (device) or raw pointers."""
    B = int(cu_gamma.shape[0]) - 1 if hasattr(cu_gamma, "shape") else None
    a = spec_chain_args()
    a.batch = B
    a.vocab = int(vocab)
    a.row_stride = int(row_stride if row_stride is not None else target_logits.shape[-1])
    a.max_gamma = int(max_gamma)
    a.total_draft_rows = int(total_draft_rows)
    a.lead_slots = int(lead_slots)
    a.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    a.target_logits = _ptr(target_logits)
    a.draft_logits = _ptr(draft_logits)
    a.cu_gamma = _ptr(cu_gamma)
    a.draft_tokens = _ptr(draft_tokens)
    a.temperature = _ptr(temperature)
    a.top_p = _ptr(top_p)
    a.top_k = _ptr(top_k)
    a.seq_id = _ptr(seq_id)
    a.committed_len = _ptr(committed_len)
    a.out_tokens = _ptr(out_tokens)
    a.num_accepted = _ptr(num_accepted)
    a.seq_flags = _ptr(seq_flags)
    a.probe_rows = _ptr(probe_rows)
    a.probe_seq = _ptr(probe_seq)
    a.uniform_override = _ptr(uniform_override)
    a.eos_token = _ptr(eos_token)
    a.max_emit = _ptr(max_emit)
    a.num_emitted = _ptr(num_emitted)
    _keep(a, target_logits, draft_logits, cu_gamma, draft_tokens, temperature, top_p, top_k,
          seq_id, committed_len, out_tokens, num_accepted, seq_flags, probe_rows, probe_seq,
          uniform_override, eos_token, max_emit, num_emitted)
    return a


def spec_verify_chain(args: spec_chain_args, workspace=None, stream=None, device=None):
    """Enqueues chain verification (see spec_verify.h). ``workspace`` is a uint8 device
    tensor (allocated here when None). Returns the workspace tensor for reuse."""
    need = spec_verify_chain_workspace_size(max(args.batch, 0), max(args.total_draft_rows, 0),
                                            max(args.vocab, 1))
    if workspace is None and args.batch > 0 and need > 0:
        workspace = _workspace(need, device or torch.device("cuda"))
    ws = _ptr(workspace)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().spec_verify_chain(ctypes.byref(args), ws, nbytes, _stream(stream)))
    return workspace


def spec_verify_chain_timed(args: spec_chain_args, events, workspace, stream=None):
    """spec_verify_chain with an EventPair recorded around its row-statistics kernel."""
    _check(lib().spec_verify_chain_timed(ctypes.byref(args), _ptr(workspace), workspace.numel(),
                                         _stream(stream), events.ptr))


def spec_verify_chain_noalloc(args: spec_chain_args, stream=None):
    """Enqueues chain verification on the library's own scratch memory (see spec_verify.h):
    nothing is allocated."""
    _check(lib().spec_verify_chain_noalloc(ctypes.byref(args), _stream(stream)))


# Bytes of the library's scratch array per GPU (SPEC_CHAIN_SCRATCH_BYTES).
CHAIN_SCRATCH_BYTES = 80 << 20


def tree_args(*, target_logits, parent, node_row, node_token, path_nodes, path_len,
              out_tokens, num_emitted, vocab, rows_per_seq, max_depth, tree_stride,
              seq_flags=None, row_stride=None):
    a = spec_tree_args()
    a.batch = int(node_token.shape[0])
    a.vocab = int(vocab)
    a.row_stride = int(row_stride if row_stride is not None else target_logits.shape[-1])
    a.num_nodes = int(node_token.shape[1])
    a.rows_per_seq = int(rows_per_seq)
    a.max_depth = int(max_depth)
    a.tree_stride = int(tree_stride)
    a.target_logits = _ptr(target_logits)
    a.parent = _ptr(parent)
    a.node_row = _ptr(node_row)
    a.node_token = _ptr(node_token)
    a.path_nodes = _ptr(path_nodes)
    a.path_len = _ptr(path_len)
    a.out_tokens = _ptr(out_tokens)
    a.num_emitted = _ptr(num_emitted)
    a.seq_flags = _ptr(seq_flags)
    _keep(a, target_logits, parent, node_row, node_token, path_nodes, path_len, out_tokens,
          num_emitted, seq_flags)
    return a


def spec_verify_tree(args: spec_tree_args, workspace=None, stream=None, device=None):
    need = spec_verify_tree_workspace_size(max(args.batch, 0), max(args.rows_per_seq, 1))
    if workspace is None and args.batch > 0 and need > 0:
        workspace = _workspace(need, device or torch.device("cuda"))
    ws = _ptr(workspace)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().spec_verify_tree(ctypes.byref(args), ws, nbytes, _stream(stream)))
    return workspace


def kv_args(*, k_cache, v_cache, path_nodes, path_len, committed_len, num_kv_heads, head_dim,
            seq_stride, slot_stride, head_stride, slot_capacity, lead_slots, max_depth,
            seq_flags=None):
    """k_cache / v_cache: lists of device tensors (one per layer) or raw pointers."""
    nl = len(k_cache)
    a = spec_kv_args()
    a.batch = int(path_len.shape[0])
    a.num_layers = nl
    a.num_kv_heads = int(num_kv_heads)
    a.head_dim = int(head_dim)
    a.seq_stride, a.slot_stride, a.head_stride = int(seq_stride), int(slot_stride), int(head_stride)
    a.slot_capacity = int(slot_capacity)
    a.lead_slots = int(lead_slots)
    a.max_depth = int(max_depth)
    arr_k = (ctypes.c_void_p * nl)(*[_ptr(t) for t in k_cache])
    arr_v = (ctypes.c_void_p * nl)(*[_ptr(t) for t in v_cache])
    a._keep = (arr_k, arr_v)  # the host arrays must live until the call returns
    a.k_cache = ctypes.cast(arr_k, _P)
    a.v_cache = ctypes.cast(arr_v, _P)
    a.path_nodes = _ptr(path_nodes)
    a.path_len = _ptr(path_len)
    a.committed_len = _ptr(committed_len)
    a.seq_flags = _ptr(seq_flags)
    _keep(a, path_nodes, path_len, committed_len, seq_flags, *k_cache, *v_cache)
    return a


def kv_commit_path(args: spec_kv_args, stream=None):
    _check(lib().kv_commit_path(ctypes.byref(args), _stream(stream)))


def kv_paged_args(*, k_cache, v_cache, block_table, path_nodes, path_len, committed_len,
                  free_list, free_count, num_kv_heads, head_dim, block_size, num_blocks,
                  block_stride, slot_stride, head_stride, lead_slots, max_depth,
                  seq_flags=None):
    """k_cache / v_cache: lists of device tensors (one per layer) or raw pointers; the block
    table is [B, max_blocks] and the free list [free_capacity] (device int32)."""
    nl = len(k_cache)
    a = spec_paged_kv_args()
    a.batch = int(block_table.shape[0])
    a.num_layers = nl
    a.num_kv_heads = int(num_kv_heads)
    a.head_dim = int(head_dim)
    a.block_size = int(block_size)
    a.max_blocks = int(block_table.shape[1])
    a.num_blocks = int(num_blocks)
    a.free_capacity = int(free_list.shape[0])
    a.lead_slots = int(lead_slots)
    a.max_depth = int(max_depth)
    a.block_stride, a.slot_stride = int(block_stride), int(slot_stride)
    a.head_stride = int(head_stride)
    arr_k = (ctypes.c_void_p * nl)(*[_ptr(t) for t in k_cache])
    arr_v = (ctypes.c_void_p * nl)(*[_ptr(t) for t in v_cache])
    a._keep = (arr_k, arr_v)  # the host arrays must live until the call returns
    a.k_cache = ctypes.cast(arr_k, _P)
    a.v_cache = ctypes.cast(arr_v, _P)
    a.block_table = _ptr(block_table)
    a.path_nodes = _ptr(path_nodes)
    a.path_len = _ptr(path_len)
    a.committed_len = _ptr(committed_len)
    a.free_list = _ptr(free_list)
    a.free_count = _ptr(free_count)
    a.seq_flags = _ptr(seq_flags)
    _keep(a, block_table, path_nodes, path_len, committed_len, free_list, free_count,
          seq_flags, *k_cache, *v_cache)
    return a


def kv_commit_paged(args: spec_paged_kv_args, stream=None):
    _check(lib().kv_commit_paged(ctypes.byref(args), _stream(stream)))


def ngram_args(*, tokens, hist_len, draft_tokens, num_drafts, ngram_min, ngram_max,
               num_draft, match_len=None, match_pos=None, seq_flags=None):
    """tokens [B, hist_stride] and draft_tokens [B, draft_stride] are device int32 tensors."""
    a = spec_ngram_args()
    a.batch = int(tokens.shape[0])
    a.hist_stride = int(tokens.shape[1])
    a.ngram_min, a.ngram_max = int(ngram_min), int(ngram_max)
    a.num_draft = int(num_draft)
    a.draft_stride = int(draft_tokens.shape[1])
    a.tokens = _ptr(tokens)
    a.hist_len = _ptr(hist_len)
    a.draft_tokens = _ptr(draft_tokens)
    a.num_drafts = _ptr(num_drafts)
    a.match_len = _ptr(match_len)
    a.match_pos = _ptr(match_pos)
    a.seq_flags = _ptr(seq_flags)
    _keep(a, tokens, hist_len, draft_tokens, num_drafts, match_len, match_pos, seq_flags)
    return a


def spec_ngram_draft(args: spec_ngram_args, stream=None):
    _check(lib().spec_ngram_draft(ctypes.byref(args), _stream(stream)))


def _tree_config(top_head, top_k_spec):
    th = (_I32 * len(top_head))(*[int(h) for h in top_head])
    flat = [int(k) for s in range(len(top_head)) for k in top_k_spec[s]]
    ks = (_I32 * max(len(flat), 1))(*flat)
    return th, ks


def spec_tree_draft_workspace_size(batch, vocab, top_head, top_k_spec) -> int:
    th, ks = _tree_config(top_head, top_k_spec)
    return int(lib().spec_tree_draft_workspace_size(int(batch), int(vocab), len(top_head),
                                                    ctypes.cast(th, _P), ctypes.cast(ks, _P)))


def tree_draft_args(*, top_head, top_k_spec, step, draft_logits, parent, node_token, node_row,
                    node_logp, position_ids, ancestor_mask, expand_nodes, vocab,
                    root_token=None, pos_base=None, seq_flags=None, row_stride=None):
    """Fills a spec_tree_draft_args; the tree arrays are [B, tree_stride] device tensors,
    ancestor_mask is [B, tree_stride, (tree_stride + 31) // 32] and expand_nodes is
    [B, expand_stride]."""
    a = spec_tree_draft_args()
    a.batch = int(parent.shape[0])
    a.vocab = int(vocab)
    a.row_stride = int(row_stride if row_stride is not None else draft_logits.shape[-1])
    a.depth = len(top_head)
    a.step = int(step)
    a.tree_stride = int(parent.shape[1])
    a.expand_stride = int(expand_nodes.shape[1])
    th, ks = _tree_config(top_head, top_k_spec)
    a._keep_cfg = (th, ks)
    a.top_head = ctypes.cast(th, _P)
    a.top_k_spec = ctypes.cast(ks, _P)
    a.draft_logits = _ptr(draft_logits)
    a.root_token = _ptr(root_token)
    a.pos_base = _ptr(pos_base)
    a.parent = _ptr(parent)
    a.node_token = _ptr(node_token)
    a.node_row = _ptr(node_row)
    a.node_logp = _ptr(node_logp)
    a.position_ids = _ptr(position_ids)
    a.ancestor_mask = _ptr(ancestor_mask)
    a.expand_nodes = _ptr(expand_nodes)
    a.seq_flags = _ptr(seq_flags)
    _keep(a, draft_logits, root_token, pos_base, parent, node_token, node_row, node_logp,
          position_ids, ancestor_mask, expand_nodes, seq_flags)
    return a


def spec_tree_draft_step(args: spec_tree_draft_args, workspace=None, stream=None, device=None):
    """Enqueues one tree-drafting step (see spec_verify.h). Returns the workspace tensor."""
    if workspace is None and args.batch > 0:
        th, ks = args._keep_cfg
        need = int(lib().spec_tree_draft_workspace_size(args.batch, max(args.vocab, 1),
                                                        args.depth, ctypes.cast(th, _P),
                                                        ctypes.cast(ks, _P)))
        if need > 0:
            workspace = _workspace(need, device or torch.device("cuda"))
    ws = _ptr(workspace)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().spec_tree_draft_step(ctypes.byref(args), ws, nbytes, _stream(stream)))
    return workspace


# ---- HIP events for the row-pass timing (spec_verify_chain_timed) -----------------------

_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(_P)]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _P, _P]
        _hip.hipEventSynchronize.argtypes = [_P]
        _hip.hipEventDestroy.argtypes = [_P]
    return _hip


class EventPair:
    """Two hipEvent_t for spec_verify_chain_timed (row-pass start / end)."""

    def __init__(self):
        h = _hiprt()
        self.ev = (_P * 2)()
        for i in range(2):
            e = _P()
            rc = h.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.ev[i] = e
        self.ptr = ctypes.cast(self.ev, _P).value

    def elapsed_ms(self) -> float:
        h = _hiprt()
        h.hipEventSynchronize(self.ev[1])
        ms = ctypes.c_float(0)
        rc = h.hipEventElapsedTime(ctypes.byref(ms), self.ev[0], self.ev[1])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        try:
            h = _hiprt()
            for i in range(2):
                h.hipEventDestroy(self.ev[i])
        except Exception:
            pass
