#!/usr/bin/env python3
"""Benchmark of the verification step on one MI355X.

A step is one spec_verify_chain call (row pass + resolve: temperature/top-p laws, acceptance
test, first rejection, residual/bonus draw, committed-length pointer) over the chain
workload B=256, gamma=8, V=128256, T=0.7, top-p 0.9 with its inputs resident in HBM.
Prints one JSON line with verify rows/s (rows = (sequence, position) target rows,
sum(gamma_b+1) per call), the row-pass kernel's achieved HBM bandwidth against 8 TB/s
(timed live with HIP events on the launch stream), and the fp64 CPU oracle timed on a
bounded sample of the same workload as a reported baseline.

  python bench.py [--steps K] [--warmup W] [--warmup-seconds S] [--gpus 1] [--no-cpu-baseline]
  python bench.py --copy-calibration     # a plain copy of known size, for counter scaling
  python bench.py --workload tree_draft  # the tree-drafting steps of one round instead
  python bench.py --workload paged_kv    # the paged KV commit of the tree workload instead
  python bench.py --workload ngram       # the n-gram prompt lookup instead
  python bench.py --workload tree        # greedy tree verify + KV commit instead
  python bench.py --workload c2|c5       # the other chain workloads (c3 is the default)
  python bench.py --workload c3_no_top_p|c3_greedy|c3_top_k_50   # c3 variants
  python bench.py --workload markov      # the vocab-4 Markov rounds (launch-bound)
  python bench.py --summarize-trace DIR [--cycle NAMES:K] [--remove-csv]  # rocprofv3 trace tables
  python bench.py --summarize-counters DIR [--remove-csv]  # tables of a rocprofv3 --pmc run

With --workload tree_draft a step is one round of tree drafting ("投机推理：小模型搭树，
大模型一次验证": top_head [1, 2, 2], top_k_spec [[6], [2, 2], [1, 1]]) over B=128 sequences
with V=151936 draft rows: three spec_tree_draft_step calls reading 128, 256 and 256 draft
rows. The rounds take three copies of the draft rows in turn (3 x 194 MB, more than the
256 MB memory-side cache), so every round reads its rows from HBM. The line reports draft
rows/s and the HBM bandwidth of the steps against 8 TB/s.

With --workload paged_kv a step is one kv_commit_paged call committing the tree workload's
accepted paths (B=128, depth <= 3) into a cache of 32 layers x K,V x 8 heads x 128 bf16 paged
in 16-slot blocks (64 shuffled blocks per sequence, 17.2 GB), releasing the surplus blocks.
The block table, lengths and free count are restored before each call, outside the events
that time it.

With --workload tree a step is one spec_verify_tree call over the tree workload (B=128,
V=151936, 5 target rows and 12 nodes per sequence, tree [6], [2, 2], [1, 1]) followed by one
kv_commit_path of the accepted paths into a contiguous cache of 32 layers x K,V x 8 heads x
128 bf16 (1024 slots per sequence, 17.2 GB). The steps take three copies of the target rows
in turn (3 x 194 MB, more than the 256 MB memory-side cache), so every call reads its rows
from HBM. The committed lengths are restored before each step, outside the events. The line reports verify rows/s and the verify call's HBM bandwidth
(the argmax kernel's rows, plus its small walk launch) against 8 TB/s; the commit's time and
bytes ride along under "kv_commit".

With --workload ngram a step is one spec_ngram_draft call over B=256 token histories of
U{1024..8192} tokens (prompt_lookup_min 1, max 4, 8 drafts); the bytes are the histories'
tokens, read once.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
# Copies of a workload's rows that the tree and tree-drafting legs take in turn: together
# they exceed the 256 MB memory-side cache, so each call reads its rows from HBM.
ROTATE = 3
METRIC = "verify rows/sec at B=256 γ=8 V=128k; achieved HBM GB/s vs peak"
SEED = 2024
SEED_DRAFT = 9090
ROW_KERNEL = "row_stats_kernel"
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "row_stats_kernel_c3.md")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Each workload's kernel sources: its kernel files and the library headers they include.
CHAIN_SOURCES = ("chain_verify.hip", "row_ops.h", "spec_device.h", "specv_internal.h")
TREE_SOURCES = ("tree_verify.hip", "kv_commit.hip", "row_ops.h", "spec_device.h",
                "specv_internal.h")
TREE_DRAFT_SOURCES = ("tree_draft.hip", "row_ops.h", "spec_device.h", "specv_internal.h")
PAGED_SOURCES = ("kv_paged.hip", "spec_device.h", "specv_internal.h")
NGRAM_SOURCES = ("ngram_draft.hip", "spec_device.h", "specv_internal.h")


def kernel_source_hash(files=None) -> str:
    """First 16 hex digits of the sha256 of the given csrc files (in this order), or of every
    csrc source in name order."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_verification_03_amd", "csrc")
    if files is None:
        files = [f for f in sorted(os.listdir(csrc)) if f.endswith((".hip", ".h", ".cpp"))]
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(x) -> dict:
    """Bytes the verification must move at least once, per call.

    The row kernel reads every logits row once: per draft position its p row and its q row
    (2 * V * 2 B; a greedy sequence's q rows are not read) plus the draft token (4 B), and per
    sequence the bonus row p_{gamma+1} (V * 2 B). The call adds the outputs (tokens,
    accepted counts, committed lengths)."""
    import numpy as np
    cu = x["cu_gamma"]
    B = len(cu) - 1
    nd = int(cu[-1])
    V = x["vocab"]
    b_of = np.repeat(np.arange(B), np.diff(cu))
    nq = int((x["temperature"][b_of] != 0).sum())  # greedy positions read no q row
    row_pass = (nd + nq + B) * V * 2 + nd * 4
    outputs = (nd + B) * 4 + B * 4 * 2
    return dict(row_pass=row_pass, call=row_pass + outputs, rows=int(np.sum(np.diff(cu) + 1)))


def read_traffic(src_hash):
    """HBM traffic per row-pass launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    if not os.path.exists(PROFILE_SUMMARY):
        return None
    text = open(PROFILE_SUMMARY).read()
    m = re.search(r"kernel source hash:\s*`?([0-9a-f]{16})", text)
    t = re.search(r"traffic per launch \(bytes\):\s*([0-9.e+]+)", text)
    if not m or not t or m.group(1) != src_hash:
        return None
    return float(t.group(1))


def _short_kernel_name(name):
    name = name.replace("specv::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", name)


def _csv_rows(d, suffix):
    import csv
    import glob
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            yield from csv.DictReader(fh)


def _grid(r):
    g = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
    w = int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 1)
    return g // max(w, 1), w


def summarize_trace(d, last=100, cycle=None):
    """Per (kernel, workgroups, workgroup size) of a rocprofv3 --kernel-trace csv run: the
    dispatch count and the mean, median, min and max duration in us, over every dispatch and
    over the last `last` ones, then the median gap between consecutive dispatches of the last
    3 * `last`. With cycle = (names, K): the dispatches of the kernels named (by prefix), in
    launch order, are cut into runs of K (one call or round each; runs that do not hold the
    same kernel sequence as the first are dropped), and each position of the run gets its
    median duration and median gap after the dispatch before it. Written to DIR/summary.txt
    and printed."""
    import statistics as st
    rows = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                   _short_kernel_name(r["Kernel_Name"])) + _grid(r)
                  for r in _csv_rows(d, "kernel_trace.csv"))
    groups = {}
    for s0, e0, n, g, w in rows:
        groups.setdefault((n, g, w), []).append((e0 - s0) / 1e3)
    out = [f"dispatches: {len(rows)}",
           f"{'kernel':58s} {'wgs':>7s} {'wg':>5s} {'n':>6s} {'avg':>9s} {'med':>9s} "
           f"{'min':>9s} {'max':>9s} | last{last}: avg med"]
    for (n, g, w), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        tail = ds[-last:]
        out.append(f"{n[:58]:58s} {g:7d} {w:5d} {len(ds):6d} {st.mean(ds):9.2f} "
                   f"{st.median(ds):9.2f} {min(ds):9.2f} {max(ds):9.2f} | "
                   f"{st.mean(tail):8.2f} {st.median(tail):8.2f}")
    gaps = {}
    tail = rows[-3 * last:]
    for a, b in zip(tail, tail[1:]):
        gaps.setdefault((a[2][:30], b[2][:30]), []).append((b[0] - a[1]) / 1e3)
    out.append("gaps between consecutive dispatches (last ones), median us:")
    out += [f"  {a} -> {b}: {st.median(v):.2f} (n={len(v)})" for (a, b), v in gaps.items()]
    if cycle:
        names, k = cycle
        sel = [r for r in rows if any(r[2].startswith(n) for n in names)]
        runs = [sel[i:i + k] for i in range(0, len(sel) - k + 1, k)]
        runs = [r for r in runs if [x[2] for x in r] == [x[2] for x in runs[0]]][-last:]
        out.append(f"runs of {k} dispatches of {', '.join(names)} (last {len(runs)}), median us:")
        for j in range(k):
            dur = st.median((r[j][1] - r[j][0]) / 1e3 for r in runs)
            gap = st.median((r[j][0] - r[j - 1][1]) / 1e3 for r in runs) if j else float("nan")
            out.append(f"  {j}: {runs[0][j][2][:40]:40s} wgs={runs[0][j][3]:6d} "
                       f"duration {dur:7.2f}  gap before {gap:6.2f}")
        out.append(f"  run (first start to last end): "
                   f"{st.median((r[-1][1] - r[0][0]) / 1e3 for r in runs):.2f}")
    return out


def summarize_counters(d):
    """Per (kernel, workgroups, counter) of a rocprofv3 --pmc csv run: the dispatch count and
    the mean, min and max of the counter summed over its instances (FETCH_SIZE and WRITE_SIZE
    are in KiB). Written to DIR/counters.txt and printed."""
    import statistics as st
    vals = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        key = (_short_kernel_name(r["Kernel_Name"]), _grid(r)[0], r["Counter_Name"])
        per = vals.setdefault(key, {})
        per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    out = []
    for (n, g, c), per in sorted(vals.items()):
        v = list(per.values())
        out.append(f"{n[:56]:56s} wgs={g:7d} {c:18s} n={len(v):4d} mean={st.mean(v):16.1f} "
                   f"min={min(v):16.1f} max={max(v):16.1f}")
    return out


def _write_summary(d, name, lines, remove_csv):
    import glob
    open(os.path.join(d, name), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))
    if remove_csv:  # the per-dispatch csv files, which can run to hundreds of MB
        for f in glob.glob(os.path.join(d, "**", "*.csv"), recursive=True):
            if f.endswith(("kernel_trace.csv", "counter_collection.csv")):
                os.remove(f)


def cpu_baseline(x, n_seq, min_seconds=10.0):
    """The fp64 oracle as it is, on the first n_seq sequences of the same workload, repeated
    until at least min_seconds of wall time have been spent in it."""
    import numpy as np
    import oracle
    cu = x["cu_gamma"][:n_seq + 1]
    nd = int(cu[-1])
    sub = dict(x)
    sub.update(target=x["target"][:nd + n_seq], draft=x["draft"][:nd], cu_gamma=cu,
               temperature=x["temperature"][:n_seq],
               top_p=None if x["top_p"] is None else x["top_p"][:n_seq],
               seq_id=x["seq_id"][:n_seq], committed_len=x["committed_len"][:n_seq],
               top_k=None if x.get("top_k") is None else x["top_k"][:n_seq])
    b_of = np.repeat(np.arange(n_seq), np.diff(cu))
    tok = oracle.draw_tokens(sub["draft"], sub["temperature"][b_of],
                             None if sub["top_p"] is None else sub["top_p"][b_of], SEED_DRAFT,
                             sub["seq_id"][b_of], sub["committed_len"][b_of] + np.arange(nd) - cu[b_of],
                             vocab=x["vocab"],
                             top_k=None if sub["top_k"] is None else sub["top_k"][b_of])
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    reps, dt = 0, 0.0
    while dt < min_seconds:
        t0 = time.perf_counter()
        oracle.verify_chain_v(sub["target"], sub["draft"], cu, tok, sub["temperature"],
                              sub["top_p"], sub["seq_id"], sub["committed_len"], seed=SEED,
                              vocab=x["vocab"], nthreads=threads, top_k=sub["top_k"])
        dt += time.perf_counter() - t0
        reps += 1
    rows = nd + n_seq
    return dict(value=rows * reps / dt, unit="verify rows/s", cores=threads, kind="oracle",
                sample=f"{n_seq} of {len(x['cu_gamma']) - 1} sequences ({rows} verify rows) "
                       f"verified {reps} times, {dt:.1f} s wall; draft tokens drawn beforehand")


def copy_calibration(nbytes=1 << 30, reps=5):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


def tree_draft_bench(args):
    """One round of tree drafting per step (see the module docstring)."""
    import numpy as np
    import torch

    import ctypes
    from draft_verification_03_amd import binding as B
    from draft_verification_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log("generating the tree-drafting workload (B=128, V=151936, top_head [1,2,2])")
    x = W.tree_draft_inputs()
    th, ks, Bn, V = x["top_head"], x["top_k_spec"], x["batch"], x["vocab"]
    n = 1 + sum(sum(k) for k in ks)
    i32 = dict(dtype=torch.int32, device="cuda")
    t = dict(parent=torch.empty((Bn, n), **i32), node_token=torch.empty((Bn, n), **i32),
             node_row=torch.empty((Bn, n), **i32),
             node_logp=torch.empty((Bn, n), dtype=torch.float32, device="cuda"),
             position_ids=torch.empty((Bn, n), **i32),
             ancestor_mask=torch.empty((Bn, n, (n + 31) // 32), **i32),
             expand_nodes=torch.empty((Bn, max(th)), **i32))
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(  # noqa: E731
        np.int16 if a.dtype == np.uint16 else a.dtype)).cuda()
    # ROTATE copies of the draft rows (3 x 194 MB), one per round in turn, so that a round
    # does not find its rows in the 256 MB memory-side cache from the round before
    root, pos = dv(x["root_token"]), dv(x["pos_base"])
    rounds = []
    for _ in range(ROTATE):
        rows = [dv(r) for r in x["rows"]]
        rounds.append([B.tree_draft_args(top_head=th, top_k_spec=ks, step=s,
                                         draft_logits=rows[s], root_token=root, pos_base=pos,
                                         vocab=V, **t) for s in range(len(th))])
    ws = torch.empty(B.spec_tree_draft_workspace_size(Bn, V, th, ks), dtype=torch.uint8,
                     device="cuda")
    L = B.lib()
    wsp, wsn = ws.data_ptr(), ws.numel()

    def round_(i, stream):
        for a in rounds[i % ROTATE]:
            rc = L.spec_tree_draft_step(ctypes.byref(a), wsp, wsn, stream)
            if rc != 0:
                raise B.SpecError(rc, B.spec_last_error())

    st = torch.cuda.current_stream().cuda_stream
    t_warm = time.time()
    done = 0
    while done < args.warmup or time.time() - t_warm < args.warmup_seconds:
        for _ in range(10):
            round_(done, st)
            done += 1
        torch.cuda.synchronize()
    log(f"timing {args.steps} rounds")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        round_(i, st)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    nrows = Bn * sum(th)
    row_bytes = nrows * V * 2
    gbs = row_bytes / (ms / 1e3) / 1e9
    log(f"round {ms * 1e3:.1f} us for {nrows} draft rows ({gbs:.0f} GB/s)")
    res = {
        "metric": "tree drafting: draft rows/s at B=128 V=151936, top_head [1,2,2], "
                  "top_k_spec [[6],[2,2],[1,1]]; achieved HBM GB/s vs peak",
        "value": nrows / (ms / 1e3), "unit": "draft rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "tree drafting round, B=128, V=151936 bf16 draft rows "
                               "N(0,2^2), top_head [1,2,2], top_k_spec [[6],[2,2],[1,1]]",
                   "draft_rows_per_round": nrows, "round_algorithmic_bytes": row_bytes,
                   "input_sets": ROTATE},
        "roofline": {"bound": "hbm", "kernel": "draft_topk_kernel + tree_grow_kernel",
                     "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                     "bytes_per_launch": row_bytes, "avg_launch_us": ms * 1e3,
                     "kernel_source_hash": kernel_source_hash(TREE_DRAFT_SOURCES)},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("timing the oracle on whole rounds")
        oracle.lib()
        t0 = time.time()
        reps = 0
        while time.time() - t0 < 10.0 or reps == 0:
            oracle.tree_draft(x["rows"], th, ks, x["root_token"], pos_base=x["pos_base"],
                              vocab=V, nthreads=16)
            reps += 1
        el = time.time() - t0
        res["cpu_baseline"] = {"value": reps * nrows / el, "unit": "draft rows/s", "cores": 16,
                               "kind": "oracle",
                               "sample": f"{reps} whole rounds ({nrows} draft rows each), "
                                         f"{el:.1f} s wall"}
    print(json.dumps(res), flush=True)


def paged_kv_bench(args):
    """The paged KV commit of the tree workload (see the module docstring)."""
    import numpy as np
    import torch

    import oracle
    from draft_verification_03_amd import binding as B
    from draft_verification_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log("generating the tree workload's accepted paths")
    x = W.tree_inputs()
    o = oracle.verify_tree(x["logits"], x["parent"], x["node_row"], x["node_token"],
                           x["rows_per_seq"], x["max_depth"], x["num_nodes"], vocab=x["vocab"])
    NL, H, Dh, S = (W.KV_SHAPE[k] for k in ("num_layers", "num_kv_heads", "head_dim", "slots"))
    Bn, bs = 128, 16
    mb = S // bs
    nb = Bn * mb
    rng = np.random.default_rng(404)
    bt0 = rng.permutation(nb).astype(np.int32).reshape(Bn, mb)
    L0, paths, plen = x["committed_len"], o["path_nodes"], o["path_len"]
    log(f"allocating the paged cache ({2 * NL * nb * bs * H * Dh * 2 / 1e9:.1f} GB)")
    caches = [[torch.empty((nb, bs, H, Dh), dtype=torch.int16, device="cuda").random_(-32768, 32767)
               for _ in range(2)] for _ in range(NL)]
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    bt_init, L_init = dv(bt0), dv(L0)
    btt, Lt = bt_init.clone(), L_init.clone()
    ft = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    fct = torch.zeros(1, dtype=torch.int32, device="cuda")
    a = B.kv_paged_args(k_cache=[c[0] for c in caches], v_cache=[c[1] for c in caches],
                        block_table=btt, path_nodes=dv(paths), path_len=dv(plen),
                        committed_len=Lt, free_list=ft, free_count=fct, num_kv_heads=H,
                        head_dim=Dh, block_size=bs, num_blocks=nb, block_stride=bs * H * Dh,
                        slot_stride=H * Dh, head_stride=Dh, lead_slots=1,
                        max_depth=x["max_depth"])

    def restore():
        btt.copy_(bt_init)
        Lt.copy_(L_init)
        fct.zero_()

    t_warm = time.time()
    done = 0
    while done < args.warmup or time.time() - t_warm < args.warmup_seconds:
        restore()
        B.kv_commit_paged(a)
        done += 1
        if done % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"timing {args.steps} calls")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        restore()
        e0.record()
        B.kv_commit_paged(a)
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    moved = sum(int((paths[b, :plen[b]] != np.arange(1, plen[b] + 1)).sum()) for b in range(Bn))
    row_bytes = NL * 2 * H * Dh * 2  # one slot's K and V rows in every layer
    nbytes = 2 * moved * row_bytes + Bn * mb * 4  # moved rows read + written, tables read
    released = int(fct.cpu()[0])
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"commit {ms * 1e3:.1f} us: {moved} rows moved ({2 * moved * row_bytes / 1e6:.1f} MB "
        f"read + written), {released} blocks released, {gbs:.0f} GB/s")
    res = {
        "metric": "paged KV commit: sequences/s at B=128, 32 layers x 8 KV heads x 128, "
                  "16-slot blocks; achieved HBM GB/s vs peak",
        "value": Bn / (ms / 1e3), "unit": "sequences/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u16", "data": "synthetic",
        "config": {"workload": "paged KV commit of the tree workload's accepted paths, B=128, "
                               "32 layers x K,V x 8 heads x 128 bf16, 16-slot blocks, 64 "
                               "shuffled blocks per sequence",
                   "rows_moved": moved, "blocks_released": released,
                   "call_algorithmic_bytes": nbytes},
        "roofline": {"bound": "hbm", "kernel": "paged_copy_kernel + paged_release_kernel",
                     "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None, "bytes_per_launch": nbytes,
                     "avg_launch_us": ms * 1e3,
                     "kernel_source_hash": kernel_source_hash(PAGED_SOURCES)},
    }
    print(json.dumps(res), flush=True)
    del caches
    torch.cuda.empty_cache()


def tree_bench(args):
    """Greedy tree verify and the contiguous KV commit of the tree workload (see the module
    docstring)."""
    import numpy as np
    import torch

    from draft_verification_03_amd import binding as B
    from draft_verification_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log("generating the tree workload (B=128, V=151936, 5 rows and 12 nodes per sequence)")
    x = W.tree_inputs()
    Bn = x["node_token"].shape[0]
    R, md, V = x["rows_per_seq"], x["max_depth"], x["vocab"]
    lg = x["logits"]
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(  # noqa: E731
        {np.dtype(np.uint16): np.int16}.get(a.dtype, a.dtype))).cuda()
    # ROTATE copies of the target rows (3 x 194 MB), one per step in turn, so that a call
    # does not find its rows in the 256 MB memory-side cache from the call before
    logit_sets = [dv(lg.reshape(-1, lg.shape[-1])) for _ in range(ROTATE)]
    pn = torch.full((Bn, md), -1, dtype=torch.int32, device="cuda")
    pl = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    out = torch.full((Bn, md + 1), -1, dtype=torch.int32, device="cuda")
    ne = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    tfl = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    parent, node_row, node_token = dv(x["parent"]), dv(x["node_row"]), dv(x["node_token"])
    tas = [B.tree_args(target_logits=lgs, parent=parent, node_row=node_row,
                       node_token=node_token, path_nodes=pn, path_len=pl, out_tokens=out,
                       num_emitted=ne, seq_flags=tfl, vocab=V, rows_per_seq=R, max_depth=md,
                       tree_stride=x["num_nodes"], row_stride=lg.shape[-1])
           for lgs in logit_sets]
    ws = torch.empty(max(B.spec_verify_tree_workspace_size(Bn, R), 1), dtype=torch.uint8,
                     device="cuda")
    NL, H, Dh, S = (W.KV_SHAPE[k] for k in ("num_layers", "num_kv_heads", "head_dim", "slots"))
    log(f"allocating the cache ({2 * NL * Bn * S * H * Dh * 2 / 1e9:.1f} GB)")
    caches = [[torch.empty((Bn, S, H, Dh), dtype=torch.int16, device="cuda").random_(-32768, 32767)
               for _ in range(2)] for _ in range(NL)]
    L_init = dv(x["committed_len"])
    Lt = L_init.clone()
    kfl = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    ka = B.kv_args(k_cache=[c[0] for c in caches], v_cache=[c[1] for c in caches],
                   path_nodes=pn, path_len=pl, committed_len=Lt, seq_flags=kfl,
                   num_kv_heads=H, head_dim=Dh, seq_stride=S * H * Dh, slot_stride=H * Dh,
                   head_stride=Dh, slot_capacity=S, lead_slots=1, max_depth=md)

    def step(i):
        B.spec_verify_tree(tas[i % ROTATE], workspace=ws)
        B.kv_commit_path(ka)

    t_warm = time.time()
    done = 0
    while done < args.warmup or time.time() - t_warm < args.warmup_seconds:
        Lt.copy_(L_init)
        step(done)
        done += 1
        if done % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
           for _ in range(args.steps)]
    for i, (e0, e1, e2) in enumerate(evs):
        Lt.copy_(L_init)
        e0.record()
        B.spec_verify_tree(tas[i % ROTATE], workspace=ws)
        e1.record()
        B.kv_commit_path(ka)
        e2.record()
    torch.cuda.synchronize()
    ms_tree = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in evs]))
    ms_kv = float(np.mean([e1.elapsed_time(e2) for _, e1, e2 in evs]))
    paths, plen = pn.cpu().numpy(), pl.cpu().numpy()
    assert not kfl.cpu().numpy().any(), "KV commit flagged a sequence"
    assert not (tfl.cpu().numpy() & B.FLAG_BAD_TREE).any(), "tree flagged as malformed"
    moved = sum(int((paths[b, :plen[b]] != np.arange(1, plen[b] + 1)).sum()) for b in range(Bn))
    rows = Bn * R
    tree_bytes = rows * V * 2
    kv_bytes = 2 * moved * NL * 2 * H * Dh * 2  # moved K and V rows, read and written
    gbs = tree_bytes / (ms_tree / 1e3) / 1e9
    kv_gbs = kv_bytes / (ms_kv / 1e3) / 1e9
    ms = ms_tree + ms_kv
    log(f"verify {ms_tree * 1e3:.1f} us ({gbs:.0f} GB/s), commit {ms_kv * 1e3:.1f} us "
        f"({moved} rows moved, {kv_bytes / 1e6:.1f} MB read + written, {kv_gbs:.0f} GB/s), "
        f"path lengths {np.bincount(plen, minlength=md + 1).tolist()}")
    res = {
        "metric": "tree verify rows/sec at B=128 V=151936, 5 rows per sequence, with the KV "
                  "commit of the accepted paths; achieved HBM GB/s vs peak",
        "value": rows / (ms / 1e3), "unit": "verify rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": "greedy tree verify, B=128, V=151936, tree [6], [2, 2], [1, 1] "
                               "(12 nodes, 5 rows), then KV commit of the accepted paths, 32 "
                               "layers x K,V x 8 heads x 128 bf16, 1024 slots",
                   "rows": rows, "rows_moved": moved, "input_sets": ROTATE},
        "roofline": {"bound": "hbm", "kernel": "tree_argmax_kernel + tree_walk_kernel",
                     "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                     "bytes_per_launch": tree_bytes, "avg_launch_us": ms_tree * 1e3,
                     "kernel_source_hash": kernel_source_hash(TREE_SOURCES)},
        "kv_commit": {"kernel": "kv_copy_kernel + kv_pointer_kernel", "us": ms_kv * 1e3,
                      "bytes": kv_bytes, "achieved": kv_gbs, "frac": kv_gbs / PEAK_HBM_GBS},
    }
    print(json.dumps(res), flush=True)
    del caches
    torch.cuda.empty_cache()


def ngram_bench(args):
    """The n-gram prompt lookup (see the module docstring)."""
    import numpy as np
    import torch

    from draft_verification_03_amd import binding as B
    from draft_verification_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log("generating the n-gram workload (B=256, 1024..8192 tokens)")
    x = W.ngram_inputs()
    Bn, g = x["batch"], 8
    tok = torch.from_numpy(x["tokens"]).cuda()
    lens = torch.from_numpy(x["hist_len"]).cuda()
    d = torch.empty((Bn, g), dtype=torch.int32, device="cuda")
    nd = torch.empty(Bn, dtype=torch.int32, device="cuda")
    a = B.ngram_args(tokens=tok, hist_len=lens, draft_tokens=d, num_drafts=nd, ngram_min=1,
                     ngram_max=4, num_draft=g)
    t_warm = time.time()
    done = 0
    while done < args.warmup or time.time() - t_warm < args.warmup_seconds:
        for _ in range(10):
            B.spec_ngram_draft(a)
        done += 10
        torch.cuda.synchronize()
    log(f"timing {args.steps} calls")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        B.spec_ngram_draft(a)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    nbytes = int(x["hist_len"].sum()) * 4 + Bn * (g + 1) * 4
    gbs = nbytes / (ms / 1e3) / 1e9
    drafted = int((nd > 0).sum())
    log(f"lookup {ms * 1e3:.1f} us for {Bn} histories ({gbs:.0f} GB/s), {drafted} drafted")
    res = {
        "metric": "n-gram prompt lookup: sequences/s at B=256, 1024..8192-token histories; "
                  "achieved HBM GB/s vs peak",
        "value": Bn / (ms / 1e3), "unit": "sequences/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": "n-gram prompt lookup, B=256 histories of U{1024..8192} tokens "
                               "(half fresh spans, half copies of earlier spans), n in [1, 4], "
                               "8 drafts",
                   "call_algorithmic_bytes": nbytes, "sequences_drafted": drafted},
        "roofline": {"bound": "hbm", "kernel": "ngram_draft_kernel", "achieved": gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": None, "bytes_per_launch": nbytes, "avg_launch_us": ms * 1e3,
                     "kernel_source_hash": kernel_source_hash(NGRAM_SOURCES)},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("timing the oracle on the whole batch")
        t0 = time.time()
        reps = 0
        while time.time() - t0 < 10.0 or reps == 0:
            oracle.ngram_draft(x["tokens"], x["hist_len"], 1, 4, g)
            reps += 1
        el = time.time() - t0
        res["cpu_baseline"] = {"value": reps * Bn / el, "unit": "sequences/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} whole batches of {Bn} histories, "
                                         f"{el:.1f} s wall, one thread"}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-seconds", type=float, default=1.0)
    ap.add_argument("--cpu-sample-seqs", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--workload", default="chain",
                    choices=["chain", "c2", "c3", "c5", "c3_no_top_p", "c3_greedy",
                             "c3_top_k_50", "markov", "tree", "tree_draft", "paged_kv",
                             "ngram"])
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--cycle", metavar="NAMES:K",
                    help="with --summarize-trace: per-position times of runs of K dispatches "
                         "of the comma-separated kernels, e.g. "
                         "draft_topk_kernel,tree_grow_kernel:6")
    ap.add_argument("--summarize-counters", metavar="DIR")
    ap.add_argument("--remove-csv", action="store_true")
    args = ap.parse_args()
    if args.summarize_trace:
        cyc = None
        if args.cycle:
            names, k = args.cycle.rsplit(":", 1)
            cyc = (names.split(","), int(k))
        _write_summary(args.summarize_trace, "summary.txt",
                       summarize_trace(args.summarize_trace, 100, cyc), args.remove_csv)
        return
    if args.summarize_counters:
        _write_summary(args.summarize_counters, "counters.txt",
                       summarize_counters(args.summarize_counters), args.remove_csv)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the verification step has no cross-GPU exchange in "
              "this build (batch sharding is independent per GPU); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload == "tree_draft":
        tree_draft_bench(args)
        return
    if args.workload == "paged_kv":
        paged_kv_bench(args)
        return
    if args.workload == "ngram":
        ngram_bench(args)
        return
    if args.workload == "tree":
        tree_bench(args)
        return
    if args.workload == "markov":
        markov_bench(args)
        return
    chain_bench(args, "c3" if args.workload == "chain" else args.workload)


# Chain workloads: what each line reports and how its inputs are held in HBM. "base" names
# the configuration the inputs come from and "mod" how a variant changes it.
CHAIN_LEGS = {
    "c2": dict(sets=16, workload="chain verify B=64 gamma=4 V=32000 bf16 logits, target "
                                 "N(0,2^2), draft = target + N(0,0.5^2), T=1, no top-k/top-p; "
                                 "16 input sets (590 MB) rotated call by call, so that the "
                                 "working set exceeds twice the 256 MB last-level cache"),
    "c3": dict(sets=1, workload="chain verify B=256 gamma=8 V=128256 bf16 logits, target "
                                "N(0,3^2) with 1% of ids +8, draft = target + N(0,1^2), T=0.7, "
                                "top-p 0.9 on p and q"),
    "c5": dict(sets=1, workload="ragged chain verify B=1024 gamma_b~U{1..8} V=128256 bf16 "
                                "logits, target N(0,2^2), draft noise sigma_b~U[0.3,1.5], "
                                "T_b~U[0.5,1.2], no top-k/top-p, bonus on full accept, pointer "
                                "rollback"),
    "c3_no_top_p": dict(sets=1, base="c3", mod=dict(top_p=None),
                        workload="the c3 chain workload without top-p (every draw reads its "
                                 "rows)"),
    "c3_greedy": dict(sets=1, base="c3", mod=dict(temperature=0.0),
                      workload="the c3 chain workload at T=0 (greedy: argmax rows, q rows "
                               "not read)"),
    "c3_top_k_50": dict(sets=1, base="c3", top_k=50,
                        workload="the c3 chain workload with top-k 50 ahead of top-p 0.9"),
}


def chain_bench(args, name):
    """One spec_verify_chain call per step over chain workload ``name`` (c2, c3, c5)."""
    import numpy as np
    import torch

    from draft_verification_03_amd import binding as B
    from draft_verification_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    leg = CHAIN_LEGS[name]
    nsets = leg["sets"]
    log(f"generating the {name} workload ({nsets} input set(s))")
    base = leg.get("base", name)
    xs = [W.chain_inputs(base, **leg.get("mod", {})) if i == 0 else
          W.chain_inputs(base, seed=W.SEEDS[base] * 1000 + i, **leg.get("mod", {}))
          for i in range(nsets)]
    if "top_k" in leg:
        for xi in xs:
            xi["top_k"] = np.full(len(xi["cu_gamma"]) - 1, leg["top_k"], np.int32)
    x = xs[0]
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(  # noqa: E731
        {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}.get(a.dtype, a.dtype))).cuda()
    calls = []
    for xi in xs:
        cu = xi["cu_gamma"]
        Bn, nd, V = len(cu) - 1, int(cu[-1]), xi["vocab"]
        tgt, drf = dv(xi["target"]), dv(xi["draft"])
        topp = None if xi["top_p"] is None else dv(xi["top_p"])
        # The drafter's tokens: one gamma = 0 round per draft row through the same library.
        b_of = np.repeat(np.arange(Bn), np.diff(cu))
        k_of = np.arange(nd) - cu[b_of]
        d_out = torch.empty(nd, dtype=torch.int32, device="cuda")
        tk = xi.get("top_k")
        da = B.chain_args(target_logits=drf, cu_gamma=dv(np.zeros(nd + 1, np.int32)),
                          temperature=dv(xi["temperature"][b_of]),
                          top_p=None if xi["top_p"] is None else dv(xi["top_p"][b_of]),
                          top_k=None if tk is None else dv(tk[b_of]),
                          seq_id=dv(xi["seq_id"][b_of]),
                          committed_len=dv((xi["committed_len"][b_of] + k_of).astype(np.int32)),
                          out_tokens=d_out,
                          num_accepted=torch.empty(nd, dtype=torch.int32, device="cuda"),
                          seed=SEED_DRAFT, vocab=V, max_gamma=0, total_draft_rows=0,
                          row_stride=xi["stride"])
        B.spec_verify_chain(da)
        torch.cuda.synchronize()
        L = dv(xi["committed_len"])
        out = torch.empty(nd + Bn, dtype=torch.int32, device="cuda")
        nacc = torch.empty(Bn, dtype=torch.int32, device="cuda")
        flags = torch.empty(Bn, dtype=torch.int32, device="cuda")
        a = B.chain_args(target_logits=tgt, draft_logits=drf, cu_gamma=dv(cu), draft_tokens=d_out,
                         temperature=dv(xi["temperature"]), top_p=topp, seq_id=dv(xi["seq_id"]),
                         top_k=None if tk is None else dv(tk),
                         committed_len=L, out_tokens=out, num_accepted=nacc, seq_flags=flags,
                         seed=SEED, vocab=V, max_gamma=int(np.diff(cu).max()),
                         total_draft_rows=nd, row_stride=xi["stride"])
        ws = torch.empty(B.spec_verify_chain_workspace_size(Bn, nd, V), dtype=torch.uint8,
                         device="cuda")
        calls.append(dict(a=a, ws=ws, L=L, nacc=nacc, flags=flags))
    # Warm-up: the W steps, continued until --warmup-seconds have passed, so that the timed
    # steps run at the GPU's settled clocks (the first few hundred milliseconds of a burst
    # of work run measurably slower). The committed lengths advance call after call; the
    # uniforms are keyed by position, so every call is a fresh round of the same shape.
    t_warm = time.time()
    done = 0
    while done < args.warmup or time.time() - t_warm < args.warmup_seconds:
        for _ in range(10):
            c = calls[done % nsets]
            B.spec_verify_chain(c["a"], workspace=c["ws"])
            done += 1
        torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    # Headline: the steps back to back with nothing between them.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        c = calls[i % nsets]
        B.spec_verify_chain(c["a"], workspace=c["ws"])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # Row-pass durations: the same steps again through spec_verify_chain_timed, which records
    # one event pair on the launch stream around the row kernel.
    evs = [B.EventPair() for _ in range(args.steps)]
    for i, e in enumerate(evs):
        c = calls[i % nsets]
        B.spec_verify_chain_timed(c["a"], e, c["ws"])
    torch.cuda.synchronize()
    row_ms = [e.elapsed_ms() for e in evs]
    ms_step = total_ms / args.steps
    abs_ = [algorithmic_bytes(xi) for xi in xs]
    # per step, averaged over the rotated sets (equal shares of the steps)
    rows = float(np.mean([ab["rows"] for ab in abs_]))
    row_pass = float(np.mean([ab["row_pass"] for ab in abs_]))
    call_bytes = float(np.mean([ab["call"] for ab in abs_]))
    value = rows / (ms_step / 1e3)
    row_avg_ms = float(np.mean(row_ms))
    achieved = row_pass / (row_avg_ms / 1e3) / 1e9
    src_hash = kernel_source_hash(CHAIN_SOURCES)
    traffic = read_traffic(src_hash) if name == "c3" else None
    fl = calls[0]["flags"].cpu().numpy()
    log(f"step {ms_step * 1e3:.1f} us, row pass {row_avg_ms * 1e3:.1f} us "
        f"({achieved:.0f} GB/s), call {call_bytes / (ms_step / 1e3) / 1e9:.0f} GB/s, "
        f"accepted/seq {calls[0]['nacc'].float().mean().item():.3f}, "
        f"top-p multi-pass sequences {int(((fl & B.FLAG_TOPP_SLOW) != 0).sum())}")
    cu = x["cu_gamma"]
    res = {
        "metric": METRIC if name == "c3" else
        f"verify rows/sec, {name} chain workload; achieved HBM GB/s vs peak",
        "value": value,
        "unit": "verify rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": leg["workload"],
                   "batch": len(cu) - 1, "max_gamma": int(np.diff(cu).max()),
                   "vocab": x["vocab"], "input_sets": nsets,
                   "verify_rows_per_call": rows, "call_algorithmic_bytes": call_bytes,
                   "call_hbm_gbs": call_bytes / (ms_step / 1e3) / 1e9},
        "roofline": {"bound": "hbm", "kernel": ROW_KERNEL, "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "bytes_per_launch": row_pass,
                     "avg_launch_us": row_avg_ms * 1e3, "kernel_source_hash": src_hash},
    }
    if not args.no_cpu_baseline:
        n = min(args.cpu_sample_seqs, len(cu) - 1)
        log(f"timing the oracle on the first {n} sequences")
        res["cpu_baseline"] = cpu_baseline(x, n)
    print(json.dumps(res), flush=True)


def markov_bench(args):
    """The vocab-4 Markov workload: one spec_verify_chain call per round (B=1, gamma=4,
    V=4), on rounds whose inputs are all resident in HBM, one call after another. A round of
    a real stream depends on the previous one's output; here the rounds' contexts and drafts
    are drawn beforehand (last token uniform, drafts a chain of the draft table), so the line
    measures the call itself: it is bound by launch latency, not by its 88 bytes (nine
    4-logit bf16 rows and four draft tokens)."""
    import numpy as np
    import torch

    from draft_verification_03_amd import binding as B
    from draft_verification_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    T, D = W.markov_tables()
    tl, dl = W.log_rows_bf16(T), W.log_rows_bf16(D)
    g, nr = 4, 2048
    rng = np.random.default_rng(W.SEEDS["markov"] + 1)
    last = rng.integers(0, 4, size=nr)
    drafts = np.zeros((nr, g), np.int32)
    cdf = np.cumsum(D, axis=1)
    for r in range(nr):
        prev = last[r]
        for j in range(g):
            prev = int(np.searchsorted(cdf[prev], rng.random(), side="right").clip(0, 3))
            drafts[r, j] = prev
    ctx = np.concatenate([last[:, None], drafts], axis=1)
    tgt = tl[ctx.reshape(-1)].reshape(nr, g + 1, 8)
    drf = dl[ctx[:, :g].reshape(-1)].reshape(nr, g, 8)
    i32 = dict(dtype=torch.int32, device="cuda")
    d_tgt = torch.from_numpy(tgt.view(np.int16)).cuda()
    d_drf = torch.from_numpy(drf.view(np.int16)).cuda()
    d_tok = torch.from_numpy(drafts).cuda()
    pos = (np.arange(nr) * 3).astype(np.int32)  # distinct positions: fresh uniforms per round
    d_L = torch.from_numpy(pos.copy()).cuda()
    d_out = torch.zeros((nr, g + 1), **i32)
    d_n = torch.zeros(nr, **i32)
    cu = torch.tensor([0, g], **i32)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.spec_verify_chain_workspace_size(1, g, 4), dtype=torch.uint8,
                     device="cuda")
    args_r = [B.chain_args(target_logits=d_tgt[r], draft_logits=d_drf[r], cu_gamma=cu,
                           draft_tokens=d_tok[r], temperature=one, committed_len=d_L[r:r + 1],
                           out_tokens=d_out[r], num_accepted=d_n[r:r + 1], seed=SEED, vocab=4,
                           max_gamma=g, total_draft_rows=g, row_stride=8) for r in range(nr)]
    t_warm = time.time()
    done = 0
    while done < args.warmup or time.time() - t_warm < args.warmup_seconds:
        for _ in range(10):
            B.spec_verify_chain(args_r[done % nr], workspace=ws)
            done += 1
        torch.cuda.synchronize()
    steps = args.steps
    log(f"timing {steps} rounds")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        B.spec_verify_chain(args_r[i % nr], workspace=ws)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    evs = [B.EventPair() for _ in range(steps)]
    for i, e in enumerate(evs):
        B.spec_verify_chain_timed(args_r[i % nr], e, ws)
    torch.cuda.synchronize()
    row_ms = float(np.mean([e.elapsed_ms() for e in evs]))
    nbytes = (2 * g + 1) * 4 * 2 + g * 4  # the rows' 4 logits each, and the draft tokens
    gbs = nbytes / (row_ms / 1e3) / 1e9
    log(f"round {ms * 1e3:.1f} us ({1e3 / ms:.0f} rounds/s), row kernel {row_ms * 1e3:.1f} us")
    res = {
        "metric": "Markov workload: verification rounds/s at B=1 gamma=4 V=4 (launch-bound)",
        "value": 1e3 / ms, "unit": "rounds/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "vocab-4 Markov rounds, Dirichlet(2) target table, draft = "
                               "target + U(-0.05,0.05) renormalised, B=1, gamma=4, T=1; 2048 "
                               "pre-drawn rounds resident in HBM, one call per round",
                   "call_algorithmic_bytes": nbytes},
        "roofline": {"bound": "hbm", "kernel": ROW_KERNEL, "achieved": gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": None, "bytes_per_launch": nbytes, "avg_launch_us": row_ms * 1e3,
                     "kernel_source_hash": kernel_source_hash(CHAIN_SOURCES),
                     "note": "launch-latency bound: 72 bytes per round"},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("timing the oracle, one call per round")
        t0 = time.time()
        reps = 0
        onef = np.ones(1, np.float32)
        while time.time() - t0 < 10.0 or reps == 0:
            r = reps % nr
            oracle.verify_chain_v(tgt[r], drf[r], np.array([0, g], np.int32), drafts[r], onef,
                                  None, np.zeros(1, np.uint32), pos[r:r + 1], seed=SEED,
                                  vocab=4, nthreads=1)
            reps += 1
        el = time.time() - t0
        res["cpu_baseline"] = {"value": reps / el, "unit": "rounds/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} rounds, one oracle call each (ctypes), "
                                         f"{el:.1f} s wall, one thread"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
