"""Benchmark: tree-indexed sparse decode attention on one MI355X.

One step = one pass of the whole hot path over one batch: zha_build_tree (summary
pyramid over the full cache) followed by zha_attend (top-level scoring, per-level top-p
selection and expansion, sparse GQA decode and split-combine) for every query head.
Default workload: single layer, 256K context (262,144 tokens), bf16, 32 query heads
over 4 KV heads, head dim 128, deep tree b = 4, L = 6, decode batch 4, p = 0.95,
clustered keys with 16 planted needles per sequence (seeded, synthetic).

Prints one JSON line. `value` is query heads per second of whole steps; the same line
reports the decode-only rate (tree prebuilt), per-kernel times from HIP events recorded
on the library's launch stream, the dominant kernel's HBM roofline, keys-read
statistics, and the CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode query-heads/s at 256K deep tree p=0.95; HBM GB/s % of peak; keys-read %"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="256k_deep")
    ap.add_argument("--p", type=float, default=None)
    ap.add_argument("--cpu-units", type=int, default=16,
                    help="(sequence, KV head) units the CPU oracle baseline runs on "
                         "(0: every unit of the batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="geometry sweep on the workload's tensors instead of the benchmark: "
                         "keys read, retained attention mass and needle recall per (b, L, p)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense comparator and the append-build timings (profiling "
                         "runs: every decode dispatch is then the tree-indexed attend's)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only copy a 2 GiB device buffer 5 times (the known-size kernel that "
                         "rocprofv3 HBM counters are scaled by) and print its bandwidth")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (by default the step is also captured as a "
                         "HIP graph and its replays are the headline timing)")
    return ap.parse_args()


# source files whose kernels a counter summary covers (a change to any of them voids it)
KERNEL_FILES = {
    "decode": ["zha_decode.hip", "zha_internal.h"],
    "pool_l1": ["zha_build.hip", "zha_internal.h"],
    "score_l1": ["zha_search.hip", "zha_internal.h"],
}


def kernel_sources_sha(kernel=None) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_indexed_sparse_amd", "csrc")
    files = KERNEL_FILES.get(kernel) or sorted(os.listdir(csrc))
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.calibrate and args.gpus == 1:
        import torch
        dev = torch.device("cuda:0")
        print(json.dumps({"copy_bytes_read": 1 << 31, "copy_bytes_written": 1 << 31,
                          "copies": 5, "copy_gbs": copy_probe(torch, dev, reps=5, warm=0)}),
              flush=True)
        return
    if args.sweep and args.gpus == 1:
        return sweep(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has "
              f"no multi-GPU path. Its (sequence, KV head) units would shard across GPUs with "
              f"no communication.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_indexed_sparse_amd as Z
    from tree_indexed_sparse_amd import _lib as LB
    import workloads as W

    lib = Z.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = W.spec(args.workload)
    p = args.p if args.p is not None else spec["p"][len(spec["p"]) // 2]
    B, T, Hq, Hkv, d, N, b, L = (spec[k] for k in ("B", "T", "Hq", "Hkv", "d", "N", "b", "L"))
    anchor = spec["anchor"]
    QH = B * T * Hq
    elem = 2 if spec["dtype"] == "bf16" else 4

    t0 = time.time()
    inp = W.gen_all(spec, device=dev)
    torch.cuda.synchronize()
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    K, V, Q, R = inp["K"], inp["V"], inp["Q"], inp["R"]

    # preallocated outputs and workspace: the timed region allocates nothing
    tree = Z.build_tree(K, R, b, L)
    O = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev)
    sel = torch.empty((B, T, Hq, N), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, T, Hq), dtype=torch.int32, device=dev)
    ws = torch.empty(Z.workspace_bytes(tree, T, Hq), dtype=torch.uint8, device=dev)

    # rebuild the pyramid in place each step (same storage, same view)
    c_tree = tree.c

    def build_into():
        LB.check(lib.zha_build_tree(K.data_ptr(), R.data_ptr(), c_tree.dtype, B, Hkv, N, N, d, b,
                                    L, tree.storage.data_ptr(), tree.storage.numel(),
                                    ctypes.byref(c_tree), torch.cuda.current_stream().cuda_stream))

    def full_step():
        build_into()
        Z.attend(Q, K, V, tree, p, anchor, out=O, sel_idx=sel, sel_count=cnt, workspace=ws)

    def attend_only():
        Z.attend(Q, K, V, tree, p, anchor, out=O, sel_idx=sel, sel_count=cnt, workspace=ws)

    def timed(fn, steps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, (time.perf_counter() - w0) * 1e3 / steps

    def per_step(fn, steps):
        # each repetition between its own pair of events: spread of the step time
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for a, z in ev:
            a.record()
            fn()
            z.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(z) for a, z in ev])
        return {"p10": round(float(np.percentile(t, 10)), 4),
                "median": round(float(np.median(t)), 4),
                "p90": round(float(np.percentile(t, 90)), 4), "reps": steps}

    # Cache flush between timed repetitions: writing 1 GiB evicts the 4 MB L2 of every XCD
    # and the 256 MB Infinity Cache, so a repetition finds none of the previous one's data
    # on chip (the flush itself sits outside the event pair).
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def flushed(fn, steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for a, z in ev:
            flush_buf.zero_()
            a.record()
            fn()
            z.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(z) for a, z in ev])
        return {"median": round(float(np.median(t)), 4), "mean": round(float(t.mean()), 4),
                "p10": round(float(np.percentile(t, 10)), 4),
                "p90": round(float(np.percentile(t, 90)), 4), "reps": steps}

    for _ in range(args.warmup):
        full_step()
    torch.cuda.synchronize()
    ms_eager, wall_eager = timed(full_step, args.steps)
    print(f"# eager step {ms_eager:.3f} ms (wall {wall_eager:.3f} ms)", file=sys.stderr, flush=True)
    ms_attend_eager, _ = timed(attend_only, args.steps)

    # The step's grids depend only on the cache capacity, so the whole step (every launch
    # of the build and of the attend) is captured once as a HIP graph and replayed: the
    # launch-bound small kernels of the search then run without per-launch host overhead.
    ms_step, ms_attend, graph = ms_eager, ms_attend_eager, False
    dist = None
    fl_step = fl_attend = None
    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    if not args.no_graph:
        g_step = capture(full_step)
        g_attend = capture(attend_only)
        for _ in range(args.warmup):
            g_step.replay()
        ms_step, wall_step = timed(g_step.replay, args.steps)
        ms_attend, _ = timed(g_attend.replay, args.steps)
        dist = per_step(g_step.replay, args.steps)
        fl_step = flushed(g_step.replay, args.steps)
        fl_attend = flushed(g_attend.replay, args.steps)
        graph = True
        print(f"# graph step {ms_step:.3f} ms (wall {wall_step:.3f} ms)", file=sys.stderr,
              flush=True)

    # dense comparator (every head over all N keys, same decode kernels) and the build:
    # one shot versus whole-top-node appends
    dws = torch.empty(Z.dense_workspace_bytes(B, Hkv, N, N, d, T, Hq), dtype=torch.uint8,
                      device=dev)
    O_dense = torch.empty_like(O)

    def dense():
        Z.dense_attend(Q, K, V, N, out=O_dense, workspace=dws)

    top = b ** L
    n_app = N // top
    ms_dense = ms_appends = float("nan")
    if not args.no_extras:
        dense()
        ms_dense, _ = timed(dense, args.steps)

    def appends():
        c_tree.N = 0
        for i in range(n_app):
            LB.check(lib.zha_tree_append(ctypes.byref(c_tree), K.data_ptr(), R.data_ptr(), top,
                                         torch.cuda.current_stream().cuda_stream))

    if not args.no_extras:
        appends()
        ms_appends, _ = timed(appends, max(1, args.steps // 4))
    ms_build, _ = timed(build_into, args.steps)
    torch.cuda.synchronize()

    # one token at a time: the last 4096 tokens of the cache appended one by one to a tree
    # over the tokens before them (each append pools exactly the nodes its token
    # completes; most complete none and launch nothing), eager launches from Python
    one_tok = None
    if not args.no_extras:
        n_one = min(4096, N)

        def one_token_appends():
            c_tree.N = N - n_one
            for _ in range(n_one):
                LB.check(lib.zha_tree_append(ctypes.byref(c_tree), K.data_ptr(), R.data_ptr(),
                                             1, torch.cuda.current_stream().cuda_stream))

        one_token_appends()
        ms_one, wall_one = timed(one_token_appends, 3)
        lib.zha_timing_enable(1)
        one_token_appends()
        lib.zha_timing_enable(0)
        tot, nl = ctypes.c_double(), ctypes.c_int64()
        LB.check(lib.zha_timing_read(LB.ZHA_K_POOL, -1, ctypes.byref(tot), ctypes.byref(nl)))
        one_tok = {"tokens": n_one, "b": b,
                   "gpu_us_per_token": round(1e3 * ms_one / n_one, 3),
                   "host_us_per_token": round(1e3 * wall_one / n_one, 3),
                   "pool_launches": nl.value,
                   "pool_kernel_us_per_token": round(1e3 * tot.value / n_one, 3),
                   "pool_kernel_us_per_launch": round(1e3 * tot.value / max(nl.value, 1), 3),
                   "note": "gpu: HIP events around the 4096 appends (the GPU idles between "
                           "launches the host issues slower than it runs them); host: wall "
                           "time of the Python loop; kernel: the pooling launches' own time"}
        build_into()
        torch.cuda.synchronize()

    # per-kernel durations: HIP events the library records around each of its launches
    lib.zha_timing_enable(1)
    ms_timed_pass, _ = timed(full_step, args.steps)
    lib.zha_timing_enable(0)

    def ktime(kind, level=-1):
        tot, n = ctypes.c_double(), ctypes.c_int64()
        LB.check(lib.zha_timing_read(kind, level, ctypes.byref(tot), ctypes.byref(n)))
        return tot.value, n.value

    kernels = {}
    for name, kind, levels in (("pool", LB.ZHA_K_POOL, range(1, L + 1)),
                               ("score", LB.ZHA_K_SCORE, range(1, L + 1)),
                               ("select", LB.ZHA_K_SELECT, range(1, L + 1)),
                               ("compact", LB.ZHA_K_COMPACT, range(1, L + 1)),
                               ("descent_top", LB.ZHA_K_DESCENT, range(1, L + 1)),
                               ("decode", LB.ZHA_K_DECODE, [0]), ("combine", LB.ZHA_K_COMBINE, [0])):
        for lv in levels:
            tot, n = ktime(kind, lv)
            if n:
                kernels[f"{name}_l{lv}" if lv else name] = dict(avg_ms=tot / n, launches=n)

    # selection statistics and algorithmic bytes from this call's outputs
    attend_only()
    torch.cuda.synchronize()
    counts = cnt.cpu().numpy().reshape(-1).astype(np.int64)
    lists = {lv: Z.level_view(tree, T, Hq, lv, ws) for lv in range(1, L + 1)}
    n1, _, c1 = lists[1]
    U = c1.size
    union_tokens = 0
    for u in range(U):
        # anchor tokens inside the unit's kept nodes are read once, not twice
        first = n1[u, :min(int(c1[u]), -(-anchor // b))].astype(np.int64)
        covered = int(sum(min(b, anchor - nd * b) for nd in first if nd * b < anchor))
        union_tokens += int(c1[u]) * b + (anchor - covered)
    kv_bytes = union_tokens * 2 * d * elem
    decode_bytes = kv_bytes + int(c1.sum()) * 8 + QH * d * elem + QH * d * 4
    frontier_rows = 0
    score_bytes = {}
    members = min(T, max(1, 16 // (Hq // Hkv))) * (Hq // Hkv)
    for lv in range(1, L + 1):
        if lv == L:
            rows = (N // b ** L) * U
            scores = rows * members
        else:
            _, pmasks, pcount = lists[lv + 1]
            rows = int(pcount.sum()) * b
            # with b a multiple of 4 a member's scores are stored only over its own frontier
            # (the children of the nodes it kept one level up); otherwise for every member
            if b % 4 == 0:
                kept = sum(int(np.unpackbits(pmasks[u, :pcount[u]].astype("<u4").view(np.uint8)).sum())
                           for u in range(pmasks.shape[0]))
                scores = kept * b
            else:
                scores = rows * members
        frontier_rows += rows
        # each union-frontier row read once (float32), the members' scores written
        score_bytes[lv] = rows * d * 4 + 4 * scores
    # a pooling launch that starts at level lv reads level lv - 1 once and writes every
    # level it fuses (b^k <= 64 rows per tile, as the library groups them)
    build_bytes = {}
    lv = 1
    while lv <= L:
        k = 1
        while k < L - lv + 1 and b ** (k + 1) <= 64:
            k += 1
        if b > 64:
            k = 1
        child = B * Hkv * (N // b ** (lv - 1)) * d * (elem if lv == 1 else 4)
        build_bytes[lv] = child + sum(B * Hkv * (N // b ** j) * d * 4 for j in range(lv, lv + k))
        lv += k
    list_bytes = 4 * int(counts.sum())
    attend_alg = kv_bytes + frontier_rows * d * 4 + QH * (d * elem + d * 4 + 4) + list_bytes
    step_alg = attend_alg + B * Hkv * N * d * elem + tree_bytes_written(B, Hkv, N, d, b, L)

    alg_bytes = {"decode": decode_bytes}
    for lv in range(1, L + 1):
        alg_bytes[f"score_l{lv}"] = score_bytes[lv]
    for lv, nbytes in build_bytes.items():
        alg_bytes[f"pool_l{lv}"] = nbytes
    # the kernel with the most time per step among those with algorithmic bytes (the fused
    # top-level walk of a small tree can take longer, but moves a few KB)
    dom = max((k for k in kernels if alg_bytes.get(k)),
              key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches"])
    dom_bytes = alg_bytes.get(dom)
    roofline = None
    if dom_bytes is not None:
        ach = dom_bytes / (kernels[dom]["avg_ms"] * 1e-3) / 1e9
        roofline = dict(kernel=dom, bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS,
                        unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4),
                        traffic=pmc_traffic(dom, args.workload), alg_bytes_per_launch=dom_bytes,
                        avg_launch_ms=round(kernels[dom]["avg_ms"], 4))

    # every kernel with algorithmic bytes, against the same peak (the roofline object above
    # is the longest of them): the decode's K/V gather, the scoring and the pooling
    kernel_rooflines = {}
    for name, nbytes in alg_bytes.items():
        if name in kernels and nbytes:
            ach = nbytes / (kernels[name]["avg_ms"] * 1e-3) / 1e9
            kernel_rooflines[name] = dict(achieved_gbs=round(ach, 1),
                                          frac=round(ach / HBM_PEAK_GBS, 4),
                                          traffic=pmc_traffic(name, args.workload),
                                          alg_bytes_per_launch=nbytes)

    kr = counts / N
    keys = dict(mean=round(100 * kr.mean(), 3), min=round(100 * kr.min(), 3),
                median=round(100 * float(np.median(kr)), 3), max=round(100 * kr.max(), 3),
                union=round(100 * union_tokens / (U * N), 3))

    copy_gbs = copy_probe(torch, dev)

    # needle recall: each planted key, in the selected list of the query head aimed at it
    sel_h = sel.cpu().numpy()
    cnt_h = cnt.cpu().numpy()
    hits = total = 0
    for bb in range(B):
        for pos, t, h in W.needle_plan(spec, bb):
            total += 1
            hits += int(pos in set(sel_h[bb, t, h, :cnt_h[bb, t, h]].tolist()))
    needles = {"planted": total, "kept_by_aimed_head": hits,
               "recall": round(hits / total, 4) if total else None}

    # FP4 router (the pages' FP4 router variant): the pyramid's MXFP4 copy written after the
    # build and scored with an MXFP4 query; the float32-router figures above are untouched
    fp4 = None
    if not args.no_extras:
        rbytes = Z.router_bytes(B, Hkv, N, d, b, L)
        rstore = torch.empty(rbytes, dtype=torch.uint8, device=dev)

        def quantize():
            LB.check(lib.zha_router_quantize(ctypes.byref(c_tree), 0, rstore.data_ptr(), rbytes,
                                             torch.cuda.current_stream().cuda_stream))

        def build_fp4():
            # an empty tree given its copy, then extended by the whole cache: the pooling
            # launches write the MXFP4 rows along with the float32 ones
            LB.check(lib.zha_build_tree(K.data_ptr(), R.data_ptr(), c_tree.dtype, B, Hkv, 0, N, d,
                                        b, L, tree.storage.data_ptr(), tree.storage.numel(),
                                        ctypes.byref(c_tree),
                                        torch.cuda.current_stream().cuda_stream))
            quantize()
            LB.check(lib.zha_tree_append(ctypes.byref(c_tree), K.data_ptr(), R.data_ptr(), N,
                                         torch.cuda.current_stream().cuda_stream))

        def step_fp4():
            build_fp4()
            attend_only()

        step_fp4()
        ms4_quant, _ = timed(quantize, args.steps)
        ms4_build, _ = timed(build_fp4, args.steps)
        if args.no_graph:
            ms4_step, _ = timed(step_fp4, args.steps)
            ms4_attend, _ = timed(attend_only, args.steps)
        else:
            g4_step = capture(step_fp4)
            g4_attend = capture(attend_only)
            ms4_step, _ = timed(g4_step.replay, args.steps)
            ms4_attend, _ = timed(g4_attend.replay, args.steps)
        lib.zha_timing_enable(1)
        timed(step_fp4, args.steps)
        lib.zha_timing_enable(0)
        k4 = {}
        for name, kind, levels in (("router", LB.ZHA_K_ROUTER, [0]),
                                   ("pool", LB.ZHA_K_POOL, range(1, L + 1)),
                                   ("score", LB.ZHA_K_SCORE, range(1, L + 1)),
                                   ("descent_top", LB.ZHA_K_DESCENT, range(1, L + 1)),
                                   ("decode", LB.ZHA_K_DECODE, [0])):
            for lv in levels:
                tot, n = ktime(kind, lv)
                if n:
                    k4[f"{name}_l{lv}" if lv else name] = round(tot / n, 4)
        attend_only()
        torch.cuda.synchronize()
        c4 = cnt.cpu().numpy()
        s4 = sel.cpu().numpy()
        n1_4, _, c1_4 = Z.level_view(tree, T, Hq, 1, ws)
        union4 = sum(int(c1_4[u]) for u in range(U)) * b
        hits4 = 0
        for bb in range(B):
            for pos, t, h in W.needle_plan(spec, bb):
                hits4 += int(pos in set(s4[bb, t, h, :c4[bb, t, h]].tolist()))
        # share of each head's float32-router selection that the FP4 router also selects
        keep = []
        for bb in range(B):
            for t in range(T):
                for h in range(Hq):
                    a = sel_h[bb, t, h, :cnt_h[bb, t, h]]
                    z = s4[bb, t, h, :c4[bb, t, h]]
                    keep.append(np.intersect1d(a, z, assume_unique=True).size / max(a.size, 1))
        kr4 = c4.reshape(-1) / N
        fp4 = {"router_bytes": rbytes, "encode_pass_ms": round(ms4_quant, 4),
               "build_ms": round(ms4_build, 4),
               "step_ms": round(ms4_step, 4),
               "query_heads_per_s": round(QH / (ms4_step * 1e-3), 1),
               "attend_ms": round(ms4_attend, 4),
               "keys_read_pct": {"mean": round(100 * kr4.mean(), 3),
                                 "union": round(100 * union4 / (U * N), 3)},
               "needle_recall": round(hits4 / needles["planted"], 4) if needles["planted"] else None,
               "f32_selection_kept": {"mean": round(float(np.mean(keep)), 4),
                                      "min": round(float(np.min(keep)), 4)},
               "kernels_ms": k4}
        c_tree.router = LB.ZHA_ROUTER_F32

    # causal multi-query: 16 queries per sequence at positions (i + 1) N / 16 - 1, each
    # searching the tree over the tokens up to its position (tree prebuilt), against the
    # dense causal comparator on the same queries
    causal = None
    if not args.no_extras:
        Tc = 16
        Qc = torch.from_numpy(W.gen_Q(dict(spec, T=Tc))).to(dev).to(K.dtype)
        posn = ((np.arange(Tc) + 1) * (N // Tc) - 1).astype(np.int32)
        posc = torch.from_numpy(np.tile(posn, (B, 1))).to(dev)
        QHc = B * Tc * Hq
        Oc = torch.empty((B, Tc, Hq, d), dtype=torch.float32, device=dev)
        selc = torch.empty((B, Tc, Hq, N), dtype=torch.int32, device=dev)
        cntc = torch.empty((B, Tc, Hq), dtype=torch.int32, device=dev)
        wsc = torch.empty(Z.workspace_bytes(tree, Tc, Hq), dtype=torch.uint8, device=dev)
        Odc = torch.empty_like(Oc)
        dwsc = torch.empty(Z.dense_workspace_bytes(B, Hkv, N, N, d, Tc, Hq), dtype=torch.uint8,
                           device=dev)
        build_into()

        def attend_c():
            Z.attend(Qc, K, V, tree, p, anchor, out=Oc, sel_idx=selc, sel_count=cntc,
                     workspace=wsc, positions=posc)

        def dense_c():
            Z.dense_attend(Qc, K, V, N, out=Odc, workspace=dwsc, positions=posc)

        attend_c()
        dense_c()
        if args.no_graph:
            ms_c, _ = timed(attend_c, args.steps)
            ms_dc, _ = timed(dense_c, args.steps)
        else:
            ms_c, _ = timed(capture(attend_c).replay, args.steps)
            ms_dc, _ = timed(capture(dense_c).replay, args.steps)
        # per-kernel durations of the causal attend (eager launches with HIP events)
        lib.zha_timing_enable(1)
        timed(attend_c, max(1, args.steps // 4))
        lib.zha_timing_enable(0)
        kernels_c = {}
        for name, kind, levels in (("score", LB.ZHA_K_SCORE, range(1, L + 1)),
                                   ("select", LB.ZHA_K_SELECT, range(0, L + 1)),
                                   ("compact", LB.ZHA_K_COMPACT, range(1, L + 1)),
                                   ("descent_top", LB.ZHA_K_DESCENT, range(1, L + 1)),
                                   ("decode", LB.ZHA_K_DECODE, [0]),
                                   ("combine", LB.ZHA_K_COMBINE, [0])):
            for lv in levels:
                tot, n = ktime(kind, lv)
                if n:
                    key = f"{name}_l{lv}" if (lv or name == "select") else name
                    kernels_c[key.replace("select_l0", "tail")] = round(tot / n, 4)
        attend_c()
        torch.cuda.synchronize()
        cc = cntc.cpu().numpy().astype(np.float64)
        vis = (posn + 1).astype(np.float64)[None, :, None]
        causal = {"queries_per_sequence": Tc, "positions": "(i + 1) N / 16 - 1, i < 16",
                  "attend_ms": round(ms_c, 4),
                  "query_heads_per_s": round(QHc / (ms_c * 1e-3), 1),
                  "dense_causal_ms": round(ms_dc, 4),
                  "kernels_ms": kernels_c,
                  "speedup_of_attend": round(ms_dc / ms_c, 3),
                  "keys_read_pct_of_seen": round(100 * float(np.mean(cc / vis)), 3),
                  "keys_read_pct_of_cache": round(100 * float(np.mean(cc / N)), 3)}

    cpu = near_ties = None
    if not args.no_cpu_baseline:
        cpu, near_ties = cpu_baseline(spec, p, anchor, args.cpu_units)

    qhs = QH / (ms_step * 1e-3)
    out = {
        "metric": METRIC,
        "value": round(qhs, 1),
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "timing": "HIP graph replay of the captured step" if graph else "eager launches",
        "eager_ms_per_step": round(ms_eager, 4),
        "step_ms_spread": dist if dist is not None else per_step(full_step, args.steps),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "d": d,
                   "N": N, "b": b, "L": L, "p": p, "anchor": anchor,
                   "step": "zha_build_tree + zha_attend", "accumulate": "fp32",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "kernel_rooflines": kernel_rooflines,
        "cpu_baseline": cpu,
        "needles": needles,
        "near_ties": near_ties,
        "attend_roofline": {"what": "zha_attend (tree prebuilt): search + decode + combine",
                            "bound": "hbm", "achieved": round(attend_alg / (ms_attend * 1e-3) / 1e9, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(attend_alg / (ms_attend * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "alg_bytes": attend_alg, "ms": round(ms_attend, 4),
                            "flushed_ms": fl_attend["median"] if fl_attend else None,
                            "flushed_frac": round(attend_alg / (fl_attend["median"] * 1e-3) / 1e9
                                                  / HBM_PEAK_GBS, 4) if fl_attend else None},
        "flushed": {"what": "1 GiB written between repetitions, outside the timed region",
                    "step_ms": fl_step, "attend_ms": fl_attend,
                    "query_heads_per_s": round(QH / (fl_step["median"] * 1e-3), 1)
                    if fl_step else None},
        "decode_only": {"ms": round(ms_attend, 4), "eager_ms": round(ms_attend_eager, 4),
                        "query_heads_per_s": round(QH / (ms_attend * 1e-3), 1),
                        "alg_bytes": attend_alg,
                        "alg_gbs": round(attend_alg / (ms_attend * 1e-3) / 1e9, 1),
                        "hbm_frac": round(attend_alg / (ms_attend * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "dense": None if args.no_extras else {
            "ms": round(ms_dense, 4),
            "kv_gbs": round(B * Hkv * N * 2 * d * elem / (ms_dense * 1e-3) / 1e9, 1),
            "query_heads_per_s": round(QH / (ms_dense * 1e-3), 1),
            "speedup_of_attend": round(ms_dense / ms_attend, 3)},
        "build": {"oneshot_ms": round(ms_build, 4), "appends": n_app,
                  "appends_ms": None if args.no_extras else round(ms_appends, 4),
                  "one_token_appends": one_tok,
                  "oneshot_in_dense_decodes":
                      None if args.no_extras else round(ms_build / ms_dense, 3)},
        "step_alg_gbs": round(step_alg / (ms_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_alg / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "keys_read_pct": keys,
        "time_split_ms": {
            "build": round(sum(v["avg_ms"] for k, v in kernels.items() if k.startswith("pool")), 4),
            "index": round(sum(v["avg_ms"] for k, v in kernels.items()
                               if k.startswith(("score", "select", "compact", "descent"))), 4),
            "attend": round(sum(v["avg_ms"] for k, v in kernels.items()
                                if k in ("decode", "combine")), 4),
            "timed_pass_ms_per_step": round(ms_timed_pass, 4)},
        "kernels": {k: {"avg_ms": round(v["avg_ms"], 4), "launches": v["launches"]}
                    for k, v in kernels.items()},
        "fp4_router": fp4,
        "causal_multi_query": causal,
        "copy_probe_gbs": copy_gbs,
        "kernel_sources": kernel_sources_sha(),
    }
    print(json.dumps(out), flush=True)


SWEEP_ROUTERS = ("f32", "mxfp4")
SWEEP_GEOMETRIES = [(2, 12), (4, 6), (4, 8), (8, 4), (16, 3), (16, 4), (64, 2), (256, 1),
                    (1024, 1)]
SWEEP_P = [0.8, 0.9, 0.95, 0.99]


def sweep(args):
    """Selection quality over tree geometries on one workload's tensors (same keys, values,
    queries and reference queries for every geometry): per (b, L, p) the keys each query
    head reads, the union over a KV head's heads, the true attention mass of the selected
    set (from dense softmax weights over all N keys), needle recall, and the attend time.
    Prints one JSON line."""
    import numpy as np
    import torch

    import tree_indexed_sparse_amd as Z
    import workloads as W

    Z.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = W.spec(args.workload)
    B, T, Hq, Hkv, d, N = (spec[k] for k in ("B", "T", "Hq", "Hkv", "d", "N"))
    G = Hq // Hkv
    anchor = spec["anchor"]
    inp = W.gen_all(spec, device=dev)
    K, V, Q, R = inp["K"], inp["V"], inp["Q"], inp["R"]
    QH = B * T * Hq
    wts = dense_weights(Q, K)
    O = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev)
    sel = torch.empty((B, T, Hq, N), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, T, Hq), dtype=torch.int32, device=dev)
    plan = [(bb, pos, t, h) for bb in range(B) for pos, t, h in W.needle_plan(spec, bb)]
    rows = []
    for (b, L) in SWEEP_GEOMETRIES:
        if N % (b ** L) or N // b > (1 << 21):
            continue
        tree = Z.build_tree(K, R, b, L)
        Z.quantize_router(tree)  # the FP4 router's copy; the float32 router is tried first
        ws = torch.empty(Z.workspace_bytes(tree, T, Hq), dtype=torch.uint8, device=dev)
        for router, p in [(r, p) for r in SWEEP_ROUTERS for p in SWEEP_P]:
            Z.set_router(tree, router)

            def run():
                Z.attend(Q, K, V, tree, p, anchor, out=O, sel_idx=sel, sel_count=cnt,
                         workspace=ws)
            run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                run()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 5
            kept_mass = selected_mass(wts, sel, cnt).cpu().numpy()
            kr = (cnt.view(-1).float() / N).cpu().numpy()
            c1 = Z.level_view(tree, T, Hq, 1, ws)[2]
            sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
            hits = sum(int(pos in set(sel_h[bb, t, h, :cnt_h[bb, t, h]].tolist()))
                       for bb, pos, t, h in plan)
            rows.append({"b": b, "L": L, "p": p, "router": router, "top_node_tokens": b ** L,
                         "keys_read_pct": round(100 * float(kr.mean()), 2),
                         "keys_read_pct_min": round(100 * float(kr.min()), 2),
                         "keys_read_pct_max": round(100 * float(kr.max()), 2),
                         "union_pct": round(100 * float(c1.sum()) * b / (c1.size * N), 2),
                         "attention_mass_kept_mean": round(float(kept_mass.mean()), 4),
                         "attention_mass_kept_min": round(float(kept_mass.min()), 4),
                         "needle_recall": round(hits / len(plan), 4) if plan else None,
                         "attend_ms": round(ms, 4)})
            print(f"# b={b} L={L} p={p} {router}: {rows[-1]}", file=sys.stderr, flush=True)
        del tree, ws
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": args.workload, "query_heads": QH, "N": N, "rows": rows}),
          flush=True)


def dense_weights(Q, K):
    """Dense softmax attention weights (scale 1/sqrt(d), float32) of every query head over
    every key of its KV head: [B * T * Hq, N]. Measurement only (the sweep's retained-mass
    column)."""
    import torch

    B, T, Hq, d = Q.shape
    Hkv, N = K.shape[1], K.shape[2]
    G = Hq // Hkv
    wts = torch.empty((B, T, Hq, N), dtype=torch.float32, device=Q.device)
    for bb in range(B):
        for g in range(Hkv):
            q = Q[bb, :, g * G:(g + 1) * G, :].float().reshape(T * G, d)
            sc = (q @ K[bb, g].float().T) / (d ** 0.5)
            wts[bb, :, g * G:(g + 1) * G, :] = torch.softmax(sc, dim=-1).reshape(T, G, N)
    return wts.reshape(B * T * Hq, N)


def selected_mass(wts, sel, cnt):
    """Share of each query head's dense attention weight that falls on its selected keys
    (the first cnt entries of its list): [B * T * Hq]."""
    import torch

    QH, N = wts.shape
    c = cnt.reshape(QH, 1).long()
    idx = sel.reshape(QH, -1)[:, :N].long()
    valid = torch.arange(idx.shape[1], device=wts.device).view(1, -1) < c
    mask = torch.zeros((QH, N), dtype=torch.float32, device=wts.device)
    mask.scatter_add_(1, torch.where(valid, idx, torch.zeros_like(idx)), valid.float())
    return (wts * (mask > 0)).sum(-1)


def tree_bytes_written(B, Hkv, N, d, b, L):
    return sum(B * Hkv * (N // b ** lv) * d * 4 for lv in range(1, L + 1))


def copy_probe(torch, dev, reps=5, warm=2):
    """Device-to-device copy bandwidth (read + write bytes / time) of a 2 GiB buffer."""
    n = 1 << 29
    a = torch.empty(n, dtype=torch.float32, device=dev)
    c = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(warm):
        c.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, c
    return round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)


def pmc_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this kernel,
    if it was taken on the current kernel sources; otherwise None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_sources") != kernel_sources_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


CPU_WORKERS = 16   # host cores a one-GPU machine gives a run


def _oracle_worker(args):
    """One worker of the CPU baseline: regenerate its units' inputs, wait for every other
    worker, then run the oracle (one BLAS thread) on them, repeating the whole pass until a
    second has gone by (the small workloads take milliseconds). Returns (start, end, the
    fragility records of one pass, passes)."""
    spec, p, anchor, units, barrier = args
    import threadpoolctl

    import oracle as O
    import workloads as W

    G = spec["Hq"] // spec["Hkv"]
    Q = W.gen_Q(spec)
    R = W.gen_R(spec)
    data = [(u, W.gen_KV_unit(spec, u[0], u[1], Q)) for u in units]

    def one_pass():
        out = []
        for (bb, g), (K_u, V_u) in data:
            levels = O.build_tree_unit(K_u, R[g], spec["b"], spec["L"])
            for t in range(spec["T"]):
                for h in range(g * G, (g + 1) * G):
                    r = O.attend_head(Q[bb, t, h], levels, K_u, V_u, spec["b"], spec["L"], p,
                                      anchor)
                    out.append((len(r.levels), sum(1 for lv in r.levels if lv.fragile),
                                [(bb, t, h, lv.level, kind, float(f"{gap:.3g}"))
                                 for lv in r.levels for kind, gap in lv.fragile]))
        return out

    barrier.wait()
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        first = one_pass()
        passes = 1
        while time.perf_counter() - t0 < 1.0:
            one_pass()
            passes += 1
        t1 = time.perf_counter()
    return t0, t1, first, passes


def cpu_baseline(spec, p, anchor, n_units, workers=CPU_WORKERS):
    """The CPU oracle, as it stands, on a bounded sample: n_units (sequence, KV head) units
    of the same workload, each running the whole path (pyramid build, descent and exact
    attention for the unit's query heads). The units are spread over `workers` processes
    (one BLAS thread each; the oracle itself is unchanged); the rate is query heads over
    the wall time from the first worker's start to the last worker's end, after every
    worker has generated its inputs."""
    import multiprocessing as mp

    all_units = [(bb, g) for bb in range(spec["B"]) for g in range(spec["Hkv"])]
    units = all_units[:n_units] if n_units > 0 else all_units
    workers = max(1, min(workers, len(units)))
    ctx = mp.get_context("spawn")
    with ctx.Manager() as mgr:
        barrier = mgr.Barrier(workers)
        jobs = [(spec, p, anchor, units[i::workers], barrier) for i in range(workers)]
        with ctx.Pool(workers) as pool:
            res = pool.map(_oracle_worker, jobs)
    t0 = min(r[0] for r in res)
    t1 = max(r[1] for r in res)
    sec = t1 - t0
    heads = sum(len(r[2]) * r[3] for r in res)     # query heads attended, every pass
    passes = min(r[3] for r in res)
    decisions = sum(x[0] for r in res for x in r[2])
    fragile = sum(x[1] for r in res for x in r[2])
    log = [x[2] for r in res for x in r[2]]
    kinds = {}
    for head in log:
        for entry in head:
            kinds[entry[4]] = kinds.get(entry[4], 0) + 1
    ties = {"decisions": decisions, "fragile_decisions": fragile,
            "heads_with_any": sum(1 for head in log if head), "heads": len(log),
            "by_kind": kinds,
            "sample": "the oracle's own decisions on the cpu_baseline units",
            "log_fields": ["sequence", "t", "h", "level", "kind", "gap"],
            "log": sorted(e for head in log for e in head)}
    full = len(units) == len(all_units)
    return {"value": round(heads / sec, 3), "unit": "query-heads/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{len(units)} of {len(all_units)} (sequence, KV head) units"
                      f"{' (the whole batch)' if full else ''}"
                      f"{f', {passes}+ passes' if passes > 1 else ''} = {heads} query heads of "
                      f"{spec['name']}, full path per unit (pyramid build + descent + "
                      f"attention), {workers} processes with one BLAS thread each, "
                      f"{sec:.1f}s wall",
            "cpu": cpu_model()}, ties


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip() + f" x{os.cpu_count()}"
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
