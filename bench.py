#!/usr/bin/env python3
"""Benchmark of the row-wise RMSNorm hot path on one MI355X.

Prints ONE JSON line. Headline (`value`): achieved HBM bandwidth of the
batched-rows kernel on the prefill batch (8192 rows x 7168, bf16 in/out,
binary32 arithmetic), counted in algorithmic bytes (x read + y written per
row, w read once), with inputs resident in HBM and the 256 MB last-level
cache defeated by rotating over 4 buffer sets (940 MB). Its timed region
(the warm-up launches, then the timed ones) runs last, after the other
sections, once the GPU's clocks have settled; the same region run first,
right after the process starts, is reported beside it. Also reported:
* single_norm: latency of one binary32 1 x 7168 norm (Lecture 04 section 2);
* batch64: the bf16 64 x 7168 batch;
* decode_step: the 327-norm decode step, eager launches vs one captured
  graph replay (Lecture 08 section 1) vs one persistent launch walking the
  table, A/A controls then ABCCBA x 2 with per-rep numbers and standard
  errors (Lecture 04 section 6.1);
* decode_step_positioned: the same step walking a ring of rows through a
  device-resident position that the step itself advances (Lecture 08
  section 2), eager vs graph;
* dispatch_floor_us: a graph-captured one-element launch, the floor under the
  graph-timed figures; the single norm and the batch are also given above it;
* decode_step_nodes: per-node time of each descriptor kernel of the step;
* persistent_check: the persistent launch on tiny independent rows (its
  dispatch plus the walkers' overlap check);
* geometry_audit: every kernel of these workloads with grid, block,
  workgroups per CU, calls and time per step, its bandwidth floor and
  measured / floor, ranked by the time per step above the floor (Lecture 04,
  Lab);
* roofline: the prefill kernel against the 8 TB/s HBM peak;
* prefill.wave_path_us: the same launches on the one-wavefront-per-row layout;
* cpu_baseline: the CPU oracle timed on this host (a reported baseline only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps D]
       python bench.py --profile-kernels     (short run for rocprofv3 counters)
       python bench.py --profile-decode      (the same, decode step: eager + persistent)
       python bench.py --profile-persistent spread|one|chained|chained_offset   (one persistent arm)
       python bench.py --profile-copy        (prefill kernel beside the copy-pattern ceilings)
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E peak, 8 TB/s
METRIC = ("RMSNorm achieved HBM GB/s (% of peak) + µs per 327-norm decode step "
          "(graph vs eager)")
ROTATE = 4
# (16-byte vectors per lane, threads per workgroup) of the copy-pattern ceilings
COPY_PATTERNS = ((1, 64), (2, 448), (1, 1024))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_bf16_8192x7168_traffic.json")
# the sources the prefill kernel is compiled from (its traffic record is tied to them)
KERNEL_SRCS = [os.path.join(ROOT, "row_wise_rmsnorm_amd", "csrc", f)
               for f in ("rmsn_kernels.hip", "rmsn_rows.h", "rmsn_common.h", "rmsn_group.h",
                         "rmsn_launch.h")] + [
    os.path.join(ROOT, "row_wise_rmsnorm_amd", "build.py")]  # the compiler flags


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stats(xs):
    m = statistics.fmean(xs)
    sd = statistics.stdev(xs) if len(xs) > 1 else 0.0
    return {"mean": m, "sd": sd, "sem": sd / math.sqrt(len(xs)) if xs else 0.0,
            "reps": [round(v, 4) for v in xs]}


def elapsed_ms(fn, count):
    """Run fn(i) for i in range(count) back to back on the current stream and
    return the HIP-event time of the whole burst in ms."""
    import torch
    s = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(s)
    for i in range(count):
        fn(i)
    b.record(s)
    b.synchronize()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def source_digest():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, only
    while the kernel source is the one the counters were taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, None
    if t.get("kernel_source_sha256") != source_digest():
        return None, t
    return t.get("bytes_per_launch"), t


# ---------------------------------------------------------------------------

def bench_prefill(rn, torch, np, wl, steps, warmup):
    rows, n = wl.PREFILL_SHAPE
    log(f"prefill: generating {rows} x {n} bf16 inputs")
    xb, wb = wl.prefill()
    dev = torch.device("cuda", 0)
    x0 = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wb.view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [x0] + [x0.clone() for _ in range(ROTATE - 1)]
    ys = [torch.empty_like(x0) for _ in range(ROTATE)]
    algo_bytes = rows * n * 2 * 2 + n * 2
    eps = float(wl.EPS)
    plan = rn.plan_query(rn.BF16, rows, n, aligned=True)

    def step(i):
        k = i % ROTATE
        rn.rmsnorm_batched_rows(xs[k], w, eps, out=ys[k])

    def timed(steps_, warmup_):
        """`warmup_` untimed launches, then the timed region: `steps_`
        launches over the rotating buffer sets; µs per launch."""
        for i in range(warmup_):
            step(i)
        torch.cuda.synchronize()
        return 1000.0 * elapsed_ms(step, steps_) / steps_

    us = timed(steps, warmup)
    # per-rep spread over 30 further bursts of `steps` launches
    reps = []
    for _ in range(30):
        reps.append(1000.0 * elapsed_ms(step, steps) / steps)
    # warm arms: one buffer set, so the last-level cache may hold part of it;
    # with the automatic (streaming) plan and with default caching forced
    warm = 1000.0 * elapsed_ms(lambda i: rn.rmsnorm_batched_rows(xs[0], w, eps, out=ys[0]),
                               steps) / steps
    rn.set_option(rn.OPT_STREAMING, 0)
    try:
        warm_cached = 1000.0 * elapsed_ms(
            lambda i: rn.rmsnorm_batched_rows(xs[0], w, eps, out=ys[0]), steps) / steps
        rot_cached = 1000.0 * elapsed_ms(step, steps) / steps
    finally:
        rn.set_option(rn.OPT_STREAMING, -1)
    # the one-wavefront-per-row layout on the same rotated launches, for comparison
    rn.set_option(rn.OPT_PATH, rn.PATH_WAVE)
    try:
        wave_plan = rn.plan_query(rn.BF16, rows, n, aligned=True)
        wave_us = 1000.0 * elapsed_ms(step, steps) / steps
    finally:
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
    # a plain device copy of the same bytes (x read, y written), rotated the
    # same way: the practical bandwidth ceiling of this traffic pattern
    copy_us = 1000.0 * elapsed_ms(lambda i: ys[i % ROTATE].copy_(xs[i % ROTATE]), steps) / steps
    # the library's streaming copy of the same bytes in three granularities:
    # 1 KB per 64-thread workgroup (the fastest pattern measured), the
    # prefill kernel's own 14 KB per workgroup of 448 threads (two 16-byte
    # vectors per lane) and 16 KB per 1024-thread workgroup
    copy_patterns = {}
    for v, b in COPY_PATTERNS:
        fn = lambda i, v=v, b=b: rn.diag_copy(xs[i % ROTATE], ys[i % ROTATE], v, b)
        for i in range(20):
            fn(i)
        copy_patterns[f"{v}x16B_per_lane_{b}_threads"] = 1000.0 * elapsed_ms(fn, steps) / steps
    # the timed kernel (automatic plan) and the WAVE kernel, another layout,
    # give the same bytes (parity with the oracle is the tests' job); the copy
    # above overwrote the output buffers, so both run once more
    rn.rmsnorm_batched_rows(xs[0], w, eps, out=ys[0])
    try:
        rn.set_option(rn.OPT_PATH, rn.PATH_WAVE)
        rn.rmsnorm_batched_rows(xs[0], w, eps, out=ys[1])
    finally:
        rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
    torch.cuda.synchronize()
    parity = bool(torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16)))
    return {
        "us_per_launch": us, "algo_bytes": algo_bytes, "plan": plan,
        "gbs": algo_bytes / (us * 1e-6) / 1e9,
        "reps_us": stats(reps), "warm_us": warm,
        "warm_gbs": algo_bytes / (warm * 1e-6) / 1e9,
        "warm_cached_us": warm_cached, "rotated_cached_us": rot_cached,
        "copy_us": copy_us, "copy_gbs": (rows * n * 4) / (copy_us * 1e-6) / 1e9,
        "copy_patterns_us": copy_patterns,
        "wave_path_us": wave_us, "wave_path_plan": wave_plan,
        "rows_per_s": rows / (us * 1e-6), "bit_exact_vs_wave_layout": parity,
        "host": (xb, wb), "timed": timed,
    }


def bench_prefill_only(rn, torch, np, wl, steps, warmup):
    """Only the rotated, timed prefill launches (for kernel-trace and counter
    runs, so the profiler's average covers exactly the launches timed here)."""
    rows, n = wl.PREFILL_SHAPE
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    xs = [torch.randn(rows, n, device=dev, generator=g).to(torch.bfloat16) for _ in range(ROTATE)]
    w = (1.0 + 0.1 * torch.randn(n, device=dev, generator=g)).to(torch.bfloat16)
    ys = [torch.empty_like(xs[0]) for _ in range(ROTATE)]
    eps = float(wl.EPS)
    step = lambda i: rn.rmsnorm_batched_rows(xs[i % ROTATE], w, eps, out=ys[i % ROTATE])
    for i in range(warmup):
        step(i)
    us = 1000.0 * elapsed_ms(step, steps) / steps
    algo = rows * n * 4 + n * 2
    return {"prefill_only": True, "launches_timed": steps, "warmup_launches": warmup,
            "us_per_launch": us, "gbs": algo / (us * 1e-6) / 1e9,
            "plan": rn.plan_query(rn.BF16, rows, n)}


def graph_us_per_launch(torch, fn, per_graph=100, replays=20, reps=30):
    """Per-launch device time of `fn` (one launch on the given stream) with no
    host in the loop: `per_graph` launches captured in one graph, replayed
    `replays` times, HIP events around the replays; `reps` repetitions. Each
    launch still pays the graph's per-node dispatch cost."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(per_graph):
            fn(s)
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        out.append(1000.0 * elapsed_ms(lambda i: g.replay(), replays) / (per_graph * replays))
    del g
    return stats(out)


def bench_single(rn, torch, np, wl):
    x, w = wl.single()
    dev = torch.device("cuda", 0)
    xd, wd = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
    yd = torch.empty_like(xd)
    eps = float(wl.EPS)
    f = lambda i: rn.rmsnorm_f32(xd, wd, eps, out=yd)
    for i in range(50):
        f(i)
    dev_us = graph_us_per_launch(torch, lambda s: rn.rmsnorm_f32(xd, wd, eps, out=yd, stream=s))
    one = [1000.0 * elapsed_ms(f, 1) for _ in range(30)]          # host call -> completion
    burst = 1000.0 * elapsed_ms(f, 1000) / 1000                     # back-to-back host calls
    algo = 7168 * 4 * 3
    return {"us_per_norm_device": dev_us,
            "gbs_device": algo / (dev_us["mean"] * 1e-6) / 1e9,
            "us_isolated_host_call": stats(one), "us_back_to_back_host_calls": burst,
            "plan": rn.plan_query(rn.F32, 1, 7168),
            "note": ("us_per_norm_device: 100 launches captured in one graph, so no host work "
                     "between launches; the host-call figures include Python and launch overhead")}


def bench_batch64(rn, torch, np, wl):
    xb, wb = wl.batch64()
    dev = torch.device("cuda", 0)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wb.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty_like(x)
    eps = float(wl.EPS)
    f = lambda i: rn.rmsnorm_batched_rows(x, w, eps, out=y)
    for i in range(50):
        f(i)
    dev_us = graph_us_per_launch(torch, lambda s: rn.rmsnorm_batched_rows(x, w, eps, out=y, stream=s))
    host = [1000.0 * elapsed_ms(f, 200) / 200 for _ in range(3)]
    algo = 64 * 7168 * 4 + 7168 * 2
    plan = rn.plan_query(rn.BF16, 64, 7168)
    return {"us_device": dev_us, "gbs_device": algo / (dev_us["mean"] * 1e-6) / 1e9,
            "us_back_to_back_host_calls": stats(host), "plan": plan,
            "workgroups_per_cu": plan["grid"] / 256.0}


def bench_dispatch_floor(rn, torch):
    """What a graph-captured launch costs with (almost) no work: torch's fill
    of one element, and this library's norm of a one-element row (one
    256-thread workgroup: one load of x and w, the sum, the inverse, one
    store). The single norm and the 64-row batch are reported against it."""
    dev = torch.device("cuda", 0)
    one = torch.zeros(1, device=dev)
    x1 = torch.ones(1, device=dev)
    w1 = torch.ones(1, device=dev)
    y1 = torch.empty(1, device=dev)
    fill = graph_us_per_launch(torch, lambda s: one.fill_(1.0), reps=10)
    norm1 = graph_us_per_launch(
        torch, lambda s: rn.rmsnorm_f32(x1, w1, 1e-6, out=y1, stream=s), reps=10)
    return {"torch_fill_1_element_us": fill, "rmsnorm_1_element_us": norm1,
            "note": ("100 launches captured in one graph, replayed; each launch pays the graph's "
                     "per-node dispatch: the floor under every graph-timed figure here")}


def bench_decode_nodes(rn, torch, np, wl, reps=10, replays=200):
    """Per-node time of the decode step's descriptor kernels, one instance at a
    time: the step's rows of one width captured as their own graph (the same
    kernels, plans and rows as the step), replay time / rows. Each width also
    on the other descriptor layout (GROUP when the plan takes BLOCK), the two
    interleaved, outputs compared bit for bit."""
    rows = wl.decode()
    dev = torch.device("cuda", 0)
    eps = float(wl.EPS)
    out = {}
    for width in sorted({len(x) for x, _ in rows}, reverse=True):
        sel = [(x, w) for x, w in rows if len(x) == width]
        xs = [torch.from_numpy(x).to(dev) for x, _ in sel]
        ws = [torch.from_numpy(w).to(dev) for _, w in sel]
        ys = [torch.empty_like(t) for t in xs]
        table, widths = rn.make_table(list(zip(xs, ws, ys)))
        plan = rn.plan_query(rn.F32, 1, width, align=-1)
        other = rn.PATH_GROUP if plan["path"] != rn.PATH_GROUP else rn.PATH_BLOCK
        graphs = {"plan": rn.SequenceGraph(table, widths, eps, rn.F32)}
        rn.set_option(rn.OPT_PATH, other)
        try:
            graphs["other"] = rn.SequenceGraph(table, widths, eps, rn.F32)
            other_plan = rn.plan_query(rn.F32, 1, width, align=-1)
        finally:
            rn.set_option(rn.OPT_PATH, rn.PATH_AUTO)
        for g in graphs.values():
            if g.status != rn.RMSN_OK:
                raise RuntimeError(f"graph capture failed: {g.capture_error}")
            for _ in range(20):
                g.launch()
        bits = {}
        for k, g in graphs.items():
            g.launch()
            torch.cuda.synchronize()
            bits[k] = [t.cpu().numpy().view(np.uint32).copy() for t in ys]
        same = all(np.array_equal(a, b) for a, b in zip(bits["plan"], bits["other"]))
        per = {"plan": [], "other": []}
        for r in range(reps):
            for k in (("plan", "other") if r % 2 == 0 else ("other", "plan")):
                g = graphs[k]
                per[k].append(1000.0 * elapsed_ms(lambda i: g.launch(), replays)
                              / (replays * len(sel)))
        out[str(width)] = {"rows_per_step": len(sel), "us_per_node": stats(per["plan"]),
                           "plan": plan, "other_layout_us_per_node": stats(per["other"]),
                           "other_layout_plan": other_plan, "bit_exact_layouts": bool(same)}
        for g in graphs.values():
            g.destroy()
    return out


def bench_persistent_check(rn, torch, np, wl, decode_steps):
    """The persistent launch's own cost: 327 independent rows of 4 elements
    (their work is negligible, so the launch time is the dispatch plus the
    first workgroup's check of which rows may overlap), against one such row
    (no check: one workgroup)."""
    dev = torch.device("cuda", 0)
    eps = float(wl.EPS)

    def arm(count):
        xs = [torch.ones(4, device=dev) for _ in range(count)]
        ws = [torch.ones(4, device=dev) for _ in range(count)]
        ys = [torch.empty(4, device=dev) for _ in range(count)]
        table, _ = rn.make_table(list(zip(xs, ws, ys)))
        fn = lambda i: rn.rmsnorm_sequence_persistent(table, count, eps, rn.F32)
        for i in range(20):
            fn(i)
        return stats([1000.0 * elapsed_ms(fn, decode_steps) / decode_steps for _ in range(4)])

    return {"check_327_rows_us": arm(327), "one_row_us": arm(1),
            "note": ("327 independent 4-element rows spread over 256 workgroups: the first "
                     "workgroup checks every pair of rows (rank sort of the outputs, searches) "
                     "while the others run the rows; one row: a single workgroup, no check")}


def geometry_audit(single, b64, dec, nodes, pre, plan_prefill):
    """Every kernel of the four timed workloads (Lecture 04, Lab: grid, block,
    calls, time, the bandwidth floor, measured over floor), ranked by the time
    per step spent above the floor."""
    peak = PEAK_HBM_GBS * 1e3          # bytes per microsecond
    cu = 256
    rows = []

    def add(workload, kernel, grid, block, calls, mean, sd, nbytes):
        floor = nbytes / peak
        rows.append({"workload": workload, "kernel": kernel, "grid": grid, "block": block,
                     "workgroups_per_cu": round(grid / cu, 4), "calls_per_step": calls,
                     "us_per_call": round(mean, 3), "sd_us": round(sd, 3),
                     "us_per_step": round(calls * mean, 3), "bytes_per_call": nbytes,
                     "floor_us": round(floor, 4), "measured_over_floor": round(mean / floor, 1),
                     "above_floor_us_per_step": round(calls * (mean - floor), 3)})

    n = 7168
    add("prefill 8192x7168 bf16", "k_rows_split (SPLIT, 7 wavefronts, 2 slices each)",
        plan_prefill["grid"], plan_prefill["block"], 1, pre["us_per_launch"],
        pre["reps_us"]["sd"], 8192 * n * 4 + n * 2)
    s = single["us_per_norm_device"]
    add("single norm 1x7168 f32", "k_rows_group (GROUP, Q=7)", single["plan"]["grid"],
        single["plan"]["block"], 1, s["mean"], s["sd"], n * 12)
    b = b64["us_device"]
    add("batch 64x7168 bf16", "k_rows_group (GROUP, Q=7)", b64["plan"]["grid"],
        b64["plan"]["block"], 1, b["mean"], b["sd"], 64 * n * 4 + n * 2)
    for width, v in nodes.items():
        wd = int(width)
        add("decode step, graph", f"k_desc_block (BLOCK, {v['plan']['chunks']} chunks), width {wd}",
            1, 256, v["rows_per_step"], v["us_per_node"]["mean"], v["us_per_node"]["sd"], wd * 12)
    step_bytes = dec["algo_bytes_per_step"]
    gdev = dec["persistent_graph_captured_us_per_step"]
    for key, name, grid in (("spread", "spread over workgroups", 256),
                            ("one_workgroup", "one workgroup", 1),
                            ("chained_table", "chained table (every row bound, run walk)", 256),
                            ("chained_offset_table",
                             "chained table read 8 elements off (dependency walk)", 256)):
        add("decode step, persistent (graph-timed)", f"k_sequence_persistent, {name}", grid, 256,
            1, gdev[key]["mean"], gdev[key]["sd"], step_bytes)
    rows.sort(key=lambda r: -r["above_floor_us_per_step"])
    return rows


WIDE_SHAPES = [("f32", 1, 1 << 14), ("f32", 1, 1 << 16), ("f32", 1, 1 << 20), ("f32", 1, 1 << 24),
               ("bf16", 1, 1 << 24), ("bf16", 16, 1 << 18), ("bf16", 64, 1 << 16)]


def bench_wide(rn, torch, np, wl):
    """Few very wide rows (beyond the pages' widths): the plain entry point
    (STREAM or SPLIT) against the workspace entry point (WIDE), graph-timed,
    outputs compared bit for bit. Not part of the default run."""
    dev = torch.device("cuda", 0)
    eps = float(wl.EPS)
    out = []
    for kind, rows, n in WIDE_SHAPES:
        x = np.stack([wl.misc_f32(4_000_000 + r, n)[0] for r in range(rows)])
        w = wl.misc_f32(4_000_000, n)[1]
        if kind == "bf16":
            code, iv = rn.BF16, torch.int16
            xd = torch.from_numpy(wl.to_bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)
            wd = torch.from_numpy(wl.to_bf16_bits(w).view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            code, iv = rn.F32, torch.int32
            xd, wd = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
        y1, y2 = torch.empty_like(xd), torch.empty_like(xd)
        plan, need = rn.workspace_query(code, rows, n)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        big = rows * n >= (1 << 22)
        kw = dict(per_graph=10, replays=5, reps=5) if big else {}
        plain = graph_us_per_launch(
            torch, lambda s: rn.rmsnorm_batched_rows(xd, wd, eps, out=y1, stream=s), **kw)
        wide = graph_us_per_launch(
            torch, lambda s: rn.rmsnorm_batched_rows_ws(xd, wd, eps, out=y2, workspace=ws,
                                                        stream=s), **kw)
        torch.cuda.synchronize()
        out.append({"dtype": kind, "rows": rows, "n": n,
                    "plain_path": rn.plan_query(code, rows, n)["path"], "plain_us": plain["mean"],
                    "ws_path": plan["path"], "ws_us": wide["mean"],
                    "bit_exact_ws_eq_plain": bool(torch.equal(y1.view(iv), y2.view(iv)))})
        log(f"wide {kind} {rows} x {n}: plain {plain['mean']:.1f} us, with workspace "
            f"{wide['mean']:.1f} us")
        del xd, wd, y1, y2, ws
    return out


def profile_wide(rn, torch, np, wl):
    """A short run for a kernel trace of the wide-row paths: every shape of
    bench_wide, 3 + 20 launches through each entry point (no graph), so the
    trace can be grouped by shape (grid size)."""
    dev = torch.device("cuda", 0)
    eps = float(wl.EPS)
    for kind, rows, n in WIDE_SHAPES:
        dt = torch.bfloat16 if kind == "bf16" else torch.float32
        g = torch.Generator(device=dev)
        g.manual_seed(rows * 131 + n)
        x = torch.randn(rows, n, device=dev, generator=g).to(dt)
        w = (1 + 0.1 * torch.randn(n, device=dev, generator=g)).to(dt)
        y = torch.empty_like(x)
        _, need = rn.workspace_query(rn.BF16 if kind == "bf16" else rn.F32, rows, n)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        for _ in range(23):
            rn.rmsnorm_batched_rows(x, w, eps, out=y)
        for _ in range(23):
            rn.rmsnorm_batched_rows_ws(x, w, eps, out=y, workspace=ws)
        torch.cuda.synchronize()
        log(f"profile wide {kind} {rows} x {n}")


def bench_decode(rn, torch, np, wl, decode_steps):
    rows = wl.decode()
    dev = torch.device("cuda", 0)
    xs = [torch.from_numpy(x).to(dev) for x, _ in rows]
    ws = [torch.from_numpy(w).to(dev) for _, w in rows]
    ys = [torch.empty_like(t) for t in xs]
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    eps = float(wl.EPS)
    g = rn.SequenceGraph(table, widths, eps, rn.F32)
    if g.status != rn.RMSN_OK:
        raise RuntimeError(f"graph capture failed: {g.capture_error}")
    eager = lambda i: rn.rmsnorm_sequence_eager(table, widths, eps, rn.F32)
    graph = lambda i: g.launch()
    persistent = lambda i: rn.rmsnorm_sequence_persistent(table, len(widths), eps, rn.F32)
    for i in range(20):
        eager(i)
        graph(i)
        persistent(i)
    torch.cuda.synchronize()
    # correctness of the timed arms: graph and persistent outputs == the eager
    # launch sequence's (parity with the oracle is the tests' job)
    for t in ys:
        t.fill_(float("nan"))
    g.launch()
    torch.cuda.synchronize()
    gbits = [t.cpu().numpy().view(np.uint32).copy() for t in ys]
    eager(0)
    torch.cuda.synchronize()
    ok = all(np.array_equal(a, t.cpu().numpy().view(np.uint32)) for a, t in zip(gbits, ys))
    for t in ys:
        t.fill_(float("nan"))
    persistent(0)
    torch.cuda.synchronize()
    ok_p = all(np.array_equal(a, t.cpu().numpy().view(np.uint32)) for a, t in zip(gbits, ys))

    def rep(fn):
        return 1000.0 * elapsed_ms(fn, decode_steps) / decode_steps   # us per step

    # A/A, B/B and C/C controls, then ABCCBA x 2 (each arm 4 reps)
    order = ["A", "A", "B", "B", "C", "C"] + ["A", "B", "C", "C", "B", "A"] * 2
    arms = {"A": eager, "B": graph, "C": persistent}
    res = {"A": [], "B": [], "C": [], "sequence": []}
    for k, a in enumerate(order):
        v = rep(arms[a])
        res["sequence"].append((a, round(v, 2)))
        if k >= 6:
            res[a].append(v)
    aa = {"eager_pair_us": [round(v, 2) for a, v in res["sequence"][:2]],
          "graph_pair_us": [round(v, 2) for a, v in res["sequence"][2:4]],
          "persistent_pair_us": [round(v, 2) for a, v in res["sequence"][4:6]]}
    e, gr, pe = stats(res["A"]), stats(res["B"]), stats(res["C"])
    # The persistent launch decides from the table what may overlap: the
    # step's norms share no memory, so its rows spread over workgroups. The
    # same table in one workgroup, and a table of the same widths whose norm j
    # reads the output of the previous norm of its width (every row bound to
    # table order), show what that is worth.
    rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 1)
    try:
        one_wg = stats([rep(persistent) for _ in range(4)])
    finally:
        rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 0)
    last, cx, src = {}, [], []
    for j, n in enumerate(widths):
        src.append(last.get(n))
        cx.append(ys[last[n]] if n in last else xs[j])
        last[n] = j
    ctable, _ = rn.make_table(list(zip(cx, ws, ys)))
    chained = lambda i: rn.rmsnorm_sequence_persistent(ctable, len(widths), eps, rn.F32)
    for t in ys:
        t.fill_(float("nan"))
    rn.rmsnorm_sequence_eager(ctable, widths, eps, rn.F32)
    torch.cuda.synchronize()
    want = [t.cpu().numpy().view(np.uint32).copy() for t in ys]
    for t in ys:
        t.fill_(float("nan"))
    chained(0)
    torch.cuda.synchronize()
    ok_c = all(np.array_equal(a, t.cpu().numpy().view(np.uint32)) for a, t in zip(want, ys))
    chained_us = stats([rep(chained) for _ in range(4)])
    # the same chains with each x 8 elements past the output it reads: the
    # rows meet at other than the same addresses, so the dependency walk
    # orders them instead of the run walk
    otable = offset_chained_table(rn, torch, xs, ws, widths)
    for t in otable[1]:
        t.fill_(float("nan"))
    rn.rmsnorm_sequence_eager(otable[0], widths, eps, rn.F32)
    torch.cuda.synchronize()
    want_o = [t.cpu().numpy().view(np.uint32).copy() for t in otable[1]]
    for t in otable[1]:
        t.fill_(float("nan"))
    rn.rmsnorm_sequence_persistent(otable[0], len(widths), eps, rn.F32)
    torch.cuda.synchronize()
    ok_o = all(np.array_equal(a, t.cpu().numpy().view(np.uint32)) for a, t in zip(want_o, otable[1]))
    # the same three arms captured in a graph (no host in the loop): the
    # persistent kernel's own time on the device
    pers_s = lambda tbl: (lambda st: rn.rmsnorm_sequence_persistent(tbl, len(widths), eps, rn.F32,
                                                                    stream=st))
    dev_spread = graph_us_per_launch(torch, pers_s(table), per_graph=50, replays=10, reps=10)
    rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 1)
    try:
        dev_one = graph_us_per_launch(torch, pers_s(table), per_graph=10, replays=5, reps=5)
    finally:
        rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 0)
    dev_chained = graph_us_per_launch(torch, pers_s(ctable), per_graph=10, replays=5, reps=5)
    dev_offset = graph_us_per_launch(torch, pers_s(otable[0]), per_graph=10, replays=5, reps=5)
    timeouts = rn.diag_walk_timeouts(reset=True)
    algo = sum(n * 12 for n in widths)
    nodes = g.node_count()
    g.destroy()
    return {
        "eager_us_per_step": e, "graph_us_per_step": gr,
        "speedup_graph_over_eager": e["mean"] / gr["mean"],
        "persistent_us_per_step": pe,
        "speedup_persistent_over_graph": gr["mean"] / pe["mean"],
        "bit_exact_persistent_eq_graph": bool(ok_p),
        "persistent_one_workgroup_us_per_step": one_wg,
        "persistent_chained_table_us_per_step": chained_us,
        "persistent_graph_captured_us_per_step": {"spread": dev_spread, "one_workgroup": dev_one,
                                                  "chained_table": dev_chained,
                                                  "chained_offset_table": dev_offset},
        "persistent_walk_timeouts": timeouts,
        "bit_exact_chained_persistent_eq_eager": bool(ok_c),
        "bit_exact_chained_offset_persistent_eq_eager": bool(ok_o),
        "persistent_note": ("the step's norms share no memory, so the persistent launch runs them "
                            "on up to 256 workgroups; one_workgroup: the whole table walked by one "
                            "workgroup; chained_table: the same widths with norm j reading the "
                            "previous same-width norm's output, so every row keeps table order "
                            "(run walk: the rows meet at the same addresses); "
                            "chained_offset_table: the same chains read 8 elements past each "
                            "output (dependency walk); "
                            "the *_us_per_step figures are host calls timed back to back, the "
                            "graph_captured ones the same launches replayed from a graph "
                            "(device time, no host in the loop)"),
        "graph_us_per_norm": gr["mean"] / len(widths),
        "eager_us_per_norm": e["mean"] / len(widths),
        "norms_per_s_graph": len(widths) / (gr["mean"] * 1e-6),
        "graph_nodes": nodes, "norms": len(widths), "steps_per_rep": decode_steps,
        "aa_controls": aa, "rep_order": res["sequence"],
        "algo_bytes_per_step": algo, "bit_exact_graph_eq_eager": bool(ok),
    }


def bench_decode_positioned(rn, torch, np, wl, decode_steps, period=4):
    """The decode step as a positioned sequence: every norm owns a ring of
    `period` rows (one 7168-element slot each, shorter rows use its start),
    the descriptor table points at slot 0, and the step's last launch advances
    a device-resident position -- so consecutive replays normalise the next
    token's rows with no host work between them (Lecture 08 section 2)."""
    rows = wl.decode()
    dev = torch.device("cuda", 0)
    slot = 7168
    xs, ws, ys = [], [], []
    for i, (x, w) in enumerate(rows):
        n = len(x)
        ring = np.zeros((period, slot), np.float32)
        ring[0, :n] = x
        for p in range(1, period):
            ring[p, :n] = wl.misc_f32(600000 + period * i + p, n)[0]
        xs.append(torch.from_numpy(ring).to(dev))
        ws.append(torch.from_numpy(w).to(dev))
        ys.append(torch.full((period, slot), float("nan"), dtype=torch.float32, device=dev))
    n_of = [len(x) for x, _ in rows]
    table, widths = rn.make_table([(xs[i][0, :n_of[i]], ws[i], ys[i][0, :n_of[i]])
                                   for i in range(len(rows))])
    d_pos = torch.zeros(1, dtype=torch.int64, device=dev)
    pos = (d_pos, slot * 4, slot * 4, period)
    eps = float(wl.EPS)
    g = rn.SequenceGraph(table, widths, eps, rn.F32, position=pos)
    if g.status != rn.RMSN_OK:
        raise RuntimeError(f"positioned capture failed: {g.capture_error}")
    eager = lambda i: rn.rmsnorm_sequence_eager(table, widths, eps, rn.F32, position=pos)
    graph = lambda i: g.launch()
    # correctness: one full cycle of the ring on the graph, every norm and
    # position, equals a cycle of the eager positioned sequence
    d_pos.zero_()
    for y in ys:
        y.fill_(float("nan"))
    torch.cuda.synchronize()
    for _ in range(period):
        eager(0)
    torch.cuda.synchronize()
    ok = int(d_pos.item()) == 0          # the update wraps the position: a full cycle
    want = [y.cpu().numpy().view(np.uint32).copy() for y in ys]
    for y in ys:
        y.fill_(float("nan"))
    for _ in range(period):
        g.launch()
    torch.cuda.synchronize()
    ok = ok and int(d_pos.item()) == 0
    ok = ok and all(np.array_equal(a, y.cpu().numpy().view(np.uint32)) for a, y in zip(want, ys))
    # the same cycle as one persistent launch per step (its norms share no
    # memory: spread over workgroups, the position advanced by its own launch)
    pers = lambda i: rn.rmsnorm_sequence_persistent(table, len(widths), eps, rn.F32, position=pos)
    for y in ys:
        y.fill_(float("nan"))
    torch.cuda.synchronize()
    for _ in range(period):
        pers(0)
    torch.cuda.synchronize()
    ok_p = int(d_pos.item()) == 0
    ok_p = ok_p and all(np.array_equal(a, y.cpu().numpy().view(np.uint32)) for a, y in zip(want, ys))
    for i in range(20):
        eager(i)
        graph(i)
    # the same kernels and update node on a ring of one position: every step
    # re-reads the same rows, as the plain decode-step arms do
    pos1 = (d_pos, slot * 4, slot * 4, 1)
    g1 = rn.SequenceGraph(table, widths, eps, rn.F32, position=pos1)
    if g1.status != rn.RMSN_OK:
        raise RuntimeError(f"positioned capture failed: {g1.capture_error}")
    graph1 = lambda i: g1.launch()
    for i in range(20):
        eager(i)
        graph(i)
        graph1(i)
    for i in range(20):
        pers(i)
    res = {"A": [], "B": [], "C": [], "D": []}
    for a in ["A", "B", "C", "D", "D", "C", "B", "A"] * 2:
        fn = {"A": eager, "B": graph, "C": graph1, "D": pers}[a]
        res[a].append(1000.0 * elapsed_ms(fn, decode_steps) / decode_steps)
    rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 1)
    try:
        pers(0)
        one_wg = [1000.0 * elapsed_ms(pers, decode_steps) / decode_steps for _ in range(2)]
    finally:
        rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 0)
    nodes = g.node_count()
    g.destroy()
    g1.destroy()
    e, gr, g1s, ps = stats(res["A"]), stats(res["B"]), stats(res["C"]), stats(res["D"])
    return {"eager_us_per_step": e, "graph_us_per_step": gr,
            "graph_period1_us_per_step": g1s, "persistent_us_per_step": ps,
            "persistent_one_workgroup_us_per_step": stats(one_wg),
            "bit_exact_one_cycle_persistent_eq_eager": bool(ok_p),
            "speedup_graph_over_eager": e["mean"] / gr["mean"], "graph_nodes": nodes,
            "period": period, "bit_exact_one_cycle_graph_eq_eager": bool(ok),
            "note": ("327 norm nodes + 1 position-update node; each replay normalises the next "
                     "position's rows, no host work between replays; graph_period1: the same "
                     "graph on a ring of one position (same rows every step); persistent: one "
                     "launch per step spread over workgroups plus the position's update launch; "
                     "ABCDDCBA x 2")}


def cpu_baseline(np, wl, host):
    """The oracle as it stands, on this host's cores, over a bounded sample of
    the prefill workload; same algorithmic-byte accounting as the GPU."""
    import oracle
    xb, wb = host
    threads = min(os.cpu_count() or 1, 16)
    rows, n = xb.shape
    per_row = n * 4
    # multi-threaded: whole batch, repeated for ~6 s
    t0 = time.perf_counter()
    passes, used = 0, 1
    while True:
        _, used = oracle.rows(xb, wb, wl.EPS, nthreads=threads)
        passes += 1
        if time.perf_counter() - t0 > 6.0:
            break
    dt = time.perf_counter() - t0
    mt_gbs = (passes * rows * per_row + passes * n * 2) / dt / 1e9
    # single thread: 512 rows, repeated for ~4 s
    sub = xb[:512]
    t0 = time.perf_counter()
    p1 = 0
    while True:
        oracle.rows(sub, wb, wl.EPS, nthreads=1)
        p1 += 1
        if time.perf_counter() - t0 > 4.0:
            break
    dt1 = time.perf_counter() - t0
    st_gbs = (p1 * 512 * per_row + p1 * n * 2) / dt1 / 1e9
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": mt_gbs, "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": (f"prefill batch 8192x7168 bf16, {passes} full passes in {dt:.1f} s on "
                       f"{used} threads; single-thread figure from 512 rows x {p1} passes"),
            "single_thread_gbs": st_gbs, "cpu_model": cpu,
            "oracle_build": "gcc -O2 -ffp-contract=off -fno-fast-math"}


def profile_kernels(rn, torch, np, wl):
    """Short run for counter collection: 5 prefill launches, 5 launches each
    of the 64-row bf16 batch and of the single binary32 row, 5 of each of the
    first two copy patterns on the prefill's buffers, and 5 copies of a 1 GiB
    buffer (a plain copy of known size to scale the counters)."""
    rows, n = wl.PREFILL_SHAPE
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    x = torch.randn(rows, n, device=dev, generator=g).to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn(n, device=dev, generator=g)).to(torch.bfloat16)
    y = torch.empty_like(x)
    for _ in range(5):
        rn.rmsnorm_batched_rows(x, w, float(wl.EPS), out=y)
    xb, yb = x[:64].contiguous(), torch.empty(64, n, device=dev, dtype=torch.bfloat16)
    for _ in range(5):
        rn.rmsnorm_batched_rows(xb, w, float(wl.EPS), out=yb)
    x1 = torch.randn(n, device=dev, generator=g)
    w1 = 1.0 + 0.1 * torch.randn(n, device=dev, generator=g)
    y1 = torch.empty_like(x1)
    for _ in range(5):
        rn.rmsnorm_f32(x1, w1, float(wl.EPS), out=y1)
    for v, b in COPY_PATTERNS[:2]:
        for _ in range(5):
            rn.diag_copy(x, y, v, b)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_kernels": "done", "rmsnorm_launches": 15,
                      "copy_bytes_each": src.numel() * 4, "copies": 5}), flush=True)


def profile_decode(rn, torch, np, wl):
    """Short run for counter collection on the decode step: one eager step
    (327 launches) and three persistent launches of the same table."""
    rows = wl.decode()
    dev = torch.device("cuda", 0)
    xs = [torch.from_numpy(x).to(dev) for x, _ in rows]
    ws = [torch.from_numpy(w).to(dev) for _, w in rows]
    ys = [torch.empty_like(t) for t in xs]
    table, widths = rn.make_table(list(zip(xs, ws, ys)))
    rn.rmsnorm_sequence_eager(table, widths, float(wl.EPS), rn.F32)
    for _ in range(3):
        rn.rmsnorm_sequence_persistent(table, len(widths), float(wl.EPS), rn.F32)
    torch.cuda.synchronize()
    print(json.dumps({"profile_decode": "done", "eager_launches": len(widths),
                      "persistent_launches": 3}), flush=True)


def profile_copy(rn, torch, np, wl, launches=200):
    """A short run for a kernel trace of the prefill kernel beside the
    copy-pattern ceilings on the same rotated buffers: 300 warm-up launches,
    then `launches` of the prefill kernel and of each pattern of
    COPY_PATTERNS (told apart in the trace by their workgroup size)."""
    rows, n = wl.PREFILL_SHAPE
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    xs = [torch.randn(rows, n, device=dev, generator=g).to(torch.bfloat16) for _ in range(ROTATE)]
    w = (1.0 + 0.1 * torch.randn(n, device=dev, generator=g)).to(torch.bfloat16)
    ys = [torch.empty_like(xs[0]) for _ in range(ROTATE)]
    eps = float(wl.EPS)
    pre = lambda i: rn.rmsnorm_batched_rows(xs[i % ROTATE], w, eps, out=ys[i % ROTATE])
    for i in range(300):
        pre(i)
    out = {"prefill_us": 1000.0 * elapsed_ms(pre, launches) / launches}
    for v, b in COPY_PATTERNS:
        fn = lambda i, v=v, b=b: rn.diag_copy(xs[i % ROTATE], ys[i % ROTATE], v, b)
        for i in range(50):
            fn(i)
        out[f"copy_{v}x16B_{b}_threads_us"] = 1000.0 * elapsed_ms(fn, launches) / launches
    print(json.dumps({"profile_copy": out, "launches": launches}), flush=True)


COPY_SWEEP = tuple((v, b) for v in (1, 2, 4) for b in (64, 128, 256, 448, 512, 768, 1024))


def profile_copy_sweep(rn, torch, np, wl, launches=200):
    """The prefill kernel beside the library's streaming copy of the same
    bytes at every geometry of COPY_SWEEP (16-byte vectors per lane x threads
    per workgroup), on the same rotated buffers, HIP-event timed, two reps in
    opposite orders: how a plain copy's time depends on the vectors each lane
    holds before its first store and on the workgroup's size."""
    rows, n = wl.PREFILL_SHAPE
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    xs = [torch.randn(rows, n, device=dev, generator=g).to(torch.bfloat16) for _ in range(ROTATE)]
    w = (1.0 + 0.1 * torch.randn(n, device=dev, generator=g)).to(torch.bfloat16)
    ys = [torch.empty_like(xs[0]) for _ in range(ROTATE)]
    eps = float(wl.EPS)
    pre = lambda i: rn.rmsnorm_batched_rows(xs[i % ROTATE], w, eps, out=ys[i % ROTATE])
    for i in range(400):
        pre(i)
    res = {}
    for rep in range(2):
        res.setdefault("prefill", []).append(1000.0 * elapsed_ms(pre, launches) / launches)
        for v, b in (COPY_SWEEP if rep == 0 else COPY_SWEEP[::-1]):
            fn = lambda i, v=v, b=b: rn.diag_copy(xs[i % ROTATE], ys[i % ROTATE], v, b)
            for i in range(30):
                fn(i)
            res.setdefault(f"copy_{v}x16B_{b}_threads", []).append(
                1000.0 * elapsed_ms(fn, launches) / launches)
        log(f"copy sweep rep {rep} done")
    print(json.dumps({"profile_copy_sweep": {k: sum(v) / len(v) for k, v in res.items()},
                      "reps_us": res, "launches": launches}), flush=True)


def offset_chained_table(rn, torch, xs, ws, widths, shift=8):
    """The decode step's widths with norm j reading the output of the previous
    norm of its width `shift` elements on (outputs padded by `shift`): every
    row bound to table order, the rows meeting at other than the same
    addresses. Returns the table and the padded outputs' row views."""
    pads = [torch.empty(n + shift, dtype=torch.float32, device=xs[0].device) for n in widths]
    ys = [p[:n] for p, n in zip(pads, widths)]
    last, cx = {}, []
    for j, n in enumerate(widths):
        cx.append(pads[last[n]][shift:shift + n] if n in last else xs[j])
        last[n] = j
    table, _ = rn.make_table(list(zip(cx, ws, ys)))
    return table, ys, pads


def profile_persistent(rn, torch, np, wl, arm, launches=200):
    """A short run of one persistent arm of the decode step, so a kernel trace
    has one row per arm: 'spread' (the step's independent rows over up to 256
    workgroups), 'one' (the whole table in one workgroup), 'chained' (each norm
    reading the previous same-width norm's output: every row in table order,
    the run walk), 'chained_offset' (the same chains read 8 elements past each
    output: the dependency walk)."""
    rows = wl.decode()
    dev = torch.device("cuda", 0)
    xs = [torch.from_numpy(x).to(dev) for x, _ in rows]
    ws = [torch.from_numpy(w).to(dev) for _, w in rows]
    ys = [torch.empty_like(t) for t in xs]
    widths = [len(x) for x, _ in rows]
    if arm == "chained":
        last, cx = {}, []
        for j, n in enumerate(widths):
            cx.append(ys[last[n]] if n in last else xs[j])
            last[n] = j
        table, _ = rn.make_table(list(zip(cx, ws, ys)))
    elif arm == "chained_offset":
        table, ys, pads = offset_chained_table(rn, torch, xs, ws, widths)
    else:
        table, _ = rn.make_table(list(zip(xs, ws, ys)))
    rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 1 if arm == "one" else 0)
    try:
        for _ in range(launches):
            rn.rmsnorm_sequence_persistent(table, len(widths), float(wl.EPS), rn.F32)
        torch.cuda.synchronize()
    finally:
        rn.set_option(rn.OPT_PERSISTENT_WORKGROUPS, 0)
    print(json.dumps({"profile_persistent": arm, "launches": launches}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed prefill launches first (the first ~300 launches after a "
                         "cold start run slower while the clocks settle)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-kernels", action="store_true")
    ap.add_argument("--profile-decode", action="store_true",
                    help="short decode-step run for counter collection")
    ap.add_argument("--profile-wide", action="store_true",
                    help="a short run of the wide-row shapes for a kernel trace")
    ap.add_argument("--profile-copy-sweep", action="store_true",
                    help="prefill kernel beside the streaming copy at 21 geometries (HIP events)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="prefill kernel and copy-pattern ceilings on the same buffers (trace)")
    ap.add_argument("--profile-persistent", choices=["spread", "one", "chained", "chained_offset"],
                    help="200 launches of one persistent arm of the decode step (kernel trace)")
    ap.add_argument("--sections", default="prefill,single,batch64,decode",
                    help="comma list of prefill,single,batch64,decode,positioned,wide (for "
                         "profiling runs; the default runs the first four; wide: few very "
                         "wide rows, plain against workspace entry point)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only; --gpus {args.gpus} is not "
              "supported (rows shard across GPUs with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import row_wise_rmsnorm_amd as rn
    import workloads as wl

    torch.cuda.set_device(0)
    if args.profile_kernels:
        profile_kernels(rn, torch, np, wl)
        return
    if args.profile_decode:
        profile_decode(rn, torch, np, wl)
        return
    if args.profile_wide:
        profile_wide(rn, torch, np, wl)
        return
    if args.profile_copy:
        profile_copy(rn, torch, np, wl)
        return
    if args.profile_copy_sweep:
        profile_copy_sweep(rn, torch, np, wl)
        return
    if args.profile_persistent:
        profile_persistent(rn, torch, np, wl, args.profile_persistent)
        return

    sections = set(args.sections.split(","))
    full = {"prefill", "single", "batch64", "decode"}
    if "prefill" in sections and sections != full:
        # a profiling run of the prefill kernel alone: only the timed launches
        pre = bench_prefill_only(rn, torch, np, wl, args.steps, args.warmup)
        print(json.dumps(pre), flush=True)
        return
    if sections != full:
        out = {}
        if "single" in sections:
            out["single_norm"] = bench_single(rn, torch, np, wl)
        if "batch64" in sections:
            out["batch64"] = bench_batch64(rn, torch, np, wl)
        if "decode" in sections:
            out["decode_step"] = bench_decode(rn, torch, np, wl, args.decode_steps)
        if "positioned" in sections:
            out["decode_step_positioned"] = bench_decode_positioned(rn, torch, np, wl,
                                                                    args.decode_steps)
        if "wide" in sections:
            out["wide_rows"] = bench_wide(rn, torch, np, wl)
        print(json.dumps(out), flush=True)
        return
    torch.cuda.synchronize()
    t_start = time.time()
    pre = bench_prefill(rn, torch, np, wl, args.steps, args.warmup)
    log(f"prefill {pre['us_per_launch']:.2f} us  {pre['gbs']:.0f} GB/s "
        f"(copy of the same bytes {pre['copy_us']:.2f} us)")
    single = bench_single(rn, torch, np, wl)
    log(f"single {single['us_per_norm_device']['mean']:.2f} us per norm (graph-captured)")
    b64 = bench_batch64(rn, torch, np, wl)
    log(f"batch64 {b64['us_device']['mean']:.2f} us (graph-captured)")
    dec = bench_decode(rn, torch, np, wl, args.decode_steps)
    gd = dec["persistent_graph_captured_us_per_step"]
    log(f"persistent, graph-timed: spread {gd['spread']['mean']:.2f} us, one workgroup "
        f"{gd['one_workgroup']['mean']:.1f} us, chained {gd['chained_table']['mean']:.1f} us, "
        f"chained 8 elements off {gd['chained_offset_table']['mean']:.1f} us; "
        f"walk timeouts {dec['persistent_walk_timeouts']}")
    log(f"decode eager {dec['eager_us_per_step']['mean']:.1f} us  "
        f"graph {dec['graph_us_per_step']['mean']:.1f} us  "
        f"persistent {dec['persistent_us_per_step']['mean']:.1f} us (one workgroup "
        f"{dec['persistent_one_workgroup_us_per_step']['mean']:.1f}, chained table "
        f"{dec['persistent_chained_table_us_per_step']['mean']:.1f})")
    floor = bench_dispatch_floor(rn, torch)
    log(f"dispatch floor: torch fill {floor['torch_fill_1_element_us']['mean']:.2f} us, "
        f"1-element norm {floor['rmsnorm_1_element_us']['mean']:.2f} us (graph-captured)")
    nodes = bench_decode_nodes(rn, torch, np, wl)
    pcheck = bench_persistent_check(rn, torch, np, wl, args.decode_steps)
    log(f"persistent check: 327 tiny rows {pcheck['check_327_rows_us']['mean']:.2f} us, "
        f"one row {pcheck['one_row_us']['mean']:.2f} us")
    decp = bench_decode_positioned(rn, torch, np, wl, args.decode_steps)
    log(f"decode positioned eager {decp['eager_us_per_step']['mean']:.1f} us  "
        f"graph {decp['graph_us_per_step']['mean']:.1f} us  "
        f"persistent {decp['persistent_us_per_step']['mean']:.1f} us "
        f"(one workgroup {decp['persistent_one_workgroup_us_per_step']['mean']:.1f})")
    # The headline launches once more, now that the GPU has run the other
    # sections: right after the process starts, the first few hundred
    # launches run up to 20% slower while the clocks settle (the figure taken
    # then is reported beside it).
    at_start = pre["us_per_launch"]
    us = pre["timed"](args.steps, args.warmup)
    pre["us_per_launch"] = us
    pre["gbs"] = pre["algo_bytes"] / (us * 1e-6) / 1e9
    pre["rows_per_s"] = wl.PREFILL_SHAPE[0] / (us * 1e-6)
    log(f"prefill, timed again after the other sections: {us:.2f} us  {pre['gbs']:.0f} GB/s "
        f"(at the start of the run {at_start:.2f} us)")
    traffic, traffic_rec = measured_traffic()
    gpu_s = time.time() - t_start
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(np, wl, pre["host"])

    gbs = pre["gbs"]
    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["us_per_launch"] / 1000.0,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("prefill batch: 8192 rows x 7168, bf16 in/out, f32 arithmetic, "
                         "x~N(0,1) with 0.1% of entries +-100, w=1+0.1N(0,1), eps=1e-6; "
                         f"{ROTATE} rotated buffer sets (940 MB) defeat the 256 MB MALL"),
            "rows": 8192, "n": 7168, "io_dtype": "bf16",
            "plan": pre["plan"], "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": pre["algo_bytes"],
            "kernel_us_per_launch": round(pre["us_per_launch"], 3),
        },
        "cpu_baseline": cpu,
        "prefill": {
            "us_per_launch_at_start": round(at_start, 3),
            "timing_note": ("the timed region (warm-up, then the timed launches) runs after "
                            "the other sections; us_per_launch_at_start is the same timed "
                            "region run first, right after the process started, and us_reps "
                            "the 30 bursts that followed it"),
            "us_reps": pre["reps_us"], "warm_us": round(pre["warm_us"], 3),
            "warm_gbs": round(pre["warm_gbs"], 1), "rows_per_s": pre["rows_per_s"],
            "warm_cached_us": round(pre["warm_cached_us"], 3),
            "rotated_cached_us": round(pre["rotated_cached_us"], 3),
            "wave_path_us": round(pre["wave_path_us"], 3),
            "wave_path_gbs": round(pre["algo_bytes"] / (pre["wave_path_us"] * 1e-6) / 1e9, 1),
            "wave_path_plan": pre["wave_path_plan"],
            "copy_reference_us": round(pre["copy_us"], 3),
            "copy_patterns_us": {k: round(v, 3) for k, v in pre["copy_patterns_us"].items()},
            "copy_patterns_note": ("rmsnorm_diag_copy of the same bytes (x read, y written), "
                                   "rotated like the timed launches: the ceiling a pure copy of "
                                   "each granularity reaches; 2x16B_per_lane_448_threads moves "
                                   "one prefill row per workgroup"),
            "copy_reference_gbs": round(pre["copy_gbs"], 1),
            "fraction_of_copy": round(pre["copy_us"] / pre["us_per_launch"], 4),
            "bit_exact_vs_wave_layout": pre["bit_exact_vs_wave_layout"],
        },
        "single_norm": single,
        "batch64": b64,
        "dispatch_floor_us": round(floor["rmsnorm_1_element_us"]["mean"], 3),
        "dispatch_floor": floor,
        "single_norm_us_above_floor": round(single["us_per_norm_device"]["mean"]
                                            - floor["rmsnorm_1_element_us"]["mean"], 3),
        "batch64_us_above_floor": round(b64["us_device"]["mean"]
                                        - floor["rmsnorm_1_element_us"]["mean"], 3),
        "decode_step": dec,
        "decode_step_nodes": nodes,
        "persistent_check": pcheck,
        "geometry_audit": geometry_audit(single, b64, dec, nodes, pre, pre["plan"]),
        "decode_step_positioned": decp,
        "traffic_record": traffic_rec,
        "gpu_section_s": round(gpu_s, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
