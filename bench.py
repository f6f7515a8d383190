#!/usr/bin/env python3
"""Benchmark of the zero-copy MoE dispatch -> expert -> combine path.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3]

One step = the whole path on one batch: plan, dispatch, expert (SwiGLU
gate/up + down), combine.  Inputs are seeded synthetic tensors already
resident in HBM when the timed region starts.  Prints ONE JSON line:
whole-step throughput (tokens/s), per-kernel times from HIP events on the
launch stream, the roofline of the dominant kernel and the CPU oracle timed
on a bounded sample of the same workload.

The path runs on one GPU: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
# arithmetic intensity (flop per HBM byte) above which a kernel is bound by
# the matrix cores rather than by HBM
RIDGE_FLOP_PER_BYTE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
FLUSH_BYTES = 1 << 30       # per flush buffer: well above L2 (8 x 4 MiB) + MALL (256 MiB)


class CacheFlush:
    """Leaves L2 and MALL cold and clean before a timed launch: 1 GiB is
    written (evicting every line, the measured kernel's own included), then
    1 GiB of another buffer is read, so the written lines go back to HBM
    now and not during the measured kernel.  With the write alone, up to
    ~260 MB of dirty flush data drained while the next kernel ran and a
    plain 0.94 GB fill timed 1.3x slower."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.w = torch.empty(FLUSH_BYTES // 2, dtype=torch.bfloat16, device=dev)
        self.r = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.sink = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        self.w.fill_(1.0)
        self.torch.amax(self.r, dim=0, out=self.sink)


def stage_work(cfg, active_experts=None):
    """Algorithmic bytes / flops per launch of each kernel (what the method
    must move or compute; not what a kernel happens to re-read).  Expert
    weights count once per expert that received rows."""
    T, H, K, E, I = cfg.T, cfg.H, cfg.K, cfg.E, cfg.I
    EA = E if active_experts is None else int(active_experts)
    TK = T * K
    w = {
        # plan: read idx twice (count, rank), write pos + expert ids, counts/offsets
        "plan_count": dict(bytes=4 * TK + 12 * E),
        "plan_rank": dict(bytes=4 * TK + 8 * TK),
        # dispatch: read x once, write K rows + 12 B metadata, read idx/pos/w
        "dispatch": dict(bytes=2 * T * H + 2 * TK * H + 24 * TK),
        # combine: read K rows, write out, read w/idx/pos
        "combine": dict(bytes=2 * TK * H + 2 * T * H + 12 * TK),
    }
    if I > 0:
        # gate/up: X rows, gate+up weights of the active experts, h out
        w["expert_gate_up"] = dict(flops=4 * TK * H * I, bytes=2 * TK * H + 4 * EA * I * H + 2 * TK * I)
        # down: h rows, down weights, y out
        w["expert_down"] = dict(flops=2 * TK * H * I, bytes=2 * TK * I + 2 * EA * H * I + 2 * TK * H)
    return w


def fp8_step_variant(cfg, moe, idx, x8, sc, w, w13, w2, out, stream, flush, n_iter, steps,
                     ms_per_step, stages, work, torch):
    """The whole step on 8-bit tokens: plan, the 8-bit dispatch, the expert
    reading the 8-bit receive rows and their scales in place, combine.
    Timed like the bf16 step (wall clock over `steps` steps), then per
    kernel with HIP events, caches flushed before each step."""
    import numpy as np

    def step8():
        moe.plan(idx, stream)
        moe.dispatch_fp8(x8, sc, w, stream)
        moe.expert(w13, w2, stream)
        moe.combine(w, out=out, stream=stream)

    for _ in range(3):
        step8()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step8()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    per = {}
    moe.set_timing(True)
    for _ in range(n_iter):
        flush()
        step8()
        torch.cuda.synchronize()
        for k, (n, t) in moe.timing_summary().items():
            if n:
                per.setdefault(k, []).append(t / n)
    moe.set_timing(False)
    ns = sc.shape[1]
    TK = cfg.T * cfg.K
    gu = dict(work["expert_gate_up"])
    # the 8-bit rows: H codes and ns scales per row instead of 2H bytes
    gu["bytes"] += TK * (cfg.H + 4 * ns) - 2 * TK * cfg.H
    res = {"ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
           "vs_bf16_step_time": round(ms / ms_per_step, 4), "stages": {}}
    for k, times in per.items():
        avg = float(np.mean(times))
        st = {"avg_ms": round(avg, 5), "median_ms": round(float(np.median(times)), 5)}
        if k in stages:
            st["vs_bf16"] = round(avg / stages[k]["avg_ms"], 3)
        if k == "expert_gate_up":
            st["alg_bytes"] = gu["bytes"]
            st["GB_s"] = round(gu["bytes"] / (avg * 1e-3) / 1e9, 1)
            st["TFLOP_s"] = round(gu["flops"] / (avg * 1e-3) / 1e12, 2)
            st["mfma_frac"] = round(st["TFLOP_s"] / BF16_PEAK_TFLOPS, 4)
        res["stages"][k] = st
    return res


def code_digest(path):
    """sha256 of a C++/HIP source with its // comments, trailing blanks and
    empty lines removed: a change to the comments keeps the digest."""
    import hashlib
    import re
    lines = []
    for line in open(path).read().split("\n"):
        line = re.sub(r"//.*$", "", line).rstrip()
        if line:
            lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


EXPERT_SOURCES = ("expert.hip", "gemm_tile.h")


def expert_digest():
    """Digest of the expert GEMM's code (the kernel file and its tile)."""
    import hashlib
    csrc = os.path.join(ROOT, "combine_symmetric_memory_amd", "csrc")
    parts = [code_digest(os.path.join(csrc, f)) for f in EXPERT_SOURCES]
    return hashlib.sha256("".join(parts).encode()).hexdigest()


def profiled_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None if there is none for this workload or the expert kernel's
    code changed since the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", "traffic_%s.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"expert_code_sha256: ([0-9a-f]+)", text)
    if not m or m.group(1) != expert_digest():
        return None
    m = re.search(r"traffic_bytes_per_launch %s: (\d+)" % re.escape(kernel), text)
    return int(m.group(1)) if m else None


def cpu_baseline(cfg, x_np, idx_np, w_np, w13_host, sample_experts, counts, nthreads):
    """The oracle, untuned, timed on the host: plan, dispatch and combine on
    the full batch (each the median of 3 runs; the oracle runs them on one
    thread), the SwiGLU expert on every row of a stratified set of experts
    (the smallest, the median and the largest) with `nthreads` threads,
    extrapolated to all T * K rows by rows per second.  Returns tokens/s."""
    import numpy as np

    from oracle import oracle as orc

    def median3(fn):
        times, out = [], None
        for _ in range(3):
            out = None
            t0 = time.perf_counter()
            out = fn()
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), out

    E, S, cap = cfg.E, cfg.S, cfg.cap
    t_plan, pl = median3(lambda: orc.plan(idx_np, E, S, cap))
    t_disp, d = median3(lambda: orc.dispatch(x_np, w_np, idx_np, pl.pos, E, S, cap))
    # combine over the receive rows: the same rows, weights and arithmetic as
    # over expert outputs (identity experts read exactly these)
    t_comb, _ = median3(lambda: orc.combine_tokens(d.disp_x, w_np, idx_np, pl.pos, E, S))
    del d
    rows = 0
    t_exp = 0.0
    if cfg.I > 0:
        for e, (w13e, w2e) in zip(sample_experts, w13_host):
            n = int(counts[e])
            X = x_np[np.nonzero((idx_np == e).any(axis=1))[0][:n]]
            t0 = time.perf_counter()
            orc.swiglu_rows(X, w13e, w2e, nthreads)
            t_exp += time.perf_counter() - t0
            rows += X.shape[0]
    per_row = t_exp / rows if rows else 0.0
    TK = cfg.T * cfg.K
    step_s = t_plan + t_disp + t_comb + TK * per_row
    sample = ("full size, median of 3: plan, dispatch and combine of all %d tokens (%d pairs), "
              "one thread each; SwiGLU expert on every row of the smallest, median and largest "
              "experts %s (%d rows) with %d threads, extrapolated to all %d rows" %
              (cfg.T, TK, list(sample_experts), rows, nthreads, TK))
    return {"value": round(cfg.T / step_s, 3), "unit": "tokens/s", "cores": int(nthreads),
            "kind": "oracle", "sample": sample,
            "stage_s": {"plan": round(t_plan, 4), "dispatch": round(t_disp, 4),
                        "combine": round(t_comb, 4), "expert_per_row": per_row,
                        "expert_extrapolated": round(TK * per_row, 3)}}


def calibrate(cfg, moe, w, out, work, stream, dev, torch, per_expert=None):
    """Reference rates on the same GPU, each timed with L2 and MALL flushed:
    a device-to-device copy of the dispatch's byte count, torch kernels with
    the byte mixes of dispatch and combine, a large bf16 GEMM through the
    vendor library (torch.matmul, hipBLASLt) and one vendor GEMM per expert,
    and combine fed a foreign expert output (the copy fallback) against the
    zero-copy view."""
    flush = CacheFlush(torch, dev)

    def time_ms(fn, n=5):
        fn()
        times = []
        for _ in range(n):
            flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)[len(times) // 2]

    cal = {}
    nb = work["dispatch"]["bytes"] // 2 * 2
    a = torch.empty(nb // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    ms = time_ms(lambda: b.copy_(a))
    cal["d2d_copy"] = {"bytes_moved": 2 * nb, "GB_s": round(2 * nb / (ms * 1e-3) / 1e9, 1)}
    del a, b
    # the byte mixes of dispatch and combine through torch's own kernels:
    # every token row written K times (a broadcast copy into [K, T, H]), and
    # the K rows of every token summed (a reduction over [T, K, H])
    T, H, K = cfg.T, cfg.H, cfg.K
    xa = torch.empty((T, H), dtype=torch.bfloat16, device=dev).fill_(1.0)
    rep = torch.empty((K, T, H), dtype=torch.bfloat16, device=dev)
    ms = time_ms(lambda: rep.copy_(xa.unsqueeze(0).expand(K, T, H)))
    mixed = 2 * T * H * (1 + K)
    cal["library_broadcast_x%d" % K] = {"bytes_moved": mixed,
                                        "GB_s": round(mixed / (ms * 1e-3) / 1e9, 1)}
    red = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    rows = rep.view(T, K, H)
    ms = time_ms(lambda: torch.sum(rows, dim=1, out=red))
    cal["library_sum_of_%d_rows" % K] = {"bytes_moved": mixed,
                                         "GB_s": round(mixed / (ms * 1e-3) / 1e9, 1)}
    del xa, rep, red, rows
    if cfg.I > 0:
        # all of the step's rows through one expert's gate+up weights
        M, N, K = cfg.T * cfg.K, 2 * cfg.I, cfg.H
        x = torch.randn(M, K, device=dev).to(torch.bfloat16)
        wt = torch.randn(K, N, device=dev).to(torch.bfloat16)   # contiguous [K, N]
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        ms = time_ms(lambda: torch.matmul(x, wt, out=y))
        cal["library_gemm"] = {"shape_MNK": [M, N, K],
                               "TFLOP_s": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        del x, wt, y
    if per_expert is not None:
        # the gate/up projection as one vendor GEMM per expert, on the same
        # rows (gathered beforehand) and weights: the straightforward
        # alternative to the grouped kernel
        xs, w13 = per_expert
        ys = [torch.empty((xe.shape[0], 2 * cfg.I), dtype=torch.bfloat16, device=dev)
              for _, xe in xs]

        def loop():
            for (e, xe), ye in zip(xs, ys):
                torch.matmul(xe, w13[e].t(), out=ye)
        ms = time_ms(loop, n=3)
        fl = sum(2.0 * xe.shape[0] * 2 * cfg.I * cfg.H for _, xe in xs)
        cal["library_gemm_per_expert_gate_up"] = {"experts": len(xs), "ms": round(ms, 4),
                                                  "TFLOP_s": round(fl / (ms * 1e-3) / 1e12, 1)}
        del ys
    # combine through the copy fallback: the expert output handed over in
    # buffers of its own (one per slot) instead of the staging views
    foreign = [torch.empty((moe.cap, cfg.H), dtype=torch.bfloat16, device=dev)
               for _ in range(cfg.S)]
    ms_view = time_ms(lambda: moe.combine(w, out=out, stream=stream))
    ms_copy = time_ms(lambda: moe.combine(w, out=out, expert_out=foreign, stream=stream))
    cal["combine_copy_fallback"] = {"view_ms": round(ms_view, 4), "foreign_ms": round(ms_copy, 4),
                                    "extra_ms": round(ms_copy - ms_view, 4)}
    del foreign, flush
    return cal


def stage_in_variant(cfg, moe, slot_total, stream, dev, torch):
    """The expert output of every slot handed over in buffers of the
    caller's and staged into the combine windows on the copy engines
    (cco_moe_stage_in_sdma, no kernel), against the same bytes moved by a
    copy kernel on the compute units (torch's device-to-device copy; the
    library's own copy fallback runs at about the same rate); then each beside
    a large vendor GEMM on another stream, to show what the copy takes from
    the compute units."""
    import numpy as np
    flush = CacheFlush(torch, dev)
    rows = [int(r) for r in slot_total]
    foreign = [torch.zeros((max(r, 1), cfg.H), dtype=torch.bfloat16, device=dev) for r in rows]
    moved = 2 * 2 * cfg.H * sum(rows)  # read + write

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def sdma(st):
        for s in range(cfg.S):
            moe.stage_in_sdma(s, foreign[s], rows[s], stream=st)

    # a copy kernel on the compute units, on the same bytes
    dst = [torch.empty_like(f) for f in foreign]

    def cu_copy(st):
        with torch.cuda.stream(st):
            for d, f in zip(dst, foreign):
                d.copy_(f)

    def alone(fn, n=5):
        fn(stream)
        ts = []
        for _ in range(n):
            flush()
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn(stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    res = {"bytes_moved": moved}
    ms = alone(sdma)
    res["sdma_ms"] = round(ms, 4)
    res["sdma_GB_s"] = round(moved / (ms * 1e-3) / 1e9, 1)
    ms = alone(cu_copy)
    res["copy_kernel_ms"] = round(ms, 4)
    res["copy_kernel_GB_s"] = round(moved / (ms * 1e-3) / 1e9, 1)
    # beside a GEMM on the compute units: the copies go on a second stream
    M, N, K = 32768, 4096, 7168
    a = torch.randn(M, K, device=dev).to(torch.bfloat16)
    b = torch.randn(K, N, device=dev).to(torch.bfloat16)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream(device=dev)

    def gemm():
        torch.matmul(a, b, out=c)

    def beside(copy):
        flush()
        torch.cuda.synchronize()
        g0, g1, c1 = ev(), ev(), ev()
        g0.record(stream)
        side.wait_event(g0)
        if copy is not None:
            copy(side)
        gemm()
        g1.record(stream)
        c1.record(side)
        torch.cuda.synchronize()
        return g0.elapsed_time(g1), max(g0.elapsed_time(g1), g0.elapsed_time(c1))

    # the three cases interleaved, so that clock and cache state drift alike
    for _ in range(3):
        gemm()
    runs = {None: [], sdma: [], cu_copy: []}
    for _ in range(7):
        for k in runs:
            runs[k].append(beside(k))

    def med(k, i):
        return float(np.median([r[i] for r in runs[k]]))
    g_alone = med(None, 0)
    g_sdma, t_sdma = med(sdma, 0), med(sdma, 1)
    g_cu, t_cu = med(cu_copy, 0), med(cu_copy, 1)
    res["gemm_shape_MNK"] = [M, N, K]
    res["gemm_alone_ms"] = round(g_alone, 4)
    res["gemm_beside_sdma_ms"] = round(g_sdma, 4)
    res["gemm_beside_copy_kernel_ms"] = round(g_cu, 4)
    res["both_done_sdma_ms"] = round(t_sdma, 4)
    res["both_done_copy_kernel_ms"] = round(t_cu, 4)
    torch.cuda.synchronize()
    del foreign, dst, a, b, c, flush
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's batch size T (routing drawn for T tokens)")
    ap.add_argument("--inter", type=int, default=None,
                    help="override the workload's SwiGLU width I (0: identity experts)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed steps, run one plain elementwise copy of 1 GiB "
                         "(reference kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the path runs on one GPU (its share of the work); "
              "--gpus %d is not supported (use --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import combine_symmetric_memory_amd as ccm
    from synth import get_config
    from synth.gen import activations, bf16_bits, expert_weights, routing

    def log(*a):
        print("[bench]", *a, file=sys.stderr, flush=True)

    over = {}
    if args.tokens is not None:
        over["T"] = args.tokens
    if args.inter is not None:
        over["I"] = args.inter
    cfg = get_config(args.workload, **over)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log("workload", cfg)
    xt = activations(cfg)
    idx_np, w_np = routing(cfg)
    x = xt.to(dev)
    idx = torch.from_numpy(idx_np).to(dev)
    w = torch.from_numpy(w_np).to(dev)
    w13, w2 = expert_weights(cfg, dev)
    need = ccm.required_slot_bytes(cfg.T, cfg.H, cfg.K, cfg.E, cfg.I, cfg.S)
    heap = ccm.SymHeap(cfg.S, need, device=0)
    moe = ccm.MoE(heap, cfg.T, cfg.H, cfg.K, cfg.E, cfg.I)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    log("heap %.2f GiB, weights %.2f GiB" % (heap.stride * cfg.S / 2**30,
        0 if w13 is None else (w13.numel() + w2.numel()) * 2 / 2**30))

    def step():
        moe.plan(idx, stream)
        moe.dispatch(x, w, stream)
        moe.expert(w13, w2, stream)
        moe.combine(w, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    code, slot_total, counts = moe.status()
    if code != ccm.CCO_OK:
        raise SystemExit("device status %s" % ccm.status_string(code))
    log("warmup done")

    # ---- timed region: exactly `steps` steps ----
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = 1e3 * wall / args.steps
    value = cfg.T * args.steps / wall
    log("timed %d steps: %.3f ms/step (events %.3f ms/step)" % (args.steps, ms_per_step,
                                                                  gpu_ms / args.steps))

    # ---- per-kernel durations: HIP events on the launch stream, one step per
    # iteration, L2 and MALL left cold and clean before each ----
    flush = CacheFlush(torch, dev)
    n_iter = max(20, min(args.steps, 50))
    per = {}
    moe.set_timing(True)
    for _ in range(n_iter):
        flush()
        step()
        torch.cuda.synchronize()
        for k, (n, ms) in moe.timing_summary().items():
            if n:
                per.setdefault(k, []).append(ms / n)
    moe.set_timing(False)
    work = stage_work(cfg, active_experts=int(np.count_nonzero(counts)))
    if "plan_count" in per and "plan_rank" not in per:
        # a batch of one plan chunk runs the whole plan in one launch
        per["plan"] = per.pop("plan_count")
        work["plan"] = dict(bytes=work["plan_count"]["bytes"] + work["plan_rank"]["bytes"])
    stages = {}
    for k, times in per.items():
        t = np.asarray(times)
        avg = float(t.mean())
        st = {"launches": len(times), "avg_ms": round(avg, 5),
              "median_ms": round(float(np.median(t)), 5),
              "p10_ms": round(float(np.percentile(t, 10)), 5),
              "p90_ms": round(float(np.percentile(t, 90)), 5)}
        wk = work.get(k, {})
        if "bytes" in wk:
            st["alg_bytes"] = wk["bytes"]
            st["GB_s"] = round(wk["bytes"] / (avg * 1e-3) / 1e9, 1)
            st["hbm_frac"] = round(st["GB_s"] / HBM_PEAK_GBS, 4)
        if "flops" in wk:
            st["alg_flops"] = wk["flops"]
            st["TFLOP_s"] = round(wk["flops"] / (avg * 1e-3) / 1e12, 2)
            st["mfma_frac"] = round(st["TFLOP_s"] / BF16_PEAK_TFLOPS, 4)
            st["flop_per_byte"] = round(wk["flops"] / wk["bytes"], 1)
        stages[k] = st
    log("stages", json.dumps(stages))

    # ---- the 8-bit dispatch (tokens quantized by the caller to OCP e4m3 in
    # 1 x 128 blocks, fp32 scales) on the same routing, timed the same way;
    # outside the step, which stays bf16 ----
    variants = {}
    if cfg.H % 128 == 0:
        from synth.gen import quantized_activations
        x8_np, sc_np = quantized_activations(cfg, block=128)
        x8 = torch.from_numpy(x8_np).to(dev)
        sc = torch.from_numpy(sc_np).to(dev)
        ns = sc.shape[1]
        del x8_np, sc_np
        moe.plan(idx, stream)
        moe.dispatch_fp8(x8, sc, w, stream)
        times = []
        moe.set_timing(True)
        for _ in range(n_iter):
            flush()
            moe.dispatch_fp8(x8, sc, w, stream)
            torch.cuda.synchronize()
            n, ms = moe.timing_summary()["dispatch_fp8"]
            times.append(ms / n)
        moe.set_timing(False)
        t = np.asarray(times)
        TK = cfg.T * cfg.K
        nbytes = cfg.T * cfg.H + TK * cfg.H + 4 * ns * (cfg.T + TK) + 24 * TK
        avg = float(t.mean())
        variants["dispatch_fp8"] = {
            "scales_per_token": ns, "launches": len(times), "avg_ms": round(avg, 5),
            "median_ms": round(float(np.median(t)), 5), "alg_bytes": nbytes,
            "GB_s": round(nbytes / (avg * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "vs_bf16_dispatch_time": round(avg / stages["dispatch"]["avg_ms"], 3)}
        if cfg.I > 0:
            variants["step_fp8"] = fp8_step_variant(cfg, moe, idx, x8, sc, w, w13, w2, out,
                                                    stream, flush, n_iter, args.steps,
                                                    ms_per_step, stages, work, torch)
        # the bf16 rows back in the receive window for what follows
        moe.dispatch(x, w, stream)
        torch.cuda.synchronize()
        del x8, sc
        log("variants", json.dumps(variants))

    if cfg.I > 0:
        variants["stage_in_sdma"] = stage_in_variant(cfg, moe, slot_total, stream, dev, torch)
        log("variants", json.dumps({"stage_in_sdma": variants["stage_in_sdma"]}))
        # the staging windows back to the step's own expert output
        moe.expert(w13, w2, stream)
        torch.cuda.synchronize()

    # roofline of the dominant kernel (the longest one), bound by HBM or by
    # the matrix cores according to its arithmetic intensity
    dom = max(stages, key=lambda k: stages[k]["avg_ms"])
    d = stages[dom]
    hbm = {"achieved": d["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": d["hbm_frac"]}
    if "alg_flops" in d:
        mfma = {"achieved": d["TFLOP_s"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": d["mfma_frac"]}
        if d["flop_per_byte"] < RIDGE_FLOP_PER_BYTE:
            roofline = dict(kernel=dom, bound="hbm", **hbm, mfma_view=mfma)
        else:
            roofline = dict(kernel=dom, bound="mfma", **mfma, hbm_view=hbm)
        roofline["flop_per_byte"] = d["flop_per_byte"]
        roofline["ridge_flop_per_byte"] = round(RIDGE_FLOP_PER_BYTE, 1)
    else:
        roofline = dict(kernel=dom, bound="hbm", **hbm)
    # the profiled counters belong to the workload as configured
    roofline["traffic"] = None if over else profiled_traffic(cfg.name, dom)

    # ---- calibrations: context for the stage rates, outside the step ----
    per_expert = None
    if cfg.I > 0:
        # each expert's rows, in its receive order, as a contiguous tensor
        order = np.argsort(idx_np.ravel(), kind="stable")
        eid = idx_np.ravel()[order]
        xs = []
        start = 0
        for e in range(cfg.E):
            n = int(counts[e])
            if n:
                rows = torch.from_numpy((order[start:start + n] // cfg.K).astype(np.int64)).to(dev)
                xs.append((e, x.index_select(0, rows)))
            start += n
        assert start == len(eid)
        per_expert = (xs, w13)
    del flush
    calibration = calibrate(cfg, moe, w, out, work, stream, dev, torch, per_expert)
    del per_expert
    log("calibration", json.dumps(calibration))

    dc_bytes = stages["dispatch"]["alg_bytes"] + stages["combine"]["alg_bytes"]
    dc_ms = stages["dispatch"]["avg_ms"] + stages["combine"]["avg_ms"]
    summary = {"dispatch_combine_GB_s": round(dc_bytes / (dc_ms * 1e-3) / 1e9, 1),
               "dispatch_combine_hbm_frac": round(dc_bytes / (dc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if cfg.I > 0:
        fl = work["expert_gate_up"]["flops"] + work["expert_down"]["flops"]
        ex_ms = stages["expert_gate_up"]["avg_ms"] + stages["expert_down"]["avg_ms"]
        summary["expert_TFLOP_s"] = round(fl / (ex_ms * 1e-3) / 1e12, 2)
        summary["expert_mfma_frac"] = round(summary["expert_TFLOP_s"] / BF16_PEAK_TFLOPS, 4)

    if args.calib_copy:
        a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        sample_experts = []
        w13_host = []
        if cfg.I > 0:
            nz = np.nonzero(counts)[0]
            order = nz[np.argsort(counts[nz], kind="stable")]
            # stratified: the smallest, the median and the largest expert
            sample_experts = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
            w13_host = [(bf16_bits(w13[e]), bf16_bits(w2[e])) for e in sample_experts]
        from oracle import oracle as orc
        nthreads = orc.default_threads()
        cpu = cpu_baseline(cfg, bf16_bits(xt), idx_np, w_np, w13_host, sample_experts, counts,
                           nthreads)
        log("cpu baseline", json.dumps(cpu))

    res = {
        "metric": "dispatch+combine HBM GB/s (% peak); expert GEMM TFLOP/s; tokens/sec",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: T=%d H=%d top-%d E=%d over %d slots, SwiGLU I=%d" %
                   (cfg.name, cfg.T, cfg.H, cfg.K, cfg.E, cfg.S, cfg.I),
                   "T": cfg.T, "H": cfg.H, "K": cfg.K, "E": cfg.E, "S": cfg.S, "I": cfg.I,
                   "seed": cfg.seed},
        "summary": summary,
        "stages": stages,
        "roofline": roofline,
        "variants": variants,
        "calibration": calibration,
        "cpu_baseline": cpu,
    }
    heap.destroy()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
