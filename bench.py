#!/usr/bin/env python3
"""Throughput of the layer-by-layer weight-streamed DiT forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large]

A step is one streamed forward over every block of the workload (H2D of all
dp shards of every block, on-GPU reconstruction into one of two slots, and
the DiT block from the other slot), for one batch of synthetic input whose
weights already sit in pinned host memory and whose activations already sit
in HBM; for the irregular workload a step is its four sequential requests
(four forwards with their drawn token counts).  W untimed steps, then K timed
steps between two device syncs.

The default workload is the largest one: 80 blocks of d 8192 (about 131 GB of
bf16 weights, held only in pinned host memory).  Its weights are drawn block by
block and handed to the library, which copies them into its pinned shards, so
host memory holds the model once.  One pinned shard store serves every pass:
the timed forwards, an untraced pass, a fully traced pass over two
consecutive forwards and a serialized pass (dlo_set_flags between them).

Prints ONE JSON line: blocks/s as ``value`` plus tokens/s, H2D GB/s, GEMM
MFMA utilisation, overlap, per-step overheads, device weight residency, a
roofline of the dominant kernel (timed with HIP events on the compute stream
around that kernel only, inside the timed region; the warm-up, traced in
full, names it, and per-kernel statistics come from a fully traced pass after
the timed steps) and the oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 and fp16 MFMA (same rate)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PCIE5_X16_GBPS = 64.0       # nominal host link per direction

KERNEL_KINDS = ["k_adaln", "k_ln1", "k_qk", "k_v", "k_attn", "k_out", "k_ln2", "k_fc1", "k_fc2"]
KERNEL_DESC = {
    "k_qk": "q,k projection GEMM", "k_v": "v projection GEMM (transposed)", "k_attn": "flash attention",
    "k_out": "out projection GEMM + gated residual", "k_fc1": "MLP up GEMM + GELU",
    "k_fc2": "MLP down GEMM + gated residual", "k_adaln": "adaLN GEMV", "k_ln1": "LayerNorm+modulate",
    "k_ln2": "LayerNorm+modulate",
}
# pages' per-step overhead of the all-gather mode (release page, "Validation":
# Ascend 910B3, Cosmos3-Nano, DP4): stream switching and Python dispatch
PAGES_STEP_OVERHEAD_MS = {"stream_switching": 72.0, "collective_calls": 10.0, "python_dispatch": 68.0}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_work(shape, T):
    """Algorithmic flops (GEMMs, attention) or HBM bytes (norm kernels) per launch."""
    d, m, c = shape.d_model, shape.d_mlp, shape.d_cond
    return {
        "k_qk": ("flop", 2.0 * T * 2 * d * d),
        "k_v": ("flop", 2.0 * T * d * d),
        "k_attn": ("flop", 4.0 * T * T * d),
        "k_out": ("flop", 2.0 * T * d * d),
        "k_fc1": ("flop", 2.0 * T * m * d),
        "k_fc2": ("flop", 2.0 * T * d * m),
        "k_adaln": ("byte", 2.0 * 6 * d * c + 4.0 * 6 * d),
        "k_ln1": ("byte", 4.0 * T * d + 2.0 * T * d),
        "k_ln2": ("byte", 4.0 * T * d + 2.0 * T * d),
    }


def host_info():
    info = {"cpu_count": os.cpu_count(), "machine": platform.machine()}
    try:
        out = subprocess.run(["lscpu"], stdout=subprocess.PIPE, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        for line in open("/proc/meminfo"):
            if line.startswith(("MemTotal", "MemAvailable")):
                k, v = line.split(":")
                info[k] = v.strip()
    except Exception:
        pass
    return info


def source_hash(path):
    """sha256[:16] of a kernel source together with the device headers it
    includes (a change to either invalidates counters taken on the kernel)."""
    h = hashlib.sha256(open(path, "rb").read())
    d = os.path.dirname(path)
    for inc in ("device_common.h", "kernels.h"):
        h.update(open(os.path.join(d, inc), "rb").read())
    return h.hexdigest()[:16]


def kernel_source(kind):
    unit = "flop" if kind in ("k_qk", "k_v", "k_attn", "k_out", "k_fc1", "k_fc2") else "byte"
    name = "attention.hip" if kind == "k_attn" else ("gemm.hip" if unit == "flop" else "norm.hip")
    return os.path.join(ROOT, "layerwise_weight_streaming_dit_amd", "csrc", name)


def traffic_from_profiles(kind, workload):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary of this workload (profiles/hbm_traffic_<workload>_dit.txt: lines
    "kind source-sha16 fetch-bytes write-bytes", copy-calibrated), only if
    the counters were taken on the current kernel source and device headers;
    else None."""
    p = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}_dit.txt")
    if not os.path.exists(p):
        return None
    want = source_hash(kernel_source(kind))
    alias = {"k_ln1": "k_ln", "k_ln2": "k_ln"}.get(kind, kind)
    for line in open(p):
        f = line.split()
        if len(f) == 4 and f[0] == alias and f[1] == want:
            return float(f[2]) + float(f[3])
    return None


def busy(rs):
    """Length of the union of intervals (the two copy engines overlap)."""
    tot, cs, ce = 0.0, None, None
    for r in sorted(rs, key=lambda r: r["start"]):
        if ce is None or r["start"] > ce:
            if ce is not None:
                tot += ce - cs
            cs, ce = r["start"], r["end"]
        else:
            ce = max(ce, r["end"])
    return tot + (ce - cs if ce is not None else 0.0)


def overlap_of(rs):
    """Overlap figures of the intervals of one forward: E = max(busy(H2D and
    reconstruction), busy(compute)) / t_forward (<= 1; 1 = the slower side
    never waits), and the hidden fraction (H2D + compute - t) / min of the
    two (1 = the faster side is entirely hidden behind the slower)."""
    stage = [r for r in rs if r["kind"] in ("h2d", "asm")]
    comp = [r for r in rs if r["kind"] == "compute"]
    t = max(r["end"] for r in rs) - min(r["start"] for r in rs)
    h, a, c, st = (busy([r for r in rs if r["kind"] == "h2d"]), busy([r for r in rs if r["kind"] == "asm"]),
                   busy(comp), busy(stage))
    return {"t_forward_ms": t, "sum_h2d_ms": h, "sum_asm_ms": a, "sum_compute_ms": c,
            "E": max(st, c) / t, "hidden_frac": (h + c - t) / min(h, c),
            "hidden_side": "compute behind H2D" if c < h else "H2D behind compute"}


def step_costs(tr, L, f):
    """Per-step costs of forward f in a trace spanning forwards f-1 and f:
    the compute stream's idle time between consecutive blocks, split into the
    wait for a block's weights (its reconstruction ended after the previous
    block's compute) and the switch itself (event wait + launch after the
    weights were ready), and the step time (last compute end to last compute
    end)."""
    comp = {(r["forward"], r["block"]): r for r in tr if r["kind"] == "compute"}
    ready = {}
    for r in tr:
        if r["kind"] == "asm":
            k = (r["forward"], r["block"])
            ready[k] = max(ready.get(k, r["end"]), r["end"])
    wait = switch = boundary = 0.0
    for b in range(L):
        prev = comp[(f, b - 1)] if b > 0 else comp[(f - 1, L - 1)]
        cur = comp[(f, b)]
        rdy = ready[(f, b)]
        w = max(0.0, rdy - prev["end"])
        sw = max(0.0, cur["start"] - max(prev["end"], rdy))
        wait += w
        switch += sw
        if b == 0:
            boundary = cur["start"] - prev["end"]
    return {"step_ms": comp[(f, L - 1)]["end"] - comp[(f - 1, L - 1)]["end"],
            "compute_idle_waiting_for_weights_ms": wait, "stream_switch_ms": switch,
            "step_boundary_gap_ms": boundary}


def cpu_baseline(wl, shapes, T, W_keep, seconds, min_blocks):
    """The oracle timed on the host cores on a bounded sample of blocks of the
    same workload at the full token count; blocks/s = blocks run / elapsed
    (a full forward would take blocks / value seconds).  `value` runs the
    oracle's arithmetic in fp32 (numpy with every BLAS thread); the oracle at
    its default fp64 is timed beside it where a block fits half the budget."""
    import numpy as np
    import synth
    from oracle import dit as D, layout as OL
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"] or [0])
    except Exception:
        threads = 0

    def timed(dtype, budget, at_least):
        x = synth.activations(T, shapes[0].d_model)
        cond = synth.conditioning(shapes[0].d_cond)
        n, elapsed = 0, 0.0
        for b in range(len(shapes)):
            shp = shapes[b]
            flat = W_keep[b] if b in W_keep else synth.block_weights(wl.wid, b, OL.block_numel(shp))
            if x.shape[1] != shp.d_model:
                x = D.width_adapter(x, shp.d_model)
            ts = time.perf_counter()
            x = D.dit_block(flat, shp, x, cond, dtype=dtype)
            elapsed += time.perf_counter() - ts
            n += 1
            log(f"cpu baseline ({np.dtype(dtype).name}): block {b} in {time.perf_counter() - ts:.1f} s")
            if elapsed >= budget and n >= at_least:
                break
        return n, elapsed

    n, elapsed = timed(np.float32, seconds, min_blocks)
    bps = n / elapsed
    out = {"value": bps, "unit": "blocks/s", "cores": threads or os.cpu_count(), "kind": "oracle",
           "sample": f"{n} of {len(shapes)} blocks of the {wl.name} workload at T={T}, numpy fp32, "
                     f"{elapsed:.1f} s of block compute (weight generation not timed); a whole "
                     f"{len(shapes)}-block forward extrapolates to {len(shapes) / bps:.0f} s",
           "tokens_per_s": bps * T / len(shapes)}
    if elapsed / n <= seconds / 2:
        n64, el64 = timed(np.float64, seconds / 2, 1)
        out["fp64"] = {"value": n64 / el64, "unit": "blocks/s",
                       "sample": f"{n64} of {len(shapes)} blocks, numpy fp64 (the oracle's default), {el64:.1f} s"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="large")
    ap.add_argument("--dp", type=int, default=0)
    ap.add_argument("--blocks", type=int, default=0,
                    help="stream only the first N blocks of the workload (per-block rates unchanged)")
    ap.add_argument("--chunk", type=int, default=0, help="H2D chunk in elements (0 = the library's default)")
    ap.add_argument("--gen-threads", type=int, default=12)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-min-blocks", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-serial", action="store_true")
    ap.add_argument("--timed-only", action="store_true",
                    help="only the warm-up and timed forwards (for counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device copy (the reconstruction kernel) so "
                         "a counter pass can scale HBM byte counters by a copy of known size")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the streamed forward has no multi-GPU path here "
              f"(asked for {max(args.gpus, world)} GPUs)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import layerwise_weight_streaming_dit_amd as dlo

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = 1 << 27  # elements: 256 MiB read + 256 MiB written
        src = torch.empty(n, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()
        dlo.op_assemble(dst, src, n)
        torch.cuda.synchronize()
        log(f"calibration copy: {2 * n} bytes read, {2 * n} bytes written")
        del src, dst
    wl = synth.workload(args.workload)
    shapes = list(wl.blocks)[: args.blocks] if args.blocks > 0 else list(wl.blocks)
    dp = args.dp or wl.dp_sizes[0]
    # a step of the irregular workload is its four sequential requests, each
    # with its own drawn token count; every other workload runs one request
    Ts = synth.request_tokens() if wl.name == "irregular" else [wl.tokens]
    T = max(Ts)
    L = len(shapes)
    dev = torch.device("cuda:0")
    numels = [dlo.block_layout(s, dp)[0] for s in shapes]
    n_keep = 0 if args.no_cpu_baseline else min(args.cpu_min_blocks, L)

    # ---- weights: drawn block by block and sharded into pinned memory; the
    # library keeps no reference to the drawn array, so host memory holds the
    # model once (plus the blocks drawn ahead)
    def load(nblocks):
        c = dlo.StreamedDiT(shapes[:nblocks], dp, T, flags=dlo.FLAG_TRACE_KERNELS, chunk_elems=args.chunk)
        keep, t_gen = {}, time.perf_counter()
        for b, flat in synth.iter_block_weights(wl.wid, numels[:nblocks], threads=args.gen_threads):
            try:
                c.load_shards(b, flat)
            except dlo.DloError as e:
                if e.code != dlo.E_HOST_OOM:
                    raise
                c.close()
                return None, b, keep
            if b < n_keep:
                keep[b] = flat
            if b % 10 == 9 or b == nblocks - 1:
                log(f"{b + 1}/{nblocks} blocks drawn and pinned ({time.perf_counter() - t_gen:.1f} s)")
        return c, nblocks, keep

    t0 = time.perf_counter()
    ctx, loaded, W_keep = load(L)
    repeats, note = 1, ""
    if ctx is None:
        # the host could not pin the whole model: stream a cyclic subset of k
        # distinct blocks, L / k forwards of the k-block context per step
        # (per-block H2D and compute are unchanged; the alternation continues
        # across forwards)
        k = max(d for d in range(1, L + 1) if L % d == 0 and d <= max(1, loaded - 2))
        log(f"pinning failed after {loaded} blocks: streaming a cyclic subset of {k} blocks")
        ctx, _, W_keep = load(k)
        repeats = L // k
        note = (f"; pinned host memory held only {loaded} of {L} blocks, so each step streams a cyclic "
                f"subset of {k} distinct blocks {repeats} times ({L} block-steps)")
    load_s = time.perf_counter() - t0
    pinned_bytes = sum(2 * dp * (-(-n // dp)) for n in numels[: len(ctx.shapes)])
    log(f"{wl.name}: {L} blocks, T={T}, dp={dp}; drawn, sharded and pinned in {load_s:.1f} s "
        f"({pinned_bytes / 1e9:.1f} GB pinned)")

    x0 = torch.from_numpy(synth.activations(T, shapes[0].d_model).reshape(-1)).to(dev)
    xbuf = torch.zeros(T * max(s.d_model for s in shapes), dtype=torch.float32, device=dev)
    xbuf[: x0.numel()] = x0
    cond = torch.from_numpy(synth.conditioning(shapes[0].d_cond)).to(dev)
    stream = torch.cuda.current_stream()

    def step():
        for _ in range(repeats):
            for t_req in Ts:
                ctx.forward(xbuf, cond, t_req)

    def kernel_stats(tr, kinds):
        """Per-kernel launch statistics of the traced forwards in tr."""
        f_first = min((r["forward"] for r in tr), default=0)

        def t_of(r):  # token count of a traced forward (the steps cycle through the requests)
            return Ts[(r["forward"] - f_first) % len(Ts)]

        def step_of(r):
            return (r["forward"] - f_first) // (len(Ts) * max(repeats, 1))

        by = {}
        for r in tr:
            if r["kind"] in kinds:
                by.setdefault(r["kind"], []).append(r)
        out = {}
        for kind in kinds:
            rs = by.get(kind, [])
            if not rs:
                continue
            ds = sorted(r["end"] - r["start"] for r in rs)
            avg = sum(ds) / len(ds)
            med = ds[len(ds) // 2]
            # work per launch follows each launch's block (widths differ
            # between blocks in the irregular workload); average work /
            # average time
            unit = kernel_work(shapes[0], T)[kind][0]
            work = sum(kernel_work(shapes[r["block"]], t_of(r))[kind][1] for r in rs) / len(rs)
            e = {"launches": len(rs), "avg_ms": avg, "median_ms": med, "max_ms": ds[-1], "total_ms": sum(ds),
                 "work_per_launch": work, "desc": KERNEL_DESC[kind],
                 "launches_over_1_5x_median": sum(1 for x in ds if x > 1.5 * med),
                 # the slowest launches: (step of the pass, block, ms)
                 "slowest": [[step_of(r), r["block"], round(r["end"] - r["start"], 4)]
                             for r in sorted(rs, key=lambda r: r["start"] - r["end"])[:4]]}
            # average launch per step of the pass (a slow stretch shows as one step)
            per_step = {}
            for r in rs:
                per_step.setdefault(step_of(r), []).append(r["end"] - r["start"])
            e["avg_ms_by_step"] = [round(sum(v) / len(v), 4) for _, v in sorted(per_step.items())]
            if unit == "flop":
                e["TFLOPs"] = work / (avg * 1e-3) / 1e12
                e["mfma_frac"] = e["TFLOPs"] / PEAK_BF16_TFLOPS
            else:
                e["GBps"] = work / (avg * 1e-3) / 1e9
                e["hbm_frac"] = e["GBps"] / PEAK_HBM_GBPS
            out[kind] = e
        return out

    # ---- warm-up, every kernel traced: it names the dominant kernel (the
    # largest median launch time x launches; the first step's cold launches
    # do not decide it)
    ctx.reserve_trace(args.warmup * repeats * len(Ts))
    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warm-up step {i + 1}/{args.warmup} done")
    wk = kernel_stats(ctx.trace(), KERNEL_KINDS)
    dom = max(wk, key=lambda k: wk[k]["median_ms"] * wk[k]["launches"]) if wk else "k_fc1"

    # ---- timed region: HIP events on the compute stream around the dominant
    # kernel only (each event pair between two kernels costs the stream a
    # little; the per-kernel statistics come from a separate pass below),
    # created before timing starts
    ctx.set_trace_kinds(1 << dlo.IV_KIND[dom])
    ctx.reserve_trace(args.steps * repeats * len(Ts))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ts = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - ts
    ms_per_step = 1e3 * elapsed / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (events {ev0.elapsed_time(ev1) / args.steps:.3f})")
    timed_dom = kernel_stats(ctx.trace(), [dom])[dom]

    # ---- every kernel traced, over up to two more steps: per-kernel statistics
    n_k = max(1, min(2, args.steps))
    ctx.set_trace_kinds(dlo.TRACE_KINDS_ALL)
    ctx.reserve_trace(n_k * repeats * len(Ts))
    torch.cuda.synchronize()
    for _ in range(n_k):
        step()
    torch.cuda.synchronize()
    kernels = kernel_stats(ctx.trace(), KERNEL_KINDS)
    log(f"kernel statistics over {n_k} more steps, every kernel traced")
    gemm_kinds = [k for k in ("k_qk", "k_v", "k_out", "k_fc1", "k_fc2") if k in kernels]
    gemm_flops = sum(kernels[k]["work_per_launch"] * kernels[k]["launches"] for k in gemm_kinds)
    gemm_ms = sum(kernels[k]["total_ms"] for k in gemm_kinds)
    gemm_util = gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS if gemm_ms else None
    unit, work = kernel_work(shapes[0], T)[dom][0], timed_dom["work_per_launch"]
    peak = PEAK_BF16_TFLOPS if unit == "flop" else PEAK_HBM_GBPS
    scale = 1e12 if unit == "flop" else 1e9
    ach = work / (timed_dom["avg_ms"] * 1e-3) / scale
    ach_med = work / (timed_dom["median_ms"] * 1e-3) / scale
    roofline = {"bound": "mfma" if unit == "flop" else "hbm", "achieved": ach, "peak": peak,
                "unit": "TFLOP/s" if unit == "flop" else "GB/s", "frac": ach / peak,
                "traffic": traffic_from_profiles(dom, wl.name),
                "kernel": f"{dom}: {KERNEL_DESC[dom]}", "avg_launch_ms": timed_dom["avg_ms"],
                "median_launch_ms": timed_dom["median_ms"], "max_launch_ms": timed_dom["max_ms"],
                "frac_by_median": ach_med / peak, "launches": timed_dom["launches"],
                "launches_over_1_5x_median": timed_dom["launches_over_1_5x_median"],
                "work_per_launch": work, "work_unit": unit,
                "timing": "HIP events around this kernel only, every launch of the timed steps"}

    # ---- untraced pass: host dispatch per step and the untraced step time
    ctx.set_flags(0)
    torch.cuda.synchronize()
    enq, enq_cpu, n_u = 0.0, 0.0, 2
    tu = time.perf_counter()
    for _ in range(n_u):
        te, tc = time.perf_counter(), time.thread_time()
        step()
        enq += time.perf_counter() - te
        enq_cpu += time.thread_time() - tc
    torch.cuda.synchronize()
    untraced_ms = 1e3 * (time.perf_counter() - tu) / n_u
    dispatch_ms = 1e3 * enq / n_u
    dispatch_cpu_ms = 1e3 * enq_cpu / n_u
    log(f"untraced: {untraced_ms:.3f} ms/step, host dispatch {dispatch_ms:.3f} ms/step "
        f"({dispatch_cpu_ms:.3f} ms of thread CPU time)")

    # one step on an idle device (no previous step to overlap its pipeline
    # fill with): the difference to the back-to-back step time is what
    # streaming across step boundaries hides
    torch.cuda.synchronize()
    ti = time.perf_counter()
    step()
    torch.cuda.synchronize()
    iso_ms = 1e3 * (time.perf_counter() - ti)

    sched = residency = costs = None
    serial = None
    if not args.timed_only:
        # ---- fully traced pass over two consecutive forwards
        ctx.set_flags(dlo.FLAG_TRACE | dlo.FLAG_TRACE_SPAN)
        ctx.reserve_trace(2)
        torch.cuda.synchronize()
        for i in range(2):
            ctx.forward(xbuf, cond, Ts[i % len(Ts)])
        torch.cuda.synchronize()
        st = ctx.stats()
        tr = ctx.trace()
        fwds = sorted({r["forward"] for r in tr})
        f0, f1 = fwds[0], fwds[-1]
        Lc = len(ctx.shapes)
        per_fwd = {f: overlap_of([r for r in tr if r["forward"] == f]) for f in (f0, f1)}
        h2d_rs = [r for r in tr if r["kind"] == "h2d"]
        asm_rs = [r for r in tr if r["kind"] == "asm"]
        h2d_busy, asm_busy = busy(h2d_rs), busy(asm_rs)
        sched = {"first_forward": per_fwd[f0], "following_forward": per_fwd[f1],
                 "h2d_GBps_busy": sum(r["bytes"] for r in h2d_rs) / (h2d_busy * 1e-3) / 1e9,
                 "assemble_GBps": 2 * sum(r["bytes"] for r in asm_rs) / (asm_busy * 1e-3) / 1e9,
                 "assemble_bytes_note": "reconstruction reads and writes each valid byte once"}
        costs = step_costs(tr, Lc, f1)
        costs.update({"host_dispatch_ms_per_step_untraced": dispatch_ms,
                      "host_dispatch_cpu_ms_per_step_untraced": dispatch_cpu_ms,
                      "host_dispatch_note": "wall and thread-CPU time of enqueuing one step (wall time includes "
                                            "waits for space in the device queues); all of it behind the GPU",
                      "pages_all_gather_overhead_ms_per_step": PAGES_STEP_OVERHEAD_MS})
        residency = {"slot_high_water_blocks": st["residency_high_water"],
                     "blocks_on_device_high_water": st["blocks_on_device_high_water"],
                     "weight_bytes_peak_in_use": st["weight_bytes_peak"],
                     "weight_bytes_allocated": st["weight_bytes_allocated"],
                     "max_block_bytes": st["max_block_bytes"],
                     "allocated_over_max_block": st["weight_bytes_allocated"] / st["max_block_bytes"],
                     "slot_bytes": st["slot_bytes"], "landing_bytes": st["landing_bytes"],
                     "landing_chunk_elems": st["landing_chunk_elems"], "workspace_bytes": st["workspace_bytes"],
                     "note": "from the traced pass over two consecutive forwards: a block counts on the device "
                             "from its first H2D start (landing buffers included) to its compute end"}
        log(f"traced pass: step {costs['step_ms']:.2f} ms, E {per_fwd[f1]['E']:.3f}, "
            f"hidden {per_fwd[f1]['hidden_frac']:.3f}, blocks on device <= {st['blocks_on_device_high_water']}")

        # ---- synchronous schedule (H2D -> wait -> reconstruct -> wait ->
        # compute), same kernels
        if not args.no_serial:
            ctx.set_flags(dlo.FLAG_SERIALIZE)
            torch.cuda.synchronize()
            tss = time.perf_counter()
            step()
            torch.cuda.synchronize()
            serial = 1e3 * (time.perf_counter() - tss)
            log(f"serialized: {serial:.2f} ms/step")
    st_all = ctx.stats()
    ctx.close()

    # pinned H2D ceiling: a plain back-to-back copy of (up to 512 MB of) one
    # block's bytes
    nbytes = min(2 * dp * (-(-numels[0] // dp)), 512 << 20)
    hsrc = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    ddst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(2):
            ddst.copy_(hsrc, non_blocking=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(side)
        for _ in range(8):
            ddst.copy_(hsrc, non_blocking=True)
        e1.record(side)
    torch.cuda.synchronize()
    h2d_ceiling = 8 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del hsrc, ddst

    cpu = None
    if not args.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0:
        cpu = cpu_baseline(wl, shapes, T, W_keep, args.cpu_seconds, args.cpu_min_blocks)

    value = L * len(Ts) * args.steps / elapsed
    shp = shapes[0]
    h2d_per_step = st_all["h2d_bytes_per_forward"] * repeats
    out = {
        "metric": "streamed DiT blocks/s & tokens/s; H2D GB/s, GEMM MFMA util, overlap %",
        "value": value,
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "precision": "weights bf16 as streamed, converted to fp16 by the reconstruction (exact for |w| >= 2^-17); "
                     "fp16 matrix-core operands; fp32 accumulation, softmax, residual and modulation",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) activations)",
        "config": {"workload": wl.description + (f"; first {L} of {wl.num_blocks} blocks streamed"
                                                 if L < wl.num_blocks else "") + note,
                   "blocks": L, "d_model": shp.d_model, "heads": shp.n_heads,
                   "d_mlp": shp.d_mlp, "d_cond": shp.d_cond, "tokens": T if len(Ts) == 1 else Ts,
                   "batch": 1, "dp_size": dp,
                   "slots": 2, "pinned_host_bytes": pinned_bytes, "parallelism": "single GPU"},
        "tokens_per_s": sum(Ts) * args.steps / elapsed,
        "token_blocks_per_s": sum(Ts) * L * args.steps / elapsed,
        "h2d_GBps_effective": h2d_per_step * len(Ts) * args.steps / elapsed / 1e9,
        "h2d_GBps_busy": sched["h2d_GBps_busy"] if sched else None,
        "h2d_ceiling_GBps": h2d_ceiling,
        "h2d_frac_of_pcie5_x16": (sched["h2d_GBps_busy"] / PCIE5_X16_GBPS) if sched else None,
        "assemble_GBps": sched["assemble_GBps"] if sched else None,
        "gemm_mfma_util": gemm_util,
        "step_boundary": {"isolated_step_ms": iso_ms, "back_to_back_ms_per_step": ms_per_step,
                          "untraced_back_to_back_ms_per_step": untraced_ms},
        "step_overhead": costs,
        "overlap": dict(sched or {}, serialized_ms_per_step=serial),
        "residency": residency,
        "kernels": kernels,
        "kernels_pass": f"{n_k} step(s) after the timed region with every kernel traced (the timed steps "
                        f"carry events around the dominant kernel only)",
        "roofline": roofline,
        "cpu_baseline": cpu,
        "setup_s": load_s,
        "gpu": torch.cuda.get_device_name(0),
        "host": host_info(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
