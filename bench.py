#!/usr/bin/env python3
"""Throughput of the layer-by-layer weight-streamed DiT forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload image]

A step is one streamed forward over every block of the workload (H2D of all
dp shards of every block, on-GPU reconstruction into one of two slots, and
the DiT block from the other slot), for one batch of synthetic input whose
weights already sit in pinned host memory and whose activations already sit
in HBM.  W untimed steps, then K timed steps between two device syncs.

Prints ONE JSON line: blocks/s as ``value`` plus tokens/s, H2D GB/s, GEMM
MFMA utilisation, overlap, a roofline of the dominant kernel (timed with HIP
events on the compute stream inside the timed region) and the oracle timed
on the host cores.
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


def traffic_from_profiles(kernel_src, kind, workload):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary (profiles/hbm_traffic_image_dit.txt: lines "kind source-sha16
    fetch-bytes write-bytes", copy-calibrated), used only for the workload the
    counters were taken on (image) and only if they were taken on the current
    kernel source and device headers; else None."""
    if workload != "image":
        return None
    p = os.path.join(ROOT, "profiles", "hbm_traffic_image_dit.txt")
    if not os.path.exists(p):
        return None
    want = source_hash(kernel_src)
    for line in open(p):
        f = line.split()
        if len(f) == 4 and f[0] == kind and f[1] == want:
            return float(f[2]) + float(f[3])
    return None


def cpu_baseline(wl, dp, T, seconds):
    """The oracle timed on the host cores on a bounded sample of blocks of the
    same workload at the full token count; blocks/s = blocks run / elapsed.
    `value` runs the oracle's arithmetic in fp32 (numpy with every BLAS
    thread); the same oracle at its default fp64 is timed on a smaller
    sample and reported beside it."""
    import numpy as np
    import synth
    from oracle import dit as D, layout as OL
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"] or [0])
    except Exception:
        threads = 0

    def timed(dtype, budget):
        x = synth.activations(T, wl.blocks[0].d_model)
        cond = synth.conditioning(wl.blocks[0].d_cond)
        n, elapsed = 0, 0.0
        for b in range(wl.num_blocks):
            shp = wl.blocks[b]
            flat = synth.block_weights(wl.wid, b, OL.block_numel(shp))
            if x.shape[1] != shp.d_model:
                x = D.width_adapter(x, shp.d_model)
            ts = time.perf_counter()
            x = D.dit_block(flat, shp, x, cond, dtype=dtype)
            elapsed += time.perf_counter() - ts
            n += 1
            if elapsed >= budget:
                break
        return n, elapsed

    n, elapsed = timed(np.float32, seconds)
    n64, el64 = timed(np.float64, seconds / 2)
    bps = n / elapsed
    return {"value": bps, "unit": "blocks/s", "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": f"{n} of {wl.num_blocks} blocks of the {wl.name} workload at T={T}, numpy fp32, "
                      f"{elapsed:.1f} s of block compute (weight generation not timed)",
            "tokens_per_s": bps * T / wl.num_blocks,
            "fp64": {"value": n64 / el64, "unit": "blocks/s",
                     "sample": f"{n64} of {wl.num_blocks} blocks, numpy fp64 (the oracle's default), {el64:.1f} s"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="image")
    ap.add_argument("--dp", type=int, default=0)
    ap.add_argument("--blocks", type=int, default=0,
                    help="stream only the first N blocks of the workload (per-block rates unchanged; "
                         "for shapes whose full weight set would not fit host memory twice)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-serial", action="store_true")
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
        print(f"[bench] calibration copy: {2 * n} bytes read, {2 * n} bytes written", file=sys.stderr, flush=True)
        del src, dst
    wl = synth.workload(args.workload)
    shapes = list(wl.blocks)[: args.blocks] if args.blocks > 0 else list(wl.blocks)
    dp = args.dp or wl.dp_sizes[0]
    T = wl.tokens
    L = len(shapes)
    dev = torch.device("cuda:0")

    t0 = time.perf_counter()
    numels = [dlo.block_layout(s, dp)[0] for s in shapes]
    W = synth.many_block_weights(wl.wid, numels)
    gen_s = time.perf_counter() - t0

    def make(flags):
        ctx = dlo.StreamedDiT(shapes, dp, T, flags=flags)
        for b in range(L):
            ctx.load_shards(b, W[b])
        return ctx

    x0 = torch.from_numpy(synth.activations(T, shapes[0].d_model).reshape(-1)).to(dev)
    xbuf = torch.zeros(T * max(s.d_model for s in shapes), dtype=torch.float32, device=dev)
    xbuf[: x0.numel()] = x0
    cond = torch.from_numpy(synth.conditioning(shapes[0].d_cond)).to(dev)
    stream = torch.cuda.current_stream()

    t1 = time.perf_counter()
    # the timed context records HIP events only on the compute stream (around
    # each kernel), so the copy and gather streams run exactly as untraced
    ctx = make(dlo.FLAG_TRACE_KERNELS)
    load_s = time.perf_counter() - t1
    print(f"[bench] {wl.name}: {L} blocks, T={T}, dp={dp}; weights generated in {gen_s:.1f} s, "
          f"sharded+pinned in {load_s:.1f} s", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        ctx.forward(xbuf, cond, T)
    torch.cuda.synchronize()
    ctx.trace()  # kernel intervals accumulate until read: drop the warm-up's
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ts = time.perf_counter()
    enqueue_s = 0.0
    ev0.record(stream)
    for _ in range(args.steps):
        te = time.perf_counter()
        ctx.forward(xbuf, cond, T)
        enqueue_s += time.perf_counter() - te
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - ts
    ev_ms = ev0.elapsed_time(ev1)
    elapsed = wall
    ms_per_step = 1e3 * elapsed / args.steps
    print(f"[bench] timed {args.steps} forwards: {ms_per_step:.3f} ms/forward (events {ev_ms / args.steps:.3f})",
          file=sys.stderr, flush=True)

    # kernel durations: every launch of the timed region
    ktr = ctx.trace()
    # one forward on an idle device (no previous forward to overlap its
    # pipeline fill with): the difference to the back-to-back step time is
    # what streaming across step boundaries hides
    iso = []
    for _ in range(3):
        torch.cuda.synchronize()
        ti = time.perf_counter()
        ctx.forward(xbuf, cond, T)
        torch.cuda.synchronize()
        iso.append(1e3 * (time.perf_counter() - ti))
    iso_ms = sorted(iso)[1]
    ctx.close()
    # schedule breakdown: a fully traced context (events on all three
    # streams), run back to back like the timed region
    fctx = make(dlo.FLAG_TRACE)
    for _ in range(3):
        fctx.forward(xbuf, cond, T)
    torch.cuda.synchronize()
    tr = fctx.trace()
    st = fctx.stats()
    fctx.close()
    by = {}
    for r in tr:
        if not r["kind"].startswith("k_"):
            by.setdefault(r["kind"], []).append(r)
    for r in ktr:
        if r["kind"].startswith("k_"):
            by.setdefault(r["kind"], []).append(r)
    dur = lambda rs: sum(r["end"] - r["start"] for r in rs)

    def busy(rs):
        # length of the union of intervals (the two copy engines overlap)
        tot, cs, ce = 0.0, None, None
        for r in sorted(rs, key=lambda r: r["start"]):
            if ce is None or r["start"] > ce:
                if ce is not None:
                    tot += ce - cs
                cs, ce = r["start"], r["end"]
            else:
                ce = max(ce, r["end"])
        return tot + (ce - cs if ce is not None else 0.0)

    h2d_ms, asm_ms, comp_ms = busy(by.get("h2d", [])), busy(by.get("asm", [])), busy(by.get("compute", []))
    t_fwd = max(r["end"] for r in tr) - min(r["start"] for r in tr)
    h2d_bytes = sum(r["bytes"] for r in by.get("h2d", []))
    asm_read = sum(r["bytes"] for r in by.get("asm", []))
    overlap_E = max(h2d_ms + asm_ms, comp_ms) / t_fwd
    hidden = (h2d_ms + comp_ms - t_fwd) / min(h2d_ms, comp_ms)
    # steady state: the staging of blocks 1..L-1 against the compute of
    # blocks 0..L-2 (what can overlap once the pipeline is full), inside the
    # window from the first staging of block 1 to the end of compute(L-2)
    steady = None
    if L >= 3:
        st_rs = [r for r in tr if r["kind"] in ("h2d", "asm") and r["block"] >= 1]
        cp_rs = [r for r in tr if r["kind"] == "compute" and r["block"] <= L - 2]
        w0 = min(r["start"] for r in st_rs if r["block"] == 1)
        w1 = max(r["end"] for r in cp_rs if r["block"] == L - 2)
        clip = lambda rs: [dict(r, start=max(r["start"], w0), end=min(r["end"], w1)) for r in rs
                           if r["end"] > w0 and r["start"] < w1]
        h_s = busy(clip([r for r in st_rs if r["kind"] == "h2d"]))
        a_s = busy(clip([r for r in st_rs if r["kind"] == "asm"]))
        c_s = busy(clip(cp_rs))
        win = w1 - w0
        steady = {"window_ms": win, "sum_h2d_ms": h_s, "sum_asm_ms": a_s, "sum_compute_ms": c_s,
                  "E": max(h_s + a_s, c_s) / win, "hidden_frac": (h_s + c_s - win) / min(h_s, c_s)}
    kernels = {}
    for kind in KERNEL_KINDS:
        rs = by.get(kind, [])
        if not rs:
            continue
        avg = dur(rs) / len(rs)
        ds = sorted(r["end"] - r["start"] for r in rs)
        # work per launch follows each launch's block (widths differ between
        # blocks in the irregular workload); average work / average time
        unit = kernel_work(shapes[0], T)[kind][0]
        work = sum(kernel_work(shapes[r["block"]], T)[kind][1] for r in rs) / len(rs)
        rate = work / (avg * 1e-3)
        # the median shows how far a few slow launches pull the average
        e = {"launches": len(rs), "avg_ms": avg, "median_ms": ds[len(ds) // 2], "max_ms": ds[-1], "total_ms": dur(rs),
             "work_per_launch": work, "desc": KERNEL_DESC[kind]}
        if unit == "flop":
            e["TFLOPs"] = rate / 1e12
            e["mfma_frac"] = rate / 1e12 / PEAK_BF16_TFLOPS
        else:
            e["GBps"] = rate / 1e9
            e["hbm_frac"] = rate / 1e9 / PEAK_HBM_GBPS
        kernels[kind] = e
    gemm_kinds = [k for k in ("k_qk", "k_v", "k_out", "k_fc1", "k_fc2") if k in kernels]
    gemm_flops = sum(kernels[k]["work_per_launch"] * kernels[k]["launches"] for k in gemm_kinds)
    gemm_ms = sum(kernels[k]["total_ms"] for k in gemm_kinds)
    gemm_util = gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS if gemm_ms else None
    dom = max(kernels, key=lambda k: kernels[k]["total_ms"])
    unit, work = kernel_work(shapes[0], T)[dom][0], kernels[dom]["work_per_launch"]
    ach = kernels[dom]["TFLOPs"] if unit == "flop" else kernels[dom]["GBps"]
    src = os.path.join(ROOT, "layerwise_weight_streaming_dit_amd", "csrc",
                       "attention.hip" if dom == "k_attn" else ("gemm.hip" if unit == "flop" else "norm.hip"))
    roofline = {"bound": "mfma" if unit == "flop" else "hbm", "achieved": ach,
                "peak": PEAK_BF16_TFLOPS if unit == "flop" else PEAK_HBM_GBPS,
                "unit": "TFLOP/s" if unit == "flop" else "GB/s",
                "frac": ach / (PEAK_BF16_TFLOPS if unit == "flop" else PEAK_HBM_GBPS),
                "traffic": traffic_from_profiles(src, dom, wl.name),
                "kernel": f"{dom}: {KERNEL_DESC[dom]}", "avg_launch_ms": kernels[dom]["avg_ms"],
                # achieved and frac use the average launch; a single launch
                # caught in one of the device's occasional multi-millisecond
                # stalls moves it, the median does not
                "median_launch_ms": kernels[dom]["median_ms"], "max_launch_ms": kernels[dom]["max_ms"],
                "work_per_launch": work, "work_unit": unit}

    # synchronous schedule (H2D -> wait -> reconstruct -> wait -> compute), same kernels
    serial = enqueue_untraced_us = None
    if not args.no_serial:
        sctx = make(dlo.FLAG_SERIALIZE)
        sctx.forward(xbuf, cond, T)
        torch.cuda.synchronize()
        n_s = max(2, args.steps // 4)
        ts = time.perf_counter()
        enq_s = 0.0
        for _ in range(n_s):
            te = time.perf_counter()
            sctx.forward(xbuf, cond, T)
            enq_s += time.perf_counter() - te
        torch.cuda.synchronize()
        serial = 1e3 * (time.perf_counter() - ts) / n_s
        enqueue_untraced_us = 1e6 * enq_s / n_s
        sctx.close()

    # pinned H2D ceiling with a plain copy of the same size as one block's shards
    nbytes = 2 * dp * (-(-numels[0] // dp))
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
    del W

    cpu = None
    if not args.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0:
        cpu = cpu_baseline(wl, dp, T, args.cpu_seconds)

    value = L * args.steps / elapsed
    shp = shapes[0]
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
        "precision": "weights bf16 (streamed, reconstructed bit-exact, widened to fp16 in registers); "
                     "fp16 matrix-core operands; fp32 accumulation, softmax, residual and modulation",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) activations)",
        "config": {"workload": wl.description + (f"; first {L} of {wl.num_blocks} blocks streamed"
                                                 if L < wl.num_blocks else ""), "blocks": L, "d_model": shp.d_model, "heads": shp.n_heads,
                   "d_mlp": shp.d_mlp, "d_cond": shp.d_cond, "tokens": T, "batch": 1, "dp_size": dp,
                   "slots": 2, "parallelism": "single GPU"},
        "tokens_per_s": T * args.steps / elapsed,
        "token_blocks_per_s": T * L * args.steps / elapsed,
        "h2d_GBps_busy": h2d_bytes / (h2d_ms * 1e-3) / 1e9 if h2d_ms else None,
        "h2d_GBps_effective": st["h2d_bytes_per_forward"] * args.steps / elapsed / 1e9,
        "h2d_ceiling_GBps": h2d_ceiling,
        "h2d_frac_of_pcie5_x16": (h2d_bytes / (h2d_ms * 1e-3) / 1e9) / PCIE5_X16_GBPS if h2d_ms else None,
        "assemble_GBps": (asm_read * 2) / (asm_ms * 1e-3) / 1e9 if asm_ms else None,
        "gemm_mfma_util": gemm_util,
        "step_boundary": {"isolated_forward_ms": iso_ms, "back_to_back_ms_per_step": ms_per_step,
                          "host_enqueue_us_per_forward": 1e6 * enqueue_s / args.steps,
                          "host_enqueue_us_per_block": 1e6 * enqueue_s / args.steps / L,
                          "host_enqueue_note": "timed context records HIP events around every kernel",
                          "host_enqueue_us_per_forward_untraced": enqueue_untraced_us},
        "overlap": {"E": overlap_E, "hidden_frac": hidden, "t_forward_ms": t_fwd, "sum_h2d_ms": h2d_ms,
                    "sum_asm_ms": asm_ms, "sum_compute_ms": comp_ms, "serialized_ms": serial,
                    "steady_state": steady},
        "residency": {"high_water_blocks": st["residency_high_water"],
                      "high_water_note": "most blocks whose slot was occupied at one instant (from the block's first "
                                         "reconstruction write to the end of its compute); 1 when each block "
                                         "travels as one transfer that lands only after the previous block computed",
                      "slot_bytes": st["slot_bytes"],
                      "landing_bytes": st["landing_bytes"], "workspace_bytes": st["workspace_bytes"]},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "gpu": torch.cuda.get_device_name(0),
        "host": host_info(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
