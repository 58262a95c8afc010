"""The streamed forward through the C ABI against the oracle, plus the
invariants the method fixes: bit-exact reconstruction, exact adaLN-Zero
identity, outputs independent of dp_size / schedule / chunking, the
two-slot schedule, and fail-closed errors."""
import numpy as np
import pytest

import synth
from oracle import dit as D, layout as OL, shard as OS, trace as OT
from gpu_util import assert_reconstructed, dev, host, within, torch

pytestmark = pytest.mark.gpu

import layerwise_weight_streaming_dit_amd as dlo


def _weights(wl, blocks=None):
    blocks = range(wl.num_blocks) if blocks is None else blocks
    return {b: synth.block_weights(wl.wid, b, OL.block_numel(wl.blocks[b])) for b in blocks}


def _ctx(shapes, dp, T, flags=0, chunk=0):
    return dlo.StreamedDiT(shapes, dp, T, flags=flags, chunk_elems=chunk)


def _run(ctx, x, cond):
    t = torch()
    T, d0 = x.shape
    xbuf = t.zeros(T * ctx.max_d, dtype=t.float32, device="cuda")
    xbuf[: T * d0] = dev(x.reshape(-1))
    out = ctx.forward(xbuf, dev(cond), T)
    t.cuda.synchronize()
    return host(out).copy()


# ------------------------------------------------------------ reconstruction

def test_debug_assemble_tiny_bit_exact():
    wl = synth.workload("tiny")
    W = _weights(wl)
    ctx = _ctx(list(wl.blocks), 4, wl.tokens)
    for b, flat in W.items():
        ctx.load_shards(b, flat)
        ref = OS.shard(flat, 4)
        for r in range(4):
            assert np.array_equal(ctx.get_shard(b, r), ref[r])
    for b, flat in W.items():
        got = ctx.debug_assemble(b)
        assert_reconstructed(got, OS.unshard(OS.shard(flat, 4), len(flat)))


@pytest.mark.parametrize("dp", [3, 8])
def test_debug_assemble_irregular_bit_exact(dp):
    wl = synth.workload("irregular")
    shapes = list(wl.blocks[:2])
    ctx = _ctx(shapes, dp, 64)
    for b in range(2):
        flat = synth.block_weights(wl.wid, b, OL.block_numel(shapes[b]))
        ctx.load_shards(b, flat)
        assert_reconstructed(ctx.debug_assemble(b), flat)


def test_debug_assemble_random_numel_sweep():
    rng = np.random.default_rng(2024)
    for it in range(12):
        dp = int(rng.integers(1, 17))
        extra = tuple(int(v) for v in rng.integers(0, 5000, size=int(rng.integers(1, 6))))
        shp = synth.BlockShape(128, 2, 128, 64, extra)
        n = OL.block_numel(shp)
        chunk = int(rng.choice([4096, 5000, 1 << 20]))
        ctx = _ctx([shp], dp, 16, chunk=chunk)
        flat = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
        ctx.load_shards(0, flat)
        print(f"dp {dp} extra {extra} chunk {chunk}", flush=True)
        assert_reconstructed(ctx.debug_assemble(0), flat)
        ctx.close()


# ---------------------------------------------------------- forward parity

def test_tiny_forward_matches_oracle():
    wl = synth.workload("tiny")
    W = _weights(wl)
    x = synth.activations(wl.tokens, 256)
    cond = synth.conditioning(256)
    ctx = _ctx(list(wl.blocks), 4, wl.tokens)
    for b, flat in W.items():
        ctx.load_shards(b, flat)
    got = _run(ctx, x, cond)
    want = D.dit_forward([W[b] for b in range(wl.num_blocks)], wl.blocks, x, cond)
    ok, ma, mr = within(got, want)
    print(f"tiny chained: max_abs {ma:.3e} max_rel {mr:.3e}")
    assert ok, (ma, mr)


def test_tiny_per_block_matches_oracle():
    wl = synth.workload("tiny")
    W = _weights(wl)
    x = synth.activations(wl.tokens, 256)
    cond = synth.conditioning(256)
    xin = x.astype(np.float64)
    for b in range(wl.num_blocks):
        ctx = _ctx([wl.blocks[b]], 4, wl.tokens)
        ctx.load_shards(0, W[b])
        got = _run(ctx, xin.astype(np.float32), cond)
        want = D.dit_block(W[b], wl.blocks[b], xin.astype(np.float32), cond)
        ok, ma, mr = within(got, want)
        assert ok, (b, ma, mr)
        xin = want
        ctx.close()


@pytest.mark.parametrize("T", [1, 5, 100, 257])
def test_tiny_ragged_tokens(T):
    wl = synth.workload("tiny")
    W = _weights(wl, [0, 1])
    shapes = list(wl.blocks[:2])
    x = synth.activations(T, 256)
    cond = synth.conditioning(256)
    ctx = _ctx(shapes, 4, 512)
    for b in range(2):
        ctx.load_shards(b, W[b])
    got = _run(ctx, x, cond)
    want = D.dit_forward([W[0], W[1]], shapes, x, cond)
    ok, ma, mr = within(got, want)
    assert ok, (T, ma, mr)


def test_smallest_block_with_all_padding_shards():
    # the smallest block the kernels accept (d 128, hd 64, MLP 128, cond 64)
    # has 148992 elements; at dp 1024 the shard size is 146 and the last three
    # shards hold only padding (degenerate shards of the ceil-division rule)
    shp = synth.BlockShape(128, 2, 128, 64)
    numel = OL.block_numel(shp)
    dp = 1024
    S = OS.shard_size(numel, dp)
    assert (dp - 1) * S >= numel  # at least one all-padding shard
    rng = np.random.default_rng(5)
    flat = synth.bf16_bits_from_f32((rng.standard_normal(numel) * 0.02).astype(np.float32))
    ctx = _ctx([shp, shp], dp, 64)
    ctx.load_shards(0, flat)
    ctx.load_shards(1, flat[::-1].copy())
    for r in (0, dp - 1):
        assert np.array_equal(ctx.get_shard(0, r), OS.shard(flat, dp)[r])
    assert_reconstructed(ctx.debug_assemble(0), flat)
    x = synth.activations(64, 128)
    cond = synth.conditioning(64)
    got = _run(ctx, x, cond)
    want = D.dit_forward([flat, flat[::-1].copy()], [shp, shp], x, cond)
    ok, ma, mr = within(got, want)
    assert ok, (ma, mr)


def _sampled_block_check(wl, b, T, dp, rows=48):
    shp = wl.blocks[b]
    flat = synth.block_weights(wl.wid, b, OL.block_numel(shp))
    x = synth.activations(T, shp.d_model)
    cond = synth.conditioning(shp.d_cond)
    ctx = _ctx([shp], dp, T)
    ctx.load_shards(0, flat)
    got = _run(ctx, x, cond)
    ctx.close()
    idx = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(b).integers(0, T, size=rows)]))
    want = D.dit_block(flat, shp, x, cond, rows=idx)
    ok, ma, mr = within(got[idx], want)
    print(f"{wl.name} block {b} T={T}: max_abs {ma:.3e} max_rel {mr:.3e}")
    assert ok, (ma, mr)


@pytest.mark.parametrize("b", [0, 27])
def test_image_block_full_size_sampled_rows(b):
    wl = synth.workload("image")
    _sampled_block_check(wl, b, wl.tokens, 4)


# --------------------------------------------------------------- invariants

def _tiny_out(dp=4, flags=0, chunk=0, W=None, x=None):
    wl = synth.workload("tiny")
    W = W or _weights(wl)
    x = synth.activations(wl.tokens, 256) if x is None else x
    ctx = _ctx(list(wl.blocks), dp, wl.tokens, flags=flags, chunk=chunk)
    for b, flat in W.items():
        ctx.load_shards(b, flat)
    out = _run(ctx, x, synth.conditioning(256))
    return out, ctx


def test_image_chained_forward_sampled_rows():
    # the whole 28-block image forward (weights streamed through both slots
    # 14 times) against the oracle's chained fp64 forward on sampled rows
    # (tests/golden/image_chain_rows.npz, written by make_image_chain.py)
    import os
    z = np.load(os.path.join(os.path.dirname(__file__), "golden", "image_chain_rows.npz"))
    wl = synth.workload("image")
    shapes = list(wl.blocks)
    numels = [OL.block_numel(s) for s in shapes]
    W = synth.many_block_weights(wl.wid, numels)
    ctx = _ctx(shapes, 4, wl.tokens)
    for b in range(len(shapes)):
        ctx.load_shards(b, W[b])
    got = _run(ctx, synth.activations(wl.tokens, 2048), synth.conditioning(256))
    ctx.close()
    ok, ma, mr = within(got[z["rows"]], z["out"])
    print(f"image chained 28 blocks: max_abs {ma:.3e} max_rel {mr:.3e}")
    assert ok, (ma, mr)


def test_outputs_identical_across_dp_chunking_and_schedule():
    base, _ = _tiny_out()
    for dp in (1, 3, 8):
        assert np.array_equal(_tiny_out(dp=dp)[0], base), dp
    assert np.array_equal(_tiny_out(chunk=4096)[0], base)
    assert np.array_equal(_tiny_out(flags=dlo.FLAG_SERIALIZE)[0], base)
    assert np.array_equal(_tiny_out(flags=dlo.FLAG_POISON_SLOTS)[0], base)


def test_chained_equals_successive_single_block_forwards():
    wl = synth.workload("tiny")
    W = _weights(wl)
    base, _ = _tiny_out(W=W)
    x = synth.activations(wl.tokens, 256)
    for b in range(wl.num_blocks):
        ctx = _ctx([wl.blocks[b]], 4, wl.tokens)
        ctx.load_shards(0, W[b])
        x = _run(ctx, x, synth.conditioning(256))
        ctx.close()
    assert np.array_equal(x, base)


def test_adaln_zero_identity_exact():
    wl = synth.workload("tiny")
    W = _weights(wl)
    for b, flat in W.items():
        tab = {p.name: p for p in OL.param_table(wl.blocks[b])}
        d = wl.blocks[b].d_model
        c = wl.blocks[b].d_cond
        flat = flat.copy()
        wada = flat[tab["Wada"].offset:tab["Wada"].offset + tab["Wada"].numel].reshape(6 * d, c)
        wada[2 * d:3 * d] = 0
        wada[5 * d:6 * d] = 0
        bada = flat[tab["bada"].offset:tab["bada"].offset + tab["bada"].numel]
        bada[2 * d:3 * d] = 0
        bada[5 * d:6 * d] = 0
        W[b] = flat
    x = synth.activations(wl.tokens, 256)
    out, _ = _tiny_out(W=W, x=x)
    assert np.array_equal(out, x)


def test_repeated_forwards_identical_and_allocate_nothing():
    t = torch()
    wl = synth.workload("tiny")
    W = _weights(wl)
    ctx = _ctx(list(wl.blocks), 4, wl.tokens)
    for b, flat in W.items():
        ctx.load_shards(b, flat)
    x = synth.activations(wl.tokens, 256)
    first = _run(ctx, x, synth.conditioning(256))
    t.cuda.synchronize()
    free0 = t.cuda.mem_get_info()[0]
    for _ in range(3):
        assert np.array_equal(_run(ctx, x, synth.conditioning(256)), first)
    t.cuda.synchronize()
    assert t.cuda.mem_get_info()[0] == free0


def test_trace_two_slot_schedule_image():
    wl = synth.workload("image")
    shapes = list(wl.blocks[:8])
    W = _weights(wl, range(8))
    ctx = _ctx(shapes, 4, wl.tokens, flags=dlo.FLAG_TRACE)
    for b in range(8):
        ctx.load_shards(b, W[b])
    x = synth.activations(wl.tokens, 2048)
    _run(ctx, x, synth.conditioning(256))
    tr = ctx.trace()
    st = ctx.stats()
    numels = [OL.block_numel(s) for s in shapes]
    errs = OT.check_trace(tr, 8, slot_capacity=st["slot_bytes"] // 2, numels=numels, dp=4)
    assert errs == [], errs[:5]
    assert st["slot_bytes"] == 2 * OT.slot_capacity_elems(numels, 4)
    # the library's residency figures are the oracle's, on the same intervals
    assert st["residency_high_water"] == OT.residency_high_water(tr, 8) <= 2
    assert st["blocks_on_device_high_water"] == OT.device_high_water(tr, 8) <= 2
    block_bytes = [2 * 4 * OS.shard_size(n, 4) for n in numels]
    assert st["weight_bytes_peak"] == OT.weight_bytes_peak(tr, 8, block_bytes)
    # every device byte that holds weights: two slots and two landing buffers
    # of one shard each = 2.5 blocks (release page, TL;DR: two layers' weights)
    assert st["max_block_bytes"] == max(block_bytes)
    assert st["weight_bytes_allocated"] == 2.5 * st["max_block_bytes"]
    assert st["weight_bytes_peak"] <= st["weight_bytes_allocated"]
    print("stats", st)


def _chain(ctx, x, cond, steps, streams=None, hold_cycles=0):
    """`steps` back-to-back forwards, each on the previous one's output (a
    denoising loop), optionally on a different stream per step.  hold_cycles
    > 0 first parks the compute stream in a bounded spin kernel, so that the
    host has enqueued every step before the GPU starts on them (the GPU then
    runs them back to back whatever the host's enqueue speed)."""
    t = torch()
    T, d0 = x.shape
    xbuf = t.zeros(T * ctx.max_d, dtype=t.float32, device="cuda")
    xbuf[: T * d0] = dev(x.reshape(-1))
    c = dev(cond)
    t.cuda.synchronize()
    if hold_cycles:
        t.cuda._sleep(hold_cycles)
    for i in range(steps):
        out = ctx.forward(xbuf, c, T, stream=None if streams is None else streams[i % len(streams)])
    t.cuda.synchronize()
    return host(out).copy()


@pytest.mark.parametrize("L", [3, 4])
def test_next_forward_first_block_streams_under_last_block(L):
    # A compute-bound shape (d 256, T 16384: attention dominates), cut into
    # several chunks per block, traced over three back-to-back forwards.
    shp = synth.BlockShape(256, 4, 1024)
    T = 16384
    W = [synth.block_weights(1, b, OL.block_numel(shp)) for b in range(L)]
    ctx = _ctx([shp] * L, 4, T, flags=dlo.FLAG_TRACE | dlo.FLAG_TRACE_SPAN, chunk=1 << 18)
    for b in range(L):
        ctx.load_shards(b, W[b])
    ctx.reserve_trace(3)
    x, cond = synth.activations(T, 256), synth.conditioning(256)
    got = _chain(ctx, x, cond, 3, hold_cycles=100_000_000)
    tr = ctx.trace()
    st_numel = OL.block_numel(shp)
    assert sorted({r["forward"] for r in tr}) == [0, 1, 2]
    errs = OT.check_trace(tr, L, slot_capacity=4 * OS.shard_size(st_numel, 4), numels=[st_numel] * L, dp=4)
    assert errs == [], errs[:5]
    assert OT.device_high_water(tr, L) == 2
    for s in range(2):
        last = [r for r in tr if r["kind"] == "compute" and r["forward"] == s and r["block"] == L - 1][0]
        nxt = [r for r in tr if r["kind"] in ("h2d", "asm") and r["forward"] == s + 1 and r["block"] == 0]
        assert len({r["chunk"] for r in nxt}) > 1
        # block 0 of step s+1 is copied and reconstructed while block L-1 of
        # step s computes, and not before block L-2 of step s released its slot
        assert max(r["end"] for r in nxt) <= last["end"], (s, max(r["end"] for r in nxt), last)
        prev = [r for r in tr if r["kind"] == "compute" and r["forward"] == s and r["block"] == L - 2][0]
        assert min(r["start"] for r in nxt) >= prev["end"]
    # the same loop untraced on a fresh context gives the same bits
    ref = _ctx([shp] * L, 4, T, chunk=1 << 18)
    for b in range(L):
        ref.load_shards(b, W[b])
    assert np.array_equal(got, _chain(ref, x, cond, 3))


def _overlap(a, b):
    """Length of the intersection of interval a with the union of intervals b."""
    segs = sorted((max(a["start"], r["start"]), min(a["end"], r["end"])) for r in b
                  if r["end"] > a["start"] and r["start"] < a["end"])
    tot, cs, ce = 0.0, None, None
    for s, e in segs:
        if ce is None or s > ce:
            tot += (ce - cs) if ce is not None else 0.0
            cs, ce = s, e
        else:
            ce = max(ce, e)
    return tot + ((ce - cs) if ce is not None else 0.0)


def test_h2d_hidden_behind_compute_when_compute_bound():
    """The method's overlap target on the compute-bound mid-video block
    (d 5120, 40 heads, MLP 20480, T 16384: ~15 ms of kernels against ~12 ms
    of H2D per block): the copies of blocks 1..L-1 run while earlier blocks
    compute, so at least 90% of their H2D time is hidden behind compute, and
    the forward takes within 10% of its summed compute plus the first
    block's staging."""
    L, T = 3, 16384
    shp = synth.workload("midvideo").blocks[0]
    ctx = _ctx([shp] * L, 4, T, flags=dlo.FLAG_TRACE)
    numels = [OL.block_numel(shp)] * L
    for b, flat in synth.iter_block_weights(3, numels, threads=8):
        ctx.load_shards(b, flat)
    x, cond = synth.activations(T, shp.d_model), synth.conditioning(256)
    _run(ctx, x, cond)  # first forward: warm-up
    ctx.trace()
    _run(ctx, x, cond)
    tr = ctx.trace()
    comp = [r for r in tr if r["kind"] == "compute"]
    h2d = [r for r in tr if r["kind"] == "h2d" and r["block"] >= 1]
    assert len(comp) == L and h2d
    h2d_time = sum(r["end"] - r["start"] for r in h2d)
    hidden = sum(_overlap(r, comp) for r in h2d)
    assert hidden >= 0.9 * h2d_time, (hidden, h2d_time)
    c = sum(r["end"] - r["start"] for r in comp)
    all_h2d = [r for r in tr if r["kind"] == "h2d"]
    busy_h2d = _overlap({"start": min(r["start"] for r in all_h2d), "end": max(r["end"] for r in all_h2d)}, all_h2d)
    assert c > busy_h2d, (c, busy_h2d)  # compute-bound, as designed
    stage0 = max(r["end"] for r in tr if r["kind"] == "asm" and r["block"] == 0) - \
        min(r["start"] for r in tr if r["kind"] == "h2d" and r["block"] == 0)
    t_fwd = max(r["end"] for r in comp) - min(r["start"] for r in tr)
    assert t_fwd <= 1.1 * (c + stage0), (t_fwd, c, stage0)
    ctx.close()


def test_forwards_on_alternating_streams_match_one_stream():
    # consecutive calls may pass different streams; each call is ordered after
    # the previous one (the context's workspace and x are shared)
    t = torch()
    wl = synth.workload("tiny")
    W = _weights(wl)
    ctxs = []
    for _ in range(2):
        c = _ctx(list(wl.blocks), 4, wl.tokens)
        for b, flat in W.items():
            c.load_shards(b, flat)
        ctxs.append(c)
    x, cond = synth.activations(wl.tokens, 256), synth.conditioning(256)
    one = _chain(ctxs[0], x, cond, 6)
    two = _chain(ctxs[1], x, cond, 6, streams=[t.cuda.Stream(), t.cuda.Stream()])
    assert np.array_equal(one, two)


def test_set_flags_reuses_one_shard_store():
    wl = synth.workload("tiny")
    W = _weights(wl)
    ctx = _ctx(list(wl.blocks), 4, wl.tokens)
    for b, flat in W.items():
        ctx.load_shards(b, flat)
    x, cond = synth.activations(wl.tokens, 256), synth.conditioning(256)
    base = _run(ctx, x, cond)
    assert ctx.trace() == []
    ctx.set_flags(dlo.FLAG_TRACE)
    assert np.array_equal(_run(ctx, x, cond), base)
    tr = ctx.trace()
    assert {"h2d", "asm", "compute", "k_fc2"} <= {r["kind"] for r in tr}
    assert OT.check_trace(tr, wl.num_blocks) == []
    ctx.set_flags(dlo.FLAG_TRACE | dlo.FLAG_SERIALIZE)
    assert np.array_equal(_run(ctx, x, cond), base)
    tr = ctx.trace()
    comp_end = {r["block"]: r["end"] for r in tr if r["kind"] == "compute"}
    assert all(r["start"] >= comp_end[r["block"] - 1] for r in tr if r["kind"] == "h2d" and r["block"] >= 1)
    ctx.set_flags(dlo.FLAG_TRACE_KERNELS)
    ctx.reserve_trace(2)
    for _ in range(2):
        assert np.array_equal(_run(ctx, x, cond), base)
    assert len(ctx.trace()) == 2 * wl.num_blocks * 10
    ctx.set_flags(0)
    assert np.array_equal(_run(ctx, x, cond), base)
    assert ctx.trace() == []
    with pytest.raises(dlo.DloError):
        ctx.set_flags(0x400)


def test_odd_block_count_alternates_slots_across_forwards():
    # 3 blocks: block 0 of each forward takes the slot the previous forward's
    # last block does not use, so consecutive forwards start in slots 0, 1, 0
    wl = synth.workload("tiny")
    shapes = list(wl.blocks[:3])
    W = _weights(wl, range(3))
    ctx = _ctx(shapes, 4, wl.tokens, flags=dlo.FLAG_TRACE)
    for b in range(3):
        ctx.load_shards(b, W[b])
    x = synth.activations(wl.tokens, 256)
    cond = synth.conditioning(256)
    outs = []
    for step in range(3):
        outs.append(_run(ctx, x, cond))
        tr = ctx.trace()
        assert OT.check_trace(tr, 3) == []
        first = {r["slot"] for r in tr if r["block"] == 0 and r["kind"] in ("asm", "compute")}
        assert first == {step % 2}, (step, first)
    fresh = _ctx(shapes, 4, wl.tokens)
    for b in range(3):
        fresh.load_shards(b, W[b])
    ref = _run(fresh, x, cond)
    for o in outs:
        assert np.array_equal(o, ref)


# ------------------------------------------------------------------ errors

def test_errors_fail_closed():
    t = torch()
    wl = synth.workload("tiny")
    ctx = _ctx(list(wl.blocks), 4, wl.tokens)
    xbuf = t.zeros(wl.tokens * 256, dtype=t.float32, device="cuda")
    cond = dev(synth.conditioning(256))
    assert ctx.forward_status(xbuf, cond, wl.tokens) == dlo.E_STATE  # nothing loaded
    W = _weights(wl)
    with pytest.raises(dlo.DloError) as e:
        ctx.load_shards(0, W[0][:-1])
    assert e.value.code == dlo.E_SHAPE
    for b, flat in W.items():
        ctx.load_shards(b, flat)
    assert ctx.forward_status(xbuf, cond, 0) == dlo.E_INVAL
    assert ctx.forward_status(xbuf, cond, wl.tokens + 1) == dlo.E_INVAL
    assert ctx.forward_status(None, cond, wl.tokens) == dlo.E_INVAL
    assert ctx.forward_status(xbuf, cond, wl.tokens) == dlo.OK
    t.cuda.synchronize()


def test_serialized_schedule_really_serializes():
    wl = synth.workload("tiny")
    W = _weights(wl)
    ctx = _ctx(list(wl.blocks), 4, wl.tokens, flags=dlo.FLAG_TRACE | dlo.FLAG_SERIALIZE)
    for b, flat in W.items():
        ctx.load_shards(b, flat)
    _run(ctx, synth.activations(wl.tokens, 256), synth.conditioning(256))
    tr = ctx.trace()
    assert OT.check_trace(tr, wl.num_blocks) == []
    comp_end = {r["block"]: r["end"] for r in tr if r["kind"] == "compute"}
    for r in tr:
        if r["kind"] == "h2d" and r["block"] >= 1:
            assert r["start"] >= comp_end[r["block"] - 1]


def test_kernel_trace_covers_every_step():
    wl = synth.workload("tiny")
    W = _weights(wl)
    ctx = _ctx(list(wl.blocks), 4, wl.tokens, flags=dlo.FLAG_TRACE_KERNELS)
    for b, flat in W.items():
        ctx.load_shards(b, flat)
    _run(ctx, synth.activations(wl.tokens, 256), synth.conditioning(256))
    tr = ctx.trace()
    kinds = {}
    for r in tr:
        kinds.setdefault(r["kind"], []).append(r)
    assert "h2d" not in kinds and "asm" not in kinds
    for k in ("compute", "k_adaln", "k_ln1", "k_qk", "k_v", "k_attn", "k_out", "k_ln2", "k_fc1", "k_fc2"):
        assert len(kinds[k]) == wl.num_blocks, k
    comp = {r["block"]: r for r in kinds["compute"]}
    for k, rs in kinds.items():
        if k.startswith("k_"):
            for r in rs:
                c = comp[r["block"]]
                assert c["start"] <= r["start"] <= r["end"] <= c["end"]


def test_kernel_trace_accumulates_until_read():
    wl = synth.workload("tiny")
    W = _weights(wl)
    ctx = _ctx(list(wl.blocks), 4, wl.tokens, flags=dlo.FLAG_TRACE_KERNELS)
    for b, flat in W.items():
        ctx.load_shards(b, flat)
    x, cond = synth.activations(wl.tokens, 256), synth.conditioning(256)
    per_forward = wl.num_blocks * 10  # block compute + 9 kernels
    for n in (1, 3):
        for _ in range(n):
            _run(ctx, x, cond)
        tr = ctx.trace()  # hands out and clears
        assert len(tr) == n * per_forward
        assert sum(r["kind"] == "k_fc2" for r in tr) == n * wl.num_blocks
        assert all(r["end"] >= r["start"] >= 0.0 for r in tr)
    assert ctx.trace() == []


def test_trace_kinds_keep_only_the_selected_kernel():
    """dlo_set_trace_kinds: with only the MLP-up kind selected, a traced
    forward records exactly one interval per block, of that kind, and its
    output equals the fully traced forward's; unknown kind bits are refused."""
    wl = synth.workload("tiny")
    W = _weights(wl)
    ctx = _ctx(list(wl.blocks), 4, wl.tokens, flags=dlo.FLAG_TRACE_KERNELS)
    for b, flat in W.items():
        ctx.load_shards(b, flat)
    x, cond = synth.activations(wl.tokens, 256), synth.conditioning(256)
    full = _run(ctx, x, cond)
    assert len(ctx.trace()) == wl.num_blocks * 10
    with pytest.raises(dlo.DloError) as e:
        ctx.set_trace_kinds(1 << 12)
    assert e.value.code == dlo.E_INVAL
    ctx.set_trace_kinds(1 << dlo.IV_KIND["k_fc1"])
    ctx.reserve_trace(2)
    one = _run(ctx, x, cond)
    tr = ctx.trace()
    assert [r["kind"] for r in tr] == ["k_fc1"] * wl.num_blocks
    assert sorted(r["block"] for r in tr) == list(range(wl.num_blocks))
    assert np.array_equal(one, full)
    ctx.set_trace_kinds(dlo.TRACE_KINDS_ALL)
    _run(ctx, x, cond)
    assert len(ctx.trace()) == wl.num_blocks * 10
