"""Full-size parity and invariants at the larger workloads: the mid video
shape, the large video shape and the irregular stress workload (two widths,
odd element counts, dp 3 and 8, per-request token counts).  Outputs the
oracle cannot afford in full are compared on sampled rows (keys and values
still come from every token)."""
import numpy as np
import pytest

import synth
from oracle import dit as D, layout as OL, shard as OS
from gpu_util import assert_reconstructed, run_forward, sample_rows, within

pytestmark = pytest.mark.gpu

import layerwise_weight_streaming_dit_amd as dlo


def _block_check(wl, b, T, dp, rows=40, flags=0):
    shp = wl.blocks[b]
    flat = synth.block_weights(wl.wid, b, OL.block_numel(shp))
    x = synth.activations(T, shp.d_model)
    cond = synth.conditioning(shp.d_cond)
    ctx = dlo.StreamedDiT([shp], dp, T, flags=flags)
    ctx.load_shards(0, flat)
    assert_reconstructed(ctx.debug_assemble(0), flat)
    got = run_forward(ctx, x, cond)
    ctx.close()
    idx = sample_rows(T, rows, b + T)
    want = D.dit_block(flat, shp, x, cond, rows=idx)
    ok, ma, mr = within(got[idx], want)
    print(f"{wl.name} block {b} T={T} dp={dp}: max_abs {ma:.3e} max_rel {mr:.3e}")
    assert ok, (ma, mr)
    return got


def test_midvideo_block_full_size():
    wl = synth.workload("midvideo")
    _block_check(wl, 0, wl.tokens, 4)


def test_large_block_full_size():
    wl = synth.workload("large")
    _block_check(wl, 79, wl.tokens, 4, rows=24)


@pytest.mark.parametrize("b,dp", [(0, 3), (1, 8)])
def test_irregular_block_at_max_tokens(b, dp):
    wl = synth.workload("irregular")
    _block_check(wl, b, wl.tokens, dp)


def test_irregular_outputs_independent_of_dp():
    wl = synth.workload("irregular")
    shp = wl.blocks[1]
    flat = synth.block_weights(wl.wid, 1, OL.block_numel(shp))
    x = synth.activations(1000, shp.d_model)
    cond = synth.conditioning(256)
    outs = []
    for dp in (1, 3, 8):
        ctx = dlo.StreamedDiT([shp], dp, 1000)
        ctx.load_shards(0, flat)
        for r in range(dp):
            assert np.array_equal(ctx.get_shard(0, r), OS.shard(flat, dp)[r])
        outs.append(run_forward(ctx, x, cond))
        ctx.close()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("dp", [3, 8])
def test_irregular_chain_with_width_changes(dp):
    """Four blocks 3072 -> 4096 -> 3072 -> 4096 at a ragged token count:
    the residual is zero-filled / truncated between widths."""
    wl = synth.workload("irregular")
    shapes = list(wl.blocks[:4])
    W = [synth.block_weights(wl.wid, b, OL.block_numel(s)) for b, s in enumerate(shapes)]
    T = 203
    x = synth.activations(T, 3072)
    cond = synth.conditioning(256)
    ctx = dlo.StreamedDiT(shapes, dp, 512)
    for b in range(4):
        ctx.load_shards(b, W[b])
    got = run_forward(ctx, x, cond)
    want = D.dit_forward(W, shapes, x, cond)
    ok, ma, mr = within(got, want)
    print(f"irregular chain dp={dp}: max_abs {ma:.3e}")
    assert ok, (ma, mr)
    # an odd number of width changes leaves the result at width 3072
    ctx3 = dlo.StreamedDiT(shapes[:3], dp, 512)
    for b in range(3):
        ctx3.load_shards(b, W[b])
    got3 = run_forward(ctx3, x, cond)
    assert got3.shape == (T, 3072)
    ok, ma, mr = within(got3, D.dit_forward(W[:3], shapes[:3], x, cond))
    assert ok, (ma, mr)


def test_irregular_sequential_requests():
    """The 24-block irregular model serves four requests with drawn token
    counts in sequence; each result equals that request run alone in a fresh
    context (bit for bit), and the first block of each request matches the
    oracle on sampled rows."""
    wl = synth.workload("irregular")
    shapes = list(wl.blocks)
    numels = [OL.block_numel(s) for s in shapes]
    W = synth.many_block_weights(wl.wid, numels)
    Ts = synth.request_tokens()
    cond = synth.conditioning(256)
    ctx = dlo.StreamedDiT(shapes, 3, max(Ts))
    for b in range(len(shapes)):
        ctx.load_shards(b, W[b])
    outs = [run_forward(ctx, synth.activations(T, 3072, seed=100 + i), cond) for i, T in enumerate(Ts)]
    ctx.close()
    for o, T in zip(outs, Ts):
        assert o.shape == (T, 4096) and np.all(np.isfinite(o))
    alone = dlo.StreamedDiT(shapes, 3, Ts[2])
    for b in range(len(shapes)):
        alone.load_shards(b, W[b])
    assert np.array_equal(run_forward(alone, synth.activations(Ts[2], 3072, seed=102), cond), outs[2])
    alone.close()
    one = dlo.StreamedDiT(shapes[:1], 3, max(Ts))
    one.load_shards(0, W[0])
    for i, T in enumerate(Ts):
        x = synth.activations(T, 3072, seed=100 + i)
        got = run_forward(one, x, cond)
        idx = sample_rows(T, 16, i)
        ok, ma, mr = within(got[idx], D.dit_block(W[0], shapes[0], x, cond, rows=idx))
        assert ok, (T, ma, mr)
