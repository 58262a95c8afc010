"""Each kernel against the oracle's definition of its step, on seeded inputs
that span several tiles and a ragged tail.  Calls go through the C ABI."""
import numpy as np
import pytest

import synth
from oracle import dit as D, shard as OS
from gpu_util import assert_reconstructed, dev, host, within, torch

pytestmark = pytest.mark.gpu

import layerwise_weight_streaming_dit_amd as dlo


def _bf16(a):
    return synth.bf16_bits_from_f32(np.asarray(a, np.float32))


def _w(a):
    """A parameter as the kernels read it from the slot: drawn as bf16 (as
    streamed), converted to fp16 patterns the way the reconstruction does."""
    return OS.as_f16_bits(_bf16(a))


def _f16(a):
    """fp16 bit patterns (activations between kernels are fp16)."""
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def f16_to_f64(bits):
    return np.ascontiguousarray(bits, np.uint16).view(np.float16).astype(np.float64)


def vt_position(j):
    """Documented layout of the transposed v buffer (include/dlo_ops.h):
    token j sits at column j with bits 2 and 3 swapped."""
    j = np.asarray(j)
    return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1)


# ------------------------------------------------------------- reconstruction

@pytest.mark.parametrize("n", [1, 7, 8, 9, 4095, 65536 + 13, (1 << 21) + 5])
@pytest.mark.parametrize("dst_off,src_off", [(0, 0), (3, 3), (5, 5), (1, 6), (7, 0)])
def test_assemble_bit_exact(n, dst_off, src_off):
    rng = np.random.default_rng(n + 31 * dst_off + src_off)
    src = rng.integers(0, 1 << 16, size=n + 16, dtype=np.uint16)
    t = torch()
    s = dev(src)
    d = t.full((n + 16,), -1, dtype=t.int16, device="cuda")
    dlo.op_assemble(d[dst_off:], s[src_off:], n)
    t.cuda.synchronize()
    out = host(d, np.uint16)
    assert_reconstructed(out[dst_off:dst_off + n], src[src_off:src_off + n])
    assert np.all(out[:dst_off] == 0xFFFF) and np.all(out[dst_off + n:] == 0xFFFF)


# ------------------------------------------------------------------- adaLN

@pytest.mark.parametrize("d,c", [(256, 256), (2048, 256), (3072, 64)])
def test_adaln(d, c):
    rng = np.random.default_rng(d + c)
    w = _w(rng.standard_normal((6 * d, c)) * 0.02)
    b = _w(rng.standard_normal(6 * d) * 0.02)
    cond = rng.standard_normal(c).astype(np.float32)
    t = torch()
    mod = t.empty(6 * d, dtype=t.float32, device="cuda")
    dlo.op_adaln(dev(w), dev(b), dev(cond), mod, 6 * d, c)
    want = f16_to_f64(w).reshape(6 * d, c) @ D.silu(cond.astype(np.float64)) + f16_to_f64(b)
    ok, ma, mr = within(host(mod), want, rtol=1e-4, atol=1e-5)
    assert ok, (ma, mr)


@pytest.mark.parametrize("rows,c", [(1, 64), (17, 320), (1003, 4096), (4099, 256)])
def test_adaln_ragged_rows(rows, c):
    # row counts that leave a workgroup's last rows empty (16 rows per
    # workgroup, 4 per wave) and widths from one lane group to the LDS limit
    rng = np.random.default_rng(rows * 7 + c)
    w = _w(rng.standard_normal((rows, c)) * 0.02)
    b = _w(rng.standard_normal(rows) * 0.02)
    cond = rng.standard_normal(c).astype(np.float32)
    mod = dev(np.full(rows + 16, np.nan, np.float32))
    dlo.op_adaln(dev(w), dev(b), dev(cond), mod, rows, c)
    got = host(mod)
    want = f16_to_f64(w).reshape(rows, c) @ D.silu(cond.astype(np.float64)) + f16_to_f64(b)
    ok, ma, mr = within(got[:rows], want, rtol=1e-4, atol=1e-5)
    assert ok, (ma, mr)
    assert np.all(np.isnan(got[rows:])), "wrote past the last row"


# ------------------------------------------------------- LayerNorm + modulate

@pytest.mark.parametrize("tokens,d_in,d", [(1, 256, 256), (37, 2048, 2048), (300, 3072, 4096),
                                           (65, 4096, 3072), (8, 8192, 8192), (5, 8, 4), (17, 1000, 1024),
                                           (6, 516, 500), (3, 4100, 6000), (2, 6000, 4100),
                                           (129, 5120, 5120), (5, 6144, 6144), (3, 6148, 6148)])
def test_ln_modulate(tokens, d_in, d):
    rng = np.random.default_rng(tokens * d)
    x = (rng.standard_normal((tokens, d_in)) * 2 + 0.5).astype(np.float32)
    shift = rng.standard_normal(d).astype(np.float32) * 0.3
    scale = rng.standard_normal(d).astype(np.float32) * 0.3
    t = torch()
    h = t.empty((tokens, d), dtype=t.int16, device="cuda")
    xo = t.full((tokens, d), float("nan"), dtype=t.float32, device="cuda") if d_in != d else None
    dlo.op_ln_modulate(dev(x), d_in, xo, dev(shift), dev(scale), h, tokens, d)
    y = D.width_adapter(x.astype(np.float64), d)
    want = D.modulate(D.layer_norm(y), shift.astype(np.float64), scale.astype(np.float64))
    ok, ma, mr = within(f16_to_f64(host(h, np.uint16)), want, rtol=2e-3, atol=2e-4)
    assert ok, (ma, mr)
    if xo is not None:
        assert np.array_equal(host(xo), y.astype(np.float32))


# --------------------------------------------------------------------- GEMM

_POISON = 0x7FFF  # NaN as fp16 and as bf16
_SENTINEL_F16, _SENTINEL_F32 = 0x1234, 12345.0


def _padded(rows_bits, ld):
    """rows_bits (uint16 [rows][cols]) in a [rows][ld] buffer whose padding is NaN."""
    buf = np.full((rows_bits.shape[0], ld), _POISON, np.uint16)
    buf[:, : rows_bits.shape[1]] = rows_bits
    return buf


def _gemm_case(epi, M, N, K, w_rows=None, seed=0, pad=None):
    """One GEMM through the C ABI; `a` is the fp16 activation and `w` the
    weight (bf16 draws as the slot holds them, fp16), except for the
    transposed-v epilogue where the roles swap.
    pad = (extra lda, extra ldw, extra ldo): the operands' row padding holds
    NaN (a read of it would poison the result) and the output's a sentinel
    that must survive."""
    rng = np.random.default_rng(seed)
    pa, pw, po = pad or (0, 0, 0)
    w_rows = N if w_rows is None else w_rows
    vt = epi == dlo.EPI_VT_F16
    a_val = rng.standard_normal((M, K)) * (0.02 if vt else 1.0)
    w_val = rng.standard_normal((w_rows, K)) * (1.0 if vt else 0.02)
    a = _w(a_val) if vt else _f16(a_val)
    w = _f16(w_val) if vt else _w(w_val)
    nb = M if vt else N
    bias = _w(rng.standard_normal(nb) * 0.1)
    gate = rng.standard_normal(N).astype(np.float32)
    x0 = rng.standard_normal((M, N)).astype(np.float32)
    if epi == dlo.EPI_GATED_F32:
        out_h = np.full((M, N + po), _SENTINEL_F32, np.float32)
        out_h[:, :N] = x0
    else:
        out_h = np.full((M, N + po), _SENTINEL_F16, np.uint16)
    out = dev(out_h)
    dlo.op_gemm(epi, dev(_padded(a, K + pa)), K + pa, dev(_padded(w, K + pw)), K + pw, w_rows, dev(bias),
                dev(gate), out, N + po, M, N, K)
    if po:
        got_all = host(out) if epi == dlo.EPI_GATED_F32 else host(out, np.uint16)
        assert np.array_equal(got_all[:, N:], out_h[:, N:]), "output padding was written"
        out = out[:, :N]
    wfull = f16_to_f64(w)[np.minimum(np.arange(N), w_rows - 1)]
    acc = f16_to_f64(a) @ wfull.T
    bf = f16_to_f64(bias)
    if epi == dlo.EPI_BIAS_F16:
        return f16_to_f64(host(out, np.uint16)), acc + bf
    if epi == dlo.EPI_BIAS_GELU_F16:
        return f16_to_f64(host(out, np.uint16)), D.gelu_tanh(acc + bf)
    if epi == dlo.EPI_GATED_F32:
        return host(out).astype(np.float64), x0 + gate.astype(np.float64) * (acc + bf)
    got = f16_to_f64(host(out, np.uint16))
    return got[:, vt_position(np.arange(N))], acc + bf[:, None]


@pytest.mark.parametrize("epi", [dlo.EPI_BIAS_F16, dlo.EPI_BIAS_GELU_F16, dlo.EPI_GATED_F32, dlo.EPI_VT_F16])
@pytest.mark.parametrize("M,N,K", [(256, 768, 256), (300, 256, 1024), (1000, 512, 512), (4096 + 17, 2048, 256),
                                   (33, 128, 128), (1, 16, 128), (700, 1040, 384)])
def test_gemm(epi, M, N, K):
    got, want = _gemm_case(epi, M, N, K, seed=M + N + K + epi)
    ok, ma, mr = within(got, want, rtol=2e-3, atol=2e-3)
    assert ok, (ma, mr)


def test_gemm_clamped_w_rows():
    # the transposed v projection: output columns past w_rows repeat the last row
    got, want = _gemm_case(dlo.EPI_VT_F16, 512, 1088, 256, w_rows=1000, seed=5)
    ok, ma, mr = within(got, want, rtol=2e-3, atol=2e-3)
    assert ok, (ma, mr)


@pytest.mark.parametrize("epi", [dlo.EPI_BIAS_F16, dlo.EPI_BIAS_GELU_F16, dlo.EPI_GATED_F32, dlo.EPI_VT_F16])
@pytest.mark.parametrize("M,N,K", [(300, 272, 256), (4096 + 40, 2048, 4096)])
def test_gemm_strided_operands(epi, M, N, K):
    # row strides past the logical extents: lda = K + 8, ldw = K + 24 and
    # ldo = N + 8 (N + 4 for fp32 rows); the second shape takes the 256x128
    # tiles with the L2 prefetch and a ragged last tile row
    po = 4 if epi == dlo.EPI_GATED_F32 else 8
    got, want = _gemm_case(epi, M, N, K, seed=M + K + epi, pad=(8, 24, po))
    ok, ma, mr = within(got, want, rtol=2e-3, atol=2e-3)
    assert ok, (ma, mr)


def test_gemm_epilogue_rounding_is_rne_exact():
    """A one-hot A makes acc = w[j][i] exactly (the bf16 weights convert to
    fp16 exactly); with bias of similar magnitude acc + bias is exact in
    fp32, so the fp16 output must be the round-to-nearest-even of that sum,
    bit for bit (ties included)."""
    rng = np.random.default_rng(77)
    M, N, K = 128, 256, 128
    a = np.zeros((M, K), np.float32)
    a[np.arange(M), np.arange(M) % K] = 1.0
    # w and bias: bf16 values whose fp32 sum has bits below bf16 precision,
    # including values exactly halfway between two fp16 numbers
    w = _w((rng.integers(-256, 256, size=(N, K)) / 64.0).astype(np.float32))
    # bias: +-(1 + m/128) * 2^e, e in [-8, -5] -- exact bf16, so every fp32
    # sum w + bias spans at most 17 significant bits (exact)
    mant = 1.0 + rng.integers(0, 128, size=N) / 128.0
    bias = _w((rng.choice([-1.0, 1.0], size=N) * mant * 2.0 ** rng.integers(-8, -4, size=N)).astype(np.float32))
    t = torch()
    out = t.empty((M, N), dtype=t.int16, device="cuda")
    dlo.op_gemm(dlo.EPI_BIAS_F16, dev(_f16(a)), K, dev(w), K, N, dev(bias), None, out, N, M, N, K)
    acc = f16_to_f64(w)[:, np.arange(M) % K].T.astype(np.float32)
    exact = acc + f16_to_f64(bias).astype(np.float32)[None, :]
    assert np.all(exact.astype(np.float64) == f16_to_f64(w)[:, np.arange(M) % K].T + f16_to_f64(bias)[None, :])
    want = exact.astype(np.float16).view(np.uint16)  # numpy rounds half to even
    ties = (exact.view(np.uint32) & 0x1FFF) == 0x1000  # halfway between two fp16 values
    assert np.any(ties)
    assert np.array_equal(host(out, np.uint16), want)


def test_gemm_large_tile_shapes():
    # 256x256 tiles (at least 256 of them); (4096, 2048, 512) has 128 such
    # tiles and a short K, so it takes two 128x128 tiles per CU
    for (M, N, K) in [(4096, 4096, 512), (4096, 2048, 512)]:
        got, want = _gemm_case(dlo.EPI_BIAS_F16, M, N, K, seed=M + N)
        ok, ma, mr = within(got, want, rtol=2e-3, atol=2e-3)
        assert ok, (M, N, K, ma, mr)


@pytest.mark.parametrize("epi,M,N,K", [(dlo.EPI_BIAS_F16, 4000, 2048, 4096), (dlo.EPI_GATED_F32, 4000, 2048, 4096),
                                         (dlo.EPI_VT_F16, 4000, 2048, 4096), (dlo.EPI_BIAS_GELU_F16, 4000, 2048, 4096),
                                         (dlo.EPI_GATED_F32, 4000, 2000, 4096), (dlo.EPI_BIAS_F16, 4000, 2000, 4096),
                                         (dlo.EPI_BIAS_F16, 4096 + 17, 4096, 1024),
                                         (dlo.EPI_GATED_F32, 4096 + 17, 4096, 1024),
                                         (dlo.EPI_BIAS_GELU_F16, 4096 + 17, 4096 - 48, 1024),
                                         (dlo.EPI_VT_F16, 4096 + 128, 4096 - 64, 1024),
                                         (dlo.EPI_BIAS_F16, 8192 + 17, 8192 - 48, 512),
                                         (dlo.EPI_BIAS_GELU_F16, 8192 + 17, 8192, 384),
                                         (dlo.EPI_GATED_F32, 8192 + 17, 8192 - 48, 512),
                                         (dlo.EPI_VT_F16, 8192 + 128, 8192 - 64, 512)])
def test_gemm_long_k_and_ragged_large_tiles(epi, M, N, K):
    """The 256x128 tile (K >= 4096 with fewer than 256 tiles of 256x256: the
    MLP-down shape class, and the transposed v projection of a d = 4096 block
    at T <= 2048) and the one-wave-per-SIMD 256x256 tile (256 tiles and
    more), with a ragged last tile row and column, every epilogue, checked on
    sampled rows (every row of the last, partial tile row included) against
    fp64 products."""
    rng = np.random.default_rng(M + N + K + epi)
    vt = epi == dlo.EPI_VT_F16
    w_rows = N - 77 if vt else N  # transposed v: columns past the last token repeat it
    a = _w(rng.standard_normal((M, K)) * 0.02) if vt else _f16(rng.standard_normal((M, K)))
    w = _f16(rng.standard_normal((w_rows, K))) if vt else _w(rng.standard_normal((N, K)) * 0.02)
    bias = _w(rng.standard_normal(M if vt else N) * 0.1)
    gate = rng.standard_normal(N).astype(np.float32)
    x0 = rng.standard_normal((M, N)).astype(np.float32)
    t = torch()
    out = dev(x0.copy()) if epi == dlo.EPI_GATED_F32 else t.empty((M, N), dtype=t.int16, device="cuda")
    dlo.op_gemm(epi, dev(a), K, dev(w), K, w_rows, dev(bias), dev(gate), out, N, M, N, K)
    rows = np.unique(np.concatenate([rng.choice(M, 48, replace=False), np.arange(M // 256 * 256, M)]))
    if vt:
        wf = f16_to_f64(w).reshape(w_rows, K)[np.minimum(np.arange(N), w_rows - 1)]
        acc = f16_to_f64(a[rows]).reshape(len(rows), K) @ wf.T + f16_to_f64(bias)[rows][:, None]
        got = f16_to_f64(host(out, np.uint16))[rows][:, vt_position(np.arange(N))]
        want = acc
    else:
        acc = f16_to_f64(a[rows]) @ f16_to_f64(w).reshape(N, K).T + f16_to_f64(bias)
        if epi == dlo.EPI_GATED_F32:
            got = host(out).astype(np.float64)[rows]
            want = x0[rows].astype(np.float64) + gate.astype(np.float64) * acc
        elif epi == dlo.EPI_BIAS_GELU_F16:
            got = f16_to_f64(host(out, np.uint16))[rows]
            want = D.gelu_tanh(acc)
        else:
            got = f16_to_f64(host(out, np.uint16))[rows]
            want = acc
    ok, ma, mr = within(got, want, rtol=2e-3, atol=2e-3)
    assert ok, (M, N, K, ma, mr)


# ---------------------------------------------------------------- attention

def _attention_case(T, H, hd, qscale=1.0, seed=0):
    rng = np.random.default_rng(seed)
    d = H * hd
    q = _f16(rng.standard_normal((T, d)) * qscale)
    k = _f16(rng.standard_normal((T, d)))
    v = _f16(rng.standard_normal((T, d)))
    tp = (T + 63) // 64 * 64
    vt = np.zeros((d, tp), np.uint16)
    vt[:, vt_position(np.arange(T))] = v.T
    qk = np.concatenate([q, k], axis=1)
    t = torch()
    o = t.empty((T, d), dtype=t.int16, device="cuda")
    dlo.op_attention(dev(qk), 2 * d, dev(vt), tp, o, d, T, H, hd)
    want = D.attention(f16_to_f64(q), f16_to_f64(k), f16_to_f64(v), H)
    return f16_to_f64(host(o, np.uint16)), want


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 129, 200, 1000])
@pytest.mark.parametrize("H,hd", [(2, 64), (2, 128)])
def test_attention(T, H, hd):
    got, want = _attention_case(T, H, hd, seed=T * hd)
    ok, ma, mr = within(got, want, rtol=5e-3, atol=5e-3)
    assert ok, (ma, mr)


@pytest.mark.parametrize("T", [65, 1000])
@pytest.mark.parametrize("H,hd", [(8, 64), (16, 128)])
def test_attention_heads_per_xcd(T, H, hd):
    # head counts divisible by 8 take the grid mapping that keeps each head's
    # query tiles on one XCD
    got, want = _attention_case(T, H, hd, seed=T + H)
    ok, ma, mr = within(got, want, rtol=5e-3, atol=5e-3)
    assert ok, (ma, mr)


@pytest.mark.parametrize("T,H,hd", [(4096, 20, 64), (2048 + 33, 32, 128)])
def test_attention_full_grid_sampled_queries(T, H, hd):
    """Sequences long enough for 256-query tiles (one workgroup per CU),
    with a head count that is not a multiple of 8 (plain grid order) and one
    that is (heads kept on one XCD), ragged last key tile included; checked
    on sampled query rows against fp64 softmax attention over all keys."""
    rng = np.random.default_rng(T + H + hd)
    d = H * hd
    q = _f16(rng.standard_normal((T, d)))
    k = _f16(rng.standard_normal((T, d)))
    v = _f16(rng.standard_normal((T, d)))
    tp = (T + 63) // 64 * 64
    vt = np.zeros((d, tp), np.uint16)
    vt[:, vt_position(np.arange(T))] = v.T
    t = torch()
    o = t.empty((T, d), dtype=t.int16, device="cuda")
    dlo.op_attention(dev(np.concatenate([q, k], axis=1)), 2 * d, dev(vt), tp, o, d, T, H, hd)
    got = f16_to_f64(host(o, np.uint16))
    rows = np.unique(np.concatenate([rng.choice(T, 24, replace=False), [0, T - 1]]))
    # the oracle's attention on the sampled query rows against every key
    want = D.attention(f16_to_f64(q)[rows], f16_to_f64(k), f16_to_f64(v), H)
    ok, ma, mr = within(got[rows], want, rtol=5e-3, atol=5e-3)
    assert ok, (T, H, hd, ma, mr)


@pytest.mark.parametrize("qscale", [4.0, 30.0])
def test_attention_peaked_softmax(qscale):
    got, want = _attention_case(300, 2, 128, qscale=qscale, seed=7)
    ok, ma, mr = within(got, want)
    assert ok, (ma, mr)
