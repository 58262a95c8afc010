"""Pins for oracle.dit: element ops against library routines and closed
forms, the block's composition through special cases that reduce to closed
form, and a full-block cross-check against PyTorch's fp64 library ops.

The pages print no numeric example of the block math, so these pins come
from the mathematics and from library routines, not from page values."""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import synth
from oracle import dit as D
from oracle import layout as L

TINY = synth.BlockShape(64, 4, 256, 32)  # d, heads (hd 16), mlp, cond


def _flat_from(shape, overrides, seed=0, std=0.02):
    """A block's flat bf16 weight: seeded N(0, std) with some parameters
    replaced by given fp32 arrays (rounded to bf16)."""
    n = L.block_numel(shape)
    rng = np.random.default_rng(seed)
    flat = synth.bf16_bits_from_f32((rng.standard_normal(n) * std).astype(np.float32))
    tab = {p.name: p for p in L.param_table(shape)}
    for name, val in overrides.items():
        p = tab[name]
        v = np.broadcast_to(np.asarray(val, np.float32), p.shape).reshape(-1)
        flat[p.offset:p.offset + p.numel] = synth.bf16_bits_from_f32(v)
    return flat


def _bf16_round(a):
    return D.bf16_bits_to_float(synth.bf16_bits_from_f32(np.asarray(a, np.float32)))


# ---------------------------------------------------------------- element ops

def test_bf16_upcast_exact():
    vals = np.array([0.0, 1.0, -2.5, 3.140625, 1e-30, -65504.0], np.float32)
    bits = synth.bf16_bits_from_f32(vals)
    up = D.bf16_bits_to_float(bits)
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(up, ref)
    # upper-half rule on raw patterns
    assert D.bf16_bits_to_float(np.array([0x3F80, 0xC000, 0x0000, 0x8000], np.uint16)).tolist() == [1.0, -2.0, 0.0, -0.0]


def test_rne_matches_torch():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal(100000) * 0.02).astype(np.float32)
    bits = synth.bf16_bits_from_f32(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)


def test_silu_matches_library():
    z = np.linspace(-20, 20, 2001)
    assert np.allclose(D.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-15)
    assert D.silu(np.array([0.0]))[0] == 0.0


def test_gelu_tanh_matches_library_and_bounds():
    z = np.linspace(-12, 12, 4801)
    ref = F.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.allclose(D.gelu_tanh(z), ref, rtol=1e-13, atol=1e-15)
    # the tanh form stays within 5e-4 of the exact erf form
    exact = 0.5 * z * (1 + scipy.special.erf(z / np.sqrt(2)))
    assert np.max(np.abs(D.gelu_tanh(z) - exact)) < 5e-4
    assert D.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(D.gelu_tanh(np.array([1.0]))[0] - 0.8411919906082768) < 1e-12
    assert abs(D.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12
    assert abs(D.gelu_tanh(np.array([-30.0]))[0]) < 1e-12


def test_layer_norm_matches_library():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((17, 96)) * 3 + 1.5
    ref = F.layer_norm(torch.from_numpy(x), (96,), eps=1e-6).numpy()
    assert np.allclose(D.layer_norm(x), ref, rtol=1e-12, atol=1e-12)
    # a constant row normalises to exactly zero
    assert np.all(D.layer_norm(np.full((2, 8), 3.25)) == 0.0)


def _attn_loops(q, k, v, heads):
    tq, d = q.shape
    hd = d // heads
    out = np.zeros_like(q)
    for h in range(heads):
        for i in range(tq):
            s = [sum(q[i, h * hd + c] * k[j, h * hd + c] for c in range(hd)) / np.sqrt(hd)
                 for j in range(k.shape[0])]
            m = max(s)
            w = [np.exp(x - m) for x in s]
            z = sum(w)
            for c in range(hd):
                out[i, h * hd + c] = sum(w[j] * v[j, h * hd + c] for j in range(k.shape[0])) / z
    return out


def test_modulate_special_cases_and_feature_broadcast():
    """adaLN modulation h (1 + scale) + shift acts per feature: zero scale
    and shift leave h unchanged, scale -1 leaves only the shift, and on a
    non-square input each feature column gets its own pair (a row-wise
    broadcast or a swapped shift/scale fails the element loop)."""
    rng = np.random.default_rng(3)
    h = rng.standard_normal((5, 3))
    z = np.zeros(3)
    assert np.array_equal(D.modulate(h, z, z), h)
    shift = rng.standard_normal(3)
    assert np.array_equal(D.modulate(h, shift, -np.ones(3)), np.broadcast_to(shift, h.shape))
    scale = rng.standard_normal(3)
    got = D.modulate(h, shift, scale)
    for t in range(5):
        for j in range(3):
            assert got[t, j] == h[t, j] * (1.0 + scale[j]) + shift[j]


def test_attention_bruteforce_tiny():
    rng = np.random.default_rng(5)
    for tq, tk in ((1, 1), (3, 5), (8, 8)):
        q, k, v = (rng.standard_normal((t, 8)) for t in (tq, tk, tk))
        assert np.allclose(D.attention(q, k, v, 2), _attn_loops(q, k, v, 2), rtol=1e-12, atol=1e-13)


def test_attention_matches_library_sdpa():
    rng = np.random.default_rng(6)
    t, d, h = 300, 64, 4
    q, k, v = (rng.standard_normal((t, d)) * 2 for _ in range(3))
    tq = torch.from_numpy(q).view(t, h, d // h).transpose(0, 1)
    tk = torch.from_numpy(k).view(t, h, d // h).transpose(0, 1)
    tv = torch.from_numpy(v).view(t, h, d // h).transpose(0, 1)
    ref = F.scaled_dot_product_attention(tq, tk, tv).transpose(0, 1).reshape(t, d).numpy()
    assert np.allclose(D.attention(q, k, v, h, query_chunk=64), ref, rtol=1e-11, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((1, 16))
    q, k = rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    assert np.array_equal(D.attention(q, k, v, 2), v)  # one key: output is v exactly
    k = np.repeat(rng.standard_normal((1, 16)), 9, axis=0)  # identical keys: mean of v
    v = rng.standard_normal((9, 16))
    q = rng.standard_normal((4, 16))
    assert np.allclose(D.attention(q, k, v, 2), np.repeat(v.mean(0, keepdims=True), 4, 0), atol=1e-14)
    # huge scores stay finite (max subtraction)
    q = rng.standard_normal((5, 16)) * 1e3
    k = rng.standard_normal((7, 16)) * 1e3
    out = D.attention(q, k, rng.standard_normal((7, 16)), 2)
    assert np.all(np.isfinite(out))


# ---------------------------------------------------------------- composition

def _xc(shape, t=12, seed=9):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((t, shape.d_model)), rng.standard_normal(shape.d_cond)


def _ada_bias(shape, shift1=0.0, scale1=0.0, gate1=0.0, shift2=0.0, scale2=0.0, gate2=0.0):
    d = shape.d_model
    parts = [np.broadcast_to(np.asarray(v, np.float64), (d,)) for v in
             (shift1, scale1, gate1, shift2, scale2, gate2)]
    return np.concatenate(parts)


def test_adaln_zero_identity_is_exact():
    """With both gates zero the block returns x bit for bit (x + 0*anything)."""
    shp = TINY
    d = shp.d_model
    base = _flat_from(shp, {}, seed=1)
    tab = {p.name: p for p in L.param_table(shp)}
    wada = D.bf16_bits_to_float(base[tab["Wada"].offset:tab["Wada"].offset + tab["Wada"].numel]).reshape(6 * d, -1)
    bada = D.bf16_bits_to_float(base[tab["bada"].offset:tab["bada"].offset + tab["bada"].numel])
    wada[2 * d:3 * d] = 0
    wada[5 * d:6 * d] = 0
    bada[2 * d:3 * d] = 0
    bada[5 * d:6 * d] = 0
    flat = _flat_from(shp, {"Wada": wada, "bada": bada}, seed=1)
    x, c = _xc(shp)
    assert np.array_equal(D.dit_block(flat, shp, x, c), x)


def test_attention_branch_closed_form():
    """scale1 = -1 makes h = shift1 for every token, so all q, k, v rows are
    equal, attention returns the v row, and with gate1 = 1, gate2 = 0:
    x_out = x + Wo (Wv s + bv) + bo.  Pins the chunk order (shift1, scale1,
    gate1 first), the 1 + scale form and v being the third third of Wqkv."""
    shp = TINY
    d = shp.d_model
    rng = np.random.default_rng(11)
    s = _bf16_round(rng.standard_normal(d))
    flat = _flat_from(shp, {"Wada": 0.0, "bada": _ada_bias(shp, shift1=s, scale1=-1.0, gate1=1.0)}, seed=2)
    prm = D.block_params(flat, shp)
    x, c = _xc(shp)
    wv, bv = prm["Wqkv"][2 * d:], prm["bqkv"][2 * d:]
    v_row = np.einsum("oi,i->o", wv, s) + bv
    want = x + (np.einsum("oi,i->o", prm["Wo"], v_row) + prm["bo"])[None, :]
    assert np.allclose(D.dit_block(flat, shp, x, c), want, rtol=1e-12, atol=1e-12)


def test_mlp_branch_closed_form():
    """gate1 = 0, scale2 = -1, shift2 = s2, gate2 = g: every row gets
    x + g * (W2 gelu(W1 s2 + b1) + b2)."""
    shp = TINY
    d = shp.d_model
    rng = np.random.default_rng(12)
    s2 = _bf16_round(rng.standard_normal(d))
    g = _bf16_round(rng.standard_normal(d))
    flat = _flat_from(shp, {"Wada": 0.0, "bada": _ada_bias(shp, shift2=s2, scale2=-1.0, gate2=g)}, seed=3)
    prm = D.block_params(flat, shp)
    x, c = _xc(shp)
    pre = np.einsum("oi,i->o", prm["W1"], s2) + prm["b1"]
    u = 0.5 * pre * (1 + np.tanh(np.sqrt(2 / np.pi) * (pre + 0.044715 * pre ** 3)))
    want = x + g * (np.einsum("oi,i->o", prm["W2"], u) + prm["b2"])
    assert np.allclose(D.dit_block(flat, shp, x, c), want, rtol=1e-12, atol=1e-12)


def test_conditioning_path():
    """Wada = 0 except the gate1 rows, which read cond through SiLU:
    gate1 = Wg silu(c) + bg.  With the attention branch made constant
    (scale1 = -1, shift1 = 0 -> h = 0, qkv = bqkv, o = bv), the update is
    gate1 * (Wo bv + bo)."""
    shp = TINY
    d, cw = shp.d_model, shp.d_cond
    rng = np.random.default_rng(13)
    wg = _bf16_round(rng.standard_normal((d, cw)) * 0.1)
    wada = np.zeros((6 * d, cw))
    wada[2 * d:3 * d] = wg
    flat = _flat_from(shp, {"Wada": wada, "bada": _ada_bias(shp, scale1=-1.0)}, seed=4)
    prm = D.block_params(flat, shp)
    x, c = _xc(shp)
    gate1 = wg @ (c / (1 + np.exp(-c))) + prm["bada"][2 * d:3 * d]
    want = x + gate1 * (prm["Wo"] @ prm["bqkv"][2 * d:] + prm["bo"])
    assert np.allclose(D.dit_block(flat, shp, x, c), want, rtol=1e-12, atol=1e-12)


def _torch_block(flat, shp, x, c):
    """The same block assembled from PyTorch fp64 library ops."""
    prm = {k: torch.from_numpy(v) for k, v in D.block_params(flat, shp).items()}
    x, c = torch.from_numpy(x), torch.from_numpy(c)
    d, h = shp.d_model, shp.n_heads
    mod = F.linear(F.silu(c), prm["Wada"], prm["bada"]).chunk(6)
    sh1, sc1, g1, sh2, sc2, g2 = mod
    hh = F.layer_norm(x, (d,), eps=1e-6) * (1 + sc1) + sh1
    q, k, v = F.linear(hh, prm["Wqkv"], prm["bqkv"]).chunk(3, dim=-1)
    t = x.shape[0]
    sp = lambda a: a.view(t, h, d // h).transpose(0, 1)
    o = F.scaled_dot_product_attention(sp(q), sp(k), sp(v)).transpose(0, 1).reshape(t, d)
    x = x + g1 * F.linear(o, prm["Wo"], prm["bo"])
    h2 = F.layer_norm(x, (d,), eps=1e-6) * (1 + sc2) + sh2
    x = x + g2 * F.linear(F.gelu(F.linear(h2, prm["W1"], prm["b1"]), approximate="tanh"), prm["W2"], prm["b2"])
    return x.numpy()


@pytest.mark.parametrize("std", [0.02, 0.3])
def test_block_matches_library_composition(std):
    shp = TINY
    flat = _flat_from(shp, {}, seed=5, std=std)
    x, c = _xc(shp, t=33)
    assert np.allclose(D.dit_block(flat, shp, x, c), _torch_block(flat, shp, x, c), rtol=1e-11, atol=1e-11)


def test_rows_subset_equals_full():
    shp = TINY
    flat = _flat_from(shp, {}, seed=6, std=0.2)
    x, c = _xc(shp, t=40)
    full = D.dit_block(flat, shp, x, c)
    rows = [0, 7, 39, 21]
    assert np.allclose(D.dit_block(flat, shp, x, c, rows=rows), full[rows], rtol=1e-13, atol=1e-13)


def test_width_adapter_and_forward_chain():
    a = synth.BlockShape(64, 4, 128, 32)
    b = synth.BlockShape(96, 6, 192, 32)
    x = np.arange(12.0).reshape(2, 6)
    assert np.array_equal(D.width_adapter(x, 8), np.hstack([x, np.zeros((2, 2))]))
    assert np.array_equal(D.width_adapter(x, 4), x[:, :4])
    flats = [_flat_from(s, {}, seed=20 + i) for i, s in enumerate((a, b, a))]
    x0, c = _xc(a, t=5)
    y = D.dit_forward(flats, (a, b, a), x0, c)
    z = D.dit_block(flats[0], a, x0, c)
    z = D.dit_block(flats[1], b, np.hstack([z, np.zeros((5, 32))]), c)
    z = D.dit_block(flats[2], a, z[:, :64], c)
    assert np.array_equal(y, z)


def test_float32_mode_close_to_float64():
    shp = TINY
    flat = _flat_from(shp, {}, seed=8, std=0.1)
    x, c = _xc(shp, t=20)
    a = D.dit_block(flat, shp, x, c, dtype=np.float64)
    b = D.dit_block(flat, shp, x, c, dtype=np.float32)
    assert b.dtype == np.float32
    assert np.allclose(a, b, rtol=1e-4, atol=1e-4)
