"""The DiT block and the chained forward, all weights resident (oracle).

The offload method changes where weights live and when they move, never a
value: reconstruction is a bit copy and the two-slot schedule only reorders
transfers.  So the oracle of the streamed forward is the plain forward with
every block's weights resident on the host.

The pages name the model family (Diffusion Transformer) and its block counts
but not the block internals.  The reading taken here is the standard DiT
block with adaLN-Zero conditioning (Peebles & Xie, "Scalable Diffusion Models
with Transformers", 2023, section 3.2 and figure 3), with these choices where
that paper leaves details to code:

* conditioning: mod = Wada @ silu(cond) + bada, split into six d-wide chunks
  in the order shift1, scale1, gate1, shift2, scale2, gate2;
* LayerNorm without affine parameters, eps = 1e-6, population variance;
* modulation h = LN(x) * (1 + scale) + shift;
* attention: non-causal multi-head softmax(q k^T / sqrt(hd)) v, q/k/v packed
  as rows [0,d), [d,2d), [2d,3d) of Wqkv, head j on columns [j*hd, (j+1)*hd);
  no mask, no positional rotation, no QK normalisation;
* MLP: GELU with the tanh approximation between W1 and W2;
* residual updates gated per feature: x += gate * branch(x).

Arithmetic runs in ``dtype`` (float64 by default) with no intermediate bf16
rounding; the bf16 weights are upcast exactly.  Between blocks of different
width (irregular workload) the residual keeps its first min(d_in, d_out)
features and zero-fills the rest.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .layout import param_table

LN_EPS = 1e-6


def bf16_bits_to_float(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to ``dtype``: a bf16 value
    is the upper half of the fp32 value with the same bits."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(dtype)


def block_params(flat_bits: np.ndarray, shape, dtype=np.float64) -> Dict[str, np.ndarray]:
    """Parameter views of one block, each upcast from its slice of the flat
    bf16 weight at the layout's offset."""
    flat_bits = np.asarray(flat_bits, dtype=np.uint16)
    out = {}
    for p in param_table(shape):
        out[p.name] = bf16_bits_to_float(flat_bits[p.offset:p.offset + p.numel], dtype).reshape(p.shape)
    return out


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    t = z.dtype.type
    c = t(np.sqrt(2.0 / np.pi))
    return t(0.5) * z * (t(1.0) + np.tanh(c * (z + t(0.044715) * z ** 3)))


def layer_norm(x: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + x.dtype.type(eps))


def modulate(h: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return h * (1.0 + scale) + shift


def adaln(params: Dict[str, np.ndarray], cond: np.ndarray):
    """The six modulation vectors (shift1, scale1, gate1, shift2, scale2, gate2)."""
    mod = params["Wada"] @ silu(cond) + params["bada"]
    return np.split(mod, 6)


def softmax(s: np.ndarray) -> np.ndarray:
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int,
              query_chunk: int = 1024) -> np.ndarray:
    """Non-causal multi-head attention.  q: [Tq, d], k, v: [Tk, d]; returns
    [Tq, d].  Query rows are independent, so they are processed in chunks to
    bound the size of the score matrix."""
    tq, d = q.shape
    hd = d // n_heads
    out = np.empty((tq, d), dtype=q.dtype)
    scale = q.dtype.type(1.0 / np.sqrt(hd))
    for j in range(n_heads):
        cols = slice(j * hd, (j + 1) * hd)
        kj, vj = k[:, cols], v[:, cols]
        for r0 in range(0, tq, query_chunk):
            qj = q[r0:r0 + query_chunk, cols]
            p = softmax((qj @ kj.T) * scale)
            out[r0:r0 + query_chunk, cols] = p @ vj
    return out


def dit_block(flat_bits: np.ndarray, shape, x: np.ndarray, cond: np.ndarray,
              rows: Optional[Sequence[int]] = None, dtype=np.float64) -> np.ndarray:
    """One DiT block applied to x [T, d]; returns the new x.

    If ``rows`` is given, only those output rows are computed (keys and values
    still come from every token), and the result has len(rows) rows."""
    prm = block_params(flat_bits, shape, dtype)
    d = shape.d_model
    x = np.asarray(x, dtype=dtype)
    cond = np.asarray(cond, dtype=dtype)
    if x.ndim != 2 or x.shape[1] != d:
        raise ValueError(f"x must be [T, {d}]")
    shift1, scale1, gate1, shift2, scale2, gate2 = adaln(prm, cond)

    h = modulate(layer_norm(x), shift1, scale1)
    wq, wk, wv = prm["Wqkv"][0:d], prm["Wqkv"][d:2 * d], prm["Wqkv"][2 * d:3 * d]
    bq, bk, bv = prm["bqkv"][0:d], prm["bqkv"][d:2 * d], prm["bqkv"][2 * d:3 * d]
    k = h @ wk.T + bk
    v = h @ wv.T + bv
    if rows is None:
        xr, hr = x, h
    else:
        idx = np.asarray(rows, dtype=np.int64)
        xr, hr = x[idx], h[idx]
    q = hr @ wq.T + bq
    o = attention(q, k, v, shape.n_heads)
    xr = xr + gate1 * (o @ prm["Wo"].T + prm["bo"])

    h2 = modulate(layer_norm(xr), shift2, scale2)
    u = gelu_tanh(h2 @ prm["W1"].T + prm["b1"])
    xr = xr + gate2 * (u @ prm["W2"].T + prm["b2"])
    return xr


def width_adapter(x: np.ndarray, d_out: int) -> np.ndarray:
    """Residual handed from a block of width d_in to one of width d_out: the
    first min(d_in, d_out) features are kept, the rest are zero."""
    t, d_in = x.shape
    out = np.zeros((t, d_out), dtype=x.dtype)
    n = min(d_in, d_out)
    out[:, :n] = x[:, :n]
    return out


def dit_forward(flat_bits_per_block: Sequence[np.ndarray], shapes: Sequence, x: np.ndarray,
                cond: np.ndarray, dtype=np.float64) -> np.ndarray:
    """The chained forward over all blocks in order, every weight resident."""
    if len(flat_bits_per_block) != len(shapes):
        raise ValueError("one flat weight per block is required")
    x = np.asarray(x, dtype=dtype)
    for flat, shp in zip(flat_bits_per_block, shapes):
        if x.shape[1] != shp.d_model:
            x = width_adapter(x, shp.d_model)
        x = dit_block(flat, shp, x, cond, dtype=dtype)
    return x
