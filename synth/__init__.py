"""Seeded synthetic inputs for the streamed DiT forward.

This module is shared by the oracle's tests and by the GPU path's tests and
benchmark.  It holds only *inputs*: the five workload shapes, the weight,
activation and conditioning generators, and the per-request token draws.  It
contains none of the method's arithmetic (no parameter layout, no sharding, no
block math); callers pass in the element count a block's flat weight has, as
computed by whichever side (oracle or library) is under test.

Input recipe (the pages run real checkpoints -- Cosmos3-Nano/Super, 72 and 128
blocks, BF16 -- which are not available here, so seeded synthetic tensors of the
same kind stand in for them; vLLM-Omni DLO page, "Models and benchmark
artefacts" in the references section):

* weights: one flat draw per (workload, block) of N(0, 1) in fp32 from numpy's
  PCG64 with seed ``1000 * workload_id + block``, times 0.02, then rounded to
  bf16 with round-to-nearest-even.  Biases are drawn the same way.
* x: N(0, 1) fp32 of shape [tokens, d], seed 7.
* cond: N(0, 1) fp32 of shape [d_cond], seed 11.
* irregular workload: per-request token counts uniform over [1000, 12000],
  seed 2026, four sequential requests.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "BlockShape",
    "Workload",
    "WORKLOADS",
    "workload",
    "weight_seed",
    "bf16_bits_from_f32",
    "block_weights",
    "many_block_weights",
    "iter_block_weights",
    "activations",
    "conditioning",
    "request_tokens",
]


@dataclasses.dataclass(frozen=True)
class BlockShape:
    """Shape of one DiT block: width, heads, MLP width, conditioning width and
    the lengths of extra vectors appended to the block's flat weight (carried
    through streaming and reconstruction but not read by the block math)."""

    d_model: int
    n_heads: int
    d_mlp: int
    d_cond: int = 256
    extra: Tuple[int, ...] = ()

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int  # seed namespace: weights use 1000 * wid + block
    name: str
    blocks: Tuple[BlockShape, ...]
    tokens: int  # token count of the single request (max for "irregular")
    dp_sizes: Tuple[int, ...]
    description: str

    @property
    def num_blocks(self) -> int:
        return len(self.blocks)


def _uniform(n: int, shape: BlockShape) -> Tuple[BlockShape, ...]:
    return tuple(shape for _ in range(n))


_ODD_EXTRAS = (1, 3, 5, 7, 9, 11, 13)
_IRREG_A = BlockShape(3072, 24, 12288, 256, _ODD_EXTRAS)
_IRREG_B = BlockShape(4096, 32, 16384, 256, _ODD_EXTRAS)

WORKLOADS = {
    "tiny": Workload(
        1, "tiny", _uniform(4, BlockShape(256, 4, 1024)), 256, (4,),
        "Tiny DiT: 4 blocks, d=256, 4 heads (hd 64), MLP 1024, 256 tokens, dp 4"),
    "image": Workload(
        2, "image", _uniform(28, BlockShape(2048, 16, 8192)), 4096, (4,),
        "Image-DiT shape: 28 blocks, d=2048, 16 heads, MLP 8192, 4096 tokens, dp 4"),
    "midvideo": Workload(
        3, "midvideo", _uniform(40, BlockShape(5120, 40, 20480)), 16384, (4,),
        "Mid video-DiT shape: 40 blocks, d=5120, 40 heads, MLP 20480, 16384 tokens, dp 4"),
    "large": Workload(
        4, "large", _uniform(80, BlockShape(8192, 64, 32768)), 8192, (4,),
        "Large video-DiT shape: 80 blocks, d=8192, 64 heads, MLP 32768, 8192 tokens, dp 4"),
    "irregular": Workload(
        5, "irregular", tuple(_IRREG_A if b % 2 == 0 else _IRREG_B for b in range(24)),
        12000, (3, 8),
        "Irregular stress: 24 blocks alternating d=3072/4096, 7 odd-length extra "
        "vectors per block, tokens U[1000,12000] per request, dp 3 or 8"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def weight_seed(wid: int, block: int) -> int:
    return 1000 * wid + block


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round-to-nearest-even.  Inputs here
    are finite draws, so no NaN special case is needed."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


_SLICE = 1 << 24  # draws converted per pass (bounds the fp32 temporaries)


def block_weights(wid: int, block: int, numel: int, std: float = 0.02) -> np.ndarray:
    """The flat bf16 weight of one block as uint16 bit patterns, N(0, std).
    Drawn and rounded slice by slice: the generator's stream continues across
    calls, so the result is the same as one draw of `numel` values, without
    a full-size fp32 copy in memory."""
    g = np.random.Generator(np.random.PCG64(weight_seed(wid, block)))
    n = int(numel)
    out = np.empty(n, dtype=np.uint16)
    for i in range(0, n, _SLICE):
        a = g.standard_normal(min(_SLICE, n - i), dtype=np.float32)
        a *= np.float32(std)
        out[i:i + a.size] = bf16_bits_from_f32(a)
    return out


def many_block_weights(wid: int, numels: Sequence[int], blocks: Optional[Sequence[int]] = None,
                       threads: int = 8) -> List[np.ndarray]:
    """block_weights for several blocks, drawn in parallel threads (numpy's
    generators release the GIL while filling)."""
    if blocks is None:
        blocks = range(len(numels))
    blocks = list(blocks)
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return list(ex.map(lambda bn: block_weights(wid, bn[0], bn[1]), zip(blocks, numels)))


def iter_block_weights(wid: int, numels: Sequence[int], threads: int = 8):
    """Yield (block, flat bf16 weight) in block order, drawing up to `threads`
    blocks ahead in parallel threads; a block's array is dropped by the caller
    once consumed, so at most about `threads` blocks are held at once."""
    from collections import deque
    numels = list(numels)
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        pending = deque()
        nxt = 0
        while nxt < len(numels) or pending:
            while nxt < len(numels) and len(pending) < max(1, threads):
                pending.append((nxt, ex.submit(block_weights, wid, nxt, numels[nxt])))
                nxt += 1
            b, fut = pending.popleft()
            yield b, fut.result()


def activations(tokens: int, d: int, seed: int = 7) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal((int(tokens), int(d)), dtype=np.float32)


def conditioning(d_cond: int = 256, seed: int = 11) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal(int(d_cond), dtype=np.float32)


def request_tokens(n: int = 4, lo: int = 1000, hi: int = 12000, seed: int = 2026) -> List[int]:
    g = np.random.Generator(np.random.PCG64(seed))
    return [int(t) for t in g.integers(lo, hi, size=n, endpoint=True)]
