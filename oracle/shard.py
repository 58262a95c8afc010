"""Ceil-divided, zero-padded weight shards and their reconstruction (oracle).

Release page, section "Weight sharding with AllGather reconstruction":

* every rank keeps 1/dp_size of a block's flattened weight; the shard length
  is the ceiling of total_numel / dp_size;
* a shard starts as zeros and receives the part of the flat weight that falls
  in [rank * shard_size, (rank + 1) * shard_size); the tail of the last
  shard(s) therefore stays zero, which makes all shards the same length, as
  the all-gather collective requires;
* at run time the full layer is rebuilt by gathering all shards into one
  buffer (all_gather_into_tensor), i.e. the concatenation of the shards in
  rank order; the first total_numel elements of it are the flat weight.

Pinning is a property of host memory, not of values, so it has no oracle.

The GPU path keeps the reconstructed layer in its matrix cores' operand type,
fp16 (a reading of the precision the pages leave to the hardware: fp16 has
the bf16 rate on these matrix cores and three more mantissa bits);
``as_f16_bits`` is that conversion, element by element.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np


def shard_size(numel: int, dp: int) -> int:
    if dp < 1 or numel < 0:
        raise ValueError("dp must be >= 1 and numel >= 0")
    return (numel + dp - 1) // dp


def shard(flat: np.ndarray, dp: int) -> List[np.ndarray]:
    """Split a 1-D flat weight into dp equal, zero-padded shards."""
    flat = np.asarray(flat)
    if flat.ndim != 1:
        raise ValueError("flat weight must be 1-D")
    numel = flat.shape[0]
    s = shard_size(numel, dp)
    shards = []
    for rank in range(dp):
        out = np.zeros(s, dtype=flat.dtype)
        lo = rank * s
        hi = min(lo + s, numel)
        if hi > lo:
            out[: hi - lo] = flat[lo:hi]
        shards.append(out)
    return shards


def all_gather(shards: Sequence[np.ndarray]) -> np.ndarray:
    """What all_gather_into_tensor returns: the shards concatenated in rank
    order (length dp * shard_size, padding included)."""
    sizes = {int(s.shape[0]) for s in shards}
    if len(sizes) != 1:
        raise ValueError("all shards must have the same length")
    return np.concatenate(list(shards))


def unshard(shards: Sequence[np.ndarray], numel: int) -> np.ndarray:
    """The reconstructed flat weight: the gathered buffer without padding."""
    full = all_gather(shards)
    if numel > full.shape[0]:
        raise ValueError("numel exceeds the gathered length")
    return full[:numel].copy()


def as_f16_bits(bf16_bits: np.ndarray) -> np.ndarray:
    """Each bf16 value (given as its 16-bit pattern) rounded to the nearest
    fp16 value, ties to even, fp16 subnormals included, magnitudes past
    fp16's range to infinity; returned as fp16 bit patterns.  Every bf16 value
    of magnitude >= 2^-17 and <= 65504 is an fp16 value already and is kept
    exactly."""
    f = (np.ascontiguousarray(bf16_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    with np.errstate(over="ignore"):
        return f.astype(np.float16).view(np.uint16)
