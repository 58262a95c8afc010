"""Per-block flat parameter layout (oracle side).

The offload backend treats each block's weights as one flattened tensor of
``total_numel`` elements and slices it (release page, section "Weight sharding
with AllGather reconstruction", the ``_shard_and_pin`` snippet); after the
gather it re-points parameters at slices of the flat buffer from cached
(offset, shape) metadata (section "Double-buffered prefetch with H2D +
AllGather overlap").  The pages do not fix the parameter order; the reading
taken here is a dense concatenation, in nn.Linear convention (weight stored
[out, in]), in this order:

    Wqkv [3d, d], bqkv [3d], Wo [d, d], bo [d], W1 [m, d], b1 [m],
    W2 [d, m], b2 [d], Wada [6d, c], bada [6d], extra_0, extra_1, ...

so numel = 4d^2 + 2dm + 6dc + 11d + m + sum(extra).
"""
from __future__ import annotations

from typing import List, NamedTuple, Tuple


class Param(NamedTuple):
    name: str
    offset: int
    shape: Tuple[int, ...]

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


def param_table(shape) -> List[Param]:
    """Parameters of one block (a ``synth.BlockShape``-like object with
    d_model, d_mlp, d_cond, extra) with their offsets into the flat weight."""
    d, m, c = shape.d_model, shape.d_mlp, shape.d_cond
    entries = [
        ("Wqkv", (3 * d, d)), ("bqkv", (3 * d,)),
        ("Wo", (d, d)), ("bo", (d,)),
        ("W1", (m, d)), ("b1", (m,)),
        ("W2", (d, m)), ("b2", (d,)),
        ("Wada", (6 * d, c)), ("bada", (6 * d,)),
    ]
    entries += [(f"extra{i}", (int(n),)) for i, n in enumerate(shape.extra)]
    out, off = [], 0
    for name, shp in entries:
        p = Param(name, off, shp)
        out.append(p)
        off += p.numel
    return out


def block_numel(shape) -> int:
    t = param_table(shape)
    return t[-1].offset + t[-1].numel
