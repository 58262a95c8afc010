"""Pins for oracle.layout: dense parameter concatenation in a fixed order."""
import numpy as np
import pytest

import synth
from oracle import layout as L


def _closed_form(d, m, c, extra=()):
    # Wqkv 3d*d + bqkv 3d + Wo d*d + bo d + W1 m*d + b1 m + W2 d*m + b2 d
    # + Wada 6d*c + bada 6d + extras
    return 4 * d * d + 2 * d * m + 6 * d * c + 11 * d + m + sum(extra)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_numel_closed_form(name):
    for shp in synth.workload(name).blocks:
        assert L.block_numel(shp) == _closed_form(shp.d_model, shp.d_mlp, shp.d_cond, shp.extra)


def test_offsets_dense_and_ordered():
    shp = synth.BlockShape(256, 4, 1024, 256, (1, 3, 5))
    t = L.param_table(shp)
    names = [p.name for p in t]
    assert names == ["Wqkv", "bqkv", "Wo", "bo", "W1", "b1", "W2", "b2", "Wada", "bada",
                     "extra0", "extra1", "extra2"]
    off = 0
    for p in t:
        assert p.offset == off
        off += int(np.prod(p.shape))
    assert off == L.block_numel(shp)
    d, m, c = 256, 1024, 256
    expect = {"Wqkv": (3 * d, d), "bqkv": (3 * d,), "Wo": (d, d), "bo": (d,), "W1": (m, d),
              "b1": (m,), "W2": (d, m), "b2": (d,), "Wada": (6 * d, c), "bada": (6 * d,)}
    for p in t:
        if p.name in expect:
            assert p.shape == expect[p.name]


def test_matrix_offsets_are_multiples_of_d():
    # All matrix views start on a multiple of d elements (>= 256), i.e. 512-byte
    # aligned inside a 512-byte-aligned flat buffer.
    for name in synth.WORKLOADS:
        for shp in synth.workload(name).blocks[:2]:
            for p in L.param_table(shp):
                if not p.name.startswith("extra"):
                    assert p.offset % shp.d_model == 0


def test_workload_sizes_match_their_descriptions():
    # mid video: "~0.63 GB per block" of bf16
    mid = synth.workload("midvideo").blocks[0]
    assert 0.62e9 < 2 * L.block_numel(mid) < 0.66e9
    # large: "~64B params, ~128 GB bf16"
    large = synth.workload("large")
    total = sum(L.block_numel(b) for b in large.blocks)
    assert 63e9 < total < 67e9
    # irregular: per-block numel not divisible by dp in {3, 8}; largest ~2x smallest
    irr = synth.workload("irregular")
    n = [L.block_numel(b) for b in irr.blocks]
    for dp in (3, 8):
        assert all(x % dp != 0 for x in n)
    assert 1.6 < max(n) / min(n) < 2.0
