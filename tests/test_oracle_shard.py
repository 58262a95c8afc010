"""Pins for oracle.shard: ceil-divided, zero-padded shards and reconstruction.

Release page, section "Weight sharding with AllGather reconstruction": shard
length is ceil(total_numel / dp_size); shard r holds the flat slice
[r*S, (r+1)*S) and zeros after it; all shards have the same length; the
gathered buffer's first total_numel elements are the flat weight.
"""
import math
import os

import numpy as np
import pytest

from oracle import shard as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_memory_facts.txt")


def _elementwise_expected(flat, dp):
    """Brute force, one element at a time: global index i of the gathered
    buffer lives in shard i // S at position i % S and holds flat[i] if
    i < numel, else zero."""
    n = len(flat)
    s = -(-n // dp)
    out = [[0] * s for _ in range(dp)]
    for i in range(dp * s):
        out[i // s][i % s] = int(flat[i]) if i < n else 0
    return out


def test_shard_size_closed_form():
    for n in list(range(0, 300)) + [10**9 + 7, 2**40 + 3, 818_012_160, 207_679_537]:
        for dp in range(1, 17):
            if n < 2**52:  # float division is exact enough here
                assert O.shard_size(n, dp) == math.ceil(n / dp)
            assert O.shard_size(n, dp) == -(-n // dp)
            assert dp * O.shard_size(n, dp) - n in range(0, dp)


def test_shard_size_rejects_bad_args():
    with pytest.raises(ValueError):
        O.shard_size(10, 0)
    with pytest.raises(ValueError):
        O.shard_size(-1, 2)


@pytest.mark.parametrize("dp", range(1, 17))
def test_shard_bruteforce_small(dp):
    rng = np.random.default_rng(dp)
    for n in range(0, 130):
        flat = rng.integers(0, 2**16, size=n, dtype=np.uint16)
        shards = O.shard(flat, dp)
        exp = _elementwise_expected(flat, dp)
        assert len(shards) == dp
        s = O.shard_size(n, dp)
        for r in range(dp):
            assert shards[r].dtype == np.uint16 and shards[r].shape == (s,)
            assert shards[r].tolist() == exp[r]
        pad = dp * s - n
        assert 0 <= pad <= max(dp - 1, 0)
        assert np.array_equal(O.unshard(shards, n), flat)


def test_shard_random_sizes_up_to_4096():
    rng = np.random.default_rng(1)
    for _ in range(400):
        n = int(rng.integers(0, 4097))
        dp = int(rng.integers(1, 17))
        flat = rng.integers(0, 2**16, size=n, dtype=np.uint16)
        shards = O.shard(flat, dp)
        s = -(-n // dp)
        gathered = O.all_gather(shards)
        assert gathered.shape == (dp * s,)
        assert np.all(gathered[n:] == 0)
        assert np.array_equal(gathered[:n], flat)
        for r in range(dp):
            lo, hi = r * s, min((r + 1) * s, n)
            if hi > lo:
                assert np.array_equal(shards[r][: hi - lo], flat[lo:hi])
            assert np.all(shards[r][max(hi - lo, 0):] == 0)


def test_bit_patterns_survive():
    # NaN / inf / negative-zero bf16 patterns must round-trip as bits.
    flat = np.array([0x7FC0, 0xFFC1, 0x7F80, 0xFF80, 0x8000, 0x0001, 0xFFFF], dtype=np.uint16)
    for dp in (1, 2, 3, 8):
        assert O.unshard(O.shard(flat, dp), len(flat)).tobytes() == flat.tobytes()


def test_degenerate_all_padding_shards():
    # numel 5, dp 8: S = 1, shards 5..7 hold only padding.
    flat = np.arange(1, 6, dtype=np.uint16)
    shards = O.shard(flat, 8)
    assert [int(s[0]) for s in shards] == [1, 2, 3, 4, 5, 0, 0, 0]
    empty = O.shard(np.zeros(0, np.uint16), 4)
    assert len(empty) == 4 and all(s.size == 0 for s in empty)


def test_unequal_shards_rejected():
    with pytest.raises(ValueError):
        O.all_gather([np.zeros(3, np.uint16), np.zeros(2, np.uint16)])


def test_pages_memory_facts():
    """Sharding stores 1/dp of every block per rank, so the pinned total over
    all ranks is the model size (up to < dp padding elements per block) and
    the per-rank share is model/dp -- the page's Super DP4 figures."""
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert rows
    for name, model_gb, dp, unsharded, sharded, per_rank in rows:
        model_gb, dp = float(model_gb), int(dp)
        numel = int(model_gb * 1e9 / 2)  # BF16 elements
        s = O.shard_size(numel, dp)
        assert dp * model_gb == pytest.approx(float(unsharded))
        assert dp * s * 2 / 1e9 == pytest.approx(float(sharded), rel=1e-9)
        assert s * 2 / 1e9 == pytest.approx(float(per_rank), rel=1e-9)


def test_as_f16_bits_every_bf16_pattern_against_struct():
    """All 65536 bf16 patterns: the oracle's conversion agrees with CPython's
    own binary16 packing (struct format 'e', round half to even), which
    raises for values too large for fp16; those must become infinities, and
    NaNs must stay NaNs."""
    import struct
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.as_f16_bits(bits)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    for b, v, g in zip(bits.tolist(), vals.tolist(), got.tolist()):
        if math.isnan(v):
            assert (g & 0x7C00) == 0x7C00 and (g & 0x03FF) != 0, hex(b)
            continue
        try:
            want = struct.unpack("<H", struct.pack("<e", v))[0]
        except OverflowError:
            want = 0xFC00 if v < 0 else 0x7C00
        assert g == want, (hex(b), v, hex(g), hex(want))


def test_as_f16_bits_special_cases():
    """Hand-derived values: exact conversions, the subnormal grid (spacing
    2^-24) with ties to even, and overflow."""
    def bf16_of(x):
        return np.array([np.float32(x).view(np.uint32) >> 16], np.uint16)
    cases = [
        (1.0, 0x3C00), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
        (2.0 ** -14, 0x0400),          # smallest fp16 normal
        (2.0 ** -17, 0x0080),          # subnormal, exact (8 significant bits fit)
        (2.0 ** -24, 0x0001),          # smallest fp16 subnormal
        (2.0 ** -25, 0x0000),          # a tie between 0 and 2^-24: to even (0)
        (1.5 * 2.0 ** -25, 0x0001),    # above the tie: up
        (3.0 * 2.0 ** -25, 0x0002),    # 1.5 * 2^-24, a tie: to even (2 * 2^-24)
        (65280.0, 0x7BF8),             # the largest bf16 value below 65504: exact
        (65536.0, 0x7C00),             # beyond fp16's range: infinity
        (-65536.0, 0xFC00),
    ]
    for x, want in cases:
        assert int(O.as_f16_bits(bf16_of(x))[0]) == want, (x, hex(int(O.as_f16_bits(bf16_of(x))[0])))
