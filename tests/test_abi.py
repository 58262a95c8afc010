"""The C-ABI library on the CPU: it loads, exports every symbol the headers
declare, and its pure host logic (layout, sizes, validation) agrees with the
oracle.  No call here reaches the GPU."""
import ctypes
import os
import re

import pytest

import synth
from oracle import layout as OL, shard as OS, trace as OT
import layerwise_weight_streaming_dit_amd as dlo
from layerwise_weight_streaming_dit_amd import _lib as L


def _declared_symbols():
    names = []
    for h in L.HEADERS:
        src = open(h).read()
        names += re.findall(r"DLO_API\s+[\w\s\*]+?\b(dlo_\w+)\s*\(", src)
    return sorted(set(names))


def test_headers_declare_the_core_calls():
    syms = _declared_symbols()
    for core in ("dlo_create", "dlo_load_shards", "dlo_forward", "dlo_destroy", "dlo_required_bytes",
                 "dlo_layout", "dlo_get_shard", "dlo_debug_assemble", "dlo_get_stats", "dlo_get_trace",
                 "dlo_last_error", "dlo_op_assemble", "dlo_op_gemm", "dlo_op_attention"):
        assert core in syms


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in _declared_symbols():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_library_layout_matches_oracle(name):
    wl = synth.workload(name)
    for shp in wl.blocks[:2]:
        for dp in wl.dp_sizes + (1, 7):
            numel, shard, params = dlo.block_layout(shp, dp)
            assert numel == OL.block_numel(shp)
            assert shard == OS.shard_size(numel, dp)
            want = [(p.name, p.offset, p.shape) for p in OL.param_table(shp)]
            assert params == want


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_required_bytes_two_slots_of_largest_block(name):
    wl = synth.workload(name)
    for dp in wl.dp_sizes:
        sz = dlo.required_bytes(list(wl.blocks), dp, wl.tokens)
        numels = [OL.block_numel(b) for b in wl.blocks]
        one_slot = OT.slot_capacity_elems(numels, dp) * 2  # bytes
        one_slot_aligned = -(-one_slot // 256) * 256
        assert sz["slots"] == 2 * one_slot_aligned
        assert sz["total"] >= sz["slots"] + sz["landing"] + sz["workspace"]
        # landing: two chunks of at most min(S_max, a quarter block, 2^27)
        # elements (+ co-alignment slack), so that every byte that ever holds
        # weights -- slots and landing buffers -- is at most 2.5 blocks
        s_max = max(OS.shard_size(n, dp) for n in numels)
        chunk = min(s_max, -(-dp * s_max // 4), 1 << 27)
        assert sz["landing"] <= 2 * (-(-(chunk + 8) * 2 // 256) * 256)
        max_block = 2 * dp * s_max
        # (+ 256-byte alignment of each of the four buffers and the landing
        # buffers' co-alignment slack)
        assert sz["slots"] + sz["landing"] <= 2.5 * max_block + 4 * 256 + 2 * 16
        if name == "image":  # four chunks of exactly one shard each
            assert sz["landing"] == 2 * 2 * s_max
            assert sz["slots"] + sz["landing"] == 2.5 * max_block


def _cfg(shapes, **kw):
    args = dict(dp=4, max_tokens=256, chunk=0, device=0, flags=0, arena=0, arena_bytes=0)
    args.update(kw)
    return L._config(shapes, args["dp"], args["max_tokens"], args["chunk"], args["device"], args["flags"],
                     args["arena"], args["arena_bytes"])


def _create_status(cfg):
    h = ctypes.c_void_p()
    return L.lib().dlo_create(ctypes.byref(cfg), ctypes.byref(h)), h


TINY = list(synth.workload("tiny").blocks)


@pytest.mark.parametrize("mutate,code", [
    (dict(dp=0), L.E_INVAL),
    (dict(max_tokens=0), L.E_INVAL),
    (dict(chunk=100), L.E_INVAL),
    (dict(arena=0, arena_bytes=1 << 30), L.E_INVAL),          # NULL arena
    (dict(arena=256, arena_bytes=1024), L.E_DEV_OOM),          # arena too small
    (dict(arena=300, arena_bytes=1 << 40), L.E_INVAL),         # misaligned arena
])
def test_create_rejects_before_touching_the_device(mutate, code):
    cfg, keep = _cfg(TINY, **mutate)
    st, h = _create_status(cfg)
    assert st == code and not h.value
    assert L.lib().dlo_last_error().decode()


@pytest.mark.parametrize("bad", [
    synth.BlockShape(200, 4, 1024),     # d not a multiple of 128
    synth.BlockShape(256, 3, 1024),     # d not divisible by heads
    synth.BlockShape(256, 8, 1024),     # head dim 32
    synth.BlockShape(256, 4, 1000),     # mlp not a multiple of 128
    synth.BlockShape(256, 4, 1024, 100),  # cond not a multiple of 64
])
def test_invalid_block_shapes_rejected(bad):
    cfg, keep = _cfg([bad], arena=256, arena_bytes=1 << 40)
    st, h = _create_status(cfg)
    assert st == L.E_INVAL
    with pytest.raises(dlo.DloError):
        dlo.block_layout(bad, 4)


def test_activations_beyond_4gib_rejected():
    # 2^20 tokens x d_mlp 8192 x 2 bytes = 16 GiB: GEMM offsets are 32-bit
    cfg, keep = _cfg([synth.BlockShape(256, 4, 8192)], max_tokens=1 << 20, arena=256, arena_bytes=1 << 40)
    assert _create_status(cfg)[0] == L.E_INVAL
    assert "4 GiB" in L.lib().dlo_last_error().decode()
    # the q,k projection output is tokens x 2 d_model: with d_mlp = d_model it
    # is the widest operand (200000 x 8192 x 2 bytes fits, x 2 does not)
    cfg, keep = _cfg([synth.BlockShape(8192, 64, 8192)], max_tokens=200000, arena=256, arena_bytes=1 << 40)
    assert _create_status(cfg)[0] == L.E_INVAL
    assert "4 GiB" in L.lib().dlo_last_error().decode()


def test_abi_version_and_mixed_cond_rejected():
    cfg, keep = _cfg(TINY, arena=256, arena_bytes=1 << 40)
    cfg.abi_version = 99
    assert _create_status(cfg)[0] == L.E_INVAL
    mixed = [synth.BlockShape(256, 4, 1024, 256), synth.BlockShape(256, 4, 1024, 128)]
    cfg, keep = _cfg(mixed, arena=256, arena_bytes=1 << 40)
    assert _create_status(cfg)[0] == L.E_INVAL


def test_null_context_calls_fail_closed():
    lib = L.lib()
    assert lib.dlo_destroy(None) == L.OK
    assert lib.dlo_forward(None, None, None, 1, None) == L.E_INVAL
    assert lib.dlo_load_shards(None, 0, None, 0) == L.E_INVAL


def test_op_validation_without_launch():
    lib = L.lib()
    fake = 4096  # never dereferenced: every call below fails validation first
    assert lib.dlo_op_gemm(0, fake, 64, fake, 64, 64, fake, None, fake, 64, 64, 64, 63, None) == L.E_SHAPE
    assert lib.dlo_op_gemm(0, fake, 64, fake, 64, 64, fake, None, fake, 64, 64, 64, 64, None) == L.E_SHAPE
    assert lib.dlo_op_gemm(0, fake, 128, fake, 128, 24, fake, None, fake, 24, 64, 24, 128, None) == L.E_SHAPE
    assert lib.dlo_op_gemm(9, fake, 128, fake, 128, 64, fake, None, fake, 64, 64, 64, 128, None) == L.E_INVAL
    assert lib.dlo_op_gemm(2, fake, 128, fake, 128, 64, fake, None, fake, 64, 64, 64, 128, None) == L.E_INVAL
    # operands are addressed with 32-bit byte offsets: more than 2^17 rows x 2^14 elements is beyond 4 GiB
    assert lib.dlo_op_gemm(0, fake, 1 << 14, fake, 128, 64, fake, None, fake, 64, (1 << 17) + 1, 64, 128, None) == L.E_SHAPE
    assert lib.dlo_op_gemm(0, fake, 128, fake, 1 << 14, (1 << 17) + 16, fake, None, fake, (1 << 17) + 16, 64, (1 << 17) + 16, 128,
                           None) == L.E_SHAPE
    assert lib.dlo_op_attention(fake, 256, fake, 64, fake, 128, 10, 1, 96, None) == L.E_SHAPE
    assert lib.dlo_op_attention(fake, 256, fake, 32, fake, 128, 40, 1, 128, None) == L.E_SHAPE
    assert lib.dlo_op_adaln(fake, fake, fake, fake, 10, 100, None) == L.E_SHAPE
    assert lib.dlo_op_ln_modulate(fake, 64, None, fake, fake, fake, 4, 8194, None) == L.E_SHAPE
    assert lib.dlo_op_assemble(fake, fake + 2, 8, None) == L.E_INVAL  # overlap
    assert lib.dlo_op_assemble(fake, fake, 0, None) == L.OK           # empty copy is a no-op


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asking for more exits with a message before
    touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
