"""Loading a streamed model from a memory-mapped safetensors checkpoint: the
pinned shards and the forward are bitwise those of an in-memory load, and the
mmap path adds no anonymous host copy of the weights."""
import numpy as np
import pytest

import synth
from oracle import layout as OL, shard as OS
from gpu_util import dev, host, torch

pytestmark = pytest.mark.gpu

import layerwise_weight_streaming_dit_amd as dlo
from layerwise_weight_streaming_dit_amd import checkpoint as C


def _forward(ctx, x, cond):
    t = torch()
    T, d0 = x.shape
    xbuf = t.zeros(T * ctx.max_d, dtype=t.float32, device="cuda")
    xbuf[: T * d0] = dev(x.reshape(-1))
    out = ctx.forward(xbuf, dev(cond), T)
    t.cuda.synchronize()
    return host(out).copy()


def test_mmap_load_matches_in_memory_load_without_a_host_copy(tmp_path):
    wl = synth.workload("image")
    L, dp, T = 6, 4, 512
    shapes = list(wl.blocks[:L])
    numels = [OL.block_numel(s) for s in shapes]
    path = str(tmp_path / "image6.safetensors")
    size = C.write(path, shapes, lambda b: synth.block_weights(wl.wid, b, numels[b]))
    model_bytes = 2 * sum(numels)
    print(f"[mmap] checkpoint {size / 1e6:.1f} MB, {L} blocks", flush=True)

    m0 = C.host_memory()
    a = dlo.StreamedDiT(shapes, dp, T)
    C.load(a, path)
    m1 = C.host_memory()

    data = np.fromfile(path, dtype=np.uint8)  # the in-memory path: the whole file in process memory
    ranges = C.plan(path, shapes)
    b = dlo.StreamedDiT(shapes, dp, T)
    for i, (off, n) in enumerate(ranges):
        b.load_shards(i, data[off: off + 2 * n].view(np.uint16))
    m2 = C.host_memory()
    del data

    grow_mmap = m1["RssAnon"] - m0["RssAnon"]
    grow_mem = m2["RssAnon"] - m1["RssAnon"]
    print(f"[mmap] anonymous RSS growth: mmap load {grow_mmap / 1e6:.1f} MB, in-memory load "
          f"{grow_mem / 1e6:.1f} MB (model {model_bytes / 1e6:.1f} MB); file-backed RSS after the mmap "
          f"load {(m1['RssFile'] - m0['RssFile']) / 1e6:.1f} MB", flush=True)
    if "Pss" in m0:
        print(f"[mmap] PSS growth: mmap load {(m1['Pss'] - m0['Pss']) / 1e6:.1f} MB (anonymous "
              f"{(m1['Pss_Anon'] - m0['Pss_Anon']) / 1e6:.1f}, file {(m1['Pss_File'] - m0['Pss_File']) / 1e6:.1f}), "
              f"in-memory load {(m2['Pss'] - m1['Pss']) / 1e6:.1f} MB (anonymous "
              f"{(m2['Pss_Anon'] - m1['Pss_Anon']) / 1e6:.1f})", flush=True)
    # pinned shard bytes: dp shards of ceil(numel / dp) elements per block, in
    # both contexts, whichever way the weights were read
    pinned = sum(dp * -(-n // dp) * 2 for n in numels)
    print(f"[mmap] pinned shard bytes per context: {pinned / 1e6:.1f} MB", flush=True)
    assert a.pinned_bytes() == b.pinned_bytes() == pinned
    # the in-memory path holds one more anonymous copy of the model than the mmap path
    assert grow_mem - grow_mmap >= 0.9 * model_bytes

    for i in (0, L - 1):
        flat = synth.block_weights(wl.wid, i, numels[i])
        ref = OS.shard(flat, dp)
        for r in range(dp):
            assert np.array_equal(a.get_shard(i, r), ref[r])
            assert np.array_equal(b.get_shard(i, r), ref[r])
    x = synth.activations(T, 2048)
    cond = synth.conditioning(256)
    assert np.array_equal(_forward(a, x, cond), _forward(b, x, cond))
    a.close()
    b.close()
