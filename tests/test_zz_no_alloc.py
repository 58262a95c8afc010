"""dlo_forward_static -- the streamed forward with its activation workspace in
the library's static device scratch, for callers that cannot allocate at call
time -- against dlo_forward on the same inputs, through the C ABI."""
import numpy as np
import pytest

import synth
from oracle import layout as OL
from gpu_util import dev, host, torch

import layerwise_weight_streaming_dit_amd as dlo
from layerwise_weight_streaming_dit_amd import _lib as L

pytestmark = pytest.mark.gpu


def _static(ctx, xbuf, cond, tokens, stream=None):
    return L.lib().dlo_forward_static(ctx._h, xbuf.data_ptr(), cond.data_ptr(), tokens, L._stream_handle(stream))


def _pair(shapes, dp, max_tokens, wid):
    W = [synth.block_weights(wid, b, OL.block_numel(s)) for b, s in enumerate(shapes)]
    ctxs = []
    for _ in range(2):
        c = dlo.StreamedDiT(shapes, dp, max_tokens)
        for b, flat in enumerate(W):
            c.load_shards(b, flat)
        ctxs.append(c)
    return ctxs


def _xbuf(x, max_d):
    t = torch()
    T, d0 = x.shape
    buf = t.zeros(T * max_d, dtype=t.float32, device="cuda")
    buf[: T * d0] = dev(x.reshape(-1))
    return buf


@pytest.mark.parametrize("workload", ["tiny", "irregular"])
def test_forward_static_matches_forward_on_two_calls(workload):
    t = torch()
    wl = synth.workload(workload)
    shapes = list(wl.blocks[:2]) if workload == "irregular" else list(wl.blocks)
    max_tokens = 256
    ref_ctx, st_ctx = _pair(shapes, wl.dp_sizes[0], max_tokens, wl.wid)
    max_d = max(s.d_model for s in shapes)
    cond = dev(synth.conditioning(256))
    # two calls in a row on the static scratch, the second with fewer tokens
    for T in (max_tokens, 77):
        x = synth.activations(T, shapes[0].d_model)
        xa, xb = _xbuf(x, max_d), _xbuf(x, max_d)
        ref = ref_ctx.forward(xa, cond, T)
        t.cuda.synchronize()
        free0 = t.cuda.mem_get_info()[0]
        assert _static(st_ctx, xb, cond, T) == dlo.OK, L.lib().dlo_last_error()
        t.cuda.synchronize()
        assert t.cuda.mem_get_info()[0] == free0  # the call allocated nothing
        d_last = shapes[-1].d_model
        got = host(xb[: T * d_last]).reshape(T, d_last)
        assert np.array_equal(got, host(ref)), (workload, T)
    ref_ctx.close()
    st_ctx.close()


def test_forward_static_rejects_before_enqueue():
    t = torch()
    wl = synth.workload("image")
    shapes = list(wl.blocks[:1])
    ctx = dlo.StreamedDiT(shapes, 4, 8192)
    xbuf = t.zeros(8192 * 2048, dtype=t.float32, device="cuda")
    cond = dev(synth.conditioning(256))
    # 8192 tokens of a d 2048 / MLP 8192 block need ~302 MB of activations
    assert _static(ctx, xbuf, cond, 8192) == dlo.E_INVAL
    assert b"static scratch" in L.lib().dlo_last_error()
    assert _static(ctx, xbuf, cond, 0) == dlo.E_INVAL
    assert _static(ctx, xbuf, cond, 1024) == dlo.E_STATE  # no shards loaded
    ctx.close()
    tr = dlo.StreamedDiT(shapes, 4, 64, flags=dlo.FLAG_TRACE)
    assert _static(tr, xbuf, cond, 64) == dlo.E_STATE
    assert b"trace" in L.lib().dlo_last_error()
    tr.close()
    t.cuda.synchronize()
