"""Helpers for the GPU tests (device copies, the contract tolerance)."""
import numpy as np

RTOL = 2e-2
ATOL = 2e-2


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    """Copy a numpy array to cuda:0 with the same bytes (uint16 -> int16)."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a).cuda()


def host(t, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, np.uint16).view(np.float16).astype(np.float64)


def assert_reconstructed(got: np.ndarray, flat_bf16: np.ndarray) -> None:
    """The reconstructed layer (fp16 patterns) is the flat bf16 weight
    converted element by element (oracle.shard.as_f16_bits), bit for bit; a
    bf16 NaN may come out as any fp16 NaN."""
    from oracle import shard as OS
    got = np.asarray(got, np.uint16)
    flat_bf16 = np.asarray(flat_bf16, np.uint16)
    assert got.shape == flat_bf16.shape
    want = OS.as_f16_bits(flat_bf16)
    nan_in = ((flat_bf16 & 0x7F80) == 0x7F80) & ((flat_bf16 & 0x007F) != 0)
    bad = np.flatnonzero((got != want) & ~nan_in)
    assert bad.size == 0, (bad[:8], got[bad[:8]], want[bad[:8]])
    g = got[nan_in]
    assert np.all(((g & 0x7C00) == 0x7C00) & ((g & 0x03FF) != 0))


def within(got, want, rtol=RTOL, atol=ATOL):
    """|got - want| <= atol + rtol * |want| everywhere; returns (ok, max_abs, max_rel)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    ok = bool(np.all(err <= atol + rtol * np.abs(want))) and bool(np.all(np.isfinite(got)))
    rel = err / np.maximum(np.abs(want), 1e-30)
    return ok, float(err.max(initial=0.0)), float(rel.max(initial=0.0))


def run_forward(ctx, x, cond):
    """One streamed forward of x [T, d_first] (numpy fp32) through a context;
    returns the [T, d_last] result as numpy."""
    t = torch()
    T, d0 = x.shape
    xbuf = t.zeros(T * ctx.max_d, dtype=t.float32, device="cuda")
    xbuf[: T * d0] = dev(np.ascontiguousarray(x, np.float32).reshape(-1))
    out = ctx.forward(xbuf, dev(np.asarray(cond, np.float32)), T)
    t.cuda.synchronize()
    return host(out).copy()


def sample_rows(T, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, size=n)]))
