"""ctypes binding of libdlo.so (include/dlo.h, include/dlo_ops.h).

Argument marshalling only: every step of the streamed forward runs in the
library's HIP kernels.  PyTorch is used for device memory (the arena, x,
cond) and streams.  Importing this module does not load the library; the
first call that needs it does, and fails loudly if it is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdlo.so")
HEADERS = [os.path.join(os.path.dirname(_HERE), "include", h) for h in ("dlo.h", "dlo_ops.h")]

ABI_VERSION = 2
OK, E_INVAL, E_SHAPE, E_STATE, E_HOST_OOM, E_DEV_OOM, E_HIP, E_POISONED = 0, -1, -2, -3, -4, -5, -6, -7
STATUS_NAMES = {0: "DLO_OK", -1: "DLO_E_INVAL", -2: "DLO_E_SHAPE", -3: "DLO_E_STATE", -4: "DLO_E_HOST_OOM",
                -5: "DLO_E_DEV_OOM", -6: "DLO_E_HIP", -7: "DLO_E_POISONED"}
FLAG_TRACE, FLAG_SERIALIZE, FLAG_POISON_SLOTS, FLAG_TRACE_KERNELS, FLAG_TRACE_SPAN = 0x1, 0x2, 0x4, 0x8, 0x10
IV_H2D, IV_ASM, IV_COMPUTE = 0, 1, 2
IV_NAMES = {0: "h2d", 1: "asm", 2: "compute", 3: "k_adaln", 4: "k_ln1", 5: "k_qk", 6: "k_v", 7: "k_attn",
            8: "k_out", 9: "k_ln2", 10: "k_fc1", 11: "k_fc2"}
IV_KIND = {name: kind for kind, name in IV_NAMES.items()}
TRACE_KINDS_ALL = 0xFFF
EPI_BIAS_F16, EPI_BIAS_GELU_F16, EPI_GATED_F32, EPI_VT_F16 = 0, 1, 2, 3


class DloError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


class BlockDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_mlp", ctypes.c_int32),
                ("d_cond", ctypes.c_int32), ("n_extra", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("extra_len", ctypes.POINTER(ctypes.c_int64))]


class Config(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("blocks", ctypes.POINTER(BlockDesc)), ("dp_size", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("landing_chunk_elems", ctypes.c_int64),
                ("device", ctypes.c_int32), ("flags", ctypes.c_uint32), ("arena", ctypes.c_void_p),
                ("arena_bytes", ctypes.c_size_t), ("copy_stream", ctypes.c_void_p),
                ("gather_stream", ctypes.c_void_p)]


class ParamDesc(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 16), ("offset", ctypes.c_int64), ("ndim", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("shape", ctypes.c_int64 * 2)]


class Interval(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("block", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("slot", ctypes.c_int32), ("landing", ctypes.c_int32), ("forward", ctypes.c_int32),
                ("bytes", ctypes.c_int64), ("start_ms", ctypes.c_double), ("end_ms", ctypes.c_double)]


class Stats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("dp_size", ctypes.c_int32), ("forwards", ctypes.c_int64),
                ("max_shard_elems", ctypes.c_int64), ("slot_bytes", ctypes.c_size_t),
                ("landing_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
                ("residency_high_water", ctypes.c_int32), ("n_intervals", ctypes.c_int32),
                ("last_forward_ms", ctypes.c_double), ("sum_h2d_ms", ctypes.c_double),
                ("sum_asm_ms", ctypes.c_double), ("sum_compute_ms", ctypes.c_double),
                ("h2d_bytes_per_forward", ctypes.c_int64), ("landing_chunk_elems", ctypes.c_int64),
                ("max_block_bytes", ctypes.c_size_t), ("weight_bytes_allocated", ctypes.c_size_t),
                ("blocks_on_device_high_water", ctypes.c_int32), ("reserved2", ctypes.c_int32),
                ("weight_bytes_peak", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGNATURES = {
    "dlo_block_layout": [ctypes.POINTER(BlockDesc), _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                         ctypes.POINTER(_I32), ctypes.POINTER(ParamDesc), _I32],
    "dlo_required_bytes": [ctypes.POINTER(Config), ctypes.POINTER(_SZ), ctypes.POINTER(_SZ),
                           ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)],
    "dlo_create": [ctypes.POINTER(Config), ctypes.POINTER(_P)],
    "dlo_load_shards": [_P, _I32, _P, _I64],
    "dlo_forward": [_P, _P, _P, _I32, _P],
    "dlo_forward_static": [_P, _P, _P, _I32, _P],
    "dlo_destroy": [_P],
    "dlo_set_flags": [_P, ctypes.c_uint32],
    "dlo_reserve_trace": [_P, _I32],
    "dlo_set_trace_kinds": [_P, ctypes.c_uint32],
    "dlo_layout": [_P, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I32),
                   ctypes.POINTER(ParamDesc), _I32],
    "dlo_get_shard": [_P, _I32, _I32, ctypes.POINTER(_P), ctypes.POINTER(_I64)],
    "dlo_debug_assemble": [_P, _I32, _P, _I64],
    "dlo_get_stats": [_P, ctypes.POINTER(Stats)],
    "dlo_get_trace": [_P, ctypes.POINTER(Interval), _I32, ctypes.POINTER(_I32)],
    "dlo_op_assemble": [_P, _P, _I64, _P],
    "dlo_op_adaln": [_P, _P, _P, _P, _I32, _I32, _P],
    "dlo_op_ln_modulate": [_P, _I32, _P, _P, _P, _P, _I32, _I32, _P],
    "dlo_op_gemm": [_I32, _P, _I32, _P, _I32, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _P],
    "dlo_op_attention": [_P, _I32, _P, _I32, _P, _I32, _I32, _I32, _I32, _P],
}

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libdlo.so (once).  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m layerwise_weight_streaming_dit_amd.build`")
        # PyTorch brings its own HIP runtime; loading it first makes the
        # library bind to that same runtime (one runtime per process) instead
        # of loading the system copy next to it.
        import torch  # noqa: F401
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = ctypes.c_int32
        l.dlo_last_error.argtypes = []
        l.dlo_last_error.restype = ctypes.c_char_p
        _lib = l
    return _lib


def check(code: int) -> None:
    if code != OK:
        raise DloError(code, lib().dlo_last_error().decode(errors="replace"))


def _blocks_array(shapes) -> tuple:
    keep = []
    arr = (BlockDesc * len(shapes))()
    for i, s in enumerate(shapes):
        extra = tuple(getattr(s, "extra", ()) or ())
        ext = (ctypes.c_int64 * max(1, len(extra)))(*extra) if extra else None
        keep.append(ext)
        arr[i] = BlockDesc(s.d_model, s.n_heads, s.d_mlp, getattr(s, "d_cond", 256), len(extra), 0,
                           ctypes.cast(ext, ctypes.POINTER(ctypes.c_int64)) if ext is not None else None)
    return arr, keep


def block_layout(shape, dp: int):
    """(numel, shard_size, [(name, offset, shape)]) of one block, from the
    library's own layout code."""
    arr, keep = _blocks_array([shape])
    numel, shard, n = _I64(), _I64(), _I32()
    out = (ParamDesc * 128)()
    check(lib().dlo_block_layout(arr, dp, ctypes.byref(numel), ctypes.byref(shard), ctypes.byref(n), out, 128))
    params = [(p.name.decode(), int(p.offset), tuple(int(p.shape[i]) for i in range(p.ndim)))
              for p in out[: n.value]]
    return int(numel.value), int(shard.value), params


def _config(shapes, dp, max_tokens, chunk=0, device=0, flags=0, arena=0, arena_bytes=0,
            copy_stream=0, gather_stream=0):
    arr, keep = _blocks_array(shapes)
    cfg = Config(ABI_VERSION, len(shapes), arr, dp, max_tokens, chunk, device, flags, arena, arena_bytes,
                 copy_stream, gather_stream)
    return cfg, (arr, keep)


def required_bytes(shapes, dp: int, max_tokens: int, chunk: int = 0) -> Dict[str, int]:
    cfg, keep = _config(shapes, dp, max_tokens, chunk)
    s, l, w, t = _SZ(), _SZ(), _SZ(), _SZ()
    check(lib().dlo_required_bytes(ctypes.byref(cfg), ctypes.byref(s), ctypes.byref(l), ctypes.byref(w),
                                   ctypes.byref(t)))
    return {"slots": s.value, "landing": l.value, "workspace": w.value, "total": t.value}


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class StreamedDiT:
    """A context of the weight-streamed forward: pinned shards on the host,
    two device slots, landing buffers and workspace carved from one torch
    allocation (the arena)."""

    def __init__(self, shapes: Sequence, dp_size: int, max_tokens: int, device: int = 0, flags: int = 0,
                 chunk_elems: int = 0, copy_stream=None, gather_stream=None):
        import torch
        self.shapes = list(shapes)
        self.dp_size = dp_size
        self.max_tokens = max_tokens
        self.flags = flags
        self.device = device
        self.sizes = required_bytes(self.shapes, dp_size, max_tokens, chunk_elems)
        self.arena = torch.empty(self.sizes["total"], dtype=torch.uint8, device=f"cuda:{device}")
        self._streams = (copy_stream, gather_stream)  # keep alive
        cfg, self._keep = _config(self.shapes, dp_size, max_tokens, chunk_elems, device, flags,
                                  self.arena.data_ptr(), self.sizes["total"],
                                  int(copy_stream.cuda_stream) if copy_stream is not None else 0,
                                  int(gather_stream.cuda_stream) if gather_stream is not None else 0)
        h = _P()
        check(lib().dlo_create(ctypes.byref(cfg), ctypes.byref(h)))
        self._h = h
        self.max_d = max(s.d_model for s in self.shapes)

    # -- load
    def load_shards(self, block: int, flat: np.ndarray) -> None:
        flat = np.ascontiguousarray(flat, dtype=np.uint16)
        check(lib().dlo_load_shards(self._h, block, flat.ctypes.data, flat.size))

    # -- forward
    def forward(self, xbuf, cond, tokens: int, stream=None):
        """xbuf: cuda fp32 tensor holding tokens * max_d floats whose first
        tokens * d_first are x; returns the [tokens, d_last] view of the
        result.  Asynchronous on `stream` (default: torch's current stream)."""
        import torch
        if xbuf.dtype != torch.float32 or not xbuf.is_cuda or not xbuf.is_contiguous():
            raise ValueError("xbuf must be a contiguous float32 CUDA tensor")
        if xbuf.numel() < tokens * self.max_d:
            raise ValueError(f"xbuf holds {xbuf.numel()} floats; tokens * max_d = {tokens * self.max_d}")
        d_cond = getattr(self.shapes[0], "d_cond", 256)
        if cond.dtype != torch.float32 or not cond.is_cuda or cond.numel() < d_cond:
            raise ValueError(f"cond must be a float32 CUDA tensor of {d_cond} elements")
        check(lib().dlo_forward(self._h, xbuf.data_ptr(), cond.data_ptr(), tokens, _stream_handle(stream)))
        d_last = self.shapes[-1].d_model
        return xbuf.view(-1)[: tokens * d_last].view(tokens, d_last)

    def forward_status(self, xbuf, cond, tokens: int, stream=None) -> int:
        """dlo_forward's raw status (for error-path tests)."""
        return lib().dlo_forward(self._h, xbuf.data_ptr() if xbuf is not None else None,
                                 cond.data_ptr() if cond is not None else None, tokens,
                                 _stream_handle(stream))

    # -- queries
    def layout(self, block: int):
        numel, shard, n = _I64(), _I64(), _I32()
        out = (ParamDesc * 128)()
        check(lib().dlo_layout(self._h, block, ctypes.byref(numel), ctypes.byref(shard), ctypes.byref(n), out, 128))
        return int(numel.value), int(shard.value), [
            (p.name.decode(), int(p.offset), tuple(int(p.shape[i]) for i in range(p.ndim))) for p in out[: n.value]]

    def pinned_bytes(self) -> int:
        """Pinned host bytes holding the loaded blocks' shards (dp_size shards
        of ceil(numel / dp_size) elements per block, 2 bytes each)."""
        total = 0
        for b in range(len(self.shapes)):
            ptr, n = _P(), _I64()
            if lib().dlo_get_shard(self._h, b, 0, ctypes.byref(ptr), ctypes.byref(n)) == OK and ptr.value:
                total += self.dp_size * int(n.value) * 2
        return total

    def get_shard(self, block: int, rank: int) -> np.ndarray:
        ptr, n = _P(), _I64()
        check(lib().dlo_get_shard(self._h, block, rank, ctypes.byref(ptr), ctypes.byref(n)))
        if n.value == 0:
            return np.zeros(0, np.uint16)
        buf = (ctypes.c_uint16 * n.value).from_address(ptr.value)
        return np.frombuffer(buf, dtype=np.uint16).copy()

    def debug_assemble(self, block: int) -> np.ndarray:
        numel = self.layout(block)[0]
        out = np.empty(numel, dtype=np.uint16)
        check(lib().dlo_debug_assemble(self._h, block, out.ctypes.data, numel))
        return out

    def set_flags(self, flags: int) -> None:
        """New DLO_FLAG_* for the forwards enqueued from now on (drops any
        recorded intervals)."""
        check(lib().dlo_set_flags(self._h, flags))
        self.flags = flags

    def set_trace_kinds(self, kinds: int) -> None:
        """Record only the interval kinds whose bit is set (bit n = kind n of
        IV_NAMES; TRACE_KINDS_ALL records all) in the traced forwards enqueued
        from now on (drops any recorded intervals)."""
        check(lib().dlo_set_trace_kinds(self._h, kinds))

    def reserve_trace(self, forwards: int) -> None:
        """Create the timing events `forwards` traced forwards need now, so
        none is created while they are enqueued."""
        check(lib().dlo_reserve_trace(self._h, forwards))

    def stats(self) -> Dict:
        s = Stats()
        check(lib().dlo_get_stats(self._h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in Stats._fields_}

    def trace(self) -> List[Dict]:
        n = _I32()
        check(lib().dlo_get_trace(self._h, None, 0, ctypes.byref(n)))
        arr = (Interval * max(1, n.value))()
        check(lib().dlo_get_trace(self._h, arr, n.value, ctypes.byref(n)))
        return [dict(kind=IV_NAMES[iv.kind], block=iv.block, chunk=iv.chunk, slot=iv.slot, landing=iv.landing,
                     forward=iv.forward, bytes=iv.bytes, start=iv.start_ms, end=iv.end_ms)
                for iv in arr[: n.value]]

    def close(self) -> None:
        if getattr(self, "_h", None):
            check(lib().dlo_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------ ops

def op_assemble(dst, src, n: int, stream=None) -> None:
    check(lib().dlo_op_assemble(dst.data_ptr(), src.data_ptr(), n, _stream_handle(stream)))


def op_adaln(w, b, cond, mod, rows: int, c: int, stream=None) -> None:
    check(lib().dlo_op_adaln(w.data_ptr(), b.data_ptr(), cond.data_ptr(), mod.data_ptr(), rows, c,
                             _stream_handle(stream)))


def op_ln_modulate(xin, d_in: int, xout, shift, scale, h, tokens: int, d: int, stream=None) -> None:
    check(lib().dlo_op_ln_modulate(xin.data_ptr(), d_in, xout.data_ptr() if xout is not None else None,
                                   shift.data_ptr(), scale.data_ptr(), h.data_ptr(), tokens, d,
                                   _stream_handle(stream)))


def op_gemm(epilogue: int, a, lda: int, w, ldw: int, w_rows: int, bias, gate, out, ldo: int, M: int, N: int,
            K: int, stream=None) -> None:
    check(lib().dlo_op_gemm(epilogue, a.data_ptr(), lda, w.data_ptr(), ldw, w_rows, bias.data_ptr(),
                            gate.data_ptr() if gate is not None else None, out.data_ptr(), ldo, M, N, K,
                            _stream_handle(stream)))


def op_attention(qk, ld_qk: int, vt, ld_vt: int, o, ld_o: int, tokens: int, heads: int, head_dim: int,
                 stream=None) -> None:
    check(lib().dlo_op_attention(qk.data_ptr(), ld_qk, vt.data_ptr(), ld_vt, o.data_ptr(), ld_o, tokens, heads,
                                 head_dim, _stream_handle(stream)))
