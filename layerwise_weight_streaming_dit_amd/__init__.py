"""MI355X-native layer-by-layer weight-streamed DiT forward.

The C-ABI library ``libdlo.so`` (include/dlo.h) holds the pinned weight
shards, the two device slots, the stream/event scheduler and the gfx950 HIP
kernels; this package is its ctypes binding.  Build the library with
``python -m layerwise_weight_streaming_dit_amd.build``.
"""
from ._lib import (  # noqa: F401
    ABI_VERSION, DloError, StreamedDiT, block_layout, required_bytes, lib, check,
    op_assemble, op_adaln, op_ln_modulate, op_gemm, op_attention,
    FLAG_TRACE, FLAG_SERIALIZE, FLAG_POISON_SLOTS, FLAG_TRACE_KERNELS, FLAG_TRACE_SPAN,
    IV_KIND, TRACE_KINDS_ALL,
    EPI_BIAS_F16, EPI_BIAS_GELU_F16, EPI_GATED_F32, EPI_VT_F16,
    OK, E_INVAL, E_SHAPE, E_STATE, E_HOST_OOM, E_DEV_OOM, E_HIP, E_POISONED,
)
