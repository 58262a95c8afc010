// Host-side launchers of the gfx950 kernels.  Each returns the HIP status of
// its launch; argument validation is the caller's job (the C ABI layer).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace dlo {

// Reconstruction of one landed chunk into its slot (all-gather stand-in):
// dst[i] = fp16(src[i]) for the n bf16 values of src.
hipError_t launch_assemble(uint16_t* dst, const uint16_t* src, int64_t n, hipStream_t s);
// Fill n fp16 elements with a quiet-NaN pattern (slot poisoning test hook).
hipError_t launch_fill_nan(uint16_t* dst, int64_t n, hipStream_t s);

hipError_t launch_adaln(const uint16_t* w, const uint16_t* b, const float* cond, float* mod,
                        int rows, int c, hipStream_t s);

hipError_t launch_ln_modulate(const float* xin, int d_in, float* xout, const float* shift,
                              const float* scale, uint16_t* h, int tokens, int d, hipStream_t s);

enum Epilogue { EPI_BIAS_F16 = 0, EPI_BIAS_GELU_F16 = 1, EPI_GATED_F32 = 2, EPI_VT_F16 = 3 };

struct GemmArgs {
  const uint16_t* a;
  const uint16_t* w;
  const uint16_t* bias;
  const float* gate;
  void* out;
  int lda, ldw, ldo;
  int M, N, K;
  int w_rows;
};
hipError_t launch_gemm(int epilogue, const GemmArgs& g, hipStream_t s);

hipError_t launch_attention(const uint16_t* qk, int ld_qk, const uint16_t* vt, int ld_vt,
                            uint16_t* o, int ld_o, int tokens, int heads, int head_dim,
                            hipStream_t s);

// The library's static device scratch (scratch.hip): kStaticScratchBytes per
// device, held from the first call on a device until the process ends.
// static_scratch returns this device's address of it; `device` must be the
// current device.
constexpr size_t kStaticScratchBytes = size_t(256) << 20;
hipError_t static_scratch(int device, void** out);

}  // namespace dlo
