// Device-side helpers shared by the gfx950 kernels of the streamed DiT forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dlo {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed pair of fp16 (lo in bits 0..15), round to nearest even
// (v_cvt_pk_f16_f32).  Activations between kernels are fp16.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// bf16 -> fp16, two at a time (bits 0..15 and 16..31 of w), round to
// nearest even.  A bf16 value has 8 significant bits and fp16 has 11.
// Magnitudes in [2^-14, 65504] are fp16 normals and convert exactly; in
// [2^-17, 2^-14) they become fp16 subnormals (spacing 2^-24), which still
// hold all 8 bits of a bf16 value there, so they convert exactly too; below
// 2^-17 they round to the subnormal grid (absolute error <= 2^-25); above
// 65504 they overflow.  The reconstruction writes the gathered layer through
// this, so the weights reach the matrix cores as fp16.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// fp16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Four fp16 (two dwords, lowest element first) -> fp32 (exact).  The dwords
// are copied out of the vector before the bit casts: a bit cast applied to a
// vector element expression (b.y) has been compiled as a cast of element 0.
__device__ __forceinline__ f32x4_t f16x4_to_f32x4(u32x2_t b) {
  const uint32_t b0 = b.x, b1 = b.y;
  const f16x2_t lo = __builtin_bit_cast(f16x2_t, b0), hi = __builtin_bit_cast(f16x2_t, b1);
  return f32x4_t{static_cast<float>(lo[0]), static_cast<float>(lo[1]), static_cast<float>(hi[0]),
                 static_cast<float>(hi[1])};
}

// Column position of token j in the transposed v buffer: inside every aligned
// group of 16 tokens, bits 2 and 3 of the offset are swapped, so that the
// 8 keys each lane of attention's P.V step needs are one aligned 16-byte run.
__device__ __forceinline__ int vt_key_position(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

// tanh-approximated GELU: 0.5 z (1 + tanh(y)), y = sqrt(2/pi) (z + 0.044715 z^3).
// Since 0.5 (1 + tanh(y)) = 1 / (1 + exp(-2y)), this is z / (1 + 2^(-2y log2 e)):
// one exp2 and one reciprocal (v_exp_f32, v_rcp_f32, about 1 ulp each) instead
// of an IEEE division.  Large |z| saturate correctly (exp2 -> inf gives -0,
// exp2 -> 0 gives z).
__device__ __forceinline__ float gelu_tanh(float z) {
  const float c0 = 2.0f * 0.7978845608028654f * 1.4426950408889634f;  // 2 sqrt(2/pi) log2(e)
  const float c1 = c0 * 0.044715f;
  const float t = z * fmaf(c1, z * z, c0);  // 2 y log2(e)
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t));
}

// SiLU z / (1 + exp(-z)) with exp2 and a reciprocal (see gelu_tanh).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// Wave-wide (64 lanes) reductions.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Raw (byte-addressed, unswizzled) buffer descriptor over `bytes` bytes from
// `base`; dword 3 selects the 32-bit data format of gfx9 raw buffer loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// 16 bytes per lane from buffer offset voff + soff straight into LDS (lane i's
// data lands at lds + 16 * i: buffer_load_dwordx4 ... lds, no staging
// registers).  The LDS address-space cast only exists in the device pass.
// Unlike global_load_lds (a FLAT-encoded access, which the compiler must
// assume may complete out of order with LDS reads, so that after one every
// wait it inserts for a fragment read becomes lgkmcnt(0)), a buffer load
// counts on vmcnt only: the compiler's waits for fragment reads stay exact
// and a wave starts multiplying as soon as its first fragments are in.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, uint16_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#endif
}

// s_waitcnt vmcnt(n) leaving lgkmcnt / expcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) leaving vmcnt / expcnt unconstrained.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

template <int V>
using IC = std::integral_constant<int, V>;

}  // namespace dlo
