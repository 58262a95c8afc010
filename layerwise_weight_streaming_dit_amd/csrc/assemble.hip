// Shard reconstruction on gfx950: the single-GPU stand-in for
// all_gather_into_tensor (vLLM-Omni release page, section "Weight sharding
// with AllGather reconstruction": the full layer is the shards concatenated in
// rank order, padding dropped).  The gathered layer is written in the
// matrix cores' operand type: each streamed bf16 value is converted to fp16
// on the way (bf16x2_to_f16x2: exact for |w| >= 2^-17), so no kernel of the
// block converts weights again.
//
// The scheduler lands each H2D chunk at the same address modulo 16 bytes as
// its destination in the slot, so the body is a 16-byte vector
// load-convert-store (global_load_dwordx4 / global_store_dwordx4, fully
// coalesced; four v_cvt_pk_f16_f32 per vector) with at most seven scalar
// elements before and after it.  The kernel is HBM bound: it reads and writes
// 2 bytes per element once.  Its grid is capped so that it
// occupies only part of the chip while the compute stream runs GEMMs, and its
// loads and stores are non-temporal: nothing reads the landing chunk again,
// and the slot is read only by the next block's GEMMs, so the copy should not
// displace the running GEMMs' operands from the caches (measured in the large
// forward: reconstruction 1.12-1.23 -> 1.24-1.29 TB/s busy, MLP up 1.5-2.5%
// faster by the median, MLP down level).
#include "device_common.h"
#include "kernels.h"

namespace dlo {

namespace {

constexpr int kAsmThreads = 256;
constexpr int kAsmUnroll = 4;
constexpr int kAsmMaxBlocks = 512;

__device__ __forceinline__ uint16_t bf16_to_f16(uint16_t b) {
  return static_cast<uint16_t>(bf16x2_to_f16x2(b));
}

__device__ __forceinline__ u32x4_t convert4(u32x4_t v) {
  return u32x4_t{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]), bf16x2_to_f16x2(v[3])};
}

__global__ __launch_bounds__(kAsmThreads) void assemble_vec_kernel(
    uint16_t* __restrict__ dst, const uint16_t* __restrict__ src, int64_t head, int64_t nvec,
    int64_t tail) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kAsmThreads + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kAsmThreads;
  if (blockIdx.x == 0 && threadIdx.x < head) dst[threadIdx.x] = bf16_to_f16(src[threadIdx.x]);
  const u32x4_t* __restrict__ s4 = reinterpret_cast<const u32x4_t*>(src + head);
  u32x4_t* __restrict__ d4 = reinterpret_cast<u32x4_t*>(dst + head);
  int64_t i = tid;
  // Unrolled body: kAsmUnroll independent 16-byte loads in flight per thread.
  for (; i + (kAsmUnroll - 1) * nthreads < nvec; i += kAsmUnroll * nthreads) {
    u32x4_t v[kAsmUnroll];
#pragma unroll
    for (int u = 0; u < kAsmUnroll; ++u) v[u] = __builtin_nontemporal_load(&s4[i + u * nthreads]);
#pragma unroll
    for (int u = 0; u < kAsmUnroll; ++u) __builtin_nontemporal_store(convert4(v[u]), &d4[i + u * nthreads]);
  }
  for (; i < nvec; i += nthreads) __builtin_nontemporal_store(convert4(__builtin_nontemporal_load(&s4[i])), &d4[i]);
  if (blockIdx.x == 0 && threadIdx.x < tail) {
    const int64_t t = head + nvec * 8 + threadIdx.x;
    dst[t] = bf16_to_f16(src[t]);
  }
}

// Fallback for source and destination that differ modulo 16 bytes.
__global__ __launch_bounds__(kAsmThreads) void assemble_scalar_kernel(
    uint16_t* __restrict__ dst, const uint16_t* __restrict__ src, int64_t n) {
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kAsmThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kAsmThreads + threadIdx.x; i < n; i += nthreads)
    dst[i] = bf16_to_f16(src[i]);
}

__global__ __launch_bounds__(kAsmThreads) void fill_nan_kernel(uint16_t* __restrict__ dst, int64_t n) {
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kAsmThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kAsmThreads + threadIdx.x; i < n; i += nthreads)
    dst[i] = 0x7e00u;
}

int grid_for(int64_t work_items) {
  int64_t b = (work_items + kAsmThreads * kAsmUnroll - 1) / (kAsmThreads * kAsmUnroll);
  if (b < 1) b = 1;
  if (b > kAsmMaxBlocks) b = kAsmMaxBlocks;
  return static_cast<int>(b);
}

}  // namespace

hipError_t launch_assemble(uint16_t* dst, const uint16_t* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const uintptr_t da = reinterpret_cast<uintptr_t>(dst), sa = reinterpret_cast<uintptr_t>(src);
  if (((da ^ sa) & 15u) == 0) {
    int64_t head = static_cast<int64_t>(((16u - (da & 15u)) & 15u) / 2u);
    if (head > n) head = n;
    const int64_t nvec = (n - head) / 8;
    const int64_t tail = (n - head) % 8;
    hipLaunchKernelGGL(assemble_vec_kernel, dim3(grid_for(nvec)), dim3(kAsmThreads), 0, s, dst, src,
                       head, nvec, tail);
  } else {
    hipLaunchKernelGGL(assemble_scalar_kernel, dim3(grid_for(n)), dim3(kAsmThreads), 0, s, dst, src, n);
  }
  return hipGetLastError();
}

hipError_t launch_fill_nan(uint16_t* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_nan_kernel, dim3(grid_for(n)), dim3(kAsmThreads), 0, s, dst, n);
  return hipGetLastError();
}

}  // namespace dlo
