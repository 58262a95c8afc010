// adaLN modulation vector and LayerNorm + modulate, the two HBM-bound
// per-token steps of the DiT block (adaLN-Zero conditioning of Peebles & Xie,
// "Scalable Diffusion Models with Transformers", section 3.2).
#include "device_common.h"
#include "kernels.h"

namespace dlo {

namespace {

constexpr int kNormThreads = 256;
constexpr int kAdaRowsPerWave = 4;

// mod[r] = W[r] . silu(cond) + b[r].  silu(cond) is staged once per workgroup
// in LDS; each wave computes kAdaRowsPerWave rows at once: the rows' loads
// (8 bytes per lane per 256 columns) and their biases are all issued before
// any arithmetic, and the rows' wave reductions are independent chains, so
// the GEMV costs a few memory round trips per wave instead of a few per row.
__global__ __launch_bounds__(kNormThreads) void adaln_kernel(const uint16_t* __restrict__ w,
                                                             const uint16_t* __restrict__ b,
                                                             const float* __restrict__ cond,
                                                             float* __restrict__ mod, int rows,
                                                             int c) {
  __shared__ float sc[4096];
  for (int j = threadIdx.x; j < c; j += kNormThreads) sc[j] = silu(cond[j]);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = (blockIdx.x * (kNormThreads / 64) + wave) * kAdaRowsPerWave;
  // rows past the end read the last row (in bounds) and store nothing
  const float bias = f16_to_f32(b[min(r0 + min(lane, kAdaRowsPerWave - 1), rows - 1)]);
  float acc[kAdaRowsPerWave];
#pragma unroll
  for (int rr = 0; rr < kAdaRowsPerWave; ++rr) acc[rr] = 0.f;
  for (int j = lane * 4; j < c; j += 256) {
    u32x2_t v[kAdaRowsPerWave];
#pragma unroll
    for (int rr = 0; rr < kAdaRowsPerWave; ++rr)
      v[rr] = *reinterpret_cast<const u32x2_t*>(w + static_cast<int64_t>(min(r0 + rr, rows - 1)) * c + j);
    const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(sc + j);
#pragma unroll
    for (int rr = 0; rr < kAdaRowsPerWave; ++rr) {
      const f32x4_t wv = f16x4_to_f32x4(v[rr]);
      acc[rr] += wv.x * s4.x + wv.y * s4.y + wv.z * s4.z + wv.w * s4.w;
    }
  }
  float mine = 0.f;
#pragma unroll
  for (int rr = 0; rr < kAdaRowsPerWave; ++rr) {
    const float t = wave_sum(acc[rr]);
    if (lane == rr) mine = t;
  }
  if (lane < kAdaRowsPerWave && r0 + lane < rows) mod[r0 + lane] = mine + bias;
}

// One wave per token row, four rows per workgroup: the row (adapted to width
// d) is held in registers, NV float4 per lane (NV * 256 >= d), so mean and
// variance are wave reductions with no LDS or barrier, and every lane has NV
// loads in flight.  The register cap keeps 4 waves per SIMD resident for
// d <= 2048, 2 up to 6144 (d = 6144 needs 232 registers and no spills);
// wider rows use the workgroup-per-row kernel below.
//
// shift and scale are shared by the workgroup's four rows: they are staged in
// LDS once (their loads overlap the rows' loads), so the output loop reads
// them from LDS -- global loads there would sit behind the previous float4's
// stores (possible aliasing) and cost a memory round trip each.
template <int NV>
__global__ __launch_bounds__(256, NV <= 8 ? 4 : 2) void ln_modulate_kernel(
    const float* __restrict__ xin, int d_in, float* __restrict__ xout, const float* __restrict__ shift,
    const float* __restrict__ scale, uint16_t* __restrict__ h, int tokens, int d) {
  __shared__ f32x4_t s_sh[NV * 64], s_sc[NV * 64];
  const int lane = threadIdx.x & 63;
  const int64_t t_raw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const bool row_ok = t_raw < tokens;  // rows past the end compute on the last row and store nothing
  const int64_t t = row_ok ? t_raw : tokens - 1;
  const float* xr = xin + t * d_in;
  const int nv = d / 4;
  const int lim = min(nv, d_in / 4);  // float4s of the row that come from xin
  f32x4_t v[NV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    // every lane loads (clamped in bounds) and zeroes what lies past the
    // input row: no divergent branch around the loads
    const int q = lane + i * 64;
    const f32x4_t l = *reinterpret_cast<const f32x4_t*>(xr + min(q, lim - 1) * 4);
    const bool in = q < lim;
    v[i] = f32x4_t{in ? l.x : 0.f, in ? l.y : 0.f, in ? l.z : 0.f, in ? l.w : 0.f};
    s += v[i].x + v[i].y + v[i].z + v[i].w;
  }
  for (int j = threadIdx.x; j < nv; j += 256) {
    s_sh[j] = *reinterpret_cast<const f32x4_t*>(shift + j * 4);
    s_sc[j] = *reinterpret_cast<const f32x4_t*>(scale + j * 4);
  }
  const float mean = wave_sum(s) / static_cast<float>(d);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int q = lane + i * 64;
    if (q < nv) {
      const f32x4_t e = v[i] - mean;
      ss += e.x * e.x + e.y * e.y + e.z * e.z + e.w * e.w;
    }
  }
  const float var = wave_sum(ss) / static_cast<float>(d);
  const float rstd = rsqrtf(var + 1e-6f);
  __syncthreads();  // shift and scale staged
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int q = lane + i * 64;
    if (row_ok && q < nv) {
      const f32x4_t sh = s_sh[q];
      const f32x4_t sc = s_sc[q];
      const f32x4_t y = (v[i] - mean) * rstd * (1.0f + sc) + sh;
      u32x2_t o;
      o.x = pack_f16x2(y.x, y.y);
      o.y = pack_f16x2(y.z, y.w);
      *reinterpret_cast<u32x2_t*>(h + t * d + q * 4) = o;
      if (xout != nullptr) *reinterpret_cast<f32x4_t*>(xout + t * d + q * 4) = v[i];
    }
  }
}

template <int THREADS>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // red may still be read from a previous reduction
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < THREADS / 64; ++i) t += red[i];
  return t;
}

// Wide rows (d > 6144): one workgroup per token row.  The row (adapted to
// width d) is held in registers, at most two float4 per thread (1024 threads
// for d = 8192, so registers stay few and occupancy high); mean and variance
// are workgroup reductions over the registers.
template <int THREADS, int NV>
__global__ __launch_bounds__(THREADS) void ln_modulate_row_kernel(
    const float* __restrict__ xin, int d_in, float* __restrict__ xout, const float* __restrict__ shift,
    const float* __restrict__ scale, uint16_t* __restrict__ h, int d) {
  __shared__ float red[THREADS / 64];
  const int64_t t = blockIdx.x;
  const float* xr = xin + t * d_in;
  const int nv = d / 4;
  f32x4_t v[NV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int q = threadIdx.x + i * THREADS;
    v[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (q < nv && q * 4 < d_in) v[i] = *reinterpret_cast<const f32x4_t*>(xr + q * 4);
    s += v[i].x + v[i].y + v[i].z + v[i].w;
  }
  // shift and scale load with the row (before any store of this thread)
  f32x4_t shv[NV], scv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int q = min(static_cast<int>(threadIdx.x) + i * THREADS, nv - 1);
    shv[i] = *reinterpret_cast<const f32x4_t*>(shift + q * 4);
    scv[i] = *reinterpret_cast<const f32x4_t*>(scale + q * 4);
  }
  const float mean = block_sum<THREADS>(s, red) / static_cast<float>(d);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int q = threadIdx.x + i * THREADS;
    if (q < nv) {
      const f32x4_t e = v[i] - mean;
      ss += e.x * e.x + e.y * e.y + e.z * e.z + e.w * e.w;
    }
  }
  const float var = block_sum<THREADS>(ss, red) / static_cast<float>(d);
  const float rstd = rsqrtf(var + 1e-6f);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int q = threadIdx.x + i * THREADS;
    if (q < nv) {
      const f32x4_t sh = shv[i];
      const f32x4_t sc = scv[i];
      const f32x4_t y = (v[i] - mean) * rstd * (1.0f + sc) + sh;
      u32x2_t o;
      o.x = pack_f16x2(y.x, y.y);
      o.y = pack_f16x2(y.z, y.w);
      *reinterpret_cast<u32x2_t*>(h + t * d + q * 4) = o;
      if (xout != nullptr) *reinterpret_cast<f32x4_t*>(xout + t * d + q * 4) = v[i];
    }
  }
}

}  // namespace

hipError_t launch_adaln(const uint16_t* w, const uint16_t* b, const float* cond, float* mod,
                        int rows, int c, hipStream_t s) {
  const int rows_per_block = (kNormThreads / 64) * kAdaRowsPerWave;
  const int grid = (rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(adaln_kernel, dim3(grid), dim3(kNormThreads), 0, s, w, b, cond, mod, rows, c);
  return hipGetLastError();
}

hipError_t launch_ln_modulate(const float* xin, int d_in, float* xout, const float* shift,
                              const float* scale, uint16_t* h, int tokens, int d, hipStream_t s) {
  if (tokens <= 0) return hipSuccess;
  const dim3 grid((tokens + 3) / 4), block(256);
#define DLO_LN(NV) \
  hipLaunchKernelGGL((ln_modulate_kernel<NV>), grid, block, 0, s, xin, d_in, xout, shift, scale, h, tokens, d)
  if (d <= 256) DLO_LN(1);
  else if (d <= 512) DLO_LN(2);
  else if (d <= 1024) DLO_LN(4);
  else if (d <= 2048) DLO_LN(8);
  else if (d <= 4096) DLO_LN(16);
  else if (d <= 6144) DLO_LN(24);
  else
    hipLaunchKernelGGL((ln_modulate_row_kernel<1024, 2>), dim3(tokens), dim3(1024), 0, s, xin, d_in, xout, shift,
                       scale, h, d);
#undef DLO_LN
  return hipGetLastError();
}

}  // namespace dlo
