// Dense projections of the DiT block on gfx950 matrix cores.
//
// acc[i][j] = sum_k A[i][k] * W[j][k]: both operands are K-contiguous
// ("NT"), which is exactly the operand layout of v_mfma_f32_32x32x16_bf16:
// lane l supplies 8 consecutive k of row (l % 32), k offset 8 * (l / 32), for
// A and for W alike, and receives a 32x32 fp32 tile in which lane l holds
// column (l % 32) and rows 8 * (r / 4) + 4 * (l / 32) + (r % 4), r = 0..15.
//
// A workgroup computes a BM x BN tile with WM x WN waves; each wave owns a
// (BM / WM) x (BN / WN) sub-tile made of 32x32 MFMA tiles.  K advances in
// steps of 64: each step's A and W tiles are staged in LDS (double-buffered,
// one barrier per step) with 16-byte chunks XOR-swizzled by row, so the
// 16-byte fragment reads of 8 consecutive rows hit distinct banks.  The next
// step's global loads are issued before the current step's MFMAs.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile order gives
// each XCD a contiguous range of tiles, walked in groups of kGroupM tile rows,
// so tiles that share A rows or W rows share an L2.
//
// Epilogues fuse the DiT block's elementwise work into the GEMM:
//   bias -> bf16 (q/k projection), bias + GELU(tanh) -> bf16 (MLP up),
//   x += gate * (acc + bias) in fp32 (attention output and MLP down, the
//   gated residual of adaLN-Zero), and per-row bias -> bf16 (the v projection
//   computed transposed, v^T = Wv h^T, which is the operand layout attention
//   needs for P V; each output column goes to its permuted key position, see
//   vt_key_position).
#include "device_common.h"
#include "kernels.h"

namespace dlo {

namespace {

constexpr int kBK = 64;
constexpr int kGroupM = 8;

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(GemmArgs g) {
  constexpr int THREADS = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int LA = BM * 8 / THREADS, LB = BN * 8 / THREADS;
  static_assert(LA * THREADS == BM * 8 && LB * THREADS == BN * 8, "tile/threads mismatch");

  __shared__ __attribute__((aligned(16))) uint16_t smA[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t smB[2][BN * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile order: XCD-contiguous ranges, grouped along M
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int nb = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int logical = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int group_span = kGroupM * tiles_n;
  const int group = logical / group_span;
  const int first_m = group * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * group_span;
  const int tile_m = first_m + in_group % gsz;
  const int tile_n = in_group / gsz;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  // ---- global -> register staging addresses (clamped rows keep loads in bounds)
  const uint16_t* pa[LA];
  const uint16_t* pb[LB];
  int la_off[LA], lb_off[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int q = tid + i * THREADS, row = q >> 3, c = q & 7;
    const int gr = min(m0 + row, g.M - 1);
    pa[i] = g.a + static_cast<int64_t>(gr) * g.lda + c * 8;
    la_off[i] = row * kBK + ((c ^ (row & 7)) << 3);
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int q = tid + i * THREADS, row = q >> 3, c = q & 7;
    const int gr = min(n0 + row, g.w_rows - 1);
    pb[i] = g.w + static_cast<int64_t>(gr) * g.ldw + c * 8;
    lb_off[i] = row * kBK + ((c ^ (row & 7)) << 3);
  }

  // ---- fragment read offsets (elements) for k-substep 0; substep ks adds
  // chunk 2*ks, applied through the same XOR.
  int fa_row[TM], fb_row[TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) fa_row[tm] = wm * WTM + tm * 32 + (lane & 31);
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) fb_row[tn] = wn * WTN + tn * 32 + (lane & 31);
  const int fchunk = lane >> 5;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

  u32x4_t ra[LA], rb[LB];
  const int nk = g.K / kBK;

#pragma unroll
  for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(pa[i]);
#pragma unroll
  for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(pb[i]);
#pragma unroll
  for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4_t*>(&smA[0][la_off[i]]) = ra[i];
#pragma unroll
  for (int i = 0; i < LB; ++i) *reinterpret_cast<u32x4_t*>(&smB[0][lb_off[i]]) = rb[i];
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int koff = (kt + 1) * kBK;
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(pa[i] + koff);
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(pb[i] + koff);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t fa[TM], fb[TN];
      const int c = ks * 2 + fchunk;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int row = fa_row[tm];
        fa[tm] = *reinterpret_cast<const bf16x8_t*>(&smA[cur][row * kBK + ((c ^ (row & 7)) << 3)]);
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int row = fb_row[tn];
        fb[tn] = *reinterpret_cast<const bf16x8_t*>(&smB[cur][row * kBK + ((c ^ (row & 7)) << 3)]);
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4_t*>(&smA[cur ^ 1][la_off[i]]) = ra[i];
#pragma unroll
      for (int i = 0; i < LB; ++i) *reinterpret_cast<u32x4_t*>(&smB[cur ^ 1][lb_off[i]]) = rb[i];
    }
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int col = n0 + wn * WTN + tn * 32 + (lane & 31);
    if (col >= g.N) continue;
    float cbias = 0.f, cgate = 0.f;
    if constexpr (EPI != EPI_ROWBIAS_BF16) cbias = bf16_to_f32(g.bias[col]);
    if constexpr (EPI == EPI_GATED_F32) cgate = g.gate[col];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WTM + tm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= g.M) continue;
        const float v = acc[tm][tn][r];
        const int64_t o = static_cast<int64_t>(row) * g.ldo + col;
        if constexpr (EPI == EPI_BIAS_BF16) {
          static_cast<uint16_t*>(g.out)[o] = f32_to_bf16(v + cbias);
        } else if constexpr (EPI == EPI_BIAS_GELU_BF16) {
          static_cast<uint16_t*>(g.out)[o] = f32_to_bf16(gelu_tanh(v + cbias));
        } else if constexpr (EPI == EPI_GATED_F32) {
          float* x = static_cast<float*>(g.out);
          x[o] = x[o] + cgate * (v + cbias);
        } else {
          // transposed v: token `col` lands at its permuted key position
          const int64_t ot = static_cast<int64_t>(row) * g.ldo + vt_key_position(col);
          static_cast<uint16_t*>(g.out)[ot] = f32_to_bf16(v + bf16_to_f32(g.bias[row]));
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_shape(int epi, const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  const dim3 grid(tiles), block(WM * WN * 64);
  switch (epi) {
    case EPI_BIAS_BF16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_BIAS_BF16>), grid, block, 0, s, g);
      break;
    case EPI_BIAS_GELU_BF16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_BIAS_GELU_BF16>), grid, block, 0, s, g);
      break;
    case EPI_GATED_F32:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_GATED_F32>), grid, block, 0, s, g);
      break;
    default:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_ROWBIAS_BF16>), grid, block, 0, s, g);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int epilogue, const GemmArgs& g, hipStream_t s) {
  // Largest tile that still gives every CU (256) at least one workgroup.
  const int64_t t256 = static_cast<int64_t>((g.M + 255) / 256) * ((g.N + 255) / 256);
  const int64_t t256x128 = static_cast<int64_t>((g.M + 255) / 256) * ((g.N + 127) / 128);
  if (t256 >= 256) return launch_shape<256, 256, 2, 4>(epilogue, g, s);
  if (t256x128 >= 256) return launch_shape<256, 128, 2, 2>(epilogue, g, s);
  return launch_shape<128, 128, 2, 2>(epilogue, g, s);
}

}  // namespace dlo
