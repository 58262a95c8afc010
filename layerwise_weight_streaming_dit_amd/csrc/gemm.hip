// Dense projections of the DiT block on gfx950 matrix cores.
//
// acc[i][j] = sum_k A[i][k] * W[j][k]: both operands are K-contiguous
// ("NT"), which is exactly the operand layout of v_mfma_f32_32x32x16_f16:
// lane l supplies 8 consecutive k of row (l % 32), k offset 8 * (l / 32), for
// A and for W alike, and receives a 32x32 fp32 tile in which lane l holds
// column (l % 32) and rows 8 * (r / 4) + 4 * (l / 32) + (r % 4), r = 0..15.
//
// A workgroup computes a BM x BN tile with WM x WN waves; each wave owns a
// (BM / WM) x (BN / WN) sub-tile made of 32x32 MFMA tiles.  K advances in
// steps of 64 through two LDS stages.  Global data moves straight into LDS
// with buffer_load_dwordx4 ... lds (no staging registers), one step
// ahead of the MFMAs that consume it; each row's 64 k values are one full
// 128-byte cache line, so every line is fetched from L2 once per tile.  One
// barrier per step both publishes a landed stage and frees the other one.
// Each wave writes 1 KB of LDS per load instruction (64 lanes x 16 bytes,
// contiguous), so the row/chunk swizzle is applied on the global side: LDS
// slot s holds row s / 8, 16-byte chunk (s % 8) ^ swz(row).
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile order gives
// each XCD a contiguous range of tiles, walked in groups of kGroupM tile rows,
// so tiles that share A rows or W rows share an L2.
//
// Precision: both operands and the biases are fp16 -- the weights are the
// streamed bf16 values as the reconstruction converted them (exact for
// |w| >= 2^-17; smaller magnitudes round to fp16's subnormal grid, |w| > 65504
// would overflow) -- and accumulation is fp32.  (fp16 operands have 3 more
// mantissa bits than bf16 at the same matrix-core rate; with bf16 activations
// the rounding error of a d = 8192 block reaches the 2e-2 output tolerance.)
//
// Epilogues fuse the DiT block's elementwise work into the GEMM:
//   bias -> fp16 (q/k projection), bias + GELU(tanh) -> fp16 (MLP up),
//   x += gate * (acc + bias) in fp32 (attention output and MLP down, the
//   gated residual of adaLN-Zero), and per-row bias -> fp16 (the v projection
//   computed transposed, v^T = Wv h^T, which is the operand layout attention
//   needs for P V; each output column goes to its permuted key position, see
//   vt_key_position).
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace dlo {

namespace {

constexpr int kBK = 64;      // K per stage: one full 128-byte line per row
constexpr int kGroupM = 4;

// 16-byte chunk swizzle of a 128-byte LDS row: keeps the fragment reads of 8
// (32 banks) or 16 (64 banks) consecutive rows on distinct banks.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(GemmArgs g) {
  constexpr int W = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int STAGE_A = BM * kBK, STAGE_B = BN * kBK;  // elements per stage
  constexpr int LA = BM / 8 / W, LB = BN / 8 / W;        // 1 KB DMA loads per wave per stage
  static_assert(LA * 8 * W == BM && LB * 8 * W == BN, "tile/waves mismatch");
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[STAGE_A];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[STAGE_A];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[STAGE_B];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[STAGE_B];

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

  // ---- per-lane global sources of the DMA loads (rows clamped in bounds):
  // LDS slot s of a stage holds row s / 8, 16-byte chunk (s % 8) ^ swz(row).
  uint32_t ga[LA], gb[LB];  // byte offsets from g.a / g.w (host checks they fit 32 bits)
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int slot = (wave * LA + i) * 64 + lane, row = slot >> 3;
    const int c = (slot & 7) ^ swz(row);
    ga[i] = (static_cast<uint32_t>(min(m0 + row, g.M - 1)) * g.lda + c * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int slot = (wave * LB + i) * 64 + lane, row = slot >> 3;
    const int c = (slot & 7) ^ swz(row);
    gb[i] = (static_cast<uint32_t>(min(n0 + row, g.w_rows - 1)) * g.ldw + c * 8) * 2u;
  }
  const int nk = g.K / kBK;

  // buffer descriptors over each operand's extent (the host checks that it
  // fits 32 bits); the per-lane offsets above never reach past it
  const __amdgpu_buffer_rsrc_t rs_a = buffer_rsrc(g.a, (static_cast<uint32_t>(g.M - 1) * g.lda + g.K) * 2u);
  const __amdgpu_buffer_rsrc_t rs_w = buffer_rsrc(g.w, (static_cast<uint32_t>(g.w_rows - 1) * g.ldw + g.K) * 2u);


  auto stageA = [&](auto S) -> uint16_t* {
    if constexpr (decltype(S)::value == 0) return sA0;
    else return sA1;
  };
  auto stageB = [&](auto S) -> uint16_t* {
    if constexpr (decltype(S)::value == 0) return sB0;
    else return sB1;
  };
  // DMA load d of K step `kstep` (clamped to the last step) into stage S:
  // d < LA are this wave's A loads, the rest its W loads.
  auto issue_one = [&](auto S, int kstep, int d) {
    const uint32_t koff = static_cast<uint32_t>(min(kstep, nk - 1)) * (kBK * 2);
    if (d < LA)
      dma16_buf(rs_a, ga[d], koff, stageA(S) + (wave * LA + d) * 512);
    else
      dma16_buf(rs_w, gb[d - LA], koff, stageB(S) + (wave * LB + d - LA) * 512);
  };
  auto issue = [&](auto S, int kstep) {
#pragma unroll
    for (int d = 0; d < LA + LB; ++d) issue_one(S, kstep, d);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

  // Fragments of one 16-wide k slice of a stage.
  auto read_frags = [&](auto S, int ks, f16x8_t (&fa)[TM], f16x8_t (&fb)[TN]) {
    const uint16_t* a = stageA(S);
    const uint16_t* b = stageB(S);
    const int c = ks * 2 + (lane >> 5);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int row = wm * WTM + tm * 32 + (lane & 31);
      fa[tm] = *reinterpret_cast<const f16x8_t*>(a + row * kBK + ((c ^ swz(row)) << 3));
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int row = wn * WTN + tn * 32 + (lane & 31);
      fb[tn] = *reinterpret_cast<const f16x8_t*>(b + row * kBK + ((c ^ swz(row)) << 3));
    }
  };
  // `after_row(tm)` runs after the MFMAs of tile row tm (used to interleave
  // the next step's DMA loads with the matrix work).
  auto mfmas = [&](const f16x8_t (&fa)[TM], const f16x8_t (&fb)[TN], auto&& after_row) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[tn], fa[tm], acc[tm][tn], 0, 0, 0);
      after_row(tm);
    }
  };
  auto nothing = [](int) {};

  // One K step on stage S: wait for this wave's loads of the step, barrier
  // (everyone's loads landed; everyone finished the previous step, whose
  // stage now receives the next step's loads), then four k slices with the
  // fragment reads of slice j+1 in flight while slice j multiplies.
  // sched_barrier(0) fences keep the compiler from sinking each read next to
  // its first use; the explicit lgkmcnt(0) before each batch of reads retires
  // the previous batch, so no wait lands between reads and the MFMAs they
  // overlap.
  f16x8_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  // The next step's LA + LB DMA loads are spread over the tile rows of the
  // first two k slices (kPer after each row), so no wave stalls on a full
  // address queue while it has MFMAs to issue.
  constexpr int kSlots = 2 * TM, kPer = (LA + LB + kSlots - 1) / kSlots;
  auto step = [&](auto S, int kt) {
    constexpr int s = decltype(S)::value;
    auto dma_after = [&](int slot) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int d = slot * kPer + j;
        if (d < LA + LB) {
          issue_one(IC<s ^ 1>{}, kt + 1, d);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // this step's loads (issued during the previous step) have landed
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    read_frags(S, 0, fa0, fb0);
    wait_lgkmcnt0();
    read_frags(S, 1, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa0, fb0, [&](int tm) { dma_after(tm); });
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    read_frags(S, 2, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa1, fb1, [&](int tm) { dma_after(TM + tm); });
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    read_frags(S, 3, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa0, fb0, nothing);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    mfmas(fa1, fb1, nothing);
  };

  issue(IC<0>{}, 0);
  // K is a multiple of two steps (128), so the ring unrolls without early exits
  for (int kt = 0; kt < nk; kt += 2) {
    step(IC<0>{}, kt);
    step(IC<1>{}, kt + 1);
  }
  wait_vmcnt<0>();  // drain the clamped tail loads before the epilogue

  // ---- epilogue.  The MFMAs above take W as their first operand, so each
  // 32x32 accumulator is a tile of C^T: lane l owns output row (l % 32) of the
  // tile and, for q = 0..3, the four consecutive output columns
  // 8q + 4(l / 32) + 0..3 (registers 4q..4q+3).  N is a multiple of 16, so a
  // group of four (or eight) columns is either wholly inside or wholly past
  // the last column.
  int col[TN][4];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int q = 0; q < 4; ++q) col[tn][q] = n0 + wn * WTN + tn * 32 + 8 * q + 4 * (lane >> 5);
  // Outputs go out through LDS.  In the C^T accumulator layout a lane holds
  // 4 consecutive columns of 32 different rows, so a direct store writes
  // 8- or 16-byte pieces of 32 rows per instruction (and the gated residual's
  // loads, placed after stores to the same buffer, could not be batched).
  // Staged row-major in the idle stage buffers (padded rows, one region per
  // wave), each instruction instead moves whole row segments: fp16 outputs
  // 8 rows x 128 bytes (the wave's 64 columns; two tile rows per pass), the
  // fp32 residual 4 rows x 256 bytes (one tile row per pass).  Interior
  // tiles store unguarded; edge tiles clamp their loads and guard their
  // stores.
  auto rows_out_lds = [&](auto guarded) {
    constexpr bool GUARD = decltype(guarded)::value;
    constexpr int RS = 72;  // LDS row stride in halves (16-byte aligned rows)
    constexpr int PR = 64;  // output rows per pass
    static_assert(WTN == 64 && WTM % PR == 0, "wave tile");
    static_assert((W / 4) * PR * RS * 2 <= STAGE_B * 2 && STAGE_B <= STAGE_A && W % 4 == 0, "epilogue region");
    __syncthreads();  // every wave is done reading the stage buffers
    const int arr = wave / (W / 4), sub = wave % (W / 4);
    uint16_t* region = (arr == 0 ? sA0 : arr == 1 ? sA1 : arr == 2 ? sB0 : sB1) + sub * PR * RS;
#pragma unroll
    for (int p = 0; p < WTM / PR; ++p) {
#pragma unroll
      for (int i = 0; i < PR / 32; ++i) {
        const int tm = p * (PR / 32) + i;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4_t v;
            v.x = acc[tm][tn][4 * q];
            v.y = acc[tm][tn][4 * q + 1];
            v.z = acc[tm][tn][4 * q + 2];
            v.w = acc[tm][tn][4 * q + 3];
            int c = tn * 32 + 8 * q + 4 * (lane >> 5);  // column in the wave's 64
            if constexpr (EPI == EPI_VT_F16) {
              // transposed v: per-row bias; tokens c..c+3 land at their
              // permuted key positions, consecutive too (the tile's first
              // column is a multiple of 16, and only bits 2 and 3 move)
              const float rb = f16_to_f32(g.bias[min(m0 + wm * WTM + tm * 32 + (lane & 31), g.M - 1)]);
              v += rb;
              c = vt_key_position(c);
            } else {
              const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(g.bias + min(col[tn][q], g.N - 4));
              v += f16x4_to_f32x4(bb);
            }
            if constexpr (EPI == EPI_BIAS_GELU_F16) {
              v.x = gelu_tanh(v.x);
              v.y = gelu_tanh(v.y);
              v.z = gelu_tanh(v.z);
              v.w = gelu_tanh(v.w);
            }
            u32x2_t w;
            w.x = pack_f16x2(v.x, v.y);
            w.y = pack_f16x2(v.z, v.w);
            *reinterpret_cast<u32x2_t*>(region + (i * 32 + (lane & 31)) * RS + c) = w;
          }
      }
#pragma unroll
      for (int k = 0; k < PR / 8; ++k) {
        const int r = k * 8 + (lane >> 3), c8 = (lane & 7) * 8;
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(region + r * RS + c8);
        const int row = m0 + wm * WTM + p * PR + r, cc = n0 + wn * WTN + c8;
        if (!GUARD || (row < g.M && cc < g.N))
          *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(g.out) + static_cast<int64_t>(row) * g.ldo + cc) = val;
      }
    }
  };
  // Gated fp32 residual: acc + bias is staged, then x = x + gate * (acc + bias)
  // (one fused multiply-add) row segment by row segment, the tile row's x
  // loads all issued before its stores.
  auto rows_out_lds_f32 = [&](auto guarded) {
    constexpr bool GUARD = decltype(guarded)::value;
    constexpr int RS = 68;  // LDS row stride in floats (16-byte aligned rows)
    static_assert(WTN == 64, "wave tile");
    static_assert((W / 4) * 32 * RS * 4 <= STAGE_B * 2 && STAGE_B <= STAGE_A && W % 4 == 0, "epilogue region");
    __syncthreads();  // every wave is done reading the stage buffers
    const int arr = wave / (W / 4), sub = wave % (W / 4);
    float* region = reinterpret_cast<float*>(arr == 0 ? sA0 : arr == 1 ? sA1 : arr == 2 ? sB0 : sB1) + sub * 32 * RS;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(g.bias + min(col[tn][q], g.N - 4));
          const f32x4_t bf = f16x4_to_f32x4(bb);
          f32x4_t v;
          v.x = acc[tm][tn][4 * q] + bf.x;
          v.y = acc[tm][tn][4 * q + 1] + bf.y;
          v.z = acc[tm][tn][4 * q + 2] + bf.z;
          v.w = acc[tm][tn][4 * q + 3] + bf.w;
          *reinterpret_cast<f32x4_t*>(region + (lane & 31) * RS + tn * 32 + 8 * q + 4 * (lane >> 5)) = v;
        }
      const int c4 = (lane & 15) * 4, cc = n0 + wn * WTN + c4;
      const f32x4_t gt = *reinterpret_cast<const f32x4_t*>(g.gate + (GUARD ? min(cc, g.N - 4) : cc));
      f32x4_t xr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = m0 + wm * WTM + tm * 32 + k * 4 + (lane >> 4);
        const int64_t off = static_cast<int64_t>(GUARD ? min(row, g.M - 1) : row) * g.ldo + (GUARD ? min(cc, g.N - 4) : cc);
        xr[k] = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(g.out) + off);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = k * 4 + (lane >> 4);
        const int row = m0 + wm * WTM + tm * 32 + r;
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(region + r * RS + c4);
        if (!GUARD || (row < g.M && cc < g.N))
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(g.out) + static_cast<int64_t>(row) * g.ldo + cc) = xr[k] + gt * v;
      }
    }
  };
  const bool interior = m0 + BM <= g.M && n0 + BN <= g.N;
  if constexpr (EPI == EPI_BIAS_F16 || EPI == EPI_BIAS_GELU_F16 || EPI == EPI_VT_F16) {
    if (interior)
      rows_out_lds(std::false_type{});
    else
      rows_out_lds(std::true_type{});
  } else {
    if (interior)
      rows_out_lds_f32(std::false_type{});
    else
      rows_out_lds_f32(std::true_type{});
  }
}

// ---------------------------------------------------------------------------
// 256 x BN tile with ONE wave per SIMD (four waves).
//   BN = 256: the waves split the tile along the dimension of the activation
//   operand, so each wave owns its own slice of the weight operand (no two
//   waves read the same weight fragments):
//     WM=1, WN=4: waves own 64 weight rows (columns of C), 256x64 per wave;
//     WM=4, WN=1: the transposed v projection (weights are the A operand),
//                 waves own 64 weight rows, 64x256 per wave.
//   BN = 128 (the long-K shapes with too few 256x256 tiles): a 2 x 2 wave
//   grid, 128x64 per wave.
// Per 64-wide K step a BN = 256 wave issues 64 MFMAs (256 fp32 accumulators
// per lane in the accumulation registers) against 40 fragment reads, a
// BN = 128 wave 32 MFMAs against 24.  With no second
// wave on the SIMD the stream is pipelined by hand:
//   * the fragments of k slice j+1 are read one after each of slice j's
//     first ten MFMAs; the stage loads are buffer loads (dma16_buf), so the
//     compiler's waits for the reads are exact and each MFMA of the next
//     slice waits only for its own fragments;
//   * the step's barrier sits before the last slice's MFMAs: every wave has
//     read all four slices of the stage by then and waited for its loads of
//     the next step, so after the barrier the next stage is complete and this
//     one may be overwritten;
//   * the loads of step kt+2 into the stage just released start right after
//     that barrier (ten during the last slice, six during the next step's
//     first slice), so they have three slices to land;
//   * load addresses are a uniform base (scalar registers, advanced per step)
//     plus a fixed per-lane offset; the LDS destination of every load is
//     uniform too, so issuing a load costs no vector instruction.
template <int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(256) void gemm_wt_kernel(GemmArgs g) {
  constexpr int BM = 256, W = 4;
  static_assert(WM * WN == W, "four waves");
  constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  constexpr int MF = TM * TN;        // MFMAs per k slice
  constexpr int STAGE_A = BM * kBK, STAGE_B = BN * kBK;
  constexpr int LA = BM / 8 / W, LB = BN / 8 / W;  // 1 KB DMA loads per wave per operand per stage
  constexpr int ND = LA + LB;        // DMA loads per wave per step
  constexpr bool A_IS_WEIGHT = EPI == EPI_VT_F16;
  constexpr int NWF = A_IS_WEIGHT ? TM : TN;  // weight fragments per slice
  static_assert(MF % NWF == 0 && TM + TN <= MF, "slice shape");
  static_assert(WTM % 64 == 0 && WTN % 64 == 0, "fragment addressing assumes an even tile count per wave");

  __shared__ __attribute__((aligned(1024))) uint16_t sA0[STAGE_A];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[STAGE_A];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[STAGE_B];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[STAGE_B];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile order: XCD-contiguous ranges, grouped along M
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int nb = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int logical = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  // groups of 8 tile rows for long-K products over 32 or more tile columns
  // (warm, same box: MLP down of the large block 8192x8192x32768 3782 ->
  // 3597 us, 8192x8192x16384 1820 -> 1789 us; shorter K or fewer columns
  // measured level or up to 2.5% slower with 8)
  const int group_m = (g.K >= 16384 && tiles_n >= 32) ? 8 : kGroupM;
  const int group_span = group_m * tiles_n;
  const int group = logical / group_span;
  const int first_m = group * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int in_group = logical - group * group_span;
  const int tile_m = first_m + in_group % gsz;
  const int tile_n = in_group / gsz;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  // ---- DMA sources: per-lane byte offsets (rows clamped in bounds) from a
  // uniform base; LDS slot s of a stage holds row s / 8, 16-byte chunk
  // (s % 8) ^ swz(row)
  uint32_t ga[LA], gb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int slot = (wave * LA + i) * 64 + lane, row = slot >> 3;
    const int c = (slot & 7) ^ swz(row);
    ga[i] = (static_cast<uint32_t>(min(m0 + row, g.M - 1)) * g.lda + c * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int slot = (wave * LB + i) * 64 + lane, row = slot >> 3;
    const int c = (slot & 7) ^ swz(row);
    gb[i] = (static_cast<uint32_t>(min(n0 + row, g.w_rows - 1)) * g.ldw + c * 8) * 2u;
  }
  const int nk = g.K / kBK;

  auto stageA = [&](auto S) -> uint16_t* {
    if constexpr (decltype(S)::value == 0) return sA0;
    else return sA1;
  };
  auto stageB = [&](auto S) -> uint16_t* {
    if constexpr (decltype(S)::value == 0) return sB0;
    else return sB1;
  };
  // buffer descriptors over each operand's extent (the host checks that it
  // fits 32 bits); the per-lane offsets above never reach past it
  const __amdgpu_buffer_rsrc_t rs_a = buffer_rsrc(g.a, (static_cast<uint32_t>(g.M - 1) * g.lda + g.K) * 2u);
  const __amdgpu_buffer_rsrc_t rs_w = buffer_rsrc(g.w, (static_cast<uint32_t>(g.w_rows - 1) * g.ldw + g.K) * 2u);
  // DMA load d (< ND) of K step `kstep` (clamped) into stage S: per-lane
  // offset plus the step's uniform byte offset
  auto issue_one = [&](auto S, int kstep, int d) {
    const uint32_t kb = static_cast<uint32_t>(min(kstep, nk - 1)) * (kBK * 2);
    if (d < LA)
      dma16_buf(rs_a, ga[d], kb, stageA(S) + (wave * LA + d) * 512);
    else
      dma16_buf(rs_w, gb[d - LA], kb, stageB(S) + (wave * LB + d - LA) * 512);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

  // Fragment pipeline: fragments double-buffered by slice parity (four
  // slices per step: parities 0, 1, 0, 1).
  f16x8_t ra[2][TM], rb[2][TN];
  // Fragment addresses.  Tile rows are 32 apart, so within a wave's rows
  // (which start at a multiple of 32) the chunk swizzle of fragment row
  // R + (lane % 32) is swz(lane % 32) ^ 4 for odd tiles and swz(lane % 32) for
  // even ones: per k slice two per-lane offsets serve every tile, the tile
  // itself being a constant offset.
  int fo[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int l = lane & 31;
      fo[ks][par] = l * kBK + ((((ks * 2 + (lane >> 5)) ^ swz(l)) ^ (4 * par)) << 3);
    }
  const int arow0 = wm * WTM * kBK, brow0 = wn * WTN * kBK;  // uniform
  auto read_frags = [&](auto S, int ks, auto P) {
    constexpr int p = decltype(P)::value;
    const uint16_t* a = stageA(S) + arow0;
    const uint16_t* b = stageB(S) + brow0;
    auto rd_a = [&] {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        ra[p][tm] = *reinterpret_cast<const f16x8_t*>(a + tm * 32 * kBK + fo[ks][tm & 1]);
    };
    auto rd_b = [&] {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        rb[p][tn] = *reinterpret_cast<const f16x8_t*>(b + tn * 32 * kBK + fo[ks][tn & 1]);
    };
    // the weight fragments first, in the order the MFMAs use them
    if constexpr (A_IS_WEIGHT) {
      rd_a();
      rd_b();
    } else {
      rd_b();
      rd_a();
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // fragment read j (< TM + TN; the weight fragments first) of k slice ks of
  // stage S into parity P
  auto read_one = [&](auto S, int ks, auto P, int j) {
    constexpr int p = decltype(P)::value;
    constexpr int NW = A_IS_WEIGHT ? TM : TN;
    const bool wfrag = j < NW;
    const int t = wfrag ? j : j - NW;
    if (A_IS_WEIGHT == wfrag)
      ra[p][t] = *reinterpret_cast<const f16x8_t*>(stageA(S) + arow0 + t * 32 * kBK + fo[ks][t & 1]);
    else
      rb[p][t] = *reinterpret_cast<const f16x8_t*>(stageB(S) + brow0 + t * 32 * kBK + fo[ks][t & 1]);
  };
  // The 16 MFMAs of the slice of parity P; after MFMA i, rd(i) (fragment
  // read i of the next slice, into parity P ^ 1) and dma(i).  The compiler's
  // LDS waits are exact (see dma16_buf): each MFMA waits only for its own
  // fragments.
  auto mfma_slice = [&](auto P, auto&& dma, auto&& rd) {
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      // weight fragment outer: each weight fragment is done with early
      const int wf = i / (MF / NWF), af = i % (MF / NWF);
      const int tm = A_IS_WEIGHT ? wf : af, tn = A_IS_WEIGHT ? af : wf;
      acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rb[p][tn], ra[p][tm], acc[tm][tn], 0, 0, 0);
      rd(i);
      dma(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // DMA loads of the step after next issued in the slice after the barrier;
  // the rest go out during the next step's first slice
  constexpr int NEARLY = ND * 5 / 8;
  static_assert(NEARLY <= MF && ND - NEARLY <= MF, "loads per slice");
  auto step = [&](auto S, int kt) {
    constexpr int s = decltype(S)::value;
    auto dma_range = [&](auto T, int kstep, int first, int count) {
      return [&, T, kstep, first, count](int i) {
        if (i < count) issue_one(T, kstep, first + i);
      };
    };
    auto none = [](int) {};
    auto reads = [&](auto T, int ks, auto P) {
      return [&, T, ks, P](int i) {
        if (i < TM + TN) read_one(T, ks, P, i);
      };
    };
    mfma_slice(IC<0>{}, dma_range(IC<s ^ 1>{}, kt + 1, NEARLY, ND - NEARLY), reads(S, 1, IC<1>{}));
    mfma_slice(IC<1>{}, none, reads(S, 2, IC<0>{}));
    mfma_slice(IC<0>{}, none, reads(S, 3, IC<1>{}));
    // step kt+1's loads have landed and slice 3 is in registers: publish the
    // next stage, release this one
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mfma_slice(IC<1>{}, dma_range(S, kt + 2, 0, NEARLY), reads(IC<s ^ 1>{}, 0, IC<0>{}));
  };

#pragma unroll
  for (int d = 0; d < ND; ++d) issue_one(IC<0>{}, 0, d);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  read_frags(IC<0>{}, 0, IC<0>{});
#pragma unroll
  for (int d = 0; d < NEARLY; ++d) issue_one(IC<1>{}, 1, d);
  wait_lgkmcnt0();
  // K is a multiple of two steps (128), so the ring unrolls without early exits
  for (int kt = 0; kt < nk; kt += 2) {
    step(IC<0>{}, kt);
    step(IC<1>{}, kt + 1);
  }
  wait_vmcnt<0>();  // drain the clamped tail loads before the epilogue
  __syncthreads();  // every wave is done with the stage buffers
  // keep the accumulator reads below (spilling them otherwise)
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue through LDS (each wave its own 32 KB region), one 32-row
  // tile row per pass.  Each 32x32 accumulator is a tile of C^T: lane l owns
  // output row (l % 32) of the tile and, for q = 0..3, the four consecutive
  // columns 8q + 4(l / 32) + 0..3.
  uint16_t* region = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sB0 : sB1;
  const bool interior = m0 + BM <= g.M && n0 + BN <= g.N;
  const int row0 = m0 + wm * WTM, col0 = n0 + wn * WTN;
  if constexpr (EPI == EPI_GATED_F32) {
    // x = x + gate * (acc + bias): staged as fp32 rows of WTN (+4) floats,
    // then whole row segments, the pass's x loads issued before its stores
    constexpr int RS = WTN + 4, LPR = WTN / 4, RPI = 64 / LPR, NI = 32 / RPI;
    float* fr = reinterpret_cast<float*>(region);
    const int c4 = (lane % LPR) * 4, cc = col0 + c4;
    const bool col_ok = cc < g.N;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = tn * 32 + 8 * q + 4 * (lane >> 5);
          const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(g.bias + min(col0 + c, g.N - 4));
          const f32x4_t bf = f16x4_to_f32x4(bb);
          f32x4_t v;
          v.x = acc[tm][tn][4 * q] + bf.x;
          v.y = acc[tm][tn][4 * q + 1] + bf.y;
          v.z = acc[tm][tn][4 * q + 2] + bf.z;
          v.w = acc[tm][tn][4 * q + 3] + bf.w;
          *reinterpret_cast<f32x4_t*>(fr + (lane & 31) * RS + c) = v;
        }
      const f32x4_t gt = *reinterpret_cast<const f32x4_t*>(g.gate + min(cc, g.N - 4));
      // half a pass at a time: its x loads, then its stores
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4_t xr[NI / 2];
#pragma unroll
        for (int k = 0; k < NI / 2; ++k) {
          const int row = row0 + tm * 32 + (h * NI / 2 + k) * RPI + lane / LPR;
          const int64_t off = static_cast<int64_t>(interior ? row : min(row, g.M - 1)) * g.ldo +
                              (interior ? cc : min(cc, g.N - 4));
          xr[k] = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(g.out) + off);
        }
#pragma unroll
        for (int k = 0; k < NI / 2; ++k) {
          const int r = (h * NI / 2 + k) * RPI + lane / LPR, row = row0 + tm * 32 + r;
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(fr + r * RS + c4);
          if (interior || (row < g.M && col_ok))
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(g.out) + static_cast<int64_t>(row) * g.ldo + cc) =
                xr[k] + gt * v;
        }
      }
    }
  } else {
    // fp16 results: staged as rows of WTN (+8) halves, then whole row
    // segments of 16 bytes per lane
    constexpr int RS = WTN + 8, LPR = WTN / 8, RPI = 64 / LPR, NI = 32 / RPI;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4_t v;
          v.x = acc[tm][tn][4 * q];
          v.y = acc[tm][tn][4 * q + 1];
          v.z = acc[tm][tn][4 * q + 2];
          v.w = acc[tm][tn][4 * q + 3];
          int c = tn * 32 + 8 * q + 4 * (lane >> 5);
          if constexpr (EPI == EPI_VT_F16) {
            // transposed v: per-row bias; tokens c..c+3 land at their
            // permuted key positions, consecutive too (the tile's first
            // column is a multiple of 16, and only bits 2 and 3 move)
            v += f16_to_f32(g.bias[min(row0 + tm * 32 + (lane & 31), g.M - 1)]);
            c = vt_key_position(c);
          } else {
            const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(g.bias + min(col0 + c, g.N - 4));
            v += f16x4_to_f32x4(bb);
          }
          if constexpr (EPI == EPI_BIAS_GELU_F16) {
            v.x = gelu_tanh(v.x);
            v.y = gelu_tanh(v.y);
            v.z = gelu_tanh(v.z);
            v.w = gelu_tanh(v.w);
          }
          u32x2_t w;
          w.x = pack_f16x2(v.x, v.y);
          w.y = pack_f16x2(v.z, v.w);
          *reinterpret_cast<u32x2_t*>(region + (lane & 31) * RS + c) = w;
        }
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int r = k * RPI + lane / LPR, c8 = (lane % LPR) * 8;
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(region + r * RS + c8);
        const int row = row0 + tm * 32 + r, cc = col0 + c8;
        if (interior || (row < g.M && cc < g.N))
          *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(g.out) + static_cast<int64_t>(row) * g.ldo + cc) = val;
      }
    }
  }
}

template <int BN, int WM, int WN, int WMV, int WNV>
hipError_t launch_wt(int epi, const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + 255) / 256) * ((g.N + BN - 1) / BN);
  const dim3 grid(tiles), block(256);
  switch (epi) {
    case EPI_BIAS_F16:
      hipLaunchKernelGGL((gemm_wt_kernel<BN, WM, WN, EPI_BIAS_F16>), grid, block, 0, s, g);
      break;
    case EPI_BIAS_GELU_F16:
      hipLaunchKernelGGL((gemm_wt_kernel<BN, WM, WN, EPI_BIAS_GELU_F16>), grid, block, 0, s, g);
      break;
    case EPI_GATED_F32:
      hipLaunchKernelGGL((gemm_wt_kernel<BN, WM, WN, EPI_GATED_F32>), grid, block, 0, s, g);
      break;
    default:
      hipLaunchKernelGGL((gemm_wt_kernel<BN, WMV, WNV, EPI_VT_F16>), grid, block, 0, s, g);
      break;
  }
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_shape(int epi, const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  const dim3 grid(tiles), block(WM * WN * 64);
  switch (epi) {
    case EPI_BIAS_F16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_BIAS_F16>), grid, block, 0, s, g);
      break;
    case EPI_BIAS_GELU_F16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_BIAS_GELU_F16>), grid, block, 0, s, g);
      break;
    case EPI_GATED_F32:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_GATED_F32>), grid, block, 0, s, g);
      break;
    default:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_VT_F16>), grid, block, 0, s, g);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int epilogue, const GemmArgs& g, hipStream_t s) {
  // Largest tile that still gives every CU (256) at least one workgroup.
  // From one 256x256 tile per CU up, the one-wave-per-SIMD kernel is ahead
  // (measured on warm operands, same results bit for bit: 1-9% on the image
  // shapes with one or two tiles per CU, 5-10% on the large and mid-video
  // shapes).  Its 256x128 form (2 x 2 waves) pays off over a long K (MLP
  // down of the image block, 4096x2048x8192: 137 -> 127 us warm, 152 -> 144
  // us by the median inside the forward, against the eight-wave-style
  // 256x128 kernel with an L2 prefetch it replaces); for short K two 128x128
  // tiles per CU (8 waves) finish first (2048x4096x2048: 34.5 vs 35.6 us).
  const int64_t t256 = static_cast<int64_t>((g.M + 255) / 256) * ((g.N + 255) / 256);
  const int64_t t256x128 = static_cast<int64_t>((g.M + 255) / 256) * ((g.N + 127) / 128);
  if (t256 >= 256) return launch_wt<256, 1, 4, 4, 1>(epilogue, g, s);
  if (t256x128 >= 256 && g.K >= 4096) return launch_wt<128, 2, 2, 2, 2>(epilogue, g, s);
  return launch_shape<128, 128, 2, 2>(epilogue, g, s);
}

}  // namespace dlo
