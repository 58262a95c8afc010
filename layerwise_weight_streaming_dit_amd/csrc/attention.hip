// Non-causal multi-head attention of the DiT block on gfx950 matrix cores,
// flash-style: the T x T scores are never materialised; each query keeps a
// running max and sum (online softmax) while key/value tiles stream through
// LDS.
//
// Orientation.  A wave owns 32 queries of one head and computes the scores
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_f16: K rows are the A
// operand (8 consecutive head-dim values per lane), the wave's Q rows the B
// operand (kept in registers for the whole key loop).  In the 32x32 result,
// lane l holds query (l % 32) and 16 of the 32 keys, so the softmax state of
// a query lives in one lane pair (l, l ^ 32): row max and row sum need one
// cross-half exchange and no LDS.
//
// Operands are fp16 (q, k, v as written by the projections, P converted from
// the fp32 probabilities), accumulation and softmax fp32.
//
// The output is accumulated transposed too, O^T += V^T P^T: P (fp16) is the B
// operand straight from the S^T registers, and V^T is the A operand.  In the
// S^T layout, lane group g = l / 32 holds key offsets {8a + 4g + b} (a in
// {0,1}, b in 0..3) of each 16-key group; the v projection writes V^T with
// bits 2 and 3 of every key offset swapped (vt_key_position), so each lane's
// 8 keys are one aligned 16-byte run and staging is a plain copy.
//
// Softmax work per score: one max, one FMA (scale and max folded), one exp2,
// one add, half a v_cvt_pk_f16_f32.  The output is rescaled only when a
// query's max grows by more than 2^8 over the reference it uses (a
// wave-uniform branch, usually taken on the first tile only): the
// probabilities are then at most 256 -- exact in fp32 and in range for fp16 --
// and the final division by the running sum is unchanged, so the result is
// the same softmax.  Key masking runs only in the last, partial tile.
//
// Tiles: 256 queries (8 waves, two per SIMD) per workgroup and one workgroup
// per CU, so each K/V tile fetched from L2 feeds 256 queries; 64 keys per
// step, K and V^T double-buffered in LDS with XOR-swizzled 16-byte chunks.
// The next tile moves from global memory straight into LDS (buffer loads
// with the LDS destination, no staging registers) while the current tile is
// processed; one barrier per step publishes it.
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace dlo {

namespace {

constexpr int kBKV = 64;           // keys per step
constexpr float kRescaleSlack = 8.0f;  // log2 of the largest unnormalised probability

// BQ queries per workgroup, 32 per wave: 256 (8 waves, one workgroup per
// CU) normally; 128 (4 waves, two workgroups per CU) when 256-query tiles
// would leave CUs idle (short sequences: T 1000, 4 heads runs in 16 instead
// of 24 us), since with enough tiles the larger tile is faster (T 4096: 154
// vs 175 us).
template <int HD, int BQ>
__global__ __launch_bounds__(BQ * 2, BQ == 256 ? 1 : 2) void attention_kernel(
    const uint16_t* __restrict__ qk, int ld_qk, const uint16_t* __restrict__ vt, int ld_vt,
    uint16_t* __restrict__ o, int ld_o, int T, int H, float scale_log2) {
  constexpr int kAttnThreads = BQ * 2;  // 64 lanes per 32 queries
  constexpr int kBQ = BQ;
  constexpr int KCH = HD / 8;           // 16-byte chunks per K row
  // 16-byte chunk swizzles, so that the 16 lanes the LDS serves together
  // (16 consecutive rows, same logical chunk) hit 16 distinct 16-byte bank
  // groups of the 256-byte bank row: 256-byte rows (K, hd 128) XOR the chunk
  // with row % 16; 128-byte rows (V^T, and K for hd 64) pair rows r and r + 8
  // in the same half of a bank row, so they also XOR with row / 8.
  auto swz = [](int row, int nch) { return nch >= 16 ? (row & 15) : ((row ^ (row >> 3)) & 7); };
  constexpr int NKK = HD / 16;                    // MFMA k-steps over the head dim
  constexpr int NIB = HD / 32;                    // 32-row blocks of O^T

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBKV * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][HD * kBKV];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int kc = lane & 31;
  // Workgroups are dispatched round-robin over the 8 XCDs (workgroup i to XCD
  // i % 8).  When the head count is a multiple of 8, head h runs entirely on
  // XCD h % 8, one head at a time per XCD, so its K and V are fetched from
  // HBM into that XCD's L2 once instead of once per XCD.
  const int nq = (T + kBQ - 1) / kBQ;
  const int bid = blockIdx.x;
  int h, qt;
  if ((H & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3;
    h = (local / nq) * 8 + xcd;
    qt = local % nq;
  } else {
    h = bid / nq;
    qt = bid % nq;
  }
  const int q0 = qt * kBQ + wave * 32;
  const int64_t kcol = static_cast<int64_t>(H) * HD + static_cast<int64_t>(h) * HD;

  // Q fragments (B operand of S^T = K Q^T).
  f16x8_t qf[NKK];
  {
    const int qrow = min(q0 + kc, T - 1);
    const uint16_t* qp = qk + static_cast<int64_t>(qrow) * ld_qk + static_cast<int64_t>(h) * HD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const f16x8_t*>(qp + kk * 16);
  }

  // Staging: every 1 KB block of a K or V^T tile is one DMA load of one wave
  // (64 lanes x 16 bytes, contiguous in LDS), so the chunk swizzle is applied
  // on the global side.  K blocks hold 512 / HD rows of HD values, V^T blocks
  // 8 rows of 64 keys.  Per-lane byte offsets: the K row is clamped to the
  // last token in the last tile; V^T columns past the last token exist
  // (ld_vt covers whole 64-key tiles).
  constexpr int NKB = HD / 8, NVBLK = HD / 8;  // 1 KB blocks per tile (K, V^T)
  constexpr int NW = kAttnThreads / 64;
  constexpr int LPW = (NKB + NVBLK) / NW;       // loads per wave per tile
  static_assert(LPW * NW == NKB + NVBLK, "loads per wave");
  constexpr int KRB = 512 / HD;                // K rows per block
  const __amdgpu_buffer_rsrc_t rs_qk =
      buffer_rsrc(qk, (static_cast<uint32_t>(T - 1) * ld_qk + static_cast<uint32_t>(2 * H * HD)) * 2u);
  const __amdgpu_buffer_rsrc_t rs_vt =
      buffer_rsrc(vt, (static_cast<uint32_t>(H * HD - 1) * ld_vt + static_cast<uint32_t>(ld_vt)) * 2u);
  int ld_row[LPW];
  uint32_t ld_col[LPW];  // K: row in the tile and byte column; V^T: byte offset
  uint32_t ld_lds[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int b = wave * LPW + i;
    if (b < NKB) {
      const int row = b * KRB + lane / KCH, slot = lane % KCH;
      ld_row[i] = row;
      ld_col[i] = static_cast<uint32_t>(kcol + ((slot ^ swz(row, KCH)) << 3)) * 2u;
      ld_lds[i] = b * 512;
    } else {
      const int vb = b - NKB, row = vb * 8 + lane / 8, slot = lane % 8;
      ld_row[i] = 0;
      ld_col[i] = (static_cast<uint32_t>(h * HD + row) * ld_vt + ((slot ^ swz(row, 8)) << 3)) * 2u;
      ld_lds[i] = vb * 512;
    }
  }
  auto load_tile = [&](int key0, int kbuf, int vbuf) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int b = wave * LPW + i;  // uniform
      if (b < NKB) {
        const uint32_t voff = static_cast<uint32_t>(min(ld_row[i], T - 1 - key0)) * ld_qk * 2u + ld_col[i];
        dma16_buf(rs_qk, voff, static_cast<uint32_t>(key0) * ld_qk * 2u, &sK[kbuf][ld_lds[i]]);
      } else {
        dma16_buf(rs_vt, ld_col[i], static_cast<uint32_t>(key0) * 2u, &sV[vbuf][ld_lds[i]]);
      }
    }
  };

  f32x16_t oacc[NIB];
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[ib][r] = 0.f;
  float m_use = -INFINITY;  // reference max (scaled, base 2) the probabilities use
  float l_run = 0.f;        // this lane's half of the running sum

  auto process = [&](auto mask_tag, int t, int cur) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // ---- scores S^T for two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int krow = kb * 32 + kc;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int c = kk * 2 + g;
        const f16x8_t a = *reinterpret_cast<const f16x8_t*>(&sK[cur][krow * HD + ((c ^ swz(krow, KCH)) << 3)]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[kk], s[kb], 0, 0, 0);
      }
    }
    // ---- max over raw scores (the scale is positive)
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (MASK) {
          const int key = t * kBKV + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= T) s[kb][r] = -INFINITY;
        }
        mloc = fmaxf(mloc, s[kb][r]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float mc = mloc * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mc > m_use + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_use, mc);
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
      l_run *= alpha;
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[ib][r] *= alpha;
      m_use = m_new;
    }
    const float nm = -m_use;
    f16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * ks + 2 * e], scale_log2, nm));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * ks + 2 * e + 1], scale_log2, nm));
          l_run += p0 + p1;
          w[e] = pack_f16x2(p0, p1);
        }
        pb[kb][ks] = __builtin_bit_cast(f16x8_t, w);
      }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      const int vrow = ib * 32 + kc;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int c = kb * 4 + ks * 2 + g;
          const f16x8_t a = *reinterpret_cast<const f16x8_t*>(&sV[cur][vrow * kBKV + ((c ^ swz(vrow, 8)) << 3)]);
          oacc[ib] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[kb][ks], oacc[ib], 0, 0, 0);
        }
    }
  };

  const int ntiles = (T + kBKV - 1) / kBKV;
  load_tile(0, 0, 0);
  wait_vmcnt<0>();
  __syncthreads();

  // every tile but the last: no key masking
  for (int t = 0; t + 1 < ntiles; ++t) {
    const int cur = t & 1;
    load_tile((t + 1) * kBKV, cur ^ 1, cur ^ 1);
    process(std::false_type{}, t, cur);
    wait_vmcnt<0>();
    __syncthreads();
  }
  // the last tile, masked only if it is partial
  if (T % kBKV != 0)
    process(std::true_type{}, ntiles - 1, (ntiles - 1) & 1);
  else
    process(std::false_type{}, ntiles - 1, (ntiles - 1) & 1);

  // ---- normalise and store: lane holds query q0 + l%32, head dims
  // ib*32 + 8*rg + 4*g + 0..3 for rg = 0..3 (four consecutive -> 8 bytes).
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  const int qrow = q0 + kc;
  if (qrow < T) {
    uint16_t* op = o + static_cast<int64_t>(qrow) * ld_o + static_cast<int64_t>(h) * HD + 4 * g;
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2_t w;
        w.x = pack_f16x2(oacc[ib][4 * rg] * inv, oacc[ib][4 * rg + 1] * inv);
        w.y = pack_f16x2(oacc[ib][4 * rg + 2] * inv, oacc[ib][4 * rg + 3] * inv);
        *reinterpret_cast<u32x2_t*>(op + ib * 32 + 8 * rg) = w;
      }
  }
}

}  // namespace

hipError_t launch_attention(const uint16_t* qk, int ld_qk, const uint16_t* vt, int ld_vt, uint16_t* o,
                            int ld_o, int tokens, int heads, int head_dim, hipStream_t s) {
  if (tokens <= 0) return hipSuccess;
  const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(head_dim)));
  // 256-query tiles unless they would leave some of the 256 CUs idle
  const bool small = static_cast<int64_t>((tokens + 255) / 256) * heads < 256;
  const int bq = small ? 128 : 256;
  const dim3 grid(((tokens + bq - 1) / bq) * heads), block(bq * 2);
#define DLO_ATTN(HD, BQ) \
  hipLaunchKernelGGL((attention_kernel<HD, BQ>), grid, block, 0, s, qk, ld_qk, vt, ld_vt, o, ld_o, tokens, heads, scale_log2)
  if (head_dim == 128) {
    if (small) DLO_ATTN(128, 128);
    else DLO_ATTN(128, 256);
  } else {
    if (small) DLO_ATTN(64, 128);
    else DLO_ATTN(64, 256);
  }
#undef DLO_ATTN
  return hipGetLastError();
}

}  // namespace dlo
