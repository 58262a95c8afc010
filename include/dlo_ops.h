/*
 * dlo_ops.h -- kernel-level entry points of the streamed DiT forward.
 *
 * Each call launches exactly the kernel dlo_forward launches for that step,
 * on the caller's stream, without a context.  They exist so each step can be
 * checked against the oracle and timed on its own.  All pointers are device
 * pointers; bf16 and fp16 values are their 16-bit patterns.  Weights arrive
 * as bf16 (as streamed) and dlo_op_assemble converts them to fp16 while
 * reconstructing, so the other calls take fp16 weights and biases, as the
 * forward's kernels read them from the slot; activations between kernels are
 * fp16 (fp16 has three more mantissa bits than bf16 and runs the matrix cores
 * at the same rate; with bf16 activations the rounding error of the widest
 * block reaches the 2e-2 output tolerance).  Calls are asynchronous
 * with respect to the host.  Shapes are validated on the host before any
 * launch (DLO_E_INVAL / DLO_E_SHAPE, nothing enqueued); a failed launch
 * returns DLO_E_HIP.  Error messages come from dlo_last_error().
 */
#ifndef DLO_OPS_H
#define DLO_OPS_H

#include "dlo.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reconstruction (the single-GPU stand-in for all_gather_into_tensor,
 * release page section "Weight sharding with AllGather reconstruction"):
 * dst[i] = fp16(src[i]) for the bf16 values src[i], i in [0, n), rounded to
 * nearest even (exact for |src[i]| >= 2^-17; rounded to fp16's subnormal grid
 * below, error <= 2^-25; inf above 65504).  Any 2-byte alignment is
 * accepted; when dst and src have the same address modulo 16 bytes the kernel
 * works in 16-byte vectors with a scalar head and tail, which is how
 * dlo_forward lands every chunk.  The ranges must not overlap. */
DLO_API dlo_status dlo_op_assemble(uint16_t* dst, const uint16_t* src, int64_t n,
                                   hipStream_t stream);

/* adaLN modulation (DiT adaLN-Zero conditioning):
 * mod[r] = sum_j w[r][j] * silu(cond[j]) + b[r] for r in [0, rows), fp32
 * accumulation.  w: fp16 [rows][c] row-major; b: fp16 [rows]; cond, mod: fp32.
 * c must be a multiple of 64 and at most 4096. */
DLO_API dlo_status dlo_op_adaln(const uint16_t* w, const uint16_t* b, const float* cond,
                                float* mod, int32_t rows, int32_t c, hipStream_t stream);

/* LayerNorm (no affine, eps 1e-6, population variance) + modulation:
 * for each token t, y = adapt(xin[t]) where xin rows have width d_in and
 * adapt keeps the first min(d_in, d) features and zero-fills the rest;
 * h[t][j] = fp16(LN(y)[j] * (1 + scale[j]) + shift[j]).  If xout is not NULL
 * the adapted row y (fp32, width d) is written to xout[t] as well (the
 * residual handed to a block of another width).  d must be a multiple of 4
 * and at most 8192; d_in a multiple of 4. */
DLO_API dlo_status dlo_op_ln_modulate(const float* xin, int32_t d_in, float* xout,
                                      const float* shift, const float* scale, uint16_t* h,
                                      int32_t tokens, int32_t d, hipStream_t stream);

/* GEMM on MFMA: acc[i][j] = sum_k a[i][k] * w[j][k] for i in [0, M), j in
 * [0, N), fp32 accumulation.  Both operands are fp16: one is a weight matrix
 * (as dlo_op_assemble writes it), the other activations: for DLO_EPI_VT_F16 `a` is
 * the weight and `w` the activation, for every other epilogue `a` is the
 * activation and `w` the weight.  Rows of w at or past w_rows are read as row
 * w_rows - 1 (so padded output columns stay finite).  Epilogues (fp16
 * results rounded to nearest even):
 *   DLO_EPI_BIAS_F16       out fp16 [M][ldo]:  out[i][j] = acc + bias[j]
 *   DLO_EPI_BIAS_GELU_F16  out fp16 [M][ldo]:  out[i][j] = gelu_tanh(acc + bias[j])
 *   DLO_EPI_GATED_F32      out fp32 [M][ldo]:  out[i][j] += gate[j] * (acc + bias[j])
 *   DLO_EPI_VT_F16         out fp16 [M][ldo]:  out[i][p(j)] = acc + bias[i]
 * where p(j) swaps bits 2 and 3 of j (the transposed v layout attention
 * reads, see dlo_op_attention).  bias is fp16, gate fp32.  M >= 1; N a
 * multiple of 16; K a multiple of 128; lda, ldw multiples of 8 and >= K;
 * ldo >= N and a multiple of 8 (of 4 for the fp32 epilogue), so that every
 * output row starts 16-byte aligned; 1 <= w_rows <= N; a, w and out 16-byte
 * aligned, bias 8-byte (column bias), gate 16-byte. */
#define DLO_EPI_BIAS_F16 0
#define DLO_EPI_BIAS_GELU_F16 1
#define DLO_EPI_GATED_F32 2
#define DLO_EPI_VT_F16 3
DLO_API dlo_status dlo_op_gemm(int32_t epilogue, const uint16_t* a, int32_t lda, const uint16_t* w,
                               int32_t ldw, int32_t w_rows, const uint16_t* bias, const float* gate,
                               void* out, int32_t ldo, int32_t M, int32_t N, int32_t K,
                               hipStream_t stream);

/* Non-causal multi-head attention on MFMA with online softmax:
 * for head h and token t, o[t][h*hd + i] = fp16(sum_s p[t][s] v[s][h*hd + i])
 * with p = softmax_s(q[t] . k[s] / sqrt(hd)), fp32 softmax and accumulation;
 * q, k, v and the probabilities enter the matrix cores as fp16.
 * q[t][c] = qk[t*ld_qk + c] and k[t][c] = qk[t*ld_qk + heads*hd + c]
 * (the q and k thirds of the QKV projection, row-major); v is given
 * transposed with its keys permuted inside every aligned group of 16:
 * v[s][c] = vt[c*ld_vt + p(s)], p(s) = s with bits 2 and 3 swapped (so the
 * eight keys one lane multiplies are one aligned 16-byte run); ld_vt >=
 * tokens rounded up to 64, a multiple of 64, and the columns that hold keys
 * >= tokens finite.  hd = head_dim in {64, 128}.  The q/k extent
 * ((tokens - 1) * ld_qk + 2 * heads * hd) and the v^T extent
 * (heads * hd * ld_vt) must each stay within 4 GiB (DLO_E_SHAPE otherwise). */
DLO_API dlo_status dlo_op_attention(const uint16_t* qk, int32_t ld_qk, const uint16_t* vt,
                                    int32_t ld_vt, uint16_t* o, int32_t ld_o, int32_t tokens,
                                    int32_t heads, int32_t head_dim, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DLO_OPS_H */
