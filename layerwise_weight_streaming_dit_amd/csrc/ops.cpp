// Kernel-level entry points: validate on the host, then launch the same
// kernel dlo_forward launches for that step.
#include <hip/hip_runtime_api.h>

#include "common.h"
#include "dlo_ops.h"
#include "kernels.h"

using namespace dlo;

namespace {

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

dlo_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DLO_E_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return DLO_OK;
}

}  // namespace

extern "C" DLO_API dlo_status dlo_op_assemble(uint16_t* dst, const uint16_t* src, int64_t n, hipStream_t s) {
  return guarded([&]() -> dlo_status {
    clear_error();
    if (n < 0) return fail(DLO_E_INVAL, "n %lld < 0", (long long)n);
    if (n == 0) return DLO_OK;
    if (dst == nullptr || src == nullptr) return fail(DLO_E_INVAL, "NULL pointer");
    if (!aligned(dst, 2) || !aligned(src, 2)) return fail(DLO_E_INVAL, "pointers must be 2-byte aligned");
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst), a = reinterpret_cast<uintptr_t>(src);
    if (d < a + size_t(n) * 2 && a < d + size_t(n) * 2) return fail(DLO_E_INVAL, "ranges overlap");
    return launched(launch_assemble(dst, src, n, s), "assemble");
  });
}

extern "C" DLO_API dlo_status dlo_op_adaln(const uint16_t* w, const uint16_t* b, const float* cond, float* mod,
                                           int32_t rows, int32_t c, hipStream_t s) {
  return guarded([&]() -> dlo_status {
    clear_error();
    if (!w || !b || !cond || !mod) return fail(DLO_E_INVAL, "NULL pointer");
    if (rows < 1) return fail(DLO_E_INVAL, "rows %d < 1", rows);
    if (c < 64 || c % 64 != 0 || c > 4096) return fail(DLO_E_SHAPE, "c %d must be a multiple of 64 in [64, 4096]", c);
    if (!aligned(w, 8) || !aligned(cond, 4) || !aligned(mod, 4)) return fail(DLO_E_INVAL, "misaligned pointer");
    return launched(launch_adaln(w, b, cond, mod, rows, c, s), "adaln");
  });
}

extern "C" DLO_API dlo_status dlo_op_ln_modulate(const float* xin, int32_t d_in, float* xout, const float* shift,
                                                 const float* scale, uint16_t* h, int32_t tokens, int32_t d,
                                                 hipStream_t s) {
  return guarded([&]() -> dlo_status {
    clear_error();
    if (!xin || !shift || !scale || !h) return fail(DLO_E_INVAL, "NULL pointer");
    if (tokens < 0) return fail(DLO_E_INVAL, "tokens %d < 0", tokens);
    if (d < 4 || d % 4 != 0 || d > 8192) return fail(DLO_E_SHAPE, "d %d must be a multiple of 4 in [4, 8192]", d);
    if (d_in < 4 || d_in % 4 != 0) return fail(DLO_E_SHAPE, "d_in %d must be a positive multiple of 4", d_in);
    if (!aligned(xin, 16) || !aligned(shift, 16) || !aligned(scale, 16) || !aligned(h, 8) ||
        (xout && !aligned(xout, 16)))
      return fail(DLO_E_INVAL, "misaligned pointer");
    return launched(launch_ln_modulate(xin, d_in, xout, shift, scale, h, tokens, d, s), "ln_modulate");
  });
}

extern "C" DLO_API dlo_status dlo_op_gemm(int32_t epilogue, const uint16_t* a, int32_t lda, const uint16_t* w,
                                          int32_t ldw, int32_t w_rows, const uint16_t* bias, const float* gate,
                                          void* out, int32_t ldo, int32_t M, int32_t N, int32_t K,
                                          hipStream_t s) {
  return guarded([&]() -> dlo_status {
    clear_error();
    if (epilogue < DLO_EPI_BIAS_F16 || epilogue > DLO_EPI_VT_F16)
      return fail(DLO_E_INVAL, "unknown epilogue %d", epilogue);
    if (!a || !w || !bias || !out) return fail(DLO_E_INVAL, "NULL pointer");
    if (epilogue == DLO_EPI_GATED_F32 && !gate) return fail(DLO_E_INVAL, "gate is NULL");
    if (M < 1 || N < 16 || N % 16 != 0 || K < 128 || K % 128 != 0)
      return fail(DLO_E_SHAPE, "M %d, N %d, K %d (N a multiple of 16, K of 128)", M, N, K);
    if (w_rows < 1 || w_rows > N) return fail(DLO_E_SHAPE, "w_rows %d outside [1, N=%d]", w_rows, N);
    if (lda < K || ldw < K || lda % 8 || ldw % 8) return fail(DLO_E_SHAPE, "lda %d / ldw %d must be >= K and multiples of 8", lda, ldw);
    // the epilogue writes 16-byte row pieces: 8 fp16 or 4 fp32 columns
    const int ldo_mult = epilogue == DLO_EPI_GATED_F32 ? 4 : 8;
    if (ldo < N || ldo % ldo_mult)
      return fail(DLO_E_SHAPE, "ldo %d must be >= N %d and a multiple of %d", ldo, N, ldo_mult);
    // the kernel addresses both operands with 32-bit byte offsets
    if ((int64_t(M - 1) * lda + K) * 2 > int64_t(UINT32_MAX) || (int64_t(w_rows - 1) * ldw + K) * 2 > int64_t(UINT32_MAX))
      return fail(DLO_E_SHAPE, "operand extent beyond 4 GiB (M %d x lda %d, w_rows %d x ldw %d)", M, lda, w_rows, ldw);
    if (!aligned(a, 16) || !aligned(w, 16)) return fail(DLO_E_INVAL, "operands must be 16-byte aligned");
    if (!aligned(out, 16) || !aligned(bias, epilogue == DLO_EPI_VT_F16 ? 2 : 8) ||
        (gate && !aligned(gate, 16)))
      return fail(DLO_E_INVAL, "out, bias or gate misaligned for vector access");
    GemmArgs g{a, w, bias, gate, out, lda, ldw, ldo, M, N, K, w_rows};
    return launched(launch_gemm(epilogue, g, s), "gemm");
  });
}

extern "C" DLO_API dlo_status dlo_op_attention(const uint16_t* qk, int32_t ld_qk, const uint16_t* vt, int32_t ld_vt,
                                               uint16_t* o, int32_t ld_o, int32_t tokens, int32_t heads,
                                               int32_t head_dim, hipStream_t s) {
  return guarded([&]() -> dlo_status {
    clear_error();
    if (!qk || !vt || !o) return fail(DLO_E_INVAL, "NULL pointer");
    if (head_dim != 64 && head_dim != 128) return fail(DLO_E_SHAPE, "head_dim %d must be 64 or 128", head_dim);
    if (tokens < 1 || heads < 1) return fail(DLO_E_SHAPE, "tokens %d, heads %d", tokens, heads);
    const int64_t d = int64_t(heads) * head_dim;
    if (ld_qk < 2 * d || ld_qk % 8) return fail(DLO_E_SHAPE, "ld_qk %d must be >= 2*d and a multiple of 8", ld_qk);
    if (ld_o < d || ld_o % 4) return fail(DLO_E_SHAPE, "ld_o %d must be >= d and a multiple of 4", ld_o);
    const int64_t tp = (int64_t(tokens) + 63) / 64 * 64;
    if (ld_vt < tp || ld_vt % 64) return fail(DLO_E_SHAPE, "ld_vt %d must be >= %lld and a multiple of 64", ld_vt, (long long)tp);
    // the kernel addresses q, k and v^T with 32-bit byte offsets
    if ((int64_t(tokens - 1) * ld_qk + 2 * d) * 2 > int64_t(UINT32_MAX) || d * ld_vt * 2 > int64_t(UINT32_MAX))
      return fail(DLO_E_SHAPE, "operand extent beyond 4 GiB (tokens %d x ld_qk %d, d %lld x ld_vt %d)", tokens, ld_qk,
                  (long long)d, ld_vt);
    if (!aligned(qk, 16) || !aligned(vt, 16) || !aligned(o, 8)) return fail(DLO_E_INVAL, "misaligned pointer");
    return launched(launch_attention(qk, ld_qk, vt, ld_vt, o, ld_o, tokens, heads, head_dim, s), "attention");
  });
}
