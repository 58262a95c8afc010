// Host-only checks of the C ABI's layout arithmetic and argument validation,
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_native_host.py (g++, no GPU).
//
// The translation units under test are layout.cpp (block layout, shard size,
// error reporting) and ops.cpp (validation and marshalling of the
// kernel-level entry points).  The kernel launchers are replaced by recorders
// below, so every call that passes validation hands its arguments to a
// launcher that records them instead of touching a device; pointers are
// fabricated addresses that are never dereferenced.
//
// Facts checked, from the release page's section "Weight sharding with
// AllGather reconstruction": the shard size is ceil(numel / dp); the flat
// weight is a dense concatenation of the parameters at cached offsets.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>

#include "dlo.h"
#include "dlo_ops.h"
#include "kernels.h"

namespace {

int g_failures = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: CHECK failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                        \
    }                                                                      \
  } while (0)

// What the recorders saw last.
struct Seen {
  int calls = 0;
  int epilogue = -1;
  dlo::GemmArgs gemm{};
  int64_t n = 0;
  int rows = 0, c = 0, tokens = 0, d = 0, d_in = 0, heads = 0, head_dim = 0;
  int ld_qk = 0, ld_vt = 0, ld_o = 0;
  const void* p0 = nullptr;
  const void* p1 = nullptr;
} g_seen;

template <typename T>
T* fake(uintptr_t addr) {
  return reinterpret_cast<T*>(addr);
}

}  // namespace

namespace dlo {

hipError_t launch_assemble(uint16_t* dst, const uint16_t* src, int64_t n, hipStream_t) {
  ++g_seen.calls;
  g_seen.p0 = dst;
  g_seen.p1 = src;
  g_seen.n = n;
  return hipSuccess;
}

hipError_t launch_fill_nan(uint16_t*, int64_t, hipStream_t) { return hipSuccess; }

hipError_t launch_adaln(const uint16_t* w, const uint16_t*, const float*, float*, int rows, int c,
                        hipStream_t) {
  ++g_seen.calls;
  g_seen.p0 = w;
  g_seen.rows = rows;
  g_seen.c = c;
  return hipSuccess;
}

hipError_t launch_ln_modulate(const float* xin, int d_in, float*, const float*, const float*, uint16_t* h,
                              int tokens, int d, hipStream_t) {
  ++g_seen.calls;
  g_seen.p0 = xin;
  g_seen.p1 = h;
  g_seen.d_in = d_in;
  g_seen.tokens = tokens;
  g_seen.d = d;
  return hipSuccess;
}

hipError_t launch_gemm(int epilogue, const GemmArgs& g, hipStream_t) {
  ++g_seen.calls;
  g_seen.epilogue = epilogue;
  g_seen.gemm = g;
  return hipSuccess;
}

hipError_t launch_attention(const uint16_t* qk, int ld_qk, const uint16_t* vt, int ld_vt, uint16_t*, int ld_o,
                            int tokens, int heads, int head_dim, hipStream_t) {
  ++g_seen.calls;
  g_seen.p0 = qk;
  g_seen.p1 = vt;
  g_seen.ld_qk = ld_qk;
  g_seen.ld_vt = ld_vt;
  g_seen.ld_o = ld_o;
  g_seen.tokens = tokens;
  g_seen.heads = heads;
  g_seen.head_dim = head_dim;
  return hipSuccess;
}

}  // namespace dlo

namespace {

bool has_error_text() { return dlo_last_error() != nullptr && dlo_last_error()[0] != '\0'; }

int64_t expected_numel(int64_t d, int64_t m, int64_t c, const int64_t* extra, int n_extra) {
  int64_t n = 3 * d * d + 3 * d + d * d + d + m * d + m + d * m + d + 6 * d * c + 6 * d;
  for (int e = 0; e < n_extra; ++e) n += extra[e];
  return n;
}

void check_layouts() {
  const int64_t extra[3] = {0, 7, 1000};
  const int shapes[][4] = {{128, 2, 128, 64}, {256, 4, 1024, 128}, {1152, 18, 4608, 256}, {2048, 16, 8192, 256},
                           {3072, 24, 12288, 256}, {128, 1, 256, 4096}};
  for (auto& s : shapes) {
    for (int n_extra = 0; n_extra <= 3; n_extra += 3) {
      dlo_block_desc b{s[0], s[1], s[2], s[3], n_extra, 0, n_extra ? extra : nullptr};
      const int64_t want = expected_numel(s[0], s[2], s[3], extra, n_extra);
      for (int dp = 1; dp <= 17; ++dp) {
        int64_t numel = -1, shard = -1;
        int32_t np = -1;
        dlo_param_desc params[16];
        CHECK(dlo_block_layout(&b, dp, &numel, &shard, &np, params, 16) == DLO_OK);
        CHECK(numel == want);
        CHECK(shard == (numel + dp - 1) / dp);
        CHECK(int64_t(dp) * shard - numel >= 0 && int64_t(dp) * shard - numel <= dp - 1);
        CHECK(np == 10 + n_extra);
        // dense concatenation in the documented order
        int64_t off = 0;
        const char* names[10] = {"Wqkv", "bqkv", "Wo", "bo", "W1", "b1", "W2", "b2", "Wada", "bada"};
        for (int i = 0; i < np; ++i) {
          CHECK(params[i].offset == off);
          if (i < 10) CHECK(strcmp(params[i].name, names[i]) == 0);
          int64_t n = 1;
          for (int k = 0; k < params[i].ndim; ++k) n *= params[i].shape[k];
          off += n;
        }
        CHECK(off == numel);
      }
      // cap below the parameter count is an error, with a message
      dlo_param_desc small[4];
      CHECK(dlo_block_layout(&b, 2, nullptr, nullptr, nullptr, small, 4) == DLO_E_INVAL);
      CHECK(has_error_text());
    }
  }
  // every invalid field is rejected with a message; nothing else is touched
  const dlo_block_desc good{256, 4, 1024, 128, 0, 0, nullptr};
  const int64_t bad_len[1] = {-1};
  dlo_block_desc bad[] = {good, good, good, good, good, good, good, good, good, good};
  bad[0].d_model = 100;     // not a multiple of 128
  bad[1].d_model = 8320;    // above 8192
  bad[2].n_heads = 3;       // does not divide d
  bad[3].n_heads = 1;       // head dim 256
  bad[4].d_mlp = 96;        // not a multiple of 128
  bad[5].d_cond = 32;       // below 64
  bad[6].d_cond = 4160;     // above 4096
  bad[7].n_extra = 65;      // too many extras
  bad[8].n_extra = 1;       // extra_len NULL
  bad[9].n_extra = 1;       // negative extra length
  bad[9].extra_len = bad_len;
  for (auto& b : bad) {
    int64_t numel = 123;
    CHECK(dlo_block_layout(&b, 4, &numel, nullptr, nullptr, nullptr, 0) == DLO_E_INVAL);
    CHECK(numel == 123);
    CHECK(has_error_text());
  }
  CHECK(dlo_block_layout(nullptr, 4, nullptr, nullptr, nullptr, nullptr, 0) == DLO_E_INVAL);
  CHECK(dlo_block_layout(&good, 0, nullptr, nullptr, nullptr, nullptr, 0) == DLO_E_INVAL);
  // a good call clears the previous message
  CHECK(dlo_block_layout(&good, 4, nullptr, nullptr, nullptr, nullptr, 0) == DLO_OK);
  CHECK(!has_error_text());
}

void check_gemm() {
  auto a = fake<uint16_t>(0x100000), w = fake<uint16_t>(0x200000), bias = fake<uint16_t>(0x300000);
  auto gate = fake<float>(0x400000);
  auto out = fake<void>(0x500000);
  // a valid call reaches the launcher with every argument in place
  g_seen = Seen{};
  CHECK(dlo_op_gemm(DLO_EPI_GATED_F32, a, 8192, w, 8192, 2048, bias, gate, out, 2048, 4096, 2048, 8192, nullptr) ==
        DLO_OK);
  CHECK(g_seen.calls == 1 && g_seen.epilogue == DLO_EPI_GATED_F32);
  const dlo::GemmArgs& g = g_seen.gemm;
  CHECK(g.a == a && g.w == w && g.bias == bias && g.gate == gate && g.out == out);
  CHECK(g.lda == 8192 && g.ldw == 8192 && g.ldo == 2048 && g.M == 4096 && g.N == 2048 && g.K == 8192 &&
        g.w_rows == 2048);
  // shape, alignment and range errors never reach the launcher
  struct Bad {
    int epi, lda, ldw, w_rows, ldo, M, N, K;
    uintptr_t a_addr, out_addr;
  } cases[] = {
      {7, 128, 128, 16, 16, 1, 16, 128, 0x100000, 0x500000},           // unknown epilogue
      {0, 128, 128, 16, 16, 0, 16, 128, 0x100000, 0x500000},           // M = 0
      {0, 128, 128, 16, 24, 1, 24, 128, 0x100000, 0x500000},           // N not a multiple of 16
      {0, 192, 192, 16, 16, 1, 16, 192, 0x100000, 0x500000},           // K not a multiple of 128
      {0, 120, 128, 16, 16, 1, 16, 128, 0x100000, 0x500000},           // lda < K
      {0, 132, 128, 16, 16, 1, 16, 128, 0x100000, 0x500000},           // lda not a multiple of 8
      {0, 128, 128, 17, 16, 1, 16, 128, 0x100000, 0x500000},           // w_rows > N
      {0, 128, 128, 16, 12, 1, 16, 128, 0x100000, 0x500000},           // ldo < N
      {0, 128, 128, 16, 16, 1, 16, 128, 0x100008, 0x500000},           // a not 16-byte aligned
      {2, 128, 128, 16, 16, 1, 16, 128, 0x100000, 0x500008},           // fp32 out not 16-byte aligned
      {0, 128, 128, 16, 16, 1, 16, 128, 0x100000, 0x500008},           // fp16 out not 16-byte aligned
      {3, 128, 128, 16, 16, 1, 16, 128, 0x100000, 0x500008},           // transposed out not 16-byte aligned
      {0, 128, 128, 16, 20, 1, 16, 128, 0x100000, 0x500000},           // fp16 ldo not a multiple of 8
      {1, 128, 128, 16, 20, 1, 16, 128, 0x100000, 0x500000},           // GELU ldo not a multiple of 8
      {0, 16384, 128, 16, 16, (1 << 17) + 1, 16, 128, 0x100000, 0x500000},  // a beyond 4 GiB
  };
  for (auto& c : cases) {
    g_seen = Seen{};
    const dlo_status st = dlo_op_gemm(c.epi, fake<uint16_t>(c.a_addr), c.lda, w, c.ldw, c.w_rows, bias, gate,
                                      fake<void>(c.out_addr), c.ldo, c.M, c.N, c.K, nullptr);
    CHECK(st == DLO_E_INVAL || st == DLO_E_SHAPE);
    CHECK(g_seen.calls == 0);
    CHECK(has_error_text());
  }
  // fp32 rows need only 4-column strides (16 bytes)
  g_seen = Seen{};
  CHECK(dlo_op_gemm(DLO_EPI_GATED_F32, a, 128, w, 128, 16, bias, gate, out, 20, 1, 16, 128, nullptr) == DLO_OK);
  CHECK(g_seen.calls == 1 && g_seen.gemm.ldo == 20);
  // the largest operand that still fits 32-bit offsets is accepted
  g_seen = Seen{};
  CHECK(dlo_op_gemm(0, a, 16384, w, 128, 16, bias, nullptr, out, 16, 1 << 17, 16, 128, nullptr) == DLO_OK);
  CHECK(g_seen.calls == 1);
  // gated epilogue needs a gate
  CHECK(dlo_op_gemm(DLO_EPI_GATED_F32, a, 128, w, 128, 16, bias, nullptr, out, 16, 1, 16, 128, nullptr) ==
        DLO_E_INVAL);
}

void check_other_ops() {
  // assemble: n = 0 is a no-op, overlap is rejected, a valid call is forwarded
  g_seen = Seen{};
  CHECK(dlo_op_assemble(nullptr, nullptr, 0, nullptr) == DLO_OK && g_seen.calls == 0);
  CHECK(dlo_op_assemble(fake<uint16_t>(0x1000), fake<uint16_t>(0x1000 + 2 * 99), 100, nullptr) == DLO_E_INVAL);
  CHECK(dlo_op_assemble(fake<uint16_t>(0x1001), fake<uint16_t>(0x9000), 100, nullptr) == DLO_E_INVAL);
  CHECK(dlo_op_assemble(fake<uint16_t>(0x1000), fake<uint16_t>(0x9000), -1, nullptr) == DLO_E_INVAL);
  CHECK(g_seen.calls == 0);
  CHECK(dlo_op_assemble(fake<uint16_t>(0x1000), fake<uint16_t>(0x1000 + 2 * 100), 100, nullptr) == DLO_OK);
  CHECK(g_seen.calls == 1 && g_seen.n == 100);

  // adaLN: c a multiple of 64 in [64, 4096]
  auto w = fake<uint16_t>(0x2000), b = fake<uint16_t>(0x3000);
  auto cond = fake<float>(0x4000), mod = fake<float>(0x5000);
  g_seen = Seen{};
  CHECK(dlo_op_adaln(w, b, cond, mod, 12288, 256, nullptr) == DLO_OK);
  CHECK(g_seen.calls == 1 && g_seen.rows == 12288 && g_seen.c == 256);
  CHECK(dlo_op_adaln(w, b, cond, mod, 12288, 96, nullptr) == DLO_E_SHAPE);
  CHECK(dlo_op_adaln(w, b, cond, mod, 12288, 4160, nullptr) == DLO_E_SHAPE);
  CHECK(dlo_op_adaln(w, b, cond, mod, 0, 256, nullptr) == DLO_E_INVAL);
  CHECK(g_seen.calls == 1);

  // LayerNorm + modulate
  auto x = fake<float>(0x10000), sh = fake<float>(0x20000), sc = fake<float>(0x30000);
  auto h = fake<uint16_t>(0x40000);
  g_seen = Seen{};
  CHECK(dlo_op_ln_modulate(x, 1152, nullptr, sh, sc, h, 4096, 2048, nullptr) == DLO_OK);
  CHECK(g_seen.calls == 1 && g_seen.d_in == 1152 && g_seen.d == 2048 && g_seen.tokens == 4096);
  CHECK(dlo_op_ln_modulate(x, 1152, nullptr, sh, sc, h, 4096, 8196, nullptr) == DLO_E_SHAPE);
  CHECK(dlo_op_ln_modulate(x, 1150, nullptr, sh, sc, h, 4096, 2048, nullptr) == DLO_E_SHAPE);
  CHECK(dlo_op_ln_modulate(fake<float>(0x10004), 1152, nullptr, sh, sc, h, 4096, 2048, nullptr) == DLO_E_INVAL);
  CHECK(dlo_op_ln_modulate(x, 1152, nullptr, sh, sc, h, -1, 2048, nullptr) == DLO_E_INVAL);
  CHECK(g_seen.calls == 1);

  // attention: head dim 64 or 128, ld_vt covers the token count rounded to 64
  auto qk = fake<uint16_t>(0x100000), vt = fake<uint16_t>(0x200000), o = fake<uint16_t>(0x300000);
  g_seen = Seen{};
  CHECK(dlo_op_attention(qk, 4096, vt, 4160, o, 2048, 4100, 16, 128, nullptr) == DLO_OK);
  CHECK(g_seen.calls == 1 && g_seen.ld_vt == 4160 && g_seen.tokens == 4100 && g_seen.heads == 16 &&
        g_seen.head_dim == 128);
  CHECK(dlo_op_attention(qk, 4096, vt, 4096, o, 2048, 4100, 16, 128, nullptr) == DLO_E_SHAPE);  // ld_vt < 4160
  CHECK(dlo_op_attention(qk, 4096, vt, 4160, o, 2048, 4100, 16, 96, nullptr) == DLO_E_SHAPE);
  CHECK(dlo_op_attention(qk, 4000, vt, 4160, o, 2048, 4100, 16, 128, nullptr) == DLO_E_SHAPE);  // ld_qk < 2d
  CHECK(dlo_op_attention(qk, 4096, vt, 4160, o, 2048, 0, 16, 128, nullptr) == DLO_E_SHAPE);
  // q/k or v^T extent beyond 4 GiB (32-bit byte offsets in the kernel)
  CHECK(dlo_op_attention(qk, 1 << 17, vt, 1 << 17, o, 2048, 1 << 15, 16, 128, nullptr) == DLO_E_SHAPE);
  CHECK(dlo_op_attention(qk, 4096, vt, 1 << 20, o, 2048, 4100, 16, 128, nullptr) == DLO_E_SHAPE);
  CHECK(g_seen.calls == 1);
}

}  // namespace

int main() {
  check_layouts();
  check_gemm();
  check_other_ops();
  if (g_failures) {
    fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
