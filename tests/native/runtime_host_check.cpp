// The streaming runtime (runtime.cpp) driven on the host, under
// AddressSanitizer + UBSan, by tests/test_native_host.py (g++, no GPU).
//
// The HIP runtime is replaced by an in-order fake: "device" memory is host
// memory, every stream executes its work at enqueue time (so the enqueue order
// is the execution order), events carry a logical timestamp, copies are
// memcpy.  The reconstruction launcher here copies the bits unchanged (the
// real kernel also converts each value to fp16, which the GPU tests check), so
// the block's compute launchers, which record their arguments, can check at
// the moment they run that the slot they read holds exactly the block's
// gathered weights.  This exercises, on the CPU, the host logic of the
// method's runtime (vLLM-Omni release page, sections "Weight sharding with
// AllGather reconstruction" and "Double-buffered prefetch with H2D + AllGather
// overlap"): shard sizing, pinned shard contents, chunking of the gather
// output, which slot each block lands in and computes from, the slot
// alternation across forwards, parameter re-pointing at the cached offsets,
// argument validation, and fail-closed behaviour after a HIP error ("DP
// multi-concurrency").  Concurrency itself is checked on the GPU.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "dlo.h"
#include "kernels.h"

// ---------------------------------------------------------------- fake HIP
struct ihipStream_t {
  int id;
};
struct ihipEvent_t {
  double t;
};

namespace {
double g_clock = 0;       // logical time, one unit per enqueued operation
int g_memcpy_calls = 0;   // hipMemcpyAsync calls so far
int g_fail_memcpy_at = -1;  // make that call fail (fail-closed test)
int g_gemm_calls = 0;       // launch_gemm calls so far
int g_event_creates = 0;    // hipEventCreate calls so far
int g_fail_event_create_at = -1;  // make that call fail (trace event test)
int g_throw_gemm_at = -1;   // make that call throw std::bad_alloc (exception test)
int g_streams = 0;
}  // namespace

extern "C" {
hipError_t hipEventCreate(hipEvent_t* e) {
  if (g_event_creates++ == g_fail_event_create_at) return hipErrorInvalidValue;
  *e = new ihipEvent_t{0};
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { return hipEventCreate(e); }
hipError_t hipEventDestroy(hipEvent_t e) {
  delete e;
  return hipSuccess;
}
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b) {
  *ms = static_cast<float>(b->t - a->t);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
  e->t = ++g_clock;
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipSetDevice(int d) { return d == 0 ? hipSuccess : hipErrorInvalidDevice; }
const char* hipGetErrorString(hipError_t) { return "fake HIP error"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipHostMalloc(void** p, size_t bytes, unsigned) {
  *p = aligned_alloc(256, (bytes + 255) / 256 * 256);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipHostFree(void* p) {
  free(p);
  return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
  memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  if (g_memcpy_calls++ == g_fail_memcpy_at) return hipErrorInvalidValue;
  ++g_clock;
  memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned) {
  *s = new ihipStream_t{++g_streams};
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) {
  delete s;
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned) { return hipSuccess; }
}

// ------------------------------------------------------- launcher recorders
namespace {

int g_failures = 0;
#define CHECK(cond)                                                            \
  do {                                                                         \
    if (!(cond)) {                                                             \
      fprintf(stderr, "%s:%d: CHECK failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                            \
    }                                                                          \
  } while (0)

struct Model {
  std::vector<dlo_block_desc> descs;
  std::vector<std::vector<int64_t>> extras;
  std::vector<std::vector<uint16_t>> flat;    // gathered bf16 weights per block
  std::vector<std::vector<dlo_param_desc>> params;
  const char* slot[2] = {nullptr, nullptr};   // slot bases inside the arena
  size_t slot_bytes = 0;
};
Model g_model;

// compute launches seen, in order
struct Launch {
  char kind;  // 'a' adaln, 'l' LayerNorm, 'g' gemm, 't' attention
  int slot;   // slot the weights were read from (-1: none)
  int block;  // block whose weights the slot held (-1: none matched)
  int epilogue;
};
std::vector<Launch> g_launches;
int64_t g_assembled = 0;  // elements reconstructed

// Which slot `p` points into, or -1.
int slot_of(const void* p) {
  for (int k = 0; k < 2; ++k) {
    const char* s = g_model.slot[k];
    if (s && static_cast<const char*>(p) >= s && static_cast<const char*>(p) < s + g_model.slot_bytes) return k;
  }
  return -1;
}

// The block whose parameter `name` lies, bit-exactly, at `p` (in slot k), or -1.
int block_at(const void* p, const char* name) {
  const int k = slot_of(p);
  if (k < 0) return -1;
  const int64_t off = (static_cast<const char*>(p) - g_model.slot[k]) / 2;
  for (size_t b = 0; b < g_model.flat.size(); ++b) {
    for (auto& pd : g_model.params[b]) {
      if (strcmp(pd.name, name) != 0 || pd.offset != off) continue;
      int64_t n = 1;
      for (int i = 0; i < pd.ndim; ++i) n *= pd.shape[i];
      if (memcmp(p, g_model.flat[b].data() + off, size_t(n) * 2) == 0) return static_cast<int>(b);
    }
  }
  return -1;
}

}  // namespace

namespace dlo {

hipError_t launch_assemble(uint16_t* dst, const uint16_t* src, int64_t n, hipStream_t) {
  ++g_clock;
  memcpy(dst, src, size_t(n) * 2);
  g_assembled += n;
  return hipSuccess;
}

hipError_t launch_fill_nan(uint16_t* dst, int64_t n, hipStream_t) {
  for (int64_t i = 0; i < n; ++i) dst[i] = 0x7fc1;
  return hipSuccess;
}

hipError_t launch_adaln(const uint16_t* w, const uint16_t*, const float*, float*, int, int, hipStream_t) {
  g_launches.push_back({'a', slot_of(w), block_at(w, "Wada"), -1});
  return hipSuccess;
}

hipError_t launch_ln_modulate(const float*, int, float*, const float*, const float*, uint16_t*, int, int,
                              hipStream_t) {
  g_launches.push_back({'l', -1, -1, -1});
  return hipSuccess;
}

hipError_t launch_gemm(int epilogue, const GemmArgs& g, hipStream_t) {
  if (g_gemm_calls++ == g_throw_gemm_at) throw std::bad_alloc();
  // the weight operand: `a` for the transposed v projection, `w` otherwise
  const uint16_t* wt = epilogue == EPI_VT_F16 ? g.a : g.w;
  const char* name = "W1";
  if (epilogue == EPI_BIAS_F16 || epilogue == EPI_VT_F16) name = "Wqkv";
  if (epilogue == EPI_GATED_F32) name = g.K == g.N ? "Wo" : "W2";
  int blk = -1;
  if (epilogue == EPI_VT_F16) {
    // v rows start 2d rows into Wqkv: check the whole Wqkv from its start
    const int d = g.M;
    blk = block_at(wt - int64_t(2) * d * d, "Wqkv");
  } else {
    blk = block_at(wt, name);
  }
  g_launches.push_back({'g', slot_of(wt), blk, epilogue});
  return hipSuccess;
}

hipError_t launch_attention(const uint16_t*, int, const uint16_t*, int, uint16_t*, int, int, int, int,
                            hipStream_t) {
  g_launches.push_back({'t', -1, -1, -1});
  return hipSuccess;
}

// The library's static device scratch: the fake kernels never touch the
// workspace, so a small host buffer stands in for it.
hipError_t static_scratch(int, void** out) {
  alignas(256) static unsigned char buf[4096];
  *out = buf;
  return hipSuccess;
}

}  // namespace dlo

namespace {

uint16_t lcg16(uint64_t& s) {
  s = s * 6364136223846793005ull + 1442695040888963407ull;
  // finite bf16 patterns: clear the exponent's top bit
  return static_cast<uint16_t>((s >> 33) & 0xbfff);
}

struct Ctx {
  dlo_ctx* ctx = nullptr;
  void* arena = nullptr;
  std::vector<float> x, cond;
};

// Build a model of the given block shapes with dp shards and a chunk limit.
dlo_status make(Ctx& c, const std::vector<dlo_block_desc>& descs, int dp, int tokens, int64_t chunk,
                uint32_t flags) {
  g_model = Model{};
  g_model.descs = descs;
  dlo_config cfg{};
  cfg.abi_version = DLO_ABI_VERSION;
  cfg.num_blocks = static_cast<int32_t>(descs.size());
  cfg.blocks = g_model.descs.data();
  cfg.dp_size = dp;
  cfg.max_tokens = tokens;
  cfg.landing_chunk_elems = chunk;
  cfg.flags = flags;
  size_t slots = 0, landing = 0, ws = 0, total = 0;
  dlo_status st = dlo_required_bytes(&cfg, &slots, &landing, &ws, &total);
  if (st != DLO_OK) return st;
  CHECK(total == slots + landing + ws);
  c.arena = aligned_alloc(256, total);
  cfg.arena = c.arena;
  cfg.arena_bytes = total;
  // a smaller arena is refused before anything is created
  cfg.arena_bytes = total - 1;
  CHECK(dlo_create(&cfg, &c.ctx) == DLO_E_DEV_OOM && c.ctx == nullptr);
  cfg.arena_bytes = total;
  st = dlo_create(&cfg, &c.ctx);
  if (st != DLO_OK) return st;
  g_model.slot_bytes = slots / 2;
  g_model.slot[0] = static_cast<const char*>(c.arena);
  g_model.slot[1] = g_model.slot[0] + slots / 2;
  uint64_t seed = 12345;
  for (size_t b = 0; b < descs.size(); ++b) {
    int64_t numel = 0;
    int32_t np = 0;
    CHECK(dlo_block_layout(&descs[b], dp, &numel, nullptr, &np, nullptr, 0) == DLO_OK);
    std::vector<dlo_param_desc> pd(np);
    CHECK(dlo_block_layout(&descs[b], dp, nullptr, nullptr, nullptr, pd.data(), np) == DLO_OK);
    g_model.params.push_back(pd);
    std::vector<uint16_t> f(numel);
    for (auto& v : f) v = lcg16(seed);
    g_model.flat.push_back(f);
    // wrong element count is refused
    CHECK(dlo_load_shards(c.ctx, static_cast<int32_t>(b), f.data(), numel - 1) == DLO_E_SHAPE);
  }
  // a forward before every block has shards is refused
  int max_d = 0;
  for (auto& d : descs) max_d = d.d_model > max_d ? d.d_model : max_d;
  c.x.assign(size_t(tokens) * max_d + 16, 0.f);
  c.cond.assign(size_t(descs[0].d_cond) + 16, 0.f);
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), tokens, nullptr) == DLO_E_STATE);
  for (size_t b = 0; b < descs.size(); ++b) {
    st = dlo_load_shards(c.ctx, static_cast<int32_t>(b), g_model.flat[b].data(),
                         static_cast<int64_t>(g_model.flat[b].size()));
    if (st != DLO_OK) return st;
  }
  return DLO_OK;
}

void destroy(Ctx& c) {
  CHECK(dlo_destroy(c.ctx) == DLO_OK);
  free(c.arena);
  c = Ctx{};
}

// Shards: S = ceil(numel / dp), shard r = flat[r S, (r + 1) S) zero-padded.
void check_shards(Ctx& c, int dp) {
  for (size_t b = 0; b < g_model.flat.size(); ++b) {
    const auto& f = g_model.flat[b];
    const int64_t numel = static_cast<int64_t>(f.size());
    const int64_t S = (numel + dp - 1) / dp;
    for (int r = 0; r < dp; ++r) {
      const uint16_t* p = nullptr;
      int64_t n = 0;
      CHECK(dlo_get_shard(c.ctx, static_cast<int32_t>(b), r, &p, &n) == DLO_OK);
      CHECK(n == S);
      for (int64_t i = 0; i < S; ++i) {
        const int64_t g = int64_t(r) * S + i;
        if (p[i] != (g < numel ? f[g] : 0)) {
          CHECK(!"shard content");
          break;
        }
      }
    }
    CHECK(dlo_get_shard(c.ctx, static_cast<int32_t>(b), dp, nullptr, nullptr) == DLO_E_INVAL);
  }
}

// One forward: every block's compute reads its own weights from slot
// (b + first_slot) % 2; returns the slot block 0 used.
int check_forward(Ctx& c, int tokens, int expect_first_slot) {
  g_launches.clear();
  g_assembled = 0;
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), tokens, nullptr) == DLO_OK);
  const size_t L = g_model.flat.size();
  CHECK(g_launches.size() == 9 * L);
  int64_t want_asm = 0;
  for (auto& f : g_model.flat) want_asm += static_cast<int64_t>(f.size());
  CHECK(g_assembled == want_asm);  // padding is never copied into a slot
  const char order[] = "alggtglgg";
  using namespace dlo;
  const int epis[] = {-1, -1, EPI_BIAS_F16, EPI_VT_F16, -1, EPI_GATED_F32, -1, EPI_BIAS_GELU_F16, EPI_GATED_F32};
  int first = -1;
  for (size_t b = 0; b < L && 9 * b + 8 < g_launches.size(); ++b) {
    for (int i = 0; i < 9; ++i) {
      const Launch& l = g_launches[9 * b + i];
      CHECK(l.kind == order[i]);
      if (l.kind == 'g') CHECK(l.epilogue == epis[i]);
      if (l.kind == 'a' || l.kind == 'g') {
        if (first < 0) first = l.slot;
        CHECK(l.slot == static_cast<int>((b + first) % 2));
        CHECK(l.block == static_cast<int>(b));  // the slot holds this block's bf16 weights, bit-exact
      }
    }
  }
  if (expect_first_slot >= 0) CHECK(first == expect_first_slot);
  return first;
}

void run_schedule_case(const std::vector<dlo_block_desc>& descs, int dp, int64_t chunk, uint32_t flags) {
  Ctx c;
  const int tokens = 8;
  CHECK(make(c, descs, dp, tokens, chunk, flags) == DLO_OK);
  if (!c.ctx) return;
  check_shards(c, dp);
  // bad arguments are refused before anything is enqueued
  const int before = g_memcpy_calls;
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), tokens + 1, nullptr) == DLO_E_INVAL);
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), 0, nullptr) == DLO_E_INVAL);
  CHECK(dlo_forward(c.ctx, c.x.data() + 1, c.cond.data(), tokens, nullptr) == DLO_E_INVAL);
  CHECK(dlo_forward(c.ctx, nullptr, c.cond.data(), tokens, nullptr) == DLO_E_INVAL);
  CHECK(g_memcpy_calls == before);
  // consecutive forwards continue the alternation: an odd block count flips
  // the slot of block 0, an even one keeps it
  const size_t L = descs.size();
  int s0 = check_forward(c, tokens, 0);
  int s1 = check_forward(c, tokens, L % 2 ? 1 - s0 : s0);
  check_forward(c, tokens, L % 2 ? 1 - s1 : s1);
  // the stand-alone reconstruction gives back every block bit-exactly
  for (size_t b = 0; b < L; ++b) {
    std::vector<uint16_t> out(g_model.flat[b].size() + 3, 0xabcd);
    CHECK(dlo_debug_assemble(c.ctx, static_cast<int32_t>(b), out.data(), static_cast<int64_t>(out.size())) ==
          DLO_OK);
    CHECK(memcmp(out.data(), g_model.flat[b].data(), g_model.flat[b].size() * 2) == 0);
    CHECK(dlo_debug_assemble(c.ctx, static_cast<int32_t>(b), out.data(), 1) == DLO_E_INVAL);
  }
  dlo_stats st{};
  CHECK(dlo_get_stats(c.ctx, &st) == DLO_OK);
  CHECK(st.num_blocks == static_cast<int32_t>(L) && st.dp_size == dp && st.forwards == 3);
  int64_t h2d = 0;
  for (auto& f : g_model.flat) h2d += 2 * int64_t(dp) * ((static_cast<int64_t>(f.size()) + dp - 1) / dp);
  CHECK(st.h2d_bytes_per_forward == h2d);
  if (flags & DLO_FLAG_TRACE) {
    // the full trace: per chunk an H2D and a reconstruction interval, per
    // block a compute interval and nine kernel intervals
    int32_t n = 0;
    CHECK(dlo_get_trace(c.ctx, nullptr, 0, &n) == DLO_OK);
    std::vector<dlo_interval> iv(n);
    CHECK(dlo_get_trace(c.ctx, iv.data(), n, &n) == DLO_OK);
    int h = 0, a = 0, comp = 0, k = 0;
    for (auto& v : iv) {
      h += v.kind == DLO_IV_H2D;
      a += v.kind == DLO_IV_ASM;
      comp += v.kind == DLO_IV_COMPUTE;
      k += v.kind >= DLO_IV_K_ADALN;
      CHECK(v.end_ms >= v.start_ms);
    }
    CHECK(h == a && h >= static_cast<int>(L) && comp == static_cast<int>(L) && k == 9 * static_cast<int>(L));
    CHECK(st.residency_high_water >= 1 && st.residency_high_water <= 2);
  }
  destroy(c);
}

// dlo_set_trace_kinds: unknown kind bits are refused; a mask keeps only its
// kinds in the kernel trace (one K_FC1 interval per block), and the full mask
// brings every compute-stream interval back.
void run_trace_kinds_case() {
  Ctx c;
  std::vector<dlo_block_desc> descs(3, dlo_block_desc{128, 2, 256, 64, 0, 0, nullptr});
  CHECK(make(c, descs, 2, 8, 0, DLO_FLAG_TRACE_KERNELS) == DLO_OK);
  if (!c.ctx) return;
  CHECK(dlo_set_trace_kinds(c.ctx, 1u << 12) == DLO_E_INVAL);
  CHECK(dlo_set_trace_kinds(nullptr, DLO_TRACE_KINDS_ALL) == DLO_E_INVAL);
  auto kinds_of_forward = [&](std::vector<int>* per_kind) {
    CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), 8, nullptr) == DLO_OK);
    int32_t n = 0;
    CHECK(dlo_get_trace(c.ctx, nullptr, 0, &n) == DLO_OK);
    std::vector<dlo_interval> iv(n);
    CHECK(dlo_get_trace(c.ctx, iv.data(), n, &n) == DLO_OK);
    per_kind->assign(12, 0);
    for (auto& v : iv)
      if (v.kind >= 0 && v.kind < 12) ++(*per_kind)[v.kind];
  };
  std::vector<int> k;
  CHECK(dlo_set_trace_kinds(c.ctx, 1u << DLO_IV_K_FC1) == DLO_OK);
  kinds_of_forward(&k);
  for (int kind = 0; kind < 12; ++kind) CHECK(k[kind] == (kind == DLO_IV_K_FC1 ? 3 : 0));
  CHECK(dlo_set_trace_kinds(c.ctx, DLO_TRACE_KINDS_ALL) == DLO_OK);
  kinds_of_forward(&k);
  CHECK(k[DLO_IV_H2D] == 0 && k[DLO_IV_ASM] == 0 && k[DLO_IV_COMPUTE] == 3);
  for (int kind = DLO_IV_K_ADALN; kind <= DLO_IV_K_FC2; ++kind) CHECK(k[kind] == 3);
  destroy(c);
}

// A HIP error during a forward poisons the context: every later call fails
// with DLO_E_POISONED, and destroy still succeeds.
void run_fail_closed_case() {
  Ctx c;
  std::vector<dlo_block_desc> descs(3, dlo_block_desc{128, 2, 256, 64, 0, 0, nullptr});
  CHECK(make(c, descs, 2, 8, 4096, 0) == DLO_OK);
  if (!c.ctx) return;
  g_fail_memcpy_at = g_memcpy_calls + 5;
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), 8, nullptr) == DLO_E_HIP);
  g_fail_memcpy_at = -1;
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), 8, nullptr) == DLO_E_POISONED);
  CHECK(dlo_load_shards(c.ctx, 0, g_model.flat[0].data(), static_cast<int64_t>(g_model.flat[0].size())) ==
        DLO_E_POISONED);
  dlo_stats st{};
  CHECK(dlo_get_stats(c.ctx, &st) == DLO_E_POISONED);
  destroy(c);
}

// A trace event that cannot be created skips its interval: the forward and
// the trace read still succeed, and every interval read has both ends.
// Kernel-only tracing accumulates over forwards, so the second forward grows
// the event pool, two creations per interval (start, end); the creation of
// its second interval's start event fails.
void run_trace_event_failure_case() {
  Ctx c;
  std::vector<dlo_block_desc> descs(3, dlo_block_desc{128, 2, 256, 64, 0, 0, nullptr});
  CHECK(make(c, descs, 2, 8, 0, DLO_FLAG_TRACE_KERNELS) == DLO_OK);
  if (!c.ctx) return;
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), 8, nullptr) == DLO_OK);
  g_fail_event_create_at = g_event_creates + 2;
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), 8, nullptr) == DLO_OK);
  CHECK(g_event_creates > g_fail_event_create_at);  // the failing creation happened
  g_fail_event_create_at = -1;
  int32_t n = 0;
  CHECK(dlo_get_trace(c.ctx, nullptr, 0, &n) == DLO_OK);
  CHECK(n == 2 * 3 * 10 - 1);  // per block: the compute interval and nine kernels
  std::vector<dlo_interval> iv(n > 0 ? n : 0);
  CHECK(dlo_get_trace(c.ctx, iv.data(), n, &n) == DLO_OK);
  for (auto& v : iv) CHECK(v.end_ms >= v.start_ms);
  destroy(c);
}

// A C++ exception inside the library (here a host allocation failure in the
// middle of a forward's enqueue) comes back as DLO_E_HOST_OOM with a message,
// not as an exception through the C ABI, and poisons the context, since work
// may already be in flight.
void run_exception_case() {
  Ctx c;
  std::vector<dlo_block_desc> descs(3, dlo_block_desc{128, 2, 256, 64, 0, 0, nullptr});
  CHECK(make(c, descs, 2, 8, 4096, 0) == DLO_OK);
  if (!c.ctx) return;
  g_throw_gemm_at = g_gemm_calls + 7;
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), 8, nullptr) == DLO_E_HOST_OOM);
  g_throw_gemm_at = -1;
  CHECK(strstr(dlo_last_error(), "allocation failed") != nullptr);
  CHECK(dlo_forward(c.ctx, c.x.data(), c.cond.data(), 8, nullptr) == DLO_E_POISONED);
  destroy(c);
}

}  // namespace

int main() {
  const dlo_block_desc small{128, 2, 256, 64, 0, 0, nullptr};
  static const int64_t extra[2] = {5, 1001};
  const dlo_block_desc wide{256, 4, 512, 64, 2, 0, extra};
  // odd block count, chunks much smaller than a shard (they span shard
  // boundaries and end in the padding), slots poisoned before every gather
  run_schedule_case({small, small, small, small, small}, 3, 4096, DLO_FLAG_POISON_SLOTS | DLO_FLAG_TRACE);
  // even block count, one transfer per block
  run_schedule_case({small, small, small, small}, 4, 0, 0);
  // mixed widths and extra parameters, dp larger than useful (all-padding shards)
  run_schedule_case({small, wide, small}, 1024, 0, DLO_FLAG_TRACE);
  // one block, dp 1 (rank-local)
  run_schedule_case({wide}, 1, 4096, DLO_FLAG_POISON_SLOTS);
  run_trace_kinds_case();
  run_fail_closed_case();
  run_exception_case();
  run_trace_event_failure_case();
  if (g_failures) {
    fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  printf("runtime host checks passed\n");
  return 0;
}
