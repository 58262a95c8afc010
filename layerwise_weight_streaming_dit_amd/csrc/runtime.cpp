// Context, pinned shard store and the two-slot streaming scheduler.
//
// The method (vLLM-Omni "Distributed Layerwise Offload" release page):
//  * section "Weight sharding with AllGather reconstruction" -- each block's
//    flat weight is kept as dp equal shards of ceil(numel / dp) elements,
//    zero-padded, in pinned host memory; the layer is rebuilt by gathering the
//    shards in rank order;
//  * section "Double-buffered prefetch with H2D + AllGather overlap" -- two
//    device slots sized to the largest block, allocated once; block b+1 is
//    copied host-to-device (copy stream) and gathered (gather stream) while
//    block b computes from the other slot; compute waits on the gather's
//    event; parameters are re-pointed from cached offsets;
//  * section "DP multi-concurrency" -- invalid work is rejected before
//    dispatch and errors fail closed.
//
// One GPU plays every rank here: all dp shards of a block are copied, in
// chunks, through two landing buffers (the per-rank receive buffers), and the
// reconstruction kernel copies each landed chunk to its place in the slot,
// dropping the zero padding.  Chunks alternate between two copy streams (two
// DMA engines), one per landing buffer: while one engine sets up its next
// transfer the other keeps the host link busy.
//
// Per block b (slot k = (b + parity) % 2) the host enqueues, without ever
// blocking:
//   copy stream j%2: per chunk j: (first two chunks: wait comp_done[k], the
//                   compute of block b-2, so no third block reaches the
//                   device); wait land_free[j%2]; H2D -> landing[j%2];
//                   record h2d_done[j%2]
//   gather stream : wait comp_done[k] (compute of block b-2 released slot k);
//                   per chunk j: wait h2d_done[j%2]; reconstruct into slot k;
//                   record land_free[j%2]; finally record asm_done[k]
//   compute stream: wait asm_done[k]; run the block from slot k;
//                   record comp_done[k]
// Events are re-recorded every block; each wait binds to the latest record
// enqueued before it, which is the intended predecessor in this enqueue order.
// Consecutive forwards continue the alternation: `parity` flips after a
// forward with an odd block count, so block 0 of the next forward always goes
// into the slot the previous forward's last block is not computing from and
// streams while that block computes.
#include <string.h>

#include <algorithm>
#include <memory>
#include <thread>
#include <vector>

#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace dlo {

namespace {

constexpr size_t kAlign = 256;
// Default H2D chunk: min(largest shard, a quarter of the largest padded block,
// 2^27 elements = 256 MiB).  The two landing buffers then add at most half a
// block, and at most 512 MiB, to the two slots' weight bytes: slots + landing
// <= 2.5 x the largest block at any dp.  Larger transfers keep the host link
// busier, since each copy carries a fixed set-up cost and each transfer's
// landing buffer is refilled only after its reconstruction, which waits for
// CUs the GEMMs hold: the 80-block d 8192 step streams at 33.5-33.7 blocks/s
// with 128 MiB transfers, 34.2-34.3 with 256 MiB and 33.9-34.0 with quarter
// blocks (409 MB, whose longer first transfer delays each block's compute);
// 8 of those blocks took 241.7 ms with 128 MiB transfers and 256.1 ms with
// 32 MiB ones.
constexpr int64_t kDefaultChunk = int64_t(1) << 27;
constexpr int64_t kMinChunk = 4096;
constexpr int kLandSlack = 8;  // landing offset (elements) used to co-align with the slot
constexpr size_t kMaxTraceEvents = size_t(1) << 20;  // bound on recorded trace events per context
// Trace events only time intervals (the host reads them after synchronizing
// the streams; no stream waits on them), so they skip the system-scope
// release a default event performs when recorded: that cache write-back sat
// between every pair of traced kernels and lengthened each traced interval.
constexpr unsigned kTraceEventFlags = hipEventDisableSystemFence;

// One H2D transfer.  The dp shards of a block sit back to back in one pinned
// region (shard r at element r * S), so their concatenation -- the gather's
// output, the flat weight followed by the zero padding -- is contiguous, and a
// chunk is a range of it that may span several shards.
struct Chunk {
  int64_t off;    // element offset in the concatenation = offset in the slot
  int64_t len;    // elements copied host -> device
  int64_t valid;  // elements reconstructed (the trailing padding is dropped)
};

// Cut a block's padded weight (dp * shard elements, of which the first numel
// are the flat weight) into equal chunks of at most `chunk` elements; lengths
// are multiples of 8 elements unless `chunk` itself is not.
std::vector<Chunk> plan_chunks(int dp, int64_t shard, int64_t numel, int64_t chunk) {
  std::vector<Chunk> out;
  const int64_t total = int64_t(dp) * shard;
  const int64_t nch = std::max<int64_t>(1, (total + chunk - 1) / chunk);
  const int64_t len = std::min(chunk, ((total + nch - 1) / nch + 7) / 8 * 8);
  for (int64_t off = 0; off < total; off += len) {
    Chunk c;
    c.off = off;
    c.len = std::min(len, total - off);
    c.valid = std::max<int64_t>(0, std::min(c.len, numel - off));
    out.push_back(c);
  }
  return out;
}

// Elements a landing buffer needs for a chunk: the chunk lands at the same
// address modulo 16 bytes as its slot destination.
int64_t landing_need(const Chunk& c) { return c.off % kLandSlack + c.len; }

struct Block {
  dlo_block_desc desc{};
  std::vector<int64_t> extra;
  BlockLayout layout;
  int64_t shard = 0;  // S_b
  uint16_t* pinned = nullptr;     // dp * S_b pinned elements, null until loaded
  std::vector<uint16_t*> shards;  // shard r = pinned + r * S_b
  std::vector<Chunk> chunks;
};

struct TraceEv {
  int kind, block, chunk, slot, landing, fwd;
  int64_t bytes;
  hipEvent_t start, end;
};

struct Workspace {
  float* mod = nullptr;
  uint16_t* h = nullptr;
  uint16_t* qk = nullptr;
  uint16_t* vt = nullptr;
  uint16_t* o = nullptr;
  uint16_t* u = nullptr;
  float* xalt = nullptr;
};

// The activation workspace of a forward over T tokens, carved from `base`
// (256-byte aligned) in a fixed order; returns the bytes it spans.  Every
// region is written by a kernel before any kernel reads it, so no region
// needs clearing.
size_t carve_workspace(char* base, size_t T, size_t d, size_t m, bool mixed, Workspace* w) {
  const size_t Tp = align_up(T, 64);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = base ? base + off : nullptr;
    off += align_up(bytes, kAlign);
    return r;
  };
  Workspace ws;
  ws.mod = reinterpret_cast<float*>(take(6 * d * 4));
  ws.h = reinterpret_cast<uint16_t*>(take(T * d * 2));
  ws.qk = reinterpret_cast<uint16_t*>(take(T * 2 * d * 2));
  ws.vt = reinterpret_cast<uint16_t*>(take(d * Tp * 2));
  ws.o = reinterpret_cast<uint16_t*>(take(T * d * 2));
  ws.u = reinterpret_cast<uint16_t*>(take(T * m * 2));
  if (mixed) ws.xalt = reinterpret_cast<float*>(take(T * d * 4));
  if (w) *w = ws;
  return off;
}

}  // namespace

}  // namespace dlo

struct dlo_ctx {
  int device = 0;
  uint32_t flags = 0;
  uint32_t trace_kinds = DLO_TRACE_KINDS_ALL;  // interval kinds recorded when tracing
  int dp = 1;
  int max_tokens = 1;
  int d_max = 0, m_max = 0;
  bool mixed_width = false;
  int64_t s_max = 0;
  int64_t chunk_elems = 0;
  size_t slot_bytes = 0, landing_bytes = 0, workspace_bytes = 0;
  std::vector<dlo::Block> blocks;
  uint16_t* slot[2] = {nullptr, nullptr};
  int parity = 0;  // slot of block 0 in the next forward
  uint16_t* landing[2] = {nullptr, nullptr};
  dlo::Workspace ws;
  hipStream_t copy_s = nullptr, copy_s2 = nullptr, gather_s = nullptr;
  bool own_copy = false, own_gather = false;
  hipEvent_t h2d_done[2] = {}, land_free[2] = {}, asm_done[2] = {}, comp_done[2] = {};
  int64_t land_counter = 0;  // global chunk counter (landing buffer parity)
  // tracing
  std::vector<hipEvent_t> ev_pool;
  size_t ev_next = 0;
  std::vector<dlo::TraceEv> trace;
  bool trace_valid = false;
  int64_t forwards = 0;
  bool poisoned = false;
  bool created_events = false;
  void* static_ws = nullptr;       // this device's address of the library's static scratch
  hipError_t static_ws_err = hipSuccess;
};

namespace dlo {

namespace {

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

dlo_status hip_fail(dlo_ctx* ctx, hipError_t e, const char* what) {
  if (ctx) ctx->poisoned = true;
  return fail(DLO_E_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

#define DLO_HIP(ctx, call)                                   \
  do {                                                       \
    hipError_t _e = (call);                                  \
    if (_e != hipSuccess) return hip_fail((ctx), _e, #call); \
  } while (0)

struct Sizes {
  size_t slot_bytes, landing_bytes, workspace_bytes, total;
  int64_t s_max, chunk;
  int d_max, m_max;
  bool mixed;
};

dlo_status validate_config(const dlo_config* cfg) {
  if (cfg == nullptr) return fail(DLO_E_INVAL, "config is NULL");
  if (cfg->abi_version != DLO_ABI_VERSION)
    return fail(DLO_E_INVAL, "abi_version %d, library is %d", cfg->abi_version, DLO_ABI_VERSION);
  if (cfg->num_blocks < 1) return fail(DLO_E_INVAL, "num_blocks %d must be >= 1", cfg->num_blocks);
  if (cfg->blocks == nullptr) return fail(DLO_E_INVAL, "blocks is NULL");
  if (cfg->dp_size < 1 || cfg->dp_size > 1024) return fail(DLO_E_INVAL, "dp_size %d outside [1, 1024]", cfg->dp_size);
  if (cfg->max_tokens < 1 || cfg->max_tokens > (1 << 20))
    return fail(DLO_E_INVAL, "max_tokens %d outside [1, 2^20]", cfg->max_tokens);
  constexpr uint32_t kKnownFlags = DLO_FLAG_TRACE | DLO_FLAG_SERIALIZE | DLO_FLAG_POISON_SLOTS |
                                   DLO_FLAG_TRACE_KERNELS | DLO_FLAG_TRACE_SPAN;
  if (cfg->flags & ~kKnownFlags) return fail(DLO_E_INVAL, "unknown flags 0x%x", cfg->flags & ~kKnownFlags);
  if (cfg->landing_chunk_elems != 0 && cfg->landing_chunk_elems < kMinChunk)
    return fail(DLO_E_INVAL, "landing_chunk_elems %lld below %lld", (long long)cfg->landing_chunk_elems,
                (long long)kMinChunk);
  const int c0 = cfg->blocks[0].d_cond;
  for (int i = 0; i < cfg->num_blocks; ++i) {
    dlo_status st = validate_block(&cfg->blocks[i], i);
    if (st != DLO_OK) return st;
    if (cfg->blocks[i].d_cond != c0)
      return fail(DLO_E_INVAL, "block %d: d_cond %d differs from block 0 (%d)", i, cfg->blocks[i].d_cond, c0);
  }
  return DLO_OK;
}

dlo_status compute_sizes(const dlo_config* cfg, Sizes* z) {
  dlo_status st = validate_config(cfg);
  if (st != DLO_OK) return st;
  z->s_max = 0;
  z->d_max = 0;
  z->m_max = 0;
  z->mixed = false;
  for (int i = 0; i < cfg->num_blocks; ++i) {
    BlockLayout L;
    st = compute_layout(&cfg->blocks[i], &L);
    if (st != DLO_OK) return st;
    z->s_max = std::max(z->s_max, ceil_div(L.numel, cfg->dp_size));
    z->d_max = std::max(z->d_max, cfg->blocks[i].d_model);
    z->m_max = std::max(z->m_max, cfg->blocks[i].d_mlp);
    if (cfg->blocks[i].d_model != cfg->blocks[0].d_model) z->mixed = true;
  }
  // GEMM and attention operands are addressed with 32-bit byte offsets: the
  // widest activation operand (tokens x max(2 d_model, d_mlp) fp16: the q,k
  // projection output or the MLP hidden layer) must stay below 4 GiB.
  if (size_t(cfg->max_tokens) * size_t(std::max(2 * z->d_max, z->m_max)) * 2 > size_t(UINT32_MAX))
    return fail(DLO_E_INVAL, "max_tokens %d too large for the widest block (activations beyond 4 GiB)",
                cfg->max_tokens);
  // largest padded block, dp * S_max elements: no chunk needs to be longer
  const int64_t padded_max = int64_t(cfg->dp_size) * z->s_max;
  z->chunk = cfg->landing_chunk_elems ? cfg->landing_chunk_elems
                                      : std::min<int64_t>({z->s_max, ceil_div(padded_max, 4), kDefaultChunk});
  z->chunk = std::max<int64_t>(z->chunk, std::min<int64_t>(kMinChunk, padded_max));
  z->chunk = std::min<int64_t>(z->chunk, padded_max);
  z->slot_bytes = align_up(size_t(2) * size_t(cfg->dp_size) * size_t(z->s_max), kAlign);
  // each landing buffer holds the largest chunk any block is cut into
  int64_t land = 0;
  for (int i = 0; i < cfg->num_blocks; ++i) {
    BlockLayout L;
    (void)compute_layout(&cfg->blocks[i], &L);
    for (const Chunk& c : plan_chunks(cfg->dp_size, ceil_div(L.numel, cfg->dp_size), L.numel, z->chunk))
      land = std::max(land, landing_need(c));
  }
  z->landing_bytes = 2 * align_up(size_t(2) * size_t(land), kAlign);
  z->workspace_bytes = carve_workspace(nullptr, size_t(cfg->max_tokens), size_t(z->d_max), size_t(z->m_max),
                                       z->mixed, nullptr);
  z->total = 2 * z->slot_bytes + z->landing_bytes + z->workspace_bytes;
  return DLO_OK;
}

// memcpy split over a few threads (large blocks are GBs; one thread copies
// at a fraction of the host's memory bandwidth).
void copy_parallel(void* dst, const void* src, size_t bytes) {
  constexpr size_t kPiece = size_t(64) << 20;
  const size_t hw = std::max(1u, std::thread::hardware_concurrency());
  const size_t nt = std::min<size_t>({8, hw, (bytes + kPiece - 1) / kPiece});
  if (nt <= 1) {
    if (bytes) memcpy(dst, src, bytes);
    return;
  }
  const size_t per = (bytes + nt - 1) / nt;
  std::vector<std::thread> pool;
  bool reserved = true;
  try {
    pool.reserve(nt - 1);
  } catch (...) {
    reserved = false;
  }
  for (size_t t = 1; t < nt; ++t) {
    const size_t lo = t * per, n = lo < bytes ? std::min(per, bytes - lo) : 0;
    if (n == 0) continue;
    auto piece = [=] { memcpy(static_cast<char*>(dst) + lo, static_cast<const char*>(src) + lo, n); };
    bool started = false;
    if (reserved) {
      try {
        pool.emplace_back(piece);
        started = true;
      } catch (...) {
      }
    }
    if (!started) piece();  // no thread for this piece: copy it here
  }
  memcpy(dst, src, std::min(per, bytes));
  for (auto& th : pool) th.join();
}

// Index of the forward being enqueued (forwards counts completed enqueues).
int fwd_index(const dlo_ctx* ctx) { return static_cast<int>(ctx->forwards); }

// Trace events one forward records under the context's current flags.
// Whether intervals of `kind` (DLO_IV_*) are recorded.
bool traced(const dlo_ctx* ctx, int kind) { return (ctx->trace_kinds >> kind) & 1u; }

size_t events_per_forward(const dlo_ctx* ctx) {
  const bool all = (ctx->flags & DLO_FLAG_TRACE) != 0;
  const bool kern = all || (ctx->flags & DLO_FLAG_TRACE_KERNELS) != 0;
  if (!kern) return 0;
  int kinds = 0;
  for (int kind = DLO_IV_K_ADALN; kind <= DLO_IV_K_FC2; ++kind) kinds += traced(ctx, kind) ? 1 : 0;
  const size_t per_chunk = all ? 2 * ((traced(ctx, DLO_IV_H2D) ? 1 : 0) + (traced(ctx, DLO_IV_ASM) ? 1 : 0)) : 0;
  size_t n = 0;
  for (auto& b : ctx->blocks)
    n += (traced(ctx, DLO_IV_COMPUTE) ? 2 : 0) + 2 * kinds + per_chunk * b.chunks.size();
  return n;
}

// Create pool events until `want` exist (bounded); false if creation failed.
bool grow_pool(dlo_ctx* ctx, size_t want) {
  want = std::min(want, kMaxTraceEvents);
  while (ctx->ev_pool.size() < want) {
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, kTraceEventFlags) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    ctx->ev_pool.push_back(e);
  }
  return true;
}

void drop_trace(dlo_ctx* ctx) {
  ctx->trace.clear();
  ctx->ev_next = 0;
  ctx->trace_valid = false;
}

hipEvent_t next_ev(dlo_ctx* ctx) {
  if (ctx->ev_next >= ctx->ev_pool.size()) {
    // kernel-only tracing accumulates over forwards: grow the pool on demand,
    // up to a bound (intervals past it are skipped until the trace is read)
    if (ctx->ev_pool.size() >= kMaxTraceEvents) return nullptr;
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, kTraceEventFlags) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;  // the interval is skipped
    }
    ctx->ev_pool.push_back(e);
  }
  return ctx->ev_pool[ctx->ev_next++];
}

// The start/end events of one traced interval: both, or neither (the
// interval is then skipped) when the pool cannot supply two.
void take_event_pair(dlo_ctx* ctx, TraceEv* t) {
  t->start = next_ev(ctx);
  t->end = t->start ? next_ev(ctx) : nullptr;
  if (t->end == nullptr) t->start = nullptr;
}

// Enqueue the H2D + reconstruction of block b into slot k on the copy and
// gather streams.  `trace` adds timed intervals; `in_forward` is false for
// the stand-alone debug path (no compute of block b-1 to wait for).
dlo_status enqueue_staging(dlo_ctx* ctx, int b, int k, bool trace, bool in_forward) {
  Block& blk = ctx->blocks[b];
  for (size_t ci = 0; ci < blk.chunks.size(); ++ci) {
    const Chunk& c = blk.chunks[ci];
    const int lb = static_cast<int>(ctx->land_counter & 1);
    ++ctx->land_counter;
    const int64_t co = c.off % kLandSlack;  // co-align landing with slot (mod 16 bytes)
    uint16_t* land = ctx->landing[lb] + co;
    hipStream_t cs = lb ? ctx->copy_s2 : ctx->copy_s;
    // copy stream of this landing buffer.  The first chunk on each of the two
    // copy streams waits for the compute of block b-2 (the last reader of
    // slot k): a block's weights reach the device only once the block two
    // places earlier is done, so at most two blocks -- the one computing and
    // the one being staged, landing buffers included -- are ever on the
    // device.  Later chunks follow on the same streams.
    if (ci < 2) DLO_HIP(ctx, hipStreamWaitEvent(cs, ctx->comp_done[k], 0));
    DLO_HIP(ctx, hipStreamWaitEvent(cs, ctx->land_free[lb], 0));
    if ((ctx->flags & DLO_FLAG_SERIALIZE) && in_forward) {
      // synchronous schedule: nothing of block b moves before block b-1 computed
      DLO_HIP(ctx, hipStreamWaitEvent(cs, ctx->comp_done[k ^ 1], 0));
    }
    TraceEv tv{};
    if (trace && traced(ctx, DLO_IV_H2D)) {
      tv = TraceEv{DLO_IV_H2D, b, static_cast<int>(ci), -1, lb, fwd_index(ctx), c.len * 2, nullptr, nullptr};
      take_event_pair(ctx, &tv);
      if (tv.start) DLO_HIP(ctx, hipEventRecord(tv.start, cs));
    }
    DLO_HIP(ctx, hipMemcpyAsync(land, blk.pinned + c.off, size_t(c.len) * 2, hipMemcpyHostToDevice, cs));
    if (tv.end) {
      DLO_HIP(ctx, hipEventRecord(tv.end, cs));
      ctx->trace.push_back(tv);
    }
    DLO_HIP(ctx, hipEventRecord(ctx->h2d_done[lb], cs));
    // gather stream
    if (ci == 0) {
      DLO_HIP(ctx, hipStreamWaitEvent(ctx->gather_s, ctx->comp_done[k], 0));
      if (ctx->flags & DLO_FLAG_POISON_SLOTS)
        DLO_HIP(ctx, launch_fill_nan(ctx->slot[k], ctx->slot_bytes / 2, ctx->gather_s));
    }
    DLO_HIP(ctx, hipStreamWaitEvent(ctx->gather_s, ctx->h2d_done[lb], 0));
    TraceEv ta{};
    if (trace && traced(ctx, DLO_IV_ASM)) {
      ta = TraceEv{DLO_IV_ASM, b, static_cast<int>(ci), k, lb, fwd_index(ctx), c.valid * 2, nullptr, nullptr};
      take_event_pair(ctx, &ta);
      if (ta.start) DLO_HIP(ctx, hipEventRecord(ta.start, ctx->gather_s));
    }
    DLO_HIP(ctx, launch_assemble(ctx->slot[k] + c.off, land, c.valid, ctx->gather_s));
    if (ta.end) {
      DLO_HIP(ctx, hipEventRecord(ta.end, ctx->gather_s));
      ctx->trace.push_back(ta);
    }
    DLO_HIP(ctx, hipEventRecord(ctx->land_free[lb], ctx->gather_s));
  }
  DLO_HIP(ctx, hipEventRecord(ctx->asm_done[k], ctx->gather_s));
  return DLO_OK;
}

// The DiT block of `b` from slot k on the compute stream, with activations in
// workspace w.
dlo_status enqueue_block_compute(dlo_ctx* ctx, int b, int k, float*& x_cur, int& d_cur, float* x_user,
                                 const float* cond, int T, hipStream_t s, bool trace, const Workspace& w) {
  const Block& blk = ctx->blocks[b];
  const BlockLayout& L = blk.layout;
  const uint16_t* base = ctx->slot[k];
  // parameter re-pointing from the cached offsets
  const uint16_t* Wqkv = base + L.off_wqkv;
  const uint16_t* bqkv = base + L.off_bqkv;
  const uint16_t* Wo = base + L.off_wo;
  const uint16_t* bo = base + L.off_bo;
  const uint16_t* W1 = base + L.off_w1;
  const uint16_t* b1 = base + L.off_b1;
  const uint16_t* W2 = base + L.off_w2;
  const uint16_t* b2 = base + L.off_b2;
  const uint16_t* Wada = base + L.off_wada;
  const uint16_t* bada = base + L.off_bada;
  const int d = blk.desc.d_model, m = blk.desc.d_mlp, H = blk.desc.n_heads, c = blk.desc.d_cond;
  const int hd = d / H;
  const int Tp = static_cast<int>(align_up(size_t(T), 64));
  float* mod = w.mod;
  // Record a timed interval around one kernel when tracing.
  auto timed = [&](int kind, auto&& launch) -> dlo_status {
    TraceEv tv{};
    if (trace && traced(ctx, kind)) {
      tv = TraceEv{kind, b, -1, k, -1, fwd_index(ctx), 0, nullptr, nullptr};
      take_event_pair(ctx, &tv);
      if (tv.start) DLO_HIP(ctx, hipEventRecord(tv.start, s));
    }
    DLO_HIP(ctx, launch());
    if (tv.end) {
      DLO_HIP(ctx, hipEventRecord(tv.end, s));
      ctx->trace.push_back(tv);
    }
    return DLO_OK;
  };
  dlo_status st;
#define DLO_STEP(kind, expr)                       \
  st = timed(kind, [&]() -> hipError_t { return (expr); }); \
  if (st != DLO_OK) return st

  DLO_STEP(DLO_IV_K_ADALN, launch_adaln(Wada, bada, cond, mod, 6 * d, c, s));
  if (d != d_cur) {
    float* x_new = (x_cur == x_user) ? w.xalt : x_user;
    DLO_STEP(DLO_IV_K_LN1, launch_ln_modulate(x_cur, d_cur, x_new, mod, mod + d, w.h, T, d, s));
    x_cur = x_new;
    d_cur = d;
  } else {
    DLO_STEP(DLO_IV_K_LN1, launch_ln_modulate(x_cur, d, nullptr, mod, mod + d, w.h, T, d, s));
  }
  // q, k projection: qk[T][2d] = h Wqk^T + bqk
  const GemmArgs gqk{w.h, Wqkv, bqkv, nullptr, w.qk, d, d, 2 * d, T, 2 * d, d, 2 * d};
  DLO_STEP(DLO_IV_K_QK, launch_gemm(EPI_BIAS_F16, gqk, s));
  // v projection, transposed: vt[d][Tp] = Wv h^T + bv (columns >= T finite)
  const GemmArgs gv{Wqkv + int64_t(2) * d * d, w.h, bqkv + 2 * d, nullptr, w.vt, d, d, Tp, d, Tp, d, T};
  DLO_STEP(DLO_IV_K_V, launch_gemm(EPI_VT_F16, gv, s));
  DLO_STEP(DLO_IV_K_ATTN, launch_attention(w.qk, 2 * d, w.vt, Tp, w.o, d, T, H, hd, s));
  // x += gate1 * (o Wo^T + bo)
  const GemmArgs go{w.o, Wo, bo, mod + 2 * d, x_cur, d, d, d, T, d, d, d};
  DLO_STEP(DLO_IV_K_OUT, launch_gemm(EPI_GATED_F32, go, s));
  DLO_STEP(DLO_IV_K_LN2, launch_ln_modulate(x_cur, d, nullptr, mod + 3 * d, mod + 4 * d, w.h, T, d, s));
  // u = gelu(h2 W1^T + b1)
  const GemmArgs g1{w.h, W1, b1, nullptr, w.u, d, d, m, T, m, d, m};
  DLO_STEP(DLO_IV_K_FC1, launch_gemm(EPI_BIAS_GELU_F16, g1, s));
  // x += gate2 * (u W2^T + b2)
  const GemmArgs g2{w.u, W2, b2, mod + 5 * d, x_cur, m, m, d, T, d, m, d};
  DLO_STEP(DLO_IV_K_FC2, launch_gemm(EPI_GATED_F32, g2, s));
#undef DLO_STEP
  return DLO_OK;
}

dlo_status check_ctx(dlo_ctx* ctx) {
  if (ctx == nullptr) return fail(DLO_E_INVAL, "context is NULL");
  if (ctx->poisoned) return fail(DLO_E_POISONED, "context poisoned by an earlier HIP error");
  return DLO_OK;
}

dlo_status sync_ctx(dlo_ctx* ctx) {
  DLO_HIP(ctx, hipStreamSynchronize(ctx->copy_s));
  DLO_HIP(ctx, hipStreamSynchronize(ctx->copy_s2));
  DLO_HIP(ctx, hipStreamSynchronize(ctx->gather_s));
  DLO_HIP(ctx, hipEventSynchronize(ctx->comp_done[0]));
  DLO_HIP(ctx, hipEventSynchronize(ctx->comp_done[1]));
  return DLO_OK;
}

void free_ctx(dlo_ctx* ctx) {
  for (auto& b : ctx->blocks)
    if (b.pinned) (void)hipHostFree(b.pinned);
  for (auto e : ctx->ev_pool) (void)hipEventDestroy(e);
  if (ctx->created_events) {
    for (int i = 0; i < 2; ++i) {
      (void)hipEventDestroy(ctx->h2d_done[i]);
      (void)hipEventDestroy(ctx->land_free[i]);
      (void)hipEventDestroy(ctx->asm_done[i]);
      (void)hipEventDestroy(ctx->comp_done[i]);
    }
  }
  if (ctx->own_copy && ctx->copy_s) (void)hipStreamDestroy(ctx->copy_s);
  if (ctx->copy_s2) (void)hipStreamDestroy(ctx->copy_s2);
  if (ctx->own_gather && ctx->gather_s) (void)hipStreamDestroy(ctx->gather_s);
  delete ctx;
}

}  // namespace

}  // namespace dlo

using namespace dlo;

namespace {

// Entry points that enqueue GPU work: a throw part-way may leave work in
// flight, so the context is poisoned (every later call fails closed) before
// the exception becomes a status.
template <class F>
dlo_status guarded_enqueue(dlo_ctx* ctx, F&& body) noexcept {
  return guarded([&]() -> dlo_status {
    try {
      return body();
    } catch (...) {
      if (ctx != nullptr) ctx->poisoned = true;
      throw;
    }
  });
}

}  // namespace

extern "C" DLO_API dlo_status dlo_required_bytes(const dlo_config* cfg, size_t* slots, size_t* landing,
                                                 size_t* workspace, size_t* total) {
  return guarded([&]() -> dlo_status {
    clear_error();
    Sizes z;
    dlo_status st = compute_sizes(cfg, &z);
    if (st != DLO_OK) return st;
    if (slots) *slots = 2 * z.slot_bytes;
    if (landing) *landing = z.landing_bytes;
    if (workspace) *workspace = z.workspace_bytes;
    if (total) *total = z.total;
    return DLO_OK;
  });
}

extern "C" DLO_API dlo_status dlo_create(const dlo_config* cfg, dlo_ctx** out) {
  return guarded([&]() -> dlo_status {
    clear_error();
    if (out == nullptr) return fail(DLO_E_INVAL, "out is NULL");
    *out = nullptr;
    Sizes z;
    dlo_status st = compute_sizes(cfg, &z);
    if (st != DLO_OK) return st;
    if (cfg->arena == nullptr) return fail(DLO_E_INVAL, "arena is NULL");
    if (reinterpret_cast<uintptr_t>(cfg->arena) % kAlign != 0) return fail(DLO_E_INVAL, "arena not 256-byte aligned");
    if (cfg->arena_bytes < z.total)
      return fail(DLO_E_DEV_OOM, "arena holds %zu bytes, %zu required", cfg->arena_bytes, z.total);

    std::unique_ptr<dlo_ctx, void (*)(dlo_ctx*)> ctx(new dlo_ctx(), free_ctx);
    ctx->device = cfg->device;
    ctx->flags = cfg->flags;
    ctx->dp = cfg->dp_size;
    ctx->max_tokens = cfg->max_tokens;
    ctx->d_max = z.d_max;
    ctx->m_max = z.m_max;
    ctx->mixed_width = z.mixed;
    ctx->s_max = z.s_max;
    ctx->chunk_elems = z.chunk;
    ctx->slot_bytes = z.slot_bytes;
    ctx->landing_bytes = z.landing_bytes;
    ctx->workspace_bytes = z.workspace_bytes;
    ctx->blocks.resize(cfg->num_blocks);
    for (int i = 0; i < cfg->num_blocks; ++i) {
      Block& b = ctx->blocks[i];
      b.desc = cfg->blocks[i];
      b.extra.assign(cfg->blocks[i].extra_len, cfg->blocks[i].extra_len + cfg->blocks[i].n_extra);
      b.desc.extra_len = b.extra.empty() ? nullptr : b.extra.data();
      st = compute_layout(&b.desc, &b.layout);
      if (st != DLO_OK) return st;
      b.shard = ceil_div(b.layout.numel, ctx->dp);
      b.chunks = plan_chunks(ctx->dp, b.shard, b.layout.numel, ctx->chunk_elems);
    }
    // carve the arena: slot 0, slot 1, landing 0, landing 1, workspace
    char* p = static_cast<char*>(cfg->arena);
    ctx->slot[0] = reinterpret_cast<uint16_t*>(p);
    p += z.slot_bytes;
    ctx->slot[1] = reinterpret_cast<uint16_t*>(p);
    p += z.slot_bytes;
    const size_t land_one = z.landing_bytes / 2;
    ctx->landing[0] = reinterpret_cast<uint16_t*>(p);
    p += land_one;
    ctx->landing[1] = reinterpret_cast<uint16_t*>(p);
    p += land_one;
    carve_workspace(p, size_t(cfg->max_tokens), size_t(z.d_max), size_t(z.m_max), z.mixed, &ctx->ws);

    DeviceGuard dg(ctx->device);
    if (!dg.ok) return fail(DLO_E_HIP, "hipSetDevice(%d) failed", ctx->device);
    dlo_ctx* c = ctx.get();
    if (cfg->copy_stream) {
      c->copy_s = cfg->copy_stream;
    } else {
      DLO_HIP(nullptr, hipStreamCreateWithFlags(&c->copy_s, hipStreamNonBlocking));
      c->own_copy = true;
    }
    DLO_HIP(nullptr, hipStreamCreateWithFlags(&c->copy_s2, hipStreamNonBlocking));
    if (cfg->gather_stream) {
      c->gather_s = cfg->gather_stream;
    } else {
      DLO_HIP(nullptr, hipStreamCreateWithFlags(&c->gather_s, hipStreamNonBlocking));
      c->own_gather = true;
    }
    for (int i = 0; i < 2; ++i) {
      DLO_HIP(nullptr, hipEventCreateWithFlags(&c->h2d_done[i], hipEventDisableTiming));
      DLO_HIP(nullptr, hipEventCreateWithFlags(&c->land_free[i], hipEventDisableTiming));
      DLO_HIP(nullptr, hipEventCreateWithFlags(&c->asm_done[i], hipEventDisableTiming));
      DLO_HIP(nullptr, hipEventCreateWithFlags(&c->comp_done[i], hipEventDisableTiming));
      c->created_events = true;
    }
    // initial records so the first waits are satisfied
    for (int i = 0; i < 2; ++i) {
      DLO_HIP(nullptr, hipEventRecord(c->land_free[i], c->gather_s));
      DLO_HIP(nullptr, hipEventRecord(c->comp_done[i], c->gather_s));
    }
    if (!grow_pool(c, events_per_forward(c))) return fail(DLO_E_HIP, "trace event creation failed");
    // the device address of the library's static scratch (dlo_forward_static),
    // taken here, at set-up, with the context's device current
    c->static_ws_err = static_scratch(c->device, &c->static_ws);
    if (c->static_ws_err != hipSuccess) (void)hipGetLastError();
    DLO_HIP(nullptr, hipStreamSynchronize(c->gather_s));
    *out = ctx.release();
    return DLO_OK;
  });
}

extern "C" DLO_API dlo_status dlo_load_shards(dlo_ctx* ctx, int32_t block, const uint16_t* flat, int64_t numel) {
  return guarded([&]() -> dlo_status {
    clear_error();
    dlo_status st = check_ctx(ctx);
    if (st != DLO_OK) return st;
    if (block < 0 || block >= static_cast<int>(ctx->blocks.size()))
      return fail(DLO_E_INVAL, "block %d outside [0, %zu)", block, ctx->blocks.size());
    Block& b = ctx->blocks[block];
    if (numel != b.layout.numel)
      return fail(DLO_E_SHAPE, "block %d: numel %lld, layout has %lld", block, (long long)numel,
                  (long long)b.layout.numel);
    if (flat == nullptr) return fail(DLO_E_INVAL, "flat weight is NULL");
    DeviceGuard dg(ctx->device);
    if (!dg.ok) return fail(DLO_E_HIP, "hipSetDevice(%d) failed", ctx->device);
    // no in-flight copy may read the shards being replaced
    DLO_HIP(ctx, hipStreamSynchronize(ctx->copy_s));
    DLO_HIP(ctx, hipStreamSynchronize(ctx->copy_s2));
    const int64_t S = b.shard;
    if (b.pinned == nullptr) {
      void* p = nullptr;
      const size_t bytes = size_t(std::max<int64_t>(int64_t(ctx->dp) * S, 1)) * 2;
      hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocDefault);
      if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return fail(DLO_E_HOST_OOM, "block %d: pinned allocation of %zu bytes failed", block, bytes);
      }
      b.pinned = static_cast<uint16_t*>(p);
      b.shards.assign(ctx->dp, nullptr);
      for (int r = 0; r < ctx->dp; ++r) b.shards[r] = b.pinned + int64_t(r) * S;
    }
    // shard r = flat[r S, min((r + 1) S, numel)) then zeros: with the shards
    // back to back this is the flat weight followed by the zero padding
    copy_parallel(b.pinned, flat, size_t(numel) * 2);
    memset(b.pinned + numel, 0, (size_t(ctx->dp) * size_t(S) - size_t(numel)) * 2);
    return DLO_OK;
  });
}

namespace dlo {
namespace {

// Validation shared by the forward entry points (before any enqueue).
dlo_status check_forward(dlo_ctx* ctx, const float* x, const float* cond, int32_t tokens) {
  dlo_status st = check_ctx(ctx);
  if (st != DLO_OK) return st;
  if (x == nullptr || cond == nullptr) return fail(DLO_E_INVAL, "x or cond is NULL");
  if (tokens < 1 || tokens > ctx->max_tokens)
    return fail(DLO_E_INVAL, "tokens %d outside [1, %d]", tokens, ctx->max_tokens);
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(cond) % 16)
    return fail(DLO_E_INVAL, "x and cond must be 16-byte aligned");
  return DLO_OK;
}

dlo_status check_loaded(dlo_ctx* ctx) {
  for (size_t i = 0; i < ctx->blocks.size(); ++i)
    if (ctx->blocks[i].shards.empty()) return fail(DLO_E_STATE, "block %zu has no shards loaded", i);
  return DLO_OK;
}

// The streamed forward with activations in workspace w (validated).
dlo_status forward_impl(dlo_ctx* ctx, float* x, const float* cond, int32_t tokens, hipStream_t stream,
                        const Workspace& w) {
  DeviceGuard dg(ctx->device);
  if (!dg.ok) return fail(DLO_E_HIP, "hipSetDevice(%d) failed", ctx->device);

  const bool trace_all = (ctx->flags & DLO_FLAG_TRACE) != 0;
  const bool trace = trace_all || (ctx->flags & DLO_FLAG_TRACE_KERNELS) != 0;
  // the full trace describes the last forward only, unless it spans forwards
  if (trace_all && !(ctx->flags & DLO_FLAG_TRACE_SPAN)) drop_trace(ctx);
  float* x_cur = x;
  int d_cur = ctx->blocks[0].desc.d_model;
  const int L = static_cast<int>(ctx->blocks.size());
  const int parity = ctx->parity;
  dlo_status st;
  // The workspace (and x) are shared with the previous call, whose last block
  // computed from slot parity ^ 1: order this call after it even if the
  // caller switched streams (free when it is the same stream).
  DLO_HIP(ctx, hipStreamWaitEvent(stream, ctx->comp_done[parity ^ 1], 0));
  for (int b = 0; b < L; ++b) {
    const int k = (b + parity) & 1;
    st = enqueue_staging(ctx, b, k, trace_all, true);
    if (st != DLO_OK) return st;
    DLO_HIP(ctx, hipStreamWaitEvent(stream, ctx->asm_done[k], 0));
    TraceEv tc{};
    if (trace && traced(ctx, DLO_IV_COMPUTE)) {
      tc = TraceEv{DLO_IV_COMPUTE, b, -1, k, -1, fwd_index(ctx), 0, nullptr, nullptr};
      take_event_pair(ctx, &tc);
      if (tc.start) DLO_HIP(ctx, hipEventRecord(tc.start, stream));
    }
    st = enqueue_block_compute(ctx, b, k, x_cur, d_cur, x, cond, tokens, stream, trace, w);
    if (st != DLO_OK) return st;
    if (tc.end) {
      DLO_HIP(ctx, hipEventRecord(tc.end, stream));
      ctx->trace.push_back(tc);
    }
    DLO_HIP(ctx, hipEventRecord(ctx->comp_done[k], stream));
  }
  if (x_cur != x)
    DLO_HIP(ctx, hipMemcpyAsync(x, x_cur, size_t(tokens) * size_t(d_cur) * 4, hipMemcpyDeviceToDevice, stream));
  if (trace) ctx->trace_valid = true;
  ctx->parity ^= L & 1;
  ++ctx->forwards;
  return DLO_OK;
}

}  // namespace
}  // namespace dlo

extern "C" DLO_API dlo_status dlo_forward(dlo_ctx* ctx, float* x, const float* cond, int32_t tokens,
                                          hipStream_t stream) {
  return guarded_enqueue(ctx, [&]() -> dlo_status {
    clear_error();
    dlo_status st = check_forward(ctx, x, cond, tokens);
    if (st == DLO_OK) st = check_loaded(ctx);
    if (st != DLO_OK) return st;
    return forward_impl(ctx, x, cond, tokens, stream, ctx->ws);
  });
}

extern "C" DLO_API dlo_status dlo_forward_static(dlo_ctx* ctx, float* x, const float* cond, int32_t tokens,
                                                 hipStream_t stream) {
  return guarded_enqueue(ctx, [&]() -> dlo_status {
    clear_error();
    dlo_status st = check_forward(ctx, x, cond, tokens);
    if (st != DLO_OK) return st;
    const size_t need = carve_workspace(nullptr, size_t(tokens), size_t(ctx->d_max), size_t(ctx->m_max),
                                        ctx->mixed_width, nullptr);
    if (need > kStaticScratchBytes)
      return fail(DLO_E_INVAL, "%d tokens need %zu bytes of activation workspace; the static scratch holds %zu",
                  tokens, need, kStaticScratchBytes);
    if (ctx->flags & (DLO_FLAG_TRACE | DLO_FLAG_TRACE_KERNELS))
      return fail(DLO_E_STATE, "tracing creates timing events; clear the trace flags for dlo_forward_static");
    if (ctx->static_ws == nullptr)
      return fail(DLO_E_STATE, "the static scratch is unavailable on device %d: %s", ctx->device,
                  hipGetErrorString(ctx->static_ws_err));
    st = check_loaded(ctx);
    if (st != DLO_OK) return st;
    Workspace w;
    carve_workspace(static_cast<char*>(ctx->static_ws), size_t(tokens), size_t(ctx->d_max), size_t(ctx->m_max),
                    ctx->mixed_width, &w);
    return forward_impl(ctx, x, cond, tokens, stream, w);
  });
}

extern "C" DLO_API dlo_status dlo_destroy(dlo_ctx* ctx) {
  return guarded([&]() -> dlo_status {
    clear_error();
    if (ctx == nullptr) return DLO_OK;
    {
      // Wait for every enqueued copy, reconstruction and block before the
      // pinned shards are freed and the caller releases the arena -- also on
      // a poisoned context: a host allocation failure poisons one with work
      // in flight on a healthy device, and after a device fault these calls
      // return the fault at once.
      DeviceGuard dg(ctx->device);
      (void)hipStreamSynchronize(ctx->copy_s);
      (void)hipStreamSynchronize(ctx->copy_s2);
      (void)hipStreamSynchronize(ctx->gather_s);
      (void)hipEventSynchronize(ctx->comp_done[0]);
      (void)hipEventSynchronize(ctx->comp_done[1]);
      (void)hipGetLastError();
    }
    free_ctx(ctx);
    return DLO_OK;
  });
}

extern "C" DLO_API dlo_status dlo_layout(dlo_ctx* ctx, int32_t block, int64_t* numel, int64_t* shard_size,
                                         int32_t* n_params, dlo_param_desc* out, int32_t cap) {
  return guarded([&]() -> dlo_status {
    clear_error();
    if (ctx == nullptr) return fail(DLO_E_INVAL, "context is NULL");
    if (block < 0 || block >= static_cast<int>(ctx->blocks.size()))
      return fail(DLO_E_INVAL, "block %d outside [0, %zu)", block, ctx->blocks.size());
    const Block& b = ctx->blocks[block];
    if (numel) *numel = b.layout.numel;
    if (shard_size) *shard_size = b.shard;
    if (n_params) *n_params = b.layout.n_params;
    if (out) {
      if (cap < b.layout.n_params) return fail(DLO_E_INVAL, "cap %d < %d parameters", cap, b.layout.n_params);
      memcpy(out, b.layout.params, sizeof(dlo_param_desc) * b.layout.n_params);
    }
    return DLO_OK;
  });
}

extern "C" DLO_API dlo_status dlo_get_shard(dlo_ctx* ctx, int32_t block, int32_t rank, const uint16_t** ptr,
                                            int64_t* n) {
  return guarded([&]() -> dlo_status {
    clear_error();
    if (ctx == nullptr || ptr == nullptr || n == nullptr) return fail(DLO_E_INVAL, "NULL argument");
    if (block < 0 || block >= static_cast<int>(ctx->blocks.size()))
      return fail(DLO_E_INVAL, "block %d outside [0, %zu)", block, ctx->blocks.size());
    if (rank < 0 || rank >= ctx->dp) return fail(DLO_E_INVAL, "rank %d outside [0, %d)", rank, ctx->dp);
    const Block& b = ctx->blocks[block];
    if (b.shards.empty()) return fail(DLO_E_STATE, "block %d has no shards loaded", block);
    *ptr = b.shards[rank];
    *n = b.shard;
    return DLO_OK;
  });
}

extern "C" DLO_API dlo_status dlo_debug_assemble(dlo_ctx* ctx, int32_t block, uint16_t* host_out, int64_t cap) {
  return guarded_enqueue(ctx, [&]() -> dlo_status {
    clear_error();
    dlo_status st = check_ctx(ctx);
    if (st != DLO_OK) return st;
    if (block < 0 || block >= static_cast<int>(ctx->blocks.size()))
      return fail(DLO_E_INVAL, "block %d outside [0, %zu)", block, ctx->blocks.size());
    Block& b = ctx->blocks[block];
    if (b.shards.empty()) return fail(DLO_E_STATE, "block %d has no shards loaded", block);
    if (host_out == nullptr || cap < b.layout.numel)
      return fail(DLO_E_INVAL, "host_out must hold %lld elements", (long long)b.layout.numel);
    DeviceGuard dg(ctx->device);
    if (!dg.ok) return fail(DLO_E_HIP, "hipSetDevice(%d) failed", ctx->device);
    const int k = block & 1;  // either slot: the staging waits until no compute reads it
    st = enqueue_staging(ctx, block, k, false, false);
    if (st != DLO_OK) return st;
    DLO_HIP(ctx, hipStreamSynchronize(ctx->gather_s));
    DLO_HIP(ctx, hipMemcpy(host_out, ctx->slot[k], size_t(b.layout.numel) * 2, hipMemcpyDeviceToHost));
    return DLO_OK;
  });
}

namespace {

// Largest number of [start, end) intervals alive at once, each weighted
// (ends sort before starts at equal times).
int64_t max_weighted_overlap(std::vector<std::pair<double, int64_t>>& ev) {
  std::sort(ev.begin(), ev.end(), [](const auto& u, const auto& v) {
    return u.first < v.first || (u.first == v.first && u.second < v.second);
  });
  int64_t cur = 0, best = 0;
  for (auto& e : ev) {
    cur += e.second;
    best = std::max(best, cur);
  }
  return best;
}

dlo_status collect_trace(dlo_ctx* ctx, std::vector<dlo_interval>& out, dlo_stats* s) {
  out.clear();
  if (!ctx->trace_valid) return DLO_OK;
  dlo_status st = sync_ctx(ctx);
  if (st != DLO_OK) return st;
  hipEvent_t base = nullptr;
  float best = 0.f;
  // base = earliest start event
  for (auto& t : ctx->trace) {
    if (!t.start) continue;
    if (!base) {
      base = t.start;
      continue;
    }
    float ms = 0.f;
    DLO_HIP(ctx, hipEventElapsedTime(&ms, base, t.start));
    if (ms < best) {
      best = ms;
    }
  }
  if (!base) return DLO_OK;
  double t_end = 0.0;
  for (auto& t : ctx->trace) {
    float a = 0.f, e = 0.f;
    DLO_HIP(ctx, hipEventElapsedTime(&a, base, t.start));
    DLO_HIP(ctx, hipEventElapsedTime(&e, base, t.end));
    dlo_interval iv{};
    iv.kind = t.kind;
    iv.block = t.block;
    iv.chunk = t.chunk;
    iv.slot = t.slot;
    iv.landing = t.landing;
    iv.forward = t.fwd;
    iv.bytes = t.bytes;
    iv.start_ms = double(a) - double(best);
    iv.end_ms = double(e) - double(best);
    t_end = std::max(t_end, iv.end_ms);
    out.push_back(iv);
  }
  if (s) {
    s->last_forward_ms = t_end;
    // busy time per stream kind: length of the union of its intervals (the
    // two copy engines overlap)
    auto busy = [&](int kind) {
      std::vector<std::pair<double, double>> v;
      for (auto& iv : out)
        if (iv.kind == kind) v.push_back({iv.start_ms, iv.end_ms});
      std::sort(v.begin(), v.end());
      double tot = 0, cs = -1e300, ce = -1e300;
      for (auto& p : v) {
        if (p.first > ce) {
          if (ce > cs) tot += ce - cs;
          cs = p.first;
          ce = p.second;
        } else {
          ce = std::max(ce, p.second);
        }
      }
      if (ce > cs) tot += ce - cs;
      return tot;
    };
    const double h = busy(DLO_IV_H2D), a = busy(DLO_IV_ASM), c = busy(DLO_IV_COMPUTE);
    s->sum_h2d_ms = h;
    s->sum_asm_ms = a;
    s->sum_compute_ms = c;
    // Residency, per block instance g = forward * L + block:
    //  * in a slot from its first reconstruction start to its compute end;
    //  * on the device from its first H2D start (landing buffers included) to
    //    its compute end;
    //  * weight bytes: a block in its slot counts its padded size, a chunk in
    //    a landing buffer counts its length from its H2D start to the end of
    //    its reconstruction.
    const int64_t L = static_cast<int64_t>(ctx->blocks.size());
    struct Span {
      double asm0 = 1e300, h2d0 = 1e300, comp1 = -1e300;
    };
    std::vector<Span> sp;
    auto at = [&](const dlo_interval& iv) -> Span& {
      const size_t g = size_t(int64_t(std::max(iv.forward, 0)) * L + iv.block);
      if (sp.size() <= g) sp.resize(g + 1);
      return sp[g];
    };
    // landing occupancy: chunk (g, j) from its H2D start to its ASM end
    std::vector<std::pair<double, int64_t>> wev;
    struct ChunkKey {
      int64_t g;
      int chunk;
      bool operator<(const ChunkKey& o) const { return g < o.g || (g == o.g && chunk < o.chunk); }
    };
    std::vector<std::pair<ChunkKey, std::pair<double, int64_t>>> h2d_start;
    std::vector<std::pair<ChunkKey, double>> asm_end;
    for (auto& iv : out) {
      const int64_t g = int64_t(std::max(iv.forward, 0)) * L + iv.block;
      if (iv.kind == DLO_IV_ASM) {
        at(iv).asm0 = std::min(at(iv).asm0, iv.start_ms);
        asm_end.push_back({ChunkKey{g, iv.chunk}, iv.end_ms});
      } else if (iv.kind == DLO_IV_H2D) {
        at(iv).h2d0 = std::min(at(iv).h2d0, iv.start_ms);
        h2d_start.push_back({ChunkKey{g, iv.chunk}, {iv.start_ms, iv.bytes}});
      } else if (iv.kind == DLO_IV_COMPUTE) {
        at(iv).comp1 = std::max(at(iv).comp1, iv.end_ms);
      }
    }
    std::sort(asm_end.begin(), asm_end.end(), [](auto& u, auto& v) { return u.first < v.first; });
    for (auto& hs : h2d_start) {
      auto it = std::lower_bound(asm_end.begin(), asm_end.end(), hs.first,
                                 [](const auto& e, const ChunkKey& k) { return e.first < k; });
      if (it == asm_end.end() || it->first.g != hs.first.g || it->first.chunk != hs.first.chunk) continue;
      wev.push_back({hs.second.first, hs.second.second});
      wev.push_back({it->second, -hs.second.second});
    }
    std::vector<std::pair<double, int64_t>> slot_ev, dev_ev;
    for (size_t g = 0; g < sp.size(); ++g) {
      const Span& q = sp[g];
      if (q.comp1 < -1e299) continue;  // compute not traced
      const int64_t bbytes = int64_t(2) * ctx->dp * ctx->blocks[g % size_t(L)].shard;
      if (q.asm0 < 1e299) {
        slot_ev.push_back({q.asm0, 1});
        slot_ev.push_back({q.comp1, -1});
        wev.push_back({q.asm0, bbytes});
        wev.push_back({q.comp1, -bbytes});
      }
      if (q.h2d0 < 1e299) {
        dev_ev.push_back({q.h2d0, 1});
        dev_ev.push_back({q.comp1, -1});
      }
    }
    s->residency_high_water = static_cast<int32_t>(max_weighted_overlap(slot_ev));
    s->blocks_on_device_high_water = static_cast<int32_t>(max_weighted_overlap(dev_ev));
    s->weight_bytes_peak = max_weighted_overlap(wev);
    s->n_intervals = static_cast<int32_t>(out.size());
  }
  return DLO_OK;
}

}  // namespace

extern "C" DLO_API dlo_status dlo_get_stats(dlo_ctx* ctx, dlo_stats* out) {
  return guarded([&]() -> dlo_status {
    clear_error();
    dlo_status st = check_ctx(ctx);
    if (st != DLO_OK) return st;
    if (out == nullptr) return fail(DLO_E_INVAL, "out is NULL");
    DeviceGuard dg(ctx->device);
    memset(out, 0, sizeof(*out));
    out->num_blocks = static_cast<int32_t>(ctx->blocks.size());
    out->dp_size = ctx->dp;
    out->forwards = ctx->forwards;
    out->max_shard_elems = ctx->s_max;
    out->slot_bytes = ctx->slot_bytes;
    out->landing_bytes = ctx->landing_bytes;
    out->workspace_bytes = ctx->workspace_bytes;
    int64_t hb = 0;
    for (auto& b : ctx->blocks) hb += int64_t(2) * ctx->dp * b.shard;
    out->h2d_bytes_per_forward = hb;
    out->landing_chunk_elems = ctx->chunk_elems;
    out->max_block_bytes = size_t(2) * size_t(ctx->dp) * size_t(ctx->s_max);
    out->weight_bytes_allocated = 2 * ctx->slot_bytes + ctx->landing_bytes;
    std::vector<dlo_interval> tmp;
    return collect_trace(ctx, tmp, out);
  });
}

extern "C" DLO_API dlo_status dlo_get_trace(dlo_ctx* ctx, dlo_interval* out, int32_t cap, int32_t* n) {
  return guarded([&]() -> dlo_status {
    clear_error();
    dlo_status st = check_ctx(ctx);
    if (st != DLO_OK) return st;
    if (n == nullptr) return fail(DLO_E_INVAL, "n is NULL");
    DeviceGuard dg(ctx->device);
    std::vector<dlo_interval> tmp;
    st = collect_trace(ctx, tmp, nullptr);
    if (st != DLO_OK) return st;
    *n = static_cast<int32_t>(tmp.size());
    if (out) {
      if (cap < *n) return fail(DLO_E_INVAL, "cap %d < %d intervals", cap, *n);
      memcpy(out, tmp.data(), sizeof(dlo_interval) * tmp.size());
      // accumulating traces (kernel-only, or spanning forwards) are consumed
      if (!(ctx->flags & DLO_FLAG_TRACE) || (ctx->flags & DLO_FLAG_TRACE_SPAN)) drop_trace(ctx);
    }
    return DLO_OK;
  });
}

extern "C" DLO_API dlo_status dlo_set_flags(dlo_ctx* ctx, uint32_t flags) {
  return guarded([&]() -> dlo_status {
    clear_error();
    dlo_status st = check_ctx(ctx);
    if (st != DLO_OK) return st;
    constexpr uint32_t kKnown = DLO_FLAG_TRACE | DLO_FLAG_SERIALIZE | DLO_FLAG_POISON_SLOTS |
                                DLO_FLAG_TRACE_KERNELS | DLO_FLAG_TRACE_SPAN;
    if (flags & ~kKnown) return fail(DLO_E_INVAL, "unknown flags 0x%x", flags & ~kKnown);
    ctx->flags = flags;
    drop_trace(ctx);
    return DLO_OK;
  });
}

extern "C" DLO_API dlo_status dlo_set_trace_kinds(dlo_ctx* ctx, uint32_t kinds) {
  return guarded([&]() -> dlo_status {
    clear_error();
    dlo_status st = check_ctx(ctx);
    if (st != DLO_OK) return st;
    if (kinds & ~DLO_TRACE_KINDS_ALL) return fail(DLO_E_INVAL, "unknown interval kinds 0x%x", kinds & ~DLO_TRACE_KINDS_ALL);
    ctx->trace_kinds = kinds;
    drop_trace(ctx);
    return DLO_OK;
  });
}

extern "C" DLO_API dlo_status dlo_reserve_trace(dlo_ctx* ctx, int32_t forwards) {
  return guarded([&]() -> dlo_status {
    clear_error();
    dlo_status st = check_ctx(ctx);
    if (st != DLO_OK) return st;
    if (forwards < 0) return fail(DLO_E_INVAL, "forwards %d < 0", forwards);
    DeviceGuard dg(ctx->device);
    if (!dg.ok) return fail(DLO_E_HIP, "hipSetDevice(%d) failed", ctx->device);
    const size_t want = ctx->ev_next + size_t(forwards) * events_per_forward(ctx);
    if (!grow_pool(ctx, want)) return fail(DLO_E_HIP, "trace event creation failed");
    return DLO_OK;
  });
}
