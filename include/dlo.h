/*
 * dlo.h -- C ABI of the layer-by-layer, weight-streamed DiT forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (vLLM-Omni "Distributed Layerwise Offload" release page):
 *   - section "Weight sharding with AllGather reconstruction": each block's
 *     flattened weight is split into dp_size equal shards of
 *     ceil(numel / dp_size) elements, zero-padded, and kept in pinned host
 *     memory; the full layer is rebuilt on the device by an all-gather;
 *   - section "Double-buffered prefetch with H2D + AllGather overlap": exactly
 *     two device slots, each the size of the largest block, allocated once;
 *     block N+1 is copied host-to-device and gathered on side streams while
 *     block N computes from the other slot; compute waits on an event before
 *     switching slots; parameters are re-pointed at slices of the slot from
 *     cached (offset, shape) metadata;
 *   - section "DP multi-concurrency": waves that cannot run are rejected before
 *     dispatch and failures close the path instead of hanging it.
 *
 * On one GPU this library plays every data-parallel rank: it holds all
 * dp_size shards of every block, copies all of them host-to-device, and a
 * reconstruction kernel stands in for all_gather_into_tensor.
 *
 * Conventions for every call:
 *   - the return value is a dlo_status: DLO_OK (0) or a negative error code;
 *     dlo_last_error() then returns a message (thread-local, valid until the
 *     next call on the same thread);
 *   - all validation happens before any GPU work is enqueued; a failed call
 *     leaves no work in flight;
 *   - after a HIP error inside dlo_forward or dlo_debug_assemble the context is
 *     poisoned: every later call on it except dlo_destroy returns
 *     DLO_E_POISONED (fail closed);
 *   - no C++ exception crosses this interface: a failed host-side allocation
 *     inside the library returns DLO_E_HOST_OOM, and when it happens while
 *     dlo_forward, dlo_forward_static or dlo_debug_assemble enqueues work, the
 *     context is poisoned as after a HIP error;
 *   - a context is not thread-safe; calls on one context must not overlap.
 *
 * Data formats:
 *   - bf16 and fp16 values travel as their 16-bit patterns (uint16_t);
 *   - a block's flat weight is the dense concatenation, in this order, of
 *       Wqkv[3d][d] bqkv[3d] Wo[d][d] bo[d] W1[m][d] b1[m] W2[d][m] b2[d]
 *       Wada[6d][c] bada[6d] extra_0[..] extra_1[..] ...
 *     with matrices row-major as [out][in] (y = x W^T + b) and q, k, v the
 *     three d-row thirds of Wqkv; extra vectors are streamed and reconstructed
 *     but not read by the block math;
 *   - activations x are fp32 row-major [tokens][d]; cond is fp32 [c].
 *
 * The block math (DiT block with adaLN-Zero conditioning, Peebles & Xie,
 * "Scalable Diffusion Models with Transformers", section 3.2):
 *     mod = Wada silu(cond) + bada = (shift1, scale1, gate1, shift2, scale2, gate2)
 *     x  += gate1 * (attn(LN(x) * (1 + scale1) + shift1) Wo^T + bo)
 *     x  += gate2 * (gelu_tanh((LN(x) * (1 + scale2) + shift2) W1^T + b1) W2^T + b2)
 * LayerNorm has no affine parameters and eps 1e-6; attention is non-causal
 * multi-head softmax(q k^T / sqrt(d / heads)) v.  Between blocks of different
 * width the residual keeps its first min(d_in, d_out) features and zero-fills
 * the rest.  Weights are streamed as bf16; the reconstruction writes the
 * gathered layer into its slot as fp16, the matrix cores' operand type (exact
 * for |w| >= 2^-17; smaller magnitudes round to fp16's subnormal grid, error
 * <= 2^-25; |w| > 65504 overflows), and every kernel of the block reads the
 * parameters in that form (biases and the adaLN weights in fp32 arithmetic);
 * activations between kernels are fp16; matrix-core accumulation, softmax,
 * the residual x and the modulation vectors are fp32.
 */
#ifndef DLO_H
#define DLO_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLO_API __attribute__((visibility("default")))
#define DLO_ABI_VERSION 2

typedef int32_t dlo_status;
#define DLO_OK 0
#define DLO_E_INVAL (-1)     /* bad argument or configuration */
#define DLO_E_SHAPE (-2)     /* element count or shape does not match the layout */
#define DLO_E_STATE (-3)     /* call not valid in the context's current state */
#define DLO_E_HOST_OOM (-4)  /* host allocation failed (pinned shards or the library's own bookkeeping) */
#define DLO_E_DEV_OOM (-5)   /* the caller's device arena is too small */
#define DLO_E_HIP (-6)       /* a HIP runtime call failed (context is poisoned) */
#define DLO_E_POISONED (-7)  /* an earlier HIP error poisoned the context */

/* Context flags (dlo_config.flags). */
#define DLO_FLAG_TRACE 0x1u        /* record a timed interval per H2D chunk,
                                      reconstruction chunk and block compute */
#define DLO_FLAG_SERIALIZE 0x2u    /* test hook: synchronous schedule (copy,
                                      wait, reconstruct, wait, compute), same
                                      kernels */
#define DLO_FLAG_POISON_SLOTS 0x4u /* test hook: fill a slot with fp16 NaN
                                      before reconstructing into it, so a read
                                      ahead of the reconstruction shows up */
#define DLO_FLAG_TRACE_KERNELS 0x8u /* record only the compute-stream intervals
                                       (block compute and each kernel): keeps
                                       events off the copy and gather streams.
                                       Without DLO_FLAG_TRACE the intervals
                                       accumulate over forwards until
                                       dlo_get_trace hands them out (at most
                                       2^19 per context; later ones are not
                                       recorded until then) */
#define DLO_FLAG_TRACE_SPAN 0x10u  /* with DLO_FLAG_TRACE: keep the intervals of
                                      consecutive forwards (each tagged with
                                      its forward index) until dlo_get_trace
                                      hands them out, so one trace shows how
                                      one forward's last block and the next
                                      forward's first block overlap */

typedef struct dlo_ctx dlo_ctx;

/* Shape of one block.  d_model must be a multiple of 128 and of n_heads with
 * d_model / n_heads in {64, 128}; d_mlp a multiple of 128; d_cond a multiple of
 * 64 and the same for every block.  extra_len lists n_extra lengths (>= 0) of
 * vectors appended to the flat weight; it is copied by dlo_create. */
typedef struct dlo_block_desc {
  int32_t d_model;
  int32_t n_heads;
  int32_t d_mlp;
  int32_t d_cond;
  int32_t n_extra;
  int32_t reserved;
  const int64_t* extra_len;
} dlo_block_desc;

typedef struct dlo_config {
  int32_t abi_version;         /* DLO_ABI_VERSION */
  int32_t num_blocks;          /* >= 1 */
  const dlo_block_desc* blocks;/* num_blocks entries, copied by dlo_create */
  int32_t dp_size;             /* number of shards per block, >= 1 */
  int32_t max_tokens;          /* largest token count dlo_forward accepts, in [1, 2^20], and
                                  max_tokens * max(2 * d_model, d_mlp) * 2 bytes below 4 GiB */
  int64_t landing_chunk_elems; /* largest H2D chunk in elements; 0 = default
                                  min(S_max, ceil(dp * S_max / 4), 2^27) with
                                  S_max the largest shard (the two landing
                                  buffers then hold at most half of the
                                  largest block); else >= 4096.
                                  A block's padded weight is split into equal
                                  chunks of at most this size (they may span
                                  shards, which sit back to back in one pinned
                                  region per block) */
  int32_t device;              /* HIP device ordinal the context runs on */
  uint32_t flags;              /* DLO_FLAG_* */
  void* arena;                 /* device memory owned by the caller, 256-byte
                                  aligned, at least dlo_required_bytes' total;
                                  must stay alive until dlo_destroy */
  size_t arena_bytes;
  hipStream_t copy_stream;     /* side stream for the H2D copies of even
                                  chunks; NULL = the library creates its own.
                                  Odd chunks go on a second copy stream the
                                  library always owns (a second DMA engine) */
  hipStream_t gather_stream;   /* side stream for reconstruction; NULL = the
                                  library creates its own */
} dlo_config;

/* One entry of a block's parameter table (cached metadata for re-pointing). */
typedef struct dlo_param_desc {
  char name[16];
  int64_t offset;   /* element offset into the block's flat weight */
  int32_t ndim;     /* 1 or 2 */
  int32_t reserved;
  int64_t shape[2];
} dlo_param_desc;

/* One timed interval of the streaming schedule (DLO_FLAG_TRACE): per H2D
 * chunk, per reconstruction chunk, per block compute and per kernel. */
#define DLO_IV_H2D 0
#define DLO_IV_ASM 1
#define DLO_IV_COMPUTE 2
/* kernels inside a block's compute interval (compute stream) */
#define DLO_IV_K_ADALN 3   /* adaLN modulation vector */
#define DLO_IV_K_LN1 4     /* LayerNorm + modulate before attention */
#define DLO_IV_K_QK 5      /* q, k projection GEMM */
#define DLO_IV_K_V 6       /* v projection GEMM (transposed output) */
#define DLO_IV_K_ATTN 7    /* attention */
#define DLO_IV_K_OUT 8     /* output projection GEMM + gated residual */
#define DLO_IV_K_LN2 9     /* LayerNorm + modulate before the MLP */
#define DLO_IV_K_FC1 10    /* MLP up GEMM + GELU */
#define DLO_IV_K_FC2 11    /* MLP down GEMM + gated residual */
typedef struct dlo_interval {
  int32_t kind;      /* DLO_IV_* */
  int32_t block;     /* block index */
  int32_t chunk;     /* chunk index within the block, -1 otherwise */
  int32_t slot;      /* slot written (ASM) or read (COMPUTE), -1 for H2D */
  int32_t landing;   /* landing buffer written (H2D) or read (ASM), -1 otherwise */
  int32_t forward;   /* index of the dlo_forward call (0 = the context's first) */
  int64_t bytes;     /* bytes moved (H2D, ASM reads) or 0 */
  double start_ms;   /* relative to the start of the forward */
  double end_ms;
} dlo_interval;

typedef struct dlo_stats {
  int32_t num_blocks;
  int32_t dp_size;
  int64_t forwards;            /* completed dlo_forward calls */
  int64_t max_shard_elems;     /* S_max = max over blocks of ceil(numel_b / dp) */
  size_t slot_bytes;           /* bytes of ONE slot = 2 * dp * S_max */
  size_t landing_bytes;        /* both landing buffers */
  size_t workspace_bytes;      /* activations and scratch */
  int32_t residency_high_water;/* most blocks in the two slots at once (a block
                                  holds its slot from its first reconstruction
                                  start to its compute end), from the traced
                                  intervals (0 if untraced) */
  int32_t n_intervals;         /* intervals the statistics below cover */
  double last_forward_ms;      /* first H2D start to last compute end (traced) */
  double sum_h2d_ms;           /* busy time (union of intervals) per kind (traced) */
  double sum_asm_ms;
  double sum_compute_ms;
  int64_t h2d_bytes_per_forward;
  /* -- device weight memory (release page, TL;DR and section "Double-buffered
   *    prefetch": two layers' weights on the device at any time) */
  int64_t landing_chunk_elems; /* H2D chunk size in use (elements) */
  size_t max_block_bytes;      /* largest padded block, 2 * dp * S_max bytes */
  size_t weight_bytes_allocated;/* slots + landing buffers: every device byte
                                  that ever holds weight data */
  int32_t blocks_on_device_high_water; /* most blocks with any weight bytes on
                                  the device at once (a block counts from its
                                  first H2D start, landing buffers included, to
                                  its compute end), traced; 0 if untraced */
  int32_t reserved2;
  int64_t weight_bytes_peak;   /* most weight bytes in use at once (blocks in
                                  slots at their padded size plus chunks in
                                  landing buffers), traced; 0 if untraced */
} dlo_stats;

/* Pure host query: the parameter table, element count and shard size of one
 * block at dp_size (release page, section "Weight sharding with AllGather
 * reconstruction": one flat buffer per layer, cut into dp_size shards of
 * ceil(numel / dp_size) elements).  out may be NULL (then only counts are
 * returned); cap is its capacity.  No device or context needed.  Errors:
 * DLO_E_INVAL for a block shape the kernels cannot run or cap too small. */
DLO_API dlo_status dlo_block_layout(const dlo_block_desc* block, int32_t dp_size,
                                    int64_t* numel, int64_t* shard_size,
                                    int32_t* n_params, dlo_param_desc* out, int32_t cap);

/* Pure host query, before dlo_create: device bytes the arena must hold.
 * slots = 2 * slot bytes (the two buffers "sized to the largest block" of the
 * release page's section "Double-buffered prefetch with H2D + AllGather
 * overlap"); landing = the two landing buffers for H2D chunks (the per-rank
 * receive buffers of the all-gather); workspace = activations for
 * max_tokens; total = the sum plus alignment.  Any output pointer may be
 * NULL.  Errors: those of dlo_create's validation. */
DLO_API dlo_status dlo_required_bytes(const dlo_config* cfg, size_t* slots, size_t* landing,
                                      size_t* workspace, size_t* total);

/* Enable layerwise offload for one model (release page, section "Quick
 * start": the feature is switched on per model with a dp_size; section
 * "Double-buffered prefetch": the two slots are allocated once, sized to the
 * largest block, and shared by every layer).  Validates cfg, computes every
 * block's layout and shard size, carves the caller's arena into slots,
 * landing buffers and workspace, and creates events (and streams if not
 * given).  Allocates no device memory: the arena stays the caller's and must
 * outlive the context.  *out is owned by the library until dlo_destroy.
 * Errors: DLO_E_INVAL (bad field, arena NULL or misaligned), DLO_E_DEV_OOM
 * (arena smaller than dlo_required_bytes' total), DLO_E_HIP (stream or event
 * creation failed; nothing is left allocated). */
DLO_API dlo_status dlo_create(const dlo_config* cfg, dlo_ctx** out);

/* Shard and pin one block (release page, section "Weight sharding with
 * AllGather reconstruction": each layer's flattened weight is padded to a
 * multiple of dp_size, cut into equal shards kept in pinned host memory, and
 * the source parameter is replaced by an empty placeholder).  numel must
 * equal the block's layout numel (else DLO_E_SHAPE).  Allocates dp_size
 * pinned host shards of S = ceil(numel / dp_size) elements (back to back in
 * one pinned region: shard r at element r * S), copies the flat weight's
 * slice into each and zero-pads the tail.  Keeps no reference to flat_bf16:
 * the caller may free it on return (the placeholder step).  Reloading a
 * block replaces its shards; waits for in-flight copies on the context's
 * streams first.  Errors: DLO_E_INVAL (block index, NULL), DLO_E_SHAPE,
 * DLO_E_HOST_OOM (pinned allocation failed; the block stays unloaded). */
DLO_API dlo_status dlo_load_shards(dlo_ctx* ctx, int32_t block, const uint16_t* flat_bf16,
                                   int64_t numel);

/* The streamed forward over every block, in order (release page, section
 * "Double-buffered prefetch with H2D + AllGather overlap": layer N+1 is copied
 * host-to-device and gathered on side streams while layer N computes from the
 * other buffer; compute waits on an event before it switches buffers; the
 * layer's parameters are re-pointed at slices of its buffer).  x: device fp32
 * [tokens][d of block 0] in, [tokens][d of the last block] out, in place;
 * its buffer must hold tokens * max_d floats.  cond: device fp32 [d_cond].
 * Enqueues on stream (the compute stream) and the context's side streams and
 * returns without waiting; the result is ready when stream reaches it.  The
 * call's work is ordered after the previous call's on this context even when
 * the two calls pass different streams (the context's workspace is shared).
 * Consecutive blocks alternate slots, and the alternation continues across
 * calls (block 0 of a call takes the slot the previous call's last block
 * does not use), so back-to-back calls -- one per denoising step -- stream
 * the next call's first block while the previous call's last block computes.
 * The copy of a block starts only after the block two places earlier has
 * finished computing, so at most two blocks' weights are on the device at
 * any time.  Errors before any enqueue: DLO_E_STATE if a block has no
 * shards, DLO_E_INVAL if tokens is outside [1, max_tokens] or a pointer is
 * NULL or misaligned; DLO_E_HIP (context poisoned) if an enqueue fails. */
DLO_API dlo_status dlo_forward(dlo_ctx* ctx, float* x, const float* cond, int32_t tokens,
                               hipStream_t stream);

/* dlo_forward for callers that cannot allocate device memory at call time
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same schedule, kernels and results as dlo_forward, but the
 * per-forward activation workspace is the library's own static device
 * scratch -- 256 MiB per device, held from the first dlo_create on that device
 * until the process ends -- instead of the arena's workspace region; the
 * call itself allocates nothing.  Every call on one device shares that
 * device's scratch: calls whose work may overlap on one device (another
 * context, another stream without ordering) race and must not be issued.
 * Nothing in the scratch needs to start cleared: each region is written
 * before it is read.  Errors before any enqueue: those of dlo_forward, plus
 * DLO_E_INVAL if `tokens` needs more than 256 MiB of activations, and
 * DLO_E_STATE if a trace flag is set (tracing creates timing events) or the
 * scratch could not be mapped on the device. */
DLO_API dlo_status dlo_forward_static(dlo_ctx* ctx, float* x, const float* cond, int32_t tokens,
                                      hipStream_t stream);

/* Tear the context down (release page, section "Double-buffered prefetch":
 * the buffers live as long as the model).  Synchronises the context's
 * streams (also on a poisoned context, whose work may still be in flight),
 * frees pinned shards, events and owned streams.  The arena returns
 * to the caller.  NULL is a no-op.  Always returns DLO_OK. */
DLO_API dlo_status dlo_destroy(dlo_ctx* ctx);

/* Change the context's flags (DLO_FLAG_*) for the forwards enqueued after
 * this call, so that one pinned shard store serves timed, traced and
 * serialized runs.  Drops recorded intervals.  Errors: DLO_E_INVAL for an
 * unknown flag, DLO_E_POISONED. */
DLO_API dlo_status dlo_set_flags(dlo_ctx* ctx, uint32_t flags);

/* Restrict the intervals that tracing records to the kinds whose bit is set
 * in `kinds` (bit n records DLO_IV kind n; DLO_TRACE_KINDS_ALL, the default,
 * records every kind).  A timed run can then carry HIP events around only
 * the kernel it measures: every event pair recorded between two kernels
 * costs the compute stream a little time.  Applies to the forwards enqueued
 * after this call, under DLO_FLAG_TRACE or DLO_FLAG_TRACE_KERNELS; the
 * summary figures of dlo_get_stats need the H2D, reconstruction and compute
 * kinds.  Drops recorded intervals.  Errors: DLO_E_INVAL for a bit past
 * DLO_IV_K_FC2, DLO_E_POISONED. */
#define DLO_TRACE_KINDS_ALL 0xFFFu
DLO_API dlo_status dlo_set_trace_kinds(dlo_ctx* ctx, uint32_t kinds);

/* Create, ahead of time, the timing events that `forwards` traced forwards
 * under the current flags need, so that no event is created while they are
 * enqueued (creating events mid-run perturbs the timings).  Errors:
 * DLO_E_INVAL (forwards < 0), DLO_E_HIP. */
DLO_API dlo_status dlo_reserve_trace(dlo_ctx* ctx, int32_t forwards);

/* The parameter table of block `block` (see dlo_block_layout). */
DLO_API dlo_status dlo_layout(dlo_ctx* ctx, int32_t block, int64_t* numel, int64_t* shard_size,
                              int32_t* n_params, dlo_param_desc* out, int32_t cap);

/* Read-only view of pinned shard `rank` of block `block` (n = shard size). */
DLO_API dlo_status dlo_get_shard(dlo_ctx* ctx, int32_t block, int32_t rank,
                                 const uint16_t** ptr, int64_t* n);

/* Run the real H2D -> landing -> reconstruction path for one block into
 * slot (block % 2), synchronously, and copy the reconstructed numel elements
 * (fp16 patterns: the flat weight converted element by element) to host_out
 * (capacity cap elements).  Must not overlap a forward. */
DLO_API dlo_status dlo_debug_assemble(dlo_ctx* ctx, int32_t block, uint16_t* host_out,
                                      int64_t cap);

/* Counters and the summary of the recorded intervals (the last traced
 * forward, or every forward recorded since the trace was last handed out
 * under DLO_FLAG_TRACE_SPAN).  Synchronises the context's streams. */
DLO_API dlo_status dlo_get_stats(dlo_ctx* ctx, dlo_stats* out);

/* The recorded intervals: those of the last traced forward (DLO_FLAG_TRACE),
 * or of every forward since the previous call that returned intervals
 * (DLO_FLAG_TRACE with DLO_FLAG_TRACE_SPAN, or DLO_FLAG_TRACE_KERNELS alone;
 * those are then cleared); cap entries at most, *n receives the number
 * recorded (call with out = NULL to size the buffer; that clears nothing).
 * Times are in ms from the earliest recorded event.  Synchronises the
 * context's streams. */
DLO_API dlo_status dlo_get_trace(dlo_ctx* ctx, dlo_interval* out, int32_t cap, int32_t* n);

/* Message of the last failed call on this thread ("" if none). */
DLO_API const char* dlo_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DLO_H */
