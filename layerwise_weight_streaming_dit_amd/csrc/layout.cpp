// Block parameter layout and error reporting (host only, no device calls).
//
// The offload backend treats a block's weights as one flattened tensor and
// re-points each parameter at a slice of the gathered buffer from cached
// (offset, shape) metadata (vLLM-Omni release page, sections "Weight sharding
// with AllGather reconstruction" and "Double-buffered prefetch with H2D +
// AllGather overlap").  The order used here is a dense concatenation:
//   Wqkv[3d][d] bqkv[3d] Wo[d][d] bo[d] W1[m][d] b1[m] W2[d][m] b2[d]
//   Wada[6d][c] bada[6d] extra_0 .. extra_{n-1}
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace dlo {

namespace {
// A fixed buffer, so that reporting an error never allocates (and so cannot
// fail itself, e.g. while a host allocation failure is being reported).
thread_local char g_last_error[512];
}

dlo_status fail(dlo_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_last_error[0] = '\0'; }

const char* last_error_cstr() { return g_last_error; }

dlo_status validate_block(const dlo_block_desc* b, int i) {
  if (b == nullptr) return fail(DLO_E_INVAL, "block %d: descriptor is NULL", i);
  if (b->d_model < 128 || b->d_model % 128 != 0 || b->d_model > 8192)
    return fail(DLO_E_INVAL, "block %d: d_model %d must be a multiple of 128 in [128, 8192]", i,
                b->d_model);
  if (b->n_heads < 1 || b->d_model % b->n_heads != 0)
    return fail(DLO_E_INVAL, "block %d: d_model %d not divisible by n_heads %d", i, b->d_model,
                b->n_heads);
  const int hd = b->d_model / b->n_heads;
  if (hd != 64 && hd != 128)
    return fail(DLO_E_INVAL, "block %d: head dim %d must be 64 or 128", i, hd);
  if (b->d_mlp < 128 || b->d_mlp % 128 != 0 || b->d_mlp > 65536)
    return fail(DLO_E_INVAL, "block %d: d_mlp %d must be a multiple of 128 in [128, 65536]", i,
                b->d_mlp);
  if (b->d_cond < 64 || b->d_cond % 64 != 0 || b->d_cond > 4096)
    return fail(DLO_E_INVAL, "block %d: d_cond %d must be a multiple of 64 in [64, 4096]", i, b->d_cond);
  if (b->n_extra < 0 || b->n_extra > kMaxExtra)
    return fail(DLO_E_INVAL, "block %d: n_extra %d outside [0, %d]", i, b->n_extra, kMaxExtra);
  if (b->n_extra > 0 && b->extra_len == nullptr)
    return fail(DLO_E_INVAL, "block %d: extra_len is NULL", i);
  for (int e = 0; e < b->n_extra; ++e)
    if (b->extra_len[e] < 0 || b->extra_len[e] > (int64_t(1) << 40))
      return fail(DLO_E_INVAL, "block %d: extra %d has bad length %lld", i, e,
                  static_cast<long long>(b->extra_len[e]));
  return DLO_OK;
}

dlo_status compute_layout(const dlo_block_desc* b, BlockLayout* L) {
  dlo_status st = validate_block(b, 0);
  if (st != DLO_OK) return st;
  const int64_t d = b->d_model, m = b->d_mlp, c = b->d_cond;
  int64_t off = 0;
  int n = 0;
  auto add = [&](const char* name, int64_t r, int64_t cdim, int64_t* slot) {
    dlo_param_desc& p = L->params[n++];
    memset(&p, 0, sizeof(p));
    snprintf(p.name, sizeof(p.name), "%s", name);
    p.offset = off;
    if (cdim > 0) {
      p.ndim = 2;
      p.shape[0] = r;
      p.shape[1] = cdim;
      off += r * cdim;
    } else {
      p.ndim = 1;
      p.shape[0] = r;
      off += r;
    }
    if (slot) *slot = p.offset;
  };
  add("Wqkv", 3 * d, d, &L->off_wqkv);
  add("bqkv", 3 * d, 0, &L->off_bqkv);
  add("Wo", d, d, &L->off_wo);
  add("bo", d, 0, &L->off_bo);
  add("W1", m, d, &L->off_w1);
  add("b1", m, 0, &L->off_b1);
  add("W2", d, m, &L->off_w2);
  add("b2", d, 0, &L->off_b2);
  add("Wada", 6 * d, c, &L->off_wada);
  add("bada", 6 * d, 0, &L->off_bada);
  for (int e = 0; e < b->n_extra; ++e) {
    char nm[16];
    snprintf(nm, sizeof(nm), "extra%d", e);
    add(nm, b->extra_len[e], 0, nullptr);
  }
  L->n_params = n;
  L->numel = off;
  return DLO_OK;
}

}  // namespace dlo

extern "C" DLO_API const char* dlo_last_error(void) { return dlo::last_error_cstr(); }

extern "C" DLO_API dlo_status dlo_block_layout(const dlo_block_desc* block, int32_t dp_size,
                                               int64_t* numel, int64_t* shard_size,
                                               int32_t* n_params, dlo_param_desc* out, int32_t cap) {
  return dlo::guarded([&]() -> dlo_status {
    dlo::clear_error();
    if (dp_size < 1) return dlo::fail(DLO_E_INVAL, "dp_size %d must be >= 1", dp_size);
    dlo::BlockLayout L;
    dlo_status st = dlo::compute_layout(block, &L);
    if (st != DLO_OK) return st;
    if (numel) *numel = L.numel;
    if (shard_size) *shard_size = dlo::ceil_div(L.numel, dp_size);
    if (n_params) *n_params = L.n_params;
    if (out) {
      if (cap < L.n_params) return dlo::fail(DLO_E_INVAL, "cap %d < %d parameters", cap, L.n_params);
      memcpy(out, L.params, sizeof(dlo_param_desc) * L.n_params);
    }
    return DLO_OK;
  });
}
