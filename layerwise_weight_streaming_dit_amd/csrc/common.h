// Host-side helpers shared by the C ABI translation units.
#pragma once

#include <stdarg.h>
#include <stdint.h>

#include <exception>
#include <new>
#include <string>

#include "dlo.h"

namespace dlo {

// Set the thread-local last-error message and return `code`.
dlo_status fail(dlo_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Runs the body of a C entry point so that no C++ exception crosses the C
// ABI: the library's only throwing operations are host-side allocations
// (std::vector growth and the like), so a failure becomes DLO_E_HOST_OOM
// with the exception's message.
template <class F>
dlo_status guarded(F&& body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(DLO_E_HOST_OOM, "host memory allocation failed");
  } catch (const std::exception& e) {
    return fail(DLO_E_HOST_OOM, "host-side failure: %s", e.what());
  } catch (...) {
    return fail(DLO_E_HOST_OOM, "host-side failure");
  }
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Parameter table of one block (the cached metadata used to re-point
// parameters at slices of a slot).  Returns DLO_OK or DLO_E_INVAL.
struct BlockLayout {
  int64_t numel = 0;
  int64_t off_wqkv = 0, off_bqkv = 0, off_wo = 0, off_bo = 0, off_w1 = 0, off_b1 = 0;
  int64_t off_w2 = 0, off_b2 = 0, off_wada = 0, off_bada = 0;
  int n_params = 0;
  dlo_param_desc params[10 + 64];
};
constexpr int kMaxExtra = 64;

dlo_status validate_block(const dlo_block_desc* b, int index);
dlo_status compute_layout(const dlo_block_desc* b, BlockLayout* out);

}  // namespace dlo
