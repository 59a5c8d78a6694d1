// Host-side argument checks shared by the C-ABI entry points.  Everything here
// runs before a launch; a failed check returns an rra_status and enqueues
// nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rra.h"
#include "rra_device.hpp"

namespace rra {

inline bool aligned(const void* p, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

// A bf16 tensor accessed with 16-byte vectors: base 16-byte aligned and a row
// stride that keeps every row 16-byte aligned.
inline bool vec_ok(const void* p, int64_t stride_elems) {
  return aligned(p, 16) && stride_elems % 8 == 0;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? RRA_OK : RRA_ERR_LAUNCH;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The multiply-high constants of n / d for 0 <= n < 2^31, 1 <= d < 2^31
// (FastDiv in the device header).
inline FastDiv make_fast_div(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t magic = ((uint64_t(1) << (31 + l)) + d - 1) / d;
  return FastDiv{d, static_cast<uint32_t>(magic), 31 + l};
}

// Per-group scales are reduced inside one 16-lane row (group 128 = 16 lanes x
// 8 values) or one 8-lane half row (group 64).
inline bool group_ok(int g) { return g == 64 || g == 128; }

}  // namespace rra

#define RRA_REQUIRE(cond, status) \
  do {                            \
    if (!(cond)) return (status); \
  } while (0)
