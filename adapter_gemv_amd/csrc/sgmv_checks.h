// Host-side argument checks shared by libsgmv's entry points.  Every check runs
// before any HIP call, so a rejected call has no effect.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/sgmv.h"

namespace sgmv_host {

constexpr int64_t kMaxDim = int64_t(1) << 22;

inline bool rank_ok(int32_t r) { return r == 16 || r == 32 || r == 64; }

inline bool ranges_overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

inline size_t matrix_bytes(int32_t rows, int64_t ld, int32_t cols) {
  if (rows <= 0) return 0;
  return (static_cast<size_t>(rows - 1) * static_cast<size_t>(ld) + static_cast<size_t>(cols)) * 2;
}

// checks shared by every device entry point; 0 when fine
inline int check_segments(int32_t n, int32_t S, int32_t min_len, int32_t max_len) {
  if (n < 0) return SGMV_ERR_SHAPE;
  if (n == 0) return SGMV_OK;
  if (S < 1 || S > n) return SGMV_ERR_SHAPE;
  if (min_len < 0 || max_len < 1 || min_len > max_len || max_len > n) return SGMV_ERR_SHAPE;
  // pigeonhole: the longest segment holds at least ceil(n/S) rows, the shortest at most n/S
  if (static_cast<int64_t>(max_len) * S < n) return SGMV_ERR_SHAPE;
  if (static_cast<int64_t>(min_len) * S > n) return SGMV_ERR_SHAPE;
  return SGMV_OK;
}

inline int check_dim(int32_t h, int64_t ld) {
  if (h < 8 || h > kMaxDim || ld < h) return SGMV_ERR_SHAPE;
  if (h % 8 != 0 || ld % 8 != 0) return SGMV_ERR_ALIGNMENT;
  return SGMV_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? SGMV_OK : SGMV_ERR_HIP; }

inline int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SGMV_ERR_HIP;
  return SGMV_OK;
}

}  // namespace sgmv_host
