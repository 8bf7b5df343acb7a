// Host-side argument checks shared by libsgmv's entry points.  Every check runs
// before any HIP call, so a rejected call has no effect.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <algorithm>
#include <cstdint>

#include "../../include/sgmv.h"

namespace sgmv_host {

constexpr int64_t kMaxDim = int64_t(1) << 22;
constexpr int kLongMin = 16;  // segments with at least this many rows use the MFMA kernels

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

// ------------------------------------------------------------------------------------
// workspace layout shared by every entry point (the same bytes serve both paths).
// Regions that must be zero between calls (counters, tagged partials) sit at the two
// ends; scratch grows from the front:
//   [0, 4)                  int32 flag bits (SGMV_FLAG_*: wait timed out, bad id, segment
//                           bounds that contradict the tables)
//   [256, 16640)            decode path: one counter per row, one per 256-byte line
//   [rowks_off, ...)        table path: split-K slice count of each sorted row
//   [v_off, ...)            table path: final float32 v of rows of long segments
//   [part_off, ...)         table path: float32 split-K partial sums
//   [dtab_off, table_end)   segment tables built on the device for n > 64 (meta word
//                           [S, min_len, max_len, n_valid], n_segments, perm, seg_starts,
//                           seg_adapter, sorted ids, A and B pointer tables)
//   ... free ...
//   [pool, end)             last pool_bytes(h_in, r) bytes of the caller's buffer (start
//                           rounded down to 256): decode path: tagged 64-bit split-K
//                           partial sums, laid out for 64 rows whatever n is
// Counters and the tagged partials are zero before a call and are left at zero by it;
// rowks, v, the partial sums and the device tables are scratch.  The scratch end grows
// with n, h_in and r and so does the size of the tagged partials at the back, so in a
// buffer of sgmv_workspace_bytes(n, h_in, r) bytes no call of at most n rows, h_in and r
// writes scratch over another such call's counters or tagged partials.
// ------------------------------------------------------------------------------------
constexpr int kMaxPoolRows = 64;
constexpr size_t kWsPoolCounters = 256;
constexpr int kCounterInts = 64;  // 256 bytes per counter

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// split-K chunk (elements of h_in) of the table path's GEMV shrink and of the decode path
inline int table_gemv_kc(int r) { return r == 16 ? 512 : 256; }
inline int pool_kc(int r) { return 8192 / r; }
// decode path: output columns per lane of an expand item (256 contiguous bytes of B; half
// as many, with twice the expand items, measured no faster on MI355X: the shorter
// epilogue was lost to the longer wait for the partial sums with more waves polling)
constexpr int pool_cpl(int r) { return 128 / r; }
// 64-bit words per row of a decode-path partial slice (r words: at least 128 bytes)
constexpr int pool_part_row(int r) { return r; }
// 64-bit words per decode-path partial slice (64 rows)
constexpr int64_t pool_slice(int r) { return static_cast<int64_t>(kMaxPoolRows) * pool_part_row(r); }

inline size_t pool_bytes(int32_t h_in, int32_t r) {
  const size_t ks = static_cast<size_t>((h_in + pool_kc(r) - 1) / pool_kc(r));
  return sizeof(uint64_t) * ks * static_cast<size_t>(pool_slice(r));
}

// start of the tagged partials inside a caller buffer of ws_bytes bytes
inline size_t pool_offset(size_t ws_bytes, int32_t h_in, int32_t r) {
  return (ws_bytes - pool_bytes(h_in, r)) / 256 * 256;
}

// rows the one-workgroup device sort handles (sgmv_build_segments_device and the decode
// entry point for 64 < n <= kDevSortMax)
constexpr int kDevSortMax = 4096;

// device segment tables inside the workspace, offsets from dtab_off
struct DevTabLayout {
  size_t meta, n_segments, perm, seg_starts, seg_adapter, sorted_ids, A_ptrs, B_ptrs, bytes;
};

inline DevTabLayout dev_tab_layout(int32_t n) {
  DevTabLayout D{};
  const size_t nn = static_cast<size_t>(n);
  D.meta = 0;
  D.n_segments = 16;
  D.perm = 256;
  D.seg_starts = align_up(D.perm + 4 * nn, 256);
  D.seg_adapter = align_up(D.seg_starts + 4 * (nn + 1), 256);
  D.sorted_ids = align_up(D.seg_adapter + 4 * nn, 256);
  D.A_ptrs = align_up(D.sorted_ids + 4 * nn, 256);
  D.B_ptrs = align_up(D.A_ptrs + 8 * nn, 256);
  D.bytes = align_up(D.B_ptrs + 8 * nn, 256);
  return D;
}

struct WsLayout {
  size_t rowks_off, v_off, part_off, dtab_off, table_end, total;
  int64_t slice;  // floats per split-K slice of the table path (n * r)
  int ks_max;     // table path: split-K slices the partial-sum area holds
};

// Layout of a call of n rows, h_in and rank r; .total is the smallest buffer that fits.
inline WsLayout ws_layout(int32_t n, int32_t h_in, int32_t r) {
  WsLayout L{};
  L.ks_max = (h_in + table_gemv_kc(r) - 1) / table_gemv_kc(r);
  const int ks_mfma = std::min(32, std::max(1, h_in / 256));  // MFMA shrink slices, at most
  if (ks_mfma > L.ks_max) L.ks_max = ks_mfma;
  L.slice = static_cast<int64_t>(n) * r;
  L.rowks_off = kWsPoolCounters + sizeof(int32_t) * kCounterInts * kMaxPoolRows;
  L.v_off = align_up(L.rowks_off + sizeof(int32_t) * static_cast<size_t>(n), 256);
  L.part_off = align_up(L.v_off + sizeof(float) * static_cast<size_t>(L.slice), 256);
  L.dtab_off = align_up(L.part_off + sizeof(float) * static_cast<size_t>(L.slice) * L.ks_max, 256);
  L.table_end = L.dtab_off + dev_tab_layout(n).bytes;
  // 256 bytes of slack so that the tagged partials' start, rounded down, stays past the
  // scratch
  L.total = L.table_end + 256 + pool_bytes(h_in, r);
  return L;
}

// Rank groups of a mixed-rank call with their scratch side by side (so that their chains
// can run concurrently): group g (ns[g] rows, rank rs[g]) uses the workspace from
// offsets[g] on, with the layout ws_layout(ns[g], h_in, rs[g]) relative to it, whose scratch
// [rowks_off, table_end) then follows the previous group's.  Groups of no rows get the
// previous offset and no room.  Returns the end of the last group's scratch, which must
// not pass the buffer's end.
inline size_t ranked_side_by_side(const int32_t* ns, const int32_t* rs, int count, int32_t h_in,
                                  size_t* offsets) {
  size_t off = 0, end = 0;
  for (int g = 0; g < count; ++g) {
    off = align_up(off, 256);
    if (offsets) offsets[g] = off;
    if (ns[g] <= 0) continue;
    const WsLayout L = ws_layout(ns[g], h_in, rs[g]);
    end = off + L.table_end;
    off += L.table_end - L.rowks_off;
  }
  return end;
}

// The table path on segment tables that live on the device (sgmv_kernels.hip): the
// tables and their meta word [S, min_len, max_len, n_valid] as written by the device sort;
// S_max bounds S.
hipError_t table_lora_add_device(hipStream_t st, int32_t dtype, int32_t r, void* y, int64_t ld_y,
                                 const void* x, int64_t ld_x, const void* const* A_ptrs,
                                 const void* const* B_ptrs, const int32_t* seg_starts,
                                 const int32_t* perm, const int32_t* meta, int32_t n,
                                 int32_t S_max, int32_t h_in, int32_t h_out, float scale,
                                 void* workspace);

}  // namespace sgmv_host
