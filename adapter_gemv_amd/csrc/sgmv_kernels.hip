// libsgmv device code for gfx950 (MI355X): the SGMV shrink and expand kernels and the
// C-ABI entry points that validate arguments and launch them.
//
// The computation is the per-adapter low-rank addition of the Punica paper summary
// (research.elamur.ai, "Summary"): every token t adds scale * (x[t] @ A[a_t]) @ B[a_t]
// to its backbone output y[t], tokens of one adapter being grouped into a segment
// (same page, "Interesting ideas", I2) so that each adapter's A and B are read once
// per call.
//
// Work split.  A segment shorter than kLongMin rows is a batch of matrix-vector
// products and is bound by reading A and B; it uses wavefront-reduction ("GEMV")
// kernels with one workgroup per (segment, K chunk) and per (segment, column
// chunk).  Longer segments (prefill) are dense contractions and go through MFMA
// tiles over 16 sorted rows.  v = x @ A is kept in float32: the shrink kernels write
// split-K partial sums to the workspace and the expand kernels add the slices in a
// fixed order, so results are reproducible run to run (no float atomics).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "../../include/sgmv.h"
#include "sgmv_checks.h"
#include "sgmv_device.h"

namespace {

using namespace sgmv_dev;
using namespace sgmv_host;

constexpr int kLongMin = 16;   // segments with at least this many rows use MFMA tiles
constexpr int kTileRows = 16;  // sorted rows per tile on the long-segment path
constexpr int kShortMax = kLongMin - 1;

// Segment that holds sorted row `row` (0 <= row < n): the number of s in [1, S] with
// seg_starts[s] <= row, since seg_starts is non-decreasing with seg_starts[0] = 0.
// Block-wide; every thread gets the result.
__device__ inline int block_find_segment(const int32_t* __restrict__ seg_starts, int S, int row,
                                         int* s_count) {
  if (threadIdx.x == 0) *s_count = 0;
  __syncthreads();
  int c = 0;
  for (int s = 1 + static_cast<int>(threadIdx.x); s <= S; s += blockDim.x) c += (seg_starts[s] <= row);
  if (c) atomicAdd(s_count, c);
  __syncthreads();
  return *s_count;
}

// ------------------------------------------------------------------------------------
// GEMV path (segments with 1 .. kShortMax rows)
// ------------------------------------------------------------------------------------
// Lane (j, g) of a wave reads row j of A[a] (= column j of A) over its own contiguous
// run of 8*KV k values, so the only cross-lane sum is over the G = 64/R lanes that
// share j.  Four waves cover consecutive k ranges and are summed through LDS.
template <int R>
struct GemvCfg {
  static constexpr int G = 64 / R;               // k groups per wave
  static constexpr int KV = (R == 64) ? 8 : 4;   // 16-byte vectors per lane and row
  static constexpr int WAVE_K = G * 8 * KV;      // k values per wave
  static constexpr int KC = 4 * WAVE_K;          // k values per workgroup (split-K chunk)
  static constexpr int MR = 16 / KV;             // token rows loaded per pass
};

template <int DT, int R>
__global__ __launch_bounds__(256) void shrink_gemv_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* const* __restrict__ A_ptrs,
    const int32_t* __restrict__ seg_starts, const int32_t* __restrict__ perm, int32_t h_in,
    float* __restrict__ part, int64_t slice, int32_t* __restrict__ rowks, int32_t ks) {
  using C = GemvCfg<R>;
  __shared__ float red[4][kShortMax][R];
  const int s = blockIdx.x, kc = blockIdx.y;
  const int seg0 = seg_starts[s];
  const int m = seg_starts[s + 1] - seg0;
  if (m <= 0 || m >= kLongMin) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane % R, g = lane / R;
  const int kbase = kc * C::KC + w * C::WAVE_K + g * 8 * C::KV;

  const uint16_t* Arow = A_ptrs[s] + static_cast<int64_t>(j) * h_in;
  uint4 a[C::KV];
#pragma unroll
  for (int v = 0; v < C::KV; ++v) {
    const int k = kbase + 8 * v;
    a[v] = (k < h_in) ? ld16(Arow + k) : zero4();
  }
  for (int i0 = 0; i0 < m; i0 += C::MR) {
    uint4 xv[C::MR][C::KV];
#pragma unroll
    for (int r = 0; r < C::MR; ++r) {
      const int i = i0 + r;
      const uint16_t* xr = nullptr;
      if (i < m) xr = x + static_cast<int64_t>(perm ? perm[seg0 + i] : seg0 + i) * ld_x;
#pragma unroll
      for (int v = 0; v < C::KV; ++v) {
        const int k = kbase + 8 * v;
        xv[r][v] = (xr && k < h_in) ? ld16(xr + k) : zero4();
      }
    }
#pragma unroll
    for (int r = 0; r < C::MR; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int v = 0; v < C::KV; ++v) acc = dot8<DT>(xv[r][v], a[v], acc);
#pragma unroll
      for (int msk = R; msk < 64; msk <<= 1) acc += __shfl_xor(acc, msk);
      if (g == 0 && i0 + r < m) red[w][i0 + r][j] = acc;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < m * R; idx += 256) {
    const int i = idx / R, jj = idx % R;
    const float sum = (red[0][i][jj] + red[1][i][jj]) + (red[2][i][jj] + red[3][i][jj]);
    part[kc * slice + static_cast<int64_t>(seg0 + i) * R + jj] = sum;
  }
  if (kc == 0)
    for (int i = threadIdx.x; i < m; i += 256) rowks[seg0 + i] = ks;
}

// Lane owns CPL = 128/R consecutive output columns: its block of B (CPL rows of the
// stored [h_out, r] array) is 256 contiguous bytes, and its slice of y is 256/R bytes.
template <int DT, int R>
__global__ __launch_bounds__(64) void expand_gemv_kernel(
    uint16_t* __restrict__ y, int64_t ld_y, const float* __restrict__ vsrc, int64_t slice,
    int32_t ks, const uint16_t* const* __restrict__ B_ptrs, const int32_t* __restrict__ seg_starts,
    const int32_t* __restrict__ perm, int32_t h_out, float scale) {
  using E = Elem<DT>;
  constexpr int CPL = 128 / R;
  constexpr int NV = 16;  // CPL * R / 8
  constexpr int YW = CPL / 2;  // 32-bit words of y per lane and row
  __shared__ float vs[kShortMax][R];
  const int s = blockIdx.x;
  const int seg0 = seg_starts[s];
  const int m = seg_starts[s + 1] - seg0;
  if (m <= 0 || m >= kLongMin) return;
  const int lane = threadIdx.x;
  const int c0 = (blockIdx.y * 64 + lane) * CPL;
  const bool cin = c0 < h_out;

  uint4 b[NV];
  const uint16_t* Bblk = B_ptrs[s] + static_cast<int64_t>(c0) * R;
#pragma unroll
  for (int v = 0; v < NV; ++v) b[v] = cin ? ld16(Bblk + 8 * v) : zero4();

  uint32_t yv[kShortMax][YW];
  uint16_t* yrow[kShortMax];
#pragma unroll
  for (int i = 0; i < kShortMax; ++i) {
    yrow[i] = nullptr;
    if (i < m) yrow[i] = y + static_cast<int64_t>(perm ? perm[seg0 + i] : seg0 + i) * ld_y + c0;
#pragma unroll
    for (int q = 0; q < YW; ++q) yv[i][q] = 0u;
    if (i < m && cin) load_words<YW>(yrow[i], yv[i]);
  }

  for (int idx = lane; idx < m * R; idx += 64) {
    const int i = idx / R, jj = idx % R;
    vs[i][jj] = sum_slices(vsrc + static_cast<int64_t>(seg0 + i) * R + jj, slice, ks);
  }
  __syncthreads();
  if (!cin) return;

#pragma unroll
  for (int i = 0; i < kShortMax; ++i) {
    if (i >= m) continue;
    float out[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      float acc = 0.f;
#pragma unroll
      for (int jj = 0; jj < R; ++jj) {
        const int e = cc * R + jj;
        acc = fmaf(vs[i][jj], elem<DT>(b[e >> 3], e & 7), acc);
      }
      const uint32_t w = yv[i][cc >> 1];
      const float yin = (cc & 1) ? E::hi(w) : E::lo(w);
      out[cc] = fmaf(scale, acc, yin);
    }
    uint32_t packed[YW];
#pragma unroll
    for (int q = 0; q < YW; ++q) packed[q] = E::pack(out[2 * q], out[2 * q + 1]);
    store_words<YW>(yrow[i], packed);
  }
}

// ------------------------------------------------------------------------------------
// long-segment path (segments with >= kLongMin rows): tiles of 16 sorted rows
// ------------------------------------------------------------------------------------
// MFMA 16x16x32: the x tile (16 rows x 32 k) is the A operand and the adapter's A
// (32 k x 16 r, read from the stored rows of A[a]) the B operand; lane l supplies
// row/column l%16 and 8 consecutive k values of group l/16.  Each lane walks its own
// contiguous 8*U-element run of k per step; the same k map is used for both
// operands, so the contraction is exact whatever order the hardware sums in.
template <int DT, int R>
__global__ __launch_bounds__(256) void shrink_mfma_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* const* __restrict__ A_ptrs,
    const int32_t* __restrict__ seg_starts, int32_t S, const int32_t* __restrict__ perm, int32_t n,
    int32_t h_in, int32_t kcm, float* __restrict__ part, int64_t slice, int32_t* __restrict__ rowks,
    int32_t ks) {
  using E = Elem<DT>;
  constexpr int U = (R == 64) ? 4 : 8;
  constexpr int NB = R / 16;
  constexpr int WSTEP = 32 * U;
  __shared__ int s_count;
  __shared__ f32x4_t red[4][NB][64];
  const int r0 = blockIdx.x * kTileRows;
  const int r1 = min(n, r0 + kTileRows);
  const int kc = blockIdx.y;
  int seg = block_find_segment(seg_starts, S, r0, &s_count);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int mrow = lane & 15, kq = lane >> 4;
  const int kw0 = kc * kcm + w * (kcm / 4);
  const int kw1 = min(h_in, kw0 + kcm / 4);

  for (int r = r0; r < r1; ++seg) {
    const int sb = seg_starts[seg], se = seg_starts[seg + 1];
    const int lo = r, hi = min(r1, se);
    r = hi;
    if (se - sb < kLongMin) continue;  // uniform across the block
    const int i = r0 + mrow;
    const uint16_t* xr = nullptr;
    if (i >= lo && i < hi) xr = x + static_cast<int64_t>(perm ? perm[i] : i) * ld_x;
    const uint16_t* A = A_ptrs[seg];
    f32x4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kb = kw0; kb < kw1; kb += WSTEP) {
      const int k = kb + kq * 8 * U;
      uint4 xv[U];
      uint4 av[NB][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k + 8 * u;
        xv[u] = (xr && kk < h_in) ? ld16(xr + kk) : zero4();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          av[nb][u] = (kk < h_in) ? ld16(A + static_cast<int64_t>(nb * 16 + mrow) * h_in + kk) : zero4();
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = E::mfma(xv[u], av[nb][u], acc[nb]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[w][nb][lane] = acc[nb];
    __syncthreads();
    if (threadIdx.x < 64 * NB) {
      const int nb = threadIdx.x >> 6, l = threadIdx.x & 63;
      const f32x4_t t = (red[0][nb][l] + red[1][nb][l]) + (red[2][nb][l] + red[3][nb][l]);
      const int jj = nb * 16 + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = r0 + 4 * (l >> 4) + e;
        if (row >= lo && row < hi) part[kc * slice + static_cast<int64_t>(row) * R + jj] = t[e];
      }
    }
    if (kc == 0)
      for (int q = lo + static_cast<int>(threadIdx.x); q < hi; q += 256) rowks[q] = ks;
    __syncthreads();
  }
}

// VALU expand over a tile of 16 sorted rows; lane owns CPL = 128/R columns as in
// expand_gemv_kernel; four waves cover consecutive column blocks.
template <int DT, int R>
__global__ __launch_bounds__(256) void expand_long_kernel(
    uint16_t* __restrict__ y, int64_t ld_y, const float* __restrict__ vsrc, int64_t slice,
    int32_t ks, const uint16_t* const* __restrict__ B_ptrs, const int32_t* __restrict__ seg_starts,
    int32_t S, const int32_t* __restrict__ perm, int32_t n, int32_t h_out, float scale) {
  using E = Elem<DT>;
  constexpr int CPL = 128 / R;
  constexpr int NV = 16;
  constexpr int YW = CPL / 2;
  __shared__ int s_count;
  __shared__ float vs[kTileRows][R];
  const int r0 = blockIdx.x * kTileRows;
  const int r1 = min(n, r0 + kTileRows);
  int seg = block_find_segment(seg_starts, S, r0, &s_count);
  const int c0 = (blockIdx.y * 256 + static_cast<int>(threadIdx.x)) * CPL;
  const bool cin = c0 < h_out;

  for (int idx = threadIdx.x; idx < (r1 - r0) * R; idx += 256) {
    const int i = idx / R, jj = idx % R;
    vs[i][jj] = sum_slices(vsrc + static_cast<int64_t>(r0 + i) * R + jj, slice, ks);
  }
  __syncthreads();
  if (!cin) return;

  for (int r = r0; r < r1; ++seg) {
    const int sb = seg_starts[seg], se = seg_starts[seg + 1];
    const int lo = r, hi = min(r1, se);
    r = hi;
    if (se - sb < kLongMin) continue;
    uint4 b[NV];
    const uint16_t* Bblk = B_ptrs[seg] + static_cast<int64_t>(c0) * R;
#pragma unroll
    for (int v = 0; v < NV; ++v) b[v] = ld16(Bblk + 8 * v);
    uint32_t yv[kTileRows][YW];
    uint16_t* yrow[kTileRows];
#pragma unroll
    for (int i = 0; i < kTileRows; ++i) {
      const int row = lo + i;
      yrow[i] = nullptr;
#pragma unroll
      for (int q = 0; q < YW; ++q) yv[i][q] = 0u;
      if (row < hi) {
        yrow[i] = y + static_cast<int64_t>(perm ? perm[row] : row) * ld_y + c0;
        load_words<YW>(yrow[i], yv[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kTileRows; ++i) {
      if (lo + i >= hi) continue;
      const int vi = lo + i - r0;
      float out[CPL];
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        float acc = 0.f;
#pragma unroll
        for (int jj = 0; jj < R; ++jj) {
          const int e = cc * R + jj;
          acc = fmaf(vs[vi][jj], elem<DT>(b[e >> 3], e & 7), acc);
        }
        const uint32_t w = yv[i][cc >> 1];
        const float yin = (cc & 1) ? E::hi(w) : E::lo(w);
        out[cc] = fmaf(scale, acc, yin);
      }
      uint32_t packed[YW];
#pragma unroll
      for (int q = 0; q < YW; ++q) packed[q] = E::pack(out[2 * q], out[2 * q + 1]);
      store_words<YW>(yrow[i], packed);
    }
  }
}

// v[i, :] = sum of the split-K slices of sorted row i, in slice order.
template <int R>
__global__ __launch_bounds__(256) void reduce_v_kernel(float* __restrict__ v,
                                                      const float* __restrict__ part, int64_t slice,
                                                      const int32_t* __restrict__ rowks, int32_t n,
                                                      int32_t ks_max) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(n) * R) return;
  const int row = static_cast<int>(idx / R);
  v[idx] = sum_slices(part + idx, slice, min(rowks[row], ks_max));
}

// ------------------------------------------------------------------------------------
// host side: sizes, validation, launches
// ------------------------------------------------------------------------------------
constexpr size_t kWsHeader = 32768;  // error flag and the decode path's counters

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline int gemv_kc(int r) {
  switch (r) {
    case 16: return GemvCfg<16>::KC;
    case 32: return GemvCfg<32>::KC;
    case 64: return GemvCfg<64>::KC;
  }
  return 0;
}

inline int mfma_wg_step(int r) { return 4 * 32 * (r == 64 ? 4 : 8); }

struct WsLayout {
  size_t rowks_off, part_off, total;
  int64_t slice;  // floats per split-K slice (n * r)
  int ks_max;
};

inline WsLayout ws_layout(int32_t n, int32_t h_in, int32_t r) {
  WsLayout L{};
  const int kc = gemv_kc(r);
  L.ks_max = (h_in + kc - 1) / kc;
  L.slice = static_cast<int64_t>(n) * r;
  L.rowks_off = kWsHeader;
  L.part_off = align_up(L.rowks_off + sizeof(int32_t) * static_cast<size_t>(n), 256);
  L.total = L.part_off + sizeof(float) * static_cast<size_t>(L.slice) * L.ks_max;
  return L;
}

// split-K chunk of the MFMA shrink: a multiple of the workgroup step, sized so that
// tiles x chunks gives roughly 2048 workgroups
inline int mfma_kcm(int32_t n, int32_t h_in, int32_t r) {
  const int step = mfma_wg_step(r);
  const int tiles = (n + kTileRows - 1) / kTileRows;
  const int steps_total = (h_in + step - 1) / step;
  int chunks = 2048 / (tiles > 0 ? tiles : 1);
  if (chunks < 1) chunks = 1;
  if (chunks > steps_total) chunks = steps_total;
  const int steps_per_chunk = (steps_total + chunks - 1) / chunks;
  return steps_per_chunk * step;
}

struct Tables {
  const uint16_t* const* ptrs;
  const int32_t* seg_starts;
  const int32_t* perm;
  int32_t n, S, min_len, max_len;
  bool use_gemv() const { return min_len < kLongMin; }
  bool use_long() const { return max_len >= kLongMin; }
};

template <int DT, int R>
hipError_t launch_shrink(hipStream_t st, const uint16_t* x, int64_t ld_x, const Tables& T,
                         int32_t h_in, const WsLayout& L, char* ws, int* ks_gemv, int* ks_long) {
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  int32_t* rowks = reinterpret_cast<int32_t*>(ws + L.rowks_off);
  *ks_gemv = *ks_long = 0;
  if (T.use_gemv()) {
    const int ks = (h_in + GemvCfg<R>::KC - 1) / GemvCfg<R>::KC;
    *ks_gemv = ks;
    hipLaunchKernelGGL((shrink_gemv_kernel<DT, R>), dim3(T.S, ks), dim3(256), 0, st, x, ld_x,
                       T.ptrs, T.seg_starts, T.perm, h_in, part, L.slice, rowks, ks);
  }
  if (T.use_long()) {
    const int kcm = mfma_kcm(T.n, h_in, R);
    const int ks = (h_in + kcm - 1) / kcm;
    *ks_long = ks;
    const int tiles = (T.n + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL((shrink_mfma_kernel<DT, R>), dim3(tiles, ks), dim3(256), 0, st, x, ld_x,
                       T.ptrs, T.seg_starts, T.S, T.perm, T.n, h_in, kcm, part, L.slice, rowks, ks);
  }
  return hipGetLastError();
}

template <int DT, int R>
hipError_t launch_expand(hipStream_t st, uint16_t* y, int64_t ld_y, const float* vsrc,
                         int64_t slice, int ks_gemv, int ks_long, const Tables& T, int32_t h_out,
                         float scale) {
  constexpr int CPL = 128 / R;
  if (T.use_gemv()) {
    const int chunks = (h_out + 64 * CPL - 1) / (64 * CPL);
    hipLaunchKernelGGL((expand_gemv_kernel<DT, R>), dim3(T.S, chunks), dim3(64), 0, st, y, ld_y,
                       vsrc, slice, ks_gemv, T.ptrs, T.seg_starts, T.perm, h_out, scale);
  }
  if (T.use_long()) {
    const int tiles = (T.n + kTileRows - 1) / kTileRows;
    const int chunks = (h_out + 256 * CPL - 1) / (256 * CPL);
    hipLaunchKernelGGL((expand_long_kernel<DT, R>), dim3(tiles, chunks), dim3(256), 0, st, y,
                       ld_y, vsrc, slice, ks_long, T.ptrs, T.seg_starts, T.S, T.perm, T.n, h_out,
                       scale);
  }
  return hipGetLastError();
}

template <int DT, int R>
hipError_t run_shrink(hipStream_t st, float* v, const uint16_t* x, int64_t ld_x, const Tables& T,
                      int32_t h_in, const WsLayout& L, char* ws) {
  int ksg, ksl;
  hipError_t e = launch_shrink<DT, R>(st, x, ld_x, T, h_in, L, ws, &ksg, &ksl);
  if (e != hipSuccess) return e;
  const int64_t total = static_cast<int64_t>(T.n) * R;
  hipLaunchKernelGGL((reduce_v_kernel<R>), dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                     0, st, v, reinterpret_cast<const float*>(ws + L.part_off), L.slice,
                     reinterpret_cast<const int32_t*>(ws + L.rowks_off), T.n, L.ks_max);
  return hipGetLastError();
}

template <int DT, int R>
hipError_t run_lora_add(hipStream_t st, uint16_t* y, int64_t ld_y, const uint16_t* x, int64_t ld_x,
                        const Tables& TA, const Tables& TB, int32_t h_in, int32_t h_out, float scale,
                        const WsLayout& L, char* ws) {
  int ksg, ksl;
  hipError_t e = launch_shrink<DT, R>(st, x, ld_x, TA, h_in, L, ws, &ksg, &ksl);
  if (e != hipSuccess) return e;
  return launch_expand<DT, R>(st, y, ld_y, reinterpret_cast<const float*>(ws + L.part_off), L.slice,
                              ksg, ksl, TB, h_out, scale);
}

template <template <int, int> class F, typename... Args>
hipError_t dispatch(int32_t dtype, int32_t r, Args&&... args) {
  if (dtype == SGMV_F16) {
    if (r == 16) return F<SGMV_F16, 16>::run(args...);
    if (r == 32) return F<SGMV_F16, 32>::run(args...);
    return F<SGMV_F16, 64>::run(args...);
  }
  if (r == 16) return F<SGMV_BF16, 16>::run(args...);
  if (r == 32) return F<SGMV_BF16, 32>::run(args...);
  return F<SGMV_BF16, 64>::run(args...);
}

template <int DT, int R>
struct ShrinkOp {
  template <typename... A>
  static hipError_t run(A... a) { return run_shrink<DT, R>(a...); }
};
template <int DT, int R>
struct ExpandOp {
  template <typename... A>
  static hipError_t run(A... a) { return launch_expand<DT, R>(a...); }
};
template <int DT, int R>
struct LoraOp {
  template <typename... A>
  static hipError_t run(A... a) { return run_lora_add<DT, R>(a...); }
};


}  // namespace

extern "C" size_t sgmv_pool_workspace_bytes_internal(int32_t n, int32_t h_in, int32_t r);

extern "C" size_t sgmv_workspace_bytes(int32_t n, int32_t h_in, int32_t r) {
  if (n < 0 || h_in < 8 || h_in > kMaxDim || !rank_ok(r)) return 0;
  const size_t a = ws_layout(n, h_in, r).total;
  // the one-launch decode path takes at most 64 rows
  const size_t b = n <= 64 ? sgmv_pool_workspace_bytes_internal(n, h_in, r) : 0;
  return a > b ? a : b;
}

extern "C" int sgmv_shrink(hipStream_t stream, int32_t dtype, float* v, const void* x, int64_t ld_x,
                           const void* const* A_ptrs, const int32_t* seg_starts,
                           const int32_t* perm, int32_t n, int32_t n_segments, int32_t min_seg_len,
                           int32_t max_seg_len, int32_t h_in, int32_t r, void* workspace,
                           size_t workspace_bytes) {
  if (dtype != SGMV_F16 && dtype != SGMV_BF16) return SGMV_ERR_UNSUPPORTED;
  if (!rank_ok(r)) return SGMV_ERR_UNSUPPORTED;
  int st = check_segments(n, n_segments, min_seg_len, max_seg_len);
  if (st) return st;
  if ((st = check_dim(h_in, ld_x))) return st;
  if (n == 0) return SGMV_OK;
  if (!v || !x || !A_ptrs || !seg_starts) return SGMV_ERR_NULL;
  if (!aligned16(x) || !aligned16(v)) return SGMV_ERR_ALIGNMENT;
  if (ranges_overlap(v, sizeof(float) * static_cast<size_t>(n) * r, x, matrix_bytes(n, ld_x, h_in)))
    return SGMV_ERR_ALIAS;
  const WsLayout L = ws_layout(n, h_in, r);
  if (!workspace || workspace_bytes < L.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SGMV_ERR_WORKSPACE;
  if ((st = check_device())) return st;
  const Tables T{reinterpret_cast<const uint16_t* const*>(A_ptrs), seg_starts, perm, n,
                 n_segments, min_seg_len, max_seg_len};
  return hip_status(dispatch<ShrinkOp>(dtype, r, stream, v, static_cast<const uint16_t*>(x), ld_x,
                                       T, h_in, L, static_cast<char*>(workspace)));
}

extern "C" int sgmv_expand(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y, const float* v,
                           const void* const* B_ptrs, const int32_t* seg_starts,
                           const int32_t* perm, int32_t n, int32_t n_segments, int32_t min_seg_len,
                           int32_t max_seg_len, int32_t r, int32_t h_out, float scale) {
  if (dtype != SGMV_F16 && dtype != SGMV_BF16) return SGMV_ERR_UNSUPPORTED;
  if (!rank_ok(r)) return SGMV_ERR_UNSUPPORTED;
  int st = check_segments(n, n_segments, min_seg_len, max_seg_len);
  if (st) return st;
  if ((st = check_dim(h_out, ld_y))) return st;
  if (n == 0) return SGMV_OK;
  if (!y || !v || !B_ptrs || !seg_starts) return SGMV_ERR_NULL;
  if (!aligned16(y) || !aligned16(v)) return SGMV_ERR_ALIGNMENT;
  if (ranges_overlap(v, sizeof(float) * static_cast<size_t>(n) * r, y, matrix_bytes(n, ld_y, h_out)))
    return SGMV_ERR_ALIAS;
  if ((st = check_device())) return st;
  const Tables T{reinterpret_cast<const uint16_t* const*>(B_ptrs), seg_starts, perm, n,
                 n_segments, min_seg_len, max_seg_len};
  return hip_status(dispatch<ExpandOp>(dtype, r, stream, static_cast<uint16_t*>(y), ld_y, v,
                                       static_cast<int64_t>(0), 1, 1, T, h_out, scale));
}

extern "C" int sgmv_lora_add(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y,
                             const void* x, int64_t ld_x, const void* const* A_ptrs,
                             const void* const* B_ptrs, const int32_t* seg_starts,
                             const int32_t* perm, int32_t n, int32_t n_segments,
                             int32_t min_seg_len, int32_t max_seg_len, int32_t h_in, int32_t h_out,
                             int32_t r, float scale, void* workspace, size_t workspace_bytes) {
  if (dtype != SGMV_F16 && dtype != SGMV_BF16) return SGMV_ERR_UNSUPPORTED;
  if (!rank_ok(r)) return SGMV_ERR_UNSUPPORTED;
  int st = check_segments(n, n_segments, min_seg_len, max_seg_len);
  if (st) return st;
  if ((st = check_dim(h_in, ld_x))) return st;
  if ((st = check_dim(h_out, ld_y))) return st;
  if (n == 0) return SGMV_OK;
  if (!y || !x || !A_ptrs || !B_ptrs || !seg_starts) return SGMV_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return SGMV_ERR_ALIGNMENT;
  if (ranges_overlap(x, matrix_bytes(n, ld_x, h_in), y, matrix_bytes(n, ld_y, h_out)))
    return SGMV_ERR_ALIAS;
  const WsLayout L = ws_layout(n, h_in, r);
  if (!workspace || workspace_bytes < L.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SGMV_ERR_WORKSPACE;
  if ((st = check_device())) return st;
  const Tables TA{reinterpret_cast<const uint16_t* const*>(A_ptrs), seg_starts, perm, n,
                  n_segments, min_seg_len, max_seg_len};
  const Tables TB{reinterpret_cast<const uint16_t* const*>(B_ptrs), seg_starts, perm, n,
                  n_segments, min_seg_len, max_seg_len};
  return hip_status(dispatch<LoraOp>(dtype, r, stream, static_cast<uint16_t*>(y), ld_y,
                                     static_cast<const uint16_t*>(x), ld_x, TA, TB, h_in, h_out,
                                     scale, L, static_cast<char*>(workspace)));
}
