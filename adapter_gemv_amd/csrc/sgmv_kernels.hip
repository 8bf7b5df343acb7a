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
// tiles of sorted rows.  v = x @ A is kept in float32: the shrink kernels write
// split-K partial sums to the workspace and the expand kernels add the slices in a
// fixed order, so results are reproducible run to run (no float atomics).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <initializer_list>
#include <mutex>
#include <type_traits>
#include <vector>

#include "../../include/sgmv.h"
#include "sgmv_checks.h"
#include "sgmv_device.h"

namespace {

using namespace sgmv_dev;
using namespace sgmv_host;

constexpr int kShortMax = kLongMin - 1;
// rows of short segments mark their slice count with this bit, so that the slices of short
// and of long rows can be summed by separate reduce_v_kernel launches
constexpr int32_t kShortRowFlag = 1 << 30;
enum ReduceRows : int32_t { kReduceAll = 0, kReduceShort = 1, kReduceLong = 2 };

// ------------------------------------------------------------------------------------
// GEMV path (segments with 1 .. kShortMax rows)
// ------------------------------------------------------------------------------------
// A wave covers WAVE_K values of k in 64-k segments.  Lane (t0 = lane / 8, c = lane % 8)
// reads 16 bytes (k values 8c .. 8c + 7 of a segment) of rows t0, t0 + 8, t0 + 16, ... of
// A[a]: one load instruction covers 8 rows × 128 contiguous bytes, whole cache lines.
// The same 16 bytes of a token row's x serve all of the lane's A rows.  The 8 lanes of a
// row add their partial sums by shuffles; four waves cover consecutive k ranges and are
// summed through LDS.
template <int R>
struct GemvCfg {
  static constexpr int WAVE_K = (R == 16) ? 128 : 64;  // k values per wave
  static constexpr int KC = 4 * WAVE_K;                // k values per workgroup (split-K chunk)
  static constexpr int SEG = WAVE_K / 64;              // 64-k segments per wave
  static constexpr int RT = R / 8;                     // A rows per lane
  static constexpr int MR = 4;                         // token rows loaded per pass
};

//
// Every row's slice count in rowks is written for the current call by whichever shrink
// sees the row first: this kernel writes it for the rows of every segment (rk_long for
// rows of long segments), the long-segment shrinks for every row of their tiles
// (rk_short for rows outside long segments).  Both write the same value for a row, so the
// reduce pass of either chain, which runs after its own shrink, never reads a count left
// by an earlier call in which the row's segment was of the other kind.  bad_flag is set
// when the long-segment kernels are not launched (the caller's max_seg_len was below
// kLongMin) and a long segment is met anyway: its rows are not computed.
template <int DT, int R>
__global__ __launch_bounds__(256) void shrink_gemv_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* const* __restrict__ A_ptrs,
    const int32_t* __restrict__ seg_starts, const int32_t* __restrict__ perm, int32_t h_in,
    float* __restrict__ part, int64_t slice, int32_t* __restrict__ rowks, int32_t ks,
    int32_t rk_long, int32_t* __restrict__ bad_flag, const int32_t* __restrict__ meta) {
  using C = GemvCfg<R>;
  __shared__ float red[4][kShortMax][R];
  // items (segment s, chunk kc) = (i % S, i / S): one per workgroup of a (S, ks) grid with
  // host tables; strided over a 1-D grid when the segment count comes from the device
  // tables' meta word
  const int S = meta ? meta[0] : static_cast<int>(gridDim.x);
  if (meta && meta[1] >= kLongMin) return;  // no short segment at all
  const int items = S * ks;
  for (int item = blockIdx.x + gridDim.x * blockIdx.y; item < items; item += gridDim.x * gridDim.y) {
  const int s = item % S, kc = item / S;
  const int seg0 = seg_starts[s];
  const int m = seg_starts[s + 1] - seg0;
  if (m >= kLongMin) {  // uniform: a long segment, computed by the MFMA kernels
    if (kc == 0) {
      for (int i = threadIdx.x; i < m; i += 256) rowks[seg0 + i] = rk_long;
      if (bad_flag && threadIdx.x == 0) raise_flag(bad_flag, kFlagSegBounds);
    }
    continue;
  }
  if (m <= 0) continue;  // uniform
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t0 = lane >> 3, c = lane & 7;
  const int kbase = kc * C::KC + w * C::WAVE_K + 8 * c;

  const gptr<const uint16_t> Ab = global_ptr(A_ptrs[s]) + static_cast<int64_t>(t0) * h_in;
  uint4 a[C::SEG][C::RT];
#pragma unroll
  for (int sk = 0; sk < C::SEG; ++sk) {
    const int k = kbase + 64 * sk;
#pragma unroll
    for (int t = 0; t < C::RT; ++t)
      a[sk][t] = (k < h_in) ? ld16(Ab + static_cast<int64_t>(8 * t) * h_in + k) : zero4();
  }
  for (int i0 = 0; i0 < m; i0 += C::MR) {
    uint4 xv[C::MR][C::SEG];
#pragma unroll
    for (int r = 0; r < C::MR; ++r) {
      const int i = i0 + r;
      gptr<const uint16_t> xr = nullptr;
      if (i < m) xr = global_ptr(x) + static_cast<int64_t>(perm ? perm[seg0 + i] : seg0 + i) * ld_x;
#pragma unroll
      for (int sk = 0; sk < C::SEG; ++sk) {
        const int k = kbase + 64 * sk;
        xv[r][sk] = (xr && k < h_in) ? ld16(xr + k) : zero4();
      }
    }
#pragma unroll
    for (int r = 0; r < C::MR; ++r) {
      float acc[C::RT];
#pragma unroll
      for (int t = 0; t < C::RT; ++t) {
        acc[t] = 0.f;
#pragma unroll
        for (int sk = 0; sk < C::SEG; ++sk) acc[t] = dot8<DT>(xv[r][sk], a[sk][t], acc[t]);
        // the 8 lanes of row 8t + t0, in a fixed butterfly
#pragma unroll
        for (int msk = 1; msk < 8; msk <<= 1) acc[t] += __shfl_xor(acc[t], msk);
      }
      // lane (t0, c) stores row 8c + t0 (every lane of the row holds its sum)
      if (i0 + r < m && c < C::RT) {
        float mine = acc[0];
#pragma unroll
        for (int t = 1; t < C::RT; ++t) mine = (c == t) ? acc[t] : mine;
        red[w][i0 + r][8 * c + t0] = mine;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < m * R; idx += 256) {
    const int i = idx / R, jj = idx % R;
    const float sum = (red[0][i][jj] + red[1][i][jj]) + (red[2][i][jj] + red[3][i][jj]);
    part[kc * slice + static_cast<int64_t>(seg0 + i) * R + jj] = sum;
  }
  if (kc == 0)
    for (int i = threadIdx.x; i < m; i += 256) rowks[seg0 + i] = ks | kShortRowFlag;
  __syncthreads();  // red is reused by the next segment
  }
}

// Lane owns CPL = 128/R consecutive output columns: its block of B (CPL rows of the
// stored [h_out, r] array) is 256 contiguous bytes, and its slice of y is 256/R bytes.
template <int DT, int R>
__global__ __launch_bounds__(64) void expand_gemv_kernel(
    uint16_t* __restrict__ y, int64_t ld_y, const float* __restrict__ vsrc, int64_t slice,
    int32_t ks, const uint16_t* const* __restrict__ B_ptrs, const int32_t* __restrict__ seg_starts,
    const int32_t* __restrict__ perm, int32_t h_out, float scale, int32_t chunks,
    const int32_t* __restrict__ meta) {
  using E = Elem<DT>;
  constexpr int CPL = 128 / R;
  constexpr int NV = 16;  // CPL * R / 8
  constexpr int YW = CPL / 2;  // 32-bit words of y per lane and row
  __shared__ float vs[kShortMax][R];
  // items (segment s, column chunk ch) = (i % S, i / S), as in shrink_gemv_kernel
  const int S = meta ? meta[0] : static_cast<int>(gridDim.x);
  if (meta && meta[1] >= kLongMin) return;  // no short segment at all
  const int items = S * chunks;
  for (int item = blockIdx.x + gridDim.x * blockIdx.y; item < items; item += gridDim.x * gridDim.y) {
  const int s = item % S, ch = item / S;
  const int seg0 = seg_starts[s];
  const int m = seg_starts[s + 1] - seg0;
  if (m <= 0 || m >= kLongMin) continue;  // uniform
  const int lane = threadIdx.x;
  const int c0 = (ch * 64 + lane) * CPL;
  const bool cin = c0 < h_out;

  uint4 b[NV];
  const gptr<const uint16_t> Bblk = global_ptr(B_ptrs[s]) + static_cast<int64_t>(c0) * R;
#pragma unroll
  for (int v = 0; v < NV; ++v) b[v] = cin ? ld16(Bblk + 8 * v) : zero4();

  uint32_t yv[kShortMax][YW];
  gptr<uint16_t> yrow[kShortMax];
#pragma unroll
  for (int i = 0; i < kShortMax; ++i) {
    yrow[i] = nullptr;
    if (i < m) yrow[i] = global_ptr(y) + static_cast<int64_t>(perm ? perm[seg0 + i] : seg0 + i) * ld_y + c0;
#pragma unroll
    for (int q = 0; q < YW; ++q) yv[i][q] = 0u;
    if (i < m && cin) load_words<YW>(yrow[i], yv[i]);
  }

  for (int idx = lane; idx < m * R; idx += 64) {
    const int i = idx / R, jj = idx % R;
    vs[i][jj] = sum_slices(vsrc + static_cast<int64_t>(seg0 + i) * R + jj, slice, ks);
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < kShortMax; ++i) {
    if (i >= m || !cin) continue;
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
  __syncthreads();  // vs is reused by the next segment
  }
}

// ------------------------------------------------------------------------------------
// long-segment path (segments with >= kLongMin rows)
// ------------------------------------------------------------------------------------
// Long segments overlapping the sorted rows [g0, g1) of a tile (at most ROWS rows), found
// in one parallel pass over seg_starts that also reads each segment's weight pointer (so
// that the pointer needs no load of its own once the segment is known): sh.seg[k],
// sh.ptr[k] for the tile's long segments k, and sh.rseg[q] = k for row g0 + q if its
// segment has at least kLongMin rows, else -1.  Returns the number of such segments
// (uniform).  A tile of ROWS rows meets at most ROWS / kLongMin + 2 long segments.
template <int ROWS>
struct TileSegs {
  static constexpr int kMax = ROWS / kLongMin + 2;
  int nseg;
  int seg[kMax], st[kMax], en[kMax];
  const uint16_t* ptr[kMax];
  int rseg[ROWS];
};

// Segment s = threadIdx.x's bounds and weight pointer, read ahead of the scan so that they
// share a round of loads with the caller rows (sh.nseg must be cleared before the caller's
// barrier; see tile_long_segments_pre).
struct SegPre {
  int st, en;
  const uint16_t* ptr;
};

__device__ inline SegPre seg_preload(const int32_t* __restrict__ seg_starts,
                                     const uint16_t* const* __restrict__ ptrs, int S) {
  SegPre p{0, 0, nullptr};
  const int s = threadIdx.x;
  if (s < S) {
    p.st = seg_starts[s];
    p.en = seg_starts[s + 1];
    p.ptr = ptrs[s];
  }
  return p;
}

template <int ROWS, int THREADS, bool PRE>
__device__ inline int tile_segments_impl(const int32_t* __restrict__ seg_starts,
                                         const uint16_t* const* __restrict__ ptrs, int S, int g0,
                                         int g1, TileSegs<ROWS>& sh, const SegPre& pre) {
  const int tid = threadIdx.x;
  if constexpr (!PRE) {
    if (tid == 0) sh.nseg = 0;
    __syncthreads();
  }
  for (int s = tid; s < S; s += THREADS) {
    int st, en;
    const uint16_t* pp;
    if (PRE && s == tid) {
      st = pre.st;
      en = pre.en;
      pp = pre.ptr;
    } else {
      st = seg_starts[s];
      en = seg_starts[s + 1];
      pp = ptrs[s];
    }
    if (en - st >= kLongMin && st < g1 && en > g0) {
      const int k = atomicAdd(&sh.nseg, 1);
      if (k < TileSegs<ROWS>::kMax) {
        sh.seg[k] = s;
        sh.st[k] = st;
        sh.en[k] = en;
        sh.ptr[k] = pp;
      }
    }
  }
  __syncthreads();
  const int nseg = min(sh.nseg, TileSegs<ROWS>::kMax);
  for (int q = tid; q < ROWS; q += THREADS) {
    const int row = g0 + q;
    int slot = -1;
    for (int k = 0; k < nseg; ++k)
      if (sh.st[k] <= row && row < sh.en[k]) slot = k;
    sh.rseg[q] = slot;
  }
  __syncthreads();
  return nseg;
}

template <int ROWS, int THREADS>
__device__ inline int tile_long_segments(const int32_t* __restrict__ seg_starts,
                                         const uint16_t* const* __restrict__ ptrs, int S, int g0,
                                         int g1, TileSegs<ROWS>& sh) {
  return tile_segments_impl<ROWS, THREADS, false>(seg_starts, ptrs, S, g0, g1, sh, SegPre{});
}

// As tile_long_segments, with segment threadIdx.x already read by seg_preload and sh.nseg
// cleared before a barrier that all threads have passed.
template <int ROWS, int THREADS>
__device__ inline int tile_long_segments_pre(const int32_t* __restrict__ seg_starts,
                                             const uint16_t* const* __restrict__ ptrs, int S,
                                             int g0, int g1, TileSegs<ROWS>& sh,
                                             const SegPre& pre) {
  return tile_segments_impl<ROWS, THREADS, true>(seg_starts, ptrs, S, g0, g1, sh, pre);
}

// Slice counts of a tile's rows for the current call (written by the tile's first K
// chunk): rows of long segments get their final v from this kernel (ks == 1, count 0) or
// ks slices; every other row is a short-segment row, whose count rk_short the GEMV shrink
// writes too.  bad_flag (non-null when the GEMV kernels are not launched, the caller's
// min_seg_len being at least kLongMin) is set if the tile meets such a row: it is not
// computed.
template <int ROWS>
__device__ inline void mark_tile_rows(const TileSegs<ROWS>& sh, int r0, int r1, int ks,
                                      int32_t rk_short, int32_t* __restrict__ rowks,
                                      int32_t* __restrict__ bad_flag) {
  bool short_row = false;
  for (int qr = threadIdx.x; qr < r1 - r0; qr += blockDim.x) {
    const bool lng = sh.rseg[qr] >= 0;
    rowks[r0 + qr] = lng ? (ks == 1 ? 0 : ks) : rk_short;
    short_row = short_row || !lng;
  }
  if (bad_flag && short_row) raise_flag(bad_flag, kFlagSegBounds);
}

// Next long run of a tile at or after row q (rows are in segment order): its slot k in
// TileSegs, or -1 when there is none; leaves q after the run's last row in the tile.
template <int ROWS>
__device__ inline int next_run(const TileSegs<ROWS>& sh, int& q) {
  while (q < ROWS && sh.rseg[q] < 0) ++q;
  if (q >= ROWS) return -1;
  const int k = sh.rseg[q];
  while (q < ROWS && sh.rseg[q] == k) ++q;
  return k;
}

// Shrink on MFMA 16x16x32 for a tile of r sorted rows and one K chunk (r = 16 and 32).
// The x rows are the A operand and the adapter's stored A rows the B operand; lane l
// supplies row (or column) l%16 and k = k0 + 8*(l/16) .. +7 of each 32-wide k step.  Each
// of the 4 waves covers all r rows and r columns (r/16 x r/16 accumulator blocks), so A
// and x are read in equal amounts; the waves take interleaved stages of UN k steps, with
// the loads of the next stage in flight while the current one is multiplied, and are
// summed through LDS in a fixed order.  Rows of several long segments in one tile are handled run by run with the
// other rows' x set to zero.  With one chunk per tile v is written directly; otherwise
// each chunk writes its slice of partial sums and reduce_v_kernel, the next launch, adds
// the slices in order (no wait on other workgroups inside this kernel).
//
// With a multiple of 8 chunks, workgroup b (on XCD b % 8) takes chunks = b mod 8, so each
// XCD's L2 keeps one eighth of the K range of the adapters' A.
constexpr int kXcds = 8;

template <int R>
struct ShrCfg {
  static_assert(R == 16 || R == 32, "r = 64 takes shrink_lds_kernel");
  static constexpr int NB = R / 16;                 // column blocks of v
  static constexpr int RB = R / 16;                 // row blocks
  static constexpr int MT = 16 * RB;                // rows per tile
  static constexpr int UN = (R == 16) ? 2 : 1;      // k steps per stage
  static constexpr int STAGE = 32 * UN;             // k per stage
  static constexpr int WAVES_PER_SIMD = 3;
  static constexpr int TARGET_WGS = (R == 16) ? 256 : 384;
};

// The LDS-staged shrink (shrink_lds_kernel, 64-row tiles) takes r = 64, and r = 16 when
// the rows of x are long (h_in > 16384), or longer than 6144 in a call that also has short
// segments (host tables, and not a rank group of a mixed-rank call, whose groups' shrinks
// run side by side: there the taller tiles measured slower, ranks 16 + 64 gate/up 110 ->
// 116 us).  Its split-K slices then need a reduce pass, which a call with short segments
// runs anyway.  Measured on MI355X for the 70B batch: r = 64 gate/up shrink
// 27.6 -> 21.0 us, down 57.6 -> 49.3 us, r = 16 down 41.6 -> 35.6 us; r = 16 calls with
// h_in = 8192: q/o 51.1 -> 47.6 us, k/v 40.1 -> 37.1, gate/up 92.9 -> 89.0.  For the 13B
// prefill batch (long segments only) the extra reduce pass makes it slower than the
// 16-row tiles of shrink_mfma_kernel (down projection, h_in = 13824: 41.6 vs 37.5 us).
inline bool shrink_lds_long_rows(int32_t h_in, bool has_short) {
  return h_in > 16384 || (has_short && h_in > 6144);
}
template <int R> constexpr int kLdsD = 3;  // stage buffers (four at r = 64: 4-9 % slower)
constexpr int kLdsMT = 64;                                  // rows per tile
constexpr int kLdsWgs = 512;  // workgroups resident at once (two per CU, for their LDS)
// Loads of one stage.  They are unconditional (out-of-range k reads offset 0 of the same
// row, rows outside the current run read a row that exists) so that the compiler can count
// them exactly and keep the next stage in flight; shr_mul zeroes what does not belong.
template <int DT, class C>
__device__ inline void shr_load(const gptr<const uint16_t> (&xr)[C::RB],
                                const gptr<const uint16_t> (&ar)[C::NB], int k0, int k_hi, int kq,
                                uint4 (&xv)[C::UN][C::RB], uint4 (&av)[C::UN][C::NB]) {
#pragma unroll
  for (int u = 0; u < C::UN; ++u) {
    const int kk = k0 + 32 * u + 8 * kq;
    const int off = (kk < k_hi) ? kk : 0;
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) xv[u][rb] = ld16(xr[rb] + off);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) av[u][nb] = ld16(ar[nb] + off);
  }
}

template <int DT, class C>
__device__ inline void shr_mul(const uint4 (&xv)[C::UN][C::RB], const uint4 (&av)[C::UN][C::NB],
                               int k0, int k_hi, int kq, const bool (&xin)[C::RB],
                               f32x4_t (&acc)[C::RB][C::NB]) {
#pragma unroll
  for (int u = 0; u < C::UN; ++u) {
    const bool in = k0 + 32 * u + 8 * kq < k_hi;
    uint4 a[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) a[nb] = in ? av[u][nb] : zero4();
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      const uint4 xa = (in && xin[rb]) ? xv[u][rb] : zero4();
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) acc[rb][nb] = Elem<DT>::mfma(xa, a[nb], acc[rb][nb]);
    }
  }
}

template <int DT, int R>
__global__ __launch_bounds__(256, ShrCfg<R>::WAVES_PER_SIMD) void shrink_mfma_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* const* __restrict__ A_ptrs,
    const int32_t* __restrict__ seg_starts, int32_t S_host, const int32_t* __restrict__ perm,
    int32_t n, int32_t h_in, int32_t kcm, int32_t ks, float* __restrict__ part, int64_t slice,
    float* __restrict__ v_out, int32_t* __restrict__ rowks, int32_t rk_short,
    int32_t* __restrict__ bad_flag, const int32_t* __restrict__ meta) {
  const int S = meta ? meta[0] : S_host;
  if (meta && meta[2] < kLongMin) return;  // no long segment at all
  using C = ShrCfg<R>;
  constexpr int NB = C::NB, RB = C::RB, UN = C::UN, STAGE = C::STAGE, MT = C::MT;
  __shared__ TileSegs<MT> sh;
  __shared__ int s_prow[MT];
  __shared__ f32x4_t red[2][RB][NB][64];

  const int b = blockIdx.x;
  int tile, kc;
  if (ks % kXcds == 0) {
    const int m = ks / kXcds, j = b / kXcds;
    tile = j / m;
    kc = b % kXcds + kXcds * (j % m);
  } else {
    tile = b / ks;
    kc = b % ks;
  }
  const int r0 = tile * MT;
  const int r1 = min(n, r0 + MT);
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int mrow = lane & 15, kq = lane >> 4;
  // one round of loads for the caller rows, the segment bounds and the A pointers
  const SegPre pre = seg_preload(seg_starts, A_ptrs, S);
  if (tid < MT) s_prow[tid] = (r0 + tid < r1) ? (perm ? perm[r0 + tid] : r0 + tid) : 0;
  if (tid == 0) sh.nseg = 0;
  __syncthreads();
  const int nseg = tile_long_segments_pre<MT, 256>(seg_starts, A_ptrs, S, r0, r1, sh, pre);
  if (kc == 0) mark_tile_rows(sh, r0, r1, ks, rk_short, rowks, bad_flag);
  if (nseg == 0) return;  // uniform
  const int k_lo = kc * kcm;
  const int k_hi = min(h_in, k_lo + kcm);
  const int nst = (k_hi - k_lo + STAGE - 1) / STAGE;

  f32x4_t acc[RB][NB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int q = 0;
  for (int sg; (sg = next_run(sh, q)) >= 0;) {
    // rows outside the run read row r0 of the tile (it exists) and are zeroed in shr_mul
    gptr<const uint16_t> xr[RB];
    bool xin[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      xin[rb] = sh.rseg[16 * rb + mrow] == sg;
      xr[rb] = global_ptr(x) + static_cast<int64_t>(s_prow[xin[rb] ? 16 * rb + mrow : 0]) * ld_x;
    }
    const gptr<const uint16_t> A = global_ptr(sh.ptr[sg]);
    gptr<const uint16_t> ar[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ar[nb] = A + static_cast<int64_t>(nb * 16 + mrow) * h_in;
    uint4 x0[UN][RB], a0[UN][NB], x1[UN][RB], a1[UN][NB];
    int k0 = k_lo + w * STAGE;
    shr_load<DT, C>(xr, ar, k0, k_hi, kq, x0, a0);
    for (int g = w; g < nst; g += 8) {
      shr_load<DT, C>(xr, ar, k0 + 4 * STAGE, k_hi, kq, x1, a1);
      shr_mul<DT, C>(x0, a0, k0, k_hi, kq, xin, acc);
      shr_load<DT, C>(xr, ar, k0 + 8 * STAGE, k_hi, kq, x0, a0);
      shr_mul<DT, C>(x1, a1, k0 + 4 * STAGE, k_hi, kq, xin, acc);
      k0 += 8 * STAGE;
    }
  }
  // fixed-order sum over the waves: (w0 + w2) + (w1 + w3)
  if (w >= 2) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[w - 2][rb][nb][lane] = acc[rb][nb];
  }
  __syncthreads();
  if (w < 2) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[w][rb][nb][lane] = acc[rb][nb] + red[w][rb][nb][lane];
  }
  __syncthreads();
  // entry e = (rb, nb, l): rows r0 + 16rb + 4(l/16) + c, column nb*16 + l%16
  for (int e = tid; e < RB * NB * 64; e += 256) {
    const int l = e & 63, nb = (e >> 6) % NB, rb = (e >> 6) / NB;
    const f32x4_t sum = red[0][rb][nb][l] + red[1][rb][nb][l];
    const int jj = nb * 16 + (l & 15);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qr = 16 * rb + 4 * (l >> 4) + c;
      if (sh.rseg[qr] < 0) continue;
      const int64_t o = static_cast<int64_t>(r0 + qr) * R + jj;
      if (ks == 1)
        v_out[o] = sum[c];
      else
        part[kc * slice + o] = sum[c];
    }
  }
}

// Shrink on MFMA with the operands staged in LDS by direct global-to-LDS loads.  Same
// product and outputs as shrink_mfma_kernel, organised to keep many bytes in flight at a
// small register cost: operands go straight from global memory into a ring of D stage
// buffers, so D - 1 stages are in flight while one is multiplied.  Tiles are 64 rows; the
// four waves split them (16 rows each, over the whole chunk) and share the stage's A
// blocks, so A is fetched once per tile and chunk for all 64 rows and no cross-wave sum is
// needed.  A stage covers STAGE values of k (128 at r = 16, 64 at r = 64), and every load
// instruction fills one block of RPB rows x STAGE k: 4 rows x 256 contiguous bytes at
// r = 16, 8 rows x 128 bytes at r = 64.  HBM serves such row runs about 1.5 times faster
// on MI355X than 16 rows x 64 bytes, the MFMA operand's own shape (a read-only probe of
// the 70B down projection's x: 117 MB in 28 instead of 35 us); the MFMA lanes read the
// blocks back through a slot map (run_slot).  A wave waits for its own loads of a stage
// (vmcnt) and its own LDS reads (lgkmcnt), then a barrier makes every wave's loads visible
// and tells each wave that all waves have finished reading the buffer it refills next.
// The stage buffers are separate LDS variables addressed with compile-time indices, so
// that the compiler can tell which loads a read depends on.
template <int R, int MT_, int D_>
struct ShrLdsCfg {
  static_assert(R == 16 || R == 64, "ranks of the LDS-staged shrink");
  static constexpr int NB = R / 16;                  // column blocks of v
  static constexpr int MT = MT_;                     // rows per tile
  static constexpr int STAGE = R == 16 ? 128 : 64;   // k per stage
  static constexpr int UN = STAGE / 32;              // MFMA k steps per stage
  static constexpr int PPR = STAGE / 8;              // 16-byte pieces per row and stage
  static constexpr int RPB = 64 / PPR;               // rows per block (one load instruction)
  static constexpr int XB = 16 / RPB;                // x blocks per wave and stage
  static constexpr int AB = R / RPB / 4;             // A blocks per wave and stage
  static constexpr int LPS = XB + AB;                // loads per wave and stage
  static constexpr int PAD = 16 / XB;                // pad slots after each block
  static constexpr int SLOTS = 64 + PAD;             // 16-byte slots per block
  static constexpr int D = D_;                       // stage buffers
  static_assert(MT == 64, "64-row tiles");
  static_assert(D >= 3 && D <= 8 && (D - 2) * LPS < 64, "ring depth");
};
template <class C>
struct ShrStage {
  uint4 a[4 * C::AB][C::SLOTS];  // block b: A rows RPB * b .. RPB * b + RPB - 1
  uint4 x[4][C::XB * C::SLOTS];  // wave w's block i (tile rows 16w + RPB * i ..) at [w][i * SLOTS]
};

// Block layout: row j (0 .. RPB - 1) of a block, 16-byte piece p (k = 8p .. 8p + 7 of the
// stage; 0 .. PPR - 1) sits in slot PPR * j + (p + j) mod PPR, and the lane that loads it
// is the slot itself.  The MFMA lanes reading one k step (16 rows, one piece each, from
// 16 / RPB consecutive blocks) then meet no bank conflict whether the LDS serves 16 lanes
// over 64 banks or 8 lanes over 32 banks at a time: the rotation by j separates the rows
// of a block, and the PAD slots after each block (16 / XB) separate the blocks.
template <int PPR>
__device__ inline int run_slot(int j, int p) { return PPR * j + ((p + j) & (PPR - 1)); }
template <int PPR>
__device__ inline int run_piece(int slot) { return ((slot & (PPR - 1)) - slot / PPR) & (PPR - 1); }

// wait until at most N vector-memory loads of this wave are in flight (gfx9 s_waitcnt:
// vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// 16 bytes per lane from src into LDS at dst + 16 * lane (dst is the same for the wave)
__device__ inline void load_to_lds(gptr<const uint16_t> src, uint4* dst) {
  __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)dst, 16, 0, 0);
}

// workgroup barrier that does not wait for the global loads in flight: it waits only for
// this wave's LDS reads (lgkmcnt 0), so that a wave past the barrier may refill a stage
// buffer that every wave has finished reading, not merely issued its reads of; the signal
// fences keep the compiler from moving LDS accesses across it
__device__ inline void barrier_no_fence() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int I, int N, class F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// above this h_in the LDS-staged shrink assigns (chunk, tile) pairs to XCDs chunk-major
constexpr int kChunkMajorMinK = 16384;

template <int DT, int R, int MT, int D>
__global__ __launch_bounds__(256) void shrink_lds_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* const* __restrict__ A_ptrs,
    const int32_t* __restrict__ seg_starts, int32_t S_host, const int32_t* __restrict__ perm,
    int32_t n, int32_t h_in, int32_t kcm, int32_t ks, float* __restrict__ part, int64_t slice,
    float* __restrict__ v_out, int32_t* __restrict__ rowks, int32_t rk_short,
    int32_t* __restrict__ bad_flag, const int32_t* __restrict__ meta) {
  using C = ShrLdsCfg<R, MT, D>;
  constexpr int NB = C::NB, UN = C::UN, STAGE = C::STAGE, PPR = C::PPR, RPB = C::RPB;
  constexpr int XB = C::XB, AB = C::AB, LPS = C::LPS;
  const int S = meta ? meta[0] : S_host;
  if (meta && meta[2] < kLongMin) return;  // no long segment at all
  __shared__ TileSegs<MT> sh;
  __shared__ int s_prow[MT];
  __shared__ ShrStage<C> b0, b1, b2, b3, b4, b5, b6, b7;
  auto buf = [&](auto J) -> ShrStage<C>& {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return b0;
    else if constexpr (j == 1) return b1;
    else if constexpr (j == 2) return b2;
    else if constexpr (j == 3) return b3;
    else if constexpr (j == 4) return b4;
    else if constexpr (j == 5) return b5;
    else if constexpr (j == 6) return b6;
    else return b7;
  };

  // Workgroup b runs on XCD b % 8.  With a multiple of 8 chunks, XCD x owns the chunks
  // kc = x (mod 8) of every tile.  Otherwise, for h_in above kChunkMajorMinK (A of several
  // MB per adapter), XCD x takes a contiguous eighth of the (chunk, tile) pairs in
  // chunk-major order, so that its L2 fetches about ks / 8 + 1 chunks of A instead of all
  // of them; at smaller h_in the pairs go tile-major (chunk-major cost 1-2 % there, for
  // little A).
  const int b = blockIdx.x;
  int tile, kc;
  if (ks % kXcds == 0) {
    const int m = ks / kXcds, j = b / kXcds;
    tile = j / m;
    kc = b % kXcds + kXcds * (j % m);
  } else if (h_in <= kChunkMajorMinK) {
    tile = b / ks;
    kc = b % ks;
  } else {
    const int tiles = static_cast<int>(gridDim.x) / ks;
    const int pairs = tiles * ks;
    const int xcd = b % kXcds, per = pairs / kXcds, rem = pairs % kXcds;
    const int idx = xcd * per + min(xcd, rem) + b / kXcds;
    kc = idx / tiles;
    tile = idx % tiles;
  }
  const int r0 = tile * MT;
  const int r1 = min(n, r0 + MT);
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int mrow = lane & 15, kq = lane >> 4;
  const SegPre pre = seg_preload(seg_starts, A_ptrs, S);
  if (tid < MT) s_prow[tid] = (r0 + tid < r1) ? (perm ? perm[r0 + tid] : r0 + tid) : 0;
  if (tid == 0) sh.nseg = 0;
  __syncthreads();
  const int nseg = tile_long_segments_pre<MT, 256>(seg_starts, A_ptrs, S, r0, r1, sh, pre);
  if (kc == 0) mark_tile_rows(sh, r0, r1, ks, rk_short, rowks, bad_flag);
  if (nseg == 0) return;  // uniform
  const int k_lo = kc * kcm;
  const int k_hi = min(h_in, k_lo + kcm);
  // stages of the chunk, padded to a multiple of D: k past the chunk loads the chunk's last
  // 16 bytes of the row again (just fetched, so a cache hit) and multiplies zeros
  const int nst = ((k_hi - k_lo + STAGE - 1) / STAGE + D - 1) / D * D;
  const int k_last = k_hi - 8;
  const int qw = 16 * w;  // this wave's first row in the tile
  // loading lane: row lane / PPR of a block, piece run_piece(lane) of the stage
  const int lrow = lane / PPR;
  const int kpiece = 8 * run_piece<PPR>(lane);
  // MFMA lane (mrow, kq): row mrow of the wave's rows (block mrow / RPB) for x, A row
  // 16 nb + mrow for column block nb; piece 4u + kq in k step u
  const int bi = mrow / RPB, bj = mrow % RPB;

  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int q = 0;
  for (int sg; (sg = next_run(sh, q)) >= 0;) {
    // rows outside the run fetch row r0 of the tile (it exists) and are zeroed below
    const bool xin = sh.rseg[qw + mrow] == sg;
    gptr<const uint16_t> xrun[XB], arun[AB];
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int qr = qw + RPB * i + lrow;
      xrun[i] = global_ptr(x) + static_cast<int64_t>(s_prow[sh.rseg[qr] == sg ? qr : 0]) * ld_x;
    }
#pragma unroll
    for (int t = 0; t < AB; ++t)
      arun[t] = global_ptr(sh.ptr[sg]) + static_cast<int64_t>(RPB * (AB * w + t) + lrow) * h_in;
    auto issue = [&](auto J, int s) {
      ShrStage<C>& st = buf(J);
      const int kk = k_lo + s * STAGE + kpiece;
      const int off = kk < k_hi ? kk : k_last;
#pragma unroll
      for (int t = 0; t < AB; ++t) load_to_lds(arun[t] + off, &st.a[AB * w + t][0]);
#pragma unroll
      for (int i = 0; i < XB; ++i) load_to_lds(xrun[i] + off, &st.x[w][i * C::SLOTS]);
    };
    auto compute = [&](auto J, int s) {
      const ShrStage<C>& st = buf(J);
      const int k0 = k_lo + s * STAGE + 8 * kq;
      // every operand is read unconditionally and masked afterwards: a read under a branch
      // made the compiler wait for every load in flight first
      uint4 xv[UN], av[UN][NB];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int slot = run_slot<PPR>(bj, 4 * u + kq);
        // (the bound is never reached; without it the compiler cannot tell this read from
        // the global-to-LDS loads in flight into the other stage buffers and waits for all
        // of them first)
        xv[u] = st.x[w][min(bi * C::SLOTS + slot, XB * C::SLOTS - 1)];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) av[u][nb] = st.a[16 * nb / RPB + bi][slot];
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const bool in = k0 + 32 * u < k_hi;
        const uint4 xa = (in && xin) ? xv[u] : zero4();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb] = Elem<DT>::mfma(xa, in ? av[u][nb] : zero4(), acc[nb]);
      }
    };
    auto step = [&](auto J, int s) {
      wait_vmem<(D - 2) * LPS>();
      barrier_no_fence();
      issue(std::integral_constant<int, (decltype(J)::value + D - 1) % D>{}, s + D - 1);
      compute(J, s);
    };
    static_for<0, D - 1>([&](auto J) { issue(J, J); });
    int s = 0;
    for (; s < nst - D; s += D) static_for<0, D>([&](auto J) { step(J, s + J); });
    step(std::integral_constant<int, 0>{}, s);  // fetches the last stage, nst - 1
    wait_vmem<0>();
    barrier_no_fence();
    static_for<1, D>([&](auto J) { compute(J, s + J); });
    barrier_no_fence();  // the next run refills the buffers
  }
  // rows qw + 4(lane/16) + c, column nb*16 + lane%16
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int qr = qw + 4 * kq + c;
    if (sh.rseg[qr] < 0) continue;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int64_t o = static_cast<int64_t>(r0 + qr) * R + nb * 16 + mrow;
      if (ks == 1)
        v_out[o] = acc[nb][c];
      else
        part[kc * slice + o] = acc[nb][c];
    }
  }
}

// Expand on MFMA 16x16x32 for a tile of TR sorted rows and TC columns, computed
// transposed: D[col, row] = sum_k Bk[col, k] * Vk[k, row], where the k dimension is 2r:
// the stored rows of B[a] twice (A operand) against scale * v split into two 16-bit
// halves, hi = round(scale*v) and lo = round(scale*v - hi) (B operand).  The products are
// exact and summed in float32; hi + lo carries 16 (bf16) or 22 (fp16) significant bits of
// scale*v.  For fp16 each row of scale*v is first multiplied by a power of two that puts
// its largest magnitude in [2^14, 2^15), and the row's sums are multiplied back by the
// inverse power (both exact), so any float32 v fits fp16's range.  B's columns are taken
// in an order that leaves every lane with 8 consecutive columns of one row (exp_load_b),
// so y is read and written with 16-byte vectors straight from the accumulators, with no
// pass through LDS: y is loaded as soon as the caller rows are known, then updated as
// y + sum in float32 and rounded once.  Tiles are 32 x 256 (64 x 128 at r = 32); at
// r = 64 a tile then reads twice as many B bytes (from L2) as y bytes, which measured
// faster than the squarer 64 x 128 tiles.
//
// Workgroup b runs on XCD b % 8 (round-robin dispatch).  Each XCD owns a contiguous range
// of column strips (and, when the strips are few, a contiguous range of the row tiles), so
// its L2 holds only that part of every B[a]; within its share the workgroups go row tile
// by row tile, so the y traffic in flight at any time covers whole rows of a few
// consecutive tiles.
// The 8 XCDs split the (strip, tile) grid as xs strip groups times 8 / xs tile groups.
// xs = 8 (each XCD a contiguous range of strips over all tiles) unless another split
// gives the busiest XCD fewer tiles to do: with fewer than 8 strips (h_out < 2048 at
// r = 16) or a strip count that 8 does not divide, whole XCDs would otherwise idle or
// finish early (for h_out = 1024, four of the eight).
inline int expand_strip_groups(int strips, int tiles) {
  int best = kXcds;
  int64_t best_load = -1;
  for (int xs = kXcds; xs >= 1; xs /= 2) {
    const int xt = kXcds / xs;
    const int64_t load = static_cast<int64_t>((strips + xs - 1) / xs) * ((tiles + xt - 1) / xt);
    if (best_load < 0 || load < best_load) {
      best_load = load;
      best = xs;
    }
  }
  return best;
}

// split-K slices of long rows that the MFMA expand adds itself (more: reduce_v_kernel
// first): four; with one-pass tiles at r = 16 (few tiles, registers to spare) sixteen, so
// that the LDS-staged shrink's slices (11 for the 70B batch) need no reduce pass there.
// Measured on MI355X, 70B mixed batch at r = 16, graph replay: k/v 36.6 -> 34.4 us; with
// two-pass tiles sixteen slices cost more occupancy than the reduce pass (q/o 48.6 -> 54.7
// us, gate/up 90.4 -> 96.8, down 70.8 -> 75.0).
template <int R, int P>
constexpr int kExpandSlices = (R == 16 && P == 1) ? 16 : 4;

// DPP control: rotate each row of 16 lanes right by 8 (lane l16 reads lane l16 ^ 8)
constexpr int kDppRowRor8 = 0x128;

template <int R, int P = 2>
struct ExpCfg {
  // rows per pass and columns per tile (TC/4 columns per wave); measured on MI355X
  static constexpr int TRP = 32;
  static constexpr int TC = (R == 32) ? 128 : 256;
  // passes over the tile's rows, one after another with the same B registers: B is read
  // once for PASSES * TRP rows (one pass when two would leave CUs without a tile)
  static constexpr int PASSES = P;
  static constexpr int TR = TRP * PASSES;            // rows per tile
  static constexpr int RB = TRP / 16, CB = TC / 64;  // 16 x 16 blocks per wave and pass
  // waves per SIMD the register budget is set for (five spill at r = 64; one-pass tiles are
  // used only when there are fewer tiles than CUs, so at most two waves per SIMD are ever
  // resident and they get the registers of two)
  static constexpr int WAVES_PER_SIMD = (P == 1) ? 2 : (R == 64) ? 4 : 5;
};

// the register budget of a launch that also adds VS split-K slices (sixteen slices need
// more registers than five waves per SIMD leave)
template <int R, int P, int VS>
constexpr int exp_waves_per_simd() {
  return (VS > 4 && ExpCfg<R, P>::WAVES_PER_SIMD > 4) ? 4 : ExpCfg<R, P>::WAVES_PER_SIMD;
}

// The B operand of one run for a wave's CB column blocks.  The blocks come in pairs whose
// 16 columns are interleaved in groups of 4: block 2p + h, lane (l16, kq) takes column
// wc + 32p + 8(l16/4) + 4h + l16%4 and B values 32s + 8kq .. +7 (mod r) of it, s < NKU.
// The products then leave lane (kq, l16) with the 8 consecutive columns
// wc + 32p + 8kq .. +7 of one row in blocks 2p and 2p + 1: 16 bytes of y.
template <int R, int CB, int NKU>
__device__ inline void exp_load_b(gptr<const uint16_t> B, int wc, int l16, int kq, int h_out,
                                  uint4 (&bop)[CB][NKU]) {
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int col = wc + 32 * (cb >> 1) + 8 * (l16 >> 2) + 4 * (cb & 1) + (l16 & 3);
#pragma unroll
    for (int s = 0; s < NKU; ++s) {
      const int j0 = (32 * s + 8 * kq) % R;
      bop[cb][s] = (col < h_out) ? ld16(B + static_cast<int64_t>(col) * R + j0) : zero4();
    }
  }
}

// VS: v comes as up to VS split-K slices (vks of them, vslice floats apart) that are added
// here in slice order; VS == 1: v is final.
template <int DT, int R, int VS, int P>
__global__ __launch_bounds__(256, (exp_waves_per_simd<R, P, VS>())) void expand_mfma_kernel(
    uint16_t* __restrict__ y, int64_t ld_y, const float* __restrict__ v, int64_t vslice, int32_t vks,
    const uint16_t* const* __restrict__ B_ptrs, const int32_t* __restrict__ seg_starts,
    int32_t S_host, const int32_t* __restrict__ perm, int32_t n, int32_t h_out, float scale,
    int32_t tiles, int32_t strips, int32_t xs, int32_t ybuf, const int32_t* __restrict__ meta) {
  const int S = meta ? meta[0] : S_host;
  if (meta && meta[2] < kLongMin) return;  // no long segment at all
  using E = Elem<DT>;
  using C = ExpCfg<R, P>;
  constexpr int TR = C::TR, TRP = C::TRP, TC = C::TC, RB = C::RB, CB = C::CB;
  constexpr int KT = 2 * R;          // k of the hi/lo product
  constexpr int NK = KT / 32;        // MFMA k-steps
  constexpr int NKU = (R >= 32) ? R / 32 : 1;  // distinct B loads per column block
  constexpr int VPT = TR * R / 256;  // v values per thread
  static_assert(CB % 2 == 0, "column blocks come in pairs");
  __shared__ TileSegs<TR> sh;
  __shared__ int s_prow[TR];  // caller row of each tile row
  // The hi/lo halves of scale * v.  Rows are padded by 16 bytes: the 16 lanes that read one
  // k range of 16 different rows then fall on 16 different bank groups instead of one.
  __shared__ __attribute__((aligned(16))) uint16_t vlds[TR][KT + 8];
  __shared__ int s_exp[TR];  // fp16: the row's sums are multiplied by 2^s_exp[row]

  // XCD x owns strip group x % xs and tile group x / xs (xs * xt = 8 groups) and walks
  // its strips tile-major
  const int b = blockIdx.x;
  const int xcd = b % kXcds, jx = b / kXcds;
  const int xt = kXcds / xs, sgi = xcd % xs, tgi = xcd / xs;
  const int sper = strips / xs, srem = strips % xs;
  const int sx0 = sgi * sper + min(sgi, srem);
  const int nsx = sper + (sgi < srem ? 1 : 0);
  const int tper = tiles / xt, trem = tiles % xt;
  const int tx0 = tgi * tper + min(tgi, trem);
  const int ntx = tper + (tgi < trem ? 1 : 0);
  if (nsx == 0 || jx >= nsx * ntx) return;
  const int tile = tx0 + jx / nsx, strip = sx0 + jx % nsx;
  const int c0 = strip * TC;
  const int g0 = tile * TR;
  const int g1 = min(n, g0 + TR);
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int kq = lane >> 4, l16 = lane & 15;
  const int wc = c0 + (TC / 4) * w;  // first column of this wave

  // one round of loads for the caller rows, the segment bounds and the B pointers; then y
  // and v go out, the segments are found from registers, and B follows without waiting
  const SegPre pre = seg_preload(seg_starts, B_ptrs, S);
  if (tid < TR) s_prow[tid] = (g0 + tid < g1) ? (perm ? perm[g0 + tid] : g0 + tid) : -1;
  if (tid == 0) sh.nseg = 0;
  __syncthreads();
  // y, 16 bytes per lane and instruction.  Products' layout: lane (kq, l16) holds row
  // ro + 16rb + l16 of the pass that starts at tile row ro, columns wc + 32p + 8kq .. +7
  // of block pair p, so one instruction covers 16 rows x 64 bytes.  With two block pairs
  // per wave (LINES), y goes in whole 128-byte lines instead: instruction h of block rb
  // covers rows ro + 16rb + 8h .. +7, lane (kq, l16) row ro + 16rb + 8h + l16 % 8 and
  // columns wc + 32(l16 / 8) + 8kq .. +7, and the sums are brought to that layout by one
  // exchange between lanes l16 and l16 ^ 8 (read-modify-writes of whole lines measured
  // 8-18 % faster on MI355X than of 16 rows x 64 bytes).
  constexpr bool LINES = CB == 4;
  const int lrow = l16 & 7, lpair = l16 >> 3;
  uint4 yv[RB][CB / 2];
  auto y_row = [&](int ro, int rb, int p) {
    return LINES ? ro + 16 * rb + 8 * p + lrow : ro + 16 * rb + l16;
  };
  auto y_col = [&](int p) { return wc + 32 * (LINES ? lpair : p) + 8 * kq; };
  auto load_y = [&](int ro) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int p = 0; p < CB / 2; ++p) {
        const int yr = s_prow[y_row(ro, rb, p)];
        const int col = y_col(p);
        yv[rb][p] = (yr >= 0 && col < h_out) ? ld16(y + static_cast<int64_t>(yr) * ld_y + col) : zero4();
      }
  };
  load_y(0);
  float vv[VPT];
  {
    float t[VS][VPT];
#pragma unroll
    for (int k = 0; k < VS; ++k)
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int idx = tid + 256 * u;
        t[k][u] = (k < vks && g0 + idx / R < g1) ? v[k * vslice + static_cast<int64_t>(g0) * R + idx] : 0.f;
      }
    // the slices' fixed order (sum_slices): partial sums p_q over slices q, q + 4, ...,
    // then (p0 + p1) + (p2 + p3), then + 0 (slices past vks are zeros)
    static_assert(VS == 1 || VS % 4 == 0, "slice sum order");
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      if constexpr (VS == 1) {
        vv[u] = t[0][u];
      } else {
        float pq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          pq[q] = t[q][u];
#pragma unroll
          for (int k = q + 4; k < VS; k += 4) pq[q] += t[k][u];
        }
        vv[u] = ((pq[0] + pq[1]) + (pq[2] + pq[3])) + 0.f;
      }
    }
  }
  if (tile_long_segments_pre<TR, 256>(seg_starts, B_ptrs, S, g0, g1, sh, pre) == 0) return;  // uniform

  // B of the tile's first long run goes out now, so that its latency overlaps the wait
  // for v.  B row c holds the r values of column
  // c; the product's k runs over the hi halves, then the lo halves, so the k-steps past r
  // reuse the same B bytes: only NKU = r / 32 distinct loads per column block.
  int q = 0;
  const int sg = next_run(sh, q);  // the tile meets a long segment, so there is a first run
  uint4 bop[CB][NKU];
  exp_load_b<R, CB, NKU>(global_ptr(sh.ptr[sg]), wc, l16, kq, h_out, bop);

#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int idx = tid + 256 * u;
    float val = (sh.rseg[idx / R] >= 0) ? scale * vv[u] : 0.f;
    if constexpr (DT == SGMV_F16) {
      // the R values of a row sit in R consecutive lanes: their largest magnitude
      float mx = fabsf(val);
#pragma unroll
      for (int msk = 1; msk < R; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk));
      const int sh_up = (mx > 0.f && mx <= 3.0e38f) ? 14 - ilogbf(mx) : 0;
      val = ldexpf(val, sh_up);
      if (idx % R == 0) s_exp[idx / R] = -sh_up;
    }
    const uint32_t hw = E::pack(val, 0.f) & 0xffffu;
    const uint32_t lw = E::pack(val - E::lo(hw), 0.f) & 0xffffu;
    vlds[idx / R][idx % R] = static_cast<uint16_t>(hw);
    vlds[idx / R][R + idx % R] = static_cast<uint16_t>(lw);
  }
  __syncthreads();

  // y is stored through a raw buffer resource over all of y with sc1 stores, which the L2
  // writes through, so the y lines are not left dirty for the write-back at the kernel's
  // end (13B prefill calls 3-6 % faster); ybuf (set on the host from the caller's whole
  // y) is 0 when y spans 4 GiB or more, past the 32-bit buffer offsets, and the stores
  // are then plain global stores
  const __amdgpu_buffer_rsrc_t yrs =
      __builtin_amdgcn_make_buffer_rsrc(static_cast<void*>(y), static_cast<short>(0), -1, kBufferRsrcWord3);
  int cur = sg;  // the run whose B is in bop
  for (int pass = 0; pass < C::PASSES; ++pass) {
    const int ro = pass * TRP;
    if (pass > 0) load_y(ro);
    int rs[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) rs[rb] = sh.rseg[ro + 16 * rb + l16];
    f32x4_t acc[RB][CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the long runs that meet this pass's rows, in increasing order (the reads are uniform)
    for (int qq = ro;;) {
      while (qq < ro + TRP && sh.rseg[qq] < 0) ++qq;
      if (qq >= ro + TRP) break;
      const int run = sh.rseg[qq];
      while (qq < ro + TRP && sh.rseg[qq] == run) ++qq;
      if (run != cur) {
        exp_load_b<R, CB, NKU>(global_ptr(sh.ptr[run]), wc, l16, kq, h_out, bop);
        cur = run;
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int lq = ro + 16 * rb + l16;
        uint4 vop[NK];
#pragma unroll
        for (int s = 0; s < NK; ++s)
          vop[s] = (rs[rb] == run) ? *reinterpret_cast<const uint4*>(&vlds[lq][32 * s + 8 * kq]) : zero4();
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int s = 0; s < NK; ++s) acc[rb][cb] = E::mfma(bop[cb][s % NKU], vop[s], acc[rb][cb]);
      }
    }
    // y + sum, rounded once, from the accumulators: in the products' layout lane (kq,
    // l16) owns 16 bytes of row ro + 16rb + l16 per block pair; with LINES, the pair that
    // is not the lane's own (p != l16 / 8) is exchanged with lane l16 ^ 8 first
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (DT == SGMV_F16) {
        const int ex = s_exp[ro + 16 * rb + l16];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][cb][i] = ldexpf(acc[rb][cb][i], ex);
      }
      if constexpr (LINES) {
        // lane l16 < 8 keeps its pair-0 sums (row l16, instruction 0) and takes the
        // pair-0 sums of row l16 + 8 (instruction 1) from lane l16 + 8, which keeps its
        // pair-1 sums (instruction 1) and takes those of row l16 (instruction 0): two DPP
        // moves that rotate each row of 16 lanes by 8, one writing lanes 0-7 of the row
        // (banks 0 and 1), the other lanes 8-15 (banks 2 and 3)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p0 = __float_as_int(acc[rb][hb][i]), p1 = __float_as_int(acc[rb][2 + hb][i]);
            acc[rb][2 + hb][i] = __int_as_float(__builtin_amdgcn_update_dpp(p1, p0, kDppRowRor8, 0xf, 0x3, false));
            acc[rb][hb][i] = __int_as_float(__builtin_amdgcn_update_dpp(p0, p1, kDppRowRor8, 0xf, 0xc, false));
          }
      }
#pragma unroll
      for (int p = 0; p < CB / 2; ++p) {
        const int col = y_col(p);
        const int tr = y_row(ro, rb, p);
        if (sh.rseg[tr] < 0 || col >= h_out) continue;
        const f32x4_t d0 = acc[rb][2 * p], d1 = acc[rb][2 * p + 1];
        const uint4 yy = yv[rb][p];
        uint4 o;
        o.x = E::pack(E::lo(yy.x) + d0[0], E::hi(yy.x) + d0[1]);
        o.y = E::pack(E::lo(yy.y) + d0[2], E::hi(yy.y) + d0[3]);
        o.z = E::pack(E::lo(yy.z) + d1[0], E::hi(yy.z) + d1[1]);
        o.w = E::pack(E::lo(yy.w) + d1[2], E::hi(yy.w) + d1[3]);
        const int64_t e = static_cast<int64_t>(s_prow[tr]) * ld_y + col;
        if (ybuf)
          __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{o.x, o.y, o.z, o.w}, yrs,
                                                 static_cast<int>(2 * e), 0, kStoreSc1);
        else
          *reinterpret_cast<uint4*>(y + e) = o;
      }
    }
  }
}

// v[i, :] = sum of the split-K slices of sorted row i, for rows whose slice count is
// nonzero (rows of long segments with one slice already have their final v) and, unless
// `which` is kReduceAll, whose segment kind (short or long) it names.  The counts are the
// current call's: the shrink of the chain that launches this pass wrote them for every row
// (with device tables, a chain whose kind of segment is absent skips its shrink, and this
// pass then exits too).  A workgroup takes 64 consecutive entries of v; wave q adds slices
// q, q + 4, q + 8, ... of each entry in that order and the four waves' sums are added as
// (w0 + w1) + (w2 + w3).
template <int R>
__global__ __launch_bounds__(256) void reduce_v_kernel(float* __restrict__ v,
                                                      const float* __restrict__ part, int64_t slice,
                                                      const int32_t* __restrict__ rowks, int32_t n,
                                                      int32_t ks_max, int32_t which,
                                                      const int32_t* __restrict__ meta) {
  if (meta) {
    if (which == kReduceShort && meta[1] >= kLongMin) return;  // no short segment
    if (which == kReduceLong && meta[2] < kLongMin) return;    // no long segment
  }
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const bool in = idx < static_cast<int64_t>(n) * R;
  const int32_t rk = in ? rowks[idx / R] : 0;
  const bool short_row = (rk & kShortRowFlag) != 0;
  const bool take = which == kReduceAll || (which == kReduceShort) == short_row;
  const int ks = take ? min(rk & ~kShortRowFlag, ks_max) : 0;
  float acc = 0.f;
  constexpr int kFly = 8;  // loads in flight per thread
  for (int k0 = q; k0 < ks; k0 += 4 * kFly) {
    float t[kFly];
#pragma unroll
    for (int u = 0; u < kFly; ++u) {
      const int k = k0 + 4 * u;
      t[u] = (k < ks) ? part[k * slice + idx] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kFly; ++u) acc += t[u];
  }
  red[q][lane] = acc;
  __syncthreads();
  if (q == 0 && ks > 0) v[idx] = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
}

// ------------------------------------------------------------------------------------
// ------------------------------------------------------------------------------------
// host side: sizes, validation, launches
// ------------------------------------------------------------------------------------
inline int gemv_kc(int r) {
  switch (r) {
    case 16: return GemvCfg<16>::KC;
    case 32: return GemvCfg<32>::KC;
    case 64: return GemvCfg<64>::KC;
  }
  return 0;
}
static_assert(GemvCfg<16>::KC == 512 && GemvCfg<32>::KC == 256 && GemvCfg<64>::KC == 256,
              "table_gemv_kc in sgmv_checks.h must match the GEMV shrink's chunk");

// split-K of the MFMA shrinks: about `target` workgroups (set per kernel and rank from
// measured sweeps on MI355X), chunks of at least 256 k rounded up to `granule`, a multiple
// of 8 chunks where there are 8 or more before the rounding (XCD-owned chunks), and no
// more slices than the workspace holds
inline void split_k(int32_t n, int32_t h_in, int ks_cap, int mt, int target, int granule,
                    int* kcm, int* ks, bool resident = false) {
  const int tiles = (n + mt - 1) / mt;
  int k = (target + tiles - 1) / tiles;
  k = min(k, max(1, h_in / 256));
  k = max(1, min(k, ks_cap));
  if (k >= 8) k -= k % 8;
  for (;;) {
    const int c = ((h_in + k - 1) / k + granule - 1) / granule * granule;
    *kcm = c;
    *ks = (h_in + c - 1) / c;
    // resident: every workgroup must fit on the GPU at once (target is that count), or
    // the last ones start only when others end and the kernel takes one of them longer
    if (!resident || k == 1 || static_cast<int64_t>(tiles) * *ks <= target) return;
    --k;
  }
}

template <class C>
inline void mfma_split(int32_t n, int32_t h_in, int ks_cap, int* kcm, int* ks) {
  split_k(n, h_in, ks_cap, C::MT, C::TARGET_WGS, 64, kcm, ks);
}

// Segment tables of one call.  With host tables S, min_len and max_len are exact.  With
// tables built on the device, meta points at their [S, min_len, max_len, n_valid] word,
// S is only an upper bound (it sizes the grids) and every kernel reads the count from meta.
struct Tables {
  const uint16_t* const* ptrs;
  const int32_t* seg_starts;
  const int32_t* perm;
  int32_t n, S, min_len, max_len;
  const int32_t* meta = nullptr;
  // a rank group of sgmv_lora_add_ranked: other groups' kernels may run beside its own
  bool in_group = false;
  // the workspace's flag word, for host tables (kernels flag tables that contradict
  // min_len / max_len)
  int32_t* flag = nullptr;
  // rows of the caller's y when they are more than n (a rank group's rows, addressed
  // through perm, lie anywhere in the whole batch's y); 0: n
  int32_t y_rows = 0;
  // whether every byte offset into y fits the 32-bit offsets of a buffer resource
  bool y_fits_buffer(int64_t ld_y, int32_t h_out) const {
    const int64_t rows = y_rows > 0 ? y_rows : n;
    return rows > 0 && ((rows - 1) * ld_y + h_out) * 2 < (int64_t(1) << 32);
  }
  bool use_gemv() const { return meta || min_len < kLongMin; }
  bool use_long() const { return meta || max_len >= kLongMin; }
  // grid of a GEMV kernel with `per` items per segment: one workgroup per item with host
  // tables; with device tables at most max_wgs workgroups striding over S_max * per items
  // (the real count is only known on the device)
  dim3 gemv_grid(int per, int max_wgs) const {
    if (!meta) return dim3(static_cast<unsigned>(S), static_cast<unsigned>(per));
    const int64_t items = static_cast<int64_t>(S) * per;
    return dim3(static_cast<unsigned>(items < max_wgs ? items : max_wgs), 1);
  }
};

// Split-K plan of one call, fixed on the host before anything is launched, so that the
// kernels of either chain can write the slice counts of the other chain's rows (see
// shrink_gemv_kernel).  bad_flag is the workspace's flag word, passed to a chain's shrink
// when the other chain is not launched.
struct Plan {
  int ksg = 0;          // GEMV shrink: split-K slices of short rows
  int ksl = 0;          // long shrink: split-K slices of long rows
  int kcm = 0;          // long shrink: K chunk
  bool lds = false;     // long shrink: the LDS-staged kernel
  int32_t* flag = nullptr;
  int32_t rk_short() const { return kShortRowFlag | ksg; }
  int32_t rk_long() const { return ksl == 1 ? 0 : ksl; }
};

template <int R>
Plan make_plan(const Tables& T, int32_t h_in, const WsLayout& L) {
  Plan P;
  P.ksg = (h_in + GemvCfg<R>::KC - 1) / GemvCfg<R>::KC;
  if constexpr (R == 64) {
    P.lds = true;
  } else {
    P.lds = R == 16 && shrink_lds_long_rows(h_in, !T.meta && !T.in_group && T.use_gemv());
  }
  if (P.lds) {
    // Chunks are whole multiples of D stages (384 k at r = 16, 256 at r = 64): for the 70B
    // batch 11 chunks at r = 16 and 16 at r = 64, which are XCD-owned (each XCD's L2 then
    // holds an eighth of A).
    if constexpr (R != 32) {
      using C = ShrLdsCfg<R, kLdsMT, kLdsD<R>>;
      split_k(T.n, h_in, L.ks_max, kLdsMT, kLdsWgs, C::STAGE * kLdsD<R>, &P.kcm, &P.ksl, true);
    }
  } else {
    if constexpr (R != 64) mfma_split<ShrCfg<R>>(T.n, h_in, L.ks_max, &P.kcm, &P.ksl);
  }
  P.flag = T.meta ? nullptr : T.flag;
  return P;
}

// short segments: P.ksg split-K slices, counted in rowks with kShortRowFlag
template <int DT, int R>
hipError_t launch_shrink_short(hipStream_t st, const uint16_t* x, int64_t ld_x, const Tables& T,
                               int32_t h_in, const WsLayout& L, char* ws, const Plan& P) {
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  int32_t* rowks = reinterpret_cast<int32_t*>(ws + L.rowks_off);
  int32_t* bad = T.use_long() ? nullptr : P.flag;
  hipLaunchKernelGGL((shrink_gemv_kernel<DT, R>), T.gemv_grid(P.ksg, 2048), dim3(256), 0, st, x,
                     ld_x, T.ptrs, T.seg_starts, T.perm, h_in, part, L.slice, rowks, P.ksg,
                     P.rk_long(), bad, T.meta);
  return hipGetLastError();
}

// long segments: the final v in v_long (P.ksl == 1) or P.ksl slices, counted in rowks
template <int DT, int R>
hipError_t launch_shrink_long(hipStream_t st, const uint16_t* x, int64_t ld_x, const Tables& T,
                              int32_t h_in, const WsLayout& L, char* ws, float* v_long,
                              const Plan& P) {
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  int32_t* rowks = reinterpret_cast<int32_t*>(ws + L.rowks_off);
  int32_t* bad = T.use_gemv() ? nullptr : P.flag;
  if (P.lds) {
    if constexpr (R != 32) {
      constexpr int MT = kLdsMT, D = kLdsD<R>;
      const int tiles = (T.n + MT - 1) / MT;
      hipLaunchKernelGGL((shrink_lds_kernel<DT, R, MT, D>), dim3(tiles * P.ksl), dim3(256), 0, st,
                         x, ld_x, T.ptrs, T.seg_starts, T.S, T.perm, T.n, h_in, P.kcm, P.ksl, part,
                         L.slice, v_long, rowks, P.rk_short(), bad, T.meta);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if constexpr (R != 64) {
    const int tiles = (T.n + ShrCfg<R>::MT - 1) / ShrCfg<R>::MT;
    hipLaunchKernelGGL((shrink_mfma_kernel<DT, R>), dim3(tiles * P.ksl), dim3(256), 0, st, x, ld_x,
                       T.ptrs, T.seg_starts, T.S, T.perm, T.n, h_in, P.kcm, P.ksl, part, L.slice,
                       v_long, rowks, P.rk_short(), bad, T.meta);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

// short segments sum ks slices of vsrc (slice stride `slice`) themselves
template <int DT, int R>
hipError_t launch_expand_short(hipStream_t st, uint16_t* y, int64_t ld_y, const float* vsrc,
                               int64_t slice, int ks, const Tables& T, int32_t h_out,
                               float scale) {
  constexpr int CPL = 128 / R;
  const int chunks = (h_out + 64 * CPL - 1) / (64 * CPL);
  hipLaunchKernelGGL((expand_gemv_kernel<DT, R>), T.gemv_grid(chunks, 8192), dim3(64), 0, st, y,
                     ld_y, vsrc, slice, ks, T.ptrs, T.seg_starts, T.perm, h_out, scale, chunks,
                     T.meta);
  return hipGetLastError();
}

// long segments read v as ks slices of vsrc (at most kExpandSlices<R, P>, r <= 32) or
// final (ks 1); tiles of P passes of 32 rows
template <int DT, int R, int P>
hipError_t launch_expand_tiles(hipStream_t st, uint16_t* y, int64_t ld_y, const float* vsrc,
                               int64_t slice, int ks, const Tables& T, int32_t h_out,
                               float scale) {
  using C = ExpCfg<R, P>;
  const int tiles = (T.n + C::TR - 1) / C::TR;
  const int strips = (h_out + C::TC - 1) / C::TC;
  const int xs = expand_strip_groups(strips, tiles);
  // each XCD takes at most ceil(strips / xs) strips of ceil(tiles / xt) tiles: pad the
  // grid to 8 equal shares
  const int64_t share = static_cast<int64_t>((tiles + kXcds / xs - 1) / (kXcds / xs)) *
                        ((strips + xs - 1) / xs);
  if (share * kXcds > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(share * kXcds));
  const int32_t ybuf = T.y_fits_buffer(ld_y, h_out) ? 1 : 0;
  if (ks > 1) {
    if constexpr (R <= 32) {
      if (ks > kExpandSlices<R, P>) return hipErrorInvalidValue;
      hipLaunchKernelGGL((expand_mfma_kernel<DT, R, kExpandSlices<R, P>, P>), grid, dim3(256), 0, st,
                         y, ld_y, vsrc, slice, ks, T.ptrs, T.seg_starts, T.S, T.perm, T.n, h_out,
                         scale, tiles, strips, xs, ybuf, T.meta);
    } else {
      return hipErrorInvalidValue;  // r = 64: reduce_v_kernel runs first
    }
  } else {
    hipLaunchKernelGGL((expand_mfma_kernel<DT, R, 1, P>), grid, dim3(256), 0, st, y, ld_y, vsrc,
                       slice, 1, T.ptrs, T.seg_starts, T.S, T.perm, T.n, h_out, scale, tiles,
                       strips, xs, ybuf, T.meta);
  }
  return hipGetLastError();
}

// Two-pass tiles (B read once for 64 rows) unless they would leave CUs without a tile:
// then one-pass tiles of 32 rows, twice as many (narrow outputs such as the 70B k/v
// projections, h_out = 1024: 132 two-pass tiles for 256 CUs).
constexpr int kCus = 256;

// at r = 32 four passes with four slices would spill registers
template <int R>
constexpr int kExpandMaxPasses = (R == 32) ? 3 : 4;

// Passes per tile: one when two-pass tiles would leave CUs without a tile; else the
// fewest passes (2 to 4) whose tiles all fit on the GPU at once, so that no tail round of
// tiles runs after the others (13B gate/up: 1728 two-pass tiles for 1280 resident
// workgroups, 1188 three-pass tiles); two when no count fits.
template <int R>
int expand_passes(int32_t n, int32_t h_out) {
  const int64_t strips = (h_out + ExpCfg<R, 2>::TC - 1) / ExpCfg<R, 2>::TC;
  auto tiles = [&](int p) { return (n + 32 * p - 1) / (32 * p) * strips; };
  if (tiles(2) < kCus) return 1;
  const int64_t resident = static_cast<int64_t>(kCus) * ExpCfg<R, 2>::WAVES_PER_SIMD;
  for (int p = 2; p <= kExpandMaxPasses<R>; ++p)
    if (tiles(p) <= resident) return p;
  return 2;
}

template <int R>
bool expand_one_pass(int32_t n, int32_t h_out) {
  return expand_passes<R>(n, h_out) == 1;
}

template <int DT, int R>
hipError_t launch_expand_long(hipStream_t st, uint16_t* y, int64_t ld_y, const float* vsrc,
                              int64_t slice, int ks, const Tables& T, int32_t h_out,
                              float scale) {
  // A rank group of a mixed-rank call shares the GPU with the other groups' kernels, so
  // the passes chosen for tiles that fit on an idle GPU do not apply; two passes measured
  // best there (70B ranks 16 + 64 gate/up: 117.8 -> 108.7 us per call against four).
  const int passes = expand_passes<R>(T.n, h_out);
  switch (T.in_group && passes > 2 ? 2 : passes) {
    case 1: return launch_expand_tiles<DT, R, 1>(st, y, ld_y, vsrc, slice, ks, T, h_out, scale);
    case 3: return launch_expand_tiles<DT, R, 3>(st, y, ld_y, vsrc, slice, ks, T, h_out, scale);
    case 4:
      if constexpr (kExpandMaxPasses<R> >= 4)
        return launch_expand_tiles<DT, R, 4>(st, y, ld_y, vsrc, slice, ks, T, h_out, scale);
      return hipErrorInvalidValue;
    default: return launch_expand_tiles<DT, R, 2>(st, y, ld_y, vsrc, slice, ks, T, h_out, scale);
  }
}

// v of every row whose slice count (rowks) is nonzero and whose kind `which` selects,
// summed in slice order
template <int R>
hipError_t launch_reduce(hipStream_t st, float* v, const Tables& T, const WsLayout& L, char* ws,
                         int32_t which) {
  const int64_t total = static_cast<int64_t>(T.n) * R;
  hipLaunchKernelGGL((reduce_v_kernel<R>), dim3(static_cast<unsigned>((total + 63) / 64)), dim3(256),
                     0, st, v, reinterpret_cast<const float*>(ws + L.part_off), L.slice,
                     reinterpret_cast<const int32_t*>(ws + L.rowks_off), T.n, L.ks_max, which,
                     T.meta);
  return hipGetLastError();
}

// whether the long chain's slices need a reduce pass before its expand: a few slices are
// added by the MFMA expand itself (r <= 32), more are summed once per row
template <int R>
bool long_needs_reduce(int ksl, int32_t n, int32_t h_out) {
  if (ksl <= 1) return false;
  if (R > 32) return true;
  const int most = expand_one_pass<R>(n, h_out) ? kExpandSlices<R, 1> : kExpandSlices<R, 2>;
  return ksl > most;
}

template <int DT, int R>
hipError_t run_shrink(hipStream_t st, float* v, const uint16_t* x, int64_t ld_x, const Tables& T,
                      int32_t h_in, const WsLayout& L, char* ws) {
  const Plan P = make_plan<R>(T, h_in, L);
  hipError_t e;
  if (T.use_gemv() && (e = launch_shrink_short<DT, R>(st, x, ld_x, T, h_in, L, ws, P)) != hipSuccess)
    return e;
  if (T.use_long() && (e = launch_shrink_long<DT, R>(st, x, ld_x, T, h_in, L, ws, v, P)) != hipSuccess)
    return e;
  if (!T.use_gemv() && P.ksl <= 1) return hipSuccess;
  return launch_reduce<R>(st, v, T, L, ws, kReduceAll);
}

template <int DT, int R>
hipError_t run_expand(hipStream_t st, uint16_t* y, int64_t ld_y, const float* v, const Tables& T,
                      int32_t h_out, float scale) {
  hipError_t e;
  if (T.use_gemv() && (e = launch_expand_short<DT, R>(st, y, ld_y, v, 0, 1, T, h_out, scale)) != hipSuccess)
    return e;
  if (T.use_long()) return launch_expand_long<DT, R>(st, y, ld_y, v, 0, 1, T, h_out, scale);
  return hipSuccess;
}

// Side streams per device for independent chains of launches in a fused call (the
// short- and long-segment chains of sgmv_lora_add, the rank groups of
// sgmv_lora_add_ranked), with one event that forks them from the caller's stream and one
// per stream that joins them back.  Forks are taken only while the caller's stream is
// being captured into a graph: replayed, the chains overlap; called eagerly, the
// cross-stream event pairs cost more host time than the overlap saves (measured on
// MI355X), so eager calls run every chain on the caller's stream.  The streams and events
// are created by the first fused call on a device that is not being captured (a capture
// before that runs every chain on the caller's stream).  One mutex keeps each call's
// record-wait-launch-record-wait sequence whole when host threads call concurrently.
// Default stream priority.
constexpr int kSideDevices = 64;
constexpr int kSideStreams = 4;
struct SideSlot {
  hipStream_t stream[kSideStreams] = {};
  hipEvent_t join[kSideStreams] = {};
  hipEvent_t fork = nullptr;
};
std::mutex g_side_mu;
SideSlot g_side[kSideDevices];

class SideStream {
 public:
  // Up to `want` side streams forked from st; count() of them are available (0: eager
  // call, capture before the streams exist, or a stream that cannot be queried).
  hipError_t fork(hipStream_t st, int want = 1) {
    lock_ = std::unique_lock<std::mutex>(g_side_mu);
    if (want <= 0) return hipSuccess;
    // a stream whose device or capture state cannot be queried gets no fork (and the
    // query's error is cleared, so that it is not taken for a launch error later)
    int dev = 0;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return hipSuccess;
    }
    if (dev < 0 || dev >= kSideDevices) return hipSuccess;
    SideSlot& slot = g_side[dev];
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess) {
      (void)hipGetLastError();
      return hipSuccess;
    }
    if (!slot.fork) {
      if (cap != hipStreamCaptureStatusNone) return hipSuccess;
      int cur = 0;
      if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      SideSlot made;
      for (int i = 0; i < kSideStreams && e == hipSuccess; ++i) {
        e = hipStreamCreateWithFlags(&made.stream[i], hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&made.join[i], hipEventDisableTiming);
      }
      if (e == hipSuccess) e = hipEventCreateWithFlags(&made.fork, hipEventDisableTiming);
      if (e != hipSuccess) {
        // release whatever was made; the slot stays empty and a later call tries again
        for (int i = 0; i < kSideStreams; ++i) {
          if (made.join[i]) (void)hipEventDestroy(made.join[i]);
          if (made.stream[i]) (void)hipStreamDestroy(made.stream[i]);
        }
        if (made.fork) (void)hipEventDestroy(made.fork);
      }
      const hipError_t er = (cur != dev) ? hipSetDevice(cur) : hipSuccess;
      if (e != hipSuccess) return e;
      slot = made;
      if (er != hipSuccess) return er;
    }
    if (cap != hipStreamCaptureStatusActive) return hipSuccess;
    const int k = want < kSideStreams ? want : kSideStreams;
    if ((e = hipEventRecord(slot.fork, st)) != hipSuccess) return e;
    slot_ = &slot;
    for (int i = 0; i < k; ++i) {
      if ((e = hipStreamWaitEvent(slot.stream[i], slot.fork, 0)) != hipSuccess) return e;
      n_ = i + 1;  // joined back even if a later wait fails
    }
    return hipSuccess;
  }

  int count() const { return n_; }

  // whether a fork from st would be taken now: st's device has its side streams and st is
  // being captured
  static bool ready(hipStream_t st) {
    std::lock_guard<std::mutex> g(g_side_mu);
    int dev = 0;
    if ((st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    if (dev < 0 || dev >= kSideDevices || !g_side[dev].fork) return false;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    return cap == hipStreamCaptureStatusActive;
  }
  hipStream_t stream(int i) const { return slot_->stream[i % n_]; }

  hipError_t join(hipStream_t st) {
    hipError_t e = hipSuccess;
    for (int i = 0; i < n_; ++i) {
      hipError_t ei = hipEventRecord(slot_->join[i], slot_->stream[i]);
      if (ei == hipSuccess) ei = hipStreamWaitEvent(st, slot_->join[i], 0);
      if (e == hipSuccess) e = ei;
    }
    n_ = 0;
    slot_ = nullptr;
    if (lock_.owns_lock()) lock_.unlock();
    return e;
  }

  ~SideStream() {
    if (lock_.owns_lock()) lock_.unlock();
  }

 private:
  std::unique_lock<std::mutex> lock_;
  SideSlot* slot_ = nullptr;
  int n_ = 0;
};

// The short segments of a fused call (decode rows: GEMV kernels) and its long segments
// (prefill rows: MFMA kernels) touch disjoint rows of x, y, v and the workspace, so they
// run as two chains of launches.  Under graph capture the short chain goes to a second
// stream forked from the caller's stream and joined back into it, and the chains overlap
// on the GPU (measured on MI355X, graph replay of the 70B mixed batch: r = 64 gate/up
// 149 -> 133 us per call, r = 16 k/v 54 -> 39 us).
template <int DT, int R>
hipError_t run_short_chain(hipStream_t st, uint16_t* y, int64_t ld_y, const uint16_t* x,
                           int64_t ld_x, const Tables& TA, const Tables& TB, int32_t h_in,
                           int32_t h_out, float scale, const WsLayout& L, char* ws) {
  const Plan P = make_plan<R>(TA, h_in, L);
  hipError_t e = launch_shrink_short<DT, R>(st, x, ld_x, TA, h_in, L, ws, P);
  if (e != hipSuccess) return e;
  float* v_long = reinterpret_cast<float*>(ws + L.v_off);
  const float* part = reinterpret_cast<const float*>(ws + L.part_off);
  // up to 16 slices are added by the GEMV expand itself; more are summed once per row
  // instead of once per column chunk
  if (P.ksg > 16) {
    if ((e = launch_reduce<R>(st, v_long, TA, L, ws, kReduceShort)) != hipSuccess) return e;
    return launch_expand_short<DT, R>(st, y, ld_y, v_long, 0, 1, TB, h_out, scale);
  }
  return launch_expand_short<DT, R>(st, y, ld_y, part, L.slice, P.ksg, TB, h_out, scale);
}

// the long chain after its shrink
template <int DT, int R>
hipError_t run_long_tail(hipStream_t st, uint16_t* y, int64_t ld_y, const Tables& TA,
                         const Tables& TB, int32_t h_out, float scale, const WsLayout& L,
                         char* ws, const Plan& P) {
  float* v_long = reinterpret_cast<float*>(ws + L.v_off);
  const float* part = reinterpret_cast<const float*>(ws + L.part_off);
  if (long_needs_reduce<R>(P.ksl, TA.n, h_out)) {
    const hipError_t e = launch_reduce<R>(st, v_long, TA, L, ws, kReduceLong);
    if (e != hipSuccess) return e;
    return launch_expand_long<DT, R>(st, y, ld_y, v_long, 0, 1, TB, h_out, scale);
  }
  if (P.ksl > 1) return launch_expand_long<DT, R>(st, y, ld_y, part, L.slice, P.ksl, TB, h_out, scale);
  return launch_expand_long<DT, R>(st, y, ld_y, v_long, 0, 1, TB, h_out, scale);
}

template <int DT, int R>
hipError_t run_long_chain(hipStream_t st, uint16_t* y, int64_t ld_y, const uint16_t* x,
                          int64_t ld_x, const Tables& TA, const Tables& TB, int32_t h_in,
                          int32_t h_out, float scale, const WsLayout& L, char* ws) {
  const Plan P = make_plan<R>(TA, h_in, L);
  float* v_long = reinterpret_cast<float*>(ws + L.v_off);
  const hipError_t e = launch_shrink_long<DT, R>(st, x, ld_x, TA, h_in, L, ws, v_long, P);
  if (e != hipSuccess) return e;
  return run_long_tail<DT, R>(st, y, ld_y, TA, TB, h_out, scale, L, ws, P);
}

// Where the short chain starts under capture.  Started with the long chain, the GEMV
// shrink (which reads every short segment's A) competes with the long shrink for memory;
// forked after the long shrink, it overlaps the long chain's reduce and expand instead.
// Measured on MI355X (70B mixed batch, graph replay), the later start wins only at r = 64
// with h_in > h_out and a wide expand (down projection 116 -> 107 us); elsewhere the
// early start is as fast or faster (r = 64 k/v 48 vs 52 us, r = 16 down 71 vs 75 us).
inline bool short_after_long_shrink(int r, int32_t h_in, int32_t h_out) {
  return r == 64 && h_in > h_out && h_out >= 4096;
}

// first error of a sequence of steps
inline hipError_t first_error(std::initializer_list<hipError_t> es) {
  for (hipError_t e : es)
    if (e != hipSuccess) return e;
  return hipSuccess;
}

template <int DT, int R>
hipError_t run_lora_add(hipStream_t st, uint16_t* y, int64_t ld_y, const uint16_t* x, int64_t ld_x,
                        const Tables& TA, const Tables& TB, int32_t h_in, int32_t h_out, float scale,
                        const WsLayout& L, char* ws) {
  const bool both = TA.use_gemv() && TA.use_long();
  if (!both) {
    if (TA.use_gemv())
      return run_short_chain<DT, R>(st, y, ld_y, x, ld_x, TA, TB, h_in, h_out, scale, L, ws);
    return run_long_chain<DT, R>(st, y, ld_y, x, ld_x, TA, TB, h_in, h_out, scale, L, ws);
  }
  const Plan P = make_plan<R>(TA, h_in, L);
  float* v_long = reinterpret_cast<float*>(ws + L.v_off);
  if (short_after_long_shrink(R, h_in, h_out) && SideStream::ready(st)) {
    // the long shrink first; the short chain, forked after it, overlaps the long chain's
    // reduce and expand instead of competing with its shrink
    hipError_t e = launch_shrink_long<DT, R>(st, x, ld_x, TA, h_in, L, ws, v_long, P);
    if (e != hipSuccess) return e;
    SideStream side;
    e = side.fork(st, 1);
    const hipStream_t ss = (e == hipSuccess && side.count() > 0) ? side.stream(0) : st;
    const hipError_t e1 =
        run_short_chain<DT, R>(ss, y, ld_y, x, ld_x, TA, TB, h_in, h_out, scale, L, ws);
    const hipError_t e2 = run_long_tail<DT, R>(st, y, ld_y, TA, TB, h_out, scale, L, ws, P);
    const hipError_t e3 = side.join(st);
    return first_error({e, e1, e2, e3});
  }
  SideStream side;
  hipError_t e = side.fork(st, 1);
  if (e != hipSuccess) return first_error({e, side.join(st)});
  if (side.count() > 0) {
    e = run_short_chain<DT, R>(side.stream(0), y, ld_y, x, ld_x, TA, TB, h_in, h_out, scale, L, ws);
    const hipError_t e2 =
        run_long_chain<DT, R>(st, y, ld_y, x, ld_x, TA, TB, h_in, h_out, scale, L, ws);
    const hipError_t e3 = side.join(st);
    return first_error({e, e2, e3});
  }
  if ((e = side.join(st)) != hipSuccess) return e;
  // both chains on the caller's stream: one reduce_v_kernel pass for all rows if either
  // kind needs one
  const float* part = reinterpret_cast<const float*>(ws + L.part_off);
  if ((e = launch_shrink_short<DT, R>(st, x, ld_x, TA, h_in, L, ws, P)) != hipSuccess) return e;
  if ((e = launch_shrink_long<DT, R>(st, x, ld_x, TA, h_in, L, ws, v_long, P)) != hipSuccess)
    return e;
  if (long_needs_reduce<R>(P.ksl, TA.n, h_out) || P.ksg > 16) {
    if ((e = launch_reduce<R>(st, v_long, TA, L, ws, kReduceAll)) != hipSuccess) return e;
    if ((e = launch_expand_short<DT, R>(st, y, ld_y, v_long, 0, 1, TB, h_out, scale)) != hipSuccess)
      return e;
    return launch_expand_long<DT, R>(st, y, ld_y, v_long, 0, 1, TB, h_out, scale);
  }
  if ((e = launch_expand_short<DT, R>(st, y, ld_y, part, L.slice, P.ksg, TB, h_out, scale)) != hipSuccess)
    return e;
  if (P.ksl > 1) return launch_expand_long<DT, R>(st, y, ld_y, part, L.slice, P.ksl, TB, h_out, scale);
  return launch_expand_long<DT, R>(st, y, ld_y, v_long, 0, 1, TB, h_out, scale);
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
  static hipError_t run(A... a) { return run_expand<DT, R>(a...); }
};
template <int DT, int R>
struct ShortChainOp {
  template <typename... A>
  static hipError_t run(A... a) { return run_short_chain<DT, R>(a...); }
};
template <int DT, int R>
struct LongChainOp {
  template <typename... A>
  static hipError_t run(A... a) { return run_long_chain<DT, R>(a...); }
};
template <int DT, int R>
struct LoraOp {
  template <typename... A>
  static hipError_t run(A... a) { return run_lora_add<DT, R>(a...); }
};


}  // namespace

namespace sgmv_host {

hipError_t table_lora_add_device(hipStream_t st, int32_t dtype, int32_t r, void* y, int64_t ld_y,
                                 const void* x, int64_t ld_x, const void* const* A_ptrs,
                                 const void* const* B_ptrs, const int32_t* seg_starts,
                                 const int32_t* perm, const int32_t* meta, int32_t n,
                                 int32_t S_max, int32_t h_in, int32_t h_out, float scale,
                                 void* workspace) {
  const WsLayout L = ws_layout(n, h_in, r);
  Tables TA{reinterpret_cast<const uint16_t* const*>(A_ptrs), seg_starts, perm, n, S_max, 1, n};
  Tables TB{reinterpret_cast<const uint16_t* const*>(B_ptrs), seg_starts, perm, n, S_max, 1, n};
  TA.meta = meta;
  TB.meta = meta;
  return dispatch<LoraOp>(dtype, r, st, static_cast<uint16_t*>(y), ld_y,
                          static_cast<const uint16_t*>(x), ld_x, TA, TB, h_in, h_out, scale, L,
                          static_cast<char*>(workspace));
}

}  // namespace sgmv_host

extern "C" int sgmv_check_workspace(hipStream_t stream, void* workspace, int32_t* flags,
                                    int32_t clear) {
  if (!workspace) return SGMV_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SGMV_ERR_WORKSPACE;
  int st = check_device();
  if (st) return st;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return SGMV_ERR_HIP;  // a read-back cannot be captured
  int32_t f = 0;
  if (hipMemcpyAsync(&f, workspace, sizeof(f), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SGMV_ERR_HIP;
  if (clear && f != 0) {
    const int32_t zero = 0;
    if (hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return SGMV_ERR_HIP;
  }
  if (flags) *flags = f;
  return f != 0 ? SGMV_ERR_DEVICE : SGMV_OK;
}

extern "C" int sgmv_upload_adapter(hipStream_t stream, void* A_pool, int64_t A_stride,
                                   void* B_pool, int64_t B_stride, int32_t slot,
                                   int32_t n_slots, const void* A_host, const void* B_host,
                                   int32_t r, int32_t h_in, int32_t h_out) {
  if (!rank_ok(r)) return SGMV_ERR_UNSUPPORTED;
  int st;
  if ((st = check_dim(h_in, h_in)) || (st = check_dim(h_out, h_out))) return st;
  if (n_slots <= 0 || slot < 0 || slot >= n_slots) return SGMV_ERR_SHAPE;
  if (A_stride < static_cast<int64_t>(r) * h_in || B_stride < static_cast<int64_t>(h_out) * r)
    return SGMV_ERR_SHAPE;
  if (A_stride % 8 != 0 || B_stride % 8 != 0) return SGMV_ERR_ALIGNMENT;
  if (!A_pool || !B_pool || !A_host || !B_host) return SGMV_ERR_NULL;
  if (!aligned16(A_pool) || !aligned16(B_pool)) return SGMV_ERR_ALIGNMENT;
  if ((st = check_device())) return st;
  const size_t a_bytes = 2 * static_cast<size_t>(r) * h_in, b_bytes = 2 * static_cast<size_t>(r) * h_out;
  char* a_dst = static_cast<char*>(A_pool) + 2 * static_cast<size_t>(slot) * A_stride;
  char* b_dst = static_cast<char*>(B_pool) + 2 * static_cast<size_t>(slot) * B_stride;
  if (hipMemcpyAsync(a_dst, A_host, a_bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipMemcpyAsync(b_dst, B_host, b_bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
    return SGMV_ERR_HIP;
  return SGMV_OK;
}

extern "C" size_t sgmv_workspace_bytes(int32_t n, int32_t h_in, int32_t r) {
  if (n < 0 || h_in < 8 || h_in > kMaxDim || !rank_ok(r)) return 0;
  return ws_layout(n, h_in, r).total;
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
  Tables T{reinterpret_cast<const uint16_t* const*>(A_ptrs), seg_starts, perm, n,
           n_segments, min_seg_len, max_seg_len};
  T.flag = static_cast<int32_t*>(workspace);
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
  return hip_status(dispatch<ExpandOp>(dtype, r, stream, static_cast<uint16_t*>(y), ld_y, v, T,
                                       h_out, scale));
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
  Tables TA{reinterpret_cast<const uint16_t* const*>(A_ptrs), seg_starts, perm, n,
            n_segments, min_seg_len, max_seg_len};
  TA.flag = static_cast<int32_t*>(workspace);
  const Tables TB{reinterpret_cast<const uint16_t* const*>(B_ptrs), seg_starts, perm, n,
                  n_segments, min_seg_len, max_seg_len};
  return hip_status(dispatch<LoraOp>(dtype, r, stream, static_cast<uint16_t*>(y), ld_y,
                                     static_cast<const uint16_t*>(x), ld_x, TA, TB, h_in, h_out,
                                     scale, L, static_cast<char*>(workspace)));
}

// Mixed ranks: each rank group runs as sgmv_lora_add on its slice of the tables (pointer
// offsets only), one group after another on the caller's stream.
extern "C" int sgmv_lora_add_ranked(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y,
                                    const void* x, int64_t ld_x, const void* const* A_ptrs,
                                    const void* const* B_ptrs, const int32_t* seg_starts,
                                    const int32_t* perm, int32_t n, const sgmv_rank_group* groups,
                                    int32_t n_groups, int32_t h_in, int32_t h_out, void* workspace,
                                    size_t workspace_bytes) {
  if (dtype != SGMV_F16 && dtype != SGMV_BF16) return SGMV_ERR_UNSUPPORTED;
  if (n < 0 || n_groups < 0) return SGMV_ERR_SHAPE;
  if (n_groups > 0 && !groups) return SGMV_ERR_NULL;
  int st;
  if ((st = check_dim(h_in, ld_x))) return st;
  if ((st = check_dim(h_out, ld_y))) return st;
  int32_t r_max = 0;
  for (int32_t g = 0; g < n_groups; ++g) {
    const sgmv_rank_group& G = groups[g];
    if (!rank_ok(G.r)) return SGMV_ERR_UNSUPPORTED;
    if ((st = check_segments(G.n, G.n_segments, G.min_seg_len, G.max_seg_len))) return st;
    if (G.row0 < 0 || G.seg0 < 0 || G.starts0 < 0 || static_cast<int64_t>(G.row0) + G.n > n)
      return SGMV_ERR_SHAPE;
    if (G.n > 0) r_max = std::max(r_max, G.r);
  }
  if (n == 0 || r_max == 0) return SGMV_OK;
  // the buffer the header asks for: room for a call of all n rows at the largest rank
  const WsLayout L_all = ws_layout(n, h_in, r_max);
  const size_t ws_need = L_all.total;
  if (!y || !x || !A_ptrs || !B_ptrs || !seg_starts || !perm) return SGMV_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return SGMV_ERR_ALIGNMENT;
  if (ranges_overlap(x, matrix_bytes(n, ld_x, h_in), y, matrix_bytes(n, ld_y, h_out)))
    return SGMV_ERR_ALIAS;
  if (!workspace || workspace_bytes < ws_need ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SGMV_ERR_WORKSPACE;
  if ((st = check_device())) return st;
  auto tables = [&](const sgmv_rank_group& G, const void* const* P) {
    Tables T{reinterpret_cast<const uint16_t* const*>(P) + G.seg0, seg_starts + G.starts0,
             perm + G.row0, G.n, G.n_segments, G.min_seg_len, G.max_seg_len, nullptr, true};
    T.flag = static_cast<int32_t*>(workspace);
    T.y_rows = n;
    return T;
  };
  // The groups touch disjoint rows.  Under graph capture, with room for every group's
  // scratch side by side in the workspace, each group's short and long chains run on
  // streams of their own and all of them overlap; otherwise the groups run one after
  // another (each as sgmv_lora_add, whose own chains overlap under capture).
  int chains = 0;
  std::vector<int32_t> gn(n_groups), gr(n_groups);
  std::vector<size_t> goff(n_groups);
  for (int32_t g = 0; g < n_groups; ++g) {
    const sgmv_rank_group& G = groups[g];
    gn[g] = G.n;
    gr[g] = G.r;
    if (G.n > 0) chains += (G.min_seg_len < kLongMin) + (G.max_seg_len >= kLongMin);
  }
  // Side by side, the groups' scratch must end where the scratch of one call of all n rows
  // at the largest rank would: then, like that call, it stays clear of the counters and
  // tagged partials of every call the buffer is sized for.
  const bool fits =
      ranked_side_by_side(gn.data(), gr.data(), n_groups, h_in, goff.data()) <= L_all.table_end;
  SideStream side;
  if (fits && chains > 1) {
    if (side.fork(stream, chains - 1) != hipSuccess) {
      (void)side.join(stream);
      return SGMV_ERR_HIP;
    }
  }
  if (side.count() > 0) {
    hipError_t e = hipSuccess;
    int k = 0;
    for (int32_t g = 0; g < n_groups; ++g) {
      const sgmv_rank_group& G = groups[g];
      if (G.n == 0) continue;
      const Tables TA = tables(G, A_ptrs), TB = tables(G, B_ptrs);
      const WsLayout L = ws_layout(G.n, h_in, G.r);
      char* ws = static_cast<char*>(workspace) + goff[g];
      const bool kinds[2] = {TA.min_len < kLongMin, TA.max_len >= kLongMin};
      for (int c = 0; c < 2; ++c) {
        if (!kinds[c]) continue;
        const hipStream_t s = (k == 0) ? stream : side.stream(k - 1);
        ++k;
        const hipError_t ec =
            c == 0 ? dispatch<ShortChainOp>(dtype, G.r, s, static_cast<uint16_t*>(y), ld_y,
                                            static_cast<const uint16_t*>(x), ld_x, TA, TB, h_in,
                                            h_out, G.scale, L, ws)
                   : dispatch<LongChainOp>(dtype, G.r, s, static_cast<uint16_t*>(y), ld_y,
                                           static_cast<const uint16_t*>(x), ld_x, TA, TB, h_in,
                                           h_out, G.scale, L, ws);
        if (e == hipSuccess) e = ec;
      }
    }
    const hipError_t ej = side.join(stream);
    return (e == hipSuccess && ej == hipSuccess) ? SGMV_OK : SGMV_ERR_HIP;
  }
  if (side.join(stream) != hipSuccess) return SGMV_ERR_HIP;
  for (int32_t g = 0; g < n_groups; ++g) {
    const sgmv_rank_group& G = groups[g];
    if (G.n == 0) continue;
    const WsLayout L = ws_layout(G.n, h_in, G.r);
    const hipError_t e = dispatch<LoraOp>(dtype, G.r, stream, static_cast<uint16_t*>(y), ld_y,
                                          static_cast<const uint16_t*>(x), ld_x,
                                          tables(G, A_ptrs), tables(G, B_ptrs), h_in, h_out,
                                          G.scale, L, static_cast<char*>(workspace));
    if (e != hipSuccess) return SGMV_ERR_HIP;
  }
  return SGMV_OK;
}
