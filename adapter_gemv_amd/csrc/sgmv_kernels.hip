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
// long-segment path (segments with >= kLongMin rows)
// ------------------------------------------------------------------------------------
constexpr int kCounterStride = kCounterInts;  // one tile counter per 256-byte line

__device__ inline void store_coherent(float* q, float v) {
  __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_coherent(const float* q) {
  return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Segments that cover the sorted rows [r0, r1) (at most 32 rows), found in one parallel
// pass over seg_starts: the segment of row r0, the rows inside the tile where a new
// segment starts, and the nearest segment starts on either side.
struct TileSegs {
  int seg0;        // segment of row r0
  uint32_t bound;  // bit q (q >= 1): a segment starts at row r0 + q
  int prev;        // first row of segment seg0
  int next;        // first segment start >= r1 (n if none)
};

struct TileSegsLds {
  int count, prev, next;
  unsigned bound;
};

__device__ inline TileSegs tile_segments(const int32_t* __restrict__ seg_starts, int S, int n,
                                         int r0, int r1, TileSegsLds* sh) {
  if (threadIdx.x == 0) {
    sh->count = 0;
    sh->prev = 0;
    sh->next = n;
    sh->bound = 0u;
  }
  __syncthreads();
  for (int s = 1 + static_cast<int>(threadIdx.x); s <= S; s += blockDim.x) {
    const int st = seg_starts[s];
    if (st <= r0) {
      atomicAdd(&sh->count, 1);
      atomicMax(&sh->prev, st);
    } else if (st < r1) {
      atomicOr(&sh->bound, 1u << (st - r0));
    } else {
      atomicMin(&sh->next, st);
    }
  }
  __syncthreads();
  TileSegs t;
  t.seg0 = sh->count;
  t.bound = sh->bound;
  t.prev = sh->prev;
  t.next = sh->next;
  return t;
}

// Run k of a tile: rows [lo, hi) of segment seg; `len` is the segment's full length.
struct Run {
  int seg, lo, hi, len;
};

// Iterates the runs of a tile in order; uniform across the block.
struct RunIter {
  TileSegs T;
  int r0, r1;
  int seg, lo, start;
  __device__ RunIter(const TileSegs& t, int r0_, int r1_)
      : T(t), r0(r0_), r1(r1_), seg(t.seg0), lo(r0_), start(t.prev) {}
  __device__ bool next(Run* run) {
    if (lo >= r1) return false;
    const uint32_t later = (lo - r0 + 1 < 32) ? (T.bound >> (lo - r0 + 1)) : 0u;
    const int hi = later ? lo + 1 + (__ffs(later) - 1) : r1;
    const int end = later ? hi : T.next;  // first row after the segment
    run->seg = seg;
    run->lo = lo;
    run->hi = hi;
    run->len = end - start;
    ++seg;
    start = hi;
    lo = hi;
    return true;
  }
};

// rows of long segments inside the tile (bit q: row r0 + q)
__device__ inline uint32_t long_rows(const TileSegs& T, int r0, int r1) {
  uint32_t mask = 0;
  RunIter it(T, r0, r1);
  Run run;
  while (it.next(&run))
    if (run.len >= kLongMin) {
      const int w = run.hi - run.lo;
      mask |= ((w >= 32) ? 0xffffffffu : ((1u << w) - 1u)) << (run.lo - r0);
    }
  return mask;
}

// Shrink on MFMA 16x16x32 for a tile of 16 sorted rows and a K chunk, with 16 waves per
// workgroup.  The x tile is the A operand and the adapter's stored A rows the B operand;
// lane l supplies row/column l%16 and k = k0 + 8*(l/16) .. +7 of each 32-wide k step, so
// the four lanes of a row read 64 contiguous bytes per load.  The chunk is cut into
// stages of 2048/r k dealt round-robin to the waves; each wave keeps the loads of its next
// stage in flight while it multiplies the current one.  The 16 wave results are added
// in a fixed order through LDS.  With one chunk per tile v is written directly;
// otherwise chunks go out as agent-scope atomic stores and the last chunk of the tile
// (per a counter on its own cache line) adds them in order, writes v and resets the
// counter.
template <int R>
struct ShrinkMfmaCfg {
  static constexpr int NB = R / 16;
  static constexpr int UN = 64 / R;         // MFMA k-steps per stage (4 loads of A per lane)
  static constexpr int STAGE = 32 * UN;     // k per stage
  static constexpr int WAVES = 16;
};

template <int DT, int R>
__device__ inline void mfma_stage_load(const uint16_t* xr, const uint16_t* A, int h_in, int k0,
                                       int k_end, int mrow, int kq, uint4 (&xv)[ShrinkMfmaCfg<R>::UN],
                                       uint4 (&av)[R / 16][ShrinkMfmaCfg<R>::UN]) {
  constexpr int UN = ShrinkMfmaCfg<R>::UN;
#pragma unroll
  for (int u = 0; u < UN; ++u) {
    const int kk = k0 + 32 * u + 8 * kq;
    const bool in = kk < k_end;
    xv[u] = (in && xr) ? ld16(xr + kk) : zero4();
#pragma unroll
    for (int nb = 0; nb < R / 16; ++nb)
      av[nb][u] = in ? ld16(A + static_cast<int64_t>(nb * 16 + mrow) * h_in + kk) : zero4();
  }
}

template <int DT, int R>
__device__ inline void mfma_stage_mul(const uint4 (&xv)[ShrinkMfmaCfg<R>::UN],
                                      const uint4 (&av)[R / 16][ShrinkMfmaCfg<R>::UN],
                                      f32x4_t (&acc)[R / 16]) {
#pragma unroll
  for (int u = 0; u < ShrinkMfmaCfg<R>::UN; ++u)
#pragma unroll
    for (int nb = 0; nb < R / 16; ++nb) acc[nb] = Elem<DT>::mfma(xv[u], av[nb][u], acc[nb]);
}

template <int DT, int R>
__global__ __launch_bounds__(1024) void shrink_mfma_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* const* __restrict__ A_ptrs,
    const int32_t* __restrict__ seg_starts, int32_t S, const int32_t* __restrict__ perm, int32_t n,
    int32_t h_in, int32_t kcm, float* __restrict__ part, int64_t slice, int32_t* __restrict__ tile_cnt,
    float* __restrict__ v_out, int32_t* __restrict__ rowks, int32_t ks) {
  using C = ShrinkMfmaCfg<R>;
  constexpr int NB = C::NB, UN = C::UN, STAGE = C::STAGE, WAVES = C::WAVES;
  __shared__ TileSegsLds s_segs;
  __shared__ int s_last;
  __shared__ f32x4_t red[WAVES / 2][NB][64];
  const int r0 = blockIdx.x * kTileRows;
  const int r1 = min(n, r0 + kTileRows);
  const int kc = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int mrow = lane & 15, kq = lane >> 4;
  const int i = r0 + mrow;
  const int prow = (i < r1) ? (perm ? perm[i] : i) : 0;  // issued with the segment pass
  const TileSegs T = tile_segments(seg_starts, S, n, r0, r1, &s_segs);
  const uint32_t lmask = long_rows(T, r0, r1);
  if (lmask == 0) return;  // uniform: no row of a long segment here
  const int k_lo = kc * kcm;
  const int k_hi = min(h_in, k_lo + kcm);
  const int nst = (k_hi - k_lo + STAGE - 1) / STAGE;

  RunIter it(T, r0, r1);
  Run run;
  while (it.next(&run)) {
    if (run.len < kLongMin) continue;  // uniform across the block
    const uint16_t* xr = (i >= run.lo && i < run.hi) ? x + static_cast<int64_t>(prow) * ld_x : nullptr;
    const uint16_t* A = A_ptrs[run.seg];
    f32x4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 x0[UN], a0[NB][UN], x1[UN], a1[NB][UN];
    mfma_stage_load<DT, R>(xr, A, h_in, k_lo + w * STAGE, k_hi, mrow, kq, x0, a0);
    for (int g = w; g < nst; g += 2 * WAVES) {
      mfma_stage_load<DT, R>(xr, A, h_in, k_lo + (g + WAVES) * STAGE, k_hi, mrow, kq, x1, a1);
      mfma_stage_mul<DT, R>(x0, a0, acc);
      mfma_stage_load<DT, R>(xr, A, h_in, k_lo + (g + 2 * WAVES) * STAGE, k_hi, mrow, kq, x0, a0);
      mfma_stage_mul<DT, R>(x1, a1, acc);
    }
    // fixed-order sum over the 16 waves: w + 8 into w, then slots 0..7 in order
    if (w >= WAVES / 2) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[w - WAVES / 2][nb][lane] = acc[nb];
    }
    __syncthreads();
    if (w < WAVES / 2) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[w][nb][lane] = acc[nb] + red[w][nb][lane];
    }
    __syncthreads();
    if (tid < NB * 256) {
      const int nb = tid >> 8, l = (tid >> 2) & 63, c = tid & 3;
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < WAVES / 2; ++q) sum += red[q][nb][l][c];
      const int row = r0 + 4 * (l >> 4) + c;
      const int jj = nb * 16 + (l & 15);
      if (row >= run.lo && row < run.hi) {
        if (ks == 1)
          v_out[static_cast<int64_t>(row) * R + jj] = sum;
        else
          store_coherent(part + kc * slice + static_cast<int64_t>(row) * R + jj, sum);
      }
    }
    __syncthreads();
  }
  if (kc == 0)
    for (int q = tid; q < r1 - r0; q += blockDim.x)
      if ((lmask >> q) & 1u) rowks[r0 + q] = 0;  // v of long rows is final, not in slices
  if (ks == 1) return;

  // publish this chunk, then let the last chunk of the tile reduce and write v
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&tile_cnt[blockIdx.x * kCounterStride], 1,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == ks - 1);
    if (s_last) __hip_atomic_store(&tile_cnt[blockIdx.x * kCounterStride], 0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  for (int idx = tid; idx < (r1 - r0) * R; idx += blockDim.x) {
    const int q = idx / R;
    if (!((lmask >> q) & 1u)) continue;
    const float* src = part + static_cast<int64_t>(r0) * R + idx;
    float acc = 0.f;
    for (int k0 = 0; k0 < ks; k0 += 8) {
      float v8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v8[u] = (k0 + u < ks) ? load_coherent(src + (k0 + u) * slice) : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v8[u];
    }
    v_out[static_cast<int64_t>(r0) * R + idx] = acc;
  }
}

// Expand on MFMA 16x16x32 for a tile of 32 sorted rows and 256 columns, computed
// transposed: D[col, row] = sum_k Bk[col, k] * Vk[k, row], where the k dimension is 2r:
// the stored rows of B[a] twice (A operand) against scale * v split into two 16-bit
// halves, hi = round(scale*v) and lo = round(scale*v - hi) (B operand).  The products are
// exact and summed in float32; hi + lo carries 16 (bf16) or 22 (fp16) significant bits of
// scale*v.  The float32 sums go through LDS so that y is read and written with whole
// 16-byte vectors (16 lanes per 256-column row): y is loaded as soon as the caller rows
// are known, then updated as y + sum in float32 and rounded once.
//
// Workgroup b runs on XCD b % 8 (round-robin dispatch).  Each XCD owns a contiguous range
// of column strips, so its L2 holds only that part of every B[a]; within the range the
// workgroups go row tile by row tile, so the y traffic in flight at any time covers whole
// rows of a few consecutive tiles.
constexpr int kExpRows = 32;
constexpr int kExpCols = 256;
constexpr int kExpPad = 4;       // floats of padding per LDS row of the sums
constexpr int kExpMaxSegs = 4;   // long segments that can overlap 32 rows: 32/16 + 2
constexpr int kXcds = 8;

// waves per SIMD the register budget is set for: 4 workgroups per CU for r = 16, fewer for
// the larger B fragments of r = 32 and 64
template <int R>
constexpr int expand_waves() { return R == 16 ? 4 : (R == 32 ? 3 : 2); }

template <int DT, int R>
__global__ __launch_bounds__(256, expand_waves<R>()) void expand_mfma_kernel(
    uint16_t* __restrict__ y, int64_t ld_y, const float* __restrict__ v,
    const uint16_t* const* __restrict__ B_ptrs, const int32_t* __restrict__ seg_starts, int32_t S,
    const int32_t* __restrict__ perm, int32_t n, int32_t h_out, float scale, int32_t tiles,
    int32_t strips) {
  using E = Elem<DT>;
  constexpr int TR = kExpRows, TC = kExpCols;
  constexpr int KT = 2 * R;          // k of the hi/lo product
  constexpr int NK = KT / 32;        // MFMA k-steps
  constexpr int VPT = TR * R / 256;  // v values per thread
  constexpr int YPT = TR * TC / 8 / 256;  // 16-byte vectors of y per thread
  __shared__ int s_nseg;
  __shared__ int s_seg[kExpMaxSegs], s_st[kExpMaxSegs], s_en[kExpMaxSegs];
  __shared__ int s_rseg[TR];  // long segment of each tile row, -1 otherwise
  __shared__ int s_prow[TR];  // caller row of each tile row
  __shared__ __attribute__((aligned(16))) uint16_t vlds[TR][KT];
  __shared__ __attribute__((aligned(16))) float dl[TR][TC + kExpPad];

  // XCD x owns strips [sx0, sx1) and walks them tile-major
  const int b = blockIdx.x;
  const int xcd = b % kXcds, jx = b / kXcds;
  const int sper = strips / kXcds, srem = strips % kXcds;
  const int sx0 = xcd * sper + min(xcd, srem);
  const int nsx = sper + (xcd < srem ? 1 : 0);
  if (nsx == 0 || jx >= nsx * tiles) return;
  const int tile = jx / nsx, strip = sx0 + jx % nsx;
  const int c0 = strip * TC;
  const int g0 = tile * TR;
  const int g1 = min(n, g0 + TR);
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int kq = lane >> 4, l16 = lane & 15;

  // caller rows first, so that y is in flight while the segments are found
  if (tid == 0) s_nseg = 0;
  if (tid < TR) s_prow[tid] = (g0 + tid < g1) ? (perm ? perm[g0 + tid] : g0 + tid) : -1;
  __syncthreads();
  // y: thread vector e = tid + 256u covers row e / 32, columns c0 + 8 * (e % 32) .. +7
  uint4 yv[YPT];
#pragma unroll
  for (int u = 0; u < YPT; ++u) {
    const int e = tid + 256 * u, q = e / (TC / 8), col = c0 + 8 * (e % (TC / 8));
    const int prow = s_prow[q];
    yv[u] = (prow >= 0 && col < h_out) ? ld16(y + static_cast<int64_t>(prow) * ld_y + col) : zero4();
  }
  float vv[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int idx = tid + 256 * u;
    vv[u] = (g0 + idx / R < g1) ? v[static_cast<int64_t>(g0) * R + idx] : 0.f;
  }
  // long segments overlapping the tile
  for (int s = tid; s < S; s += 256) {
    const int st = seg_starts[s], en = seg_starts[s + 1];
    if (en - st >= kLongMin && st < g1 && en > g0) {
      const int k = atomicAdd(&s_nseg, 1);
      if (k < kExpMaxSegs) {
        s_seg[k] = s;
        s_st[k] = st;
        s_en[k] = en;
      }
    }
  }
  __syncthreads();
  const int nseg = min(s_nseg, kExpMaxSegs);
  if (nseg == 0) return;  // uniform
  if (tid < TR) {
    const int row = g0 + tid;
    int sg = -1;
    for (int k = 0; k < nseg; ++k)
      if (s_st[k] <= row && row < s_en[k]) sg = s_seg[k];
    s_rseg[tid] = sg;
  }
  __syncthreads();

#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int idx = tid + 256 * u;
    const float val = (s_rseg[idx / R] >= 0) ? scale * vv[u] : 0.f;
    const uint32_t hw = E::pack(val, 0.f) & 0xffffu;
    const uint32_t lw = E::pack(val - E::lo(hw), 0.f) & 0xffffu;
    vlds[idx / R][idx % R] = static_cast<uint16_t>(hw);
    vlds[idx / R][R + idx % R] = static_cast<uint16_t>(lw);
  }
  __syncthreads();

  int rs[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) rs[rb] = s_rseg[16 * rb + l16];
  f32x4_t acc[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the long segments of the tile, in increasing order (the reads are uniform)
  int q = 0;
  for (;;) {
    while (q < TR && s_rseg[q] < 0) ++q;
    if (q >= TR) break;
    const int sg = s_rseg[q];
    while (q < TR && s_rseg[q] == sg) ++q;
    const uint16_t* B = B_ptrs[sg];
    uint4 bop[4][NK];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = c0 + 64 * w + 16 * cb + l16;
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        const int j0 = (32 * s + 8 * kq) % R;
        bop[cb][s] = (col < h_out) ? ld16(B + static_cast<int64_t>(col) * R + j0) : zero4();
      }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int lq = 16 * rb + l16;
      uint4 vop[NK];
#pragma unroll
      for (int s = 0; s < NK; ++s)
        vop[s] = (rs[rb] == sg) ? *reinterpret_cast<const uint4*>(&vlds[lq][32 * s + 8 * kq]) : zero4();
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int s = 0; s < NK; ++s) acc[rb][cb] = E::mfma(bop[cb][s], vop[s], acc[rb][cb]);
    }
  }
  // lane: D rows 4*kq .. +3 of column block cb = tile columns 64w + 16cb + 4kq .. +3,
  // D column l16 = tile row 16rb + l16
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      *reinterpret_cast<f32x4_t*>(&dl[16 * rb + l16][64 * w + 16 * cb + 4 * kq]) = acc[rb][cb];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < YPT; ++u) {
    const int e = tid + 256 * u, q2 = e / (TC / 8), cc = 8 * (e % (TC / 8)), col = c0 + cc;
    if (s_rseg[q2] < 0 || col >= h_out) continue;
    const f32x4_t d0 = *reinterpret_cast<const f32x4_t*>(&dl[q2][cc]);
    const f32x4_t d1 = *reinterpret_cast<const f32x4_t*>(&dl[q2][cc + 4]);
    uint4 o;
    o.x = E::pack(E::lo(yv[u].x) + d0[0], E::hi(yv[u].x) + d0[1]);
    o.y = E::pack(E::lo(yv[u].y) + d0[2], E::hi(yv[u].y) + d0[3]);
    o.z = E::pack(E::lo(yv[u].z) + d1[0], E::hi(yv[u].z) + d1[1]);
    o.w = E::pack(E::lo(yv[u].w) + d1[2], E::hi(yv[u].w) + d1[3]);
    *reinterpret_cast<uint4*>(y + static_cast<int64_t>(s_prow[q2]) * ld_y + col) = o;
  }
}

// v[i, :] = sum of the split-K slices of sorted row i, in slice order, for rows whose
// slice count is nonzero (rows of long segments already have their final v).
template <int R>
__global__ __launch_bounds__(256) void reduce_v_kernel(float* __restrict__ v,
                                                      const float* __restrict__ part, int64_t slice,
                                                      const int32_t* __restrict__ rowks, int32_t n,
                                                      int32_t ks_max) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(n) * R) return;
  const int row = static_cast<int>(idx / R);
  const int ks = min(rowks[row], ks_max);
  if (ks > 0) v[idx] = sum_slices(part + idx, slice, ks);
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

// split-K chunk of the MFMA shrink: about 256 workgroups in all (one per CU), at most 8
// chunks per tile, each a multiple of 128 k (a whole number of stages for every rank)
inline int mfma_kcm(int32_t n, int32_t h_in, int32_t r) {
  (void)r;
  const int stage = ShrinkMfmaCfg<16>::STAGE;
  const int tiles = (n + kTileRows - 1) / kTileRows;
  int chunks = (256 + tiles - 1) / (tiles > 0 ? tiles : 1);
  if (chunks < 1) chunks = 1;
  if (chunks > 8) chunks = 8;
  const int stages = (h_in + stage - 1) / stage;
  if (chunks > stages) chunks = stages;
  return ((stages + chunks - 1) / chunks) * stage;
}

struct Tables {
  const uint16_t* const* ptrs;
  const int32_t* seg_starts;
  const int32_t* perm;
  int32_t n, S, min_len, max_len;
  bool use_gemv() const { return min_len < kLongMin; }
  bool use_long() const { return max_len >= kLongMin; }
};

// shrink kernels: short segments leave split-K slices (ks_gemv of them, counted in rowks),
// long segments leave their final v in v_long
template <int DT, int R>
hipError_t launch_shrink(hipStream_t st, const uint16_t* x, int64_t ld_x, const Tables& T,
                         int32_t h_in, const WsLayout& L, char* ws, float* v_long, int* ks_gemv) {
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  int32_t* rowks = reinterpret_cast<int32_t*>(ws + L.rowks_off);
  *ks_gemv = 0;
  if (T.use_gemv()) {
    const int ks = (h_in + GemvCfg<R>::KC - 1) / GemvCfg<R>::KC;
    *ks_gemv = ks;
    hipLaunchKernelGGL((shrink_gemv_kernel<DT, R>), dim3(T.S, ks), dim3(256), 0, st, x, ld_x,
                       T.ptrs, T.seg_starts, T.perm, h_in, part, L.slice, rowks, ks);
  }
  if (T.use_long()) {
    const int kcm = mfma_kcm(T.n, h_in, R);
    const int ks = (h_in + kcm - 1) / kcm;
    const int tiles = (T.n + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL((shrink_mfma_kernel<DT, R>), dim3(tiles, ks), dim3(1024), 0, st, x, ld_x,
                       T.ptrs, T.seg_starts, T.S, T.perm, T.n, h_in, kcm, part, L.slice,
                       reinterpret_cast<int32_t*>(ws + L.tile_cnt_off), v_long, rowks, ks);
  }
  return hipGetLastError();
}

// expand kernels: short segments sum ks_gemv slices of vsrc (slice stride `slice`), long
// segments read their final v from v_long
template <int DT, int R>
hipError_t launch_expand(hipStream_t st, uint16_t* y, int64_t ld_y, const float* vsrc,
                         int64_t slice, int ks_gemv, const float* v_long, const Tables& T,
                         int32_t h_out, float scale) {
  constexpr int CPL = 128 / R;
  if (T.use_gemv()) {
    const int chunks = (h_out + 64 * CPL - 1) / (64 * CPL);
    hipLaunchKernelGGL((expand_gemv_kernel<DT, R>), dim3(T.S, chunks), dim3(64), 0, st, y, ld_y,
                       vsrc, slice, ks_gemv, T.ptrs, T.seg_starts, T.perm, h_out, scale);
  }
  if (T.use_long()) {
    // each XCD takes ceil(strips / 8) strips at most: pad the grid to 8 equal shares
    const int tiles = (T.n + kExpRows - 1) / kExpRows;
    const int strips = (h_out + kExpCols - 1) / kExpCols;
    const int64_t share = static_cast<int64_t>(tiles) * ((strips + kXcds - 1) / kXcds);
    if (share * kXcds > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((expand_mfma_kernel<DT, R>), dim3(static_cast<unsigned>(share * kXcds)),
                       dim3(256), 0, st, y, ld_y, v_long, T.ptrs, T.seg_starts, T.S, T.perm, T.n,
                       h_out, scale, tiles, strips);
  }
  return hipGetLastError();
}

template <int DT, int R>
hipError_t run_shrink(hipStream_t st, float* v, const uint16_t* x, int64_t ld_x, const Tables& T,
                      int32_t h_in, const WsLayout& L, char* ws) {
  int ksg;
  hipError_t e = launch_shrink<DT, R>(st, x, ld_x, T, h_in, L, ws, v, &ksg);
  if (e != hipSuccess) return e;
  if (!T.use_gemv()) return hipSuccess;
  const int64_t total = static_cast<int64_t>(T.n) * R;
  hipLaunchKernelGGL((reduce_v_kernel<R>), dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                     0, st, v, reinterpret_cast<const float*>(ws + L.part_off), L.slice,
                     reinterpret_cast<const int32_t*>(ws + L.rowks_off), T.n, L.ks_max);
  return hipGetLastError();
}

template <int DT, int R>
hipError_t run_expand(hipStream_t st, uint16_t* y, int64_t ld_y, const float* v, const Tables& T,
                      int32_t h_out, float scale) {
  return launch_expand<DT, R>(st, y, ld_y, v, 0, 1, v, T, h_out, scale);
}

template <int DT, int R>
hipError_t run_lora_add(hipStream_t st, uint16_t* y, int64_t ld_y, const uint16_t* x, int64_t ld_x,
                        const Tables& TA, const Tables& TB, int32_t h_in, int32_t h_out, float scale,
                        const WsLayout& L, char* ws) {
  int ksg;
  float* v_long = reinterpret_cast<float*>(ws + L.v_off);
  hipError_t e = launch_shrink<DT, R>(st, x, ld_x, TA, h_in, L, ws, v_long, &ksg);
  if (e != hipSuccess) return e;
  return launch_expand<DT, R>(st, y, ld_y, reinterpret_cast<const float*>(ws + L.part_off), L.slice,
                              ksg, v_long, TB, h_out, scale);
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
struct LoraOp {
  template <typename... A>
  static hipError_t run(A... a) { return run_lora_add<DT, R>(a...); }
};


}  // namespace

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
  const Tables TA{reinterpret_cast<const uint16_t* const*>(A_ptrs), seg_starts, perm, n,
                  n_segments, min_seg_len, max_seg_len};
  const Tables TB{reinterpret_cast<const uint16_t* const*>(B_ptrs), seg_starts, perm, n,
                  n_segments, min_seg_len, max_seg_len};
  return hip_status(dispatch<LoraOp>(dtype, r, stream, static_cast<uint16_t*>(y), ld_y,
                                     static_cast<const uint16_t*>(x), ld_x, TA, TB, h_in, h_out,
                                     scale, L, static_cast<char*>(workspace)));
}
