// libsgmv decode path for gfx950: one launch per SGMV call for batches of up to 64
// tokens whose adapters live in pools (A_pool[a], B_pool[a] at fixed strides) and
// whose adapter ids are already on the device.
//
// Everything the Punica pages put in one SGMV call happens inside this one kernel
// (paper summary on research.elamur.ai, "Summary" and "Interesting ideas" I1/I2):
//   * grouping by adapter: every workgroup loads the batch's ids (one coalesced load)
//     and finds the rows that share its adapter with one wavefront ballot -- the same
//     row sets, in the same caller order, as the stable sort's segments;
//   * shrink items (adapter rows within a block of 16 caller rows, K chunk) compute
//     float32 partial sums of v = x @ A[a] on MFMA 16x16x32 tiles and publish each one
//     with a nonzero tag in the same 64-bit agent-scope atomic store;
//   * expand items (caller row, column chunk) load their slice of B[a] and of y while
//     the shrink runs, poll the row's tagged partial sums until every one is present,
//     add them in a fixed order and write y = y + scale * v @ B[a] with one rounding.
// Items are ordered shrink-first in the grid (one wave per item).
// Workgroups are dispatched in index order within each XCD, so every shrink item a
// waiting expand item depends on has already been placed on a CU; shrink items never
// wait, hence the waits end (they are also bounded, and flag the workspace if the bound
// is hit).  The last expand item of a row (per a counter on its own 256-byte line) clears
// the row's partials and the counter, leaving the workspace ready for the next call
// without a memset (safe under HIP graph capture).  The device-side stable sort itself is
// available as sgmv_build_segments_device.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/sgmv.h"
#include "sgmv_checks.h"
#include "sgmv_device.h"

namespace {

using namespace sgmv_dev;
using namespace sgmv_host;

constexpr int kPoolMaxN = kMaxPoolRows;  // tokens per call on this path (one wavefront)
constexpr int kCounterStride = kCounterInts;  // one counter per 256-byte line (no sharing)
constexpr int kSpinLimit = 1 << 22;      // bounded wait (about 0.1 s), then flag and exit
constexpr int kItemsPerWg = 1;           // work items per workgroup (one per wave): more
                                         // workgroups spread the loads over more CUs
constexpr uint32_t kNoKey = 0xffffffffu;

// v of lane (lane ^ S), S in {1, 2, 4}: DPP quad permutations for 1 and 2, a swizzle
// (and-mask 31, xor-mask 4) for 4
template <int S>
__device__ inline uint32_t xor_lane(uint32_t v) {
  if constexpr (S == 1) return __builtin_amdgcn_mov_dpp(v, 0xb1, 0xf, 0xf, true);  // [1,0,3,2]
  if constexpr (S == 2) return __builtin_amdgcn_mov_dpp(v, 0x4e, 0xf, 0xf, true);  // [2,3,0,1]
  if constexpr (S == 4) return __builtin_amdgcn_ds_swizzle(v, 0x101f);
}

// an empty asm that takes v in a VGPR: everything that computes v is done before it
__device__ inline void pin(float& v) { asm volatile("" : "+v"(v)); }

// One stage of the transpose of B's words within groups of GC lanes.  bw holds the 16
// loads of a lane, four words each (load u in bw[4u .. 4u+3]); lanes q and q ^ S swap
// load GC*t + k (held by the lane whose bit S differs from k's) for every t and k.
template <int GC, int S>
__device__ inline void transpose_stage(uint32_t (&bw)[64], int q) {
  if constexpr (S < GC) {
    const bool hi = (q & S) != 0;
#pragma unroll
    for (int t = 0; t < 16 / GC; ++t)
#pragma unroll
      for (int k = 0; k < GC; ++k) {
        if (k & S) continue;
        const int lo_u = GC * t + k, hi_u = GC * t + (k | S);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t& a = bw[4 * lo_u + d];
          uint32_t& c = bw[4 * hi_u + d];
          const uint32_t r = xor_lane<S>(hi ? a : c);
          if (hi) a = r; else c = r;
        }
      }
  }
}

// ------------------------------------------------------------------------------------
// segment plan of one batch, computed by a single wavefront
// ------------------------------------------------------------------------------------
// Lane p ends up holding the p-th smallest key (id << 6 | caller row): a stable sort by
// adapter id, since the caller row breaks ties.  Rows with an id outside
// [0, n_adapters) get no key and are skipped.
struct WavePlan {
  uint32_t key;     // per lane: sorted key at position lane, kNoKey past the valid rows
  uint64_t starts;  // bit p set: sorted position p starts a segment
  int S;            // number of segments
  int n_valid;      // rows with a valid id
  bool bad_id;      // some id was out of range
};

__device__ inline WavePlan wave_plan(const int32_t* __restrict__ ids, int n, int n_adapters) {
  const int lane = threadIdx.x & 63;
  uint32_t key = kNoKey;
  bool bad = false;
  if (lane < n) {
    const int id = ids[lane];
    if (id >= 0 && id < n_adapters)
      key = (static_cast<uint32_t>(id) << 6) | static_cast<uint32_t>(lane);
    else
      bad = true;
  }
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(key), j));
      const bool ascending = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      const uint32_t lo = key < other ? key : other, hi = key < other ? other : key;
      key = (lower == ascending) ? lo : hi;
    }
  }
  const uint32_t prev = static_cast<uint32_t>(__shfl_up(static_cast<int>(key), 1));
  const bool valid = key != kNoKey;
  const bool start = valid && (lane == 0 || (key >> 6) != (prev >> 6));
  WavePlan P;
  P.key = key;
  P.starts = __ballot(start);
  P.S = __popcll(P.starts);
  P.n_valid = __popcll(__ballot(valid));
  P.bad_id = __ballot(bad) != 0;
  return P;
}

// sorted position where segment s starts (s < popcount(mask))
__device__ inline int nth_set_bit(uint64_t mask, int s) {
  for (int t = 0; t < s; ++t) mask &= mask - 1;
  return __ffsll(static_cast<long long>(mask)) - 1;
}

struct SegInfo {
  int a;     // adapter
  int seg0;  // first sorted position
  int m;     // rows
};

__device__ inline SegInfo segment_of(const WavePlan& P, int s) {
  SegInfo g;
  g.seg0 = nth_set_bit(P.starts, s);
  const uint64_t later = (g.seg0 >= 63) ? 0ull : (P.starts & ~((2ull << g.seg0) - 1ull));
  const int end = later ? (__ffsll(static_cast<long long>(later)) - 1) : P.n_valid;
  g.m = end - g.seg0;
  g.a = static_cast<int>(static_cast<uint32_t>(__shfl(static_cast<int>(P.key), g.seg0)) >> 6);
  return g;
}

// caller row of sorted position q (q may differ per lane; every lane must call)
__device__ inline int caller_row(const WavePlan& P, int q) {
  return static_cast<int>(static_cast<uint32_t>(__shfl(static_cast<int>(P.key), q & 63)) & 63u);
}

// ------------------------------------------------------------------------------------
// a1 on the device: write the segment tables (for callers that want them, and tests)
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void segments_from_ids_kernel(
    const int32_t* __restrict__ ids, int32_t n, int32_t n_adapters, int32_t* __restrict__ perm,
    int32_t* __restrict__ seg_starts, int32_t* __restrict__ seg_adapter,
    int32_t* __restrict__ n_segments) {
  const int lane = threadIdx.x;
  const WavePlan P = wave_plan(ids, n, n_adapters);
  if (lane < P.n_valid) perm[lane] = static_cast<int32_t>(P.key & 63u);
  if ((P.starts >> lane) & 1ull) {
    const int s = __popcll(P.starts & ((1ull << lane) - 1ull));
    seg_starts[s] = lane;
    seg_adapter[s] = static_cast<int32_t>(P.key >> 6);
  }
  if (lane == 0) {
    seg_starts[P.S] = P.n_valid;
    n_segments[0] = P.bad_id ? -1 : P.S;
  }
}

// ------------------------------------------------------------------------------------
// a1 on the device for up to kDevSortMax rows: rank by counting, then one scan
// ------------------------------------------------------------------------------------
// Row i's sorted position is the number of valid rows with a smaller id plus the number
// of earlier rows with the same id: the stable sort by adapter id.  rank_kernel computes
// it for every row (each workgroup holds all ids in LDS and each thread counts for one
// row) and scatters the row and its id to that position.  tables_kernel, one workgroup,
// then finds the segment starts in the sorted ids (where the id changes), numbers them
// with an exclusive scan and writes the tables.  Rows with an id outside [0, n_adapters)
// are left out (their perm entries are -1 past the valid rows).
struct SortOut {
  int32_t* perm;            // [n]
  int32_t* seg_starts;      // [S + 1]
  int32_t* seg_adapter;     // [S]
  int32_t* n_segments;      // [1]: S, or -1 if an id was out of range
  int32_t* sorted_ids;      // [n] scratch: the id at each sorted position
  int32_t* meta;            // nullable: [S, min_len, max_len, n_valid]
  const uint16_t** A_ptrs;  // nullable: per-segment pointers into the pools
  const uint16_t** B_ptrs;
  const uint16_t* A_pool;
  const uint16_t* B_pool;
  int64_t A_stride, B_stride;
  int32_t* ws_flag;         // nullable: set to 2 if an id was out of range
};

constexpr int kRankThreads = 1024;  // 16 waves: 64 rows per workgroup, the ids split 16 ways
constexpr int kRankRows = 64;
constexpr int kTabThreads = 1024;
constexpr int32_t kNoId = 0x7fffffff;  // larger than every valid id

__global__ __launch_bounds__(kRankThreads) void rank_kernel(const int32_t* __restrict__ ids,
                                                            int32_t n, int32_t n_adapters,
                                                            SortOut o) {
  __shared__ __attribute__((aligned(16))) int32_t sid[kDevSortMax + 16];
  constexpr int W = kRankThreads / 64;
  __shared__ int part[W][kRankRows];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = (n + 15) / 16 * 16;
  for (int j = tid; j < n16; j += kRankThreads) {
    int v = kNoId;
    if (j < n) {
      const int id = ids[j];
      if (id >= 0 && id < n_adapters) v = id;
    }
    sid[j] = v;
  }
  __syncthreads();
  const int i = blockIdx.x * kRankRows + lane;
  const int me = (i < n) ? sid[i] : kNoId;
  // wave w counts over ids [j0, j1), 16 at a time (four 16-byte LDS reads in flight)
  const int share = (n16 / 16 + W - 1) / W * 16;
  const int j0 = w * share, j1 = min(n16, j0 + share);
  int before = 0;
  for (int j = j0; j < j1; j += 16) {
    int4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = *reinterpret_cast<const int4*>(&sid[j + 4 * u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jj = j + 4 * u;
      before += (q[u].x < me) + (q[u].y < me) + (q[u].z < me) + (q[u].w < me);
      before += (q[u].x == me && jj < i) + (q[u].y == me && jj + 1 < i) +
                (q[u].z == me && jj + 2 < i) + (q[u].w == me && jj + 3 < i);
    }
  }
  part[w][lane] = before;
  __syncthreads();
  if (w == 0 && i < n && me != kNoId) {
    int pos = 0;
#pragma unroll
    for (int q = 0; q < W; ++q) pos += part[q][lane];
    o.perm[pos] = i;
    o.sorted_ids[pos] = me;
  }
}

__global__ __launch_bounds__(kTabThreads) void tables_kernel(const int32_t* __restrict__ ids,
                                                              int32_t n, int32_t n_adapters,
                                                              SortOut o) {
  constexpr int T = kTabThreads, PER = kDevSortMax / kTabThreads;
  __shared__ int32_t sid[kDevSortMax];
  __shared__ int pos[kDevSortMax + 1];
  __shared__ int wsum[T / 64];
  __shared__ int s_valid, s_bad, s_min, s_max, s_S;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) {
    s_valid = 0;
    s_bad = 0;
    s_min = 0x7fffffff;
    s_max = 0;
  }
  __syncthreads();
  // the ids (to count the valid rows) and the sorted ids are read in the same round; the
  // sorted ids past the valid rows are stale and never looked at
  int nv = 0;
  for (int i = tid; i < n; i += T) {
    const int id = ids[i];
    sid[i] = o.sorted_ids[i];
    if (id >= 0 && id < n_adapters) ++nv;
  }
  if (nv) atomicAdd(&s_valid, nv);
  __syncthreads();
  const int n_valid = s_valid;
  if (tid == 0 && n_valid < n) s_bad = 1;
  for (int p = n_valid + tid; p < n; p += T) o.perm[p] = -1;
  // thread t takes sorted positions PER*t .. PER*t + PER-1
  int starts = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int p = PER * tid + u;
    if (p < n_valid && (p == 0 || sid[p - 1] != sid[p])) ++starts;
  }
  int incl = starts;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int up = __shfl_up(incl, d);
    if (lane >= d) incl += up;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int q = 0; q < T / 64; ++q) {
    if (q < wv) before += wsum[q];
    total += wsum[q];
  }
  int seg = before + incl - starts;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int p = PER * tid + u;
    if (p < n_valid && (p == 0 || sid[p - 1] != sid[p])) {
      pos[seg] = p;
      o.seg_starts[seg] = p;
      o.seg_adapter[seg] = sid[p];
      ++seg;
    }
  }
  if (tid == 0) {
    pos[total] = n_valid;
    o.seg_starts[total] = n_valid;
    s_S = total;
  }
  __syncthreads();
  const int S = s_S;
  for (int sg = tid; sg < S; sg += T) {
    const int len = pos[sg + 1] - pos[sg];
    atomicMin(&s_min, len);
    atomicMax(&s_max, len);
    if (o.A_ptrs) {
      const int64_t a = sid[pos[sg]];
      o.A_ptrs[sg] = o.A_pool + a * o.A_stride;
      o.B_ptrs[sg] = o.B_pool + a * o.B_stride;
    }
  }
  __syncthreads();
  if (tid == 0) {
    o.n_segments[0] = s_bad ? -1 : S;
    if (o.meta) {
      o.meta[0] = S;
      o.meta[1] = S ? s_min : 0;
      o.meta[2] = s_max;
      o.meta[3] = n_valid;
    }
    if (s_bad && o.ws_flag)
      raise_flag(o.ws_flag, kFlagBadId);
  }
}

// Grouping for the fused call (sgmv_lora_add_pool, 64 < n <= 4096), one workgroup: rows
// of one adapter are made contiguous, which is all the paper summary's idea I2 needs; the
// order of the groups and of the rows inside a group is not the sorted one (the results
// do not depend on it: every row's sums are formed alone, in a fixed order).  Each id goes
// into an LDS hash table of 2 * kDevSortMax slots (open addressing), which counts its rows;
// a scan over the slots gives every group its first row and its segment number, and each
// row then takes the next free position of its group.  Writes the same tables as the
// sort (perm, seg_starts, seg_adapter, pointer tables, meta, n_segments, flag).
constexpr int kGroupThreads = 1024;
constexpr int kGroupSlots = 2 * kDevSortMax;
constexpr int kGroupPer = kDevSortMax / kGroupThreads;     // rows per thread
constexpr int kSlotsPer = kGroupSlots / kGroupThreads;     // slots per thread
static_assert(kGroupSlots == 1 << 13, "the slot hash keeps 13 bits");

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ ids,
                                                              int32_t n, int32_t n_adapters,
                                                              SortOut o) {
  constexpr int T = kGroupThreads, W = T / 64;
  __shared__ int key[kGroupSlots];  // adapter id of the slot, -1 = empty
  __shared__ int cnt[kGroupSlots];  // rows of the slot, then its next free position
  __shared__ int wrows[W], wsegs[W], wsrows[W], wssegs[W];
  __shared__ int s_bad, s_min, s_max, s_rows, s_segs;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int u = 0; u < kSlotsPer; ++u) {
    key[tid + T * u] = -1;
    cnt[tid + T * u] = 0;
  }
  if (tid == 0) {
    s_bad = 0;
    s_min = 0x7fffffff;
    s_max = 0;
  }
  __syncthreads();
  // insert: thread t takes rows t, t + T, ...  Consecutive lanes with the same id (a
  // request's rows) form a run whose first lane does the table work for the whole run, so
  // that a batch of few adapters does not serialise on a few LDS addresses.
  int slot[kGroupPer], rank[kGroupPer], head_lane[kGroupPer], run_len[kGroupPer];
#pragma unroll
  for (int u = 0; u < kGroupPer; ++u) {
    const int i = tid + T * u;
    int id = (i < n) ? ids[i] : -1;
    if (i < n && (id < 0 || id >= n_adapters)) {
      s_bad = 1;
      id = -1;
    }
    const bool valid = id >= 0;
    const int prev = __shfl_up(id, 1);
    const bool head = valid && (lane == 0 || prev != id);
    const uint64_t heads = __ballot(head);
    const uint64_t bounds = heads | __ballot(!valid);
    const uint64_t upto = (lane == 63) ? ~0ull : ((2ull << lane) - 1);
    const uint64_t below = heads & upto;
    const int hl = below ? 63 - __clzll(below) : lane;
    const uint64_t above = bounds & ~upto;
    const int len = (above ? __ffsll(static_cast<long long>(above)) - 1 : 64) - lane;
    int h = -1;
    if (head) {
      h = static_cast<int>((static_cast<uint32_t>(id) * 2654435761u) >> 19);  // 13 bits
      for (int probe = 0; probe < kGroupSlots; ++probe) {
        const int old = atomicCAS(&key[h], -1, id);
        if (old == -1 || old == id) break;
        h = (h + 1) & (kGroupSlots - 1);
      }
      atomicAdd(&cnt[h], len);
    }
    const int hs = __shfl(h, hl);
    slot[u] = valid ? hs : -1;
    rank[u] = lane - hl;
    head_lane[u] = hl;
    run_len[u] = head ? len : 0;
  }
  __syncthreads();
  // scan over the slots: thread t owns slots kSlotsPer*t .. +kSlotsPer-1.  Groups of at
  // least kLongMin rows come first, then the short ones, so that the long segments start
  // at row 0 and the MFMA tiles meet as few short rows as a sorted batch does.
  int lr = 0, ls = 0, sr = 0, ss = 0;  // long rows / segments, short rows / segments
#pragma unroll
  for (int u = 0; u < kSlotsPer; ++u) {
    const int c = cnt[kSlotsPer * tid + u];
    if (c >= kLongMin) {
      lr += c;
      ++ls;
    } else if (c > 0) {
      sr += c;
      ++ss;
    }
  }
  int ilr = lr, ils = ls, isr = sr, iss = ss;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int a0 = __shfl_up(ilr, d), a1 = __shfl_up(ils, d), a2 = __shfl_up(isr, d),
              a3 = __shfl_up(iss, d);
    if (lane >= d) {
      ilr += a0;
      ils += a1;
      isr += a2;
      iss += a3;
    }
  }
  if (lane == 63) {
    wrows[wv] = ilr;
    wsegs[wv] = ils;
    wsrows[wv] = isr;
    wssegs[wv] = iss;
  }
  __syncthreads();
  int lrow = ilr - lr, lseg = ils - ls, srow = isr - sr, sseg = iss - ss;
  int tlr = 0, tls = 0, tsr = 0, tss = 0;  // totals
  for (int q = 0; q < W; ++q) {
    if (q < wv) {
      lrow += wrows[q];
      lseg += wsegs[q];
      srow += wsrows[q];
      sseg += wssegs[q];
    }
    tlr += wrows[q];
    tls += wsegs[q];
    tsr += wsrows[q];
    tss += wssegs[q];
  }
  srow += tlr;  // short groups after all long ones
  sseg += tls;
  if (tid == 0) {
    s_rows = tlr + tsr;
    s_segs = tls + tss;
  }
  int mn = 0x7fffffff, mx = 0;
#pragma unroll
  for (int u = 0; u < kSlotsPer; ++u) {
    const int sl = kSlotsPer * tid + u;
    const int c = cnt[sl];
    if (c > 0) {
      const bool lng = c >= kLongMin;
      const int seg = lng ? lseg : sseg;
      const int row0 = lng ? lrow : srow;
      const int a = key[sl];
      o.seg_starts[seg] = row0;
      o.seg_adapter[seg] = a;
      if (o.A_ptrs) {
        o.A_ptrs[seg] = o.A_pool + static_cast<int64_t>(a) * o.A_stride;
        o.B_ptrs[seg] = o.B_pool + static_cast<int64_t>(a) * o.B_stride;
      }
      mn = min(mn, c);
      mx = max(mx, c);
      cnt[sl] = row0;  // from now on: the group's next free position
      if (lng) {
        lrow += c;
        ++lseg;
      } else {
        srow += c;
        ++sseg;
      }
    }
  }
  if (mx > 0) {
    atomicMin(&s_min, mn);
    atomicMax(&s_max, mx);
  }
  __syncthreads();
  // every run takes the next positions of its group, in row order inside the run
#pragma unroll
  for (int u = 0; u < kGroupPer; ++u) {
    int base = 0;
    if (run_len[u] > 0) base = atomicAdd(&cnt[slot[u]], run_len[u]);
    base = __shfl(base, head_lane[u]);
    if (slot[u] >= 0) o.perm[base + rank[u]] = tid + T * u;
  }
  const int n_valid = s_rows, S = s_segs;
  for (int p = n_valid + tid; p < n; p += T) o.perm[p] = -1;
  if (tid == 0) {
    o.seg_starts[S] = n_valid;
    o.n_segments[0] = s_bad ? -1 : S;
    if (o.meta) {
      o.meta[0] = S;
      o.meta[1] = S ? s_min : 0;
      o.meta[2] = s_max;
      o.meta[3] = n_valid;
    }
    if (s_bad && o.ws_flag)
      raise_flag(o.ws_flag, kFlagBadId);
  }
}

inline hipError_t launch_device_sort(hipStream_t st, const int32_t* ids, int32_t n,
                                     int32_t n_adapters, const SortOut& o) {
  hipLaunchKernelGGL(rank_kernel, dim3((n + kRankRows - 1) / kRankRows), dim3(kRankThreads), 0, st,
                     ids, n, n_adapters, o);
  hipLaunchKernelGGL(tables_kernel, dim3(1), dim3(kTabThreads), 0, st, ids, n, n_adapters, o);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// fused shrink + expand
// ------------------------------------------------------------------------------------
// Work items are keyed by a *leader* row: the first caller row of each adapter.  One
// coalesced load of the ids and one ballot give every workgroup its adapter and the
// set of rows that share it (the same rows, in the same caller order, as the stable
// sort's segment; the order of segments does not change the result).  Split-K partial
// sums are indexed by caller row.  Each is one 64-bit word, the float32 bits in the low
// half and a nonzero tag in the high half, written and read with agent-scope atomics:
// a reader that sees the tag sees the value, with no L2 write-back or invalidate
// between XCDs and no separate ready counter.
// ------------------------------------------------------------------------------------
// phase timestamps (profiling builds only, compiled with -DSGMV_PHASE_STAMPS)
// ------------------------------------------------------------------------------------
// Lane 0 of every wave of the one-launch kernels writes the 100 MHz real-time counter at
// fixed points of its item to stamps[blockIdx.x * kStampSlots + i] with an ordinary
// vector store, after waiting for all of the wave's memory operations where `wait` says
// so.  Points: 0 wave start, 1 ids in registers, then for a shrink item 2 A and x loaded,
// 3 tagged partial sums issued, 4 their stores acknowledged; for an expand item 2 B and y
// loaded, 3 every partial sum present, 4 y stored (issued), 5 y store acknowledged, 6 item
// done.  Normal builds compile no stamp.
[[maybe_unused]] constexpr int kStampSlots = 8;
[[maybe_unused]] constexpr int kStampMaxWgs = 8192;  // launches with a larger grid write no stamps
#ifdef SGMV_PHASE_STAMPS
#define SGMV_STAMP(p, i, wait)                                                              \
  do {                                                                                      \
    if (wait) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                              \
    if ((p).stamps && (threadIdx.x & 63) == 0)                                              \
      (p).stamps[blockIdx.x * kStampSlots + (i)] = __builtin_amdgcn_s_memrealtime();        \
  } while (0)
#else
#define SGMV_STAMP(p, i, wait) \
  do {                         \
  } while (0)
#endif

struct PoolArgs {
  uint16_t* y;
  const uint16_t* x;
  const int32_t* ids;
  const uint16_t* A;
  const uint16_t* B;
  int64_t ld_y, ld_x, A_stride, B_stride;
  int32_t n, n_adapters, h_in, h_out;
  int32_t KS, NS;
  int32_t b_delay;  // expand items: short sleeps before their B loads
  float scale;
  int32_t* ws_flag;
  int32_t* counters;
  uint64_t* part;
  uint64_t* stamps;  // profiling builds: this launch's phase timestamps, or NULL
};

struct Leader {
  int a;          // adapter
  uint64_t rows;  // caller rows that use it
};

constexpr uint64_t kPartTag = 1ull << 32;

__device__ inline void store_partial(uint64_t* q, float v) {
  __hip_atomic_store(q, kPartTag | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t load_partial(const uint64_t* q) {
  return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// shrink item: partial v over k in [kc*KC, (kc+1)*KC) for the adapter's rows within
// one block of 16 caller rows (blk).  MFMA 16x16x32; in k step u, lane l supplies MFMA
// row/column l%16 with k values 32u + 8(l/16) .. +7 of both operands, so one load
// instruction reads 64 contiguous bytes of each of 16 rows and two consecutive steps
// fill whole cache lines.
template <int DT, int R>
__device__ inline void shrink_item(const PoolArgs& p, const Leader& L, int blk, int kc) {
  using E = Elem<DT>;
  constexpr int U = 256 / R;
  constexpr int NB = R / 16;
  constexpr int KC = 32 * U;
  const int lane = threadIdx.x & 63;
  const int mrow = lane & 15, kq = lane >> 4;
  const gptr<const uint16_t> A = global_ptr(p.A) + static_cast<int64_t>(L.a) * p.A_stride;
  const int kbase = kc * KC + kq * 8;
  uint4 av[NB][U];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = kbase + 32 * u;
      av[nb][u] = (kk < p.h_in) ? ld16(A + static_cast<int64_t>(nb * 16 + mrow) * p.h_in + kk)
                                : zero4();
    }
  const int64_t slice = pool_slice(R);
  const uint32_t bm = static_cast<uint32_t>(L.rows >> (16 * blk)) & 0xffffu;
  const int row = 16 * blk + mrow;
  const gptr<const uint16_t> xr =
      ((bm >> mrow) & 1u) ? global_ptr(p.x) + static_cast<int64_t>(row) * p.ld_x : nullptr;
  uint4 xv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int kk = kbase + 32 * u;
    xv[u] = (xr && kk < p.h_in) ? ld16(xr + kk) : zero4();
  }
  SGMV_STAMP(p, 2, true);
  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = E::mfma(xv[u], av[nb][u], acc[nb]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * (lane >> 4) + e;
    if ((bm >> r) & 1u) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        store_partial(p.part + kc * slice + static_cast<int64_t>(16 * blk + r) * pool_part_row(R) + nb * 16 + mrow,
                      acc[nb][e]);
    }
  }
  SGMV_STAMP(p, 3, false);
  SGMV_STAMP(p, 4, true);
}

// expand item: one caller row r and the 64 * CPL columns from c0 = nc * 64 * CPL
// (CPL = pool_cpl(R)), whose rows of the stored [h_out, r] B[a] are 16 KB of contiguous
// memory.  Load instruction u reads 1 KB of it: lane l gets the 8 rank values 8q .. 8q+7
// of column c0 + u * 64/GC + l / GC, where GC = R / 8 lanes share a column and
// q = l % GC.  A transpose within each group of GC lanes (DPP quad permutations, and a
// swizzle for the third stage at r = 64) then leaves lane l with every rank value of the
// columns of the loads u = GC*t + q, t < 16/GC, i.e. columns c0 + 64t + q * 64/GC + l / GC,
// so that every load of B covers whole cache lines and every y access 64 consecutive
// columns.  Keying expand items by row spreads an adapter
// with many rows over as many wavefronts.  The y loads are issued first; the B loads wait
// `p.b_delay` short sleeps (chosen on the host from the bytes the shrink items fetch), so
// that A and x, which the partial sums wait for, reach the CUs before B competes with
// them for HBM.  B is transposed and widened to float32 while the shrink runs.
template <int DT, int R>
__device__ inline void expand_item(const PoolArgs& p, const Leader& L, int r, int nc) {
  using E = Elem<DT>;
  constexpr int GC = R / 8;     // lanes per column of B in the loads
  constexpr int G = 64 / R;     // lane groups when reading the partial sums
  constexpr int NV = 16;        // 16-byte loads of B per lane: 16 KB per item
  constexpr int CPI = 64 / GC;  // columns per load instruction
  constexpr int NT = 16 / GC;   // columns per lane
  static_assert(NV * 64 * 8 == 64 * pool_cpl(R) * R, "an item covers 16 KB of B");
  const int lane = threadIdx.x & 63;
  const int q = lane % GC, m = lane / GC;
  const int c0 = nc * 64 * pool_cpl(R);
  const int cq = c0 + q * CPI + m;  // the lane's column for t = 0; + 64t for t

  // unconditional loads keep the compiler's wait counts exact: columns past h_out read
  // column 0 and store nothing
  const gptr<uint16_t> yrow = global_ptr(p.y) + static_cast<int64_t>(r) * p.ld_y;
  uint32_t yv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = cq + 64 * t;
    yv[t] = *(yrow + (c < p.h_out ? c : 0));
  }
  asm volatile("" ::: "memory");  // keep the y loads ahead of the delay
  for (int i = 0; i < p.b_delay; ++i) __builtin_amdgcn_s_sleep(1);
  const gptr<const uint16_t> Bad = global_ptr(p.B) + static_cast<int64_t>(L.a) * p.B_stride + 8 * q;
  uint32_t bw[4 * NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int c = c0 + u * CPI + m;
    const u32x4_t v = *(gptr<const u32x4_t>)(Bad + static_cast<int64_t>(c < p.h_out ? c : 0) * R);
#pragma unroll
    for (int d = 0; d < 4; ++d) bw[4 * u + d] = v[d];
  }
  asm volatile("" ::: "memory");  // keep the B loads ahead of the polling below

  // v[r, j]: lane (j = lane % R, g = lane / R) takes slices g, g+G, ... of column j,
  // polls them until every tag is present and adds them in order; the G lane groups are
  // then combined by a fixed butterfly, so every lane ends with the same sum.  The first
  // two slices of each group are loaded before B is transposed (their loads go out right
  // after B's and return behind them), the rest in batches of 8.
  const int64_t slice = pool_slice(R);
  const uint64_t* src = p.part + static_cast<int64_t>(r) * pool_part_row(R) + (lane % R);
  const int g = lane / R;
  uint64_t w0[2];
  auto load_first = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // unconditional: slices past KS read slice KS - 1
      const int k = g + u * G;
      w0[u] = load_partial(src + (k < p.KS ? k : p.KS - 1) * slice);
    }
  };
  load_first();
  // the transpose takes bw from here on: after the poll's loads have been issued
#pragma unroll
  for (int i = 0; i < 4 * NV; ++i) asm volatile("" : "+v"(bw[i])::"memory");
  transpose_stage<GC, 1>(bw, q);
  transpose_stage<GC, 2>(bw, q);
  transpose_stage<GC, 4>(bw, q);
  // bf[t * R + j] = B[column of t, j], pinned in registers here so that none of this
  // work is left for after the poll
  float bf[NT * R];
#pragma unroll
  for (int e = 0; e < NT * R; ++e) {
    bf[e] = (e & 1) ? E::hi(bw[e >> 1]) : E::lo(bw[e >> 1]);
    pin(bf[e]);
  }
  SGMV_STAMP(p, 2, true);

  float acc = 0.f;
  for (int spins = 0;; ++spins) {
    bool ready = true;
#pragma unroll
    for (int u = 0; u < 2; ++u) ready = ready && (g + u * G >= p.KS || (w0[u] >> 32) != 0);
    if (__ballot(!ready) == 0) break;
    if (spins >= kSpinLimit) {
      if (lane == 0) raise_flag(p.ws_flag, kFlagWaitTimeout);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    load_first();
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
    acc += (g + u * G < p.KS) ? __uint_as_float(static_cast<uint32_t>(w0[u])) : 0.f;
  for (int k0 = 2 * G; k0 < p.KS; k0 += 8 * G) {
    uint64_t w[8];
    for (int spins = 0;; ++spins) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + g + u * G;
        w[u] = (k < p.KS) ? load_partial(src + k * slice) : kPartTag;
      }
      bool ready = true;
#pragma unroll
      for (int u = 0; u < 8; ++u) ready = ready && (w[u] >> 32) != 0;
      if (__ballot(!ready) == 0) break;
      if (spins >= kSpinLimit) {
        if (lane == 0) raise_flag(p.ws_flag, kFlagWaitTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += __uint_as_float(static_cast<uint32_t>(w[u]));
  }
  SGMV_STAMP(p, 3, false);
  // count this reader; whether it is the row's last is looked at after the y store
  int old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(&p.counters[r * kCounterStride], 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
  for (int msk = R; msk < 64; msk <<= 1) acc += __shfl_xor(acc, msk);
  // broadcast v[r, :] to scalar registers while every lane is active
  float vj[R];
#pragma unroll
  for (int jj = 0; jj < R; ++jj)
    vj[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), jj));
  float out[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) out[t] = 0.f;
#pragma unroll
  for (int jj = 0; jj < R; ++jj)
#pragma unroll
    for (int t = 0; t < NT; ++t) out[t] = fmaf(vj[jj], bf[t * R + jj], out[t]);
  uint16_t yo[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    yo[t] = static_cast<uint16_t>(E::pack(fmaf(p.scale, out[t], E::lo(yv[t])), 0.f));
  // y row r as a raw buffer of h_out elements: the hardware drops the stores of columns
  // past its end, so every item issues the same store instructions, with no branch, and
  // the wait for the row counter below covers that atomic alone: the last reader's
  // clearing of the partial sums then goes out while the y stores are still in flight
  // (cold decode7b calls 5.18 -> 5.07 us).  The stores carry sc1 (device scope): the L2
  // writes them through, so they are not left dirty for the write-back at the kernel's end
  // (5.09 -> 4.92 us; the non-temporal hint alone changed nothing).  The base address is
  // uniform; readfirstlane keeps the buffer resource in scalar registers.
  const uint64_t ya = reinterpret_cast<uint64_t>(p.y + static_cast<int64_t>(r) * p.ld_y);
  const uint64_t yu =
      (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ya >> 32))) << 32) |
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ya)));
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(yu), static_cast<short>(0), 2 * p.h_out, kBufferRsrcWord3);
#pragma unroll
  for (int t = 0; t < NT; ++t)
    __builtin_amdgcn_raw_buffer_store_b16(yo[t], yrs, 2 * (cq + 64 * t), 0, kStoreSc1);
  // the counter's value is looked at only after the y stores have been issued
  asm volatile("" : "+v"(old)::"memory");
  SGMV_STAMP(p, 4, false);
  SGMV_STAMP(p, 5, true);

  // the last of row r's NS readers clears the row's partials and its counter, leaving
  // both at zero for the next call
  if (__builtin_amdgcn_readfirstlane(old) == p.NS - 1) {
    uint64_t* row = p.part + static_cast<int64_t>(r) * pool_part_row(R);
    for (int idx = lane; idx < p.KS * R; idx += 64)
      __hip_atomic_store(row + (idx / R) * slice + (idx % R), 0ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0)
      __hip_atomic_store(&p.counters[r * kCounterStride], 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  SGMV_STAMP(p, 6, true);
}

// Grid: n * KS shrink items (caller row r = i % n, chunk i / n; active when r is the
// first row of its adapter within its block of 16 rows), then n * NS expand items
// (caller row r = i % n, column chunk i / n), kItemsPerWg items per workgroup (one per
// wave).
// Every shrink item an expand item waits for sits in a lower-numbered workgroup.
// The kernel body, given lane's adapter id (the id of caller row `lane`, -1 past n).
template <int DT, int R>
__device__ inline void pool_items(const PoolArgs& p, int id) {
  SGMV_STAMP(p, 1, true);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n_shrink = p.n * p.KS;
  const int shrink_wgs = (n_shrink + kItemsPerWg - 1) / kItemsPerWg;
  const int b = blockIdx.x;
  if (b == 0 && wv == 0) {
    const bool bad = __ballot(lane < p.n && (id < 0 || id >= p.n_adapters)) != 0;
    if (bad && lane == 0) raise_flag(p.ws_flag, kFlagBadId);
  }
  Leader L;
  if (b < shrink_wgs) {
    // item (row r, chunk kc) works iff r is its adapter's first row within r's block
    const int it = kItemsPerWg * b + wv;
    if (it >= n_shrink) return;
    const int r = it % p.n, kc = it / p.n;
    const int a = __builtin_amdgcn_readlane(id, r);
    if (a < 0 || a >= p.n_adapters) return;
    L.a = a;
    L.rows = __ballot(lane < p.n && id == a);
    const int blk = r >> 4;
    const uint32_t bm = static_cast<uint32_t>(L.rows >> (16 * blk)) & 0xffffu;
    if (bm & ((1u << (r & 15)) - 1u)) return;
    shrink_item<DT, R>(p, L, blk, kc);
  } else {
    const int it = kItemsPerWg * (b - shrink_wgs) + wv;
    if (it >= p.n * p.NS) return;
    const int r = it % p.n, nc = it / p.n;
    const int a = __builtin_amdgcn_readlane(id, r);
    if (a < 0 || a >= p.n_adapters) return;
    L.a = a;
    L.rows = __ballot(lane < p.n && id == a);
    expand_item<DT, R>(p, L, r, nc);
  }
}

// Adapter ids in device memory: every wave starts with one coalesced load of them.
template <int DT, int R>
__global__ __launch_bounds__(64 * kItemsPerWg) void lora_add_pool_kernel(PoolArgs p) {
  SGMV_STAMP(p, 0, false);
  const int lane = threadIdx.x & 63;
  pool_items<DT, R>(p, lane < p.n ? p.ids[lane] : -1);
}

// Adapter ids carried in the kernel arguments (checked on the host before the launch).
// They reach the waves with the rest of the arguments, so the loads of A and B are the
// first memory accesses that depend on them: no global load of the ids precedes them.
struct PoolIds {
  int32_t id[kPoolMaxN];
};

template <int DT, int R>
__global__ __launch_bounds__(64 * kItemsPerWg) void lora_add_ids_kernel(PoolArgs p, PoolIds ids) {
  SGMV_STAMP(p, 0, false);
  const int lane = threadIdx.x & 63;
  const int raw = ids.id[lane];  // every lane loads: the load need not wait for p.n
  pool_items<DT, R>(p, lane < p.n ? raw : -1);
}

template <int DT, int R>
hipError_t launch_pool(hipStream_t st, const PoolArgs& p) {
  const int grid = (p.n * p.KS + kItemsPerWg - 1) / kItemsPerWg +
                   (p.n * p.NS + kItemsPerWg - 1) / kItemsPerWg;
  hipLaunchKernelGGL((lora_add_pool_kernel<DT, R>), dim3(grid), dim3(64 * kItemsPerWg), 0, st, p);
  return hipGetLastError();
}

template <int DT, int R>
hipError_t launch_ids(hipStream_t st, const PoolArgs& p, const PoolIds& ids) {
  const int grid = (p.n * p.KS + kItemsPerWg - 1) / kItemsPerWg +
                   (p.n * p.NS + kItemsPerWg - 1) / kItemsPerWg;
  hipLaunchKernelGGL((lora_add_ids_kernel<DT, R>), dim3(grid), dim3(64 * kItemsPerWg), 0, st, p,
                     ids);
  return hipGetLastError();
}

}  // namespace

extern "C" int sgmv_build_segments_device(hipStream_t stream, const int32_t* adapter_ids,
                                          int32_t n, int32_t n_adapters, int32_t* perm,
                                          int32_t* seg_starts, int32_t* seg_adapter,
                                          int32_t* n_segments) {
  if (n < 0 || n > kDevSortMax || n_adapters <= 0 || n_adapters > (1 << 24)) return SGMV_ERR_SHAPE;
  if (!seg_starts || !n_segments || (n > 0 && (!adapter_ids || !perm || !seg_adapter)))
    return SGMV_ERR_NULL;
  int st = check_device();
  if (st) return st;
  if (n <= kPoolMaxN) {
    hipLaunchKernelGGL(segments_from_ids_kernel, dim3(1), dim3(64), 0, stream, adapter_ids, n,
                       n_adapters, perm, seg_starts, seg_adapter, n_segments);
  } else {
    // the sorted ids go to seg_adapter first (it has n entries); tables_kernel reads them
    // into LDS before it writes the segments' adapters there
    SortOut o{};
    o.perm = perm;
    o.seg_starts = seg_starts;
    o.seg_adapter = seg_adapter;
    o.n_segments = n_segments;
    o.sorted_ids = seg_adapter;
    return hip_status(launch_device_sort(stream, adapter_ids, n, n_adapters, o));
  }
  return hip_status(hipGetLastError());
}

namespace {

// Host checks of the pool entry points' arguments other than the workspace (no HIP call).
int check_pool_args(int32_t dtype, void* y, int64_t ld_y, const void* x, int64_t ld_x,
                    const int32_t* adapter_ids, int32_t n, const void* A_pool, int64_t A_stride,
                    const void* B_pool, int64_t B_stride, int32_t n_adapters, int32_t h_in,
                    int32_t h_out, int32_t r) {
  if (dtype != SGMV_F16 && dtype != SGMV_BF16) return SGMV_ERR_UNSUPPORTED;
  if (!rank_ok(r)) return SGMV_ERR_UNSUPPORTED;
  if (n < 0 || n > kDevSortMax || n_adapters <= 0 || n_adapters > (1 << 24)) return SGMV_ERR_SHAPE;
  int st = check_dim(h_in, ld_x);
  if (st) return st;
  if ((st = check_dim(h_out, ld_y))) return st;
  if (A_stride < static_cast<int64_t>(r) * h_in || B_stride < static_cast<int64_t>(h_out) * r)
    return SGMV_ERR_SHAPE;
  if (A_stride % 8 != 0 || B_stride % 8 != 0) return SGMV_ERR_ALIGNMENT;
  if (n == 0) return SGMV_OK;
  if (!y || !x || !adapter_ids || !A_pool || !B_pool) return SGMV_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(A_pool) || !aligned16(B_pool))
    return SGMV_ERR_ALIGNMENT;
  if (ranges_overlap(x, matrix_bytes(n, ld_x, h_in), y, matrix_bytes(n, ld_y, h_out)))
    return SGMV_ERR_ALIAS;
  return SGMV_OK;
}

// Host checks shared by the pool entry points (no HIP call).
int check_pool_call(int32_t dtype, void* y, int64_t ld_y, const void* x, int64_t ld_x,
                    const int32_t* adapter_ids, int32_t n, const void* A_pool, int64_t A_stride,
                    const void* B_pool, int64_t B_stride, int32_t n_adapters, int32_t h_in,
                    int32_t h_out, int32_t r, void* workspace, size_t workspace_bytes) {
  int st = check_pool_args(dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool, A_stride, B_pool,
                           B_stride, n_adapters, h_in, h_out, r);
  if (st || n == 0) return st;
  if (!workspace || workspace_bytes < sgmv_workspace_bytes(n, h_in, r) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SGMV_ERR_WORKSPACE;
  return SGMV_OK;
}

#ifdef SGMV_PHASE_STAMPS
// profiling builds: the stamp buffer attached by sgmv_phase_stamps_attach, used round robin
// one launch's slice at a time
uint64_t* g_stamp_buf = nullptr;
int64_t g_stamp_cap = 0, g_stamp_next = 0;
uint64_t* next_stamps(int grid) {
  if (!g_stamp_buf || grid > kStampMaxWgs) return nullptr;
  return g_stamp_buf + (g_stamp_next++ % g_stamp_cap) * static_cast<int64_t>(kStampMaxWgs) * kStampSlots;
}
#else
uint64_t* next_stamps(int) { return nullptr; }
#endif

// Short sleeps (64 clocks each) before an expand item loads B: about the time HBM takes
// to deliver what the shrink items fetch (the distinct adapters' A and the rows of x),
// kDelayPerMiB per MiB (tuned on MI355X), at most kDelayMax.
constexpr double kDelayPerMiB = 5.0;
constexpr int kDelayMax = 160;
int32_t b_delay(int distinct, int n, int h_in, int r) {
  const double mib = 2.0 * h_in * (static_cast<double>(distinct) * r + n) / (1 << 20);
  const double d = kDelayPerMiB * mib;
  return static_cast<int32_t>(d < kDelayMax ? d + 0.5 : kDelayMax);
}

// Arguments of the one-launch kernels (n <= 64).
PoolArgs pool_args(void* y, int64_t ld_y, const void* x, int64_t ld_x, const int32_t* adapter_ids,
                   int32_t n, const void* A_pool, int64_t A_stride, const void* B_pool,
                   int64_t B_stride, int32_t n_adapters, int32_t h_in, int32_t h_out, int32_t r,
                   float scale, void* workspace, size_t workspace_bytes) {
  PoolArgs p;
  p.y = static_cast<uint16_t*>(y);
  p.x = static_cast<const uint16_t*>(x);
  p.ids = adapter_ids;
  p.A = static_cast<const uint16_t*>(A_pool);
  p.B = static_cast<const uint16_t*>(B_pool);
  p.ld_y = ld_y;
  p.ld_x = ld_x;
  p.A_stride = A_stride;
  p.B_stride = B_stride;
  p.n = n;
  p.n_adapters = n_adapters;
  p.h_in = h_in;
  p.h_out = h_out;
  p.KS = (h_in + pool_kc(r) - 1) / pool_kc(r);
  const int cols = 64 * pool_cpl(r);
  p.NS = (h_out + cols - 1) / cols;  // 64 lanes x pool_cpl(r) columns per item
  p.b_delay = 0;
  p.scale = scale;
  char* ws = static_cast<char*>(workspace);
  p.ws_flag = reinterpret_cast<int32_t*>(ws);
  p.counters = reinterpret_cast<int32_t*>(ws + kWsPoolCounters);
  p.part = reinterpret_cast<uint64_t*>(ws + pool_offset(workspace_bytes, h_in, r));
  p.stamps = next_stamps(n * (p.KS + p.NS));
  return p;
}

}  // namespace

extern "C" int sgmv_lora_add_pool(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y,
                                  const void* x, int64_t ld_x, const int32_t* adapter_ids,
                                  int32_t n, const void* A_pool, int64_t A_stride,
                                  const void* B_pool, int64_t B_stride, int32_t n_adapters,
                                  int32_t h_in, int32_t h_out, int32_t r, float scale,
                                  void* workspace, size_t workspace_bytes) {
  int st = check_pool_call(dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool, A_stride, B_pool,
                           B_stride, n_adapters, h_in, h_out, r, workspace, workspace_bytes);
  if (st || n == 0) return st;
  if ((st = check_device())) return st;

  if (n > kPoolMaxN) {
    // device grouping into the workspace, then the table path on those tables
    char* wsb = static_cast<char*>(workspace);
    const WsLayout L = ws_layout(n, h_in, r);
    const DevTabLayout D = dev_tab_layout(n);
    char* dt = wsb + L.dtab_off;
    SortOut o{};
    o.perm = reinterpret_cast<int32_t*>(dt + D.perm);
    o.seg_starts = reinterpret_cast<int32_t*>(dt + D.seg_starts);
    o.seg_adapter = reinterpret_cast<int32_t*>(dt + D.seg_adapter);
    o.n_segments = reinterpret_cast<int32_t*>(dt + D.n_segments);
    o.meta = reinterpret_cast<int32_t*>(dt + D.meta);
    o.A_ptrs = reinterpret_cast<const uint16_t**>(dt + D.A_ptrs);
    o.B_ptrs = reinterpret_cast<const uint16_t**>(dt + D.B_ptrs);
    o.A_pool = static_cast<const uint16_t*>(A_pool);
    o.B_pool = static_cast<const uint16_t*>(B_pool);
    o.A_stride = A_stride;
    o.B_stride = B_stride;
    o.ws_flag = reinterpret_cast<int32_t*>(wsb);
    o.sorted_ids = reinterpret_cast<int32_t*>(dt + D.sorted_ids);
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kGroupThreads), 0, stream, adapter_ids, n,
                       n_adapters, o);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e);
    const int32_t S_max = n < n_adapters ? n : n_adapters;
    return hip_status(table_lora_add_device(
        stream, dtype, r, y, ld_y, x, ld_x, reinterpret_cast<const void* const*>(o.A_ptrs),
        reinterpret_cast<const void* const*>(o.B_ptrs), o.seg_starts, o.perm, o.meta, n, S_max,
        h_in, h_out, scale, workspace));
  }

  PoolArgs p = pool_args(y, ld_y, x, ld_x, adapter_ids, n, A_pool, A_stride, B_pool, B_stride,
                         n_adapters, h_in, h_out, r, scale, workspace, workspace_bytes);
  p.b_delay = b_delay(n < n_adapters ? n : n_adapters, n, h_in, r);  // ids unknown here
  hipError_t e;
  if (dtype == SGMV_F16) {
    e = (r == 16) ? launch_pool<SGMV_F16, 16>(stream, p)
        : (r == 32) ? launch_pool<SGMV_F16, 32>(stream, p) : launch_pool<SGMV_F16, 64>(stream, p);
  } else {
    e = (r == 16) ? launch_pool<SGMV_BF16, 16>(stream, p)
        : (r == 32) ? launch_pool<SGMV_BF16, 32>(stream, p) : launch_pool<SGMV_BF16, 64>(stream, p);
  }
  return hip_status(e);
}

namespace {

// Number of distinct values among ids[0 .. n), n <= 64 (open addressing in a table of 128).
int distinct_ids(const int32_t* ids, int32_t n) {
  uint32_t tab[128] = {};  // id + 1, 0 = empty
  int count = 0;
  for (int i = 0; i < n; ++i) {
    const uint32_t key = static_cast<uint32_t>(ids[i]) + 1u;
    uint32_t h = (key * 2654435761u) >> 25;
    while (tab[h] != 0 && tab[h] != key) h = (h + 1) & 127u;
    if (tab[h] == 0) {
      tab[h] = key;
      ++count;
    }
  }
  return count;
}

// The one-launch kernel with host ids on a workspace that the caller's checks accepted.
int run_host_ids(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y, const void* x,
                 int64_t ld_x, const int32_t* adapter_ids, int32_t n, const void* A_pool,
                 int64_t A_stride, const void* B_pool, int64_t B_stride, int32_t n_adapters,
                 int32_t h_in, int32_t h_out, int32_t r, float scale, void* workspace,
                 size_t workspace_bytes) {
  PoolArgs p = pool_args(y, ld_y, x, ld_x, nullptr, n, A_pool, A_stride, B_pool, B_stride,
                         n_adapters, h_in, h_out, r, scale, workspace, workspace_bytes);
  PoolIds ids;
  for (int i = 0; i < kPoolMaxN; ++i) ids.id[i] = i < n ? adapter_ids[i] : -1;
  p.b_delay = b_delay(distinct_ids(adapter_ids, n), n, h_in, r);
  hipError_t e;
  if (dtype == SGMV_F16) {
    e = (r == 16) ? launch_ids<SGMV_F16, 16>(stream, p, ids)
        : (r == 32) ? launch_ids<SGMV_F16, 32>(stream, p, ids)
                    : launch_ids<SGMV_F16, 64>(stream, p, ids);
  } else {
    e = (r == 16) ? launch_ids<SGMV_BF16, 16>(stream, p, ids)
        : (r == 32) ? launch_ids<SGMV_BF16, 32>(stream, p, ids)
                    : launch_ids<SGMV_BF16, 64>(stream, p, ids);
  }
  return hip_status(e);
}

// host-side check of host ids: each in [0, n_adapters)
int check_host_ids(const int32_t* adapter_ids, int32_t n, int32_t n_adapters) {
  for (int i = 0; i < n; ++i)
    if (adapter_ids[i] < 0 || adapter_ids[i] >= n_adapters) return SGMV_ERR_ADAPTER_ID;
  return SGMV_OK;
}

}  // namespace

extern "C" int sgmv_lora_add_host_ids(hipStream_t stream, int32_t dtype, void* y, int64_t ld_y,
                                      const void* x, int64_t ld_x, const int32_t* adapter_ids,
                                      int32_t n, const void* A_pool, int64_t A_stride,
                                      const void* B_pool, int64_t B_stride, int32_t n_adapters,
                                      int32_t h_in, int32_t h_out, int32_t r, float scale,
                                      void* workspace, size_t workspace_bytes) {
  if (n > kPoolMaxN) return SGMV_ERR_SHAPE;
  int st = check_pool_call(dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool, A_stride, B_pool,
                           B_stride, n_adapters, h_in, h_out, r, workspace, workspace_bytes);
  if (st || n == 0) return st;
  if ((st = check_host_ids(adapter_ids, n, n_adapters))) return st;
  if ((st = check_device())) return st;
  // the kernel reads no id from memory: the ids travel in its arguments
  return run_host_ids(stream, dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool, A_stride, B_pool,
                      B_stride, n_adapters, h_in, h_out, r, scale, workspace, workspace_bytes);
}

// ------------------------------------------------------------------------------------
// allocation-free variant of sgmv_lora_add_host_ids
// ------------------------------------------------------------------------------------
// The one-launch kernel's scratch (flag word, per-row counters, tagged partial sums) in a
// static device array instead of a caller workspace: zero when the code object is loaded,
// and every call that completes leaves its counters and partial sums at zero again.  In
// host code `scratch` names a host-side stand-in; its device address comes from
// hipGetSymbolAddress, once per device, and only that address reaches a kernel.
constexpr size_t kScratchPartMax = size_t(8) << 20;  // tagged partial sums, at most
constexpr size_t kScratchBytes =
    kWsPoolCounters + sizeof(int32_t) * kCounterInts * kMaxPoolRows + 256 + kScratchPartMax;
static_assert(kScratchBytes % 256 == 0, "scratch layout");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// the device address of `scratch` on the current device (looked up once per device)
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return SGMV_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SGMV_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SGMV_OK;
}

}  // namespace

extern "C" int sgmv_lora_add_host_ids_noalloc(hipStream_t stream, int32_t dtype, void* y,
                                              int64_t ld_y, const void* x, int64_t ld_x,
                                              const int32_t* adapter_ids, int32_t n,
                                              const void* A_pool, int64_t A_stride,
                                              const void* B_pool, int64_t B_stride,
                                              int32_t n_adapters, int32_t h_in, int32_t h_out,
                                              int32_t r, float scale) {
  if (n > kPoolMaxN) return SGMV_ERR_SHAPE;
  int st = check_pool_args(dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool, A_stride, B_pool,
                           B_stride, n_adapters, h_in, h_out, r);
  if (st || n == 0) return st;
  if (pool_bytes(h_in, r) > kScratchPartMax) return SGMV_ERR_WORKSPACE;
  if ((st = check_host_ids(adapter_ids, n, n_adapters))) return st;
  if ((st = check_device())) return st;
  if (stream) {
    int sdev = -1, cur = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || hipGetDevice(&cur) != hipSuccess ||
        sdev != cur)
      return SGMV_ERR_HIP;  // the scratch used is the current device's
  }
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return run_host_ids(stream, dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool, A_stride, B_pool,
                      B_stride, n_adapters, h_in, h_out, r, scale, ws, kScratchBytes);
}

#ifdef SGMV_PHASE_STAMPS
// Profiling builds only (not declared in the public header): attach a device buffer of
// `launches` * 8192 * 8 uint64 words; each later one-launch call writes its waves' phase
// timestamps into the next launch's slice (round robin).  NULL detaches.  Returns the
// number of launches stamped since the last attach.
extern "C" int64_t sgmv_phase_stamps_attach(uint64_t* device_buf, int64_t launches) {
  const int64_t done = g_stamp_next;
  g_stamp_buf = launches > 0 ? device_buf : nullptr;
  g_stamp_cap = launches > 0 ? launches : 0;
  g_stamp_next = 0;
  return done;
}
#endif
