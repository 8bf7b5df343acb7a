// Host side of libsgmv that needs no GPU: status strings and the segment-metadata
// builder.  The builder is the "sort the batch by adapter" step of the Punica paper
// summary (research.elamur.ai, "Interesting ideas", I2): a stable sort of the caller's
// rows by adapter id, so that every adapter's rows form one contiguous
// segment, followed by the per-segment adapter pointer table that lets one launch
// gather each segment's own A and B.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/sgmv.h"

extern "C" int sgmv_abi_version(void) { return SGMV_ABI_VERSION; }

extern "C" const char* sgmv_status_string(int status) {
  switch (status) {
    case SGMV_OK: return "ok";
    case SGMV_ERR_NULL: return "a required pointer is NULL";
    case SGMV_ERR_SHAPE: return "inconsistent size, stride or segment bound";
    case SGMV_ERR_ALIGNMENT: return "pointer not 16-byte aligned or dimension not a multiple of 8";
    case SGMV_ERR_ADAPTER_ID: return "adapter id out of range";
    case SGMV_ERR_UNSUPPORTED: return "unsupported dtype or rank";
    case SGMV_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case SGMV_ERR_ALIAS: return "output overlaps an input";
    case SGMV_ERR_HIP: return "HIP runtime error";
    case SGMV_ERR_DEVICE: return "a device-side check flagged the workspace";
    default: return "unknown status";
  }
}

extern "C" int sgmv_build_segments(const int32_t* adapter_ids, int32_t n, int32_t n_adapters,
                                   int32_t* perm, int32_t* seg_starts, int32_t* seg_adapter,
                                   int32_t* n_segments, int32_t* min_seg_len,
                                   int32_t* max_seg_len) {
  if (n < 0 || n_adapters <= 0) return SGMV_ERR_SHAPE;
  if (!seg_starts || !n_segments || (n > 0 && (!adapter_ids || !perm || !seg_adapter)))
    return SGMV_ERR_NULL;

  // Runs of equal ids in caller order (a request's rows are usually contiguous), so that
  // the work below is per run and per distinct id, not per row or per pool entry.
  struct Run {
    int32_t id, row0, len;
  };
  std::vector<Run> runs;
  for (int32_t t = 0; t < n;) {
    const int32_t a = adapter_ids[t];
    if (a < 0 || a >= n_adapters) return SGMV_ERR_ADAPTER_ID;
    int32_t u = t + 1;
    while (u < n && adapter_ids[u] == a) ++u;
    runs.push_back({a, t, u - t});
    t = u;
  }
  // one segment per distinct id, in increasing id order
  std::vector<int32_t> ids(runs.size());
  for (size_t i = 0; i < runs.size(); ++i) ids[i] = runs[i].id;
  std::sort(ids.begin(), ids.end());
  ids.erase(std::unique(ids.begin(), ids.end()), ids.end());
  const int32_t S = static_cast<int32_t>(ids.size());
  std::vector<int32_t> seg_of(runs.size()), next(static_cast<size_t>(S) + 1, 0);
  for (size_t i = 0; i < runs.size(); ++i) {
    seg_of[i] = static_cast<int32_t>(std::lower_bound(ids.begin(), ids.end(), runs[i].id) - ids.begin());
    next[seg_of[i] + 1] += runs[i].len;
  }
  int32_t lo = n, hi = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int32_t cnt = next[s + 1];
    if (cnt < lo) lo = cnt;
    if (cnt > hi) hi = cnt;
    next[s + 1] += next[s];  // next[s] = first sorted position of segment s
    seg_starts[s] = next[s];
    seg_adapter[s] = ids[s];
  }
  seg_starts[S] = n;
  // scatter the runs in caller order: the rows of one adapter keep their relative order
  // (a stable sort)
  for (size_t i = 0; i < runs.size(); ++i) {
    int32_t* dst = perm + next[seg_of[i]];
    for (int32_t v = 0; v < runs[i].len; ++v) dst[v] = runs[i].row0 + v;
    next[seg_of[i]] += runs[i].len;
  }

  *n_segments = S;
  if (min_seg_len) *min_seg_len = (n > 0) ? lo : 0;
  if (max_seg_len) *max_seg_len = hi;
  return SGMV_OK;
}

extern "C" int sgmv_build_ptr_table(const uint64_t* adapter_base, int32_t n_adapters,
                                    const int32_t* seg_adapter, int32_t n_segments,
                                    uint64_t* seg_ptrs) {
  if (n_adapters <= 0 || n_segments < 0) return SGMV_ERR_SHAPE;
  if (n_segments == 0) return SGMV_OK;
  if (!adapter_base || !seg_adapter || !seg_ptrs) return SGMV_ERR_NULL;
  for (int32_t s = 0; s < n_segments; ++s) {
    const int32_t a = seg_adapter[s];
    if (a < 0 || a >= n_adapters) return SGMV_ERR_ADAPTER_ID;
    const uint64_t p = adapter_base[a];
    if (p == 0) return SGMV_ERR_NULL;
    if (p % 16 != 0) return SGMV_ERR_ALIGNMENT;
    seg_ptrs[s] = p;
  }
  return SGMV_OK;
}

// Mixed ranks: the same counting sort with (rank class, adapter id) as the key.  Each
// non-empty rank class becomes one group with its own relative segment starts, so that
// the fused call can run every group through the kernels built for its rank.
extern "C" int sgmv_build_segments_ranked(const int32_t* adapter_ids, int32_t n,
                                          int32_t n_adapters, const int32_t* adapter_rank,
                                          int32_t* perm, int32_t* seg_starts,
                                          int32_t* seg_adapter, sgmv_rank_group* groups,
                                          int32_t* n_groups) {
  if (n < 0 || n_adapters <= 0) return SGMV_ERR_SHAPE;
  if (!seg_starts || !groups || !n_groups || !adapter_rank ||
      (n > 0 && (!adapter_ids || !perm || !seg_adapter)))
    return SGMV_ERR_NULL;
  for (int32_t a = 0; a < n_adapters; ++a) {
    const int32_t r = adapter_rank[a];
    if (r != 16 && r != 32 && r != 64) return SGMV_ERR_UNSUPPORTED;
  }
  for (int32_t t = 0; t < n; ++t)
    if (adapter_ids[t] < 0 || adapter_ids[t] >= n_adapters) return SGMV_ERR_ADAPTER_ID;

  std::vector<int32_t> count(static_cast<size_t>(n_adapters), 0), slot(count.size(), 0);
  for (int32_t t = 0; t < n; ++t) ++count[adapter_ids[t]];
  int32_t G = 0, S = 0, row = 0;
  for (int32_t r = 16; r <= 64; r *= 2) {
    sgmv_rank_group g{};
    g.r = r;
    g.row0 = row;
    g.seg0 = S;
    g.starts0 = S + G;
    g.min_seg_len = n;
    g.max_seg_len = 0;
    g.scale = 1.0f;
    for (int32_t a = 0; a < n_adapters; ++a) {
      const int32_t cnt = count[a];
      if (adapter_rank[a] != r || cnt == 0) continue;
      seg_starts[S + G] = row - g.row0;
      seg_adapter[S] = a;
      slot[a] = row;
      row += cnt;
      ++S;
      if (cnt < g.min_seg_len) g.min_seg_len = cnt;
      if (cnt > g.max_seg_len) g.max_seg_len = cnt;
    }
    if (row == g.row0) continue;  // no rows of this rank
    g.n = row - g.row0;
    g.n_segments = S - g.seg0;
    seg_starts[S + G] = g.n;
    groups[G++] = g;
  }
  for (int32_t t = 0; t < n; ++t) perm[slot[adapter_ids[t]]++] = t;
  *n_groups = G;
  return SGMV_OK;
}
