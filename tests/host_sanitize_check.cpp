// Host code of libsgmv under AddressSanitizer and UndefinedBehaviorSanitizer: the segment
// builders and the pointer table (sgmv_segments.cpp), the adapter slot cache
// (sgmv_cache.cpp) and the argument checks and
// workspace layout (sgmv_checks.h), driven over random and edge-case inputs, including
// every rejection.  Built with g++ (no GPU code) and run by tests/test_host_abi.py; prints
// "ok <count>" and exits 0 when every case behaves, any sanitizer report aborts the run.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../adapter_gemv_amd/csrc/sgmv_checks.h"

using namespace sgmv_host;

static long g_checks = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    ++g_checks;                                                        \
    if (!(cond)) {                                                     \
      std::printf("failed at line %d: %s\n", __LINE__, #cond);         \
      std::exit(1);                                                    \
    }                                                                  \
  } while (0)

// The builder's outputs describe a stable sort of ids: perm is a permutation, segments
// cover the sorted rows in ascending adapter order, and rows of one adapter keep their
// caller order.
static void check_sorted(const std::vector<int32_t>& ids, const std::vector<int32_t>& perm,
                         const std::vector<int32_t>& starts, const std::vector<int32_t>& seg_ad,
                         int S, int lo, int hi) {
  const int n = static_cast<int>(ids.size());
  std::vector<char> seen(n, 0);
  for (int i = 0; i < n; ++i) {
    EXPECT(perm[i] >= 0 && perm[i] < n && !seen[perm[i]]);
    seen[perm[i]] = 1;
  }
  EXPECT(starts[0] == 0 && starts[S] == n);
  int mn = n, mx = 0;
  for (int s = 0; s < S; ++s) {
    EXPECT(starts[s] < starts[s + 1]);
    if (s > 0) EXPECT(seg_ad[s - 1] < seg_ad[s]);
    for (int i = starts[s]; i < starts[s + 1]; ++i) {
      EXPECT(ids[perm[i]] == seg_ad[s]);
      if (i > starts[s]) EXPECT(perm[i - 1] < perm[i]);
    }
    const int len = starts[s + 1] - starts[s];
    mn = len < mn ? len : mn;
    mx = len > mx ? len : mx;
  }
  EXPECT(lo == (n ? mn : 0) && hi == mx);
}

static void builder_cases() {
  std::mt19937 rng(7);
  const int ns[] = {0, 1, 2, 15, 16, 17, 64, 65, 300, 2112, 4096};
  const int Ps[] = {1, 2, 7, 64, 5000};
  for (int n : ns)
    for (int P : Ps) {
      std::vector<int32_t> ids(n);
      for (auto& t : ids) t = static_cast<int32_t>(rng() % P);
      // buffers sized exactly as the header asks (seg_starts n + 1, the others n)
      std::vector<int32_t> perm(n), starts(n + 1), seg_ad(n > 0 ? n : 1);
      int32_t S = -1, lo = -1, hi = -1;
      EXPECT(sgmv_build_segments(ids.data(), n, P, perm.data(), starts.data(), seg_ad.data(), &S,
                                 &lo, &hi) == SGMV_OK);
      check_sorted(ids, perm, starts, seg_ad, S, lo, hi);
      // the optional outputs may be NULL
      EXPECT(sgmv_build_segments(ids.data(), n, P, perm.data(), starts.data(), seg_ad.data(), &S,
                                 nullptr, nullptr) == SGMV_OK);
      // pointer table over the segments, then the same with a misaligned base
      std::vector<uint64_t> base(P), out(S > 0 ? S : 1);
      for (int a = 0; a < P; ++a) base[a] = (uint64_t(1) << 40) + uint64_t(a) * 4096;
      EXPECT(sgmv_build_ptr_table(base.data(), P, seg_ad.data(), S, out.data()) == SGMV_OK);
      for (int s = 0; s < S; ++s) EXPECT(out[s] == base[seg_ad[s]]);
      if (S > 0) {
        base[seg_ad[0]] += 8;
        EXPECT(sgmv_build_ptr_table(base.data(), P, seg_ad.data(), S, out.data()) ==
               SGMV_ERR_ALIGNMENT);
      }
      // an id out of range, at either end of the batch
      if (n > 0) {
        std::vector<int32_t> bad = ids;
        bad[n - 1] = P;
        EXPECT(sgmv_build_segments(bad.data(), n, P, perm.data(), starts.data(), seg_ad.data(),
                                   &S, &lo, &hi) == SGMV_ERR_ADAPTER_ID);
        bad[n - 1] = ids[n - 1];
        bad[0] = -1;
        EXPECT(sgmv_build_segments(bad.data(), n, P, perm.data(), starts.data(), seg_ad.data(),
                                   &S, &lo, &hi) == SGMV_ERR_ADAPTER_ID);
      }
    }
  int32_t S = 0;
  std::vector<int32_t> v(8);
  EXPECT(sgmv_build_segments(nullptr, 4, 2, v.data(), v.data(), v.data(), &S, nullptr, nullptr) ==
         SGMV_ERR_NULL);
  EXPECT(sgmv_build_segments(v.data(), -1, 2, v.data(), v.data(), v.data(), &S, nullptr, nullptr) ==
         SGMV_ERR_SHAPE);
  EXPECT(sgmv_build_segments(v.data(), 4, 0, v.data(), v.data(), v.data(), &S, nullptr, nullptr) ==
         SGMV_ERR_SHAPE);
  const int32_t one = 0;
  uint64_t base = 1 << 20, out = 0;
  EXPECT(sgmv_build_ptr_table(&base, 1, &one, 1, &out) == SGMV_OK && out == base);
  const int32_t far = 1;
  EXPECT(sgmv_build_ptr_table(&base, 1, &far, 1, &out) == SGMV_ERR_ADAPTER_ID);
}

static void ranked_cases() {
  std::mt19937 rng(11);
  const int ranks[] = {16, 32, 64};
  for (int n : {0, 1, 40, 300, 2112})
    for (int P : {1, 3, 50}) {
      std::vector<int32_t> ids(n), rank(P);
      for (auto& t : ids) t = static_cast<int32_t>(rng() % P);
      for (auto& r : rank) r = ranks[rng() % 3];
      std::vector<int32_t> perm(n > 0 ? n : 1), starts(n + 3), seg_ad(n > 0 ? n : 1);
      sgmv_rank_group groups[3];
      int32_t G = -1;
      EXPECT(sgmv_build_segments_ranked(ids.data(), n, P, rank.data(), perm.data(), starts.data(),
                                        seg_ad.data(), groups, &G) == SGMV_OK);
      int rows = 0;
      for (int g = 0; g < G; ++g) {
        EXPECT(groups[g].row0 == rows && groups[g].n > 0);
        if (g > 0) EXPECT(groups[g - 1].r < groups[g].r);
        for (int i = 0; i < groups[g].n; ++i) EXPECT(rank[ids[perm[rows + i]]] == groups[g].r);
        EXPECT(starts[groups[g].starts0] == 0 &&
               starts[groups[g].starts0 + groups[g].n_segments] == groups[g].n);
        rows += groups[g].n;
      }
      EXPECT(rows == n);
      if (n > 0) {
        rank[ids[0]] = 24;
        EXPECT(sgmv_build_segments_ranked(ids.data(), n, P, rank.data(), perm.data(),
                                          starts.data(), seg_ad.data(), groups, &G) ==
               SGMV_ERR_UNSUPPORTED);
        rank[ids[0]] = 16;
        ids[n / 2] = P;
        EXPECT(sgmv_build_segments_ranked(ids.data(), n, P, rank.data(), perm.data(),
                                          starts.data(), seg_ad.data(), groups, &G) ==
               SGMV_ERR_ADAPTER_ID);
      }
    }
}

// the slot cache over random batches: every key of a batch gets one slot, distinct keys
// distinct slots, misses are exactly the keys that were not resident, and the cache never
// holds more keys than slots
static void cache_cases() {
  std::mt19937 rng(5);
  for (int n_slots : {1, 3, 17, 64}) {
    sgmv_slot_cache* c = nullptr;
    EXPECT(sgmv_slot_cache_create(n_slots, &c) == SGMV_OK && c);
    std::vector<int64_t> resident_before;
    for (int round = 0; round < 400; ++round) {
      const int n = static_cast<int>(rng() % (2 * n_slots + 3));
      std::vector<int64_t> keys(n);
      for (auto& k : keys) k = static_cast<int64_t>(rng() % (3 * n_slots + 1)) - 5;
      std::vector<int32_t> slots(n > 0 ? n : 1), ms(n > 0 ? n : 1), was(n > 0 ? n : 1);
      std::vector<int64_t> mk(n > 0 ? n : 1);
      for (int t = 0; t < n; ++t) EXPECT(sgmv_slot_cache_lookup(c, keys[t], &was[t]) == SGMV_OK);
      int32_t miss = -1;
      const int st = sgmv_slot_cache_map(c, keys.data(), n, slots.data(), mk.data(), ms.data(), &miss);
      std::vector<int64_t> distinct;
      for (int t = 0; t < n; ++t) {
        bool seen = false;
        for (int64_t d : distinct) seen = seen || d == keys[t];
        if (!seen) distinct.push_back(keys[t]);
      }
      if (static_cast<int>(distinct.size()) > n_slots) {
        EXPECT(st == SGMV_ERR_SHAPE);
        continue;
      }
      EXPECT(st == SGMV_OK);
      int expect_miss = 0;
      for (int64_t d : distinct) {
        int first = -1;
        for (int t = 0; t < n && first < 0; ++t)
          if (keys[t] == d) first = t;
        expect_miss += was[first] < 0;
      }
      EXPECT(miss == expect_miss);
      for (int t = 0; t < n; ++t) {
        EXPECT(slots[t] >= 0 && slots[t] < n_slots);
        int32_t now = -2;
        EXPECT(sgmv_slot_cache_lookup(c, keys[t], &now) == SGMV_OK && now == slots[t]);
        if (was[t] >= 0) EXPECT(was[t] == slots[t]);
        for (int u = 0; u < t; ++u) EXPECT((keys[u] == keys[t]) == (slots[u] == slots[t]));
      }
      if (n > 0 && round % 7 == 0) {
        EXPECT(sgmv_slot_cache_evict(c, keys[0]) == SGMV_OK);
        int32_t gone = 0;
        EXPECT(sgmv_slot_cache_lookup(c, keys[0], &gone) == SGMV_OK && gone == -1);
        EXPECT(sgmv_slot_cache_evict(c, keys[0]) == SGMV_ERR_ADAPTER_ID);
      }
    }
    sgmv_slot_cache_destroy(c);
  }
  sgmv_slot_cache* c = nullptr;
  EXPECT(sgmv_slot_cache_create(0, &c) == SGMV_ERR_SHAPE && c == nullptr);
  EXPECT(sgmv_slot_cache_create(4, nullptr) == SGMV_ERR_NULL);
  sgmv_slot_cache_destroy(nullptr);
}

static void check_cases() {
  // segment bounds, including extreme values (no overflow in the pigeonhole products)
  EXPECT(check_segments(0, 0, 0, 0) == SGMV_OK);
  EXPECT(check_segments(-1, 1, 1, 1) == SGMV_ERR_SHAPE);
  EXPECT(check_segments(32, 32, 1, 1) == SGMV_OK);
  EXPECT(check_segments(32, 16, 1, 1) == SGMV_ERR_SHAPE);
  EXPECT(check_segments(INT_MAX, INT_MAX, INT_MAX, INT_MAX) == SGMV_ERR_SHAPE);
  EXPECT(check_segments(INT_MAX, 1, INT_MAX, INT_MAX) == SGMV_OK);
  EXPECT(check_segments(INT_MAX, INT_MAX, 1, 1) == SGMV_OK);
  EXPECT(check_segments(100, 3, 0, 100) == SGMV_OK);
  EXPECT(check_segments(100, 3, 40, 30) == SGMV_ERR_SHAPE);
  // dimensions and strides
  EXPECT(check_dim(4096, 4096) == SGMV_OK);
  EXPECT(check_dim(4092, 4096) == SGMV_ERR_ALIGNMENT);
  EXPECT(check_dim(4096, 4092) == SGMV_ERR_SHAPE);
  EXPECT(check_dim(INT_MAX, LLONG_MAX) == SGMV_ERR_SHAPE);
  EXPECT(check_dim(8, LLONG_MAX - 7) == SGMV_OK);
  // byte ranges: matrix_bytes of the largest accepted shapes fits in size_t
  EXPECT(matrix_bytes(0, 4096, 4096) == 0);
  EXPECT(matrix_bytes(4096, 1 << 22, 1 << 22) == (size_t(4095) * (1 << 22) + (1 << 22)) * 2);
  const char* p = reinterpret_cast<const char*>(uintptr_t(1) << 40);
  EXPECT(ranges_overlap(p, 64, p + 63, 1));
  EXPECT(!ranges_overlap(p, 64, p + 64, 1));
  EXPECT(!ranges_overlap(p, 0, p, 16));
  // workspace layout over the accepted range of sizes
  for (int n : {0, 1, 64, 65, 4096, 1 << 20})
    for (int h : {8, 4096, 28672, int(kMaxDim)})
      for (int r : {16, 32, 64}) {
        const WsLayout L = ws_layout(n, h, r);
        EXPECT(L.rowks_off <= L.v_off && L.v_off <= L.part_off && L.part_off <= L.dtab_off &&
               L.dtab_off < L.table_end && L.table_end + pool_bytes(h, r) < L.total);
        EXPECT(pool_offset(L.total, h, r) >= L.table_end && pool_offset(L.total, h, r) % 256 == 0);
      }
  int32_t gn[3] = {0, 700, 1}, gr[3] = {16, 32, 64};
  size_t off[3];
  const size_t end = ranked_side_by_side(gn, gr, 3, 8192, off);
  EXPECT(off[0] == 0 && off[1] == 0 && off[2] > off[1] && end > off[2]);
  // status strings exist for every code and for unknown ones
  for (int code = -3; code < 16; ++code) EXPECT(sgmv_status_string(code) != nullptr);
  EXPECT(sgmv_abi_version() == SGMV_ABI_VERSION);
}

int main() {
  builder_cases();
  ranked_cases();
  cache_cases();
  check_cases();
  std::printf("ok %ld\n", g_checks);
  return 0;
}
