// Host check of the workspace layout rule: in a buffer sized for the largest of a set of
// shapes, no call of any smaller shape writes scratch over the tagged partials of any
// other such call (the counters sit at a fixed place before all scratch), and every
// region stays inside the buffer; and the rank groups of a mixed-rank call fit side by
// side in the buffer sized for all their rows at the largest rank.  Built and run by
// tests/test_host_abi.py; prints "ok" and exits 0 when the rule holds.
#include <algorithm>
#include <cstdio>
#include <vector>

#include "../adapter_gemv_amd/csrc/sgmv_checks.h"

using namespace sgmv_host;

int main() {
  const std::vector<int> ns = {1, 16, 17, 63, 64, 65, 300, 1000, 2048, 2112, 4096};
  const std::vector<int> hs = {8, 264, 1024, 4096, 5120, 8192, 13824, 28672};
  const std::vector<int> rs = {16, 32, 64};
  const size_t front_zero_end = kWsPoolCounters + sizeof(int32_t) * kCounterInts * kMaxPoolRows;
  long checks = 0;
  for (int N : ns)
    for (int H : hs)
      for (int R : rs) {
        const size_t W = ws_layout(N, H, R).total;
        for (int n : ns) {
          if (n > N) continue;
          for (int h : hs) {
            if (h > H) continue;
            for (int r : rs) {
              if (r > R) continue;
              const WsLayout Li = ws_layout(n, h, r);
              const size_t pool = pool_offset(W, h, r);
              if (Li.rowks_off < front_zero_end || Li.table_end > pool ||
                  pool + pool_bytes(h, r) > W || pool % 256 != 0) {
                std::printf("bad layout: call (%d,%d,%d) in buffer for (%d,%d,%d)\n", n, h, r, N, H, R);
                return 1;
              }
              // this call's scratch against every other call's zero regions
              for (int n2 : ns) {
                if (n2 > N) continue;
                for (int h2 : hs) {
                  if (h2 > H) continue;
                  for (int r2 : rs) {
                    if (r2 > R) continue;
                    ++checks;
                    if (Li.table_end > pool_offset(W, h2, r2)) {
                      std::printf("overlap: scratch of (%d,%d,%d) reaches the tagged partials of (%d,%d,%d) "
                                  "in a buffer for (%d,%d,%d)\n", n, h, r, n2, h2, r2, N, H, R);
                      return 1;
                    }
                  }
                }
              }
            }
          }
        }
      }
  // mixed-rank calls: sgmv_lora_add_ranked puts the groups' scratch side by side only when
  // it ends within the scratch of one call of all rows at the largest rank (a call the
  // buffer is sized for, whose scratch the loops above keep clear of every zero region);
  // then each group's scratch starts after the counters and after the previous group's.
  // Groups of distinct ranks with at least 16 rows each (the mixed-rank workloads) always
  // fit that way.
  long fits = 0;
  const std::vector<int> Ns = {2, 65, 300, 2112, 4096};
  for (int N : Ns)
    for (int H : hs)
      for (int R : rs) {
        const size_t W = ws_layout(N, H, R).total;
        for (int parts = 2; parts <= 3; ++parts)
          for (int cut = 1; cut < 8; ++cut) {
            int32_t gn[3], gr[3];
            size_t off[3];
            int left = N;
            for (int g = 0; g < parts; ++g) {
              gn[g] = (g == parts - 1) ? left : std::min(left, (N * cut) / (8 * (parts - 1)) + g);
              left -= gn[g];
              gr[g] = rs[(g + cut) % rs.size()];
              if (gr[g] > R) gr[g] = R;
            }
            const size_t end = ranked_side_by_side(gn, gr, parts, H, off);
            ++checks;
            bool distinct = true, tall = true;
            for (int g = 0; g < parts; ++g) {
              tall = tall && gn[g] >= 16;
              for (int g2 = 0; g2 < g; ++g2) distinct = distinct && gr[g] != gr[g2];
            }
            if (end > ws_layout(N, H, R).table_end) {
              if (distinct && tall) {
                std::printf("ranked: groups of distinct ranks, %d rows (H %d, R %d, %d parts, cut %d) "
                            "do not fit side by side\n", N, H, R, parts, cut);
                return 1;
              }
              continue;  // run one after another
            }
            ++fits;
            size_t prev_end = front_zero_end;
            for (int g = 0; g < parts; ++g) {
              if (gn[g] <= 0) continue;
              const WsLayout L = ws_layout(gn[g], H, gr[g]);
              if (off[g] % 256 != 0 || off[g] + L.rowks_off < prev_end) {
                std::printf("ranked: group %d overlaps (N %d, H %d, R %d)\n", g, N, H, R);
                return 1;
              }
              prev_end = off[g] + L.table_end;
            }
          }
      }
  if (fits == 0) {
    std::printf("ranked: no partition fits side by side\n");
    return 1;
  }
  std::printf("ok %ld\n", checks);
  return 0;
}
