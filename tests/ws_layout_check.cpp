// Host check of the workspace layout rule: in a buffer sized for the largest of a set of
// shapes, no call of any smaller shape writes scratch over the tagged partials of any
// other such call (the counters sit at a fixed place before all scratch), and every
// region stays inside the buffer.  Built and run by
// tests/test_host_abi.py; prints "ok" and exits 0 when the rule holds.
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
  std::printf("ok %ld\n", checks);
  return 0;
}
