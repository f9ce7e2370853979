// Drives the expert cache's slot policy (csrc/expert_cache_policy.h) from
// stdin so that a test can compare it with a model of the documented rules.
//   first line:  E S
//   then one request per line:
//     a <protect_from or -1> <n> <ids...>   acquire (-1: nothing protected)
//     p <n> <ids...>                        pin resident experts
//     u                                     unpin all
// After each request it prints "ok <hits> <e:s>..." or "fail", then the slot
// of every expert (-1 if not resident).
#include <cstdint>
#include <cstdio>
#include <limits>
#include <vector>

#include "expert_cache_policy.h"

int main() {
  int E = 0, S = 0;
  if (std::scanf("%d %d", &E, &S) != 2) return 2;
  qmoe::SlotPolicy pol(E, S);
  char op[4];
  while (std::scanf("%3s", op) == 1) {
    if (op[0] == 'a') {
      long long prot = 0;
      int n = 0;
      if (std::scanf("%lld %d", &prot, &n) != 2) return 2;
      std::vector<int> need(n);
      for (int& e : need)
        if (std::scanf("%d", &e) != 1) return 2;
      std::vector<std::pair<int, int>> loads;
      int hits = 0;
      const uint64_t from = prot < 0 ? std::numeric_limits<uint64_t>::max() : (uint64_t)prot;
      if (pol.acquire(need, from, loads, hits)) {
        std::printf("ok %d", hits);
        for (const auto& l : loads) std::printf(" %d:%d", l.first, l.second);
        std::printf("\n");
      } else {
        std::printf("fail\n");
      }
    } else if (op[0] == 'p') {
      int n = 0;
      if (std::scanf("%d", &n) != 1) return 2;
      std::vector<int> ex(n);
      for (int& e : ex)
        if (std::scanf("%d", &e) != 1) return 2;
      pol.pin(ex);
      std::printf("pinned %d\n", pol.n_pinned());
    } else if (op[0] == 'u') {
      pol.unpin_all();
      std::printf("pinned 0\n");
    } else {
      return 2;
    }
    for (int e = 0; e < E; ++e) std::printf("%d%c", pol.slot_of(e), e + 1 < E ? ' ' : '\n');
  }
  std::printf("clock %llu evictions %llu\n", (unsigned long long)pol.clock(),
              (unsigned long long)pol.evictions());
  return 0;
}
