// Host harness for the decode-unit lookup of pod_units.h (the packing and
// selection arithmetic the kernels use, with the per-group scan done
// sequentially).  Reads "N T T2 k nb" then N context lengths on stdin, prints
// one line "r s S base t0 t1" per unit in unit order, or "miss" for a unit
// the lookup does not find.
#include <cstdio>
#include <vector>

#include "../../prefill_decode_hybrid_amd/csrc/pod_units.h"

int main() {
  int N = 0, T = 0, T2 = 0, k = 0, nb = 1;
  if (std::scanf("%d %d %d %d %d", &N, &T, &T2, &k, &nb) != 5 || N < 1 || T < 1 || T2 < 1 || k < 0 || k > 1 ||
      (nb != 1 && nb != pod::kRemBuckets))
    return 2;
  std::vector<int32_t> ctx(N);
  int maxlen = 0;
  for (int i = 0; i < N; ++i) {
    if (std::scanf("%d", &ctx[i]) != 1) return 2;
    maxlen = ctx[i] > maxlen ? ctx[i] : maxlen;
  }
  int start[pod::kUnitPhases + 1];
  pod::unit_phase_starts(ctx.data(), N, T, T2, k, nb, start);
  for (int u = 0; u < start[pod::unit_phases(k, nb)] + 1; ++u) {
    int r = -1, s = -1, S = -1, base = -1;
    if (pod::unit_locate_seq(ctx.data(), N, maxlen, T, T2, k, nb, start, u, r, s, S, base)) {
      int t0 = 0, t1 = 0;
      pod::unit_range(ctx[r], T, T2, k, s, t0, t1);
      std::printf("%d %d %d %d %d %d\n", r, s, S, base, t0, t1);
    } else {
      std::printf("miss\n");
    }
  }
  return 0;
}
