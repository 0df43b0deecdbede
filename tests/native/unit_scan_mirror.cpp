// Host harness for the decode-unit lookup of pod_units.h (the packing and
// selection arithmetic the kernels use, with the per-group scan done
// sequentially).  Reads "N T" then N context lengths on stdin, prints one
// line "r s S base" per unit in unit order, or "miss" for a unit the lookup
// does not find.
#include <cstdio>
#include <vector>

#include "../../prefill_decode_hybrid_amd/csrc/pod_units.h"

int main() {
  int N = 0, T = 0;
  if (std::scanf("%d %d", &N, &T) != 2 || N < 1 || T < 1) return 2;
  std::vector<int32_t> ctx(N);
  int maxlen = 0;
  long long units = 0, full = 0;
  for (int i = 0; i < N; ++i) {
    if (std::scanf("%d", &ctx[i]) != 1) return 2;
    maxlen = ctx[i] > maxlen ? ctx[i] : maxlen;
    units += (ctx[i] + T - 1) / T;
    full += ctx[i] / T;
  }
  for (long long u = 0; u < units + 1; ++u) {
    int r = -1, s = -1, S = -1, base = -1;
    if (pod::unit_locate_seq(ctx.data(), N, maxlen, T, (int)full, (int)u, r, s, S, base))
      std::printf("%d %d %d %d\n", r, s, S, base);
    else
      std::printf("miss\n");
  }
  return 0;
}
