// Numbering of the decode wave units (request r, token split s), shared by
// the kernels and a host mirror of their lookup.  Plain integer code: no HIP
// types, so a host compiler can build it.
//
// A request of L keys is cut into splits of two lengths: `a` long splits of T
// keys from its start, then the remaining L - a*T keys ("the tail") in short
// splits of T2 <= T keys, the last one possibly shorter.  With k = 0, a =
// L / T and the tail is the remainder, one split (T2 = T); with k = 1, the
// last full long split joins the tail, which is then cut into pieces of T2
// (a = L / T - 1, or 0 when L < 2T).  Units are numbered long phase first:
// the long splits of every request (request by request), then the short
// ones, so the last tasks to be claimed are short and the decode's end is
// balanced across the machine (paper §4.2.3 cuts decode work into one-warp
// virtual CTAs; their lengths and order are this design's choice).  The
// partial record of (r, s) is base(r) + s, with base(r) = the splits of the
// requests before r, so the splits of one request are adjacent.
//
// A wave finds its unit's request with one prefix scan per 64 requests over
// a packed count: (splits of the request) << 16 | (splits of the request in
// the unit's phase), summed as uint32_t.  Each half stays below 2^16 because
// a request has at most kUnitMaxSplits splits and 64 * 1023 < 65536, so the
// halves never carry into each other or into the sign bit.  A request has at
// most ceil(L / T2) splits, so T2 >= L / 1023 keeps it within the bound.
#pragma once

#include <cstdint>

#if defined(__HIP__)  // compiled as HIP: callable from kernels too
#define POD_HD __attribute__((host, device, always_inline)) inline
#else
#define POD_HD inline
#endif

namespace pod {

constexpr int kUnitMaxSplits = 1023;  // splits of one request
constexpr int kUnitScanLanes = 64;    // requests per scan step
static_assert((uint64_t)kUnitScanLanes * kUnitMaxSplits < (1u << 16), "packed unit counts overflow 16 bits");

// Long splits of a request of L keys.
POD_HD int unit_long(int L, int T, int k) {
  const int F = L / T;
  return F > k ? F - k : 0;
}
// Short splits of the same request (the tail cut into pieces of T2).
POD_HD int unit_short(int L, int T, int T2, int k) {
  const int tail = L - unit_long(L, T, k) * T;
  return (tail + T2 - 1) / T2;
}

// Packed (splits of the request, splits in the phase) of a request of L keys.
POD_HD uint32_t unit_pack(int L, int T, int T2, int k, bool short_phase) {
  const uint32_t a = (uint32_t)unit_long(L, T, k), b = (uint32_t)unit_short(L, T, T2, k);
  return ((a + b) << 16) | (short_phase ? b : a);
}
POD_HD uint32_t unit_total(uint32_t x) { return x >> 16; }
POD_HD uint32_t unit_phase(uint32_t x) { return x & 0xffffu; }

// Given the request found for phase-local unit u (its packed own count `own`
// and inclusive packed prefix `incl` within its scan group, plus the phase
// and record counts `key_acc`, `base_acc` of the groups before), the split
// index s, the split count S and the record base of the request.  The short
// splits of a request follow its long ones.
POD_HD void unit_select(uint32_t u, bool short_phase, uint32_t key_acc, uint32_t base_acc, uint32_t own,
                        uint32_t incl, int& s, int& S, int& base) {
  S = (int)unit_total(own);
  const int idx = (int)(u - key_acc - (unit_phase(incl) - unit_phase(own)));
  s = short_phase ? S - (int)unit_phase(own) + idx : idx;
  base = (int)(base_acc + unit_total(incl)) - S;
}

// Keys [t0, t1) of split s of a request of L keys.
POD_HD void unit_range(int L, int T, int T2, int k, int s, int& t0, int& t1) {
  const int a = unit_long(L, T, k);
  if (s < a) {
    t0 = s * T;
    t1 = t0 + T;
  } else {
    t0 = a * T + (s - a) * T2;
    t1 = t0 + T2 < L ? t0 + T2 : L;
  }
}

// Host mirror of the kernels' lookup (the per-group prefix scan done
// sequentially instead of across lanes).  ctx[N] are the context lengths
// (clamped to maxlen), n_long = the number of long-phase units.  Returns
// false for a unit past the last one.
inline bool unit_locate_seq(const int32_t* ctx, int N, int maxlen, int T, int T2, int k, int n_long, int unit,
                            int& r, int& s, int& S, int& base) {
  const bool sp = unit >= n_long;
  const uint32_t u = (uint32_t)(sp ? unit - n_long : unit);
  uint32_t key_acc = 0, base_acc = 0;
  for (int c0 = 0; c0 < N; c0 += kUnitScanLanes) {
    uint32_t own[kUnitScanLanes], incl[kUnitScanLanes], run = 0;
    for (int lane = 0; lane < kUnitScanLanes; ++lane) {
      const int idx = c0 + lane;
      int L = idx < N ? (ctx[idx] < maxlen ? ctx[idx] : maxlen) : 0;
      L = L > 0 ? L : 0;
      own[lane] = unit_pack(L, T, T2, k, sp);
      run += own[lane];
      incl[lane] = run;
    }
    const uint32_t total = incl[kUnitScanLanes - 1];
    if (u < key_acc + unit_phase(total)) {
      int first = 0;
      while (!(key_acc + unit_phase(incl[first]) > u)) ++first;
      r = c0 + first;
      unit_select(u, sp, key_acc, base_acc, own[first], incl[first], s, S, base);
      return true;
    }
    key_acc += unit_phase(total);
    base_acc += unit_total(total);
  }
  return false;
}

}  // namespace pod
