// Numbering of the decode wave units (request r, token split s), shared by
// the kernels and a host mirror of their lookup.  Plain integer code: no HIP
// types, so a host compiler can build it.
//
// A request of L keys with split length T has S = ceil(L / T) splits: L / T
// full ones and, if T does not divide L, one shorter remainder.  Units are
// numbered longest first: the full splits of every request (request by
// request), then the remainders, so the last tasks to be claimed are the
// short ones (paper §4.2.3 cuts decode work into one-warp virtual CTAs; how
// they are ordered is this design's choice).  The partial record of (r, s)
// is base(r) + s, with base(r) = the splits of the requests before r, so the
// splits of one request are adjacent.
//
// A wave finds its unit's request with one prefix scan per 64 requests over
// a packed count: (splits of the request) << 16 | (splits of the request in
// the unit's phase), summed as uint32_t.  Each half stays below 2^16 because
// a request has at most kUnitMaxSplits splits and 64 * 1023 < 65536, so the
// halves never carry into each other or into the sign bit.
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

// Packed (splits of the request, splits in the phase) of a request of L keys.
POD_HD uint32_t unit_pack(int L, int T, bool rem_phase) {
  const uint32_t full = (uint32_t)(L / T), part = (L % T) ? 1u : 0u;
  return ((full + part) << 16) | (rem_phase ? part : full);
}
POD_HD uint32_t unit_total(uint32_t x) { return x >> 16; }
POD_HD uint32_t unit_phase(uint32_t x) { return x & 0xffffu; }

// Given the request found for phase-local unit u (its packed own count `own`
// and inclusive packed prefix `incl` within its scan group, plus the phase
// and record counts `key_acc`, `base_acc` of the groups before), the split
// index s, the split count S and the record base of the request.
POD_HD void unit_select(uint32_t u, bool rem_phase, uint32_t key_acc, uint32_t base_acc, uint32_t own, uint32_t incl,
                        int& s, int& S, int& base) {
  S = (int)unit_total(own);
  s = rem_phase ? S - 1 : (int)(u - key_acc - (unit_phase(incl) - unit_phase(own)));
  base = (int)(base_acc + unit_total(incl)) - S;
}

// Host mirror of the kernels' lookup (the per-group prefix scan done
// sequentially instead of across lanes).  ctx[N] are the context lengths
// (clamped to maxlen), full = the number of full-split units.  Returns false
// for a unit past the last one.
inline bool unit_locate_seq(const int32_t* ctx, int N, int maxlen, int T, int full, int unit, int& r, int& s, int& S,
                            int& base) {
  const bool rem = unit >= full;
  const uint32_t u = (uint32_t)(rem ? unit - full : unit);
  uint32_t key_acc = 0, base_acc = 0;
  for (int c0 = 0; c0 < N; c0 += kUnitScanLanes) {
    uint32_t own[kUnitScanLanes], incl[kUnitScanLanes], run = 0;
    for (int lane = 0; lane < kUnitScanLanes; ++lane) {
      const int idx = c0 + lane;
      int L = idx < N ? (ctx[idx] < maxlen ? ctx[idx] : maxlen) : 0;
      L = L > 0 ? L : 0;
      own[lane] = unit_pack(L, T, rem);
      run += own[lane];
      incl[lane] = run;
    }
    const uint32_t total = incl[kUnitScanLanes - 1];
    if (u < key_acc + unit_phase(total)) {
      int first = 0;
      while (!(key_acc + unit_phase(incl[first]) > u)) ++first;
      r = c0 + first;
      unit_select(u, rem, key_acc, base_acc, own[first], incl[first], s, S, base);
      return true;
    }
    key_acc += unit_phase(total);
    base_acc += unit_total(total);
  }
  return false;
}

}  // namespace pod
