// Numbering of the decode wave units (request r, token split s), shared by
// the kernels and a host mirror of their lookup.  Plain integer code: no HIP
// types, so a host compiler can build it.
//
// A request of L keys is cut into splits of two lengths: `a` long splits of T
// keys from its start, then the remaining L - a*T keys ("the tail") in short
// splits of T2 <= T keys, the last one possibly shorter.  With k = 0, a =
// L / T and the tail is the remainder, one split (T2 = T); with k = 1, the
// last full long split joins the tail, which is then cut into pieces of T2
// (a = L / T - 1, or 0 when L < 2T).
//
// Units are numbered in phases, longest work first, so the last tasks to be
// claimed are the short ones and the decode's end is balanced across the
// machine (paper §4.2.3 cuts decode work into one-warp virtual CTAs; their
// lengths and order are this design's choice): phase 0 holds the long
// splits of every request, request by request.  With k = 0 the remainders
// follow in kRemBuckets phases by length, the longest eighth of [0, T)
// first (within a phase, request by request): an approximate
// longest-processing-time order.  With k = 1 phase 1 holds every request's
// short splits.  The partial record of (r, s) is base(r) + s, with base(r) =
// the splits of the requests before r, so the splits of one request are
// adjacent and the merge order does not depend on the unit order.
//
// A wave finds its unit's request with one prefix scan per 64 requests over
// a packed count: (splits of the request) << 16 | (units of the request in
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
constexpr int kRemBuckets = 8;        // remainder phases (k = 0), by length
constexpr int kUnitPhases = 1 + kRemBuckets;
static_assert((uint64_t)kUnitScanLanes * kUnitMaxSplits < (1u << 16), "packed unit counts overflow 16 bits");
static_assert(kRemBuckets == 8, "remainder phases are eighths of the split");

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

// Remainder phase (k = 0) of a remainder of 1 <= rem < T keys, with nb = 1
// (every remainder in phase 1, request order) or nb = kRemBuckets (1 for the
// longest eighth of [0, T), kRemBuckets for the shortest; T is a multiple of
// 16, so the eighths j T / 8 are exact: compares instead of a division).
POD_HD int unit_rem_phase(int rem, int T, int nb) {
  if (nb == 1) return 1;
  int ph = kRemBuckets;
  for (int j = 1; j < kRemBuckets; ++j) ph -= rem >= ((j * T) >> 3) ? 1 : 0;
  return ph;
}
// Phases in use: the long splits, then one short phase (k = 1) or nb
// remainder phases (k = 0).
POD_HD int unit_phases(int k, int nb) { return 1 + (k ? 1 : nb); }
// Units of a request of L keys in phase ph.
POD_HD uint32_t unit_count(int L, int T, int T2, int k, int ph, int nb) {
  const int a = unit_long(L, T, k);
  if (ph == 0) return (uint32_t)a;
  if (k) return ph == 1 ? (uint32_t)unit_short(L, T, T2, k) : 0u;
  const int rem = L - a * T;
  return rem > 0 && unit_rem_phase(rem, T, nb) == ph ? 1u : 0u;
}

// Packed (splits of the request, units in phase ph) of a request of L keys;
// the same counts as unit_long, unit_short and unit_count with one division
// for k = 0 (the scan evaluates this for every request).
POD_HD uint32_t unit_pack(int L, int T, int T2, int k, int ph, int nb) {
  const int F = L / T;
  const int a = F > k ? F - k : 0;
  const int tail = L - a * T;
  int b, c;
  if (k == 0) {
    b = tail > 0 ? 1 : 0;
    c = ph == 0 ? a : (tail > 0 && unit_rem_phase(tail, T, nb) == ph ? 1 : 0);
  } else {
    b = (tail + T2 - 1) / T2;
    c = ph == 0 ? a : (ph == 1 ? b : 0);
  }
  return ((uint32_t)(a + b) << 16) | (uint32_t)c;
}
POD_HD uint32_t unit_total(uint32_t x) { return x >> 16; }
POD_HD uint32_t unit_phase(uint32_t x) { return x & 0xffffu; }

// Given the request found for phase-local unit u (its packed own count `own`
// and inclusive packed prefix `incl` within its scan group, plus the phase
// and record counts `key_acc`, `base_acc` of the groups before), the split
// index s, the split count S and the record base of the request.  A
// request's units of a phase past 0 are its last splits.
POD_HD void unit_select(uint32_t u, int ph, uint32_t key_acc, uint32_t base_acc, uint32_t own, uint32_t incl,
                        int& s, int& S, int& base) {
  S = (int)unit_total(own);
  const int idx = (int)(u - key_acc - (unit_phase(incl) - unit_phase(own)));
  s = ph > 0 ? S - (int)unit_phase(own) + idx : idx;
  base = (int)(base_acc + unit_total(incl)) - S;
}

// Phase of a unit, given the first unit of each of the np phases in use
// (start[0] = 0, non-decreasing, start[np] = all units).
POD_HD int unit_phase_of(const int* start, int np, int unit) {
  int ph = 0;
  for (int q = 1; q < np; ++q) ph = unit >= start[q] ? q : ph;
  return ph;
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
// (clamped to maxlen), start[] the first unit of every phase in use.
// Returns false for a unit past the last one.
inline bool unit_locate_seq(const int32_t* ctx, int N, int maxlen, int T, int T2, int k, int nb, const int* start,
                            int unit, int& r, int& s, int& S, int& base) {
  const int np = unit_phases(k, nb);
  if (unit < 0 || unit >= start[np]) return false;
  const int ph = unit_phase_of(start, np, unit);
  const uint32_t u = (uint32_t)(unit - start[ph]);
  uint32_t key_acc = 0, base_acc = 0;
  for (int c0 = 0; c0 < N; c0 += kUnitScanLanes) {
    uint32_t own[kUnitScanLanes], incl[kUnitScanLanes], run = 0;
    for (int lane = 0; lane < kUnitScanLanes; ++lane) {
      const int idx = c0 + lane;
      int L = idx < N ? (ctx[idx] < maxlen ? ctx[idx] : maxlen) : 0;
      L = L > 0 ? L : 0;
      own[lane] = unit_pack(L, T, T2, k, ph, nb);
      run += own[lane];
      incl[lane] = run;
    }
    const uint32_t total = incl[kUnitScanLanes - 1];
    if (u < key_acc + unit_phase(total)) {
      int first = 0;
      while (!(key_acc + unit_phase(incl[first]) > u)) ++first;
      r = c0 + first;
      unit_select(u, ph, key_acc, base_acc, own[first], incl[first], s, S, base);
      return true;
    }
    key_acc += unit_phase(total);
    base_acc += unit_total(total);
  }
  return false;
}

// First unit of each phase in use for a batch (start[np] = all units).
inline void unit_phase_starts(const int32_t* ctx, int N, int T, int T2, int k, int nb, int* start) {
  const int np = unit_phases(k, nb);
  long long acc = 0;
  for (int ph = 0; ph < np; ++ph) {
    start[ph] = (int)acc;
    for (int i = 0; i < N; ++i) acc += unit_count(ctx[i] > 0 ? ctx[i] : 0, T, T2, k, ph, nb);
  }
  start[np] = (int)acc;
}

}  // namespace pod
