// Host-side planner; see pod_plan.h.
#include "pod_plan.h"

#include <algorithm>
#include <cmath>
#include <vector>

#include "../../include/pod_attn.h"

namespace pod {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int check_shape(const Shape& s) {
  if (s.hq <= 0 || s.hkv <= 0 || s.d <= 0 || s.page <= 0) return POD_ERR_INVALID_ARG;
  if (s.hq % s.hkv != 0) return POD_ERR_UNSUPPORTED;
  const int G = s.hq / s.hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return POD_ERR_UNSUPPORTED;
  if (s.page != kPageSize) return POD_ERR_UNSUPPORTED;
  if (s.dtype == kBf16) {
    if (s.d != 64 && s.d != 128) return POD_ERR_UNSUPPORTED;
  } else if (s.dtype == kF32) {
    if (s.d != 64) return POD_ERR_UNSUPPORTED;
  } else {
    return POD_ERR_UNSUPPORTED;
  }
  return POD_OK;
}

static void tile_geometry(const Shape& s, int wg, int& rpw, int& hpt, int& row_waves, int& rpt, int& hgroups) {
  rpw = rows_per_wave(s.dtype, wg);
  hpt = std::min(s.G, kWavesPerWG);
  row_waves = kWavesPerWG / hpt;
  rpt = rpw * row_waves;
  hgroups = s.G / hpt;
}

void derive_capacities(const Shape& s, Limits& lim) {
  // the largest counts over the envelopes this handle may plan with
  lim.cap_tiles = 0;
  lim.cap_prefill_tasks = 1;
  lim.cap_rowhead_tasks = 0;
  for (int wg : {2, 4}) {
    if (!envelope_allowed(s.dtype, lim.wg_per_cu, wg)) continue;
    int rpw, hpt, rw, rpt, hg;
    tile_geometry(s, wg, rpw, hpt, rw, rpt, hg);
    const int64_t slots = (int64_t)lim.num_cus * wg;
    // max_chunk_len bounds the rows of all chunks of a call; each chunk but
    // the first may add one partial row block
    const int64_t rows = std::max(1, lim.max_chunk_len);
    const int64_t tiles = (ceil_div(rows, rpt) + std::min<int64_t>(kMaxChunks, rows) - 1) * s.hkv * hg;
    const int64_t finest = ceil_div(std::max(1, lim.max_context),
                                    s.dtype == kBf16 ? kMinPrefillSplitKeys : kMinPrefillSplitKeysF32);
    int64_t tasks = std::max<int64_t>({1, std::max(lim.cap_waves, 2) * slots + tiles,
                                       tiles * ceil_div(std::max(1, lim.max_context), kMaxSplitKeys)});
    if (lim.cap_waves < 0) tasks = std::max(tasks, tiles * finest);
    if (lim.prefill_splits > 0) tasks = std::max(tasks, tiles * std::min<int64_t>(lim.prefill_splits, finest));
    lim.cap_tiles = std::max(lim.cap_tiles, tiles);
    lim.cap_prefill_tasks = std::max(lim.cap_prefill_tasks, tasks);
    lim.cap_rowhead_tasks = std::max<int64_t>(lim.cap_rowhead_tasks, tasks * rpw * kWavesPerWG);
  }
  int64_t total = lim.max_total_context > 0 ? lim.max_total_context
                                            : (int64_t)lim.max_num_decode * lim.max_context;
  lim.cap_wave_tasks =
      (int64_t)s.hkv * (lim.max_num_decode + ceil_div(total, min_split_tokens(s.dtype, lim.max_context)));
}

WorkspaceLayout workspace_layout(const Shape& s, const Limits& lim) {
  WorkspaceLayout w;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  size_t at = 0;
  w.ctrl = at;
  at = align(at + kCtrlWords * 4);
  w.tickets = at;
  at = align(at + kTicketSlots * 4);
  w.p_cnt = at;
  at = align(at + (size_t)std::max<int64_t>(1, lim.cap_tiles) * 4);
  w.d_cnt = at;
  at = align(at + (size_t)std::max(1, lim.max_num_decode) * s.hkv * 4);
  w.p_part = at;
  at = align(at + (size_t)lim.cap_rowhead_tasks * (s.d + 2) * 4);
  w.d_part = at;
  const int G = s.hq / s.hkv;
  const size_t rec = ((size_t)G * (s.d + 2) + 3) & ~size_t(3);  // 16-byte records
  at = align(at + (size_t)std::max<int64_t>(1, lim.cap_wave_tasks) * rec * 4);
  w.trace = at;
  if (lim.record_roles)
    w.trace_bytes = (size_t)(lim.cap_prefill_tasks + (lim.cap_wave_tasks + kWavesPerWG - 1) / kWavesPerWG + 1) *
                    kTraceRecordBytes;
  at = align(at + w.trace_bytes);
  w.total = at;
  return w;
}

WorkspaceLayout workspace_layout_for_plan(const Shape& s, const Plan& pl) {
  Limits lim;
  lim.cap_tiles = pl.has_p ? pl.tiles : 0;
  bool split = false;
  for (int k = 0; pl.has_p && k < pl.n_chunks; ++k) split |= pl.ch[k].splits > 1;
  lim.cap_prefill_tasks = split ? pl.p_tasks : 0;  // partials only where tiles are split
  lim.cap_rowhead_tasks = lim.cap_prefill_tasks * pl.rows_per_wave * kWavesPerWG;
  lim.max_num_decode = pl.has_d ? pl.N : 0;
  lim.cap_wave_tasks = pl.has_d ? pl.d_wave_tasks : 0;
  return workspace_layout(s, lim);
}

static void reduce_share(int64_t a, int64_t b, int& num, int& den) {
  // prefill share a / (a + b) as num / kShareDen, at least 1 of each role
  double rho = (double)a / (double)(a + b);
  num = (int)std::lround(rho * kShareDen);
  num = std::min(kShareDen - 1, std::max(1, num));
  den = kShareDen;
}

// Plan one call for the envelope of `wg` co-resident workgroups per CU.
static int plan_wg(const Shape& s, const Limits& lim, int wg, int mode, const PrefillIn& p, const DecodeIn& d,
                   Plan* out) {
  if (!out) return POD_ERR_INVALID_ARG;
  int rc = check_shape(s);
  if (rc) return rc;
  Plan pl;
  pl.mode = mode;
  pl.num_cus = lim.num_cus;
  pl.wg_per_cu = wg;
  pl.policy = lim.policy;
  if (lim.num_cus <= 0) return POD_ERR_INVALID_ARG;

  bool want_p = (mode == kModeHybrid || mode == kModePrefill);
  bool want_d = (mode == kModeHybrid || mode == kModeDecode);
  if (mode == kModePrefill && !p.present) return POD_ERR_INVALID_ARG;
  if (mode == kModeDecode && !d.present) return POD_ERR_INVALID_ARG;
  if (mode == kModeHybrid && !p.present && !d.present) return POD_ERR_INVALID_ARG;
  if (mode == kModeHybrid && !d.present) pl.fallback = 1;
  if (mode == kModeHybrid && !p.present) pl.fallback = 2;
  pl.has_p = want_p && p.present;
  pl.has_d = want_d && d.present;

  const int64_t slots = (int64_t)lim.num_cus * wg;

  if (pl.has_p) {
    if (p.n < 1 || p.n > kMaxChunks || p.stride < 0) return POD_ERR_INVALID_ARG;
    int64_t rows = 0;
    int row_base[kMaxChunks], order[kMaxChunks];
    for (int c = 0; c < p.n; ++c) {
      const int64_t Lp = (int64_t)p.C[c] + p.P0[c];
      if (p.C[c] < 1 || p.P0[c] < 0 || Lp > lim.max_context) return POD_ERR_INVALID_ARG;
      if (p.stride > 0 && ceil_div(Lp, kPageSize) > p.stride) return POD_ERR_INVALID_ARG;
      row_base[c] = (int)rows;
      rows += p.C[c];
      order[c] = c;
    }
    if (rows > lim.max_chunk_len) return POD_ERR_INVALID_ARG;
    tile_geometry(s, wg, pl.rows_per_wave, pl.heads_per_tile, pl.row_waves, pl.rows_per_tile,
                  pl.head_groups);
    // Tasks run chunk by chunk, the longest key range first (its tiles take
    // longest), the caller's order among equals.
    std::stable_sort(order, order + p.n,
                     [&](int a, int b) { return p.C[a] + p.P0[a] > p.C[b] + p.P0[b]; });
    pl.n_chunks = p.n;
    pl.stride = p.stride;
    int64_t tiles = 0;
    double work = 0.0;  // tiles x keys
    for (int k = 0; k < p.n; ++k) {
      ChunkPlan& ch = pl.ch[k];
      ch.src = order[k];
      ch.C = p.C[ch.src];
      ch.P0 = p.P0[ch.src];
      ch.Lp = ch.C + ch.P0;
      ch.row_base = row_base[ch.src];
      ch.row_blocks = (int)ceil_div(ch.C, pl.rows_per_tile);
      ch.tiles = ch.row_blocks * s.hkv * pl.head_groups;
      ch.tile_base = (int)tiles;
      tiles += ch.tiles;
      work += (double)ch.tiles * ch.Lp;
    }
    if (tiles > lim.cap_tiles) return POD_ERR_WORKSPACE;
    pl.tiles = (int)tiles;
    const int bn = keys_per_block(s.dtype);
    // KV splits.  When the tiles do not fill the machine, the average tile
    // is split s_par ways -- enough for one wave of workgroups, and at most
    // cap_waves waves in all (paper §4.2.3 caps chunked-prefill splits at
    // two waves so that the prefill cannot crowd out the decodes) -- and
    // each chunk in proportion to its key range, so tasks carry similar
    // numbers of keys; a split added for parallelism keeps at least
    // min_keys keys, and no split exceeds kMaxSplitKeys (its page ids are
    // staged in LDS).  Without the cap (cap_waves < 0) every tile is split
    // as finely as min_keys allows; prefill_splits > 0 fixes the count.
    const int min_keys = s.dtype == kBf16 ? kMinPrefillSplitKeys : kMinPrefillSplitKeysF32;
    auto assign = [&](int64_t s_par) {
      int64_t tasks = 0;
      for (int k = 0; k < p.n; ++k) {
        ChunkPlan& ch = pl.ch[k];
        int64_t sp = 1;
        if (lim.prefill_splits > 0) {
          sp = std::min<int64_t>(lim.prefill_splits, ceil_div(ch.Lp, min_keys));
        } else if (lim.cap_waves < 0) {
          sp = ceil_div(ch.Lp, min_keys);
        } else if (s_par > 1) {
          sp = (int64_t)std::floor((double)s_par * (double)tiles * ch.Lp / work);
          sp = std::max<int64_t>(1, std::min<int64_t>(sp, ceil_div(ch.Lp, min_keys)));
        }
        sp = std::max<int64_t>(sp, ceil_div(ch.Lp, kMaxSplitKeys));
        ch.split_keys = (int)round_up(ceil_div(ch.Lp, sp), bn);
        ch.splits = (int)ceil_div(ch.Lp, ch.split_keys);  // drop splits left empty by rounding
        ch.task_base = (int)tasks;
        tasks += (int64_t)ch.tiles * ch.splits;
      }
      return tasks;
    };
    int64_t s_par = 1;
    if (tiles < slots && lim.cap_waves > 0)
      s_par = std::max<int64_t>(1, std::min<int64_t>(ceil_div(slots, tiles), lim.cap_waves * slots / tiles));
    int64_t tasks = assign(s_par);
    if (tasks > lim.cap_prefill_tasks) tasks = assign(1);
    bool split = false;
    for (int k = 0; k < p.n; ++k) {
      split |= pl.ch[k].splits > 1;
      if (pl.ch[k].split_keys > kMaxSplitKeys) return POD_ERR_WORKSPACE;
    }
    if (tasks > (1LL << 30) || (split && tasks > lim.cap_prefill_tasks)) return POD_ERR_WORKSPACE;
    pl.p_tasks = (int)tasks;
  }

  if (pl.has_d) {
    if (d.N < 1 || d.N > lim.max_num_decode || d.stride < 1 || !d.ctx_host) return POD_ERR_INVALID_ARG;
    int64_t total = 0;
    int longest = 0;
    for (int r = 0; r < d.N; ++r) {
      int L = d.ctx_host[r];
      if (L < 1 || L > lim.max_context || (int64_t)L > (int64_t)d.stride * kPageSize)
        return POD_ERR_INVALID_ARG;
      total += L;
      longest = std::max(longest, L);
    }
    int64_t cap_total = lim.max_total_context > 0 ? lim.max_total_context
                                                  : (int64_t)lim.max_num_decode * lim.max_context;
    if (total > cap_total) return POD_ERR_INVALID_ARG;
    pl.N = d.N;
    pl.d_total = total;
    pl.d_max = longest;
  }

  // Prefill workgroups kept running per CU (CU-balanced policy), in 1/256
  // of a workgroup.  One decode workgroup per CU already streams KV at the
  // chip's bandwidth, while a prefill tile runs about 1.45x slower with one
  // workgroup per CU than with two.  So from the time each role needs alone
  // (prefill: its FLOPs at the tile's rate, or one task's duration if the
  // chunk has few tasks):
  //  * prefill longer: prefill takes every slot and decode fills its tail;
  //  * prefill under 4/11 of decode: decode first, prefill fills the tail.
  //    Decode streams KV at ~83% of the HBM peak on its own, so a short
  //    prefill has little to hide behind; sharing the CUs with it slowed
  //    the decode by more than the prefill took alone (measured on every
  //    512-token chunk of a 16K prompt beside 64 16K decodes, on
  //    1024-token chunks up to offset 11K and 2048-token chunks up to 4K;
  //    from 12K and 6K on, the overlap below won);
  //  * otherwise, a large batch: the roles overlap on every CU (the
  //    method's premise) with 1.375 prefill slots per CU on average -- a
  //    decode workgroup beside a prefill one streams at close to its full
  //    rate while the prefill keeps its tail short (measured on the
  //    long-context batch and on late 1024- and 2048-token chunks of a 16K
  //    prompt beside 64 16K decodes: 1.375 at least as fast as 1.5 on every
  //    one, up to 3% faster, and both well ahead of 1.25 and 1.75);
  //  * otherwise (a small batch): as many prefill slots as prefill tasks,
  //    so every tile starts at once beside the decodes.
  if (pl.has_p && pl.has_d) {
    const double es = s.dtype == kBf16 ? 2.0 : 4.0;
    double f_p = 0.0, t_task = 0.0;
    for (int k = 0; k < pl.n_chunks; ++k) {
      const ChunkPlan& ch = pl.ch[k];
      f_p += 4.0 * s.d * s.hq * ((double)ch.C * ch.P0 + 0.5 * ch.C * (ch.C + 1.0));
      t_task = std::max(t_task, (double)std::min(ch.Lp, ch.split_keys) * kPrefillSecondsPerKey);
    }
    const double t_p = std::max(t_task, f_p / (s.dtype == kBf16 ? kPrefillFlopsBf16 : kPrefillFlopsF32));
    const double t_d = 2.0 * s.hkv * s.d * es * (double)pl.d_total / kDecodeBytesPerS;
    pl.t_prefill = t_p;
    pl.t_decode = t_d;
    if (lim.slots_x256 > 0)
      pl.cu_prefill_x256 = std::min(lim.slots_x256, 256 * wg);
    else if (t_p >= t_d)
      pl.cu_prefill_x256 = 256 * wg;
    else if (2.75 * t_p < t_d)
      pl.cu_prefill_x256 = 0;
    else if (t_d >= kOverlapMinSeconds)
      pl.cu_prefill_x256 = 176 * wg;  // 1.375 of 2 slots
    else
      pl.cu_prefill_x256 = (int)std::max<int64_t>(1, std::min<int64_t>(128 * wg, 256LL * pl.p_tasks / lim.num_cus));
  }

  if (pl.has_d) {
    // Decode token splits.  Every wave task pays a start (locate the unit,
    // page ids, first loads) and a merge, so tasks are as long as the load
    // balance allows: about one wave task per 1.6 resident decode waves, and
    // no longer than the median context, so a batch of very unequal contexts
    // keeps enough tasks to balance (measured: 4096-token splits beat 1024 by
    // ~6% on the 64 x 16K batch; 2048 beat 1024 and 4096 on 256 log-uniform
    // contexts; 512 beat 256 and 1024 on 32 contexts of 1-4K).  The split
    // depends on the decode batch alone, so a decode's result is the same
    // bits whether or not a prefill chunk shares its launch.
    std::vector<int> lens(d.ctx_host, d.ctx_host + d.N);
    std::nth_element(lens.begin(), lens.begin() + d.N / 2, lens.end());
    const int64_t median = lens[d.N / 2];
    pl.d_median = (int)median;
    const int64_t target = (int64_t)lim.num_cus * 5;
    int64_t T = round_up(std::min(ceil_div(pl.d_total * s.hkv, target), median), kPageSize);
    T = std::min<int64_t>(kMaxSplitTokens, std::max<int64_t>(min_split_tokens(s.dtype, lim.max_context), T));
    if (lim.split_tokens > 0) T = lim.split_tokens;
    pl.T = (int)T;
    // Optionally the tail of every request (its last full long split and
    // the remainder) is cut into short splits, numbered after all long ones,
    // so the decode's last tasks are short.  Not the planner's choice: side
    // by side on MI355X, quarter-length tail splits made the long-context
    // batch 6% slower fused and 10% slower alone (the decode streams best
    // with one T-token unit per resident wave), the decode-heavy batch 4%
    // slower, and only the prefill-heavy batch 2% faster (its decode runs in
    // the prefill's tail).
    int64_t T2 = T;
    if (lim.tail_split_tokens > 0) T2 = lim.tail_split_tokens;
    if (T2 >= T) {
      pl.T2 = (int)T;
      pl.tail_k = 0;
    } else {
      pl.T2 = (int)T2;
      pl.tail_k = 1;
    }
    // the kernels' unit scan holds at most kMaxSplitsPerRequest splits per
    // request; a request has at most ceil(L / T2) of them
    if (ceil_div(pl.d_max, pl.T2) > kMaxSplitsPerRequest) return POD_ERR_UNSUPPORTED;
    // Units are numbered phase by phase: the long splits, then the tail
    // splits (k = 1) or the remainders.  A decode-only launch takes the
    // remainders longest first in eight length classes, which shortened its
    // end on 256 log-uniform contexts (decode alone 1088-1094 -> 1050-1059
    // us), and so does a decode-first fused launch of several rounds, whose
    // decode runs the same way (workgroup-id order, below) with the short
    // prefill in its tail.  Other fused launches keep request order: there
    // the prefill fills the decode's end and the length classes cost 1-3%
    // in the lookup.  The order never changes a result (a split's record
    // index does not depend on it), nor the number of units.
    int64_t per_phase[kUnitPhases] = {};
    auto count_units = [&](int nb) {
      const int np_nb = unit_phases(pl.tail_k, nb);
      int64_t n = 0;
      for (int ph = 0; ph < kUnitPhases; ++ph) per_phase[ph] = 0;
      for (int r = 0; r < d.N; ++r)
        for (int ph = 0; ph < np_nb; ++ph)
          per_phase[ph] += unit_count(d.ctx_host[r], pl.T, pl.T2, pl.tail_k, ph, nb);
      for (int ph = 0; ph < np_nb; ++ph) n += per_phase[ph];
      return n;
    };
    const int64_t units = count_units(1);
    if (units > (1LL << 30)) return POD_ERR_WORKSPACE;
    const bool decode_first_rounds = pl.has_p && wg == 2 && !lim.persistent && lim.policy == kPolicyCuBalanced &&
                                     pl.cu_prefill_x256 == 0 && ceil_div(units * s.hkv, kWavesPerWG) > slots;
    pl.rem_buckets = (!pl.has_p || decode_first_rounds) ? kRemBuckets : 1;
    if (pl.rem_buckets != 1) count_units(pl.rem_buckets);
    const int np = unit_phases(pl.tail_k, pl.rem_buckets);
    int64_t acc = 0;
    for (int ph = 0; ph < np; ++ph) {
      pl.phase_start[ph] = (int)acc;
      acc += per_phase[ph];
    }
    for (int ph = np; ph <= kUnitPhases; ++ph) pl.phase_start[ph] = (int)acc;
    int64_t wt = units * s.hkv;
    if (wt > lim.cap_wave_tasks || wt > (1LL << 30)) return POD_ERR_WORKSPACE;
    pl.d_wave_tasks = (int)wt;
    pl.d_wg_tasks = (int)ceil_div(wt, kWavesPerWG);
  }

  pl.grid = (pl.has_p ? pl.p_tasks : 0) + (pl.has_d ? pl.d_wg_tasks : 0);
  // A prefill-first launch of several rounds (the prefill takes every slot
  // and outlasts one round) hands the roles out by proportional tickets: the
  // decode workgroups then run spread over the launch beside prefill tiles
  // instead of after them, where the last prefill round's ragged end left
  // most slots idle (prefill-heavy batch, side by side in one process:
  // 2320-2324 -> 2273 us; 1-2% on two earlier boxes).  Prefill slots fixed
  // in the config keep the CU-balanced rule they ask for.
  if (pl.has_p && pl.has_d && !lim.persistent && lim.policy == kPolicyCuBalanced && lim.slots_x256 == 0 &&
      pl.cu_prefill_x256 == 256 * wg && pl.grid > slots)
    pl.policy = kPolicyProportional;
  // Roles by workgroup id instead of claims, when that runs the same
  // schedule without the claims' atomics in front of the work: decode first
  // with every decode workgroup resident at once, or a launch whose whole
  // grid is resident at once (prefill first: the dispatcher spreads the
  // first workgroup ids over the CUs).  A decode-first launch of several
  // rounds also hands the decode tasks to the first ids, in the decode-only
  // launch's length-class order, and the prefill's to the last: on 256
  // log-uniform decodes beside a 256-row chunk, 1082 us against 1102-1123
  // with claims in request order and 1096 for the split launches back to
  // back (by id in request order it measured 1117, prefill first by id 1097
  // with the classes and 1133 without).  Other launches of several rounds
  // keep the claims, which balance the CUs and XCDs as workgroups come and
  // go.
  if (pl.has_p && pl.has_d && !lim.persistent && lim.policy == kPolicyCuBalanced) {
    if (pl.cu_prefill_x256 == 0 && pl.d_wg_tasks <= slots)
      pl.fixed_order = 2;
    else if (pl.grid <= slots)
      pl.fixed_order = 1;
    else if (pl.cu_prefill_x256 == 0 && pl.rem_buckets != 1)
      pl.fixed_order = 2;
  }
  // Prefill waves issue above co-resident decode waves where the prefill is
  // the longer role or runs in the decode's tail.  When a decode-first
  // launch starts every workgroup in the first round, the decode is the
  // critical path from the start, and the roles issue at equal priority
  // (measured: the small Llama-3-8B batch 81.5 -> 77.5 us; decode-first
  // chunks of a 16K prompt beside 64 16K decodes, whose prefill runs in the
  // decode's tail, lost 4-6% at equal priority).
  if (pl.fixed_order == 2 && pl.grid <= slots) pl.prefill_priority = 0;
  if (pl.has_p && pl.has_d && lim.persistent) {
    pl.persistent = true;  // every resident slot loops over the queues
    pl.grid = (int)std::min<int64_t>(pl.grid, slots);
  }
  if (pl.has_p && pl.has_d) {
    if (lim.policy == kPolicyHalf) {
      pl.share_num = 1;
      pl.share_den = 2;
    } else {
      reduce_share(pl.p_tasks, pl.d_wg_tasks, pl.share_num, pl.share_den);
    }
  } else {
    pl.share_num = pl.has_p ? 1 : 0;
    pl.share_den = 1;
  }
  *out = pl;
  return POD_OK;
}

int make_plan(const Shape& s, const Limits& lim, int mode, const PrefillIn& p, const DecodeIn& d, Plan* out) {
  if (lim.wg_per_cu == 2 || lim.wg_per_cu == 4) return plan_wg(s, lim, lim.wg_per_cu, mode, p, d, out);
  // Runtime choice between the envelopes (paper §4.2.2 and §5.4.1 pick two
  // or four CTAs per SM per batch).  Measured on MI355X with these tiles:
  // the 16-row prefill tile of the four-workgroup envelope runs 1.3-1.6x
  // slower than the 32-row tile (the same LDS and DMA bytes per block for
  // half the FLOPs), so every hybrid batch tried -- prefill- and
  // decode-dominated, short and long contexts -- was faster with two
  // workgroups per CU; decode alone was 2-5% faster with four when all its
  // workgroups start in one round of four per CU, and slower when it takes
  // several.  So: four for a call without prefill whose decode workgroups
  // fit one round of four per CU, two otherwise (and always for fp32 and
  // the persistent grid, which have only that envelope).
  Plan p2;
  int rc = plan_wg(s, lim, 2, mode, p, d, &p2);
  if (rc) return rc;
  if (envelope_allowed(s.dtype, 0, 4) && !lim.persistent && p2.has_d && !p2.has_p) {
    Plan p4;
    if (plan_wg(s, lim, 4, mode, p, d, &p4) == POD_OK && (int64_t)p4.d_wg_tasks <= (int64_t)lim.num_cus * 4) {
      *out = p4;
      return POD_OK;
    }
  }
  *out = p2;
  return POD_OK;
}

}  // namespace pod
