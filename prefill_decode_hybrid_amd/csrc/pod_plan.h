// Host-side planner for hybrid-batch attention.  Plain C++17: no HIP calls,
// so it is unit-testable on a machine without a GPU.
//
// A plan turns one call's shapes into the task lists the kernels walk:
//  * prefill tiles (chunk, row block, kv head, head group), each split into
//    KV ranges when there are too few tiles to fill the machine.  The number of
//    prefill tasks is capped at `cap_waves` waves of resident workgroups so a
//    chunk cannot flood the launch (paper §4.2.3 caps chunked-prefill splits
//    at two full waves);
//  * decode wave tasks (request, kv head, token split), one 64-lane wave each
//    (paper §4.2.3, virtual decode CTAs of one warp), four per workgroup;
//  * the fused launch's role mix: prefill workgroups kept per CU for the
//    default CU-balanced policy (from the time each role needs alone), or
//    the ticket share of the proportional and 50:50 policies (paper §5.4.2);
//  * the chunk table when one call carries several prefill chunks.
#pragma once

#include <cstdint>

#include "pod_units.h"

namespace pod {

enum { kBf16 = 0, kF32 = 1 };
enum { kModeHybrid = 0, kModePrefill = 1, kModeDecode = 2 };
enum { kPolicyCuBalanced = 0, kPolicyProportional = 1, kPolicyHalf = 2, kPolicyStatic = 3 };

constexpr int kPageSize = 16;
constexpr int kWavesPerWG = 4;
constexpr int kSplitIdRegs = 4;         // page-id registers of a decode wave (64 ids each)
constexpr int kMaxSplitTokens = 64 * kPageSize * kSplitIdRegs;  // 4096 tokens per decode wave task
constexpr int kMinSplitTokens = 256;
constexpr int kMinSplitTokensF32 = 64;  // the fp32 decode wave is latency-bound: shorter splits
constexpr int kMaxSplitsPerRequest = kUnitMaxSplits;  // 64 requests' split counts share 16 bits of the unit scan
constexpr int kMaxContext = kMaxSplitsPerRequest * kMinSplitTokens;  // 261888 tokens

// Shortest decode split for `dtype` that keeps every context up to
// `max_context` within kMaxSplitsPerRequest splits.
inline int min_split_tokens(int dtype, int max_context) {
  const int base = dtype == kBf16 ? kMinSplitTokens : kMinSplitTokensF32;
  const int need = ((max_context + kMaxSplitsPerRequest - 1) / kMaxSplitsPerRequest + kPageSize - 1) / kPageSize * kPageSize;
  return base > need ? base : need;
}
// Fewest keys a split added for parallelism keeps: a bf16 tile streams a
// 64-key block in ~2.5 us, so shorter splits cost more in merges than they
// gain; the fp32 tile (one row per lane on the vector unit) is ~30x slower
// per key, so one 32-key block is worth a split.
constexpr int kMinPrefillSplitKeys = 1024;
constexpr int kMinPrefillSplitKeysF32 = 32;
constexpr int kMaxSplitKeys = 16384;       // page ids of one split are staged in LDS
constexpr int kShareDen = 64;
constexpr int kMaxChunks = 64;             // prefill chunks of one call (the table travels in the kernel arguments)
// Throughput of the split kernels on MI355X, used only to pick the fused
// launch's per-CU prefill slots: prefill FLOP/s (bf16 and fp32 tiles) and
// decode bytes/s over the whole chip, and the decode time below which a
// batch is too small to gain from running the roles side by side.  The
// choice changes where tasks run, never the result.
constexpr double kPrefillFlopsBf16 = 7.5e14;
constexpr double kPrefillFlopsF32 = 1.0e13;
constexpr double kDecodeBytesPerS = 5.8e12;
constexpr double kOverlapMinSeconds = 200e-6;
constexpr double kPrefillSecondsPerKey = 39e-9;  // one bf16 tile task, two workgroups per CU

struct Shape {
  int dtype = kBf16, hq = 0, hkv = 0, G = 0, d = 0, page = kPageSize;
};

struct Limits {
  int max_chunk_len = 0, max_num_decode = 0, max_context = 0;
  int64_t max_total_context = 0;
  int wg_per_cu = 2;  // co-resident workgroups per CU: 2, 4, or 0 (chosen per batch)
  int cap_waves = 2;  // prefill tasks added for parallelism fill at most this many waves; -1: no cap
  int prefill_splits = 0;  // KV splits per prefill tile; 0: from the batch
  int policy = kPolicyCuBalanced;
  int slots_x256 = 0;  // prefill slots per CU for the CU-balanced policy; 0: from the batch
  int split_tokens = 0;  // decode tokens per wave task; 0: from the batch
  int tail_split_tokens = 0;  // decode tail split length; 0: no tail splits
  bool persistent = false;  // fused launch as a resident grid looping over the queues
  bool record_roles = false;  // fused launches write one record per task (role trace)
  int num_cus = 0;
  // capacities derived by derive_capacities()
  int64_t cap_prefill_tasks = 0, cap_wave_tasks = 0, cap_tiles = 0;
  int64_t cap_rowhead_tasks = 0;  // prefill tasks x row-heads per task (split partials)
};

// Prefill chunks of one call in the caller's order.  stride: page-table
// row stride of chunk c (row c of the table); 0 for the single-chunk call,
// whose table is one row.
struct PrefillIn {
  bool present = false;
  int n = 0, stride = 0;
  int C[kMaxChunks] = {}, P0[kMaxChunks] = {};
};

// One chunk of a plan.  Chunks are laid out in task order (longest key
// range first); src is the caller's index of the chunk.
struct ChunkPlan {
  int src = 0, C = 0, P0 = 0, Lp = 0;
  int row_blocks = 0, tiles = 0, splits = 0, split_keys = 0;
  int task_base = 0, tile_base = 0, row_base = 0;
};

struct DecodeIn {
  bool present = false;
  int N = 0, stride = 0;
  const int32_t* ctx_host = nullptr;
};

struct Plan {
  int mode = 0, fallback = 0, num_cus = 0, wg_per_cu = 0, grid = 0;
  // prefill
  bool has_p = false;
  int n_chunks = 0, stride = 0;
  ChunkPlan ch[kMaxChunks];
  int rows_per_wave = 0, heads_per_tile = 0, row_waves = 0, rows_per_tile = 0, head_groups = 0;
  int tiles = 0, p_tasks = 0;  // over all chunks
  // decode
  bool has_d = false;
  int N = 0, T = 0, d_wave_tasks = 0, d_wg_tasks = 0;
  int d_max = 0;        // longest decode context
  int d_median = 0;     // median decode context
  int64_t d_total = 0;  // sum of decode contexts
  int T2 = 0, tail_k = 0;  // short (tail) split length, long splits moved to the tail (pod_units.h)
  int rem_buckets = 1;  // remainder phases of the unit numbering (kRemBuckets: decode-only and decode-first multi-round fused launches)
  int phase_start[kUnitPhases + 1] = {};  // first decode unit of every phase (pod_units.h)
  // fused scheduling
  int share_num = 0, share_den = 1, cu_prefill_x256 = 0, policy = 0;
  bool persistent = false;  // the fused launch is a resident grid of workgroups
  int fixed_order = 0;  // 0: roles claimed; 1 / 2: prefill / decode tasks by workgroup id first (no claims)
  int prefill_priority = 1;  // issue priority of prefill waves beside decode waves (0 or 1)
  double t_prefill = 0.0, t_decode = 0.0;  // each role's time alone, as estimated for the role mix
};

// Rows of one wave's query block and keys per staged KV block, per dtype
// and resource envelope (2 or 4 workgroups per CU; fp32 has only 2).
inline int rows_per_wave(int dtype, int wg) { return dtype == kBf16 ? (wg == 4 ? 16 : 32) : 64; }
// The envelopes a handle may plan with (wg_per_cu 0 allows both for bf16).
inline bool envelope_allowed(int dtype, int wg_config, int wg) {
  if (wg == 4 && dtype != kBf16) return false;
  return wg_config == 0 ? (wg == 2 || wg == 4) : wg == wg_config;
}

inline int keys_per_block(int dtype) { return dtype == kBf16 ? 64 : 32; }

// 0 if (dtype, G, d, page) is built, else the status code to return.
int check_shape(const Shape& s);

// Fill the capacity fields of `lim` for shape `s`.
void derive_capacities(const Shape& s, Limits& lim);

struct WorkspaceLayout {
  size_t ctrl = 0, tickets = 0, p_cnt = 0, d_cnt = 0, p_part = 0, d_part = 0, trace = 0, total = 0;
  size_t trace_bytes = 0;  // role-trace records (0 when not recording)
};
constexpr int kTraceRecordBytes = 32;  // cu key, role, task, pad, start and end times
WorkspaceLayout workspace_layout(const Shape& s, const Limits& lim);
// The workspace one planned call uses (counters and partials for exactly its tasks).
WorkspaceLayout workspace_layout_for_plan(const Shape& s, const Plan& pl);

// Validate one call and plan it.  Returns 0 or a negative pod_status.
int make_plan(const Shape& s, const Limits& lim, int mode, const PrefillIn& p,
              const DecodeIn& d, Plan* out);

constexpr int kTicketSlots = 2048;  // (xcc, se, sh, cu) keys
constexpr int kCtrlWords = 64;
constexpr int kXcdQueues = 8;         // per-XCD task queues (queue x holds tasks x, x+8, ...)
// Fused-launch control words.  Each workgroup of a launch whose roles are
// claimed counts itself out (kCtrlExit) after its last claim; the last one
// out clears the words, so every launch -- also a replay of a captured
// graph -- starts on clean words, with no host-side state.
constexpr int kCtrlPrefillHeads = 0;  // [0..7] prefill queue heads
constexpr int kCtrlDecodeHeads = 8;   // [8..15] decode workgroup-task queue heads
constexpr int kCtrlPrefillDone = 16;  // set once a claim found every prefill queue empty
constexpr int kCtrlDecodeDone = 17;   // set once a claim found every decode queue empty
constexpr int kCtrlExit = 18;         // workgroups done claiming
constexpr int kCtrlUsed = 19;         // words a launch may dirty
static_assert(kCtrlUsed <= kCtrlWords, "control words");

}  // namespace pod
