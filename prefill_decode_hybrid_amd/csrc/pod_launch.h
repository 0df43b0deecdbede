// Kernel parameter block and launch entry points shared by the host runtime
// (pod_attn.cpp) and the kernels (pod_kernels.hip).  Plain types only.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "pod_plan.h"

namespace pod {

// One prefill chunk as the kernels see it.  Its tasks are
// task_base .. task_base + tiles * splits - 1 (tiles = row_blocks * hkv *
// head_groups), its tiles tile_base .., its query/output rows row_base ..
// row_base + C - 1 of the packed q and o, and its page ids start at entry
// pt_base of the prefill page table.
struct PfChunk {
  int task_base, tile_base, row_base, pt_base;
  int C, P0, splits, split_keys, row_blocks;
};

struct PodParams {
  // paged KV pool [num_pages, 16, hkv, d]
  const void* k_pool;
  const void* v_pool;
  uint32_t num_pages;
  int hq, hkv;
  float scale_log2;  // softmax scale * log2(e): scores live in the base-2 domain

  // prefill chunks, in task order
  const void* qp;
  void* op;
  const int32_t* pt_p;
  int rows_per_tile, heads_per_tile, head_groups, p_tasks, n_chunks;
  PfChunk ch[kMaxChunks];  // read with a uniform index from the kernel-argument segment
  float* p_part;     // [task]: acc [row-head][d], m [row-head], l [row-head]
  uint32_t* p_cnt;   // [tile] arrival counters, 0 between calls

  // decode batch
  const void* qd;
  void* od;
  const int32_t* pt_d;
  const int32_t* ctx;
  int stride, N, d_units, d_wave_tasks, d_wg_tasks;
  int T, T2, tail_k; // long and short split lengths, long splits moved to the short phase (pod_units.h)
  int ctx_cap;       // device context lengths are clamped to this (the batch's largest host length)
  int phase_start[kUnitPhases + 1];  // first decode unit of every phase (pod_units.h)
  float* d_part;     // records [kv head][unit]: [G][d] acc, [G] m, [G] l, 16-byte padded
  uint32_t* d_cnt;   // [request][kv head] arrival counters, 0 between calls

  // fused launch
  uint32_t* ctrl;     // control words (pod_plan.h kCtrl*), zero at launch, left zero
  uint32_t* tickets;  // per-CU words: ticket counters, or running prefill | decode << 16
  int share_num, share_den, cu_prefill_x256, policy, grid;
  int fixed_order;   // fused launch: 1 / 2 = the first workgroup ids run the prefill / decode tasks
  int prefill_priority;  // 1: prefill waves issue above decode waves (s_setprio)
  // role trace (fused launches): task t's record at trace + 32 * (prefill t,
  // or p_tasks + decode workgroup task t); nullptr when not recording
  char* trace;
};

// The parameter block is the kernels' only argument (kernel arguments are
// limited to 4 KiB).
static_assert(sizeof(PodParams) <= 4096, "kernel argument block");

enum { kKernelHybrid = 0, kKernelPrefill = 1, kKernelDecode = 2 };

// Launch one kernel for `which` with geometry from `pl`.  Returns a hipError_t.
int launch(int which, int dtype, int d, int G, const PodParams& p, const Plan& pl, hipStream_t s);

// 1 if a kernel is built for (dtype, d, G).
int have_kernel(int dtype, int d, int G);

// Fixed device scratch of the allocation-free entry point: its size, and its
// address on `device` (looked up once per device, with that device
// current).  0 or a hipError_t.
size_t scratch_bytes();
int scratch_address(int device, void** out);
// Zero `bytes` (a multiple of 4) at `p` with a fill kernel (no memset node
// in a captured graph).  Returns a hipError_t.
int launch_zero(void* p, size_t bytes, hipStream_t s);
// Measured-peak kernels: `bytes` of `buf` read by `workgroups` workgroups
// (each wave a contiguous bytes / (4 workgroups) slice, a multiple of 16
// KB), and `workgroups` x 4 waves x `iters` x 16 MFMAs of 32x32x16 bf16.
int launch_peak_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, hipStream_t s);
int launch_peak_mfma(int workgroups, int iters, uint32_t* sink, hipStream_t s);

}  // namespace pod
