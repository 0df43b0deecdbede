// C ABI of the hybrid-batch attention library: handle, validation, planning,
// workspace and launch.  Declarations and contracts are in include/pod_attn.h.
#include "../../include/pod_attn.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>

#include "pod_launch.h"
#include "pod_plan.h"

static_assert(POD_MAX_CHUNKS == pod::kMaxChunks, "chunk limit of the ABI and the planner");

struct pod_attn_handle {
  pod::Shape shape;
  pod::Limits lim;
  float sm_scale = 0.0f;
  int device = 0;
  char* ws = nullptr;
  pod::WorkspaceLayout lay;
  pod_attn_stats stats{};
  int64_t traced_tasks = 0;  // records of the last fused launch that recorded its roles
  char err[256] = {0};
};

namespace {

int validate_config(const pod_attn_config* c, pod::Shape& s, pod::Limits& lim, float& scale) {
  if (!c) return POD_ERR_INVALID_ARG;
  s.dtype = c->dtype;
  s.hq = c->num_q_heads;
  s.hkv = c->num_kv_heads;
  s.d = c->head_dim;
  s.page = c->page_size;
  if (s.hq <= 0 || s.hkv <= 0 || s.d <= 0 || s.page <= 0) return POD_ERR_INVALID_ARG;
  s.G = s.hq % s.hkv == 0 ? s.hq / s.hkv : 0;
  int rc = pod::check_shape(s);
  if (rc) return rc;
  if (c->max_chunk_len < 1 || c->max_num_decode < 1 || c->max_context < 1 || c->max_total_context < 0)
    return POD_ERR_INVALID_ARG;
  // a request has at most kMaxSplitsPerRequest decode splits of at least kMinSplitTokens
  if ((int64_t)c->max_context > (int64_t)pod::kMaxContext) return POD_ERR_UNSUPPORTED;
  if (!(c->sm_scale >= 0.0f) || !std::isfinite(c->sm_scale)) return POD_ERR_INVALID_ARG;
  if (c->wg_per_cu != 0 && c->wg_per_cu != 2 && c->wg_per_cu != 4) return POD_ERR_INVALID_ARG;
  if (c->persistent != 0 && c->persistent != 1) return POD_ERR_INVALID_ARG;
  // the four-workgroup envelope is built for bf16 and launched one workgroup per task
  if (c->wg_per_cu == 4 && (s.dtype != pod::kBf16 || c->persistent)) return POD_ERR_UNSUPPORTED;
  if (c->prefill_split_cap_waves < -1) return POD_ERR_INVALID_ARG;
  if (c->prefill_splits < 0) return POD_ERR_INVALID_ARG;
  if (c->policy < pod::kPolicyCuBalanced || c->policy > pod::kPolicyStatic) return POD_ERR_INVALID_ARG;
  if (c->prefill_slots_x256 < 0 || c->prefill_slots_x256 > 4 * 256) return POD_ERR_INVALID_ARG;
  if (c->record_roles != 0 && c->record_roles != 1) return POD_ERR_INVALID_ARG;
  if (c->decode_split_tokens != 0 &&
      (c->decode_split_tokens % pod::kPageSize != 0 ||
       c->decode_split_tokens < pod::min_split_tokens(s.dtype, c->max_context) ||
       c->decode_split_tokens > pod::kMaxSplitTokens))
    return POD_ERR_INVALID_ARG;
  if (c->decode_tail_split_tokens < 0 ||
      (c->decode_tail_split_tokens > 0 &&
       (c->decode_tail_split_tokens % pod::kPageSize != 0 ||
        c->decode_tail_split_tokens < pod::min_split_tokens(s.dtype, c->max_context) ||
        c->decode_tail_split_tokens > pod::kMaxSplitTokens)))
    return POD_ERR_INVALID_ARG;
  lim.max_chunk_len = c->max_chunk_len;
  lim.max_num_decode = c->max_num_decode;
  lim.max_context = c->max_context;
  lim.max_total_context = c->max_total_context;
  lim.wg_per_cu = c->persistent ? 2 : c->wg_per_cu;
  lim.cap_waves = c->prefill_split_cap_waves ? c->prefill_split_cap_waves : 2;
  lim.prefill_splits = c->prefill_splits;
  lim.record_roles = c->record_roles != 0;
  lim.policy = c->policy;
  lim.slots_x256 = c->prefill_slots_x256;
  lim.split_tokens = c->decode_split_tokens;
  lim.tail_split_tokens = c->decode_tail_split_tokens;
  lim.persistent = c->persistent != 0;
  scale = c->sm_scale > 0.0f ? c->sm_scale : 1.0f / std::sqrt((float)s.d);
  return POD_OK;
}

void fill_stats(const pod::Plan& pl, pod_attn_stats* st) {
  std::memset(st, 0, sizeof *st);
  st->mode = pl.mode;
  st->fallback = pl.fallback;
  st->num_cus = pl.num_cus;
  st->wg_per_cu = pl.wg_per_cu;
  st->grid = pl.grid;
  st->prefill_rows_per_tile = pl.rows_per_tile;
  st->prefill_heads_per_tile = pl.heads_per_tile;
  st->prefill_tiles = pl.tiles;
  st->prefill_chunks = pl.has_p ? pl.n_chunks : 0;
  st->persistent = pl.persistent ? 1 : 0;
  st->fixed_order = pl.fixed_order;
  st->prefill_priority = pl.prefill_priority;
  st->prefill_splits = pl.has_p ? pl.ch[0].splits : 0;
  st->prefill_split_keys = pl.has_p ? pl.ch[0].split_keys : 0;
  st->prefill_tasks = pl.has_p ? pl.p_tasks : 0;
  st->decode_split_tokens = pl.T;
  st->decode_tail_split_tokens = pl.has_d && pl.tail_k ? pl.T2 : 0;
  st->decode_wave_tasks = pl.has_d ? pl.d_wave_tasks : 0;
  st->decode_wg_tasks = pl.has_d ? pl.d_wg_tasks : 0;
  st->decode_unit_classes = pl.has_d ? pl.rem_buckets : 0;
  st->share_num = pl.share_num;
  st->share_den = pl.share_den;
  st->cu_prefill_x256 = pl.cu_prefill_x256;
  st->policy = pl.policy;
}

int hip_fail(pod_attn_handle* h, hipError_t e, const char* what) {
  if (h) std::snprintf(h->err, sizeof h->err, "%s: %s", what, hipGetErrorString(e));
  return POD_ERR_HIP;
}

// The prefill half of a call: device buffers plus the chunk shapes.
struct PrefillView {
  const void* q = nullptr;
  void* o = nullptr;
  const int32_t* pt = nullptr;
  pod::PrefillIn in;
};

int prefill_one(const pod_prefill_args* a, PrefillView& v) {
  if (!a) return POD_OK;
  if (!a->q || !a->o || !a->page_table) return POD_ERR_INVALID_ARG;
  v.q = a->q;
  v.o = a->o;
  v.pt = a->page_table;
  v.in.present = true;
  v.in.n = 1;
  v.in.C[0] = a->chunk_len;
  v.in.P0[0] = a->chunk_offset;
  return POD_OK;
}

int prefill_many(const pod_prefill_batch* b, PrefillView& v) {
  if (!b) return POD_OK;
  if (!b->q || !b->o || !b->page_table || !b->chunk_lens_host || !b->chunk_offsets_host)
    return POD_ERR_INVALID_ARG;
  if (b->num_chunks < 1 || b->num_chunks > POD_MAX_CHUNKS || b->page_table_stride < 1) return POD_ERR_INVALID_ARG;
  v.q = b->q;
  v.o = b->o;
  v.pt = b->page_table;
  v.in.present = true;
  v.in.n = b->num_chunks;
  v.in.stride = b->page_table_stride;
  for (int c = 0; c < b->num_chunks; ++c) {
    v.in.C[c] = b->chunk_lens_host[c];
    v.in.P0[c] = b->chunk_offsets_host[c];
  }
  return POD_OK;
}

pod::DecodeIn decode_in(const pod_decode_args* a) {
  pod::DecodeIn d;
  if (a) {
    d.present = true;
    d.N = a->num_decode;
    d.stride = a->page_table_stride;
    d.ctx_host = a->context_lens_host;
  }
  return d;
}

int check_decode(const pod_decode_args* d) {
  if (d && (!d->q || !d->o || !d->page_table || !d->context_lens || !d->context_lens_host))
    return POD_ERR_INVALID_ARG;
  return POD_OK;
}

// The kernels' parameter block for plan `pl` over workspace `ws` laid out as `lay`.
void fill_params(const pod::Shape& s, float sm_scale, char* ws, const pod::WorkspaceLayout& lay, const pod::Plan& pl,
                 const void* k_pool, const void* v_pool, int64_t num_pages, const PrefillView& pv,
                 const pod_decode_args* da, pod::PodParams& p) {
  p = pod::PodParams{};
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.num_pages = (uint32_t)num_pages;
  p.hq = s.hq;
  p.hkv = s.hkv;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.ctrl = reinterpret_cast<uint32_t*>(ws + lay.ctrl);
  p.tickets = reinterpret_cast<uint32_t*>(ws + lay.tickets);
  p.p_cnt = reinterpret_cast<uint32_t*>(ws + lay.p_cnt);
  p.d_cnt = reinterpret_cast<uint32_t*>(ws + lay.d_cnt);
  p.p_part = reinterpret_cast<float*>(ws + lay.p_part);
  p.d_part = reinterpret_cast<float*>(ws + lay.d_part);
  p.trace = lay.trace_bytes ? ws + lay.trace : nullptr;
  if (pl.has_p) {
    p.qp = pv.q;
    p.op = pv.o;
    p.pt_p = pv.pt;
    p.rows_per_tile = pl.rows_per_tile;
    p.heads_per_tile = pl.heads_per_tile;
    p.head_groups = pl.head_groups;
    p.p_tasks = pl.p_tasks;
    p.n_chunks = pl.n_chunks;
    for (int k = 0; k < pl.n_chunks; ++k) {
      const pod::ChunkPlan& c = pl.ch[k];
      p.ch[k] = pod::PfChunk{c.task_base, c.tile_base, c.row_base, c.src * pl.stride,
                             c.C, c.P0, c.splits, c.split_keys, c.row_blocks};
    }
  }
  if (pl.has_d) {
    p.qd = da->q;
    p.od = da->o;
    p.pt_d = da->page_table;
    p.ctx = da->context_lens;
    p.stride = da->page_table_stride;
    p.N = pl.N;
    p.T = pl.T;
    p.T2 = pl.T2;
    p.tail_k = pl.tail_k;
    p.d_wave_tasks = pl.d_wave_tasks;
    p.d_units = pl.d_wave_tasks / s.hkv;
    for (int ph = 0; ph <= pod::kUnitPhases; ++ph) p.phase_start[ph] = pl.phase_start[ph];
    p.ctx_cap = pl.d_max;
    p.d_wg_tasks = pl.d_wg_tasks;
  }
  p.share_num = pl.share_num;
  p.share_den = pl.share_den;
  p.cu_prefill_x256 = pl.cu_prefill_x256;
  p.policy = pl.policy;
  p.fixed_order = pl.fixed_order;
  p.prefill_priority = pl.prefill_priority;
  p.grid = pl.grid;
}

int kernel_of(const pod::Plan& pl) {
  if (!pl.has_d) return pod::kKernelPrefill;
  if (!pl.has_p) return pod::kKernelDecode;
  return pod::kKernelHybrid;
}

int run(pod_attn_handle* h, int mode, const void* k_pool, const void* v_pool, int64_t num_pages,
        const PrefillView& pv, const pod_decode_args* da, pod_stream_t stream) {
  if (!h || !k_pool || !v_pool || num_pages < 1 || num_pages > 0xffffffffLL) return POD_ERR_INVALID_ARG;
  int rc = check_decode(da);
  if (rc) return rc;
  pod::Plan pl;
  rc = pod::make_plan(h->shape, h->lim, mode, pv.in, decode_in(da), &pl);
  if (rc) return rc;

  const pod::Shape& s = h->shape;
  pod::PodParams p;
  fill_params(s, h->sm_scale, h->ws, h->lay, pl, k_pool, v_pool, num_pages, pv, da, p);
  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) return hip_fail(h, e, "hipSetDevice");
  if (pl.grid > 0) {
    e = (hipError_t)pod::launch(kernel_of(pl), s.dtype, s.d, s.G, p, pl, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(h, e, "kernel launch");
  }
  fill_stats(pl, &h->stats);
  if (p.trace && kernel_of(pl) == pod::kKernelHybrid) h->traced_tasks = (int64_t)pl.p_tasks + pl.d_wg_tasks;
  return POD_OK;
}

int plan_only(const pod_attn_config* cfg, int32_t num_cus, int32_t mode, const PrefillView& pv,
              const pod_decode_args* decode, pod_attn_stats* out) {
  if (!out || num_cus < 1 || mode < 0 || mode > 2) return POD_ERR_INVALID_ARG;
  pod::Shape s;
  pod::Limits lim;
  float scale = 0.0f;
  int rc = validate_config(cfg, s, lim, scale);
  if (rc) return rc;
  rc = check_decode(decode);
  if (rc) return rc;
  lim.num_cus = num_cus;
  pod::derive_capacities(s, lim);
  pod::Plan pl;
  rc = pod::make_plan(s, lim, mode, pv.in, decode_in(decode), &pl);
  if (rc) return rc;
  fill_stats(pl, out);
  return POD_OK;
}

}  // namespace

extern "C" {

int pod_attn_create(const pod_attn_config* cfg, pod_attn_handle** out) {
  if (!out) return POD_ERR_INVALID_ARG;
  *out = nullptr;
  pod::Shape s;
  pod::Limits lim;
  float scale = 0.0f;
  int rc = validate_config(cfg, s, lim, scale);
  if (rc) return rc;
  if (!pod::have_kernel(s.dtype, s.d, s.G)) return POD_ERR_UNSUPPORTED;

  int dev = cfg->device;
  hipError_t e;
  if (dev < 0) {
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return POD_ERR_HIP;
  }
  e = hipSetDevice(dev);
  if (e != hipSuccess) return POD_ERR_HIP;
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus <= 0) return POD_ERR_HIP;
  lim.num_cus = cus;
  pod::derive_capacities(s, lim);

  pod_attn_handle* h = new (std::nothrow) pod_attn_handle();
  if (!h) return POD_ERR_WORKSPACE;
  h->shape = s;
  h->lim = lim;
  h->sm_scale = scale;
  h->device = dev;
  h->lay = pod::workspace_layout(s, lim);
  e = hipMalloc(reinterpret_cast<void**>(&h->ws), h->lay.total);
  if (e != hipSuccess) {
    delete h;
    return POD_ERR_WORKSPACE;
  }
  // counters and queue heads start at zero; kernels restore them after each call
  e = hipMemset(h->ws, 0, h->lay.p_part);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(h->ws);
    delete h;
    return POD_ERR_HIP;
  }
  *out = h;
  return POD_OK;
}

int pod_attn_destroy(pod_attn_handle* h) {
  if (!h) return POD_OK;
  int rc = POD_OK;
  if (hipSetDevice(h->device) != hipSuccess || hipDeviceSynchronize() != hipSuccess) rc = POD_ERR_HIP;
  if (h->ws && hipFree(h->ws) != hipSuccess) rc = POD_ERR_HIP;
  delete h;
  return rc;
}

int pod_attn_hybrid(pod_attn_handle* h, const void* k_pool, const void* v_pool, int64_t num_pages,
                    const pod_prefill_args* prefill, const pod_decode_args* decode, pod_stream_t stream) {
  PrefillView pv;
  const int rc = prefill_one(prefill, pv);
  return rc ? rc : run(h, pod::kModeHybrid, k_pool, v_pool, num_pages, pv, decode, stream);
}

int pod_attn_hybrid_noalloc(const pod_attn_config* cfg, const void* k_pool, const void* v_pool, int64_t num_pages,
                            const pod_prefill_args* prefill, const pod_decode_args* decode, pod_stream_t stream) {
  pod::Shape s;
  pod::Limits lim;
  float scale = 0.0f;
  int rc = validate_config(cfg, s, lim, scale);
  if (rc) return rc;
  if (!k_pool || !v_pool || num_pages < 1 || num_pages > 0xffffffffLL) return POD_ERR_INVALID_ARG;
  if (!pod::have_kernel(s.dtype, s.d, s.G)) return POD_ERR_UNSUPPORTED;
  rc = check_decode(decode);
  if (rc) return rc;
  if (lim.record_roles) return POD_ERR_UNSUPPORTED;  // no trace region in the fixed scratch
  PrefillView pv;
  rc = prefill_one(prefill, pv);
  if (rc) return rc;

  int dev = cfg->device;
  hipError_t e = hipSuccess;
  if (dev < 0) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipSetDevice(dev);
  int cus = 0;
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus <= 0) return POD_ERR_HIP;
  lim.num_cus = cus;
  pod::derive_capacities(s, lim);
  pod::Plan pl;
  rc = pod::make_plan(s, lim, pod::kModeHybrid, pv.in, decode_in(decode), &pl);
  if (rc) return rc;
  // the workspace this call needs, laid out in the device's fixed scratch
  const pod::WorkspaceLayout lay = pod::workspace_layout_for_plan(s, pl);
  if (lay.total > pod::scratch_bytes()) return POD_ERR_WORKSPACE;
  void* base = nullptr;
  if (pod::scratch_address(dev, &base) != 0 || !base) return POD_ERR_HIP;

  pod::PodParams p;
  fill_params(s, scale, static_cast<char*>(base), lay, pl, k_pool, v_pool, num_pages, pv, decode, p);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // counters and control words start at zero whatever the last call left
  if (pod::launch_zero(base, lay.p_part, st) != 0) return POD_ERR_HIP;
  if (pl.grid > 0 && pod::launch(kernel_of(pl), s.dtype, s.d, s.G, p, pl, st) != 0) return POD_ERR_HIP;
  return POD_OK;
}

int pod_attn_prefill_only(pod_attn_handle* h, const void* k_pool, const void* v_pool, int64_t num_pages,
                          const pod_prefill_args* prefill, pod_stream_t stream) {
  if (!prefill) return POD_ERR_INVALID_ARG;
  PrefillView pv;
  const int rc = prefill_one(prefill, pv);
  return rc ? rc : run(h, pod::kModePrefill, k_pool, v_pool, num_pages, pv, nullptr, stream);
}

int pod_attn_decode_only(pod_attn_handle* h, const void* k_pool, const void* v_pool, int64_t num_pages,
                         const pod_decode_args* decode, pod_stream_t stream) {
  if (!decode) return POD_ERR_INVALID_ARG;
  return run(h, pod::kModeDecode, k_pool, v_pool, num_pages, PrefillView{}, decode, stream);
}

int pod_attn_hybrid_varlen(pod_attn_handle* h, const void* k_pool, const void* v_pool, int64_t num_pages,
                           const pod_prefill_batch* prefill, const pod_decode_args* decode, pod_stream_t stream) {
  PrefillView pv;
  const int rc = prefill_many(prefill, pv);
  return rc ? rc : run(h, pod::kModeHybrid, k_pool, v_pool, num_pages, pv, decode, stream);
}

int pod_attn_prefill_only_varlen(pod_attn_handle* h, const void* k_pool, const void* v_pool, int64_t num_pages,
                                 const pod_prefill_batch* prefill, pod_stream_t stream) {
  if (!prefill) return POD_ERR_INVALID_ARG;
  PrefillView pv;
  const int rc = prefill_many(prefill, pv);
  return rc ? rc : run(h, pod::kModePrefill, k_pool, v_pool, num_pages, pv, nullptr, stream);
}

int pod_attn_peak_read(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* sink, pod_stream_t stream) {
  if (!buf || !sink || workgroups < 1 || bytes < 1) return POD_ERR_INVALID_ARG;
  const int64_t waves = (int64_t)workgroups * pod::kWavesPerWG;
  // each wave's slice: a whole number of 16 KB register buffers, at most 1 GiB
  if (bytes % (waves * 16384) != 0 || bytes / waves > (int64_t(1) << 30)) return POD_ERR_INVALID_ARG;
  const int e = pod::launch_peak_read(buf, (size_t)bytes, workgroups, sink, reinterpret_cast<hipStream_t>(stream));
  return e == 0 ? POD_OK : POD_ERR_HIP;
}

int pod_attn_peak_mfma(int32_t workgroups, int32_t iters, uint32_t* sink, pod_stream_t stream) {
  if (!sink || workgroups < 1 || iters < 1) return POD_ERR_INVALID_ARG;
  const int e = pod::launch_peak_mfma(workgroups, iters, sink, reinterpret_cast<hipStream_t>(stream));
  return e == 0 ? POD_OK : POD_ERR_HIP;
}

int pod_attn_role_trace(pod_attn_handle* h, pod_attn_task_record* out, int32_t capacity, int32_t* count) {
  if (!h || !count || capacity < 0 || (capacity > 0 && !out)) return POD_ERR_INVALID_ARG;
  if (!h->lay.trace_bytes) return POD_ERR_INVALID_ARG;  // the handle does not record roles
  static_assert(sizeof(pod_attn_task_record) == pod::kTraceRecordBytes, "trace record layout");
  *count = (int32_t)h->traced_tasks;
  const int64_t n = std::min<int64_t>(capacity, h->traced_tasks);
  if (n <= 0) return POD_OK;
  hipError_t e = hipSetDevice(h->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(out, h->ws + h->lay.trace, (size_t)n * sizeof(pod_attn_task_record), hipMemcpyDeviceToHost);
  return e == hipSuccess ? POD_OK : hip_fail(h, e, "role trace copy");
}

int pod_attn_get_stats(const pod_attn_handle* h, pod_attn_stats* out) {
  if (!h || !out) return POD_ERR_INVALID_ARG;
  *out = h->stats;
  return POD_OK;
}

int pod_attn_plan(const pod_attn_config* cfg, int32_t num_cus, int32_t mode, const pod_prefill_args* prefill,
                  const pod_decode_args* decode, pod_attn_stats* out) {
  PrefillView pv;
  const int rc = prefill_one(prefill, pv);
  return rc ? rc : plan_only(cfg, num_cus, mode, pv, decode, out);
}

int pod_attn_plan_varlen(const pod_attn_config* cfg, int32_t num_cus, int32_t mode,
                         const pod_prefill_batch* prefill, const pod_decode_args* decode, pod_attn_stats* out) {
  PrefillView pv;
  const int rc = prefill_many(prefill, pv);
  return rc ? rc : plan_only(cfg, num_cus, mode, pv, decode, out);
}

const char* pod_attn_status_string(int status) {
  switch (status) {
    case POD_OK: return "ok";
    case POD_ERR_INVALID_ARG: return "invalid argument";
    case POD_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case POD_ERR_WORKSPACE: return "workspace too small for this batch";
    case POD_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* pod_attn_last_error(const pod_attn_handle* h) { return h ? h->err : ""; }

}  // extern "C"
