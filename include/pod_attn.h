/*
 * pod_attn.h -- C ABI of the hybrid-batch attention library (gfx950).
 *
 * One call computes exact softmax attention for a hybrid batch: one causal
 * chunked-prefill request (or, through the _varlen calls, up to
 * POD_MAX_CHUNKS of them) plus many single-token decode requests over a
 * paged grouped-query KV cache.  The batch shape is the one POD-Attention is
 * built for (paper §2.1: a hybrid batch commonly holds one prefill chunk and
 * several decodes; §3: both sets of inputs reach one attention call), and
 * the fused entry point computes both halves in a single kernel launch in
 * which each workgroup picks its role after dispatch from what its compute
 * unit is already running (paper §4.1, SM-aware CTA scheduling; §4.3, CTA-ID
 * remapping inside one fused kernel).  The split entry points compute one
 * half each; run one after the other on one stream or on two streams, they
 * are the serial and stream-parallel baselines (paper §3.2, FA_Serial and
 * FA_Streams).
 *
 * Math (the result is the plain definition; fusion only changes where and
 * when tiles run, Silicon & Systems digest, "Virtual CTAs and SM-aware
 * balance"):
 *   head h uses kv head g = h / (Hq / Hkv);
 *   key j of a request sits at pool[page_table[j / page_size]][j % page_size][g][:];
 *   O = sum_j softmax_j(sm_scale * q . K_j) V_j over the visible keys:
 *     prefill chunk row i (absolute position chunk_offset + i): j <= chunk_offset + i
 *     decode request r: j < context_lens[r]
 *
 * Layouts (row-major, element type = config dtype for q, k, v and o):
 *   k_pool, v_pool : [num_pages, page_size, Hkv, head_dim]
 *   prefill q, o   : [chunk_len, Hq, head_dim]
 *   decode  q, o   : [num_decode, Hq, head_dim]
 *   page tables    : int32 physical page ids; the prefill table has at least
 *                    ceil((chunk_offset + chunk_len) / page_size) entries, the
 *                    decode table is [num_decode, page_table_stride].
 * The prefill chunk's own keys (positions chunk_offset .. +chunk_len-1) and
 * each decode's current token must already be written into the pool.
 *
 * Ownership: the caller owns every buffer passed in (all device pointers
 * except context_lens_host) and the stream.  The handle owns its device
 * workspace (task queues, merge partials, counters), allocated once by
 * pod_attn_create from the limits in the config and freed by destroy.
 *
 * Asynchrony: every compute call enqueues on `stream` and returns without a
 * host synchronisation.  Argument validation runs first; when it fails,
 * nothing is enqueued.  Device page ids outside [0, num_pages) are clamped
 * to that range (memory-safe, result undefined).  The device context lengths
 * must equal context_lens_host (the host copy sizes the launch).
 *
 * Concurrency: a handle is not thread-safe.  pod_attn_prefill_only and
 * pod_attn_decode_only use disjoint workspace, so one of each may run at the
 * same time on two streams; two concurrent calls of the same entry point,
 * or a hybrid call concurrent with anything else, on one handle race.
 *
 * Graphs: a compute call enqueues exactly one kernel launch and no memset or
 * copy, and every launch leaves the workspace's counters and control words
 * as it found them (zero), with no host-side state between calls; a call
 * may therefore be captured into a HIP graph and replayed, provided the
 * batch shape (which sizes the launch on the host) stays the one captured.
 */
#ifndef POD_ATTN_H
#define POD_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream (hipStream_t); NULL is the device's default stream. */
typedef struct ihipStream_t *pod_stream_t;
typedef struct pod_attn_handle pod_attn_handle;

enum pod_status {
    POD_OK = 0,
    POD_ERR_INVALID_ARG = -1, /* null pointer, length < 1, offset < 0, limit exceeded   */
    POD_ERR_UNSUPPORTED = -2, /* shape/dtype combination not built (see create)        */
    POD_ERR_WORKSPACE = -3,   /* the batch needs more workspace than create reserved   */
    POD_ERR_HIP = -4          /* a HIP runtime call failed; see pod_attn_last_error     */
};

enum pod_dtype { POD_BF16 = 0, POD_F32 = 1 };

/* Role policy of the fused launch.  The default follows the paper's
 * SM-aware scheduling (§4.1): a workgroup looks at how many prefill and
 * decode workgroups already run on its compute unit and takes the role that
 * is short of its share.  The others are the paper's comparison points:
 * proportional and 50:50 ticket sequences (§5.4.2) and a fixed split by
 * workgroup id, i.e. CTA-parallel fusion without SM awareness (§3.3). */
enum pod_policy {
    POD_POLICY_CU_BALANCED = 0,  /* per-CU running counts; prefill slots from the batch
                                    (a prefill-first launch of several rounds takes the
                                    proportional rule instead; the stats report it)     */
    POD_POLICY_PROPORTIONAL = 1, /* per-CU tickets, prefill share = prefill / all tasks */
    POD_POLICY_HALF = 2,         /* per-CU tickets alternating prefill and decode       */
    POD_POLICY_STATIC = 3        /* workgroup id decides the role, no CU awareness      */
};

typedef struct {
    int32_t dtype;            /* POD_BF16 or POD_F32                                   */
    int32_t num_q_heads;      /* Hq                                                    */
    int32_t num_kv_heads;     /* Hkv; Hq / Hkv must be 1, 2, 4 or 8                    */
    int32_t head_dim;         /* 64 or 128 (POD_F32: 64 only)                          */
    int32_t page_size;        /* 16                                                    */
    float sm_scale;           /* softmax scale; 0 selects 1/sqrt(head_dim)             */
    int32_t max_chunk_len;    /* most prefill rows a call may pass (all chunks)        */
    int32_t max_num_decode;   /* largest decode batch                                  */
    int32_t max_context;      /* largest decode context and largest offset+chunk;
                                 at most 261888 (POD_ERR_UNSUPPORTED above)            */
    int64_t max_total_context;/* largest sum of decode contexts; 0: max_num_decode*max_context */
    int32_t wg_per_cu;        /* resource envelope: co-resident workgroups per CU.
                                 2: <= 256 registers per lane and ~68 KB LDS per
                                 workgroup, 32-row prefill tiles, decode by page pairs;
                                 4 (bf16 only, not persistent): <= 128 registers and
                                 <= 40 KB LDS, 16-row prefill tiles, decode page by
                                 page; 0: chosen per call from its batch (paper §4.2.2
                                 picks 2 or 4 per batch; measured here: 4 for a call
                                 without prefill whose decode workgroups all start in
                                 one round of 4 per CU, else 2).  With a fixed envelope
                                 the fused call equals the split calls bit for bit;
                                 with 0 they may pick different envelopes, whose
                                 results differ in rounding only                      */
    int32_t prefill_split_cap_waves; /* KV splits added to fill the machine stop at one
                                 wave of resident workgroups and at most this many waves
                                 (paper §4.2.3 caps splits at two waves); 0 -> 2;
                                 -1: no cap, every tile split as finely as the minimum
                                 split (1024 keys bf16, 32 fp32) allows              */
    int32_t policy;           /* enum pod_policy                                       */
    int32_t device;           /* HIP device ordinal; -1 selects the current device     */
    int32_t prefill_slots_x256; /* CU-balanced policy: prefill workgroups kept running per
                                 CU, in 1/256 of a workgroup (1 .. 1024, at most 256 *
                                 the envelope's workgroups per CU); 0 selects the
                                 planner's choice from the batch                      */
    int32_t decode_split_tokens; /* tokens per decode wave task, a multiple of 16 up to
                                 4096 and at least 256 (bf16) or 64 (fp32) and
                                 max_context / 1023; 0 selects the planner's choice, which
                                 depends on the decode batch alone (so a decode's result
                                 has the same bits in fused and decode-only launches)  */
    int32_t persistent;         /* 1: the fused launch is a resident grid (CUs x
                                 wg_per_cu workgroups) that loops over the task queues
                                 until both are empty, instead of one workgroup per
                                 task; same tasks and results.  0: one per task       */
    int32_t prefill_splits;     /* KV splits per prefill tile (at most one per minimum
                                 split); 0 selects the planner's choice above        */
    int32_t record_roles;       /* 1: fused launches write one pod_attn_task_record per
                                 task (read with pod_attn_role_trace); 0: none        */
    int32_t decode_tail_split_tokens; /* > 0: the tail of every decode request (its
                                 last full split and the remainder) is cut into splits
                                 of this many tokens, numbered after every other split
                                 so a launch's last decode tasks are short: a multiple
                                 of 16, at least the decode split minimum above; not
                                 below the decode split means no tail splits.  0: no
                                 tail splits (the planner's choice: measured faster
                                 on every batch but the prefill-heavy one)            */
} pod_attn_config;

/* One task of a fused launch as it ran: the virtual-workgroup mix the
 * Silicon & Systems digest asks the runtime to report ("Isolation and
 * predictability").  cu_key = XCC << 8 | shader engine << 5 | shader array
 * << 4 | CU of the compute unit the workgroup ran on; role 0 prefill, 1
 * decode; task its index in that role's list; start and end read from the
 * chip-wide 100 MHz real-time counter when the workgroup began the task and
 * when all its waves were done with it. */
typedef struct {
    uint32_t cu_key;
    int32_t role;
    int32_t task;
    int32_t reserved;
    uint64_t start;
    uint64_t end;
} pod_attn_task_record;

typedef struct {
    const void *q;              /* device [chunk_len, Hq, head_dim]                    */
    void *o;                    /* device [chunk_len, Hq, head_dim]                    */
    const int32_t *page_table;  /* device, >= ceil((chunk_offset+chunk_len)/page_size) */
    int32_t chunk_len;          /* >= 1                                                */
    int32_t chunk_offset;       /* >= 0: tokens of this request already in the cache  */
} pod_prefill_args;

typedef struct {
    const void *q;              /* device [num_decode, Hq, head_dim]                   */
    void *o;                    /* device [num_decode, Hq, head_dim]                   */
    const int32_t *page_table;  /* device [num_decode, page_table_stride]              */
    int32_t page_table_stride;  /* >= ceil(max context / page_size)                    */
    const int32_t *context_lens;      /* device [num_decode], each >= 1                */
    const int32_t *context_lens_host; /* host copy of the same values (plans the launch) */
    int32_t num_decode;         /* >= 1                                                */
} pod_decode_args;

/* Several prefill chunks in one call.  The paper's hybrid batch commonly
 * holds one chunk (§2.1); a scheduler that packs chunks of several prompts
 * passes them here.  Chunk c is its own request: rows row_c .. row_c +
 * chunk_lens[c] - 1 of q and o, where row_c is the sum of the earlier chunk
 * lengths, row i of it at absolute position chunk_offsets[c] + i seeing keys
 * 0 .. chunk_offsets[c] + i of its own page table (row c of page_table).
 * The sum of the chunk lengths must not exceed max_chunk_len of the config.
 * With one chunk the result equals pod_attn_hybrid's bit for bit. */
#define POD_MAX_CHUNKS 64
typedef struct {
    const void *q;              /* device [sum of chunk_lens, Hq, head_dim]            */
    void *o;                    /* device [sum of chunk_lens, Hq, head_dim]            */
    const int32_t *page_table;  /* device [num_chunks, page_table_stride]              */
    int32_t page_table_stride;  /* >= ceil((chunk_offset+chunk_len)/page_size) of every chunk */
    const int32_t *chunk_lens_host;    /* host [num_chunks], each >= 1                 */
    const int32_t *chunk_offsets_host; /* host [num_chunks], each >= 0                 */
    int32_t num_chunks;         /* 1 .. POD_MAX_CHUNKS                                 */
} pod_prefill_batch;

/* What the last call (or pod_attn_plan) decided; the runtime report the
 * Silicon & Systems digest asks for ("Isolation and predictability"):
 * the virtual-workgroup mix, tile choices and the reason for a fallback. */
typedef struct {
    int32_t mode;               /* 0 hybrid, 1 prefill only, 2 decode only            */
    int32_t fallback;           /* 0 none; 1 hybrid without decode ran prefill only;
                                   2 hybrid without prefill ran decode only            */
    int32_t num_cus;            /* compute units the plan was made for                 */
    int32_t wg_per_cu;          /* resident workgroups per CU assumed                  */
    int32_t grid;               /* workgroups launched                                 */
    int32_t prefill_rows_per_tile, prefill_heads_per_tile;
    int32_t prefill_tiles;      /* (row block, kv head, head group) tiles              */
    int32_t prefill_splits;     /* KV splits per tile (of the first chunk in task order,
                                   the one with the longest key range)                */
    int32_t prefill_split_keys; /* keys per split (same chunk)                         */
    int32_t prefill_tasks;      /* tiles * splits over all chunks (prefill workgroups) */
    int32_t decode_split_tokens;/* tokens per decode wave task                         */
    int32_t decode_wave_tasks;  /* (request, kv head, token split) units, one wave each */
    int32_t decode_wg_tasks;    /* decode workgroups (4 wave tasks each)               */
    int32_t share_num, share_den; /* prefill share of each CU's tickets               */
    int32_t cu_prefill_x256;    /* CU-balanced policy: prefill workgroups kept per CU,
                                   averaged over CUs, in 1/256                        */
    int32_t policy;
    int32_t prefill_chunks;     /* prefill chunks of the call (0 without prefill)     */
    int32_t persistent;         /* 1 if the fused launch ran as a resident grid       */
    int32_t fixed_order;        /* fused launch: 0 roles claimed after dispatch; 1 / 2
                                   the prefill / decode tasks went to the first
                                   workgroup ids (a launch resident in one round, or
                                   decode first over several rounds)                 */
    int32_t prefill_priority;   /* 1: prefill waves issued above co-resident decode
                                   waves; 0: equal (a decode-first launch whose
                                   workgroups all start in the first round)         */
    int32_t decode_tail_split_tokens; /* tokens per tail split of a decode request;
                                   0 when the tail is one split                      */
    int32_t decode_unit_classes;/* 8: the requests' shorter remainder splits run
                                   longest first in eight length classes (decode-only
                                   launches and decode-first fused launches of several
                                   rounds); 1: request order; 0 without decodes      */
} pod_attn_stats;

/* Validate `cfg`, pick the device, reserve the workspace.  Returns POD_OK and
 * a handle in *out, or an error and *out = NULL. */
int pod_attn_create(const pod_attn_config *cfg, pod_attn_handle **out);

/* Free the workspace (synchronises the device first).  NULL is a no-op. */
int pod_attn_destroy(pod_attn_handle *h);

/* Fused hybrid batch: both halves in one kernel launch.  Either half may be
 * NULL; the call then runs the other half alone and records why in stats. */
int pod_attn_hybrid(pod_attn_handle *h, const void *k_pool, const void *v_pool, int64_t num_pages,
                    const pod_prefill_args *prefill, const pod_decode_args *decode,
                    pod_stream_t stream);

/* pod_attn_hybrid without a handle, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It allocates nothing: `cfg` is validated as by
 * pod_attn_create (its limits bound the batch the same way), the plan is
 * made for the device named in cfg->device (-1: the current one, which the
 * call makes current either way), and the workspace is a fixed scratch
 * array of POD_NOALLOC_SCRATCH_BYTES in the library's device memory, one
 * copy per GPU, reserved when the library's code is loaded on that GPU and
 * held until the process ends.  The call enqueues two kernels on `stream`:
 * a fill that zeroes the scratch's counters and control words (whatever an
 * earlier call left there), then the fused launch; outputs are bit for bit
 * those of pod_attn_hybrid on the same batch and config.  A batch whose
 * workspace (counters, prefill-split and decode-split partials) exceeds the
 * scratch returns POD_ERR_WORKSPACE before anything is enqueued, and a
 * config with record_roles = 1 POD_ERR_UNSUPPORTED (no trace region); other
 * errors as for pod_attn_create and pod_attn_hybrid (a HIP failure is
 * POD_ERR_HIP; there is no handle, so no error text and no stats).  All
 * calls on one GPU share its scratch: calls that overlap in time on one GPU
 * (two streams, two threads) race and give undefined results. */
#define POD_NOALLOC_SCRATCH_BYTES (64u << 20)
int pod_attn_hybrid_noalloc(const pod_attn_config *cfg, const void *k_pool, const void *v_pool,
                            int64_t num_pages, const pod_prefill_args *prefill,
                            const pod_decode_args *decode, pod_stream_t stream);

/* Prefill half only (the compute-bound baseline kernel). */
int pod_attn_prefill_only(pod_attn_handle *h, const void *k_pool, const void *v_pool,
                          int64_t num_pages, const pod_prefill_args *prefill, pod_stream_t stream);

/* Decode half only (the bandwidth-bound baseline kernel). */
int pod_attn_decode_only(pod_attn_handle *h, const void *k_pool, const void *v_pool,
                         int64_t num_pages, const pod_decode_args *decode, pod_stream_t stream);

/* The same three calls with several prefill chunks (pod_prefill_batch).
 * Chunks run longest key range first; their tiles share the launch like
 * the tiles of one chunk.  Errors as above, and POD_ERR_INVALID_ARG for
 * num_chunks outside 1 .. POD_MAX_CHUNKS, a page_table_stride below a
 * chunk's page count, or chunk lengths summing above max_chunk_len. */
int pod_attn_hybrid_varlen(pod_attn_handle *h, const void *k_pool, const void *v_pool,
                           int64_t num_pages, const pod_prefill_batch *prefill,
                           const pod_decode_args *decode, pod_stream_t stream);
int pod_attn_prefill_only_varlen(pod_attn_handle *h, const void *k_pool, const void *v_pool,
                                 int64_t num_pages, const pod_prefill_batch *prefill,
                                 pod_stream_t stream);
int pod_attn_plan_varlen(const pod_attn_config *cfg, int32_t num_cus, int32_t mode,
                         const pod_prefill_batch *prefill, const pod_decode_args *decode,
                         pod_attn_stats *out);

/* Role trace of the last fused call (pod_attn_hybrid or _varlen) made by a
 * handle created with record_roles = 1: waits for the device, then copies up
 * to `capacity` records into `out` (host memory, prefill tasks first, then
 * decode workgroup tasks) and sets *count to the number the launch wrote
 * (0 if no fused call recorded yet).  POD_ERR_INVALID_ARG if the handle does
 * not record roles.  A diagnostic call: it synchronises the device. */
int pod_attn_role_trace(pod_attn_handle *h, pod_attn_task_record *out, int32_t capacity, int32_t *count);

/* Measured peaks, for a roofline fraction against what the chip sustains
 * next to the published peaks (the reproduction test of the Silicon &
 * Systems digest, "A reproduction and procurement test", asks for achieved
 * memory bandwidth and tensor-core activity).  Both enqueue one kernel on
 * `stream` and return at once; the caller times them with events.
 *
 * pod_attn_peak_read: `workgroups` workgroups of four waves read all `bytes`
 * of device buffer `buf` once, each wave a contiguous slice of
 * bytes / (4 workgroups) with nontemporal 16-byte loads.  The slice must be
 * a multiple of 16384 bytes and at most 1 GiB (POD_ERR_INVALID_ARG
 * otherwise).  `sink` is a device word written only if the XOR of the data
 * equals 0x9e3779b9 (it keeps the loads; a zero-filled buffer never writes).
 *
 * pod_attn_peak_mfma: `workgroups` x 4 waves x `iters` x 16
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) in four independent chains per
 * wave on register operands; `sink` as above. */
int pod_attn_peak_read(const void *buf, int64_t bytes, int32_t workgroups, uint32_t *sink,
                       pod_stream_t stream);
int pod_attn_peak_mfma(int32_t workgroups, int32_t iters, uint32_t *sink, pod_stream_t stream);

/* Copy the plan of the last successful compute call into *out. */
int pod_attn_get_stats(const pod_attn_handle *h, pod_attn_stats *out);

/* Host-only planning: validate the arguments against `cfg` and fill *out with
 * the plan a call in `mode` (0 hybrid, 1 prefill only, 2 decode only) would
 * launch on `num_cus` compute units.  Touches no device; device pointers in
 * the arguments are only checked for NULL. */
int pod_attn_plan(const pod_attn_config *cfg, int32_t num_cus, int32_t mode,
                  const pod_prefill_args *prefill, const pod_decode_args *decode,
                  pod_attn_stats *out);

/* Static description of a status code. */
const char *pod_attn_status_string(int status);

/* Text of the last HIP error seen by this handle ("" if none). */
const char *pod_attn_last_error(const pod_attn_handle *h);

#ifdef __cplusplus
}
#endif

#endif /* POD_ATTN_H */
