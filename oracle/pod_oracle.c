/*
 * fp64 CPU oracle for hybrid-batch attention.  TEST INFRASTRUCTURE ONLY:
 * nothing on the product path may link, load or call this file; only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg do.
 *
 * What it computes is the plain definition of exact softmax attention, not
 * any tiled or fused algorithm.  The POD-Attention pages state that fusing
 * prefill and decode leaves the attention result unchanged (the Silicon &
 * Systems digest, "Virtual CTAs and SM-aware balance"), and that the kernel
 * is FlashAttention-style exact tiling (same digest, opening section; paper
 * §A.1 says it is built on FlashAttention 2.6.1).  So the oracle is the
 * textbook formula:
 *
 *   for query q of head h, kv head g = floor(h / G) with G = Hq / Hkv
 *   (grouped-query attention, listed among the works the paper builds on),
 *   key j of a request lives at pool[page_table[j / B]][j % B][g][:]
 *   (paged KV cache, PagedAttention, same list);
 *     s_j = scale * sum_k q_k K_jk                  for j in the visible set
 *     O   = sum_j exp(s_j - m) V_j / sum_j exp(s_j - m),  m = max_j s_j
 *
 * Visible sets (chunked prefill in a hybrid batch, paper §2.1):
 *   prefill row i of a chunk at offset P0 sees keys j <= P0 + i
 *     -> written as an explicit mask test over all keys of the request;
 *   decode request r with context L_r sees keys j < L_r
 *     -> written as a loop bound.
 * The two formulations are deliberately different so that a test can check
 * that they agree where they must (decoding row i over context P0+i+1).
 *
 * Arithmetic: inputs are upcast exactly (bf16 and f32 -> double), every
 * product and sum is fp64, two passes (max, then exp/sum), plain index order.
 * Parallel over (row, head) / (request, head) with OpenMP; each output is
 * computed by one thread in a fixed order, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BF16 0
#define ORACLE_F32 1

static double elem(const void *base, int dtype, size_t idx)
{
    if (dtype == ORACLE_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[idx];
}

/* index of element k of kv head g of logical key j of a request */
static size_t kv_index(const int32_t *page_table, int page_size, int hkv, int d,
                       int64_t j, int g, int k)
{
    int64_t page = page_table[j / page_size];
    int64_t slot = j % page_size;
    return (size_t)(((page * page_size + slot) * hkv + g) * (int64_t)d + k);
}

/* Softmax-weighted average of the rows of V over keys 0..n_keys-1 for which
 * visible(j) holds: visible is either "j <= limit" (prefill) or every key
 * below n_keys (decode, limit < 0).  q is one query row, already in fp64. */
static void attend(const double *q, int d, double scale,
                   const double *K, const double *V, int64_t n_keys,
                   int64_t limit, double *scores, double *out, double *lse)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j) {
        if (limit >= 0 && !(j <= limit))
            continue;
        double s = 0.0;
        for (int k = 0; k < d; ++k)
            s += q[k] * K[j * d + k];
        s *= scale;
        scores[j] = s;
        if (s > m)
            m = s;
    }
    double l = 0.0;
    for (int k = 0; k < d; ++k)
        out[k] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        if (limit >= 0 && !(j <= limit))
            continue;
        double e = exp(scores[j] - m);
        l += e;
        for (int k = 0; k < d; ++k)
            out[k] += e * V[j * d + k];
    }
    for (int k = 0; k < d; ++k)
        out[k] /= l;
    if (lse)
        *lse = m + log(l);
}

/* gather keys 0..n-1 of kv head g of one request into contiguous fp64 rows */
static void gather(const void *pool, int dtype, const int32_t *page_table,
                   int page_size, int hkv, int d, int64_t n, int g, double *dst)
{
    for (int64_t j = 0; j < n; ++j)
        for (int k = 0; k < d; ++k)
            dst[j * d + k] = elem(pool, dtype, kv_index(page_table, page_size, hkv, d, j, g, k));
}

static int check_heads(int hq, int hkv, int d, int page_size)
{
    return hq > 0 && hkv > 0 && d > 0 && page_size > 0 && hq % hkv == 0;
}

/*
 * Prefill chunk of chunk_len query rows at absolute positions
 * chunk_offset .. chunk_offset+chunk_len-1.  q: [chunk_len, hq, d].
 * page_table covers ceil((chunk_offset+chunk_len)/page_size) pages.
 * rows: which rows to compute (NULL -> 0..chunk_len-1), nrows entries.
 * out: [nrows, hq, d]; lse: [nrows, hq] or NULL.  Returns 0, or -1 on bad args.
 */
int pod_oracle_prefill(int dtype, int hq, int hkv, int d, int page_size,
                       const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *page_table, int chunk_len, int chunk_offset,
                       double scale, const int32_t *rows, int nrows,
                       double *out, double *lse)
{
    if (!check_heads(hq, hkv, d, page_size) || chunk_len < 1 || chunk_offset < 0 || nrows < 0)
        return -1;
    if (!rows)
        nrows = chunk_len;
    for (int r = 0; r < nrows; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= chunk_len))
            return -1;
    const int G = hq / hkv;
    const int64_t n_keys = (int64_t)chunk_offset + chunk_len;
    double *K = malloc(sizeof(double) * (size_t)n_keys * d);
    double *V = malloc(sizeof(double) * (size_t)n_keys * d);
    if (!K || !V) {
        free(K);
        free(V);
        return -1;
    }
    for (int g = 0; g < hkv; ++g) {
        gather(k_pool, dtype, page_table, page_size, hkv, d, n_keys, g, K);
        gather(v_pool, dtype, page_table, page_size, hkv, d, n_keys, g, V);
        const int64_t work = (int64_t)nrows * G;
#pragma omp parallel
        {
            double *qd = malloc(sizeof(double) * d);
            double *scores = malloc(sizeof(double) * (size_t)n_keys);
#pragma omp for schedule(dynamic, 1)
            for (int64_t w = 0; w < work; ++w) {
                int r = (int)(w / G);
                int h = g * G + (int)(w % G);
                int row = rows ? rows[r] : r;
                for (int k = 0; k < d; ++k)
                    qd[k] = elem(q, dtype, ((size_t)row * hq + h) * d + k);
                attend(qd, d, scale, K, V, n_keys, (int64_t)chunk_offset + row, scores,
                       out + ((size_t)r * hq + h) * d, lse ? lse + (size_t)r * hq + h : NULL);
            }
            free(qd);
            free(scores);
        }
    }
    free(K);
    free(V);
    return 0;
}

/*
 * Decode requests: q [num_decode, hq, d]; page_table [num_decode, stride];
 * context_lens [num_decode] (>= 1).  reqs selects requests (NULL -> all),
 * out [nreqs, hq, d]; lse [nreqs, hq] or NULL.  Returns 0, or -1 on bad args.
 */
int pod_oracle_decode(int dtype, int hq, int hkv, int d, int page_size,
                      const void *q, const void *k_pool, const void *v_pool,
                      const int32_t *page_table, int stride,
                      const int32_t *context_lens, int num_decode, double scale,
                      const int32_t *reqs, int nreqs, double *out, double *lse)
{
    if (!check_heads(hq, hkv, d, page_size) || num_decode < 0 || stride < 1 || nreqs < 0)
        return -1;
    if (!reqs)
        nreqs = num_decode;
    for (int r = 0; r < nreqs; ++r) {
        int req = reqs ? reqs[r] : r;
        if (req < 0 || req >= num_decode || context_lens[req] < 1 ||
            (int64_t)context_lens[req] > (int64_t)stride * page_size)
            return -1;
    }
    const int G = hq / hkv;
    const int64_t work = (int64_t)nreqs * hkv;
    int ok = 1;
#pragma omp parallel
    {
        double *qd = malloc(sizeof(double) * d);
        double *K = NULL, *V = NULL, *scores = NULL;
        int64_t cap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < work; ++w) {
            int r = (int)(w / hkv);
            int g = (int)(w % hkv);
            int req = reqs ? reqs[r] : r;
            int64_t L = context_lens[req];
            if (L > cap) {
                free(K);
                free(V);
                free(scores);
                K = malloc(sizeof(double) * (size_t)L * d);
                V = malloc(sizeof(double) * (size_t)L * d);
                scores = malloc(sizeof(double) * (size_t)L);
                cap = L;
                if (!K || !V || !scores) {
                    ok = 0;
                    cap = 0;
                    continue;
                }
            }
            const int32_t *pt = page_table + (size_t)req * stride;
            gather(k_pool, dtype, pt, page_size, hkv, d, L, g, K);
            gather(v_pool, dtype, pt, page_size, hkv, d, L, g, V);
            for (int hh = 0; hh < G; ++hh) {
                int h = g * G + hh;
                for (int k = 0; k < d; ++k)
                    qd[k] = elem(q, dtype, ((size_t)req * hq + h) * d + k);
                attend(qd, d, scale, K, V, L, -1, scores,
                       out + ((size_t)r * hq + h) * d, lse ? lse + (size_t)r * hq + h : NULL);
            }
        }
        free(qd);
        free(K);
        free(V);
        free(scores);
    }
    return ok ? 0 : -1;
}
