/*
 * oracle.c -- plain fp64 CPU oracle for ragged paged attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  The GPU product path never
 * calls it and shares no code, header or constant with it.
 *
 * What it computes (source: "Ragged Paged Attention: A High-Performance and
 * Flexible LLM Inference Kernel for TPU", abstract, and the rocketrecap talk
 * summary, points 00:01:30, 00:06:36 and the glossary entries "FlashAttention",
 * "KV-Cache", "PagedAttention", "Mixed Batching"):
 *   1. the newly projected K/V of every token of a ragged batch are written into
 *      a paged KV cache (the fused KV-cache update);
 *   2. every query token then attends, with exact softmax attention, over its
 *      request's keys/values, read through that request's page table.
 * FlashAttention is exact attention, so the oracle is the plain definition of
 * softmax attention, not the tiled online-softmax algorithm.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - context_lens[r] counts the tokens already in the cache before this call;
 *     the request's total length is L_r = context_lens[r] + q_r.
 *   - query i of request r sits at position c_r + i; with the causal mask it
 *     sees keys 0..c_r+i (bottom-right alignment); without it, keys 0..L_r-1.
 *   - grouped-query attention: q head h reads kv head h / (Hq/Hkv).
 *   - K and V caches are separate arrays of shape [P, S, Hkv, D]; a cache row
 *     has the same shape as a row of k_new / v_new.
 *   - every floating-point step is fp64; bf16 inputs widen exactly.
 *
 * Parity pins: tests/test_oracle.py checks this file against a dense gathered
 * numpy formulation, torch's CPU scaled_dot_product_attention in fp64,
 * closed forms and invariants (page permutation, request order, V shift and
 * linearity), and the exact scatter.  None of those share code with it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Result codes of oracle_check.  Kept local: the GPU library has its own. */
enum {
    ORC_OK = 0,
    ORC_BAD_SHAPE = 1,
    ORC_BAD_CU_Q_LENS = 2,
    ORC_BAD_CONTEXT = 3,
    ORC_TOO_LONG = 4,
    ORC_BAD_PAGE = 5,
    ORC_BAD_SLOT = 6,
    ORC_DUP_SLOT = 7,
};

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Preconditions of the call.  Returns ORC_OK or the first violated rule.
 * page_table is [R, max_pages] row-major; only its first ceil(L_r/S) entries
 * of row r are meaningful.
 */
int oracle_check(int R, int T, int Hq, int Hkv, int D, int S, int P, int max_pages,
                 const int32_t *page_table, const int32_t *cu_q_lens,
                 const int32_t *context_lens, const int32_t *slot_mapping)
{
    if (R < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || S <= 0 || P < 0 || max_pages < 0)
        return ORC_BAD_SHAPE;
    if (Hq % Hkv != 0)
        return ORC_BAD_SHAPE;
    if (cu_q_lens[0] != 0 || cu_q_lens[R] != T)
        return ORC_BAD_CU_Q_LENS;
    for (int r = 0; r < R; ++r)
        if (cu_q_lens[r + 1] < cu_q_lens[r])
            return ORC_BAD_CU_Q_LENS;
    for (int r = 0; r < R; ++r)
        if (context_lens[r] < 0)
            return ORC_BAD_CONTEXT;
    for (int r = 0; r < R; ++r) {
        long long L = (long long)context_lens[r] + (cu_q_lens[r + 1] - cu_q_lens[r]);
        if (L > (long long)max_pages * S)
            return ORC_TOO_LONG;
        long long npages = (L + S - 1) / S;
        for (long long p = 0; p < npages; ++p) {
            int32_t page = page_table[(long long)r * max_pages + p];
            if (page < 0 || page >= P)
                return ORC_BAD_PAGE;
        }
    }
    /* Every new token must be written where its request's page table says its
     * position lives, and no slot may be written twice. */
    unsigned char *seen = (unsigned char *)calloc((size_t)P * S + 1, 1);
    if (!seen)
        return ORC_BAD_SHAPE;
    int rc = ORC_OK;
    for (int r = 0; r < R && rc == ORC_OK; ++r) {
        for (int t = cu_q_lens[r]; t < cu_q_lens[r + 1]; ++t) {
            long long pos = (long long)context_lens[r] + (t - cu_q_lens[r]);
            long long want = (long long)page_table[(long long)r * max_pages + pos / S] * S + pos % S;
            if ((long long)slot_mapping[t] != want) {
                rc = ORC_BAD_SLOT;
                break;
            }
            if (seen[want]) {
                rc = ORC_DUP_SLOT;
                break;
            }
            seen[want] = 1;
        }
    }
    free(seen);
    return rc;
}

/*
 * The KV-cache update: cache row slot_mapping[t] (page slot/S, in-page index
 * slot%S) of every kv head receives the new row of token t.  A bit copy; all
 * other cache rows keep their bits.  Works in place on the arrays given.
 */
void oracle_scatter(int T, int Hkv, int D, int S,
                    const uint16_t *k_new, const uint16_t *v_new, const int32_t *slot_mapping,
                    uint16_t *k_cache, uint16_t *v_cache)
{
    for (int t = 0; t < T; ++t) {
        long long slot = slot_mapping[t];
        long long page = slot / S, in_page = slot % S;
        for (int h = 0; h < Hkv; ++h) {
            long long dst = ((page * S + in_page) * Hkv + h) * (long long)D;
            long long src = ((long long)t * Hkv + h) * D;
            for (int d = 0; d < D; ++d) {
                k_cache[dst + d] = k_new[src + d];
                v_cache[dst + d] = v_new[src + d];
            }
        }
    }
}

/* Shared description of one attention problem (already-scattered cache). */
typedef struct {
    int R, T, Hq, Hkv, D, S, max_pages, causal;
    double scale;
    const uint16_t *q, *k_cache, *v_cache;
    const int32_t *page_table, *cu_q_lens, *context_lens;
} problem;

/* Cache row index (page * S + in-page index) of position j of request r. */
static long long cache_row(const problem *p, int r, long long j)
{
    long long page = p->page_table[(long long)r * p->max_pages + j / p->S];
    return page * p->S + j % p->S;
}

/*
 * Softmax attention of query token t, q head h, in fp64:
 *   s_j = scale * sum_d q[t,h,d] * K[row(j), h/G, d]   for j in the visible set
 *   out = sum_j exp(s_j - max s) V[row(j), h/G, :] / sum_j exp(s_j - max s)
 * scores must hold L_r doubles.
 */
static void attend_one(const problem *p, int r, int t, int h, double *scores, double *out)
{
    const int G = p->Hq / p->Hkv;
    const int hk = h / G;
    const int D = p->D;
    const long long c = p->context_lens[r];
    const long long L = c + (p->cu_q_lens[r + 1] - p->cu_q_lens[r]);
    const long long pos = c + (t - p->cu_q_lens[r]);
    const long long nvis = p->causal ? pos + 1 : L;

    const uint16_t *qrow = p->q + ((long long)t * p->Hq + h) * D;
    double smax = -INFINITY;
    for (long long j = 0; j < nvis; ++j) {
        const uint16_t *krow = p->k_cache + (cache_row(p, r, j) * p->Hkv + hk) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += widen_bf16(qrow[d]) * widen_bf16(krow[d]);
        scores[j] = p->scale * dot;
        if (scores[j] > smax)
            smax = scores[j];
    }
    double denom = 0.0;
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    for (long long j = 0; j < nvis; ++j) {
        double w = exp(scores[j] - smax);
        denom += w;
        const uint16_t *vrow = p->v_cache + (cache_row(p, r, j) * p->Hkv + hk) * D;
        for (int d = 0; d < D; ++d)
            out[d] += w * widen_bf16(vrow[d]);
    }
    for (int d = 0; d < D; ++d)
        out[d] /= denom;
}

static long long max_len(const problem *p)
{
    long long m = 1;
    for (int r = 0; r < p->R; ++r) {
        long long L = (long long)p->context_lens[r] + (p->cu_q_lens[r + 1] - p->cu_q_lens[r]);
        if (L > m)
            m = L;
    }
    return m;
}

/* Request index of every token, from cu_q_lens. */
static int *token_requests(const problem *p)
{
    int *req = (int *)malloc(sizeof(int) * (size_t)(p->T > 0 ? p->T : 1));
    for (int r = 0; r < p->R; ++r)
        for (int t = p->cu_q_lens[r]; t < p->cu_q_lens[r + 1]; ++t)
            req[t] = r;
    return req;
}

/*
 * Attention for every (token, q head): out is [T, Hq, D] fp64.
 * The cache must already hold the new tokens (oracle_scatter first).
 */
void oracle_attention(int R, int T, int Hq, int Hkv, int D, int S, int max_pages,
                      const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                      const int32_t *page_table, const int32_t *cu_q_lens,
                      const int32_t *context_lens, double scale, int causal, double *out)
{
    problem p = {R, T, Hq, Hkv, D, S, max_pages, causal, scale,
                 q, k_cache, v_cache, page_table, cu_q_lens, context_lens};
    const long long Lmax = max_len(&p);
    int *req = token_requests(&p);
    const long long rows = (long long)T * Hq;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)Lmax);
#pragma omp for schedule(dynamic, 1)
        for (long long row = 0; row < rows; ++row) {
            int t = (int)(row / Hq), h = (int)(row % Hq);
            attend_one(&p, req[t], t, h, scores, out + row * D);
        }
        free(scores);
    }
    free(req);
}

/*
 * Attention for a chosen list of (token, q head) pairs only: out is [n, D].
 * Used to sample outputs of batches too large to evaluate in full.
 */
void oracle_attention_rows(int R, int T, int Hq, int Hkv, int D, int S, int max_pages,
                           const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                           const int32_t *page_table, const int32_t *cu_q_lens,
                           const int32_t *context_lens, double scale, int causal,
                           int n, const int32_t *tokens, const int32_t *heads, double *out)
{
    problem p = {R, T, Hq, Hkv, D, S, max_pages, causal, scale,
                 q, k_cache, v_cache, page_table, cu_q_lens, context_lens};
    const long long Lmax = max_len(&p);
    int *req = token_requests(&p);
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)Lmax);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; ++i)
            attend_one(&p, req[tokens[i]], tokens[i], heads[i], scores, out + (long long)i * D);
        free(scores);
    }
    free(req);
}
