/*
 * ragged_attn.h -- C ABI of libragged_attn: ragged paged attention with the
 * KV-cache update fused in, for AMD Instinct MI355X (gfx950).
 *
 * The operation (source: "Ragged Paged Attention: A High-Performance and
 * Flexible LLM Inference Kernel for TPU", abstract; rocketrecap.com summary
 * of the talk on that paper, points 00:01:30 "PagedAttention and
 * mixed-batch problem" and 00:06:36 "kernel fusion of KV cache and
 * attention", glossary entries "FlashAttention", "KV-Cache", "Mixed
 * Batching", "PagedAttention", "Ragged Tensors"):
 *
 *   A batch holds R requests.  Request r brings q_r new tokens
 *   (q_r = cu_q_lens[r+1] - cu_q_lens[r]; 1 for a decode step, more for a
 *   prefill chunk, 0 allowed) on top of c_r = context_lens[r] tokens already
 *   in the paged KV cache.  Its total length is L_r = c_r + q_r; position j
 *   of the request lives in cache row (page_table[r][j / S], j % S).
 *
 *   1. KV-cache update: for every new token t and kv head h,
 *        k_cache[slot_mapping[t] / S][slot_mapping[t] % S][h][:] = k_new[t][h][:]
 *      and likewise for v.  A bit copy; no other cache row changes.
 *   2. Attention: the i-th new token of request r (position c_r + i) and
 *      q head h, reading kv head h / (Hq / Hkv), attends with exact softmax
 *      attention over positions 0 .. c_r + i (causal, bottom-right aligned)
 *      or 0 .. L_r - 1 (non-causal):
 *        out[t][h][:] = sum_j softmax_j(scale * q[t][h] . K_j) V_j
 *
 * Layouts (row-major, no padding, bf16 = IEEE bfloat16 bit patterns):
 *   q            [T][Hq][D]             bf16, device
 *   k_new, v_new [T][Hkv][D]            bf16, device
 *   k_cache,
 *   v_cache      [P][S][Hkv][D]         bf16, device, updated in place
 *   page_table   [R][max_pages_per_req] int32, device
 *   cu_q_lens    [R + 1]                int32, device (and a host copy)
 *   context_lens [R]                    int32, device (and a host copy)
 *   slot_mapping [T]                    int32, device; must equal
 *                page_table[r][(c_r+i)/S] * S + (c_r+i) % S for token i of r
 *   out          [T][Hq][D]             bf16, device, written
 *
 * Supported: D in {64, 128, 256}; S a multiple of 16, at most 1024 (the kernels
 * walk the cache in 16-row blocks of a page); any Hq / Hkv >= 1 with
 * Hq % Hkv == 0 (decode rows run in blocks of 16 query heads per kv head;
 * above 16 the cache pages a decode request reads are streamed once per
 * block; prefill rows of groups above 256 heads run the generic kernel);
 * L_r < 2^30 (key positions are 32-bit inside the kernels).
 *
 * Ownership and concurrency: the caller owns every buffer, the workspace
 * included; ra_forward allocates no device memory and keeps no data
 * between calls (ra_forward_noalloc, below, uses a static device array
 * instead of the workspace).  Host pointers are read during the call only.
 * ra_forward is asynchronous on `stream` (a hipStream_t; NULL is the null
 * stream) and never synchronises.  A batch with both decode and prefill
 * requests runs its prefill kernel on a second stream beside the decode
 * kernel, forked from and joined back into `stream` with events (capturable
 * in a graph); that stream and its two events are created per calling
 * thread and device on first use and live until the process ends (so one
 * thread's graph capture never absorbs another thread's eager calls).
 * `out` must not alias any input.  A slot written by this call must not be
 * read, as prior context, by any request of the same call.  Two calls that
 * share a workspace must be ordered on one stream.
 *
 * Errors: every entry point returns a status and never aborts; the detail of
 * the last failure on the calling thread is in ra_last_error().
 */
#ifndef RAGGED_ATTN_H
#define RAGGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RA_OK = 0,
    RA_E_NULL = 1,        /* a required pointer is NULL */
    RA_E_SHAPE = 2,       /* sizes are inconsistent or negative */
    RA_E_UNSUPPORTED = 3, /* valid, but outside what the library is built for */
    RA_E_METADATA = 4,    /* metadata violates a precondition (ra_validate_metadata) */
    RA_E_WORKSPACE = 5,   /* workspace missing, too small or misaligned */
    RA_E_HIP = 6          /* a HIP runtime call or kernel launch failed */
} ra_status;

typedef struct {
    int32_t num_reqs;          /* R >= 0 */
    int32_t total_tokens;      /* T = cu_q_lens[R] */
    int32_t num_q_heads;       /* Hq */
    int32_t num_kv_heads;      /* Hkv, divides Hq */
    int32_t head_dim;          /* D */
    int32_t page_size;         /* S */
    int32_t num_pages;         /* P, pages in k_cache / v_cache */
    int32_t max_pages_per_req; /* columns of page_table */
    float softmax_scale;       /* 0 means 1 / sqrt(D) */
    int32_t causal;            /* nonzero: causal mask, bottom-right aligned */
} ra_shape;

/* Kernel variants.  RA_VARIANT_AUTO lets the dispatcher pick from the batch's
 * decode/prefill mix (the distribution-aware dispatch of the paper's
 * abstract, technique (3)); the others force one path for A/B runs. */
typedef enum {
    RA_VARIANT_AUTO = 0,
    RA_VARIANT_GENERIC = 1,     /* one simple VALU kernel for every request */
    RA_VARIANT_SPECIALISED = 2, /* decode kernel + MFMA prefill kernel */
    RA_VARIANT_UNFUSED = 3      /* ablation of the fusion (the paper's technique of fusing the
                                   KV-cache update into the kernel): the specialised kernels
                                   without the update, preceded by a separate scatter kernel;
                                   same results.  Batches the specialised kernels do not take
                                   run the generic kernel, fused. */
} ra_variant;

/*
 * Bytes of device workspace ra_forward needs for this batch (work lists,
 * merge counters and the partial results of decode requests that several
 * workgroups share).  Host copies of cu_q_lens [R+1] and context_lens [R]
 * are read; with both NULL the result is the bound that covers every batch
 * of the shape's R requests and T new tokens planned on the device (see
 * ra_forward; a batch planned from host copies may need more when short
 * chunks run in the decode kernel).  Returns 0 when the shape is invalid or only one host copy is
 * given.  The size does not depend on the variant.
 */
size_t ra_workspace_bytes(const ra_shape *shape, const int32_t *cu_q_lens_host,
                          const int32_t *context_lens_host);

/*
 * The fused call: KV-cache update plus attention, as defined above.
 *
 * cu_q_lens_host / context_lens_host: host copies of the device metadata;
 * they must hold the same values (the dispatcher plans from them).  Both
 * NULL: the call plans on the device instead (the analogue of the pages'
 * metadata offload, talk summary 00:16:06): a one-workgroup plan kernel
 * builds the work lists and counts from the device metadata, and every grid
 * is sized from the bounds R = num_reqs and T = total_tokens, so no launch
 * parameter depends on the lengths and a call captured in a graph stays
 * valid for any batch of R requests and T new tokens (the workspace then
 * needs ra_workspace_bytes(shape, NULL, NULL)).  A mixed batch then runs its
 * kernels one after the other.
 * workspace: device memory of at least ra_workspace_bytes() bytes, 256-byte
 * aligned; its contents on entry do not matter.
 * Checks are O(1) plus O(R) over the host metadata (cu_q_lens monotone and
 * ending at T, c_r >= 0, L_r <= max_pages_per_req * S); the full
 * O(T + pages) validation of page_table and slot_mapping is the separate
 * ra_validate_metadata.  A call whose page_table or slot_mapping break the
 * rules listed there, or whose device cu_q_lens / context_lens differ from
 * the host copies, is undefined.  With RA_VALIDATE=1 in the environment the
 * call first copies the device metadata to the host (synchronising on
 * `stream`), checks that cu_q_lens and context_lens equal the host copies
 * and runs ra_validate_metadata on it, returning RA_E_METADATA (nothing
 * launched) on a violation; that mode refuses a stream under graph capture
 * (RA_E_UNSUPPORTED).
 * Returns RA_OK once the work is enqueued on `stream`.
 */
ra_status ra_forward(const ra_shape *shape,
                     const void *q, const void *k_new, const void *v_new,
                     void *k_cache, void *v_cache,
                     const int32_t *page_table, const int32_t *cu_q_lens,
                     const int32_t *context_lens, const int32_t *slot_mapping,
                     const int32_t *cu_q_lens_host, const int32_t *context_lens_host,
                     void *out, void *workspace, size_t workspace_bytes, void *stream);

/* ra_forward with an explicit variant (RA_VARIANT_AUTO behaves as ra_forward). */
ra_status ra_forward_variant(const ra_shape *shape,
                             const void *q, const void *k_new, const void *v_new,
                             void *k_cache, void *v_cache,
                             const int32_t *page_table, const int32_t *cu_q_lens,
                             const int32_t *context_lens, const int32_t *slot_mapping,
                             const int32_t *cu_q_lens_host, const int32_t *context_lens_host,
                             void *out, void *workspace, size_t workspace_bytes, void *stream,
                             int32_t variant);

/*
 * ra_forward_variant that also times each kernel of the call with
 * caller-created hipEvent_t handles: events[2 s] and events[2 s + 1] are the
 * start and stop of stage s = 0 plan kernel, 1 prefill kernel, 2 decode
 * kernel, 3 decode merge kernel.  Each pair is given to that kernel's launch
 * (hipExtLaunchKernel), so it brackets the kernel's execution alone, without
 * the launch gap before it; a stage whose kernel does not run has its pair
 * recorded back to back on `stream`, so its duration reads as ~0 (the plan
 * kernel runs only for decode-only batches of more than 512 requests and
 * batches with prefill chunks of more than 64; the unfused variant's scatter
 * kernel is timed with the plan stage; the generic variant runs as the
 * prefill kernel).  A batch with both decode and prefill requests runs its
 * kernels one after the other in a profiled call.  n_events must be 8;
 * events are not created, synchronised or destroyed by the library.
 */
ra_status ra_forward_profiled(const ra_shape *shape,
                              const void *q, const void *k_new, const void *v_new,
                              void *k_cache, void *v_cache,
                              const int32_t *page_table, const int32_t *cu_q_lens,
                              const int32_t *context_lens, const int32_t *slot_mapping,
                              const int32_t *cu_q_lens_host, const int32_t *context_lens_host,
                              void *out, void *workspace, size_t workspace_bytes, void *stream,
                              int32_t variant, void *const *events, int32_t n_events);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ra_forward
 * without a workspace argument.  Its work lists and decode partials live in a
 * static device array of 64 MiB that each device the library runs on holds
 * from the library's load until the process ends (the address is looked up
 * once per device, on the first call with that device current).  A batch
 * whose ra_workspace_bytes() exceeds 64 MiB is refused with RA_E_WORKSPACE
 * before anything is launched (Llama-3-8B shapes need about 17 MB whatever
 * the batch's context lengths; short chunks that would widen that past the
 * limit in the decode kernel run in the prefill kernel instead).  The call allocates nothing itself: a batch
 * with both decode and prefill requests runs its kernels one after the other
 * on `stream`, without the side stream ra_forward may create.  All calls on
 * one device share the array and each call overwrites what the last one left
 * there (its contents on entry do not matter): calls that may overlap on one
 * device (different streams or threads) race, and the caller must order them.
 * Otherwise as ra_forward (same arguments, checks and results).
 */
ra_status ra_forward_noalloc(const ra_shape *shape,
                             const void *q, const void *k_new, const void *v_new,
                             void *k_cache, void *v_cache,
                             const int32_t *page_table, const int32_t *cu_q_lens,
                             const int32_t *context_lens, const int32_t *slot_mapping,
                             const int32_t *cu_q_lens_host, const int32_t *context_lens_host,
                             void *out, void *stream);

/*
 * Full metadata validation on host copies; touches no GPU.  Checks:
 * cu_q_lens[0] == 0, non-decreasing, cu_q_lens[R] == T; c_r >= 0;
 * L_r <= max_pages_per_req * S; the first ceil(L_r / S) page-table entries of
 * every request lie in [0, P); slot_mapping agrees with the page table; no
 * slot is written twice; Hq % Hkv == 0.  Returns RA_OK or RA_E_METADATA /
 * RA_E_SHAPE / RA_E_NULL with the first failure in ra_last_error().
 */
ra_status ra_validate_metadata(const ra_shape *shape, const int32_t *page_table_host,
                               const int32_t *cu_q_lens_host, const int32_t *context_lens_host,
                               const int32_t *slot_mapping_host);

/* Static description of a status code. */
const char *ra_status_str(ra_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *ra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RAGGED_ATTN_H */
