// api.cpp -- the C ABI of libragged_attn: argument checks, metadata
// validation, workspace sizing and the distribution-aware dispatcher.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/ragged_attn.h"
#include "launch.hpp"
#include "plan.hpp"

namespace {

thread_local std::string g_last_error;

ra_status fail(ra_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

// O(1) checks of the shape itself.
ra_status check_shape(const ra_shape *s) {
    if (!s) return fail(RA_E_NULL, "shape is NULL");
    if (s->num_reqs < 0 || s->total_tokens < 0 || s->num_pages < 0 || s->max_pages_per_req < 0)
        return fail(RA_E_SHAPE, "negative size (R=%d T=%d P=%d max_pages=%d)", s->num_reqs,
                    s->total_tokens, s->num_pages, s->max_pages_per_req);
    if (s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->head_dim <= 0 || s->page_size <= 0)
        return fail(RA_E_SHAPE, "heads, head_dim and page_size must be positive");
    if (s->num_q_heads % s->num_kv_heads != 0)
        return fail(RA_E_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    s->num_q_heads, s->num_kv_heads);
    if (!(s->softmax_scale >= 0.f) || isinf(s->softmax_scale))
        return fail(RA_E_SHAPE, "softmax_scale must be finite and >= 0 (0 = 1/sqrt(D))");
    const int D = s->head_dim;
    if (!(D == 64 || D == 128 || D == 256))
        return fail(RA_E_UNSUPPORTED, "head_dim %d not supported (64, 128, 256)", D);
    if (s->page_size % 16 != 0 || s->page_size > 1024)
        return fail(RA_E_UNSUPPORTED, "page_size %d not supported (a multiple of 16, at most 1024)",
                    s->page_size);
    const long long rows = (long long)s->num_pages * s->page_size * s->num_kv_heads * D;
    if (rows > (1LL << 40)) return fail(RA_E_UNSUPPORTED, "cache too large");
    return RA_OK;
}

// O(R) checks of the host copies of cu_q_lens and context_lens.  Both NULL
// means planning on the device from the bounds R and T (nothing to check).
ra_status check_host_lens(const ra_shape *s, const int32_t *cu, const int32_t *ctx) {
    if (!cu && !ctx) return RA_OK;
    if (!cu || !ctx) return fail(RA_E_NULL, "give both host copies (cu_q_lens, context_lens) or neither");
    const int R = s->num_reqs;
    if (cu[0] != 0) return fail(RA_E_METADATA, "cu_q_lens[0] = %d, must be 0", cu[0]);
    for (int r = 0; r < R; ++r) {
        if (cu[r + 1] < cu[r])
            return fail(RA_E_METADATA, "cu_q_lens decreases at request %d", r);
        if (ctx[r] < 0) return fail(RA_E_METADATA, "context_lens[%d] = %d < 0", r, ctx[r]);
        const long long L = (long long)ctx[r] + (cu[r + 1] - cu[r]);
        if (L > (long long)s->max_pages_per_req * s->page_size)
            return fail(RA_E_METADATA, "request %d: length %lld exceeds max_pages_per_req * S", r, L);
        // The kernels index key positions (and tiles past them) in 32 bits.
        if (L >= (1LL << 30))
            return fail(RA_E_UNSUPPORTED, "request %d: length %lld of 2^30 tokens or more", r, L);
    }
    if (cu[R] != s->total_tokens)
        return fail(RA_E_METADATA, "cu_q_lens[R] = %d but total_tokens = %d", cu[R], s->total_tokens);
    return RA_OK;
}

// RA_VALIDATE=1 (environment): copy the device metadata to the host (a
// synchronising copy on the call's stream), check that cu_q_lens and
// context_lens equal the host copies the dispatcher plans from, and run the
// full ra_validate_metadata before anything is launched.
ra_status validate_device_metadata(const ra_shape *s, const int32_t *page_table,
                                   const int32_t *cu_q_lens, const int32_t *context_lens,
                                   const int32_t *slot_mapping, const int32_t *cu_h,
                                   const int32_t *ctx_h, hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess)
        return fail(RA_E_HIP, "RA_VALIDATE: hipStreamIsCapturing failed");
    if (cs != hipStreamCaptureStatusNone)
        return fail(RA_E_UNSUPPORTED, "RA_VALIDATE=1 copies the metadata to the host and cannot run "
                                      "while the stream is being captured");
    const int R = s->num_reqs, T = s->total_tokens;
    std::vector<int32_t> pt((size_t)R * s->max_pages_per_req), cu((size_t)R + 1), ctx((size_t)R), sm((size_t)T);
    auto get = [&](std::vector<int32_t> &dst, const int32_t *src) {
        return dst.empty() ? hipSuccess
                           : hipMemcpyAsync(dst.data(), src, dst.size() * sizeof(int32_t),
                                            hipMemcpyDeviceToHost, stream);
    };
    hipError_t e = get(pt, page_table);
    if (e == hipSuccess) e = get(cu, cu_q_lens);
    if (e == hipSuccess) e = get(ctx, context_lens);
    if (e == hipSuccess) e = get(sm, slot_mapping);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(RA_E_HIP, "RA_VALIDATE: metadata copy failed: %s", hipGetErrorString(e));
    for (int r = 0; r <= R && cu_h; ++r)
        if (cu[r] != cu_h[r])
            return fail(RA_E_METADATA, "device cu_q_lens[%d] = %d, host copy %d", r, cu[r], cu_h[r]);
    for (int r = 0; r < R && ctx_h; ++r)
        if (ctx[r] != ctx_h[r])
            return fail(RA_E_METADATA, "device context_lens[%d] = %d, host copy %d", r, ctx[r], ctx_h[r]);
    return ra_validate_metadata(s, pt.data(), cu.data(), ctx.data(), sm.data());
}

bool validate_requested() {
    const char *v = getenv("RA_VALIDATE");
    return v && v[0] == '1' && v[1] == '\0';
}

}  // namespace

extern "C" {

const char *ra_status_str(ra_status s) {
    switch (s) {
        case RA_OK: return "RA_OK";
        case RA_E_NULL: return "RA_E_NULL: required pointer is NULL";
        case RA_E_SHAPE: return "RA_E_SHAPE: inconsistent or negative sizes";
        case RA_E_UNSUPPORTED: return "RA_E_UNSUPPORTED: outside the built configurations";
        case RA_E_METADATA: return "RA_E_METADATA: metadata violates a precondition";
        case RA_E_WORKSPACE: return "RA_E_WORKSPACE: workspace missing or too small";
        case RA_E_HIP: return "RA_E_HIP: HIP runtime failure";
    }
    return "unknown status";
}

const char *ra_last_error(void) { return g_last_error.c_str(); }

size_t ra_workspace_bytes(const ra_shape *shape, const int32_t *cu_q_lens_host,
                          const int32_t *context_lens_host) {
    if (check_shape(shape) != RA_OK) return 0;
    if (check_host_lens(shape, cu_q_lens_host, context_lens_host) != RA_OK) return 0;
    ra::Plan plan;
    ra::make_plan(*shape, cu_q_lens_host, context_lens_host, &plan);
    return plan.workspace_bytes;
}

ra_status ra_validate_metadata(const ra_shape *s, const int32_t *page_table,
                               const int32_t *cu, const int32_t *ctx, const int32_t *slot) {
    g_last_error.clear();
    ra_status st = check_shape(s);
    if (st != RA_OK && st != RA_E_UNSUPPORTED) return st;
    if (!page_table && s->num_reqs > 0 && s->max_pages_per_req > 0)
        return fail(RA_E_NULL, "page_table is NULL");
    if (!slot && s->total_tokens > 0) return fail(RA_E_NULL, "slot_mapping is NULL");
    st = check_host_lens(s, cu, ctx);
    if (st != RA_OK) return st;
    const int R = s->num_reqs, S = s->page_size, P = s->num_pages, M = s->max_pages_per_req;
    for (int r = 0; r < R; ++r) {
        const long long L = (long long)ctx[r] + (cu[r + 1] - cu[r]);
        const long long np = (L + S - 1) / S;
        for (long long i = 0; i < np; ++i) {
            const int32_t pg = page_table[(size_t)r * M + i];
            if (pg < 0 || pg >= P)
                return fail(RA_E_METADATA, "page_table[%d][%lld] = %d outside [0, %d)", r, i, pg, P);
        }
    }
    std::vector<unsigned char> seen((size_t)P * S, 0);
    for (int r = 0; r < R; ++r) {
        for (int t = cu[r]; t < cu[r + 1]; ++t) {
            const long long pos = (long long)ctx[r] + (t - cu[r]);
            const long long want = (long long)page_table[(size_t)r * M + pos / S] * S + pos % S;
            if ((long long)slot[t] != want)
                return fail(RA_E_METADATA, "slot_mapping[%d] = %d, page table gives %lld", t,
                            slot[t], want);
            if (seen[(size_t)want])
                return fail(RA_E_METADATA, "slot %lld written twice (token %d)", want, t);
            seen[(size_t)want] = 1;
        }
    }
    return RA_OK;
}

}  // extern "C"

namespace {

// The fused call behind every forward entry point.  allow_side_stream lets
// a mixed batch overlap its prefill kernel on a second stream.
ra_status forward_impl(const ra_shape *s, const void *q, const void *k_new, const void *v_new,
                       void *k_cache, void *v_cache, const int32_t *page_table,
                       const int32_t *cu_q_lens, const int32_t *context_lens,
                       const int32_t *slot_mapping, const int32_t *cu_h, const int32_t *ctx_h,
                       void *out, void *workspace, size_t workspace_bytes, void *stream,
                       int32_t variant, void *const *events, int32_t n_events, bool allow_side_stream,
                       bool short_chunks = true) {
    g_last_error.clear();
    if (events && n_events != ra::kNumStageEvents)
        return fail(RA_E_SHAPE, "n_events must be %d", ra::kNumStageEvents);
    if (events)
        for (int k = 0; k < n_events; ++k)
            if (!events[k]) return fail(RA_E_NULL, "events[%d] is NULL", k);
    ra_status st = check_shape(s);
    if (st != RA_OK) return st;
    st = check_host_lens(s, cu_h, ctx_h);
    if (st != RA_OK) return st;
    if (variant < RA_VARIANT_AUTO || variant > RA_VARIANT_UNFUSED)
        return fail(RA_E_SHAPE, "unknown variant %d", variant);
    const bool has_tokens = s->total_tokens > 0;
    if (has_tokens && (!q || !k_new || !v_new || !out || !slot_mapping))
        return fail(RA_E_NULL, "q, k_new, v_new, out and slot_mapping are required");
    if (s->num_reqs > 0 && (!cu_q_lens || !context_lens || !page_table))
        return fail(RA_E_NULL, "cu_q_lens, context_lens and page_table are required");
    if ((has_tokens || s->num_reqs > 0) && (!k_cache || !v_cache))
        return fail(RA_E_NULL, "k_cache and v_cache are required");

    ra::Plan plan;
    ra::make_plan(*s, cu_h, ctx_h, &plan, short_chunks);
    if (workspace_bytes < plan.workspace_bytes)
        return fail(RA_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    plan.workspace_bytes);
    if (plan.workspace_bytes > 0 && (!workspace || ((uintptr_t)workspace & 255u)))
        return fail(RA_E_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
    if (!has_tokens) return RA_OK;
    if (validate_requested()) {
        st = validate_device_metadata(s, page_table, cu_q_lens, context_lens, slot_mapping, cu_h, ctx_h,
                                      (hipStream_t)stream);
        if (st != RA_OK) return st;
    }

    ra::Params p{};
    p.prefill_only = 0;
    p.dq_max = plan.dq_max;
    p.skip_scatter = (variant == RA_VARIANT_UNFUSED && plan.specialised_ok) ? 1 : 0;
    p.q = (const ra::bf16_t *)q;
    p.k_new = (const ra::bf16_t *)k_new;
    p.v_new = (const ra::bf16_t *)v_new;
    p.k_cache = (ra::bf16_t *)k_cache;
    p.v_cache = (ra::bf16_t *)v_cache;
    p.page_table = page_table;
    p.cu_q_lens = cu_q_lens;
    p.context_lens = context_lens;
    p.slot_mapping = slot_mapping;
    p.out = (ra::bf16_t *)out;
    p.R = s->num_reqs;
    p.T = s->total_tokens;
    p.Hq = s->num_q_heads;
    p.Hkv = s->num_kv_heads;
    p.D = s->head_dim;
    p.S = s->page_size;
    p.max_pages = s->max_pages_per_req;
    p.causal = s->causal ? 1 : 0;
    const float scale = s->softmax_scale > 0.f ? s->softmax_scale : 1.0f / sqrtf((float)s->head_dim);
    p.scale_log2 = scale * 1.4426950408889634f;

    hipStream_t hs = (hipStream_t)stream;
    ra::StageEvents ev(events, hs);
    hipError_t err = hipSuccess;
    const char *what = "";
    if (variant == RA_VARIANT_GENERIC || !plan.specialised_ok) {
        what = "generic kernel";
        err = ev.empty(ra::kStagePlan);
        if (err == hipSuccess) err = ra::launch_generic(p, hs, ev.start(ra::kStagePrefill), ev.stop(ra::kStagePrefill));
        if (err == hipSuccess) err = ev.empty(ra::kStageDecode);
        if (err == hipSuccess) err = ev.empty(ra::kStageMerge);
    } else {
        what = "specialised kernels";
        err = ra::launch_plan(p, plan, workspace, hs, ev, allow_side_stream);
    }
    if (err != hipSuccess)
        return fail(RA_E_HIP, "%s launch failed: %s", what, hipGetErrorString(err));
    return RA_OK;
}

}  // namespace

extern "C" {

ra_status ra_forward_profiled(const ra_shape *s, const void *q, const void *k_new, const void *v_new,
                              void *k_cache, void *v_cache, const int32_t *page_table,
                              const int32_t *cu_q_lens, const int32_t *context_lens,
                              const int32_t *slot_mapping, const int32_t *cu_h, const int32_t *ctx_h,
                              void *out, void *workspace, size_t workspace_bytes, void *stream,
                              int32_t variant, void *const *events, int32_t n_events) {
    return forward_impl(s, q, k_new, v_new, k_cache, v_cache, page_table, cu_q_lens, context_lens,
                        slot_mapping, cu_h, ctx_h, out, workspace, workspace_bytes, stream, variant,
                        events, n_events, true);
}

ra_status ra_forward_variant(const ra_shape *s, const void *q, const void *k_new, const void *v_new,
                             void *k_cache, void *v_cache, const int32_t *page_table,
                             const int32_t *cu_q_lens, const int32_t *context_lens,
                             const int32_t *slot_mapping, const int32_t *cu_h, const int32_t *ctx_h,
                             void *out, void *workspace, size_t workspace_bytes, void *stream,
                             int32_t variant) {
    return ra_forward_profiled(s, q, k_new, v_new, k_cache, v_cache, page_table, cu_q_lens,
                               context_lens, slot_mapping, cu_h, ctx_h, out, workspace,
                               workspace_bytes, stream, variant, nullptr, 0);
}

ra_status ra_forward(const ra_shape *s, const void *q, const void *k_new, const void *v_new,
                     void *k_cache, void *v_cache, const int32_t *page_table,
                     const int32_t *cu_q_lens, const int32_t *context_lens,
                     const int32_t *slot_mapping, const int32_t *cu_h, const int32_t *ctx_h,
                     void *out, void *workspace, size_t workspace_bytes, void *stream) {
    return ra_forward_variant(s, q, k_new, v_new, k_cache, v_cache, page_table, cu_q_lens,
                              context_lens, slot_mapping, cu_h, ctx_h, out, workspace,
                              workspace_bytes, stream, RA_VARIANT_AUTO);
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: its workspace is a static device
// array of kScratchBytes (each device the library runs on holds its own copy
// from module load until the process ends).
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;

}  // namespace

// Host code must not pass this name to a kernel: it stands for the host-side
// shadow of the array.  The device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device, set once

// Device address of `scratch` on the current device (looked up once per
// device, with that device current).
ra_status scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RA_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(RA_E_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(RA_E_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return RA_OK;
}

}  // namespace

extern "C" {

ra_status ra_forward_noalloc(const ra_shape *s, const void *q, const void *k_new, const void *v_new,
                             void *k_cache, void *v_cache, const int32_t *page_table,
                             const int32_t *cu_q_lens, const int32_t *context_lens,
                             const int32_t *slot_mapping, const int32_t *cu_h, const int32_t *ctx_h,
                             void *out, void *stream) {
    g_last_error.clear();
    ra_status st = check_shape(s);
    if (st != RA_OK) return st;
    st = check_host_lens(s, cu_h, ctx_h);
    if (st != RA_OK) return st;
    ra::Plan plan;
    ra::make_plan(*s, cu_h, ctx_h, &plan);
    // Short chunks in the decode kernel widen the partial slots; if that
    // does not fit, they run in the prefill kernel instead.
    bool short_chunks = true;
    if (plan.workspace_bytes > kScratchBytes && plan.dq_max > 1) {
        short_chunks = false;
        ra::make_plan(*s, cu_h, ctx_h, &plan, false);
    }
    if (plan.workspace_bytes > kScratchBytes)
        return fail(RA_E_WORKSPACE, "the batch needs %zu bytes of workspace; the static scratch holds %zu",
                    plan.workspace_bytes, kScratchBytes);
    void *ws = nullptr;
    if (plan.workspace_bytes > 0) {
        st = scratch_address(&ws);
        if (st != RA_OK) return st;
    }
    // No side stream (creating one allocates): a mixed batch runs its
    // kernels one after the other on `stream`.
    return forward_impl(s, q, k_new, v_new, k_cache, v_cache, page_table, cu_q_lens, context_lens,
                        slot_mapping, cu_h, ctx_h, out, ws, kScratchBytes, stream, RA_VARIANT_AUTO,
                        nullptr, 0, false, short_chunks);
}

}  // extern "C"
