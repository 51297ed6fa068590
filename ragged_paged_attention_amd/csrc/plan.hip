// plan.hip -- host planning, the device plan kernel and the launch sequence
// of the specialised path.
#include <stdlib.h>

#include <algorithm>
#include <cmath>

#include "launch.hpp"
#include "plan.hpp"

namespace ra {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

}  // namespace

void make_plan(const ra_shape &s, const int32_t *cu, const int32_t *ctx, Plan *plan, bool short_chunks) {
    Plan pl;
    const int R = s.num_reqs, Hq = s.num_q_heads, Hkv = s.num_kv_heads, D = s.head_dim;
    const int G = Hq / Hkv;
    pl.bounds = !cu || !ctx;
    // Short chunks (2 <= q new tokens, q G <= kShortColumns query columns)
    // run in the decode kernel, whose Q^T columns then hold q tokens x G heads
    // in blocks of 16 (one grid slice each).  dq_max is the largest q of the
    // smallest block count (1 or 2) that takes every such chunk of the batch;
    // more than one block is used only when those wider chunks hold at least
    // half of the decode kernel's pages (the extra slices also stream the
    // pages of every other decode request, for no column); otherwise the
    // wider chunks go to the prefill kernel.  RA_SHORT_CHUNKS=0 in the
    // environment sends all chunks to the prefill kernel.  Not when planning
    // on the device: the partial slots would need the wider column count.
    if (!pl.bounds && short_chunks && G <= kShortColumns / 2) {
        const char *env = getenv("RA_SHORT_CHUNKS");
        const bool on = !(env && env[0] == '0');
        int qmax = 0;
        for (int r = 0; r < R && on; ++r) {
            const int q = cu[r + 1] - cu[r];
            if (q >= 2 && q * G <= kShortColumns) qmax = std::max(qmax, q);
        }
        const int dq1 = 16 / G;  // one block
        if (qmax > 0 && qmax <= dq1) {
            pl.dq_max = dq1;
        } else if (qmax > 0) {
            const int dq = kShortColumns / G;
            long long wide = 0, all = 0;
            for (int r = 0; r < R; ++r) {
                const int q = cu[r + 1] - cu[r];
                if (q < 1 || q > dq) continue;
                const long long nb = decode_blocks(ctx[r], q);
                all += nb;
                if (q > dq1) wide += nb;
            }
            pl.dq_max = 2 * wide >= all ? dq : std::max(1, dq1);
        }
    }
    pl.cw = pl.dq_max * G;
    long long np = 0;
    for (int r = 0; r < R && !pl.bounds; ++r) {
        const int q = cu[r + 1] - cu[r];
        if (decode_kind(q, pl.dq_max)) {
            ++pl.n_decode_reqs;
            const long long nb = decode_blocks(ctx[r], q);  // 16-row blocks of pages
            np += nb;
            pl.max_decode_pages = (int)std::max<long long>(pl.max_decode_pages, nb);
        } else if (q > 1) {
            ++pl.n_prefill_reqs;
        }
    }
    pl.n_decode_pages = (int)np;
    if (pl.bounds) {
        // Every request may be a decode request or a prefill chunk.
        pl.n_decode_reqs = R;
        pl.n_prefill_reqs = R;
    }
    pl.decode_hw = pl.bounds ? decode_heads_per_group(D, Hkv, 0, 0)
                             : decode_heads_per_group(D, Hkv, np, pl.n_decode_reqs);
    pl.decode_hgroups = Hkv / pl.decode_hw;
    pl.decode_wg_cap = pl.n_decode_reqs ? std::max(1, kMaxDecodeWorkgroups / pl.decode_hgroups) : 0;
    pl.q_tile = prefill_supports(D, G) ? prefill_rows(D) / G : 0;
    // The decode kernel takes any group size (blocks of 16 query heads), the
    // prefill kernel up to 256.
    pl.specialised_ok = (s.page_size % 16 == 0) && (D == 64 || D == 128 || D == 256) &&
                        (pl.n_prefill_reqs == 0 || pl.q_tile > 0);
    double dec_bytes = 0, pre_flops = 0;
    if (pl.bounds && pl.q_tile > 0) {
        // Chunks of q >= 2 tokens: sum over them of ceil(q / q_tile) is at
        // most T / q_tile + (their number), and there are at most
        // min(R, T / 2) of them.
        const long long T = s.total_tokens;
        const long long tiles = (T + pl.q_tile - 1) / pl.q_tile + std::min<long long>(R, T / 2);
        pl.n_prefill_items = (int)std::min<long long>(tiles * Hkv, 1LL << 30);
    }
    int q_first = -1, c_first = -1;
    pl.uniform_prefill = !pl.bounds;
    for (int r = 0; r < R && !pl.bounds; ++r) {
        const int q = cu[r + 1] - cu[r];
        if (q > pl.dq_max && pl.q_tile > 0) pl.n_prefill_items += (int)ceil_div(q, pl.q_tile) * Hkv;
        if (q > pl.dq_max) {
            if (q_first < 0) q_first = q, c_first = ctx[r];
            else if (q != q_first || ctx[r] != c_first) pl.uniform_prefill = false;
        }
        if (decode_kind(q, pl.dq_max)) dec_bytes += (double)(ctx[r] + q) * Hkv * D * 4;
        if (q > pl.dq_max) {
            const double c = ctx[r];
            const double pairs = s.causal ? q * c + 0.5 * q * (q + 1.0) : (double)q * (c + q);
            pre_flops += pairs * s.num_q_heads * 4.0 * D;
        }
    }
    // Share of the compute units the decode kernel starts on when a mixed
    // batch runs its prefill kernel beside it: the decode part of the two
    // estimated times (about 6.5 TB/s and 750 TFLOP/s), within [0.4, 0.9].
    if (dec_bytes > 0 && pre_flops > 0) {
        const double td = dec_bytes / 6.5e12, tp = pre_flops / 7.5e14;
        pl.decode_share_pm = (int)(1000 * std::min(0.9, std::max(0.4, td / (td + tp))));
    }
    const int nd = pl.n_decode_reqs;
    // Two partial slots per workgroup, (kv heads of the group) x cw query
    // columns each.  The slots and the workgroup table are sized for the larger of
    // the chosen head-group size and the long-context one, so that the
    // workspace does not depend on the context lengths.
    const int hw_long = decode_heads_per_group(D, Hkv, 0, 0);
    auto wg_cap = [&](int hw) { return std::max(1, kMaxDecodeWorkgroups / (Hkv / hw)); };
    auto slot_heads = [&](int hw) { return (size_t)(Hkv / hw) * wg_cap(hw) * 2 * hw * pl.cw; };
    const size_t part_heads = std::max(slot_heads(pl.decode_hw), slot_heads(hw_long));
    const int cap_max = std::max(wg_cap(pl.decode_hw), wg_cap(hw_long));
    size_t off = 0;
    // The decode list holds the decode requests (plan kernel) or every
    // request (no plan kernel): R entries cover both.
    pl.off_dreq = off;
    off = align256(off + sizeof(int32_t) * (size_t)(nd ? R : 0));
    pl.off_dpfx = off;
    off = align256(off + sizeof(int32_t) * (size_t)(nd ? R + 1 : 0));
    pl.off_wstart = off;
    off = align256(off + sizeof(int32_t) * (size_t)(nd ? cap_max : 0));
    pl.off_part_o = off;
    off = align256(off + sizeof(float) * (nd ? part_heads * D : 0));
    pl.off_part_ml = off;
    off = align256(off + sizeof(float) * (nd ? part_heads * 2 : 0));
    pl.off_ppfx = off;
    off = align256(off + sizeof(int32_t) * ((size_t)R + 1));
    pl.off_prefill = off;
    off = align256(off + 2 * sizeof(int4) * (size_t)pl.n_prefill_items);
    pl.off_counts = off;
    off = align256(off + sizeof(int32_t) * (pl.bounds ? 4 : 0));
    // A batch without new tokens launches nothing and needs no workspace.
    pl.workspace_bytes = (nd == 0 && pl.n_prefill_reqs == 0) ? 0 : off;
    *plan = pl;
}

namespace {

constexpr int kPlanThreads = 1024;

// Block-wide exclusive scan of three counters at once (Hillis-Steele in LDS);
// returns the exclusive prefixes in v and the block totals in tot.
__device__ void scan3(int (*buf)[kPlanThreads], int v[3], int tot[3]) {
    const int tid = threadIdx.x;
    const int own[3] = {v[0], v[1], v[2]};
    for (int k = 0; k < 3; ++k) buf[k][tid] = v[k];
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        int add[3];
        for (int k = 0; k < 3; ++k) add[k] = tid >= off ? buf[k][tid - off] : 0;
        __syncthreads();
        for (int k = 0; k < 3; ++k) buf[k][tid] += add[k];
        __syncthreads();
    }
    for (int k = 0; k < 3; ++k) {
        v[k] = buf[k][tid] - own[k];
        tot[k] = buf[k][kPlanThreads - 1];
    }
    __syncthreads();
}

// Prefix arrays up to this many entries are searched in LDS.
constexpr int kPlanLds = 4096;

// Index of the last entry <= x of the non-decreasing array a[0..n) (global
// memory or LDS).
template <typename P>
__device__ int last_le(P a, int n, int x) {
    int lo = 0, hi = n;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// Writes, from the device metadata: the decode request list and its flat page
// prefix, the first decode request of every decode workgroup, the
// per-request prefix of prefill items and the prefill items themselves
// (longest query tiles of a request first; two int4 per item:
// {r, kv head, first query, first token}, {context, new tokens, 0, 0}).
// Mirrors make_plan.  At most max_items items are written: the workspace
// holds that many (the count the host planned from its copies of the same
// metadata).
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t *cu, const int32_t *ctx, int R, int dq_max, int q_tile, int Hkv, int nwg, int max_items,
    int32_t *dreq, int32_t *dpfx, int32_t *wstart, int32_t *ppfx, int4 *pre, int32_t *counts) {
    __shared__ int buf[3][kPlanThreads];
    __shared__ int dpfx_l[kPlanLds + 1], ppfx_l[kPlanLds + 1];  // LDS copies for the searches
    const int tid = threadIdx.x;
    int base[3] = {0, 0, 0};  // decode requests, decode pages, prefill items
    for (int r0 = 0; r0 < R; r0 += kPlanThreads) {
        const int r = r0 + tid;
        int n[3] = {0, 0, 0};
        if (r < R) {
            const int q = cu[r + 1] - cu[r];
            if (decode_kind(q, dq_max)) {
                n[0] = 1;
                n[1] = decode_blocks(ctx[r], q);
            } else if (q > 1 && q_tile > 0) {
                n[2] = (q + q_tile - 1) / q_tile * Hkv;
            }
        }
        int ex[3] = {n[0], n[1], n[2]}, tot[3];
        scan3(buf, ex, tot);
        if (n[0]) {
            const int i = base[0] + ex[0];
            dreq[i] = r;
            dpfx[i] = base[1] + ex[1];
            if (i <= kPlanLds) dpfx_l[i] = base[1] + ex[1];
        }
        if (r < R) {
            ppfx[r] = base[2] + ex[2];
            if (r <= kPlanLds) ppfx_l[r] = base[2] + ex[2];
        }
        for (int k = 0; k < 3; ++k) base[k] += tot[k];
    }
    const int nd = base[0], np = base[1], npre = base[2];
    // Planning on the device: the decode grid was sized from bounds; only
    // the first nwg of its workgroups per head group take pages, so that
    // none between a request's first and last is empty.
    if (counts) nwg = max(1, min(nwg, np / kMinDecodePages));
    if (tid == 0) {
        if (counts) {  // planning on the device: the kernels read the real counts
            counts[0] = nd;
            counts[1] = np;
            counts[2] = min(npre, max_items);
            counts[3] = nwg;
        }
        dpfx[nd] = np;
        ppfx[R] = npre;
        if (nd <= kPlanLds) dpfx_l[nd] = np;
        if (R <= kPlanLds) ppfx_l[R] = npre;
    }
    __syncthreads();  // the arrays above are read back below
    for (int b = tid; b < nwg && nd > 0; b += kPlanThreads) {
        const int g0 = (int)(((long long)b * np) / nwg);
        wstart[b] = nd <= kPlanLds ? last_le(dpfx_l, nd + 1, g0) : last_le(dpfx, nd + 1, g0);
    }
    for (int k = tid; k < min(npre, max_items); k += kPlanThreads) {
        const int r = R <= kPlanLds ? last_le(ppfx_l, R + 1, k) : last_le(ppfx, R + 1, k);
        const int p0 = R <= kPlanLds ? ppfx_l[r] : ppfx[r];
        const int p1 = R <= kPlanLds ? ppfx_l[r + 1] : ppfx[r + 1];
        const int local = k - p0;
        const int ntiles = (p1 - p0) / Hkv;
        const int rank = local / Hkv, hk = local - rank * Hkv;
        const int qt = ntiles - 1 - rank;  // longest key ranges first
        const int t0 = cu[r], q = cu[r + 1] - t0;
        pre[2 * k] = make_int4(r, hk, qt * q_tile, t0);
        pre[2 * k + 1] = make_int4(ctx[r], q, 0, 0);
    }
}

// The KV-cache update alone (the unfused ablation): one thread per 16-byte
// chunk of a new row, K and V.
__global__ __launch_bounds__(256) void scatter_kernel(Params p) {
    const int cpr = p.D / 8;
    const long long n = (long long)p.T * p.Hkv * cpr;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
        const int col = (int)(i % cpr);
        const long long th = i / cpr;  // token * Hkv + head
        const int t = (int)(th / p.Hkv), h = (int)(th - (long long)t * p.Hkv);
        const size_t src = (size_t)th * p.D + 8 * col;
        const size_t dst = ((size_t)p.slot_mapping[t] * p.Hkv + h) * p.D + 8 * col;
        *reinterpret_cast<uint4 *>(p.k_cache + dst) = *reinterpret_cast<const uint4 *>(p.k_new + src);
        *reinterpret_cast<uint4 *>(p.v_cache + dst) = *reinterpret_cast<const uint4 *>(p.v_new + src);
    }
}

// Concurrent mixed batches: the prefill kernel runs on a second stream next
// to the decode kernel (MFMA-bound and HBM-bound work on different compute
// units).  One side stream and two fork/join events per calling thread and
// device, created on first use and kept until the process ends, so a thread
// that captures a graph and a thread that launches eagerly never share them.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};

thread_local SideStream g_side[64];

hipError_t side_stream(SideStream **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    SideStream &ss = g_side[dev];
    if (!ss.s) {
        e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
        if (e != hipSuccess) return e;
    }
    *out = &ss;
    return hipSuccess;
}

// The prefill items of a mixed batch start on the compute units the decode
// kernel leaves free (nwg of its fill workgroups per head group hold
// cus * nwg / fill units) and run in rounds of about one item per unit.
// With only a few rounds a partial last round costs nearly a whole one, so
// the split moves to the nearer of the two that end the items on whole
// rounds, keeping the decode kernel on 40-90 % of the units.  (Mixed
// workload, 96 decode requests and 512 prefill items: 0.53 of the units,
// 4.2 rounds, 442 us per call; 0.5 and 0.6, 4 and 5 rounds, 430 us.)
int whole_prefill_rounds(int nwg, int fill, int cus, int items) {
    // (The caller caps the result at its full decode grid: with little decode
    // work that grid is far below fill, and a split sized in compute units
    // would ask for more workgroups than the batch has pages.)
    if (fill <= 0 || cus <= 0 || items <= 0 || nwg >= fill) return nwg;
    const double dec = (double)cus * nwg / fill;  // units the decode kernel holds
    const int free_units = cus - (int)dec;
    if (free_units <= 0) return nwg;
    const int rounds = (items + free_units - 1) / free_units;
    if (rounds > 8) return nwg;  // the last of many rounds matters little
    int best = nwg;
    double best_d = 1e30;
    for (int r = std::max(1, rounds - 1); r <= rounds; ++r) {
        const int need = (items + r - 1) / r;  // units that run the items in r rounds
        const int dec_units = cus - need;
        if (dec_units < 0.4 * cus || dec_units > 0.9 * cus) continue;
        const double d = std::fabs(dec_units - dec);
        if (d < best_d) {
            best_d = d;
            best = std::max(1, (int)((long long)fill * dec_units / cus));
        }
    }
    return best;
}

int env_int(const char *name, int dflt) {
    const char *v = getenv(name);
    return v ? atoi(v) : dflt;
}

}  // namespace

hipError_t launch_plan(const Params &p, const Plan &plan, void *workspace, hipStream_t stream,
                       const StageEvents &ev, bool allow_overlap) {
    char *w = (char *)workspace;
    DecodeWork dw;
    dw.dreq = (const int32_t *)(w + plan.off_dreq);
    dw.dpfx = (const int32_t *)(w + plan.off_dpfx);
    dw.wstart = (const int32_t *)(w + plan.off_wstart);
    dw.part_o = (float *)(w + plan.off_part_o);
    dw.part_ml = (float *)(w + plan.off_part_ml);
    dw.nd = plan.n_decode_reqs;
    dw.np = plan.n_decode_pages;
    dw.nwg = 0;
    dw.hw = plan.decode_hw;
    dw.cw = plan.cw;
    // Planning on the device: the plan kernel writes the real counts here,
    // and every grid below is sized from bounds.
    dw.counts = plan.bounds ? (const int32_t *)(w + plan.off_counts) : nullptr;
    // Small batches skip the plan kernel: the decode and prefill kernels find
    // their own work, and the decode list is then every request of the batch.
    // Every prefill workgroup repeats its search over all requests, which pays
    // only with one request per lane (at most kSelfPlanPrefillReqs); a batch
    // with prefill chunks and more requests runs the plan kernel (measured,
    // 512 requests x 64 tokens: 354 us planning in every workgroup, 259 us
    // with the plan kernel's list).  Decode-only batches plan in the kernel up
    // to kSelfPlanReqs requests (one search per decode workgroup).
    const bool has_decode = plan.n_decode_reqs > 0, has_prefill = plan.n_prefill_items > 0;
    const bool self_plan = !plan.bounds && p.R <= (has_prefill ? kSelfPlanPrefillReqs : kSelfPlanReqs) &&
                           env_int("RA_SELF_PLAN", 1) != 0;
    dw.self_plan = self_plan ? 1 : 0;
    if (self_plan && has_decode) dw.nd = p.R;
    // Short contexts (at most 40 16-row blocks per decode request on
    // average, none longer than four times the mean): whole requests per
    // workgroup, an equal share of the list each, so no request is cut and
    // no merge kernel runs.
    const long long nd_dec = plan.n_decode_reqs, np_dec = plan.n_decode_pages;
    dw.whole = (self_plan && has_decode && np_dec <= 40 * nd_dec &&
                (long long)plan.max_decode_pages * nd_dec <= 4 * np_dec &&
                env_int("RA_DECODE_WHOLE", 1) != 0) ? 1 : 0;
    hipError_t err = hipSuccess;
    // A batch with both kinds of work runs its prefill kernel beside the
    // decode kernel (not when the caller times the stages), and the decode
    // kernel then leaves part of the compute units to it at first.
    const bool overlap = allow_overlap && !plan.bounds && !ev.events && has_decode && has_prefill &&
                         env_int("RA_MIXED_OVERLAP", 1) != 0;
    if (has_decode) {
        int fill = 0, cus = 0;
        err = decode_workgroups(p, plan, dw.whole ? dw.nd : 0, &dw.nwg, &fill, &cus);
        if (err != hipSuccess) return err;
        if (overlap) {
            // The reduced grid never exceeds the one computed above, which
            // respects the pages per workgroup and the workspace's slots.
            const int full = dw.nwg;
            const int per_mille = env_int("RA_MIXED_DECODE_SHARE", plan.decode_share_pm);
            dw.nwg = std::max(1, std::min(full, (int)((long long)full * per_mille / 1000)));
            if (env_int("RA_MIXED_ROUNDS", 1) != 0)
                dw.nwg = std::min(full, whole_prefill_rounds(dw.nwg, fill, cus, plan.n_prefill_items));
        }
        // The workspace holds partial slots for decode_wg_cap workgroups per
        // head group.
        if (dw.nwg > plan.decode_wg_cap) return hipErrorInvalidValue;
    }
    int4 *pre = (int4 *)(w + plan.off_prefill);
    // Stage kStagePlan: the unfused ablation's scatter kernel and the plan
    // kernel, whichever run (the first launch takes the start event, the
    // last the stop event).
    if (!p.skip_scatter && self_plan) {
        err = ev.empty(kStagePlan);
        if (err != hipSuccess) return err;
    }
    if (p.skip_scatter) {
        // Unfused ablation: the cache update runs first as its own kernel.
        const long long chunks = (long long)p.T * p.Hkv * (p.D / 8);
        const int blocks = (int)std::min<long long>((chunks + 255) / 256, 4096);
        err = launch_kernel(scatter_kernel, dim3(blocks), dim3(256), 0, stream, ev.start(kStagePlan),
                            self_plan ? ev.stop(kStagePlan) : nullptr, p);
        if (err == hipSuccess) err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (!self_plan) {
        err = launch_kernel(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream,
                            p.skip_scatter ? nullptr : ev.start(kStagePlan), ev.stop(kStagePlan),
                            p.cu_q_lens, p.context_lens, p.R, plan.dq_max, plan.q_tile, p.Hkv, dw.nwg,
                            plan.n_prefill_items, (int32_t *)dw.dreq, (int32_t *)dw.dpfx,
                            (int32_t *)dw.wstart, (int32_t *)(w + plan.off_ppfx), pre, (int32_t *)dw.counts);
        if (err == hipSuccess) err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (overlap) {
        SideStream *ss = nullptr;
        err = side_stream(&ss);
        // The decode kernel is queued first so that its (persistent)
        // workgroups take their compute units before the prefill items do.
        if (err == hipSuccess) err = hipEventRecord(ss->fork, stream);
        if (err == hipSuccess) err = launch_decode(p, dw, stream, ev);
        if (err == hipSuccess) err = hipStreamWaitEvent(ss->s, ss->fork, 0);
        if (err == hipSuccess) err = launch_prefill(p, plan, pre, self_plan, nullptr, true, ss->s);
        if (err == hipSuccess) err = hipEventRecord(ss->join, ss->s);
        if (err == hipSuccess) err = hipStreamWaitEvent(stream, ss->join, 0);
        return err;
    }
    if (has_prefill)
        err = launch_prefill(p, plan, pre, self_plan, dw.counts, false, stream, ev.start(kStagePrefill),
                             ev.stop(kStagePrefill));
    else
        err = ev.empty(kStagePrefill);
    if (err == hipSuccess) {
        if (has_decode) {
            err = launch_decode(p, dw, stream, ev);  // stages kStageDecode and kStageMerge
        } else {
            err = ev.empty(kStageDecode);
            if (err == hipSuccess) err = ev.empty(kStageMerge);
        }
    }
    return err;
}

}  // namespace ra
