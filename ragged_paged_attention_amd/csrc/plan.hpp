// plan.hpp -- the distribution-aware dispatcher: how a batch is cut into
// work and which kernels run (internal to the library).
//
// The batch is classified per request from the host copies of cu_q_lens and
// context_lens: q_r == 1 is a decode request, q_r > 1 a prefill chunk,
// q_r == 0 has nothing to do.
//
// Decode: the pages of all decode requests, in request order, form one flat
// list of NP pages; a persistent grid of NW workgroups per kv-head group
// takes NP / NW consecutive pages each (stream-K style), so every compute
// unit streams the same number of bytes whatever the context lengths.  A
// request cut by a workgroup boundary is finished by a merge kernel that
// log-sum-exp combines the partial (m, l, o) of its workgroups.
//
// Prefill: chunks are cut into query tiles of `q_tile` tokens per kv head.
// Self-planned batches hand the items out longest first across requests
// (self_plan_prefill_item), or, when every request is a prefill chunk of the
// same length and context and the kernel loops over its items, in request
// order; the plan kernel writes them request by request.
//
// The host computes counts and the workspace layout only.  Decode-only
// batches of at most kSelfPlanReqs requests, and batches with prefill chunks
// of at most kSelfPlanPrefillReqs, need no further planning: the decode and
// prefill kernels find their own work from the device metadata.  Larger
// batches run a one-workgroup plan kernel that writes the decode request
// list, the workgroup start table and the prefill items from the device
// copies of the same metadata, so no host-to-device copy is needed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/ragged_attn.h"
#include "common.hpp"

namespace ra {

// Largest batch whose decode and prefill kernels find their own work with a
// wave scan over the requests; larger batches run the plan kernel.
constexpr int kSelfPlanReqs = 512;
// Largest batch with prefill chunks that plans inside the kernels (one
// request per lane of the prefill kernel's search).
constexpr int kSelfPlanPrefillReqs = 64;

// Key blocks (16 rows) a decode-kernel request with c prior and q new tokens reads.
__host__ __device__ inline int decode_blocks(int c, int q) { return (c + q + 15) >> 4; }

// Whether a request with q new tokens runs in the decode kernel.
__host__ __device__ inline bool decode_kind(int q, int dq_max) { return q >= 1 && q <= dq_max; }

// Query columns per kv head a short chunk may bring to the decode kernel
// (q tokens x G heads), and the 16-column blocks (grid slices) of cw columns.
// Every slice runs the whole page pipeline, and a decode workgroup is bound
// by its page rate, not by HBM: two slices beat the prefill kernel on such
// chunks (128 x 8 tokens after 2048, G = 4: 3.77 against 3.44 TB/s), four
// did not (64 x 16: 2.19 against 3.22 TB/s).
constexpr int kShortColumns = 32;
__host__ __device__ inline int decode_column_blocks(int cw) { return (cw + 15) / 16; }

// Sum (or max) over the wavefront, the same in every lane: DPP within each
// row of 16 lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror), then the four row results read as scalars.
template <bool MAX>
__device__ __forceinline__ int wave_reduce_i(int x) {
    auto op = [](int a, int b) { return MAX ? max(a, b) : a + b; };
    x = op(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
    x = op(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
    x = op(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false));
    x = op(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false));
    return op(op(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
              op(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Prefill item k of a batch of KR * 64 requests at most, found without the
// plan kernel.  Items go out longest first: in decreasing order of the key
// tiles (key_tile keys each) they read, ties in request order, then rank
// (query tile from the last one back), then kv head: with one item per
// workgroup the hardware starts workgroups in index order as compute units
// free up, so this is longest-processing-time-first scheduling across all
// requests, and with one workgroup per unit looping over the items in snake
// order the units get even sums of item lengths.  Every lane of the calling
// wavefront must take part: lane l holds requests l, l + 64, ... (one round
// trip of loads, from cu / ctxl); a binary search over the tile count, each
// step a wave sum of per-request counts in closed form, finds the tile count
// of item k, and a wave scan finds its request, whose metadata the owning
// lane already holds.  A result that falls outside the batch (not expected)
// turns the item into a no-op (it.x = -1).
template <int KR, typename Ptr>
__device__ __forceinline__ void self_plan_prefill_item_k(const Params &p, int k, int q_tile, int key_tile,
                                                         int4 &it, int4 &it2, Ptr cu, Ptr ctxl) {
    const int lane = threadIdx.x & 63, R = p.R, Hkv = p.Hkv;
    // Query tiles: a shift when q_tile is a power of two (G a power of two).
    const bool pow2 = (q_tile & (q_tile - 1)) == 0;
    const int qsh = __builtin_ctz(q_tile);
    auto tiles_of = [&](int x) { return pow2 ? (x + q_tile - 1) >> qsh : (x + q_tile - 1) / q_tile; };
    int t0s[KR], q[KR], c[KR], nt[KR];
    int tmax = 0;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
        const int r = 64 * j + lane;
        t0s[j] = r < R ? cu[r] : 0;
        const int qr = r < R ? cu[r + 1] - t0s[j] : 0;
        q[j] = qr > p.dq_max ? qr : 0;  // decode-kernel and empty requests have no prefill items
        c[j] = r < R ? ctxl[r] : 0;
        nt[j] = tiles_of(q[j]);
        if (q[j]) tmax = max(tmax, (c[j] + q[j] + key_tile - 1) / key_tile);
    }
    tmax = wave_reduce_i<true>(tmax);
    // Ranks of request slot j whose key range ends at or past key x - 1 (at
    // least x keys visible to the tile's last row): rank 0 (the last query
    // tile) ends at c + q, rank rho >= 1 at c + (nt - rho) q_tile; without
    // the causal mask every rank ends at c + q.
    auto cnt_ge = [&](int j, int x) {
        if (q[j] == 0 || c[j] + q[j] < x) return 0;
        const int a = x - c[j];
        if (!p.causal || a <= 0) return nt[j];
        return 1 + max(0, min(nt[j] - 1, nt[j] - tiles_of(a)));
    };
    // Items that read at least lam key tiles.
    auto at_least = [&](int lam) {
        const int x = (lam - 1) * key_tile + 1;
        int s = 0;
#pragma unroll
        for (int j = 0; j < KR; ++j)
            if (64 * j < R) s += cnt_ge(j, x);
        return wave_reduce_i<false>(s) * Hkv;
    };
    // Largest lam with more than k items reading at least lam tiles.
    int lo = 1, hi = tmax + 1;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (at_least(mid) > k) lo = mid;
        else hi = mid;
    }
    const int m = k - at_least(lo + 1);  // position among the items of exactly lo tiles
    const int x_eq = (lo - 1) * key_tile + 1, x_more = lo * key_tile + 1;
    int base = 0, hit_j = -1, hit_ln = 0, hit_excl = 0, hit_rank0 = 0;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
        if (64 * j >= R) break;
        const int r = 64 * j + lane;
        const int longer = cnt_ge(j, x_more);
        const int n = (cnt_ge(j, x_eq) - longer) * Hkv;
        int incl = n;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off, 64);
            if (lane >= off) incl += t;
        }
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(r < R && base + incl > m);
        if (hit) {
            hit_ln = __builtin_ctzll(hit);
            hit_j = j;
            hit_excl = __builtin_amdgcn_readlane(base + incl - n, hit_ln);
            hit_rank0 = __builtin_amdgcn_readlane(longer, hit_ln);
            break;
        }
        base += __builtin_amdgcn_readlane(incl, 63);
    }
    const int j = __builtin_amdgcn_readfirstlane(hit_j);
    const int ln = __builtin_amdgcn_readfirstlane(hit_ln);
    const int local = m - __builtin_amdgcn_readfirstlane(hit_excl);
    const int rank = __builtin_amdgcn_readfirstlane(hit_rank0) + local / Hkv, hk = local % Hkv;
    // The request's metadata from the lane that holds it.
    int t0v = 0, qv = 0, cv = 0;
#pragma unroll
    for (int jj = 0; jj < KR; ++jj)
        if (jj == j) {
            t0v = t0s[jj];
            qv = q[jj];
            cv = c[jj];
        }
    const int r = 64 * j + ln;
    const int t0 = __builtin_amdgcn_readlane(t0v, ln), qr = __builtin_amdgcn_readlane(qv, ln);
    const int ctx = __builtin_amdgcn_readlane(cv, ln);
    const int ntiles = tiles_of(qr);
    if (j < 0 || r >= R || local < 0 || m < 0 || qr <= 1 || rank >= ntiles) {
        it = make_int4(-1, 0, 0, 0);
        it2 = make_int4(0, 0, 0, 0);
        return;
    }
    it = make_int4(r, hk, (ntiles - 1 - rank) * q_tile, t0);
    it2 = make_int4(ctx, qr, 0, 0);
}

// As above for a batch of at most kSelfPlanPrefillReqs requests, reading
// cu_q_lens and context_lens from the device metadata.
__device__ __forceinline__ void self_plan_prefill_item(const Params &p, int k, int q_tile, int key_tile,
                                                       int4 &it, int4 &it2) {
    static_assert(kSelfPlanPrefillReqs == 64, "one request per lane");
    self_plan_prefill_item_k<1>(p, k, q_tile, key_tile, it, it2, p.cu_q_lens, p.context_lens);
}

// The same from copies in LDS (cu: R + 1 entries, ctx: R entries), which a
// kernel that plans once per item takes at its start: vector memory
// operations complete in issue order, so global loads here would wait for
// every store and load the kernel has in flight.
typedef const __attribute__((address_space(3))) int32_t *lds_i32_ptr;
__device__ __forceinline__ void self_plan_prefill_item_lds(const Params &p, int k, int q_tile, int key_tile,
                                                           int4 &it, int4 &it2, lds_i32_ptr cu, lds_i32_ptr ctx) {
    static_assert(kSelfPlanPrefillReqs == 64, "one request per lane");
    self_plan_prefill_item_k<1>(p, k, q_tile, key_tile, it, it2, cu, ctx);
}

// Upper bound of decode workgroups per call (all head groups together); it
// sizes the partial-result slots of the workspace independently of the GPU.
constexpr int kMaxDecodeWorkgroups = 512;
// Fewest pages a decode workgroup's range holds: the grid never has more
// workgroups per head group than decode pages / kMinDecodePages, so every
// workgroup between the first and last of a request owns pages (and a
// partial result the merge kernel reads).
constexpr int kMinDecodePages = 4;

struct Plan {
    // Planning on the device from upper bounds (no host copies of the
    // lengths): the counts below are bounds, the plan kernel always runs and
    // writes the real counts to the workspace, and no launch depends on them.
    bool bounds = false;
    // Requests with 1 <= q <= dq_max new tokens run in the decode kernel,
    // whose 16 Q^T columns then hold q tokens x G heads (dq_max = 16 / G when
    // the batch has such short chunks, else 1); cw: columns per kv head in
    // the decode partial slots (dq_max G).
    int dq_max = 1, cw = 0;
    // classification
    int n_decode_reqs = 0, n_prefill_reqs = 0;
    // decode
    int n_decode_pages = 0;     // NP: pages of all decode requests
    int max_decode_pages = 0;   // pages of the longest decode request
    int decode_hw = 0;          // kv heads per decode workgroup
    int decode_hgroups = 0;     // Hkv / decode_hw
    int decode_wg_cap = 0;      // workgroups per head group the workspace is sized for
    // prefill
    int q_tile = 0;             // query tokens per prefill work item
    int n_prefill_items = 0;    // (request, kv head, query tile) triples
    bool uniform_prefill = false; // every prefill chunk has the same length and context
    int decode_share_pm = 1000; // mixed batches: per mille of the decode grid launched beside prefill
    // which path runs
    bool specialised_ok = false;
    // workspace layout (byte offsets, 256-aligned)
    size_t off_dreq = 0, off_dpfx = 0, off_wstart = 0;
    size_t off_part_o = 0, off_part_ml = 0;
    size_t off_ppfx = 0, off_prefill = 0;
    size_t off_counts = 0;      // int32 {decode requests, decode pages, prefill items, decode
                                // workgroups per head group} (bounds mode)
    size_t workspace_bytes = 0;
};

// The decode work description the decode kernel reads (all in the workspace).
struct DecodeWork {
    const int32_t *dreq;    // [nd]      request id of the i-th decode request
    const int32_t *dpfx;    // [nd]      first flat page of decode request i
    const int32_t *wstart;  // [nwg]     decode request holding workgroup b's first page
    float *part_o;          // [nhg][nwg][2][HW*G][D] partial o (unnormalised)
    float *part_ml;         // [nhg][nwg][2][HW*G][2] partial (m, l)
    int nd, np, nwg;        // decode requests, flat pages, workgroups per head group
    int hw;                 // kv heads per workgroup
    int cw;                 // query columns per kv head in a partial slot
    int whole;              // 1: workgroup b takes the whole requests [b nd / nwg, (b+1) nd / nwg)
                            // of the list (short contexts, self_plan only): nothing to merge
    int self_plan;          // 1: no plan kernel; the list is every request of the batch (nd =
                            // R, dreq unused), the decode kernel finds its own start and writes
                            // dpfx of the decode requests for the merge kernel
    const int32_t *counts;  // planning on the device: {nd, np, prefill items, workgroups} written
                            // by the plan kernel (nd, np and nwg above are then only bounds; the
                            // launched workgroups past counts[3] exit), else null
};

// Optional hipEvents recorded at the stage boundaries of one call.
// Profiled calls: a start and a stop event per stage (plan, prefill, decode,
// merge), given to the stage's kernel launch itself (hipExtLaunchKernel),
// so that each pair brackets the kernel's execution alone; a stage that
// launches nothing has its pair recorded back to back.
constexpr int kNumStages = 4, kNumStageEvents = 2 * kNumStages;
enum Stage { kStagePlan = 0, kStagePrefill = 1, kStageDecode = 2, kStageMerge = 3 };
struct StageEvents {
    void *const *events;
    hipStream_t stream;
    StageEvents(void *const *e, hipStream_t s) : events(e), stream(s) {}
    hipEvent_t start(int stage) const { return events ? (hipEvent_t)events[2 * stage] : nullptr; }
    hipEvent_t stop(int stage) const { return events ? (hipEvent_t)events[2 * stage + 1] : nullptr; }
    hipError_t empty(int stage) const {
        if (!events) return hipSuccess;
        hipError_t e = hipEventRecord(start(stage), stream);
        return e == hipSuccess ? hipEventRecord(stop(stage), stream) : e;
    }
};

// cu_h / ctx_h: host copies of cu_q_lens and context_lens, or both null to
// plan from the upper bounds R and T alone (bounds mode).  short_chunks:
// short chunks may run in the decode kernel (which widens the partial slots).
void make_plan(const ra_shape &s, const int32_t *cu_h, const int32_t *ctx_h, Plan *plan,
               bool short_chunks = true);

// allow_overlap: a mixed batch may run its prefill kernel on the calling
// thread's side stream beside the decode kernel (otherwise the kernels run
// one after the other on `stream`).
hipError_t launch_plan(const Params &p, const Plan &plan, void *workspace, hipStream_t stream,
                       const StageEvents &ev, bool allow_overlap);

// Kernels of the specialised path.
// kv heads per decode workgroup for this head_dim, kv-head count and batch
// (blocks: 16-row page blocks of all nd decode requests).
int decode_heads_per_group(int D, int Hkv, long long blocks, int nd);
// Decode workgroups per head group to launch on the current device (whole:
// list entries when each workgroup takes whole requests, else 0); fill (if
// not null) receives the count that puts one on every compute unit's
// resident slots, cus (if not null) the device's compute units.
hipError_t decode_workgroups(const Params &p, const Plan &plan, int whole, int *nwg, int *fill, int *cus);
// Launches the decode kernel and the merge kernel (stages kStageDecode and
// kStageMerge of ev).
hipError_t launch_decode(const Params &p, const DecodeWork &dw, hipStream_t stream,
                         const StageEvents &ev);
// items: the plan kernel's list, or null when the kernel finds its own
// items (self_plan_prefill_item).
// counts: planning on the device (the item count is counts[2], the grid is
// sized from the bound plan.n_prefill_items), else null.
// spread: one workgroup per item (a mixed batch's prefill kernel beside the
// decode kernel); else, up to head_dim 128, one workgroup per compute unit
// that loops over its items.
// ev_start / ev_stop (may be null): events given to the kernel launch.
hipError_t launch_prefill(const Params &p, const Plan &plan, const int4 *items, bool self_plan,
                          const int32_t *counts, bool spread, hipStream_t stream,
                          hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
bool prefill_supports(int D, int G);
// Query rows (heads x tokens) of one prefill workgroup for this head_dim.
int prefill_rows(int D);

}  // namespace ra
