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
//
// The host computes counts and the workspace layout only.  Batches of at
// most kSelfPlanReqs requests need no further planning: the decode and
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

// Prefill item k of a batch of at most kSelfPlanReqs requests, found
// without the plan kernel: the item the plan kernel would
// write at position k (requests in order; per request its query tiles,
// longest key range first, each for every kv head).  Every lane of the
// calling wavefront must take part: lane l holds requests l, l + 64, ...
// (one round trip of loads) and a wave scan of their item counts finds the
// request of item k.
__device__ __forceinline__ void self_plan_prefill_item(const Params &p, int k, int q_tile, int4 &it,
                                                       int4 &it2) {
    constexpr int KR = kSelfPlanReqs / 64;
    const int lane = threadIdx.x & 63, R = p.R;
    int q[KR];
#pragma unroll
    for (int j = 0; j < KR; ++j) {
        const int r = 64 * j + lane;
        q[j] = r < R ? p.cu_q_lens[r + 1] - p.cu_q_lens[r] : 0;
    }
    int base = 0, hit_r = 0, hit_excl = 0;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
        if (64 * j >= R) break;
        const int r = 64 * j + lane;
        const int n = q[j] > 1 ? (q[j] + q_tile - 1) / q_tile * p.Hkv : 0;
        int incl = n;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off, 64);
            if (lane >= off) incl += t;
        }
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(r < R && base + incl > k);
        if (hit) {
            const int ln = __builtin_ctzll(hit);
            hit_r = 64 * j + ln;
            hit_excl = __shfl(base + incl - n, ln, 64);
            break;
        }
        base += __shfl(incl, 63, 64);
    }
    const int r = __builtin_amdgcn_readfirstlane(hit_r);
    const int local = k - __builtin_amdgcn_readfirstlane(hit_excl);
    const int t0 = p.cu_q_lens[r], qr = p.cu_q_lens[r + 1] - t0;
    const int ntiles = (qr + q_tile - 1) / q_tile;
    const int rank = local / p.Hkv, hk = local - rank * p.Hkv;
    it = make_int4(r, hk, (ntiles - 1 - rank) * q_tile, t0);
    it2 = make_int4(p.context_lens[r], qr, 0, 0);
}

// Upper bound of decode workgroups per call (all head groups together); it
// sizes the partial-result slots of the workspace independently of the GPU.
constexpr int kMaxDecodeWorkgroups = 512;

struct Plan {
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
    int decode_share_pm = 1000; // mixed batches: per mille of the decode grid launched beside prefill
    // which path runs
    bool specialised_ok = false;
    // workspace layout (byte offsets, 256-aligned)
    size_t off_dreq = 0, off_dpfx = 0, off_wstart = 0;
    size_t off_part_o = 0, off_part_ml = 0;
    size_t off_ppfx = 0, off_prefill = 0;
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
    int whole;              // 1: workgroup b takes the whole requests [b nd / nwg, (b+1) nd / nwg)
                            // of the list (short contexts, self_plan only): nothing to merge
    int self_plan;          // 1: no plan kernel; the list is every request of the batch (nd =
                            // R, dreq unused), the decode kernel finds its own start and writes
                            // dpfx of the decode requests for the merge kernel
};

// Optional hipEvents recorded at the stage boundaries of one call.
constexpr int kNumStageEvents = 5;
struct StageEvents {
    void *const *events;
    hipStream_t stream;
    StageEvents(void *const *e, hipStream_t s) : events(e), stream(s) {}
    hipError_t record(int k) const {
        return events ? hipEventRecord((hipEvent_t)events[k], stream) : hipSuccess;
    }
};

void make_plan(const ra_shape &s, const int32_t *cu_h, const int32_t *ctx_h, Plan *plan);

hipError_t launch_plan(const Params &p, const Plan &plan, void *workspace, hipStream_t stream,
                       const StageEvents &ev);

// Kernels of the specialised path.
// kv heads per decode workgroup for this head_dim, kv-head count and batch
// (blocks: 16-row page blocks of all nd decode requests).
int decode_heads_per_group(int D, int Hkv, long long blocks, int nd);
// Decode workgroups per head group to launch on the current device (whole:
// list entries when each workgroup takes whole requests, else 0).
hipError_t decode_workgroups(const Params &p, const Plan &plan, int whole, int *nwg);
// Launches the decode kernel, records event 3, launches the merge kernel.
hipError_t launch_decode(const Params &p, const DecodeWork &dw, hipStream_t stream,
                         const StageEvents &ev);
// items: the plan kernel's list, or null when the kernel finds its own
// items (self_plan_prefill_item; batches without decode requests).
hipError_t launch_prefill(const Params &p, const Plan &plan, const int4 *items, bool self_plan,
                          hipStream_t stream);
bool prefill_supports(int D, int G);
// Query rows (heads x tokens) of one prefill workgroup for this head_dim.
int prefill_rows(int D);

}  // namespace ra
