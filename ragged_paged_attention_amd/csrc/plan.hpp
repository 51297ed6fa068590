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
// The host computes counts and the workspace layout only; a one-workgroup
// plan kernel writes the decode request lists, the workgroup start table and
// the prefill items from the device copies of the same metadata, so no
// host-to-device copy is needed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/ragged_attn.h"
#include "common.hpp"

namespace ra {

// Largest batch of decode requests whose decode kernel plans its own start
// (a wave scan over the requests; larger or mixed batches run the plan kernel).
constexpr int kSelfPlanReqs = 512;

// Upper bound of decode workgroups per call (all head groups together); it
// sizes the partial-result slots of the workspace independently of the GPU.
constexpr int kMaxDecodeWorkgroups = 512;

struct Plan {
    // classification
    int n_decode_reqs = 0, n_prefill_reqs = 0;
    // decode
    int n_decode_pages = 0;     // NP: pages of all decode requests
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
    const int32_t *dpfx;    // [nd + 1]  first flat page of decode request i
    const int32_t *wstart;  // [nwg]     decode request holding workgroup b's first page
    float *part_o;          // [nhg][nwg][2][HW*G][D] partial o (unnormalised)
    float *part_ml;         // [nhg][nwg][2][HW*G][2] partial (m, l)
    int nd, np, nwg;        // decode requests, flat pages, workgroups per head group
    int hw;                 // kv heads per workgroup
    int self_plan;          // 1: every request is a decode request, dreq is the identity and
                            // the decode kernel finds its own start (no plan kernel); it then
                            // writes dreq / dpfx for the merge kernel
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
// Decode workgroups per head group to launch on the current device.
hipError_t decode_workgroups(const Params &p, const Plan &plan, int *nwg);
// Launches the decode kernel, records event 3, launches the merge kernel.
hipError_t launch_decode(const Params &p, const DecodeWork &dw, hipStream_t stream,
                         const StageEvents &ev);
hipError_t launch_prefill(const Params &p, const Plan &plan, const int4 *items,
                          hipStream_t stream);
bool prefill_supports(int D, int G);
// Query rows (heads x tokens) of one prefill workgroup for this head_dim.
int prefill_rows(int D);

}  // namespace ra
