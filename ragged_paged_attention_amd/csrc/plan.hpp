// plan.hpp -- the distribution-aware dispatcher: how a batch is cut into
// work items and which kernels run (internal to the library).
//
// The batch is classified per request from the host copies of cu_q_lens and
// context_lens: q_r == 1 is a decode request, q_r > 1 a prefill chunk,
// q_r == 0 has nothing to do.  Decode requests are cut along the key axis
// into splits of `split_tokens` keys (flash-decoding style), so that short
// and long contexts alike spread over all compute units; requests with more
// than one split get a log-sum-exp merge.  Prefill chunks are cut into query
// tiles of `q_tile` tokens per kv head.  The host computes only the counts
// and the workspace layout; a one-workgroup plan kernel writes the item
// lists from the device copies of the same metadata, so no host-to-device
// copy is needed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/ragged_attn.h"
#include "common.hpp"

namespace ra {

struct Plan {
    // classification
    int n_decode_reqs = 0, n_prefill_reqs = 0;
    // decode
    int split_tokens = 0;       // keys per decode split (multiple of the page size)
    int n_decode_items = 0;     // (request, split) pairs; each runs Hkv wavefronts
    int n_merge = 0;            // decode requests with more than one split
    int n_parts = 0;            // partial results written by split requests
    // prefill
    int q_tile = 0;             // query tokens per prefill work item
    int n_prefill_items = 0;    // (request, kv head, query tile) triples
    // which path runs
    bool specialised_ok = false;
    // workspace layout (byte offsets, 256-aligned)
    size_t off_decode = 0, off_merge = 0, off_prefill = 0;
    size_t off_part_o = 0, off_part_ml = 0;
    size_t workspace_bytes = 0;
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
// kv heads per decode workgroup for this head_dim and kv-head count.
int decode_heads_per_group(int D, int Hkv);
hipError_t launch_decode(const Params &p, const Plan &plan, const int4 *items, float *part_o,
                         float *part_ml, hipStream_t stream);
hipError_t launch_merge(const Params &p, const Plan &plan, const int4 *items, const float *part_o,
                        const float *part_ml, hipStream_t stream);
hipError_t launch_prefill(const Params &p, const Plan &plan, const int4 *items,
                          hipStream_t stream);
bool prefill_supports(int D, int G);

}  // namespace ra
