// plan.hip -- host planning, the device plan kernel, the split-KV merge
// kernel and the launch sequence of the specialised path.
#include <algorithm>

#include "launch.hpp"
#include "plan.hpp"

namespace ra {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kNumCUs = 256;
// Wavefronts the decode kernel keeps resident per CU at its register budget.
constexpr int kDecodeWavesPerCU = 12;

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Keys per decode split: enough (request, split, kv head) wavefronts to fill
// every CU about three times over, a power of two between 256 and 1024
// (the decode kernel holds one split's page ids in one VGPR: <= 64 pages).
int choose_split(long long decode_keys, int Hkv, int S) {
#ifdef RA_DECODE_SPLIT
    if (RA_DECODE_SPLIT > 0) return RA_DECODE_SPLIT;
#endif
    const long long target_waves = (long long)kNumCUs * kDecodeWavesPerCU * 3;
    long long c = (decode_keys * Hkv + target_waves - 1) / target_waves;
    long long p2 = 256;
    while (p2 < c && p2 < 1024) p2 <<= 1;
    return (int)std::max<long long>(p2, S);
}

}  // namespace

void make_plan(const ra_shape &s, const int32_t *cu, const int32_t *ctx, Plan *plan) {
    Plan pl;
    const int R = s.num_reqs, Hq = s.num_q_heads, Hkv = s.num_kv_heads, D = s.head_dim;
    const int G = Hq / Hkv;
    long long decode_keys = 0;
    for (int r = 0; r < R; ++r) {
        const int q = cu[r + 1] - cu[r];
        if (q == 1) {
            ++pl.n_decode_reqs;
            decode_keys += (long long)ctx[r] + 1;
        } else if (q > 1) {
            ++pl.n_prefill_reqs;
        }
    }
    pl.split_tokens = choose_split(decode_keys, Hkv, s.page_size);
    pl.q_tile = prefill_supports(D, G) ? 128 / G : 0;
    pl.specialised_ok = (s.page_size == 16) && (D == 64 || D == 128 || D == 256) && G <= 16 &&
                        (pl.n_prefill_reqs == 0 || pl.q_tile > 0);
    for (int r = 0; r < R; ++r) {
        const int q = cu[r + 1] - cu[r];
        const long long L = (long long)ctx[r] + q;
        if (q == 1) {
            const int ns = ceil_div(L, pl.split_tokens);
            pl.n_decode_items += ns;
            if (ns > 1) {
                ++pl.n_merge;
                pl.n_parts += ns;
            }
        } else if (q > 1 && pl.q_tile > 0) {
            pl.n_prefill_items += ceil_div(q, pl.q_tile) * Hkv;
        }
    }
    size_t off = 0;
    pl.off_decode = off;
    off = align256(off + sizeof(int4) * (size_t)pl.n_decode_items);
    pl.off_merge = off;
    off = align256(off + sizeof(int4) * (size_t)pl.n_merge);
    pl.off_prefill = off;
    off = align256(off + sizeof(int4) * (size_t)pl.n_prefill_items);
    pl.off_part_o = off;
    off = align256(off + sizeof(float) * (size_t)pl.n_parts * Hq * D);
    pl.off_part_ml = off;
    off = align256(off + sizeof(float) * 2 * (size_t)pl.n_parts * Hq);
    pl.workspace_bytes = off;
    *plan = pl;
}

namespace {

// Block-wide inclusive scan (Hillis-Steele) of four counters at once.
__device__ void scan4(int (*buf)[1024], int v[4]) {
    const int tid = threadIdx.x;
    for (int k = 0; k < 4; ++k) buf[k][tid] = v[k];
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int add[4];
        for (int k = 0; k < 4; ++k) add[k] = tid >= off ? buf[k][tid - off] : 0;
        __syncthreads();
        for (int k = 0; k < 4; ++k) buf[k][tid] += add[k];
        __syncthreads();
    }
    for (int k = 0; k < 4; ++k) v[k] = buf[k][tid];
}

// Writes the decode, merge and prefill item lists from the device metadata.
// Mirrors make_plan; every slot past the device's own counts (up to the
// capacities the host sized) gets r = -1, which the consumers skip.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t *cu, const int32_t *ctx, int R,
                                                    int split, int q_tile, int Hkv, int4 *dec,
                                                    int cap_dec, int4 *mrg, int cap_mrg,
                                                    int4 *pre, int cap_pre, int cap_parts) {
    __shared__ int buf[4][1024];
    const int tid = threadIdx.x;
    int base[4] = {0, 0, 0, 0};  // decode items, merge items, partial slots, prefill items
    for (int r0 = 0; r0 < R; r0 += 1024) {
        const int r = r0 + tid;
        int n[4] = {0, 0, 0, 0};
        int q = 0, L = 0;
        if (r < R) {
            q = cu[r + 1] - cu[r];
            L = ctx[r] + q;
            if (q == 1) {
                n[0] = (L + split - 1) / split;
                if (n[0] > 1) {
                    n[1] = 1;
                    n[2] = n[0];
                }
            } else if (q > 1 && q_tile > 0) {
                n[3] = (q + q_tile - 1) / q_tile * Hkv;
            }
        }
        int incl[4] = {n[0], n[1], n[2], n[3]};
        scan4(buf, incl);
        int o[4];
        for (int k = 0; k < 4; ++k) o[k] = base[k] + incl[k] - n[k];
        if (n[0] > 0) {
            const int part0 = n[2] > 0 ? o[2] : -1;
            for (int sidx = 0; sidx < n[0]; ++sidx) {
                const int idx = o[0] + sidx;
                const bool parts_ok = part0 < 0 || o[2] + n[2] <= cap_parts;
                if (idx < cap_dec)
                    dec[idx] = make_int4(parts_ok ? r : -1, sidx * split, min(L, (sidx + 1) * split),
                                         part0 < 0 ? -1 : part0 + sidx);
            }
            if (n[1] && o[1] < cap_mrg && o[2] + n[2] <= cap_parts)
                mrg[o[1]] = make_int4(r, o[2], n[0], 0);
        }
        if (n[3] > 0) {
            const int ntiles = n[3] / Hkv;
            for (int k = 0; k < ntiles; ++k) {
                const int qt = ntiles - 1 - k;  // longest key ranges first
                for (int hk = 0; hk < Hkv; ++hk) {
                    const int idx = o[3] + k * Hkv + hk;
                    if (idx < cap_pre) pre[idx] = make_int4(r, hk, qt * q_tile, 0);
                }
            }
        }
        for (int k = 0; k < 4; ++k) base[k] += buf[k][1023];
        __syncthreads();
    }
    for (int i = base[0] + tid; i < cap_dec; i += 1024) dec[i] = make_int4(-1, 0, 0, -1);
    for (int i = base[1] + tid; i < cap_mrg; i += 1024) mrg[i] = make_int4(-1, 0, 0, 0);
    for (int i = base[3] + tid; i < cap_pre; i += 1024) pre[i] = make_int4(-1, 0, 0, 0);
}

// Log-sum-exp merge of the split partials of one decode request and q head:
//   M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// (m is kept in the exp2 domain).  One wavefront, lanes over head_dim.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(Params p, const int4 *items, const float *part_o,
                                                   const float *part_ml) {
    const int4 it = items[blockIdx.x];
    if (it.x < 0) return;
    const int h = blockIdx.y, lane = threadIdx.x;
    const int t = p.cu_q_lens[it.x];
    const int base = it.y, ns = it.z;
    float M = -INFINITY;
    for (int sidx = 0; sidx < ns; ++sidx)
        M = fmaxf(M, part_ml[((size_t)(base + sidx) * p.Hq + h) * 2]);
    constexpr int E = D / 64;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    float den = 0.f;
    for (int sidx = 0; sidx < ns; ++sidx) {
        const size_t row = (size_t)(base + sidx) * p.Hq + h;
        const float w = fast_exp2(part_ml[row * 2] - M);
        den += w * part_ml[row * 2 + 1];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += w * part_o[row * D + lane + 64 * e];
    }
    const float inv = 1.f / den;
    bf16_t *orow = p.out + ((size_t)t * p.Hq + h) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[lane + 64 * e] = (bf16_t)f32_to_bf16(acc[e] * inv);
}

}  // namespace

hipError_t launch_merge(const Params &p, const Plan &plan, const int4 *items, const float *part_o,
                        const float *part_ml, hipStream_t stream) {
    dim3 grid(plan.n_merge, p.Hq);
    switch (p.D) {
        case 64: hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, stream, p, items, part_o, part_ml); break;
        case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(64), 0, stream, p, items, part_o, part_ml); break;
        case 256: hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(64), 0, stream, p, items, part_o, part_ml); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_plan(const Params &p, const Plan &plan, void *workspace, hipStream_t stream,
                       const StageEvents &ev) {
    char *w = (char *)workspace;
    int4 *dec = (int4 *)(w + plan.off_decode);
    int4 *mrg = (int4 *)(w + plan.off_merge);
    int4 *pre = (int4 *)(w + plan.off_prefill);
    float *part_o = (float *)(w + plan.off_part_o);
    float *part_ml = (float *)(w + plan.off_part_ml);
    hipError_t err = ev.record(0);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, p.cu_q_lens, p.context_lens,
                       p.R, plan.split_tokens, plan.q_tile, p.Hkv, dec, plan.n_decode_items, mrg,
                       plan.n_merge, pre, plan.n_prefill_items, plan.n_parts);
    err = hipGetLastError();
    if (err == hipSuccess) err = ev.record(1);
    if (err == hipSuccess && plan.n_prefill_items > 0) err = launch_prefill(p, plan, pre, stream);
    if (err == hipSuccess) err = ev.record(2);
    if (err == hipSuccess && plan.n_decode_items > 0)
        err = launch_decode(p, plan, dec, part_o, part_ml, stream);
    if (err == hipSuccess) err = ev.record(3);
    if (err == hipSuccess && plan.n_merge > 0) err = launch_merge(p, plan, mrg, part_o, part_ml, stream);
    if (err == hipSuccess) err = ev.record(4);
    return err;
}

}  // namespace ra
