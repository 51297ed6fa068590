// generic.hip -- the simple fused kernel: correct for every supported shape,
// used as the GENERIC variant and as a cross-check of the specialised kernels.
//
// One wavefront per (new token t, kv head hk, block of up to 16 of the G =
// Hq/Hkv query heads of the group).  The first block's wavefront copies the
// token's new K/V row of that head into its cache slot (the fused KV-cache
// update); every wavefront then computes exact attention for its query heads
// with an online softmax over chunks of 64 keys, one key per lane:
//   scores  : each lane dots its key row with the G query rows (fp32 VALU);
//   softmax : chunk max / sum by wave reductions, running (m, l) per head;
//   PV      : the 64 keys are walked in turn, each lane owning D/64 columns.
// Keys at positions < c_r are read from the cache through the page table;
// keys at positions >= c_r (this call's new tokens) are read from k_new /
// v_new, which holds the same values and never races with the update.
#include "common.hpp"
#include "launch.hpp"

namespace ra {

namespace {

constexpr int kMaxG = 16;
constexpr int kMaxD = 256;

__global__ __launch_bounds__(64) void generic_kernel(Params p) {
    const int t = blockIdx.x;
    const int hk = blockIdx.y;
    const int lane = threadIdx.x;
    const int G = p.Hq / p.Hkv;
    const int hq0 = hk * G + kMaxG * blockIdx.z;  // first query head of this block
    const int Gb = min(kMaxG, G - kMaxG * (int)blockIdx.z);  // query heads of this block
    const int D = p.D;

    const int r = request_of_token(p.cu_q_lens, p.R, t);
    const int t0 = p.cu_q_lens[r];
    const int c = p.context_lens[r];
    const int i = t - t0;
    const int L = c + (p.cu_q_lens[r + 1] - t0);
    const int nvis = p.causal ? c + i + 1 : L;
    if (p.prefill_only && L - c == 1) return;

    // KV-cache update for (t, hk), by the first head block.
    if (blockIdx.z == 0) {
        const size_t dst = ((size_t)p.slot_mapping[t] * p.Hkv + hk) * D;
        const size_t src = ((size_t)t * p.Hkv + hk) * D;
        for (int d = lane; d < D; d += 64) {
            p.k_cache[dst + d] = p.k_new[src + d];
            p.v_cache[dst + d] = p.v_new[src + d];
        }
    }

    __shared__ float qs[kMaxG][kMaxD];
    __shared__ float ps[kMaxG][64];
    __shared__ const bf16_t *vrows[64];

    for (int g = 0; g < Gb; ++g) {
        const bf16_t *qrow = p.q + ((size_t)t * p.Hq + hq0 + g) * D;
        for (int d = lane; d < D; d += 64) qs[g][d] = bf16_to_f32(qrow[d]);
    }
    __syncthreads();

    float m[kMaxG], l[kMaxG], acc[kMaxG][kMaxD / 64];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < kMaxD / 64; ++e) acc[g][e] = 0.f;
    }

    for (int j0 = 0; j0 < nvis; j0 += 64) {
        const int j = j0 + lane;
        const bool valid = j < nvis;
        const bf16_t *krow = nullptr, *vrow = nullptr;
        if (valid) {
            if (j < c) {
                const size_t page = (size_t)p.page_table[(size_t)r * p.max_pages + j / p.S];
                const size_t row = page * p.S + j % p.S;
                krow = p.k_cache + (row * p.Hkv + hk) * D;
                vrow = p.v_cache + (row * p.Hkv + hk) * D;
            } else {
                const size_t tt = (size_t)t0 + (j - c);
                krow = p.k_new + (tt * p.Hkv + hk) * D;
                vrow = p.v_new + (tt * p.Hkv + hk) * D;
            }
        }
        float s[kMaxG];
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) s[g] = 0.f;
        if (valid) {
            for (int d = 0; d < D; d += 8) {
                const uint4 kv = *reinterpret_cast<const uint4 *>(krow + d);
                const float kf[8] = {bf16_lo(kv.x), bf16_hi(kv.x), bf16_lo(kv.y), bf16_hi(kv.y),
                                     bf16_lo(kv.z), bf16_hi(kv.z), bf16_lo(kv.w), bf16_hi(kv.w)};
#pragma unroll
                for (int g = 0; g < kMaxG; ++g) {
                    if (g < Gb) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) s[g] += qs[g][d + e] * kf[e];
                    }
                }
            }
        }
        vrows[lane] = vrow;
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) {
            if (g < Gb) {
                const float sg = valid ? s[g] * p.scale_log2 : -INFINITY;
                const float mn = fmaxf(m[g], wave_max(sg));
                const float alpha = fast_exp2(m[g] - mn);
                const float pg = valid ? fast_exp2(sg - mn) : 0.f;
                l[g] = l[g] * alpha + wave_sum(pg);
                m[g] = mn;
#pragma unroll
                for (int e = 0; e < kMaxD / 64; ++e) acc[g][e] *= alpha;
                ps[g][lane] = pg;
            }
        }
        __syncthreads();
        const int nk = min(64, nvis - j0);
        for (int jj = 0; jj < nk; ++jj) {
            const bf16_t *vr = vrows[jj];
#pragma unroll
            for (int e = 0; e < kMaxD / 64; ++e) {
                const int d = lane + 64 * e;
                if (d < D) {
                    const float vf = bf16_to_f32(vr[d]);
#pragma unroll
                    for (int g = 0; g < kMaxG; ++g)
                        if (g < Gb) acc[g][e] += ps[g][jj] * vf;
                }
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
        if (g < Gb) {
            const float inv = 1.f / l[g];
            bf16_t *orow = p.out + ((size_t)t * p.Hq + hq0 + g) * D;
#pragma unroll
            for (int e = 0; e < kMaxD / 64; ++e) {
                const int d = lane + 64 * e;
                if (d < D) orow[d] = (bf16_t)f32_to_bf16(acc[g][e] * inv);
            }
        }
    }
}

}  // namespace

hipError_t launch_generic(const Params &p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
    if (p.T == 0) {
        hipError_t e = ev_start ? hipEventRecord(ev_start, stream) : hipSuccess;
        return (e == hipSuccess && ev_stop) ? hipEventRecord(ev_stop, stream) : e;
    }
    dim3 grid(p.T, p.Hkv, (p.Hq / p.Hkv + kMaxG - 1) / kMaxG);
    hipError_t e = launch_kernel(generic_kernel, grid, dim3(64), 0, stream, ev_start, ev_stop, p);
    return e != hipSuccess ? e : hipGetLastError();
}

bool generic_supports(int D) { return D % 8 == 0 && D <= kMaxD; }

}  // namespace ra
