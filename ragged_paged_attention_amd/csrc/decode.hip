// decode.hip -- the HBM-bound decode kernel (requests with one new token).
//
// Work unit: one wavefront per (request r, key split [kb, ke), kv head hk);
// the G = Hq/Hkv query heads of the group share every K/V byte it reads
// (grouped-query attention), so the cache is read exactly once.
//
// Per 16-token page (the page is the MFMA tile):
//   * K rows go from HBM straight into registers with 16-byte loads, already
//     in the A-operand layout of v_mfma_f32_16x16x32_bf16 (lane = key row,
//     8 consecutive head_dim elements), and the scores are computed
//     transposed, S^T = K . Q^T, with Q^T (zero-padded to 16 heads) as B;
//   * the S^T accumulator layout (lane = head, 4 keys per lane) is already
//     the B-operand layout of v_mfma_f32_16x16x16_bf16 for O^T = V^T . P^T,
//     so P never leaves its registers;
//   * V rows go to LDS as loaded (row-major) and come back as the V^T
//     operand through the gfx950 transposing read ds_read_b64_tr_b16: each
//     16-lane group points its lanes at 4 rows x 4 column quads, and lane j
//     receives column j of the 4 rows (4 consecutive keys);
//   * the online softmax runs on S^T: per-head max across the 4 lane groups
//     by two cross-lane steps, running sum kept per lane and reduced once;
//   * loads run PF pages ahead of the compute (register ring), and the
//     split's page ids are fetched once into a VGPR and read with readlane.
// The split that holds the new token's position writes its K/V row into the
// cache (the fused update); attention reads that key from k_new/v_new.
// Splits of a request with more than one split write unnormalised partials
// (o, m, l) that the merge kernel combines; single-split requests write out.
#include "launch.hpp"
#include "plan.hpp"

namespace ra {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Orders this wavefront's LDS accesses (a workgroup is one wave, and the LDS
// unit executes one wave's operations in order): a compiler-only fence.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

__device__ __forceinline__ short4_t lds_read_tr16(const bf16_t *p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(const_cast<bf16_t *>(p)));
}

template <int D>
struct DecodeTile {
    static constexpr int KS = D / 32;  // 16x16x32 k-steps over head_dim
    short8_t k[KS];
    short8_t v[KS];
};

template <int D, int PF>
__global__ __launch_bounds__(64) void decode_kernel(Params p, const int4 *__restrict__ items,
                                                    float *__restrict__ part_o,
                                                    float *__restrict__ part_ml) {
    constexpr int KS = D / 32;
    constexpr int MB = D / 16;   // O^T row blocks of 16 head_dim elements
    constexpr int RS = D + 16;   // LDS row stride (elements): 4 rows hit distinct banks
    __shared__ __attribute__((aligned(16))) bf16_t vs[16 * RS];

    const int lane = threadIdx.x;
    const int n16 = lane & 15, kg = lane >> 4;
    const int hk = blockIdx.x;
    const int4 it = items[blockIdx.y];
    const int r = it.x;
    if (r < 0) return;
    const int kb = it.y, ke = it.z, part = it.w;
    const int G = p.Hq / p.Hkv;
    const int Hkv = p.Hkv;
    const int t0 = p.cu_q_lens[r];
    const int c = p.context_lens[r];

    // Fused KV-cache update of the new token (position c) for this kv head.
    if (c >= kb && c < ke) {
        const size_t dst = ((size_t)p.slot_mapping[t0] * Hkv + hk) * D;
        const size_t src = ((size_t)t0 * Hkv + hk) * D;
        for (int ch = lane; ch < D / 8; ch += 64) {
            reinterpret_cast<uint4 *>(p.k_cache + dst)[ch] = reinterpret_cast<const uint4 *>(p.k_new + src)[ch];
            reinterpret_cast<uint4 *>(p.v_cache + dst)[ch] = reinterpret_cast<const uint4 *>(p.v_new + src)[ch];
        }
    }

    // Q^T as the B operand: lane (head n16, group kg) holds q[t0][hk*G + n16][32ks + 8kg .. +8].
    short8_t qb[KS];
    {
        const bool hv = n16 < G;
        const bf16_t *qrow = p.q + ((size_t)t0 * p.Hq + hk * G + (hv ? n16 : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const short8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
            const short8_t x = *reinterpret_cast<const short8_t *>(qrow + 32 * ks + 8 * kg);
            qb[ks] = hv ? x : z;
        }
    }

    const int pg0 = kb >> 4, pg1 = (ke + 15) >> 4;
    const int32_t *ptab = p.page_table + (size_t)r * p.max_pages;
    const int pid_vec = (pg0 + lane < pg1) ? ptab[pg0 + lane] : 0;

    auto load_page = [&](int pg, DecodeTile<D> &tile) {
        const int pid = __builtin_amdgcn_readlane(pid_vec, pg - pg0);
        const int jr = pg * 16 + n16;
        const bool valid = jr < ke;
        // Rows past the split read (and then zero) the split's first key, so
        // every lane's address is a valid row.
        const int j = valid ? jr : kb;
        const int pidj = valid ? pid : __builtin_amdgcn_readlane(pid_vec, 0);
        const bf16_t *kr, *vr;
        if (j < c) {
            const size_t row = ((size_t)pidj * 16 + (j & 15)) * Hkv + hk;
            kr = p.k_cache + row * D;
            vr = p.v_cache + row * D;
        } else {
            const size_t row = ((size_t)t0 + (j - c)) * Hkv + hk;
            kr = p.k_new + row * D;
            vr = p.v_new + row * D;
        }
        const short8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const short8_t x = *reinterpret_cast<const short8_t *>(kr + 32 * ks + 8 * kg);
            tile.k[ks] = valid ? x : z;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const short8_t x = *reinterpret_cast<const short8_t *>(vr + 32 * ks + 8 * kg);
            tile.v[ks] = valid ? x : z;
        }
    };

    float4_t o[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = p.scale_log2;
    // Transposing-read address of this lane: row 4kg + n16/4, column quad n16%4.
    const bf16_t *vt_base = vs + (4 * kg + (n16 >> 2)) * RS + 4 * (n16 & 3);

    auto process_page = [&](int pg, const DecodeTile<D> &tile) {
        // S^T[key][head] for the 16 keys of this page.
        float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tile.k[ks], qb[ks], s, 0, 0, 0);
        // V rows into LDS (row = key, as loaded).
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            *reinterpret_cast<short8_t *>(vs + n16 * RS + 32 * ks + 8 * kg) = tile.v[ks];
        // Online softmax; this lane holds keys pg*16 + 4kg + i of head n16.
        const int jb = pg * 16 + 4 * kg;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = (jb + i < ke) ? s[i] * sl2 : -INFINITY;
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - mn);
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - mn);
        l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        m_run = mn;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
        const uint32_t p01 = cvt_pk_bf16(pr[0], pr[1]);
        const uint32_t p23 = cvt_pk_bf16(pr[2], pr[3]);
        short4_t pb;
        pb[0] = (short)(p01 & 0xffff);
        pb[1] = (short)(p01 >> 16);
        pb[2] = (short)(p23 & 0xffff);
        pb[3] = (short)(p23 >> 16);
        wave_lds_fence();
        // O^T[d][head] += V^T[d][key] . P^T[key][head]; A = V^T by transposing reads.
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const short4_t va = lds_read_tr16(vt_base + 16 * mb);
            o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[mb], 0, 0, 0);
        }
        wave_lds_fence();
    };

    if (PF == 1) {
        DecodeTile<D> ta, tb;
        load_page(pg0, ta);
        for (int pg = pg0; pg < pg1; pg += 2) {
            if (pg + 1 < pg1) load_page(pg + 1, tb);
            process_page(pg, ta);
            if (pg + 1 >= pg1) break;
            if (pg + 2 < pg1) load_page(pg + 2, ta);
            process_page(pg + 1, tb);
        }
    } else {
        DecodeTile<D> ta, tb, tc;
        load_page(pg0, ta);
        if (pg0 + 1 < pg1) load_page(pg0 + 1, tb);
        for (int pg = pg0; pg < pg1; pg += 3) {
            if (pg + 2 < pg1) load_page(pg + 2, tc);
            process_page(pg, ta);
            if (pg + 1 >= pg1) break;
            if (pg + 3 < pg1) load_page(pg + 3, ta);
            process_page(pg + 1, tb);
            if (pg + 2 >= pg1) break;
            if (pg + 4 < pg1) load_page(pg + 4, tb);
            process_page(pg + 2, tc);
        }
    }

    // Row sums: add the four lane groups of each head.
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);

    if (n16 < G) {
        const int h = hk * G + n16;
        if (part < 0) {
            const float inv = 1.f / l_tot;
            bf16_t *orow = p.out + ((size_t)t0 * p.Hq + h) * D;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                uint2 w;
                w.x = cvt_pk_bf16(o[mb][0] * inv, o[mb][1] * inv);
                w.y = cvt_pk_bf16(o[mb][2] * inv, o[mb][3] * inv);
                *reinterpret_cast<uint2 *>(orow + 16 * mb + 4 * kg) = w;
            }
        } else {
            float *prow = part_o + ((size_t)part * p.Hq + h) * D;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                *reinterpret_cast<float4_t *>(prow + 16 * mb + 4 * kg) = o[mb];
            if (kg == 0) {
                part_ml[((size_t)part * p.Hq + h) * 2] = m_run;
                part_ml[((size_t)part * p.Hq + h) * 2 + 1] = l_tot;
            }
        }
    }
}

}  // namespace

hipError_t launch_decode(const Params &p, const Plan &plan, const int4 *items, float *part_o,
                         float *part_ml, hipStream_t stream) {
    dim3 grid(p.Hkv, plan.n_decode_items);
    switch (p.D) {
        case 64: hipLaunchKernelGGL((decode_kernel<64, 2>), grid, dim3(64), 0, stream, p, items, part_o, part_ml); break;
        case 128: hipLaunchKernelGGL((decode_kernel<128, 2>), grid, dim3(64), 0, stream, p, items, part_o, part_ml); break;
        case 256: hipLaunchKernelGGL((decode_kernel<256, 1>), grid, dim3(64), 0, stream, p, items, part_o, part_ml); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ra
