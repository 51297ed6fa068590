// decode.hip -- the HBM-bound decode kernel (requests with one new token).
//
// Work unit: one workgroup per (request r, key split [kb, ke), group of HW
// kv heads), one wavefront per kv head; the G = Hq/Hkv query heads of a kv
// head share every K/V byte its wavefront reads (grouped-query attention),
// so the cache is read exactly once.
//
// Per 16-token page:
//   * the workgroup loads the page's K and V blocks of its HW heads with
//     16-byte loads in address order (each token row holds the HW heads
//     side by side, so a page arrives as 16 contiguous segments of up to
//     2 KiB), keeping PF pages in flight in a register ring, and stores the
//     page to one of two LDS stages with an XOR chunk swizzle;
//   * each wavefront reads its head's K rows from LDS in the A-operand
//     layout of v_mfma_f32_16x16x32_bf16 (lane = key row, 8 consecutive
//     head_dim elements) and computes the scores transposed, S^T = K . Q^T,
//     with Q^T (zero-padded to 16 heads) as B;
//   * the S^T accumulator layout (lane = head, 4 keys per lane) is already
//     the B-operand layout of v_mfma_f32_16x16x16_bf16 for O^T = V^T . P^T,
//     so P never leaves its registers; V^T comes from the row-major V tile
//     through the gfx950 transposing read ds_read_b64_tr_b16 (each 16-lane
//     group points its lanes at 4 rows x 4 column quads, and lane j receives
//     column j of the 4 rows);
//   * the online softmax runs on S^T: per-head max across the 4 lane groups
//     by two cross-lane steps, running sum kept per lane and reduced once;
//     the accumulator is rescaled only when a max grows past a headroom.
// The split that holds the new token's position writes its K/V rows into the
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

// Prefetch depth (pages in flight per workgroup) per head_dim.
#ifndef RA_DECODE_PF64
#define RA_DECODE_PF64 3
#endif
#ifndef RA_DECODE_PF128
#define RA_DECODE_PF128 3
#endif
#ifndef RA_DECODE_PF256
#define RA_DECODE_PF256 2
#endif

// Headroom of the lazy softmax rescale, in log2 units.
constexpr float kLazyLog2 = 8.f;

// Shape constants of one decode workgroup: HW kv heads, one wavefront each.
template <int D, int HW>
struct DecodeCfg {
    static constexpr int KS = D / 32;            // 16x16x32 k-steps of QK^T
    static constexpr int MB = D / 16;            // 16-row blocks of O^T
    static constexpr int CPH = D / 8;            // 16-byte chunks per head row
    static constexpr int CPR = HW * CPH;         // chunks per row segment (HW heads)
    static constexpr int NTHR = 64 * HW;         // threads
    static constexpr int NC = 16 * CPR / NTHR;   // chunks per thread per tensor and page (= D/32)
    static constexpr int SWM = (CPH < 16 ? CPH : 16) - 1;  // chunk swizzle mask
    static constexpr int HEAD = 16 * D;          // one head's page tile in LDS (elements)
    static constexpr int TENSOR = HW * HEAD;     // one tensor's page block in LDS
    static constexpr int STAGE = 2 * TENSOR;     // K block then V block
    static constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(bf16_t);  // two stages
};

template <int NC>
struct DecodeTile {
    short8_t k[NC];
    short8_t v[NC];
};

template <int D, int HW, int PF>
__global__ __launch_bounds__(64 * HW) void decode_kernel(Params p, const int4 *__restrict__ items,
                                                         float *__restrict__ part_o,
                                                         float *__restrict__ part_ml) {
    using C = DecodeCfg<D, HW>;
    constexpr int KS = C::KS, MB = C::MB, CPH = C::CPH, CPR = C::CPR, NTHR = C::NTHR,
                  NC = C::NC, SWM = C::SWM, HEAD = C::HEAD, TENSOR = C::TENSOR,
                  STAGE = C::STAGE;
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n16 = lane & 15, kg = lane >> 4;
    const int4 it = items[blockIdx.y];
    const int r = it.x;
    if (r < 0) return;
    const int kb = it.y, ke = it.z, part = it.w;
    const int Hkv = p.Hkv, G = p.Hq / Hkv;
    const int hk0 = blockIdx.x * HW;  // first kv head of this workgroup
    const int hk = hk0 + w;           // this wavefront's kv head
    const int t0 = p.cu_q_lens[r];
    const int c = p.context_lens[r];  // position of the new token; keys 0..c

    // Fused KV-cache update of the new token (position c), heads hk0..hk0+HW-1.
    if (c >= kb && c < ke) {
        const size_t dst = ((size_t)p.slot_mapping[t0] * Hkv + hk0) * D;
        const size_t src = ((size_t)t0 * Hkv + hk0) * D;
        for (int ch = tid; ch < CPR; ch += NTHR) {
            reinterpret_cast<uint4 *>(p.k_cache + dst)[ch] = reinterpret_cast<const uint4 *>(p.k_new + src)[ch];
            reinterpret_cast<uint4 *>(p.v_cache + dst)[ch] = reinterpret_cast<const uint4 *>(p.v_new + src)[ch];
        }
    }

    // Q^T as the B operand: lane (head n16, group kg) holds q[t0][hk*G + n16][32ks + 8kg .. +8].
    short8_t qb[KS];
    {
        const bool hv = n16 < G;
        const bf16_t *qrow = p.q + ((size_t)t0 * p.Hq + hk * G + (hv ? n16 : 0)) * D;
        const short8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const short8_t x = *reinterpret_cast<const short8_t *>(qrow + 32 * ks + 8 * kg);
            qb[ks] = hv ? x : z;
        }
    }

    const int pg0 = kb >> 4, pg1 = (ke + 15) >> 4;  // <= 64 pages per split
    const int32_t *ptab = p.page_table + (size_t)r * p.max_pages;
    const int pid_vec = (pg0 + lane < pg1) ? ptab[pg0 + lane] : 0;

    // Cooperative, contiguous page-block loads: chunk u of this thread is the
    // 16-byte chunk tid + NTHR*u of the page's HW-head row segments (row j,
    // head hh of the group, dim chunk dc); it lands in LDS at head hh, row j,
    // chunk dc ^ (j & SWM) (an XOR swizzle that keeps the MFMA-layout reads
    // below free of bank conflicts).
    int row_u[NC], gofs_u[NC], lofs_u[NC], nofs_u[NC];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
        const int q = tid + NTHR * u;
        const int j = q / CPR, cc = q - j * CPR;
        const int hh = cc / CPH, dc = cc - hh * CPH;
        row_u[u] = j;
        gofs_u[u] = (j * Hkv + hk0 + hh) * D + 8 * dc;
        nofs_u[u] = (hk0 + hh) * D + 8 * dc;
        lofs_u[u] = hh * HEAD + j * D + 8 * (dc ^ (j & SWM));
    }
    const size_t page_elems = (size_t)16 * Hkv * D;
    const bf16_t *knew = p.k_new + (size_t)t0 * Hkv * D;
    const bf16_t *vnew = p.v_new + (size_t)t0 * Hkv * D;

    auto load_page = [&](int pg, DecodeTile<NC> &tile) {
        const size_t pid = (size_t)__builtin_amdgcn_readlane(pid_vec, pg - pg0);
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            // Positions >= c are the new token (read from k_new / v_new: the
            // same bits, and never the slot this launch writes) or lie past
            // the request (their scores are masked; reading the new row keeps
            // the stand-in V finite, so 0 * V stays 0).
            const bool cached = pg * 16 + row_u[u] < c;
            const bf16_t *ks = cached ? p.k_cache + pid * page_elems + gofs_u[u] : knew + nofs_u[u];
            const bf16_t *vs = cached ? p.v_cache + pid * page_elems + gofs_u[u] : vnew + nofs_u[u];
            tile.k[u] = *reinterpret_cast<const short8_t *>(ks);
            tile.v[u] = *reinterpret_cast<const short8_t *>(vs);
        }
    };
    auto store_page = [&](int stage, const DecodeTile<NC> &tile) {
        bf16_t *kbase = smem + stage * STAGE;
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            *reinterpret_cast<short8_t *>(kbase + lofs_u[u]) = tile.k[u];
            *reinterpret_cast<short8_t *>(kbase + TENSOR + lofs_u[u]) = tile.v[u];
        }
    };

    float4_t o[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = p.scale_log2;
    const int kend = min(ke, c + 1);
    // This lane's K row (A operand) and V^T transposing-read row.
    const int vrow = 4 * kg + (n16 >> 2);

    auto compute_page = [&](int pg, int stage) {
        const bf16_t *kt = smem + stage * STAGE + w * HEAD;
        const bf16_t *vt = kt + TENSOR;
        // S^T[key][head] = K . Q^T for the 16 keys of this page.
        float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int dc = 4 * ks + kg;
            const short8_t a = *reinterpret_cast<const short8_t *>(kt + n16 * D + 8 * (dc ^ (n16 & SWM)));
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], s, 0, 0, 0);
        }
        // Online softmax; this lane holds keys pg*16 + 4kg + i of head n16.
        const int jb = pg * 16 + 4 * kg;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = (jb + i < kend) ? s[i] * sl2 : -INFINITY;
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // Lazy rescale: the reference max m_run moves only when some head's
        // page max exceeds it by more than kLazyLog2 (P <= 2^kLazyLog2
        // otherwise).  o and l share the reference, so o / l is unchanged.
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyLog2)) {
            const float mn = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - mn);
            l_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
            m_run = mn;
        }
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - m_run);
        l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        const uint32_t p01 = cvt_pk_bf16(pr[0], pr[1]);
        const uint32_t p23 = cvt_pk_bf16(pr[2], pr[3]);
        short4_t pb;
        pb[0] = (short)(p01 & 0xffff);
        pb[1] = (short)(p01 >> 16);
        pb[2] = (short)(p23 & 0xffff);
        pb[3] = (short)(p23 >> 16);
        // O^T[d][head] += V^T[d][key] . P^T[key][head]; A = V^T by transposing
        // reads: lane reads row vrow, columns 16mb + 4(n16 & 3) .. +4.
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int e = 16 * mb + 4 * (n16 & 3);
            const int dc = e >> 3;
            const short4_t va = lds_read_tr16(vt + vrow * D + 8 * (dc ^ (vrow & SWM)) + (e & 7));
            o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[mb], 0, 0, 0);
        }
    };

    // Ring of PF + 1 page tiles in registers: pages pg+1 .. pg+PF are in
    // flight while page pg goes to LDS stage pg & 1 and is computed.  One
    // barrier per page: a stage is rewritten two pages later, after every
    // wavefront has passed the barrier that follows its last read.
    constexpr int NR = PF + 1;
    DecodeTile<NC> ring[NR];
#pragma unroll
    for (int k = 0; k < PF; ++k)
        if (pg0 + k < pg1) load_page(pg0 + k, ring[k]);
    for (int pg = pg0; pg < pg1; pg += NR) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            if (pg + k >= pg1) break;
            if (pg + k + PF < pg1) load_page(pg + k + PF, ring[(k + PF) % NR]);
            store_page((pg + k) & 1, ring[k]);
            __syncthreads();
            compute_page(pg + k, (pg + k) & 1);
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
                uint2 wv;
                wv.x = cvt_pk_bf16(o[mb][0] * inv, o[mb][1] * inv);
                wv.y = cvt_pk_bf16(o[mb][2] * inv, o[mb][3] * inv);
                *reinterpret_cast<uint2 *>(orow + 16 * mb + 4 * kg) = wv;
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

template <int D, int HW, int PF>
hipError_t launch_decode_cfg(const Params &p, const Plan &plan, const int4 *items, float *part_o,
                             float *part_ml, hipStream_t stream) {
    using C = DecodeCfg<D, HW>;
    static bool configured = false;
    if (!configured) {
        hipError_t e = hipFuncSetAttribute((const void *)decode_kernel<D, HW, PF>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)C::LDS_BYTES);
        if (e != hipSuccess) return e;
        configured = true;
    }
    dim3 grid(p.Hkv / HW, plan.n_decode_items);
    hipLaunchKernelGGL((decode_kernel<D, HW, PF>), grid, dim3(64 * HW), C::LDS_BYTES, stream, p,
                       items, part_o, part_ml);
    return hipGetLastError();
}

template <int D, int PF>
hipError_t launch_decode_d(const Params &p, const Plan &plan, const int4 *items, float *part_o,
                           float *part_ml, hipStream_t stream) {
    switch (decode_heads_per_group(D, p.Hkv)) {
        case 8: if constexpr (D <= 128) return launch_decode_cfg<D, 8, PF>(p, plan, items, part_o, part_ml, stream); break;
        case 4: return launch_decode_cfg<D, 4, PF>(p, plan, items, part_o, part_ml, stream);
        case 2: return launch_decode_cfg<D, 2, PF>(p, plan, items, part_o, part_ml, stream);
        case 1: return launch_decode_cfg<D, 1, PF>(p, plan, items, part_o, part_ml, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

int decode_heads_per_group(int D, int Hkv) {
    // Largest HW in {8, 4, 2, 1} dividing Hkv whose row segment (HW heads of
    // one token row) is at most 2 KiB: one page block then arrives as 16
    // contiguous segments.
    for (int hw = 8; hw > 1; hw >>= 1)
        if (Hkv % hw == 0 && hw * D * 2 <= 2048) return hw;
    return 1;
}

hipError_t launch_decode(const Params &p, const Plan &plan, const int4 *items, float *part_o,
                         float *part_ml, hipStream_t stream) {
    switch (p.D) {
        case 64: return launch_decode_d<64, RA_DECODE_PF64>(p, plan, items, part_o, part_ml, stream);
        case 128: return launch_decode_d<128, RA_DECODE_PF128>(p, plan, items, part_o, part_ml, stream);
        case 256: return launch_decode_d<256, RA_DECODE_PF256>(p, plan, items, part_o, part_ml, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ra
