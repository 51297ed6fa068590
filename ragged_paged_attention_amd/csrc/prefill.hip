// prefill.hip -- the MFMA-bound kernel for prefill chunks (requests with more
// than one new token), with the KV-cache update fused in (prefill_pp_kernel,
// head_dim 64, 128 and 256).
//
// Work unit: one workgroup of 8 wavefronts per (request r, kv head hk, query
// tile of QT = floor(256/G) tokens), read from the plan kernel's item list
// or, for batches of at most kSelfPlanPrefillReqs requests, found by the workgroup
// itself (self_plan_prefill_item).  Its 256 query rows are the G query heads
// of the group times the tile's tokens (row R: head R / QT, token R % QT; the
// last 256 - G QT rows are idle), so one K/V tile in LDS serves every head
// that reads it (grouped-query attention); wavefront w owns rows 32 w ..
// 32 w + 31.
//
// Key tiles of N keys (64, or 32 at head_dim 256) stream through four LDS
// stages with direct-to-LDS 16-byte loads (global_load_lds_dwordx4): no
// registers hold data in flight.  Each loading wavefront fetches N/4 key rows
// of a tile (inside one 16-row block of a cache page, so their page id is one
// scalar load); lane l of a 1 KiB load lands at byte 16 l, and each lane
// fetches the chunk that makes the LDS layout XOR swizzled (K chunk c of row
// j at position c ^ (j & SWM)), so the MFMA-layout reads below are free of
// bank conflicts.  Keys at positions < c_r come from the cache through the
// page table, positions >= c_r from k_new/v_new; positions past the tile's
// last visible key read that key again (finite, and masked).
//
// Per tile and wavefront (v_mfma_f32_32x32x16_bf16 throughout):
//   S^T[key][row] = K . Q^T     A = K rows from LDS (16 B per lane),
//                               B = Q^T held in registers for the whole loop
//                               (its last four k-steps in LDS at head_dim 256);
//   online softmax on S^T       each lane owns one query row: the row max is
//                               an in-lane max plus one cross-half step; the
//                               scale is folded into one FMA before exp2; the
//                               accumulator is rescaled only when a row max
//                               grows past a headroom (lazy rescale);
//   O^T[d][row] += V^T . P^T    B = P^T straight from the S^T accumulators
//                               (converted to bf16 with v_cvt_pk_bf16_f32),
//                               A = V^T by ds_read_b64_tr_b16 from the
//                               row-major V tile: each 16-lane group points
//                               at 4 key rows x 4 column quads and lane j
//                               receives column j of those 4 keys.
// Causal masking: tiles beyond the last row's position are never loaded;
// tiles beyond a wavefront's last position are skipped by that wavefront; the
// mask is applied only on tiles that cross a row's limit.
// The workgroup copies the new K/V rows of its own query tokens into the
// cache (each (token, kv head) row is written exactly once).
#include <type_traits>

#include "launch.hpp"
#include "plan.hpp"

namespace ra {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ short4_t lds_read_tr16(const bf16_t *p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(const_cast<bf16_t *>(p)));
}

// 16 bytes from global memory straight into LDS: lane l's chunk lands at
// lds_base + 16 l (lds_base is the same for the whole wavefront).
__device__ __forceinline__ void load_lds16(const bf16_t *g, bf16_t *lds_base) {
    __builtin_amdgcn_global_load_lds((const void *)g, (__attribute__((address_space(3))) void *)lds_base,
                                     16, 0, 0);
}

// Metadata the kernel never writes, read through the constant address space
// (a scalar load when the address is uniform).
__device__ __forceinline__ int ld_meta(const int32_t *a, size_t i) {
    return ((const __attribute__((address_space(4))) int32_t *)a)[i];
}

__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off, 64));
    return x;
}

// Headroom of the lazy softmax rescale, in log2 units.
constexpr float kLazyLog2 = 8.f;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wavefront are outstanding (expcnt and lgkmcnt left at their maximum).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// LDS operand prefetch depth of the prefill kernel.
#ifndef RA_PP_KPF
#define RA_PP_KPF 2
#endif
#ifndef RA_PP_VPF
#define RA_PP_VPF 2
#endif

// ---------------------------------------------------------------------------
// Two groups.
//
// The eight wavefronts form two groups, waves 0-3 and waves 4-7, one wave of
// each per SIMD.  Per key tile a wavefront runs two phases:
//   A(t): the exponentials of tile t-1 (VALU-heavy) and S(t) = K(t) . Q^T;
//   B(t): O += V(t-1) . P(t-1) (MFMA-heavy) and the (masked) row max of S(t).
// Group 1 runs one phase behind group 0 (it passes one extra barrier first,
// group 0 one extra barrier last), so on every SIMD one wave is in an A
// phase while the other is in a B phase: the exponentials of one wave run
// under the MFMAs of the other.  Every phase ends at a workgroup barrier.
//
// Tile t lives in LDS stage t % 4 (separate K and V arrays per stage).  Group
// 0 issues the direct-to-LDS loads of tile t+2 at the start of its B(t) --
// N/4 key rows per wavefront -- and waits for tile t+1 at its end;
// by then every reader of the stage's previous tile (t-2) has passed a
// barrier.  The loop is unrolled by the four stages so that every LDS access
// names its stage array at compile time; the compiler can then tell the
// transposing V reads apart from the loads in flight into other stages and
// does not drain the load queue before them.
// ---------------------------------------------------------------------------
template <int I>
using ic = std::integral_constant<int, I>;

template <int D>
struct PingPongCfg {
    // 64-key tiles up to head_dim 128; 32-key tiles at 256 (the same 32 MFMAs
    // per tile and wavefront, and four stages still fit in LDS).
    static constexpr int NW = 8, MW = 32, N = D > 128 ? 32 : 64;
    static constexpr int NTHR = 64 * NW, ROWS = NW * MW;
    static constexpr int KB = N / 32, KS = D / 16, MD = D / 32, CPR = D / 8;
    static constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;  // K chunk swizzle mask
    static constexpr int VSS = CPR >= 16 ? 4 : 2;           // V chunk swizzle step
    static constexpr int TILE = N * D;                      // elements of one K (or V) tile
    static constexpr int RWL = N / 4;                       // key rows per loading wave and tile
    static constexpr int RPI = 64 / CPR;                    // rows per 1 KiB wavefront load
    static constexpr int IPL = RWL / RPI;                   // loads per loading wave, tensor and tile
    static constexpr int NE = KB * 16;                      // scores per lane and tile
    static constexpr int EP = NE / 2;                       // exponential pairs per lane and tile
    static constexpr int NB = (N / 16) * MD;                // B chunks
    static constexpr int EB = NE / NB;                      // row-max elements per B chunk
    static constexpr int KPF = RA_PP_KPF, VPF = RA_PP_VPF;  // LDS read prefetch depth (k-steps, B chunks)
    // The last QKS k-steps of Q^T sit in LDS instead of registers at head_dim
    // 256, where O (128 registers) and all of Q^T (64) would leave too few
    // registers for two wavefronts per SIMD; 32 KiB, so LDS holds 160 KiB.
    static constexpr int QKS = D > 128 ? 4 : 0;
    static constexpr int KQR = KS - QKS;                    // k-steps of Q^T in registers
    static constexpr int QCH = 2 * QKS;                     // 16-byte chunks per row in LDS
    static_assert(16 % RWL == 0 && RWL % RPI == 0, "a loading wave's rows of a tile lie in one 16-row block");
    static_assert(EB >= 1 && NE % NB == 0, "B chunks split the scores evenly");
};

template <int D>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(Params p, const int4 *__restrict__ items, int self_plan,
                                                            int q_tile) {
    using C = PingPongCfg<D>;
    constexpr int ROWS = C::ROWS, N = C::N, KB = C::KB, KS = C::KS, MD = C::MD, CPR = C::CPR,
                  SWM = C::SWM, VSS = C::VSS, TILE = C::TILE, RWL = C::RWL, RPI = C::RPI, IPL = C::IPL,
                  NTHR = C::NTHR, NE = C::NE, EP = C::EP, NB = C::NB, EB = C::EB, KPF = C::KPF,
                  VPF = C::VPF, KQR = C::KQR, QCH = C::QCH;
    // One array per stage and tensor (see above).
    __shared__ __attribute__((aligned(16))) bf16_t k0[TILE], k1[TILE], k2[TILE], k3[TILE];
    __shared__ __attribute__((aligned(16))) bf16_t v0[TILE], v1[TILE], v2[TILE], v3[TILE];
    // Q^T k-steps KQR .. KS-1: row R's chunk c at c ^ ((R >> 1) & (QCH - 1)),
    // so the 16 rows a 16-lane group reads hit 16 different bank groups.
    // Every lane reads back only what it wrote itself.
    __shared__ __attribute__((aligned(16))) bf16_t qlds[QCH ? ROWS * 8 * QCH : 8];
    auto kst = [&](auto s) -> bf16_t * {
        constexpr int S = decltype(s)::value;
        if constexpr (S == 0) return k0;
        else if constexpr (S == 1) return k1;
        else if constexpr (S == 2) return k2;
        else return k3;
    };
    auto vst = [&](auto s) -> bf16_t * {
        constexpr int S = decltype(s)::value;
        if constexpr (S == 0) return v0;
        else if constexpr (S == 1) return v1;
        else if constexpr (S == 2) return v2;
        else return v3;
    };

    // The item carries everything the prologue needs, so that every load of
    // the prologue (new K/V rows, Q, the first two tiles) goes out at once.
    int4 it, it2;
    if (self_plan) {
        self_plan_prefill_item(p, blockIdx.x, q_tile, N, it, it2);
    } else {
        it = items[2 * blockIdx.x];
        it2 = items[2 * blockIdx.x + 1];
    }
    const int r = it.x;
    if (r < 0) return;
    const int hk = it.y, q0 = it.z, t0 = it.w, c = it2.x, qlen = it2.y;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar wavefront index
    const int grp = w >> 2;
    const int l = tid & 63, n32 = l & 31, h2 = l >> 5;
    const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv, QT = ROWS / G;
    const int L = c + qlen;
    const int tile_q = min(QT, qlen - q0);
    const int kv_end = p.causal ? c + q0 + tile_q : L;  // keys 0 .. kv_end-1 are visible to someone
    const int ntiles = (kv_end + N - 1) / N;
    const size_t prow = (size_t)r * p.max_pages;

    // Fused KV-cache update, the new rows of this tile's tokens for kv head
    // hk: loaded here with the other prologue loads, stored after them.
    const int kv_chunks = p.skip_scatter ? 0 : tile_q * CPR;
    // Two 16-byte chunks per thread and tensor cover tile_q <= 64 rows (at
    // head_dim 128; G >= 4); larger tiles copy the rest after the prologue.
    constexpr int KVU = 2;
    short8_t kvk[KVU], kvv[KVU];
    int kvslot[KVU];
#pragma unroll
    for (int i = 0; i < KVU; ++i) {
        const int idx = tid + i * NTHR;
        if (idx < kv_chunks) {
            const int row = idx / CPR, col = idx - row * CPR;
            const int t = t0 + q0 + row;
            const size_t src = ((size_t)t * Hkv + hk) * D + 8 * col;
            kvslot[i] = p.slot_mapping[t];
            kvk[i] = *reinterpret_cast<const short8_t *>(p.k_new + src);
            kvv[i] = *reinterpret_cast<const short8_t *>(p.v_new + src);
        }
    }

    // A value the compiler must recompute from here at each use instead of
    // keeping derived values live across the loop, where registers are short.
    auto opaque = [](uint32_t x) {
        asm volatile("" : "+v"(x));
        return x;
    };

    // This lane's query row R = 32 w + n32: head g = R / QT, token i = R % QT.
    const int R = 32 * w + n32;
    // When G does not divide 256 the last 256 % G rows belong to no head.
    const int gh = R / QT;
    const int iq = R - gh * QT;
    const bool rvalid = iq < tile_q && gh < G;
    const int qi = q0 + (rvalid ? iq : 0);
    const int lim = rvalid ? (p.causal ? c + qi : L - 1) : -1;  // last visible key
    short8_t qb[KS];
    const int qoff0 = QCH ? R * 8 * QCH + 8 * (h2 ^ ((R >> 1) & (QCH - 1))) : 0;
    auto qoff = [&](int ks) { return (int)opaque((uint32_t)qoff0) ^ (16 * (ks - KQR)); };
    {
        // Q^T as the B operand: lane holds q[t0 + qi][hk*G + g][16ks + 8h2 .. +8].
        const bf16_t *qrow = p.q + ((size_t)(t0 + qi) * Hq + hk * G + min(gh, G - 1)) * D + 8 * h2;
        const short8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const short8_t x = *reinterpret_cast<const short8_t *>(qrow + 16 * ks);
            if (ks < KQR) qb[ks] = rvalid ? x : z;
            else *reinterpret_cast<short8_t *>(qlds + qoff(ks)) = rvalid ? x : z;
        }
    }
    auto q_lds = [&](int ks) { return *reinterpret_cast<const short8_t *>(qlds + qoff(ks)); };
    const int lim4 = lim - 4 * h2;             // masks compare key offsets inside a lane's group of 4
    const int wave_end = wave_max_i(lim + 1);  // keys this wavefront needs
    const int wave_lim_min = wave_min_i(rvalid ? lim : 0x7fffffff);
    const int ntw = min(ntiles, (wave_end + N - 1) / N);  // tiles this wavefront computes

    // Loads (group 0 only): wavefront w fills key rows RWL w .. RWL w + RWL - 1
    // of a tile, inside one 16-row block of a cache page or of k_new / v_new.  Per-lane
    // element offsets inside that row block (the chunk each lane fetches makes
    // the LDS layout swizzled: K chunk c of row j at c ^ (j & SWM), V chunk c
    // at c ^ VSS (j & 3)).
    auto v_swizzle = [](int row) { return ((row & 3) * VSS) & SWM; };
    // Load u of wavefront w covers tile rows RWL w + RPI u + lrow; the three
    // terms occupy disjoint bits, so the swizzle of load u is that of lrow
    // XOR a wave-uniform constant: one base offset per tensor (bytes) plus a
    // uniform row step.
    const int lrow = l / CPR, lpc = l - lrow * CPR;
    const uint32_t lbase_k = 2u * ((lrow * Hkv + hk) * D + 8 * (lpc ^ (lrow & SWM)));
    const uint32_t lbase_v = 2u * ((lrow * Hkv + hk) * D + 8 * (lpc ^ v_swizzle(lrow)));
    // (The load addresses are recomputed at every issue, through opaque, by a
    // few VALU of group 0.)
    const size_t rstride = (size_t)Hkv * D;  // elements per token row
    const size_t ustride = 2 * RPI * rstride;  // bytes between loads u and u+1
    const bf16_t *const kcache = p.k_cache, *const vcache = p.v_cache;
    const bf16_t *const knew = p.k_new + (size_t)t0 * rstride, *const vnew = p.v_new + (size_t)t0 * rstride;
    auto issue_tile = [&](int tile, auto s) {
        bf16_t *kd = kst(s) + RWL * w * D, *vd = vst(s) + RWL * w * D;
        const uint32_t bk = opaque(lbase_k), bv = opaque(lbase_v);
        auto lofs_k = [&](int u) { return bk ^ (16u * ((RWL * w + RPI * u) & SWM)); };
        auto lofs_v = [&](int u) { return bv ^ (16u * (uint32_t)v_swizzle(RWL * w + RPI * u)); };
        const int jw = tile * N + RWL * w;  // first key row of this wavefront
        if (jw + RWL - 1 < kv_end && (jw + RWL - 1 < c || jw >= c)) {
            // All RWL rows are visible and come from one tensor: uniform
            // base + 32-bit lane offset.
            const char *kb, *vb;
            if (jw < c) {
                const size_t page = (size_t)ld_meta(p.page_table, prow + jw / p.S);
                const size_t row0 = page * p.S + jw % p.S;  // 16 | S: the RWL rows share a page
                kb = (const char *)(kcache + row0 * rstride);
                vb = (const char *)(vcache + row0 * rstride);
            } else {
                kb = (const char *)(knew + (size_t)(jw - c) * rstride);
                vb = (const char *)(vnew + (size_t)(jw - c) * rstride);
            }
#pragma unroll
            for (int u = 0; u < IPL; ++u) {
                load_lds16((const bf16_t *)(kb + u * ustride + lofs_k(u)), kd + RPI * u * D);
                load_lds16((const bf16_t *)(vb + u * ustride + lofs_v(u)), vd + RPI * u * D);
            }
        } else {
            // The rows hold the cache / new-token boundary or the last
            // visible key: per-lane sources; rows past the end repeat the
            // last visible key (finite, and masked).
            const int jp = min(jw, kv_end - 1);
            const size_t page = (size_t)ld_meta(p.page_table, prow + jp / p.S);
#pragma unroll
            for (int u = 0; u < IPL; ++u) {
                const int lr = (int)opaque(lrow);
                const int kr = RPI * u + lr;
                const int j = min(jw + kr, kv_end - 1);
                const uint32_t d_k = lofs_k(u) - 2u * lr * Hkv * D, d_v = lofs_v(u) - 2u * lr * Hkv * D;
                const size_t crow = (page * p.S + j % p.S) * rstride;
                const size_t nrow = (size_t)(j - c) * rstride;
                const bool cached = j < c;
                const char *kr_ = (const char *)(cached ? kcache + crow : knew + nrow);
                const char *vr_ = (const char *)(cached ? vcache + crow : vnew + nrow);
                load_lds16((const bf16_t *)(kr_ + d_k), kd + RPI * u * D);
                load_lds16((const bf16_t *)(vr_ + d_v), vd + RPI * u * D);
            }
        }
    };

    // Per-lane LDS offsets (elements) of the MFMA-layout reads: K row n32
    // (+ 32 kb), dim chunk 2 ks + h2; V^T rows 4 h2 + (l & 15) / 4 (+ 16 s16,
    // + 8 for the upper 4 keys), dims 32 md + 16 (n32 / 16) + 4 (l & 3) .. +4.
    // The swizzles only flip offset bits that the k-step (16 ks elements) and
    // the dim block (32 md) occupy, so every offset is the first one XOR a
    // constant: one register each instead of one per k-step / dim block.
    const int koff0 = n32 * D + 8 * (h2 ^ (n32 & SWM));
    const int voff0 = [&] {
        const int vr0 = 4 * h2 + ((l & 15) >> 2);
        const int col = 16 * (n32 >> 4) + 4 * (l & 3);
        return vr0 * D + 8 * ((col >> 3) ^ v_swizzle(vr0)) + (col & 7);
    }();
    // At head_dim 256 the XORs are redone at every read (one VALU each):
    // kept live across the loop, the 24 offsets would push Q out of registers.
    auto koff = [&](int ks) {
        if constexpr (D > 128) return (int)opaque((uint32_t)koff0) ^ (16 * ks);
        else return koff0 ^ (16 * ks);
    };
    auto voff = [&](int md) {
        if constexpr (D > 128) return (int)opaque((uint32_t)voff0) ^ (32 * md);
        else return voff0 ^ (32 * md);
    };
    const float16_t zero16 = {};
    const float sl2 = p.scale_log2;

    float16_t o[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) o[md] = zero16;
    float m_run = -INFINITY, l_run = 0.f;
    float16_t sbuf[2][KB];  // S of tiles t (t & 1) and t-1
    short8_t pb[N / 16];    // P^T of tile t-1 as bf16 B operands

    // Element e of a lane's scores is s[e / 16][e % 16], key
    // 32 (e / 16) + 8 ((e % 16) / 4) + 4 h2 + e % 4 of the tile.
    auto key_of = [](int e) { return 32 * (e / 16) + 8 * ((e % 16) >> 2) + (e & 3); };
    auto masked_tile = [&](int tile) { return tile * N + N - 1 > wave_lim_min; };
    auto rescale = [&](float mx) {
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyLog2)) {
            const float mn = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - mn);
            l_run *= alpha;
#pragma unroll
            for (int md = 0; md < MD; ++md) o[md] *= alpha;
            m_run = mn;
        }
    };
    auto cross_half_max = [&](float mx) { return fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2; };

    // ---- phase pieces
    // S(t) = K(t) . Q^T alone (first tile of a wavefront).
    auto qk_only = [&](auto sk, float16_t (&s)[KB]) {
        const bf16_t *Ks = kst(sk);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const short8_t a = *reinterpret_cast<const short8_t *>(Ks + 32 * kb * D + koff(ks));
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ks < KQR ? qb[ks] : q_lds(ks), ks ? s[kb] : zero16, 0, 0, 0);
            }
    };
    // Exponentials of a tile's scores alone (last tile of a wavefront).
    auto exp_only = [&](const float16_t (&s)[KB]) {
        const float nref = -m_run;
        float lsum = 0.f;
#pragma unroll
        for (int s16 = 0; s16 < N / 16; ++s16) {
            uint32_t w4[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int e = 8 * s16 + 2 * e2;
                const float a = fast_exp2(fmaf(s[e / 16][e % 16], sl2, nref));
                const float b = fast_exp2(fmaf(s[(e + 1) / 16][(e + 1) % 16], sl2, nref));
                w4[e2] = cvt_pk_bf16(a, b);
                lsum = pair_sum_bf16(w4[e2], lsum);  // the row sum of the rounded P
            }
            pb[s16] = __builtin_bit_cast(short8_t, w4);
        }
        l_run += lsum;
    };
    // O += V . P over one tile alone.
    auto pv_only = [&](auto sv) {
        const bf16_t *Vs = vst(sv);
#pragma unroll
        for (int s16 = 0; s16 < N / 16; ++s16)
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const bf16_t *v = Vs + 16 * s16 * D + voff(md);
                const short4_t lo = lds_read_tr16(v);
                const short4_t hi = lds_read_tr16(v + 8 * D);
                const short8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s16], o[md], 0, 0, 0);
            }
    };
    // Row max of S(t) alone, masking keys past each row's last one if MASKED.
    auto max_only = [&](auto masked, int t, float16_t (&s)[KB]) {
        float mx = -INFINITY;
        const int thr = lim4 - t * N;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            float v = s[e / 16][e % 16];
            if constexpr (decltype(masked)::value) {
                v = key_of(e) > thr ? -INFINITY : v;
                s[e / 16][e % 16] = v;
            }
            mx = fmaxf(mx, v);
        }
        return cross_half_max(mx);
    };
    // A(t): exponentials of S(t-1) (VALU) interleaved with the MFMAs of S(t),
    // one chunk per k-step (EP / KS pairs each: 2 at head_dim 128, one every
    // other k-step at 256); the compiler may reorder only inside a chunk.
    auto a_full = [&](auto sk, float16_t (&sn)[KB], const float16_t (&so)[KB]) {
        const bf16_t *Ks = kst(sk);
        const float nref = -m_run;
        float lsum = 0.f;
        uint32_t pk[NE / 2];
        // K operands (and the Q^T operands held in LDS) KPF k-steps ahead.
        short8_t ka[KPF + 1][KB], qa[KPF + 1];
        auto read_k = [&](int ks, short8_t (&dst)[KB], short8_t &qdst) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) dst[kb] = *reinterpret_cast<const short8_t *>(Ks + 32 * kb * D + koff(ks));
            if (ks >= KQR) qdst = q_lds(ks);
        };
#pragma unroll
        for (int ks = 0; ks < KPF; ++ks) read_k(ks, ka[ks], qa[ks]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + KPF < KS) read_k(ks + KPF, ka[(ks + KPF) % (KPF + 1)], qa[(ks + KPF) % (KPF + 1)]);
            const short8_t qop = ks < KQR ? qb[ks] : qa[ks % (KPF + 1)];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % (KPF + 1)][kb], qop, ks ? sn[kb] : zero16, 0, 0, 0);
#pragma unroll
            for (int x = ks * EP / KS; x < (ks + 1) * EP / KS; ++x) {
                const int e = 2 * x;
                const float a = fast_exp2(fmaf(so[e / 16][e % 16], sl2, nref));
                const float b = fast_exp2(fmaf(so[(e + 1) / 16][(e + 1) % 16], sl2, nref));
                pk[e / 2] = cvt_pk_bf16(a, b);
                lsum = pair_sum_bf16(pk[e / 2], lsum);  // the row sum of the rounded P
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run += lsum;
#pragma unroll
        for (int s16 = 0; s16 < N / 16; ++s16) {
            const uint32_t w4[4] = {pk[4 * s16], pk[4 * s16 + 1], pk[4 * s16 + 2], pk[4 * s16 + 3]};
            pb[s16] = __builtin_bit_cast(short8_t, w4);
        }
    };
    // B(t): O += V(t-1) . P(t-1) (MFMA) interleaved with the row max of S(t),
    // one chunk per (16-key step, 32-dim block).
    auto b_full = [&](auto masked, int t, auto sv, float16_t (&sn)[KB]) {
        const bf16_t *Vs = vst(sv);
        const int thr = lim4 - t * N;
        float mx = -INFINITY;
        // V^T operands VPF chunks ahead (LDS latency exceeds one MFMA).
        short8_t va[VPF + 1];
        auto read_v = [&](int j) {
            const bf16_t *v = Vs + 16 * (j / MD) * D + voff(j % MD);
            const short4_t lo = lds_read_tr16(v);
            const short4_t hi = lds_read_tr16(v + 8 * D);
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
#pragma unroll
        for (int j = 0; j < VPF; ++j) va[j] = read_v(j);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int s16 = j / MD, md = j % MD;
            if (j + VPF < NB) va[(j + VPF) % (VPF + 1)] = read_v(j + VPF);
            o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j % (VPF + 1)], pb[s16], o[md], 0, 0, 0);
#pragma unroll
            for (int x = 0; x < EB; ++x) {
                const int e = j * EB + x;
                float v = sn[e / 16][e % 16];
                if constexpr (decltype(masked)::value) {
                    v = key_of(e) > thr ? -INFINITY : v;
                    sn[e / 16][e % 16] = v;
                }
                mx = fmaxf(mx, v);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        return cross_half_max(mx);
    };

    // ---- phases of tile t, t % 4 == U (stage constants)
    const int T = ntiles;
    auto phase_a = [&](auto U, int t) {
        constexpr int u = decltype(U)::value;
        float16_t(&sn)[KB] = sbuf[u & 1];
        float16_t(&so)[KB] = sbuf[(u + 1) & 1];
        const bool has_exp = t >= 1 && t <= ntw, has_qk = t < ntw;
        if (has_exp && has_qk) {
            a_full(ic<u>(), sn, so);
        } else {
            if (has_exp) exp_only(so);
            if (has_qk) qk_only(ic<u>(), sn);
        }
    };
    auto phase_b = [&](auto U, int t) {
        constexpr int u = decltype(U)::value;
        float16_t(&sn)[KB] = sbuf[u & 1];
        // Every B phase of group 0 issues one tile (past the last tile it
        // reloads the last one into a stage nobody reads), so the wait below
        // is the same everywhere.
        if (grp == 0) issue_tile(min(t + 2, T - 1), ic<(u + 2) & 3>());
        const bool has_pv = t >= 1 && t <= ntw, has_max = t < ntw;
        if (has_pv && has_max) {
            const float mx = masked_tile(t) ? b_full(std::true_type(), t, ic<(u + 3) & 3>(), sn)
                                            : b_full(std::false_type(), t, ic<(u + 3) & 3>(), sn);
            rescale(mx);
        } else {
            if (has_pv) pv_only(ic<(u + 3) & 3>());
            if (has_max) {
                const float mx = masked_tile(t) ? max_only(std::true_type(), t, sn)
                                                : max_only(std::false_type(), t, sn);
                rescale(mx);
            }
        }
        // Tile t+1 must be in LDS; tile t+2 may stay in flight.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * IPL));
    };

    // Workgroup barrier for the phases.  Each wavefront has consumed its LDS
    // reads before it arrives, and group 0 has waited for the loads the next
    // phase reads, so no fence is needed; the memory clobber keeps the
    // compiler from moving LDS accesses across it.  (A fence here would also
    // wait for the loads still in flight.)
    auto barrier = [] { asm volatile("s_barrier" ::: "memory"); };

    // Prologue: tiles 0 and 1 in flight with the Q and new K/V loads; all
    // of them waited for, then the cache rows stored.
    if (grp == 0) {
        issue_tile(0, ic<0>());
        issue_tile(min(1, T - 1), ic<1>());
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
#pragma unroll
    for (int i = 0; i < KVU; ++i) {
        const int idx = tid + i * NTHR;
        if (idx < kv_chunks) {
            const int col = idx % CPR;
            const size_t dst = ((size_t)kvslot[i] * Hkv + hk) * D + 8 * col;
            *reinterpret_cast<short8_t *>(p.k_cache + dst) = kvk[i];
            *reinterpret_cast<short8_t *>(p.v_cache + dst) = kvv[i];
        }
    }
    for (int idx = tid + KVU * NTHR; idx < kv_chunks; idx += NTHR) {
        const int row = idx / CPR, col = idx - row * CPR;
        const int t = t0 + q0 + row;
        const size_t dst = ((size_t)p.slot_mapping[t] * Hkv + hk) * D + 8 * col;
        const size_t src = ((size_t)t * Hkv + hk) * D + 8 * col;
        *reinterpret_cast<uint4 *>(p.k_cache + dst) = *reinterpret_cast<const uint4 *>(p.k_new + src);
        *reinterpret_cast<uint4 *>(p.v_cache + dst) = *reinterpret_cast<const uint4 *>(p.v_new + src);
    }
    // The loads above were waited for by every wavefront; the cache stores
    // need not complete before the loop (a fence here would wait for them).
    barrier();
    if (grp == 1) barrier();     // group 1 starts one phase late

    auto step = [&](auto U, int t) {
        phase_a(U, t);
        barrier();
        phase_b(U, t);
        barrier();
    };
    for (int tb = 0; tb <= T; tb += 4) {
        step(ic<0>(), tb);
        if (tb + 1 > T) break;
        step(ic<1>(), tb + 1);
        if (tb + 2 > T) break;
        step(ic<2>(), tb + 2);
        if (tb + 3 > T) break;
        step(ic<3>(), tb + 3);
    }
    if (grp == 0) barrier();  // matches group 1's extra barrier
    // No direct-to-LDS load may still be writing when the workgroup retires.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (rvalid) {
        const float inv = 1.f / l_tot;
        bf16_t *orow = p.out + ((size_t)(t0 + qi) * Hq + hk * G + gh) * D;
#pragma unroll
        for (int md = 0; md < MD; ++md) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint2 v;
                v.x = cvt_pk_bf16(o[md][4 * q4] * inv, o[md][4 * q4 + 1] * inv);
                v.y = cvt_pk_bf16(o[md][4 * q4 + 2] * inv, o[md][4 * q4 + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + 32 * md + 8 * q4 + 4 * h2) = v;
            }
        }
    }
}

template <int D>
hipError_t launch_prefill_d(const Params &p, const Plan &plan, const int4 *items, bool self_plan,
                            hipStream_t stream) {
    hipLaunchKernelGGL(prefill_pp_kernel<D>, dim3(plan.n_prefill_items), dim3(PingPongCfg<D>::NTHR), 0, stream,
                       p, items, self_plan ? 1 : 0, plan.q_tile);
    return hipGetLastError();
}

}  // namespace

bool prefill_supports(int D, int G) { return (D == 64 || D == 128 || D == 256) && G >= 1 && G <= 16; }

int prefill_rows(int D) {
    switch (D) {
        case 64: return PingPongCfg<64>::ROWS;
        case 128: return PingPongCfg<128>::ROWS;
        case 256: return PingPongCfg<256>::ROWS;
        default: return 0;
    }
}

hipError_t launch_prefill(const Params &p, const Plan &plan, const int4 *items, bool self_plan,
                          hipStream_t stream) {
    switch (p.D) {
        case 64: return launch_prefill_d<64>(p, plan, items, self_plan, stream);
        case 128: return launch_prefill_d<128>(p, plan, items, self_plan, stream);
        case 256: return launch_prefill_d<256>(p, plan, items, self_plan, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ra
