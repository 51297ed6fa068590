// prefill.hip -- the MFMA-bound kernel for prefill chunks (requests with more
// than one new token), with the KV-cache update fused in (prefill_pp_kernel,
// head_dim 64, 128 and 256).
//
// Work item: (request r, kv head hk, query tile of QT = floor(256/G)
// tokens), read from the plan kernel's item list or, for batches of at most
// kSelfPlanPrefillReqs requests, found by the kernel itself
// (self_plan_prefill_item).  A workgroup of 8 wavefronts runs one item at a
// time (one per workgroup, or a list of them per workgroup: see the kernel).
// The item's 256 query rows are the G query heads of the group times the
// tile's tokens (row R: head R / QT, token R % QT; the last 256 - G QT rows
// are idle), so one K/V tile in LDS serves every head that reads it
// (grouped-query attention); wavefront w owns rows 32 w .. 32 w + 31.
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
//                               (its last four k-steps in LDS at head_dim 256;
//                               up to 128 the rows come in through LDS);
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
// The workgroup copies the new K/V rows of its item's tokens into the cache
// (each (token, kv head) row is written exactly once), and writes the output
// rows through LDS up to head_dim 128 so that every store covers whole rows.
#include <stdlib.h>

#include <algorithm>
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

// Rows that see fewer than this many keys have weights of order one; their
// PV products take P as a bf16 hi + lo pair.
constexpr int kFewKeys = 64;

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

// Every workgroup runs a list of items: item_at(i) for i = 0, 1, ... while
// below the item count (counts[2] when the plan kernel counted them on the
// device, else n_items).  With one workgroup per compute unit the rounds go
// out in a snake order (round i from the first workgroup up when i is even,
// from the last one down when odd), which keeps the sum of item lengths per
// workgroup even when the items come longest first, or in request order when
// every request has the same shape; a grid of one workgroup per
// item (rounds = 1) leaves the balancing to the hardware's dispatch.
// self_plan: 0 items from the list, 1 found by the kernel longest first,
// 2 | rg << 8 in closed form for prefill-only batches of one chunk shape:
// requests in groups of rg, each group longest first (rg = 1: request order).
// While one item's key tiles run, the workgroup reads its next item;
// between two items it issues the next item's first loads (Q rows, first two
// key tiles) right behind the current item's output stores.
//
// LOOP: the workgroup loops over items (one workgroup per compute unit, head
// dim up to 128).  Without it the kernel takes one item per workgroup (head
// dim 256, where the loop's extra live state would push a Q operand out of
// registers, and mixed batches, whose prefill items spread over the units the
// decode kernel frees); it then copies the new K/V rows through registers in
// its start instead of through LDS in its last phase.
template <int D, bool LOOP>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(Params p, const int4 *__restrict__ items, int self_plan,
                                                            int q_tile, const int32_t *__restrict__ counts,
                                                            int n_items) {
    using C = PingPongCfg<D>;
    constexpr int ROWS = C::ROWS, N = C::N, KB = C::KB, KS = C::KS, MD = C::MD, CPR = C::CPR,
                  SWM = C::SWM, VSS = C::VSS, TILE = C::TILE, RWL = C::RWL, RPI = C::RPI, IPL = C::IPL,
                  NE = C::NE, EP = C::EP, NB = C::NB, EB = C::EB, KPF = C::KPF, VPF = C::VPF, KQR = C::KQR,
                  QCH = C::QCH;
    // One array per stage and tensor (see above).
    // (1 KiB aligned, so that the bank pattern of every swizzle holds
    // whatever else the kernel keeps in LDS.)
    __shared__ __attribute__((aligned(1024))) bf16_t k0[TILE], k1[TILE], k2[TILE], k3[TILE];
    __shared__ __attribute__((aligned(1024))) bf16_t v0[TILE], v1[TILE], v2[TILE], v3[TILE];
    // Q^T k-steps KQR .. KS-1: row R's chunk c at c ^ ((R >> 1) & (QCH - 1)),
    // so the 16 rows a 16-lane group reads hit 16 different bank groups.
    // Every lane reads back only what it wrote itself.
    __shared__ __attribute__((aligned(16))) bf16_t qlds[QCH ? ROWS * 8 * QCH : 8];
    // Up to head_dim 128 (where LDS has room) a self-planning kernel finds
    // the items of its first kRounds rounds once, at its start (wavefront w
    // those of rounds w, w + 8, ...), from copies of cu_q_lens and
    // context_lens of its at most 64 requests, and keeps them here (8 ints
    // a round); later rounds search at the item's start.
    constexpr bool LMETA = LOOP && D <= 128;
    constexpr int NMETA = 2 * kSelfPlanPrefillReqs + 1, kRounds = 64;
    __shared__ int32_t lmeta[LMETA ? NMETA : 1];
    __shared__ int32_t lround[LMETA ? 8 * kRounds : 1];
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

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar wavefront index
    const int grp = w >> 2;
    const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv, QT = ROWS / G;
    const size_t rstride = (size_t)Hkv * D;  // elements per token row

    // A value the compiler must recompute from here at each use instead of
    // keeping derived values live across the loop, where registers are short.
    auto opaque = [](uint32_t x) {
        asm volatile("" : "+v"(x));
        return x;
    };

    // ---- the item list
    const int n = counts ? ld_meta(counts, 2) : n_items;
    const int nb = gridDim.x, b = blockIdx.x;
    auto item_at = [&](int i) { return (i & 1) ? (i + 1) * nb - 1 - b : i * nb + b; };
    auto fetch = [&](int k, int4 &it, int4 &it2) {
        if ((self_plan & 0xff) == 2) {
            // Every request a prefill chunk of the same length q and context
            // c: requests in groups of rg (self_plan >> 8), each group's items
            // longest first (a request's last query tile first, then request,
            // then kv head), in closed form.  With rg = 1 this is request
            // order, the plan kernel's; the items that run together read the
            // K/V of a few requests and share L2.
            const int rg = max(1, self_plan >> 8);
            int qr, cx;
            if constexpr (LMETA) {
                qr = __builtin_amdgcn_readfirstlane(lmeta[1] - lmeta[0]);
                cx = __builtin_amdgcn_readfirstlane(lmeta[kSelfPlanPrefillReqs + 1]);
            } else {
                qr = ld_meta(p.cu_q_lens, 1) - ld_meta(p.cu_q_lens, 0);
                cx = ld_meta(p.context_lens, 0);
            }
            const int ntiles = (qr + q_tile - 1) / q_tile, per = ntiles * p.Hkv;
            const int g = k / (rg * per), kk = k - g * rg * per;
            const int gs = min(rg, p.R - g * rg);  // requests in group g
            const int rank = kk / max(1, gs * p.Hkv), rem = kk - rank * gs * p.Hkv;
            const int r = g * rg + rem / p.Hkv, hk = rem % p.Hkv;
            if (gs < 1 || r >= p.R || qr <= 1) {
                it = make_int4(-1, 0, 0, 0);
                it2 = make_int4(0, 0, 0, 0);
            } else {
                it = make_int4(r, hk, (ntiles - 1 - rank) * q_tile, r * qr);
                it2 = make_int4(cx, qr, 0, 0);
            }
        } else if (self_plan) {
            if constexpr (LMETA) {
                const lds_i32_ptr lm = (lds_i32_ptr)lmeta;
                self_plan_prefill_item_lds(p, k, q_tile, N, it, it2, lm, lm + kSelfPlanPrefillReqs + 1);
            } else {
                self_plan_prefill_item(p, k, q_tile, N, it, it2);
            }
        } else {
            const int32_t *li = reinterpret_cast<const int32_t *>(items) + 8 * (size_t)k;
            it = make_int4(ld_meta(li, 0), ld_meta(li, 1), ld_meta(li, 2), ld_meta(li, 3));
            it2 = make_int4(ld_meta(li, 4), ld_meta(li, 5), 0, 0);
        }
    };
    // Geometry of an item (wave-uniform).
    struct Geo {
        int r, hk, q0, t0, c, qlen, tile_q, kv_end, ntiles;
    };
    auto geo = [&](const int4 &it, const int4 &it2) {
        Geo g;
        g.r = it.x;
        g.hk = it.y;
        g.q0 = it.z;
        g.t0 = it.w;
        g.c = it2.x;
        g.qlen = it2.y;
        g.tile_q = min(QT, g.qlen - g.q0);
        g.kv_end = p.causal ? g.c + g.q0 + g.tile_q : g.c + g.qlen;  // keys 0 .. kv_end-1 are visible to someone
        g.ntiles = (g.kv_end + N - 1) / N;
        return g;
    };

    // Workgroup barrier for the phases.  Each wavefront has consumed its LDS
    // reads before it arrives, and group 0 has waited for the loads the next
    // phase reads, so no fence is needed; the memory clobber keeps the
    // compiler from moving LDS accesses across it.  (A fence here would also
    // wait for the loads still in flight.)
    auto barrier = [] { asm volatile("s_barrier" ::: "memory"); };

    int i_round = 0;
    if (item_at(0) >= n) return;
    const bool listed = LMETA && self_plan;
    if (listed) {
        const int t = threadIdx.x, R = p.R;
        if (t <= R) lmeta[t] = p.cu_q_lens[t];
        if (t < R) lmeta[kSelfPlanPrefillReqs + 1 + t] = p.context_lens[t];
        __syncthreads();
        for (int i = w; i < kRounds && item_at(i) < n; i += 8) {
            int4 a, c;
            fetch(item_at(i), a, c);
            if ((threadIdx.x & 63) == 0) {
                int32_t *d = lround + 8 * i;
                d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w; d[4] = c.x; d[5] = c.y;
            }
        }
        __syncthreads();
    }
    // Item of round i: from the list above, else found now.
    auto fetch_round = [&](int i, int4 &it, int4 &it2) {
        if (listed && i < kRounds) {
            const int32_t *d = lround + 8 * i;
            it = make_int4(__builtin_amdgcn_readfirstlane(d[0]), __builtin_amdgcn_readfirstlane(d[1]),
                           __builtin_amdgcn_readfirstlane(d[2]), __builtin_amdgcn_readfirstlane(d[3]));
            it2 = make_int4(__builtin_amdgcn_readfirstlane(d[4]), __builtin_amdgcn_readfirstlane(d[5]), 0, 0);
        } else {
            fetch(item_at(i), it, it2);
        }
    };
    int4 it, it2;
    fetch_round(0, it, it2);
    for (;;) {
        // Values derived from the lane index are recomputed for every item
        // (from an opaque copy of it): hoisted out of the item loop they
        // would stay live across the key-tile loop and push registers out.
        const int tid = (int)opaque(threadIdx.x);
        const int l = tid & 63, n32 = l & 31, h2 = l >> 5;
        // This lane's query row R = 32 w + n32: head g = R / QT, token i = R % QT.
        // When G does not divide 256 the last 256 % G rows belong to no head.
        const int R = 32 * w + n32;
        const int gh = R / QT;
        const int iq = R - gh * QT;

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
        const uint32_t lbase_k0 = 2u * (lrow * Hkv * D + 8 * (lpc ^ (lrow & SWM)));
        const uint32_t lbase_v0 = 2u * (lrow * Hkv * D + 8 * (lpc ^ v_swizzle(lrow)));
        const size_t ustride = 2 * RPI * rstride;  // bytes between loads u and u+1
        const bf16_t *const kcache = p.k_cache, *const vcache = p.v_cache;
        auto issue_tile = [&](const Geo &g, int tile, auto s) {
            bf16_t *kd = kst(s) + RWL * w * D, *vd = vst(s) + RWL * w * D;
            // (The load addresses are recomputed at every issue, through opaque, by a
            // few VALU of group 0.)
            const uint32_t hoff = 2u * g.hk * D;
            const uint32_t bk = opaque(lbase_k0) + hoff, bv = opaque(lbase_v0) + hoff;
            auto lofs_k = [&](int u) { return bk ^ (16u * ((RWL * w + RPI * u) & SWM)); };
            auto lofs_v = [&](int u) { return bv ^ (16u * (uint32_t)v_swizzle(RWL * w + RPI * u)); };
            const bf16_t *const knew = p.k_new + (size_t)g.t0 * rstride, *const vnew = p.v_new + (size_t)g.t0 * rstride;
            const size_t prow = (size_t)g.r * p.max_pages;
            const int c = g.c, kv_end = g.kv_end;
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

        // Q^T as the B operand: lane holds q[t0 + qi][hk*G + g][16ks + 8h2 .. +8]
        // for k-step ks.  Up to head_dim 128 the rows come in through LDS: the
        // direct-to-LDS loads of an item's Q rows go out at the end of the
        // previous item (or at its own start) into stages 2 and 3, free until
        // the item's phase B(0) loads tile 2 there.  Wavefront w's 32 rows fill
        // its own 64 D-byte area row-major, laid out like a K tile (chunk c of
        // row j at c ^ (j & SWM)), so that one 1 KiB load covers whole rows and
        // the MFMA-layout reads back are free of bank conflicts.  At head_dim
        // 256 (Q rows of 16 KiB per wavefront, twice the free space) they load
        // into registers at the item's start; there the last QKS k-steps then
        // go to LDS.  Rows of no head or token read zeros.
        constexpr bool QSTAGE = D <= 128;
        short8_t qb[KS];
        const int qoff0 = QCH ? R * 8 * QCH + 8 * (h2 ^ ((R >> 1) & (QCH - 1))) : 0;
        auto qoff = [&](int ks) { return (int)opaque((uint32_t)qoff0) ^ (16 * (ks - KQR)); };
        auto valid_row = [&](const Geo &g, int row) {
            const int h = row / QT;
            return row - h * QT < g.tile_q && h < G;
        };
        auto row_valid = [&](const Geo &g) { return iq < g.tile_q && gh < G; };
        // Element offset of row `row` (any of the 256) of the item in q / out.
        auto row_elem = [&](const Geo &g, int row) {
            const int h = row / QT, i = row - h * QT;
            const bool v = i < g.tile_q && h < G;
            return ((size_t)(g.t0 + g.q0 + (v ? i : 0)) * Hq + g.hk * G + min(h, G - 1)) * D;
        };
        auto q_row = [&](const Geo &g) { return p.q + row_elem(g, R) + 8 * h2; };
        // Wavefront w's row area up to head_dim 128 (32 rows x D, row-major,
        // K-tile swizzle): half of stage 2 or 3's K or V array.
        bf16_t *const warea = [&]() -> bf16_t * {
            static_assert(!QSTAGE || 2 * 32 * D == TILE, "two wavefronts' rows fill one stage array");
            bf16_t *a = (w >> 1) == 0 ? k2 : (w >> 1) == 1 ? v2 : (w >> 1) == 2 ? k3 : v3;
            return a + (w & 1) * 32 * D;
        }();
        // Load / store u (u < KS) of the wavefront's rows moves rows RPI u + lrow,
        // lane chunk slot lpc, i.e. row chunk lpc ^ (row & SWM), at element
        // RPI u D + 8 l of the area.
        auto area_chunk = [&](int u) { return lpc ^ ((RPI * u + lrow) & SWM); };
        auto issue_q = [&](const Geo &g) {
            if constexpr (QSTAGE) {
    #pragma unroll
                for (int u = 0; u < KS; ++u) {
                    const int row = 32 * w + RPI * u + (int)opaque(lrow);
                    load_lds16(p.q + row_elem(g, row) + 8 * area_chunk(u), warea + RPI * u * D);
                }
            }
        };
        // After the item's loads have landed.
        auto take_q = [&](const Geo &g) {
            const bool rvalid = row_valid(g);
            const short8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
            if constexpr (QSTAGE) {
    #pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int off = n32 * D + 8 * ((2 * ks + h2) ^ (n32 & SWM));
                    const short8_t x = *reinterpret_cast<const short8_t *>(warea + off);
                    qb[ks] = rvalid ? x : z;
                }
            } else {
    #pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (!rvalid) qb[ks] = z;
                    if (ks >= KQR) *reinterpret_cast<short8_t *>(qlds + qoff(ks)) = qb[ks];
                }
            }
        };
        auto load_q_regs = [&](const Geo &g) {
            if constexpr (!QSTAGE) {
                const bf16_t *qrow = q_row(g);
    #pragma unroll
                for (int ks = 0; ks < KS; ++ks) qb[ks] = *reinterpret_cast<const short8_t *>(qrow + 16 * ks);
            }
        };
        auto q_lds = [&](int ks) { return *reinterpret_cast<const short8_t *>(qlds + qoff(ks)); };

        // Fused KV-cache update (group 0, in its last phase of an item, which
        // has no other work): the new K/V rows of the item's tokens for kv
        // head hk go global -> LDS through the K arrays of stages T % 4 and
        // (T + 3) % 4 (K rows, V rows), which no wavefront reads any more and
        // no load is still writing (the reloads of the last B phases go to
        // the other two), then LDS -> cache at slot_mapping.  A round moves
        // one array's worth of chunks per tensor (64 tokens at head_dim 128);
        // instruction i of wavefront w covers chunks 256 i + 64 w + lane of
        // the round, and each lane reads back its own chunks.
        auto kst_rt = [&](int st) -> bf16_t * { return st == 0 ? k0 : st == 1 ? k1 : st == 2 ? k2 : k3; };
        auto copy_kv = [&](const Geo &g) {
            constexpr int PER = TILE / 8, NI = PER / 256;  // chunks per array, loads per wavefront
            static_assert(PER % 256 == 0, "whole wavefront loads per array");
            const int chunks = p.skip_scatter ? 0 : g.tile_q * CPR;
            bf16_t *const ka = kst_rt(g.ntiles & 3), *const va = kst_rt((g.ntiles + 3) & 3);
            for (int base = 0; base < chunks; base += PER) {
                int slot[NI];
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int y0 = 256 * i + 64 * w;  // first chunk of this wavefront load
                    if (base + y0 < chunks) {
                        const int x = min(base + y0 + l, chunks - 1);
                        const int row = x / CPR, col = x - row * CPR;
                        const int t = g.t0 + g.q0 + row;
                        const size_t src = ((size_t)t * Hkv + g.hk) * D + 8 * col;
                        slot[i] = p.slot_mapping[t];
                        load_lds16(p.k_new + src, ka + 8 * y0);
                        load_lds16(p.v_new + src, va + 8 * y0);
                    }
                }
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int y0 = 256 * i + 64 * w;
                    const int x = base + y0 + l;
                    if (base + y0 < chunks && x < chunks) {
                        const int col = x % CPR;
                        const size_t d = ((size_t)slot[i] * Hkv + g.hk) * D + 8 * col;
                        *reinterpret_cast<short8_t *>(p.k_cache + d) =
                            *reinterpret_cast<const short8_t *>(ka + 8 * (y0 + l));
                        *reinterpret_cast<short8_t *>(p.v_cache + d) =
                            *reinterpret_cast<const short8_t *>(va + 8 * (y0 + l));
                    }
                }
            }
        };

        // Without the item loop the new K/V rows go through registers: two
        // 16-byte chunks per thread and tensor (tile_q CPR <= 1024 chunks),
        // loaded with the item's first loads and stored once they have landed;
        // larger tiles copy the rest there too.
        constexpr int KVU = LOOP ? 1 : 2;
        short8_t kvk[KVU], kvv[KVU];
        int kvslot[KVU];
        auto load_kv = [&](const Geo &g) {
            const int kv_chunks = p.skip_scatter ? 0 : g.tile_q * CPR;
#pragma unroll
            for (int i = 0; i < KVU; ++i) {
                const int idx = tid + i * 512;
                if (idx < kv_chunks) {
                    const int row = idx / CPR, col = idx - row * CPR;
                    const int t = g.t0 + g.q0 + row;
                    const size_t src = ((size_t)t * Hkv + g.hk) * D + 8 * col;
                    kvslot[i] = p.slot_mapping[t];
                    kvk[i] = *reinterpret_cast<const short8_t *>(p.k_new + src);
                    kvv[i] = *reinterpret_cast<const short8_t *>(p.v_new + src);
                }
            }
        };
        auto store_kv = [&](const Geo &g) {
            const int kv_chunks = p.skip_scatter ? 0 : g.tile_q * CPR;
#pragma unroll
            for (int i = 0; i < KVU; ++i) {
                const int idx = tid + i * 512;
                if (idx < kv_chunks) {
                    const size_t d = ((size_t)kvslot[i] * Hkv + g.hk) * D + 8 * (idx % CPR);
                    *reinterpret_cast<short8_t *>(p.k_cache + d) = kvk[i];
                    *reinterpret_cast<short8_t *>(p.v_cache + d) = kvv[i];
                }
            }
            for (int idx = tid + KVU * 512; idx < kv_chunks; idx += 512) {
                const int row = idx / CPR, col = idx - row * CPR;
                const int t = g.t0 + g.q0 + row;
                const size_t d = ((size_t)p.slot_mapping[t] * Hkv + g.hk) * D + 8 * col;
                const size_t src = ((size_t)t * Hkv + g.hk) * D + 8 * col;
                *reinterpret_cast<uint4 *>(p.k_cache + d) = *reinterpret_cast<const uint4 *>(p.k_new + src);
                *reinterpret_cast<uint4 *>(p.v_cache + d) = *reinterpret_cast<const uint4 *>(p.v_new + src);
            }
        };

        // What an item needs first, issued at the end of the previous item (or
        // before the first): its first two key tiles (group 0) and its Q rows
        // (up to head_dim 128).
        auto issue_start = [&](const Geo &g) {
            if (g.r < 0) return;
            if (grp == 0) {
                issue_tile(g, 0, ic<0>());
                if (g.ntiles > 1) issue_tile(g, 1, ic<1>());
            }
            issue_q(g);
            if constexpr (!LOOP) load_kv(g);
        };

        const Geo g = geo(it, it2);
        if (i_round == 0) issue_start(g);
        // At head_dim 256 the Q rows load into registers here, behind the
        // item's first tiles.
        if (g.r >= 0) load_q_regs(g);
        // The next item, read (or found) while this one's loads are in flight.
        const bool more = item_at(i_round + 1) < n;
        int4 nit = make_int4(-1, 0, 0, 0), nit2 = make_int4(0, 0, 0, 0);
        if (LOOP && more) fetch_round(i_round + 1, nit, nit2);
        if (g.r >= 0) {
            const int c = g.c, q0 = g.q0, t0 = g.t0, hk = g.hk;
            const int L = c + g.qlen;
            const int ntiles = g.ntiles;
            const bool rvalid = row_valid(g);
            const int qi = q0 + (rvalid ? iq : 0);
            const int lim = rvalid ? (p.causal ? c + qi : L - 1) : -1;  // last visible key
            const int lim4 = lim - 4 * h2;             // masks compare key offsets inside a lane's group of 4
            const int wave_end = wave_max_i(lim + 1);  // keys this wavefront needs
            const int wave_lim_min = wave_min_i(rvalid ? lim : 0x7fffffff);
            const int ntw = min(ntiles, (wave_end + N - 1) / N);  // tiles this wavefront computes

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
            const bool few_rows = wave_lim_min < kFewKeys - 1;
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
            // O += V . P over one tile alone (P^T given as bf16 B operands).
            auto pv_with = [&](auto sv, const short8_t (&pp)[N / 16]) {
                const bf16_t *Vs = vst(sv);
#pragma unroll
                for (int s16 = 0; s16 < N / 16; ++s16)
#pragma unroll
                    for (int md = 0; md < MD; ++md) {
                        const bf16_t *v = Vs + 16 * s16 * D + voff(md);
                        const short4_t lo = lds_read_tr16(v);
                        const short4_t hi = lds_read_tr16(v + 8 * D);
                        const short8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pp[s16], o[md], 0, 0, 0);
                    }
            };
            auto pv_only = [&](auto sv) { pv_with(sv, pb); };
            // Exponentials of a masked tile (one that crosses some row's last key)
            // of a wavefront with rows that see fewer than kFewKeys keys, as a bf16
            // hi + lo pair: hi goes to pb for the PV product of the next phase, and
            // O += V . lo right here, so the weights keep ~16 bits.  With one bf16
            // P, a row that sees a handful of keys has weights of order one, and
            // their relative rounding (2^-9 each) plus the output's own rounding can
            // exceed 1e-2 on values of a few units; rows that see more keys have
            // small weights whose rounding errors average out.  The rescale that
            // follows the next row max applies to both halves alike.
            auto exp_lo_pv = [&](const float16_t (&s)[KB], auto sv) {
                const float nref = -m_run;
                float lsum = 0.f;
                short8_t plo[N / 16];
#pragma unroll
                for (int s16 = 0; s16 < N / 16; ++s16) {
                    uint32_t w4[4], l4[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const int e = 8 * s16 + 2 * e2;
                        const float a = fast_exp2(fmaf(s[e / 16][e % 16], sl2, nref));
                        const float b = fast_exp2(fmaf(s[(e + 1) / 16][(e + 1) % 16], sl2, nref));
                        w4[e2] = cvt_pk_bf16(a, b);
                        l4[e2] = cvt_pk_bf16(a - bf16_lo(w4[e2]), b - bf16_hi(w4[e2]));
                        lsum = pair_sum_bf16(w4[e2], lsum);
                        lsum = pair_sum_bf16(l4[e2], lsum);
                    }
                    pb[s16] = __builtin_bit_cast(short8_t, w4);
                    plo[s16] = __builtin_bit_cast(short8_t, l4);
                }
                l_run += lsum;
                pv_with(sv, plo);
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
                // A masked tile t-1 of a wavefront with few-key rows takes the hi +
                // lo path (its V is still in LDS: stage (t-1) % 4 is reloaded only
                // at B(t+1)), without interleaving.
                const bool lo = has_exp && few_rows && masked_tile(t - 1);
                if (has_exp && has_qk && !lo) {
                    a_full(ic<u>(), sn, so);
                } else {
                    if (has_exp) {
                        if (lo) exp_lo_pv(so, ic<(u + 3) & 3>());
                        else exp_only(so);
                    }
                    if (has_qk) qk_only(ic<u>(), sn);
                }
            };
            auto phase_b = [&](auto U, int t) {
                constexpr int u = decltype(U)::value;
                float16_t(&sn)[KB] = sbuf[u & 1];
                // Every B phase of group 0 issues one tile (past the last tile it
                // reloads the last one into a stage nobody reads), so the wait below
                // is the same everywhere.  (Skipping those reloads, with the wait
                // made conditional to match, made every B phase ~150 cycles slower.)
                if (grp == 0) issue_tile(g, min(t + 2, T - 1), ic<(u + 2) & 3>());
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

            // Start: the tiles and Q rows have landed; Q goes to registers (every
            // wavefront has read its staging area before the first barrier, so
            // tile 2 may reuse it from B(0) on).
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            take_q(g);
            if constexpr (!LOOP) store_kv(g);
            barrier();
            if (grp == 1) barrier();  // group 1 starts one phase late

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
            if (grp == 0) {
                if constexpr (LOOP) copy_kv(g);
                // The reloads of the last B phases have landed before anyone
                // writes LDS again (the output and the next item's loads).
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                barrier();  // matches group 1's extra barrier
            }

            // Output, 1 / l applied and rounded to bf16.  Up to head_dim 128 each
            // lane's row goes to the wavefront's row area first, then whole rows
            // go out, 16 bytes per lane (the accumulator layout holds 8 bytes of a
            // row per lane and 32-dim block: stored directly, every store touches
            // 32 rows).  At head_dim 256 the rows go out directly (staged there,
            // the extra live state pushed a Q operand out of registers in the
            // key-tile loop).
            const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
            const float inv = rvalid ? 1.f / l_tot : 0.f;
            if constexpr (QSTAGE) {
#pragma unroll
                for (int md = 0; md < MD; ++md) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        uint2 v;
                        v.x = cvt_pk_bf16(o[md][4 * q4] * inv, o[md][4 * q4 + 1] * inv);
                        v.y = cvt_pk_bf16(o[md][4 * q4 + 2] * inv, o[md][4 * q4 + 3] * inv);
                        const int off = n32 * D + 8 * ((4 * md + q4) ^ (n32 & SWM)) + 4 * h2;
                        *reinterpret_cast<uint2 *>(warea + off) = v;
                    }
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wavefront's own LDS writes are done
#pragma unroll
                for (int u = 0; u < KS; ++u) {
                    const int row = 32 * w + RPI * u + lrow;
                    if (valid_row(g, row)) {
                        const short8_t x = *reinterpret_cast<const short8_t *>(warea + RPI * u * D + 8 * l);
                        *reinterpret_cast<short8_t *>(p.out + row_elem(g, row) + 8 * area_chunk(u)) = x;
                    }
                }
            } else if (rvalid) {
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
        if (!LOOP || !more) break;
        // Every LDS read of this item is done and its output stores are out:
        // the next item's first loads go out behind them.
        issue_start(geo(nit, nit2));
        it = nit;
        it2 = nit2;
        ++i_round;
    }
    // No direct-to-LDS load may still be writing when the workgroup retires
    // (every tile load was waited for in the phases; this covers a workgroup
    // whose last item was empty).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

template <int D>
hipError_t launch_prefill_d(const Params &p, const Plan &plan, const int4 *items, bool self_plan,
                            const int32_t *counts, bool spread, hipStream_t stream, hipEvent_t ev_start,
                            hipEvent_t ev_stop) {
    // One workgroup per compute unit (LDS holds one), looping over the items,
    // up to head_dim 128 unless spread; else one workgroup per item (with
    // planning on the device, per bound item: those past the count exit).
    // The loop's items are dealt out in a fixed order, which balances when
    // the list is longest first (self-planned) or every chunk has the same
    // shape; the plan kernel's list of ragged chunks is in request order, and
    // there one workgroup per item, which the hardware starts as compute units
    // free up, balances better (100 x 512-token chunks after 0-8K tokens of
    // context: 4.31 ms looping, 4.14 ms one per workgroup; uniform batches
    // gain 4-27 % from the loop, e.g. 128 x 256 tokens 292 -> 230 us).
    // RA_PREFILL_LOOP=0 / 1 (environment) overrides the choice, for tests.
    const int n = std::max(1, plan.n_prefill_items);
    bool loop = D <= 128 && !spread && (self_plan || plan.bounds || plan.uniform_prefill);
    if (const char *env = getenv("RA_PREFILL_LOOP")) {
        if (env[0] == '0') loop = false;
        else if (env[0] == '1') loop = D <= 128 && !spread;
    }
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // Self-planned item order: longest first (1), or, when every request is a
    // prefill chunk of one length and context, requests in groups of rg, each
    // group longest first (2 | rg << 8): the items that run together then
    // share the K/V of a few requests in L2.  The loop takes rg = 1 (request
    // order; same machine, 64 x 1024 tokens 859 -> 777 us, 32 x 512 155 -> 145
    // us, 64 x 256 after 1024 tokens 407 -> 365 us; 4 x 2048 within 1 %).
    // One item per workgroup needs longest first for the hardware's hand-out
    // of workgroups to balance (head_dim 256, 4 x 2048 in request order: 231
    // against 177 us), so there rg is the requests whose items fill the
    // compute units once, and each group is handed out longest first.
    // RA_PREFILL_ORDER=0 (environment) keeps longest first, for tests.
    const char *order_env = getenv("RA_PREFILL_ORDER");
    const bool uniform_all = plan.uniform_prefill && plan.n_prefill_reqs == p.R && plan.n_decode_reqs == 0 &&
                             p.R > 0 && !(order_env && order_env[0] == '0');
    const int rg = loop ? 1 : std::max(1, cus / std::max(1, plan.n_prefill_items / std::max(1, p.R)));
    const int mode = !self_plan ? 0 : uniform_all ? (2 | (std::min(rg, 1 << 20) << 8)) : 1;
    if (loop) {
        // RA_PREFILL_WGS (environment) caps the looping grid, for tuning and
        // for tests of many rounds per workgroup.
        if (const char *env = getenv("RA_PREFILL_WGS")) {
            const int forced = atoi(env);
            if (forced > 0) cus = std::min(cus, forced);
        }
        e = launch_kernel(prefill_pp_kernel<D, D <= 128>, dim3(std::min(std::max(1, cus), n)),
                          dim3(PingPongCfg<D>::NTHR), 0, stream, ev_start, ev_stop, p, items, mode, plan.q_tile,
                          counts, plan.n_prefill_items);
    } else {
        e = launch_kernel(prefill_pp_kernel<D, false>, dim3(n), dim3(PingPongCfg<D>::NTHR), 0, stream, ev_start,
                          ev_stop, p, items, mode, plan.q_tile, counts, plan.n_prefill_items);
    }
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace

// A workgroup's 256 rows hold floor(256 / G) tokens of each of the G query
// heads, so groups of up to 256 heads fit (larger groups run the generic
// kernel).
bool prefill_supports(int D, int G) { return (D == 64 || D == 128 || D == 256) && G >= 1 && G <= 256; }

int prefill_rows(int D) {
    switch (D) {
        case 64: return PingPongCfg<64>::ROWS;
        case 128: return PingPongCfg<128>::ROWS;
        case 256: return PingPongCfg<256>::ROWS;
        default: return 0;
    }
}

hipError_t launch_prefill(const Params &p, const Plan &plan, const int4 *items, bool self_plan,
                          const int32_t *counts, bool spread, hipStream_t stream, hipEvent_t ev_start,
                          hipEvent_t ev_stop) {
    switch (p.D) {
        case 64: return launch_prefill_d<64>(p, plan, items, self_plan, counts, spread, stream, ev_start, ev_stop);
        case 128: return launch_prefill_d<128>(p, plan, items, self_plan, counts, spread, stream, ev_start, ev_stop);
        case 256: return launch_prefill_d<256>(p, plan, items, self_plan, counts, spread, stream, ev_start, ev_stop);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ra
