// decode.hip -- the HBM-bound decode kernel (requests with one new token).
//
// Work split (stream-K): the pages of all decode requests, in request order,
// form one flat list; a persistent grid of workgroups per group of HW kv
// heads takes equal consecutive ranges of it, so every compute unit streams
// the same number of bytes however ragged the contexts are.  A workgroup
// walks its range request by request ("segments"); a segment that is a whole
// request writes the output, otherwise the workgroup writes a partial
// (m, l, o) to a slot of its own, and a small merge kernel that follows
// combines the partials of each such request by log-sum-exp.  Batches of
// short contexts instead give each workgroup whole requests (an equal share
// of the request list), so nothing is cut and no merge kernel runs.  Up to
// kSelfPlanReqs requests the workgroups find their ranges themselves (a wave
// scan over the requests' page counts); larger batches read the start table
// the plan kernel writes.
//
// One wavefront per kv head; the G = Hq/Hkv query heads of a kv head share
// every K/V byte its wavefront reads (grouped-query attention), so the cache
// is read exactly once when G <= 16.  Larger groups are cut into blocks of 16
// query heads on the grid's third dimension: each block's workgroups stream
// the same pages, at the same time and on the same XCD, so that the blocks
// after the first mostly find them in L2.  Per 16-token page:
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
//     so P never leaves its registers (as a bf16 hi + lo pair, two MFMAs,
//     keeping P to ~16 bits); V^T comes from the row-major V tile
//     through the gfx950 transposing read ds_read_b64_tr_b16 (each 16-lane
//     group points its lanes at 4 rows x 4 column quads, and lane j receives
//     column j of the 4 rows);
//   * the online softmax runs on S^T: per-head max across the 4 lane groups
//     by two cross-lane steps, running sum kept per lane and reduced once;
//     the accumulator is rescaled only when a max grows past a headroom.
// A short prefill chunk (q new tokens with q G <= 32, as in speculative
// verification or the tail of a chunked prefill) runs here too: its Q^T
// columns are the q tokens x G heads (column n: token n / G, head n % G;
// blocks of 16 columns on the grid's third dimension, like head blocks),
// each column with its own causal limit, and its q new K/V rows are read
// from k_new / v_new.  The workgroup that computes a page block holding new
// tokens writes their K/V rows into the cache (the fused update); attention
// reads those keys from k_new/v_new, so no workgroup reads a slot this
// launch writes.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "launch.hpp"
#include "plan.hpp"

namespace ra {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

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
#define RA_DECODE_PF128 2
#endif
#ifndef RA_DECODE_PF256
#define RA_DECODE_PF256 1
#endif

// 1: P enters PV as a bf16 hi + lo pair (two MFMAs); 0: hi only.
#ifndef RA_DECODE_P_LO
#define RA_DECODE_P_LO 1
#endif

// 1: K/V pages are read with non-temporal loads (each byte is read once;
// on this part streaming reads then run ~12% faster); 0: ordinary loads.
#ifndef RA_DECODE_NT
#define RA_DECODE_NT 1
#endif

// NT: non-temporal loads (off where several column slices of the grid read
// the same pages and should find them in L2).
template <bool NT>
__device__ __forceinline__ short8_t stream_load(const bf16_t *src) {
    const short8_t *p = reinterpret_cast<const short8_t *>(src);
    if constexpr (NT && RA_DECODE_NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// Page ids a decode workgroup stages in LDS at a time.
constexpr int kNumPids = 2048;

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

// One request as the decode walk sees it.
struct DecodeReq {
    int i;     // index in the decode request list
    int r;     // request id
    int t0;    // its first new token
    int q;     // new tokens (1, or a short chunk)
    int c;     // context length = position of the first new token
    int pfx;   // first flat page
    int pend;  // one past its last flat page
};

// Metadata the kernel never writes, read through the constant address space:
// with a uniform address the load is a scalar load, so the value lands in an
// SGPR and waiting for it never waits for the K/V vector loads in flight.
__device__ __forceinline__ int ld_meta(const int32_t *a, size_t i) {
    return ((const __attribute__((address_space(4))) int32_t *)a)[i];
}

// Decode request i of the list, whose first flat page is pfx.  Without a
// plan kernel the list is every request of the batch, and those that are
// not decode requests hold no pages (the walks step over them).
__device__ __forceinline__ DecodeReq make_req(const Params &p, const DecodeWork &dw, int i, int pfx) {
    DecodeReq q;
    q.i = i;
    q.r = dw.self_plan ? i : ld_meta(dw.dreq, i);
    q.t0 = ld_meta(p.cu_q_lens, q.r);
    q.q = ld_meta(p.cu_q_lens, q.r + 1) - q.t0;
    q.c = ld_meta(p.context_lens, q.r);
    const bool decode = !dw.self_plan || decode_kind(q.q, p.dq_max);
    q.pfx = pfx;
    q.pend = pfx + (decode ? decode_blocks(q.c, q.q) : 0);
    return q;
}

// The decode request after q.
__device__ __forceinline__ DecodeReq next_req(const Params &p, const DecodeWork &dw, const DecodeReq &q) {
    return make_req(p, dw, q.i + 1, q.pend);
}

// Batches of at most kSelfPlanReqs requests need no plan kernel: every
// wavefront finds the request holding its workgroup's first flat page g0
// itself, from the prefix sums of the requests' block counts (zero for
// requests that are not decode requests; lane l holds requests l, l + 64,
// ...: one round trip of loads, then a wave scan per 64 requests), and
// wavefront 0 of head group 0 writes the first flat page of the decode
// requests that start inside [g0, g1) for the merge kernel.  Returns
// {request, its first flat page}.
__device__ __forceinline__ int2 self_plan_first(const Params &p, const DecodeWork &dw, int g0, int g1,
                                                bool write_list) {
    constexpr int KR = kSelfPlanReqs / 64;
    const int lane = threadIdx.x & 63, R = p.R;
    int nb[KR];
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const int r = 64 * k + lane;
        const int qn = r < R ? p.cu_q_lens[r + 1] - p.cu_q_lens[r] : 0;
        nb[k] = decode_kind(qn, p.dq_max) ? decode_blocks(p.context_lens[r], qn) : 0;
    }
    int base = 0, first = -1, first_pfx = 0;
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        if (64 * k >= R) break;
        int incl = nb[k];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off, 64);
            if (lane >= off) incl += t;
        }
        const int r = 64 * k + lane;
        const int excl = base + incl - nb[k];
        if (write_list && nb[k] > 0 && excl >= g0 && excl < g1) const_cast<int32_t *>(dw.dpfx)[r] = excl;
        if (first < 0) {
            const unsigned long long hit = __builtin_amdgcn_ballot_w64(r < R && base + incl > g0);
            if (hit) {
                const int ln = __builtin_ctzll(hit);
                first = 64 * k + ln;
                first_pfx = __shfl(excl, ln, 64);
            }
        }
        base += __shfl(incl, 63, 64);
    }
    return make_int2(__builtin_amdgcn_readfirstlane(first), __builtin_amdgcn_readfirstlane(first_pfx));
}

// Whole-request ranges (short contexts, no plan kernel): workgroup b takes
// list entries [x0, x1); returns the flat pages {before x0, before x1}, from
// the same wave scan as above.
__device__ __forceinline__ int2 self_plan_range(const Params &p, int x0, int x1) {
    constexpr int KR = kSelfPlanReqs / 64;
    const int lane = threadIdx.x & 63, R = p.R;
    int nb[KR];
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const int r = 64 * k + lane;
        const int qn = r < R ? p.cu_q_lens[r + 1] - p.cu_q_lens[r] : 0;
        nb[k] = decode_kind(qn, p.dq_max) ? decode_blocks(p.context_lens[r], qn) : 0;
    }
    int base = 0, at0 = 0, at1 = 0;
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        if (64 * k >= R) break;
        int incl = nb[k];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off, 64);
            if (lane >= off) incl += t;
        }
        const int excl = base + incl - nb[k];
        if (x0 >= 64 * k && x0 < 64 * k + 64) at0 = __shfl(excl, x0 - 64 * k, 64);
        if (x1 >= 64 * k && x1 < 64 * k + 64) at1 = __shfl(excl, x1 - 64 * k, 64);
        base += __shfl(incl, 63, 64);
    }
    if (x1 >= R) at1 = base;
    return make_int2(__builtin_amdgcn_readfirstlane(at0), __builtin_amdgcn_readfirstlane(at1));
}

// Workgroup holding flat page g when NP pages are cut into nwg equal ranges
// [floor(b NP / nwg), floor((b+1) NP / nwg)).
__device__ __forceinline__ int wg_of_page(long long g, int np, int nwg) {
    return (int)(((g + 1) * nwg + np - 1) / np) - 1;
}

// Partial slot of workgroup b for a request whose first page lies in
// workgroup b_first: slot 1 of b when the request starts inside b's range
// (it is b's last segment), else slot 0 (b's first segment).
__device__ __forceinline__ int partial_slot(int hg, int b, int b_first, int nwg) {
    return (hg * nwg + b) * 2 + (b == b_first ? 1 : 0);
}

// Workgroups of up to 4 wavefronts at head_dim up to 128 ask for two
// wavefronts per SIMD (two or more workgroups per compute unit): the kernel
// then fits in 256 registers without spilling, where the unconstrained
// allocation (about 270 with accumulation registers) left one.
template <int D, int HW, int PF, bool NT>
__global__ __launch_bounds__(64 * HW, (D <= 128 && HW <= 4) ? 2 : 1) void decode_kernel(Params p, DecodeWork dw) {
    using C = DecodeCfg<D, HW>;
    constexpr int KS = C::KS, MB = C::MB, CPH = C::CPH, CPR = C::CPR, NTHR = C::NTHR,
                  NC = C::NC, SWM = C::SWM, HEAD = C::HEAD, TENSOR = C::TENSOR,
                  STAGE = C::STAGE;
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
    __shared__ int pid_lds[kNumPids];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n16 = lane & 15, kg = lane >> 4;
    const int hg = blockIdx.x, b = blockIdx.y, hb = blockIdx.z;  // hb: block of 16 query columns
    // (planning on the device: the page and workgroup counts the plan
    // kernel wrote; the launched workgroups past them have nothing to do)
    const int np = dw.counts ? ld_meta(dw.counts, 1) : dw.np;
    const int nwg = dw.counts ? ld_meta(dw.counts, 3) : dw.nwg;
    if (b >= nwg) return;
    // The workgroup's flat pages [g0, g1): an equal share of all pages, or
    // (whole-request mode) the pages of an equal share of the requests.
    int g0, g1, x0 = 0;
    if (dw.whole) {
        x0 = (int)(((long long)b * dw.nd) / nwg);
        const int2 g = self_plan_range(p, x0, (int)(((long long)(b + 1) * dw.nd) / nwg));
        g0 = g.x;
        g1 = g.y;
    } else {
        g0 = (int)(((long long)b * np) / nwg);
        g1 = (int)(((long long)(b + 1) * np) / nwg);
    }
    if (g0 >= g1) return;
    const int Hkv = p.Hkv, G = p.Hq / Hkv;
    const int hk0 = hg * HW;   // first kv head of this workgroup
    const int hk = hk0 + w;    // this wavefront's kv head
    const size_t page_elems = (size_t)16 * Hkv * D;

    // Cooperative, contiguous page-block loads: chunk u of this thread is the
    // 16-byte chunk tid + NTHR*u of the page's HW-head row segments (row j,
    // head hh of the group, dim chunk dc); it lands in LDS at head hh, row j,
    // chunk dc ^ (j & SWM) (an XOR swizzle that keeps the MFMA-layout reads
    // below free of bank conflicts).
    // Every chunk of a thread has the same head and dim chunk; its row
    // advances by RPU = NTHR / CPR per chunk.
    constexpr int RPU = NTHR / CPR;
    static_assert(NTHR % CPR == 0, "a thread's chunks must share their column");
    const int j0 = tid / CPR, cc = tid - j0 * CPR;
    const int hh = cc / CPH, dc0 = cc - hh * CPH;
    const int gofs0 = (j0 * Hkv + hk0 + hh) * D + 8 * dc0;  // + RPU*u rows of Hkv*D
    const int nofs = (hk0 + hh) * D + 8 * dc0;
    auto lds_ofs = [&](int u) {
        const int j = j0 + RPU * u;
        return hh * HEAD + j * D + 8 * (dc0 ^ (j & SWM));
    };

    // ---- page ids: the workgroup's flat pages, kNumPids at a time, go to
    // LDS in one cooperative pass (a scalar walk over the requests they
    // belong to), so that the page loop never waits on a memory round trip
    // for an id --------------------------------------------------------------
    DecodeReq first_q;
    if (dw.whole) {
        first_q = make_req(p, dw, x0, g0);
    } else if (dw.self_plan) {
        const int2 f = self_plan_first(p, dw, g0, g1, hg == 0 && hb == 0 && w == 0);
        first_q = make_req(p, dw, f.x, f.y);
    } else {
        const int first = ld_meta(dw.wstart, b);
        first_q = make_req(p, dw, first, ld_meta(dw.dpfx, first));
    }
    DecodeReq fq = first_q;  // fill cursor
    int pid_base = g0;                       // flat page held in pid_lds[0]
    auto fill_pids = [&]() {
        const int ge = min(pid_base + kNumPids, g1);
        while (pid_base >= fq.pend) fq = next_req(p, dw, fq);
        for (;;) {
            const int sb = max(pid_base, fq.pfx), se = min(ge, fq.pend);
            // Entries are 16-row blocks: block k of a request is sub-block
            // k % (S / 16) of its page k / (S / 16).
            const int32_t *row = p.page_table + (size_t)fq.r * p.max_pages;
            const int spb = p.S >> 4;
            for (int x = tid; x < se - sb; x += NTHR) {
                const int k = sb - fq.pfx + x;
                pid_lds[sb - pid_base + x] = row[k / spb] * spb + k % spb;
            }
            if (fq.pend >= ge) break;
            fq = next_req(p, dw, fq);
        }
        __syncthreads();
    };
    fill_pids();

    // ---- load cursor: walks the flat pages g0.. in order, PF ahead ---------
    DecodeReq lq = first_q;
    // Pages past the workgroup's range (the ring's last PF loads) read the
    // new-token rows of the current request instead: the instruction stream
    // stays the same on every path, so the compiler's wait counts stay exact
    // (a path without the prefetch would make it wait for every load), and
    // those few rows are cache hits.
    auto load_page = [&](int g, DecodeTile<NC> &tile) {
        const bool real = g < g1;
        size_t pid = 0;
        int pr = 0;
        if (real) {
            if (g - pid_base >= kNumPids) {  // next batch of ids (all waves are here)
                __syncthreads();
                pid_base += kNumPids;
                fill_pids();
            }
            while (g >= lq.pend) lq = next_req(p, dw, lq);
            pr = g - lq.pfx;  // page index inside the request
            pid = (size_t)__builtin_amdgcn_readfirstlane(pid_lds[g - pid_base]);
        }
        const bf16_t *knew = p.k_new + (size_t)lq.t0 * Hkv * D;
        const bf16_t *vnew = p.v_new + (size_t)lq.t0 * Hkv * D;
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            // Positions c .. c+q-1 are the new tokens (read from k_new /
            // v_new: the same bits, and never the slots this launch writes);
            // positions past the request (their scores are masked) read the
            // last new row, which keeps the stand-in V finite, so 0 * V
            // stays 0.
            const int pos = pr * 16 + j0 + RPU * u;
            const bool cached = real && pos < lq.c;
            const size_t nrow = (size_t)min(max(pos - lq.c, 0), lq.q - 1) * Hkv * D;
            const int gofs = gofs0 + RPU * u * Hkv * D;
            const bf16_t *ksrc = cached ? p.k_cache + pid * page_elems + gofs : knew + nrow + nofs;
            const bf16_t *vsrc = cached ? p.v_cache + pid * page_elems + gofs : vnew + nrow + nofs;
            tile.k[u] = stream_load<NT>(ksrc);
            tile.v[u] = stream_load<NT>(vsrc);
        }
    };
    auto store_page = [&](int stage, const DecodeTile<NC> &tile) {
        bf16_t *kbase = smem + stage * STAGE;
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int lo = lds_ofs(u);
            *reinterpret_cast<short8_t *>(kbase + lo) = tile.k[u];
            *reinterpret_cast<short8_t *>(kbase + TENSOR + lo) = tile.v[u];
        }
    };

    // ---- compute cursor: the request being accumulated ---------------------
    DecodeReq cq = lq;
    while (cq.pend == cq.pfx) cq = next_req(p, dw, cq);  // (a range may start at a request without pages)
    short8_t qb[KS];
    // This lane's query column: 16 per head block; column col of a request
    // with q new tokens is token col / G, head col % G, and exists when
    // col < q G.  Set per request by load_q, with the column's last visible
    // key.
    const int col = 16 * hb + n16;
    bool hv = false;
    int icol = 0, gcol = 0, clim = 0;
    // Q^T as the B operand: lane (column n16, group kg) holds q[t0 + icol][hk*G + gcol][32ks + 8kg .. +8].
    auto load_q = [&]() {
        hv = col < cq.q * G;
        icol = hv ? col / G : 0;
        gcol = hv ? col - icol * G : 0;
        clim = p.causal ? cq.c + icol : cq.c + cq.q - 1;
        const bf16_t *qrow = p.q + ((size_t)(cq.t0 + icol) * p.Hq + hk * G + gcol) * D;
        const short8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const short8_t x = *reinterpret_cast<const short8_t *>(qrow + 32 * ks + 8 * kg);
            qb[ks] = hv ? x : z;
        }
    };
    load_q();

    float4_t o[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = p.scale_log2;
    // This lane's V^T transposing-read row.
    const int vrow = 4 * kg + (n16 >> 2);

    auto compute_page = [&](int pr, int stage) {
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
        // Online softmax; this lane holds keys pr*16 + 4kg + i of column
        // n16, visible up to the column's limit.
        const int jb = pr * 16 + 4 * kg;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = (jb + i <= clim) ? s[i] * sl2 : -INFINITY;
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // Lazy rescale: the reference max m_run moves only when some head's
        // page max exceeds it by more than kLazyLog2 (P <= 2^kLazyLog2
        // otherwise).  o and l share the reference, so o / l is unchanged.
        // A column that has seen no visible key yet (m_run = -inf: a short
        // chunk's early token in a segment of later keys) keeps o = l = 0,
        // and its weights are 0, not exp2(-inf + inf).
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyLog2)) {
            const float mn = fmaxf(m_run, mx);
            const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mn);
            l_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
            m_run = mn;
        }
        const float mref = m_run == -INFINITY ? 0.f : m_run;
        float pr4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr4[i] = fast_exp2(sc[i] - mref);
        l_run += (pr4[0] + pr4[1]) + (pr4[2] + pr4[3]);
        // P as a bf16 pair hi + lo (lo = the rounding residue of hi), so the
        // PV product keeps ~16 bits of P: the MFMA work is negligible next to
        // the page's HBM time, and the only rounding left is the output's.
        short4_t pb_hi, pb_lo;
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            const uint32_t hi = cvt_pk_bf16(pr4[i], pr4[i + 1]);
            const float r0 = pr4[i] - __uint_as_float(hi << 16);
            const float r1 = pr4[i + 1] - __uint_as_float(hi & 0xffff0000u);
            const uint32_t lo = cvt_pk_bf16(r0, r1);
            pb_hi[i] = (short)(hi & 0xffff);
            pb_hi[i + 1] = (short)(hi >> 16);
            pb_lo[i] = (short)(lo & 0xffff);
            pb_lo[i + 1] = (short)(lo >> 16);
        }
        // O^T[d][head] += V^T[d][key] . P^T[key][head]; A = V^T by transposing
        // reads: lane reads row vrow, columns 16mb + 4(n16 & 3) .. +4.
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int e = 16 * mb + 4 * (n16 & 3);
            const int dc = e >> 3;
            const short4_t va = lds_read_tr16(vt + vrow * D + 8 * (dc ^ (vrow & SWM)) + (e & 7));
            o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_hi, o[mb], 0, 0, 0);
#if RA_DECODE_P_LO
            o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_lo, o[mb], 0, 0, 0);
#endif
        }
    };

    // End of a segment (the part of request cq inside this workgroup): write
    // the output when the segment is the whole request, otherwise a partial;
    // the last workgroup of the request to finish merges the partials.
    auto finish_segment = [&]() {
        float l_tot = l_run + __shfl_xor(l_run, 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        // (whole-request ranges never cut a request)
        const int b_first = dw.whole ? b : wg_of_page(cq.pfx, np, nwg);
        const int b_last = dw.whole ? b : wg_of_page(cq.pend - 1, np, nwg);
        bf16_t *orow = p.out + ((size_t)(cq.t0 + icol) * p.Hq + hk * G + gcol) * D;
        if (b_first == b_last) {
            if (hv) {
                const float inv = 1.f / l_tot;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    uint2 wv;
                    wv.x = cvt_pk_bf16(o[mb][0] * inv, o[mb][1] * inv);
                    wv.y = cvt_pk_bf16(o[mb][2] * inv, o[mb][3] * inv);
                    *reinterpret_cast<uint2 *>(orow + 16 * mb + 4 * kg) = wv;
                }
            }
            return;
        }
        // Partial slot: a workgroup's last segment (the request starts inside
        // its range) uses slot 1, its first segment slot 0.  The merge kernel
        // combines the slots of the request's workgroups after this launch
        // (a kernel boundary makes them visible without device-wide fences,
        // which flush the L2 of every XCD and would stall the streaming).
        if (hv) {
            const size_t sidx = (size_t)partial_slot(hg, b, b_first, nwg) * (HW * dw.cw) + w * dw.cw + col;
            float *prow = dw.part_o + sidx * D;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                *reinterpret_cast<float4_t *>(prow + 16 * mb + 4 * kg) = o[mb];
            if (kg == 0) {
                dw.part_ml[sidx * 2] = m_run;
                dw.part_ml[sidx * 2 + 1] = l_tot;
            }
        }
    };

    // One flat page through the pipeline: fused KV update on the request's
    // last page, scores/softmax/PV, and the end of the segment.
    auto step = [&](int g, int stage) {
        const int pr = g - cq.pfx;
        if (lane < CPH && hb == 0 && !p.skip_scatter) {
            // Fused KV-cache update of the new tokens in this block
            // (positions c .. c+q-1), this wavefront's kv head: the rows are
            // in the LDS tile already (loaded from k_new / v_new), so the
            // copies wait on no global load.
            const int pos_end = min(cq.c + cq.q, pr * 16 + 16);
            for (int pos = max(cq.c, pr * 16); pos < pos_end; ++pos) {
                const int j = pos & 15, dc = lane;
                const bf16_t *kt = smem + stage * STAGE + w * HEAD + j * D + 8 * (dc ^ (j & SWM));
                const short8_t kr = *reinterpret_cast<const short8_t *>(kt);
                const short8_t vr = *reinterpret_cast<const short8_t *>(kt + TENSOR);
                const size_t dst = ((size_t)ld_meta(p.slot_mapping, cq.t0 + pos - cq.c) * Hkv + hk) * D + 8 * dc;
                *reinterpret_cast<short8_t *>(p.k_cache + dst) = kr;
                *reinterpret_cast<short8_t *>(p.v_cache + dst) = vr;
            }
        }
        compute_page(pr, stage);
        if (g == cq.pend - 1 || g == g1 - 1) {
            finish_segment();
            if (g + 1 < g1) {
                // (requests without pages hold no flat page: skip them)
                do cq = next_req(p, dw, cq);
                while (cq.pend == cq.pfx);
                load_q();
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) o[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
                m_run = -INFINITY;
                l_run = 0.f;
            }
        }
    };

    // Ring of PF + 1 page tiles in registers: pages g+1 .. g+PF are in flight
    // while page g goes to LDS stage g & 1 and is computed.  One barrier per
    // page: a stage is rewritten two pages later, after every wavefront has
    // passed the barrier that follows its last read.
    constexpr int NR = PF + 1;
    DecodeTile<NC> ring[NR];
#pragma unroll
    for (int k = 0; k < PF; ++k) load_page(g0 + k, ring[k]);
    for (int g = g0; g < g1; g += NR) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            if (g + k >= g1) break;
            load_page(g + k + PF, ring[(k + PF) % NR]);
            store_page((g + k) & 1, ring[k]);
            __syncthreads();
            step(g + k, (g + k) & 1);
        }
    }
}

// Log-sum-exp merge of the partials of every decode request that several
// workgroups share: one single-wavefront workgroup per (request, kv head),
// lanes laid out like the decode accumulators (eight-wavefront workgroups,
// one per head group, took 7.4 against 6.4 us per call on 128 requests).
//   M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// (m is kept in the exp2 domain).
template <int D, int HW>
__global__ __launch_bounds__(64) void decode_merge_kernel(Params p, DecodeWork dw) {
    constexpr int MB = D / 16;
    const int i = blockIdx.x, hg = blockIdx.y / HW;  // (requests on x: more than 65535 of them fit)
    // Planning on the device: the grid covers every request, the list holds
    // counts[0] decode requests.
    if (dw.counts && i >= ld_meta(dw.counts, 0)) return;
    const int np = dw.counts ? ld_meta(dw.counts, 1) : dw.np;
    const int nwg = dw.counts ? ld_meta(dw.counts, 3) : dw.nwg;
    const int r = dw.self_plan ? i : ld_meta(dw.dreq, i);
    const int t0 = ld_meta(p.cu_q_lens, r);
    const int qn = ld_meta(p.cu_q_lens, r + 1) - t0;
    if (dw.self_plan && !decode_kind(qn, p.dq_max)) return;  // not a decode-kernel request
    const int pfx = ld_meta(dw.dpfx, i), pend = pfx + decode_blocks(ld_meta(p.context_lens, r), qn);
    const int b_first = wg_of_page(pfx, np, nwg);
    const int b_last = wg_of_page(pend - 1, np, nwg);
    if (b_first == b_last) return;  // written by the decode kernel
    const int lane = threadIdx.x & 63, w = blockIdx.y % HW;
    const int n16 = lane & 15, kg = lane >> 4;
    const int G = p.Hq / p.Hkv;
    // Query columns n16, n16 + 16, ... of this wavefront's kv head (column
    // n: token n / G, head n % G of the request's q new tokens).
    for (int col = n16; col < qn * G; col += 16) {
        const int hl = w * dw.cw + col;  // column inside the head group's slot
        // One pass with a running max; the slots are read kU at a time so
        // that their loads are in flight together (a request rarely spans
        // more than two workgroups; four at a time, mostly repeating the
        // last slot, made the kernel ~2 us slower).
        constexpr int kU = 2;
        float M = -INFINITY, den = 0.f;
        float4_t acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
        for (int b0 = b_first; b0 <= b_last; b0 += kU) {
            float ms[kU], ls[kU];
            float4_t os[kU][MB];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int bb = min(b0 + u, b_last);
                const size_t sidx = (size_t)partial_slot(hg, bb, b_first, nwg) * (HW * dw.cw) + hl;
                ms[u] = dw.part_ml[sidx * 2];
                ls[u] = dw.part_ml[sidx * 2 + 1];
                const float *prow = dw.part_o + sidx * D;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) os[u][mb] = *reinterpret_cast<const float4_t *>(prow + 16 * mb + 4 * kg);
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (b0 + u > b_last) break;
                // (a segment with no key visible to this column: m = -inf,
                // l = o = 0, nothing to add)
                if (ms[u] == -INFINITY) continue;
                const float mn = fmaxf(M, ms[u]);
                const float a = fast_exp2(M - mn), wgt = fast_exp2(ms[u] - mn);
                den = den * a + wgt * ls[u];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[mb] = acc[mb] * a + wgt * os[u][mb];
                M = mn;
            }
        }
        const float inv = 1.f / den;
        const int icol = col / G;
        bf16_t *orow = p.out + ((size_t)(t0 + icol) * p.Hq + (hg * HW + w) * G + col - icol * G) * D;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            uint2 wv;
            wv.x = cvt_pk_bf16(acc[mb][0] * inv, acc[mb][1] * inv);
            wv.y = cvt_pk_bf16(acc[mb][2] * inv, acc[mb][3] * inv);
            *reinterpret_cast<uint2 *>(orow + 16 * mb + 4 * kg) = wv;
        }
    }
}

template <int D, int HW, int PF>
hipError_t configure_decode() {
    static bool configured = false;
    if (!configured) {
        hipError_t e = hipFuncSetAttribute((const void *)decode_kernel<D, HW, PF, true>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)DecodeCfg<D, HW>::LDS_BYTES);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)decode_kernel<D, HW, PF, false>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)DecodeCfg<D, HW>::LDS_BYTES);
        if (e != hipSuccess) return e;
        configured = true;
    }
    return hipSuccess;
}

// Workgroups of this configuration resident at once on the whole device.
template <int D, int HW, int PF>
hipError_t decode_capacity(int *cap) {
    hipError_t e = configure_decode<D, HW, PF>();
    if (e != hipSuccess) return e;
    int dev = 0, cus = 0, per_cu = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<D, HW, PF, true>, 64 * HW,
                                                         DecodeCfg<D, HW>::LDS_BYTES);
    if (e != hipSuccess) return e;
    *cap = std::max(1, cus * std::max(1, per_cu));
    return hipSuccess;
}

template <int D, int HW, int PF>
hipError_t launch_decode_cfg(const Params &p, const DecodeWork &dw, hipStream_t stream,
                             const StageEvents &ev) {
    hipError_t e = configure_decode<D, HW, PF>();
    if (e != hipSuccess) return e;
    // One slice of the grid per 16 query columns of a kv head (G heads, or
    // q tokens x G heads of a short chunk); the slices of one page range
    // (same x, y) are 8k workgroups apart, on one XCD, and resident together,
    // so they read each page from HBM about once and from L2 otherwise.
    const int slices = decode_column_blocks(dw.cw);
    const dim3 grid(p.Hkv / HW, dw.nwg, slices);
    const size_t lds = DecodeCfg<D, HW>::LDS_BYTES;
    e = launch_kernel(slices == 1 ? decode_kernel<D, HW, PF, true> : decode_kernel<D, HW, PF, false>, grid,
                      dim3(64 * HW), (uint32_t)lds, stream, ev.start(kStageDecode), ev.stop(kStageDecode), p, dw);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dw.whole) return ev.empty(kStageMerge);  // no request is cut: nothing to merge
    const dim3 mgrid(dw.nd, p.Hkv);
    e = launch_kernel(decode_merge_kernel<D, HW>, mgrid, dim3(64), 0, stream, ev.start(kStageMerge),
                      ev.stop(kStageMerge), p, dw);
    return e != hipSuccess ? e : hipGetLastError();
}

// Calls f.template operator()<HW>() with the compile-time head-group size.
template <int D, int PF, typename F>
hipError_t with_hw(int hw, F &&f) {
    switch (hw) {
        case 8: if constexpr (D <= 128) return f(std::integral_constant<int, 8>()); break;
        case 4: return f(std::integral_constant<int, 4>());
        case 2: return f(std::integral_constant<int, 2>());
        case 1: return f(std::integral_constant<int, 1>());
        default: break;
    }
    return hipErrorInvalidValue;
}

template <int D, int PF>
hipError_t launch_decode_d(const Params &p, const DecodeWork &dw, hipStream_t stream,
                           const StageEvents &ev) {
    return with_hw<D, PF>(dw.hw, [&](auto hw) {
        return launch_decode_cfg<D, decltype(hw)::value, PF>(p, dw, stream, ev);
    });
}

template <int D, int PF>
hipError_t capacity_d(int hw_, int *cap) {
    return with_hw<D, PF>(hw_, [&](auto hw) { return decode_capacity<D, decltype(hw)::value, PF>(cap); });
}

}  // namespace

int decode_heads_per_group(int D, int Hkv, long long blocks, int nd) {
    // RA_DECODE_HW (environment) overrides the choice, for tuning, when it is
    // one of the sizes below and divides Hkv.
    if (const char *env = getenv("RA_DECODE_HW")) {
        const int hw = atoi(env);
        if ((hw == 1 || hw == 2 || hw == 4 || (hw == 8 && D <= 128)) && Hkv % hw == 0) return hw;
    }
    // Largest HW in {8, 4, 2, 1} dividing Hkv whose row segment (HW heads of
    // one token row) is at most 2 KiB: one page block then arrives as 16
    // contiguous segments.  Short contexts (at most kShortBlocks 16-row
    // blocks per request on average) take 8 heads as two groups of 4: twice
    // the workgroups, half the LDS each, two per compute unit, which hides
    // more of the start-up latency of their short page ranges (measured:
    // 27.8 -> 23.1 us per call at 128 requests x 128 tokens, equal at 1024
    // tokens, slower from 2048).
    constexpr long long kShortBlocks = 40;
    for (int hw = 8; hw > 1; hw >>= 1)
        if (Hkv % hw == 0 && hw * D * 2 <= 2048) {
            if (hw == 8 && nd > 0 && blocks <= kShortBlocks * nd) return 4;
            return hw;
        }
    return 1;
}

hipError_t decode_workgroups(const Params &p, const Plan &plan, int whole, int *nwg, int *fill, int *cus) {
    int cap = 0;
    hipError_t e;
    switch (p.D) {
        case 64: e = capacity_d<64, RA_DECODE_PF64>(plan.decode_hw, &cap); break;
        case 128: e = capacity_d<128, RA_DECODE_PF128>(plan.decode_hw, &cap); break;
        case 256: e = capacity_d<256, RA_DECODE_PF256>(plan.decode_hw, &cap); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if (cus) {
        int dev = 0;
        e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    // One resident wave of workgroups, none with fewer than kMinDecodePages pages.
    // RA_DECODE_WGS (environment) overrides the resident count, for tuning.
    const char *env = getenv("RA_DECODE_WGS");
    const int forced = env ? atoi(env) : 0;
    // More than 16 query columns per kv head (groups of more than 16 heads,
    // or wide short chunks) launch one grid slice per block of 16 columns:
    // together they fill the resident slots once.
    const int hblocks = decode_column_blocks(plan.cw);
    if (forced > 0) cap = forced * plan.decode_hgroups * hblocks;
    int n = std::max(1, cap / (plan.decode_hgroups * hblocks));
    if (fill) *fill = n;  // workgroups per head group that fill every compute unit once
    n = std::min(n, plan.decode_wg_cap);
    // (planning on the device: the page count is unknown here; workgroups
    // whose range is empty exit at once)
    if (!plan.bounds) n = std::min(n, whole > 0 ? whole : std::max(1, plan.n_decode_pages / kMinDecodePages));
    // With several slices, a multiple of 8 workgroups per slice keeps the
    // slices of one page range on one XCD (workgroups go to XCDs round robin).
    if (hblocks > 1 && n >= 8) n -= n % 8;
    *nwg = n;
    return hipSuccess;
}

hipError_t launch_decode(const Params &p, const DecodeWork &dw, hipStream_t stream,
                         const StageEvents &ev) {
    switch (p.D) {
        case 64: return launch_decode_d<64, RA_DECODE_PF64>(p, dw, stream, ev);
        case 128: return launch_decode_d<128, RA_DECODE_PF128>(p, dw, stream, ev);
        case 256: return launch_decode_d<256, RA_DECODE_PF256>(p, dw, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ra
