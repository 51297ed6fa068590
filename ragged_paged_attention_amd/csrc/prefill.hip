// prefill.hip -- the MFMA-bound kernel for prefill chunks (requests with more
// than one new token), with the KV-cache update fused in.
//
// Work unit: one workgroup of 4 wavefronts per (request r, kv head hk, query
// tile of Mq = 128/G tokens).  Its 128 query rows are the G query heads of
// the group times the Mq tokens, so one K/V tile in LDS serves every head
// that reads it (grouped-query attention).  Wave w owns rows 32w..32w+31.
//
// Key tiles of N keys (64 for head_dim <= 128, 32 for 256) stream through
// two LDS stages: while the MFMA units work on stage t, the next tile's
// 16-byte global loads are in flight in registers, and land in the other
// stage before the one barrier per tile.  Keys at positions < c_r come from
// the cache through the page table, positions >= c_r from k_new/v_new.
//
// Per tile and wave (v_mfma_f32_32x32x16_bf16 throughout):
//   S^T[key][row] = K . Q^T     A = K rows from LDS (16 B per lane),
//                               B = Q^T held in registers for the whole loop;
//   online softmax on S^T       each lane owns one query row: the row max is
//                               an in-lane max plus one cross-half step, and
//                               the rescale of O^T is lane-local;
//   O^T[d][row] += V^T . P^T    B = P^T straight from the S^T accumulators
//                               (converted to bf16 with v_cvt_pk_bf16_f32),
//                               A = V^T by ds_read_b64_tr_b16 from the
//                               row-major V tile: each 16-lane group points
//                               at 4 key rows x 4 column quads and lane j
//                               receives column j of those 4 keys.
// Causal masking: tiles beyond the last row's position are never loaded;
// tiles beyond a wave's last position are skipped by that wave; the mask
// is applied only on tiles that cross a row's limit.
// The workgroup copies the new K/V rows of its own query tokens into the
// cache (each (token, kv head) row is written exactly once).
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

template <int D>
struct PrefillCfg {
    static constexpr int N = D <= 128 ? 64 : 32;  // keys per tile
    static constexpr int KS = D / 16;              // QK k-steps
    static constexpr int MBK = N / 32;             // 32-key blocks of S^T per tile
    static constexpr int MD = D / 32;              // 32-wide head_dim blocks of O^T
    static constexpr int RS = D + 16;              // LDS row stride (elements)
    static constexpr int CH = D / 8;               // 16-byte chunks per row
    static constexpr int LD = N * CH / 256;        // chunks per thread per tensor per tile
    static constexpr int MIN_WAVES = D <= 128 ? 2 : 1;
};

template <int D>
__global__ __launch_bounds__(256, PrefillCfg<D>::MIN_WAVES) void prefill_kernel(
    Params p, const int4 *__restrict__ items) {
    using C = PrefillCfg<D>;
    constexpr int N = C::N, KS = C::KS, MBK = C::MBK, MD = C::MD, RS = C::RS, CH = C::CH,
                  LD = C::LD;
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
    // smem: [stage 0: K | V][stage 1: K | V], each N x RS elements

    const int4 it = items[blockIdx.x];
    const int r = it.x;
    if (r < 0) return;
    const int hk = it.y, q0 = it.z;
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, n32 = l & 31, h2 = l >> 5;
    const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv, Mq = 128 / G;
    const int t0 = p.cu_q_lens[r];
    const int qlen = p.cu_q_lens[r + 1] - t0;
    const int c = p.context_lens[r];
    const int L = c + qlen;
    const int tile_q = min(Mq, qlen - q0);
    const int kv_end = p.causal ? c + q0 + tile_q : L;
    const int ntiles = (kv_end + N - 1) / N;
    const int32_t *ptab = p.page_table + (size_t)r * p.max_pages;

    // Fused KV-cache update: the new rows of this tile's tokens, kv head hk.
    for (int idx = tid; idx < tile_q * CH; idx += 256) {
        const int row = idx / CH, col = idx - row * CH;
        const int t = t0 + q0 + row;
        const size_t dst = ((size_t)p.slot_mapping[t] * Hkv + hk) * D + 8 * col;
        const size_t src = ((size_t)t * Hkv + hk) * D + 8 * col;
        *reinterpret_cast<uint4 *>(p.k_cache + dst) = *reinterpret_cast<const uint4 *>(p.k_new + src);
        *reinterpret_cast<uint4 *>(p.v_cache + dst) = *reinterpret_cast<const uint4 *>(p.v_new + src);
    }

    // This lane's query row.
    const int R = 32 * w + n32;
    const int g = R / Mq, iq = R - g * Mq;
    const bool row_valid = iq < tile_q;
    const int i = q0 + (row_valid ? iq : 0);
    const int head = hk * G + g;
    const int lim = row_valid ? (p.causal ? c + i : L - 1) : kv_end - 1;  // last visible key
    const int wave_end = wave_max_i(row_valid ? lim : -1) + 1;
    const int wave_lim_min = wave_min_i(row_valid ? lim : 0x7fffffff);

    // Q^T as the B operand: lane holds q[t0 + i][head][16ks + 8h2 .. +8].
    short8_t qb[KS];
    {
        const bf16_t *qrow = p.q + ((size_t)(t0 + i) * Hq + head) * D + 8 * h2;
        const short8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const short8_t x = *reinterpret_cast<const short8_t *>(qrow + 16 * ks);
            qb[ks] = row_valid ? x : z;
        }
    }

    // Register-staged tile loads (16 B chunks, consecutive threads along a row).
    short8_t kreg[LD], vreg[LD];
    auto load_tile = [&](int tile) {
        const int j0 = tile * N;
        const short8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < LD; ++k) {
            const int q = tid + 256 * k;
            const int row = q / CH, col = q - row * CH;
            const int j = j0 + row;
            const bool valid = j < kv_end;
            const int je = valid ? j : kv_end - 1;
            size_t rowaddr;
            if (je < c) {
                const size_t page = (size_t)ptab[je >> 4];
                rowaddr = ((page * 16 + (je & 15)) * Hkv + hk) * D;
            } else {
                rowaddr = (((size_t)t0 + (je - c)) * Hkv + hk) * D;
            }
            const bool from_cache = je < c;
            const bf16_t *kb = from_cache ? p.k_cache : p.k_new;
            const bf16_t *vb = from_cache ? p.v_cache : p.v_new;
            const short8_t xk = *reinterpret_cast<const short8_t *>(kb + rowaddr + 8 * col);
            const short8_t xv = *reinterpret_cast<const short8_t *>(vb + rowaddr + 8 * col);
            kreg[k] = valid ? xk : z;
            vreg[k] = valid ? xv : z;
        }
    };
    auto store_tile = [&](int stage) {
        bf16_t *ks = smem + stage * 2 * N * RS;
        bf16_t *vs = ks + N * RS;
#pragma unroll
        for (int k = 0; k < LD; ++k) {
            const int q = tid + 256 * k;
            const int row = q / CH, col = q - row * CH;
            *reinterpret_cast<short8_t *>(ks + row * RS + 8 * col) = kreg[k];
            *reinterpret_cast<short8_t *>(vs + row * RS + 8 * col) = vreg[k];
        }
    };

    float16_t o[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[md][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = p.scale_log2;
    // Transposing-read lane address inside a V tile: row 4h2 + (j>>2), column
    // 16*(n32>>4) + 4*(j&3) with j = l & 15.
    const int vt_off = (4 * h2 + ((l & 15) >> 2)) * RS + 16 * (n32 >> 4) + 4 * (l & 3);

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int tile = 0; tile < ntiles; ++tile) {
        const int stage = tile & 1;
        if (tile + 1 < ntiles) load_tile(tile + 1);
        const int j0 = tile * N;
        if (j0 < wave_end) {
            const bf16_t *Ks = smem + stage * 2 * N * RS;
            const bf16_t *Vs = Ks + N * RS;
            float16_t s[MBK];
#pragma unroll
            for (int mb = 0; mb < MBK; ++mb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const short8_t a = *reinterpret_cast<const short8_t *>(
                        Ks + (32 * mb + n32) * RS + 16 * ks + 8 * h2);
                    s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], s[mb], 0, 0, 0);
                }
            }
            // Scale into the exp2 domain; mask keys past this row's limit.
            const bool need_mask = j0 + N - 1 > wave_lim_min;
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < MBK; ++mb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = s[mb][e] * sl2;
                    if (need_mask) {
                        const int key = j0 + 32 * mb + 8 * (e >> 2) + 4 * h2 + (e & 3);
                        v = key > lim ? -INFINITY : v;
                    }
                    s[mb][e] = v;
                    mx = fmaxf(mx, v);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mn = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - mn);
            m_run = mn;
            float lsum = 0.f;
            short8_t pb[MBK][2];
#pragma unroll
            for (int mb = 0; mb < MBK; ++mb) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    uint32_t w4[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const float pa = fast_exp2(s[mb][8 * s2 + 2 * e2] - mn);
                        const float pc = fast_exp2(s[mb][8 * s2 + 2 * e2 + 1] - mn);
                        lsum += pa + pc;
                        w4[e2] = cvt_pk_bf16(pa, pc);
                    }
                    pb[mb][s2] = __builtin_bit_cast(short8_t, w4);
                }
            }
            l_run = l_run * alpha + lsum;
#pragma unroll
            for (int md = 0; md < MD; ++md) o[md] *= alpha;
            // O^T += V^T . P^T over the tile's keys, 16 per MFMA.
#pragma unroll
            for (int mb = 0; mb < MBK; ++mb) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const bf16_t *vb = Vs + (32 * mb + 16 * s2) * RS + vt_off;
#pragma unroll
                    for (int md = 0; md < MD; ++md) {
                        const short4_t lo = lds_read_tr16(vb + 32 * md);
                        const short4_t hi = lds_read_tr16(vb + 8 * RS + 32 * md);
                        const short8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[mb][s2], o[md], 0, 0, 0);
                    }
                }
            }
        }
        if (tile + 1 < ntiles) store_tile(stage ^ 1);
        __syncthreads();
    }

    if (row_valid) {
        const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
        const float inv = 1.f / l_tot;
        bf16_t *orow = p.out + ((size_t)(t0 + i) * Hq + head) * D;
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
    } else {
        (void)__shfl_xor(l_run, 32, 64);
    }
}

template <int D>
hipError_t launch_prefill_d(const Params &p, const Plan &plan, const int4 *items, hipStream_t stream) {
    using C = PrefillCfg<D>;
    const size_t lds = (size_t)2 * 2 * C::N * C::RS * sizeof(bf16_t);
    static bool configured = false;
    if (!configured) {
        hipError_t e = hipFuncSetAttribute((const void *)prefill_kernel<D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    hipLaunchKernelGGL(prefill_kernel<D>, dim3(plan.n_prefill_items), dim3(256), lds, stream, p, items);
    return hipGetLastError();
}

}  // namespace

bool prefill_supports(int D, int G) {
    return (D == 64 || D == 128 || D == 256) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

hipError_t launch_prefill(const Params &p, const Plan &plan, const int4 *items, hipStream_t stream) {
    switch (p.D) {
        case 64: return launch_prefill_d<64>(p, plan, items, stream);
        case 128: return launch_prefill_d<128>(p, plan, items, stream);
        case 256: return launch_prefill_d<256>(p, plan, items, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ra
