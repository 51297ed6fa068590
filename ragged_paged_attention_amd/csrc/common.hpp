// common.hpp -- device helpers shared by the libragged_attn kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef uint16_t bf16_t;  // raw IEEE bfloat16 bits

// Parameters of one fused call, as the kernels see them.
struct Params {
    const bf16_t *q;        // [T][Hq][D]
    const bf16_t *k_new;    // [T][Hkv][D]
    const bf16_t *v_new;    // [T][Hkv][D]
    bf16_t *k_cache;        // [P][S][Hkv][D]
    bf16_t *v_cache;        // [P][S][Hkv][D]
    const int32_t *page_table;    // [R][max_pages]
    const int32_t *cu_q_lens;     // [R+1]
    const int32_t *context_lens;  // [R]
    const int32_t *slot_mapping;  // [T]
    bf16_t *out;            // [T][Hq][D]
    int32_t R, T, Hq, Hkv, D, S, max_pages, causal;
    float scale_log2;       // softmax scale * log2(e): scores live in the exp2 domain
    int32_t prefill_only;   // generic kernel: skip tokens of decode (q_r == 1) requests
    int32_t skip_scatter;   // attention kernels leave the cache alone (a separate scatter ran)
    int32_t dq_max;         // requests with 1 <= q_r <= dq_max run in the decode kernel (one
                            // decode token, or a short chunk of q_r G <= 32 query columns)
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Low / high bf16 of a packed pair, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Request owning token t: the largest r with cu_q_lens[r] <= t (empty requests
// share a cu_q_lens value with the next one and are skipped by "largest").
__device__ __forceinline__ int request_of_token(const int32_t *cu_q_lens, int R, int t) {
    int lo = 0, hi = R;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (cu_q_lens[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

}  // namespace ra

namespace ra {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair with the hardware convert (v_cvt_pk_bf16_f32,
// round to nearest even); lo lands in the low half.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    const float2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float pair_sum_bf16(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}

}  // namespace ra
