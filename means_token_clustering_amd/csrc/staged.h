// Device helpers of the staged kernels (k-means steps, centroid attention,
// local window, backward pass, exact attention): lane-group reductions, dot
// products and the softmax exponential. The single-launch kernels do not use
// them.
#pragma once

#include "common.h"

namespace ca {

// (value, index) lexicographic minimum: the smaller value wins, and on equal
// values the smaller index wins. NaN never wins against a number.
__device__ __forceinline__ bool lex_less(float a, int ia, float b, int ib) {
    return (a < b) || (a == b && ia < ib) || (b != b && a == a);
}

// a . b over 16 (64) elements with four independent fma chains joined in a
// fixed order: a quarter of the dependent latency of one chain.
__device__ __forceinline__ float dot16(const float *a, const float *b) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
        s0 = fmaf(a[c], b[c], s0);
        s1 = fmaf(a[c + 1], b[c + 1], s1);
        s2 = fmaf(a[c + 2], b[c + 2], s2);
        s3 = fmaf(a[c + 3], b[c + 3], s3);
    }
    return (s0 + s1) + (s2 + s3);
}
__device__ __forceinline__ float dot64(const float *a, const float *b) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int c = 0; c < 64; c += 4) {
        s0 = fmaf(a[c], b[c], s0);
        s1 = fmaf(a[c + 1], b[c + 1], s1);
        s2 = fmaf(a[c + 2], b[c + 2], s2);
        s3 = fmaf(a[c + 3], b[c + 3], s3);
    }
    return (s0 + s1) + (s2 + s3);
}

// Sum over the four lanes 4q .. 4q+3 through DPP quad permutes (no LDS
// round trip); the adds are commutative, so all four lanes get the same bits.
__device__ __forceinline__ float quad_sum(float x) {
    const float y = x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                            __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
    return y + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                   __builtin_bit_cast(int, y), 0x4E, 0xF, 0xF, false));            // [2,3,0,1]
}

// Wave-wide integer min / max (all 64 lanes must be active and converged).
__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) v = min(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) v = max(v, __shfl_xor(v, off));
    return v;
}

// exp(x) for softmax weights, as 2^(x log2 e) on the hardware exp2 unit.
__device__ __forceinline__ float exp_f32(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

}  // namespace ca
