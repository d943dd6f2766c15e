// Shared device helpers of the cluster attention library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "clusterattn.h"

namespace ca {

constexpr int kD = 64;          // head dimension supported by the kernels
constexpr int kMaxClusters = 256;
constexpr int kWave = 64;

// Grouped K/V heads: query slice s = b * H + h reads K and V of slice
// b * (H / G) + h / G, G query heads sharing one K/V head (G = 1: its own).
__host__ __device__ __forceinline__ long kv_slice(long s, int H, int G) {
    return G == 1 ? s : (s / H) * (H / G) + (s % H) / G;
}

// bf16 storage is carried as raw uint16 bit patterns.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Load 4 consecutive elements (16 B for fp32, 8 B for bf16) as floats.
template <typename T>
__device__ __forceinline__ float4 load4(const T *p);

template <>
__device__ __forceinline__ float4 load4<float>(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}

template <>
__device__ __forceinline__ float4 load4<bf16_t>(const bf16_t *p) {
    uint2 u = *reinterpret_cast<const uint2 *>(p);
    float4 r;
    r.x = __uint_as_float(u.x << 16);
    r.y = __uint_as_float(u.x & 0xffff0000u);
    r.z = __uint_as_float(u.y << 16);
    r.w = __uint_as_float(u.y & 0xffff0000u);
    return r;
}

template <typename T>
__device__ __forceinline__ void store4(T *p, float4 v);

template <>
__device__ __forceinline__ void store4<float>(float *p, float4 v) {
    *reinterpret_cast<float4 *>(p) = v;
}

template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *p, float4 v) {
    uint2 u;
    u.x = static_cast<uint32_t>(f32_to_bf16(v.x)) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
    u.y = static_cast<uint32_t>(f32_to_bf16(v.z)) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
    *reinterpret_cast<uint2 *>(p) = u;
}

// (value, index) lexicographic minimum: the smaller value wins, and on equal
// values the smaller index wins. NaN never wins against a number.
__device__ __forceinline__ bool lex_less(float a, int ia, float b, int ib) {
    return (a < b) || (a == b && ia < ib) || (b != b && a == a);
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

// Host-side launch helpers live in the .hip files; declared here so the
// C-ABI translation unit can call them.
namespace ca {

// Listing-compatible variants of the clustering and the gather (the
// ClusterAttention listing on the "Hooshaai/svd-sst2-roberta-cluster" page,
// its k-means routine and forward).
struct Variant {
    int init_step;     // 0: initial rows floor(k L / Kc); > 0: rows k * init_step
    bool keep_empty;   // an empty cluster keeps its previous centroid (else zero)
    bool soft;         // gather sum_k softmax_k(q . mu_k / sqrt(d)) V^cent_k
};

// Row of Q that initialises cluster k (increasing in k, below L for Kc <= L).
__host__ __device__ inline int init_row(int k, int L, int Kc, int init_step) {
    return init_step > 0 ? k * init_step : (int)(((long)k * L) / Kc);
}

// mu == nullptr: the centroids are the initial rows of Q (init_row with
// init_step); mu_init, if not null, then receives them.
hipError_t launch_kmeans_assign(const void *Q, const float *mu, int S, int L, int Kc,
                                ca_dtype_t dt, int32_t *assign, float *part_sum,
                                int32_t *part_cnt, hipStream_t st, int init_step = 0,
                                float *mu_init = nullptr);
hipError_t launch_centroid_partials(const void *Q, const int32_t *assign, int S, int L, int Kc,
                                    ca_dtype_t dt, float *part_sum, int32_t *part_cnt,
                                    hipStream_t st);
int kmeans_tiles(int L);
// keep_empty: an empty cluster leaves its row of mu as it was
hipError_t launch_centroid_reduce(const float *part_sum, const int32_t *part_cnt, int nblk,
                                  int S, int Kc, float *mu, int32_t *counts, hipStream_t st,
                                  bool keep_empty = false);

int xattn_splits(int L);
// valid: key-padding mask [B, L] (nonzero = real token) or nullptr; slice s
// belongs to batch row s / H. G: query heads per K/V head (see kv_slice).
// stats (nullable, [S, Kc, 2]): per row the largest scaled logit and the sum
// of exp(logit - largest).
hipError_t launch_centroid_xattn(const float *mu, const void *K, const void *V, int S, int L,
                                 int Kc, ca_dtype_t dt, const uint8_t *valid, int H, int G,
                                 float *vcent, float *partials, hipStream_t st,
                                 float *stats = nullptr);

// Window |i - j| <= r. With oloc == nullptr the gather + fusion epilogue
// writes out; mu != nullptr selects the soft gather over the centroids mu.
hipError_t launch_local_window(const void *Q, const void *K, const void *V, int S, int L, int r,
                               ca_dtype_t dt, const float *vcent, const int32_t *assign, int Kc,
                               float alpha, const uint8_t *valid, int H, int G, void *out,
                               float *oloc, hipStream_t st, const float *mu = nullptr);
hipError_t launch_gather_fuse(const float *vcent, const int32_t *assign, const float *oloc, int S,
                              int L, int Kc, float alpha, ca_dtype_t dt, void *out,
                              hipStream_t st);

// Backward pass (backward.hip): buffers and sizes of one launch sequence.
// Q, dO, dQ [B, H, L, 64]; K, V, dK, dV [B, Hkv, L, 64] (storage dtype);
// assign [B, H, L]; the rest fp32 workspace: mu, vcent, dvc, dmu [S, Kc, 64],
// counts [S, Kc], cstat [S, Kc, 2] (row max and sum of the centroid
// softmax), part [S, tiles, Kc, 64], lstat [S, L] (max, sum, D, 0 of the
// local softmax), dal [S * tiles]; dalpha (nullable) one float.
struct BwdArgs {
    const void *Q, *K, *V, *dO;
    const int32_t *assign;
    const uint8_t *valid;
    int B, H, Hkv, L, Kc, r;
    float alpha;
    const float *mu;
    const int32_t *counts;
    const float *vcent, *cstat;
    float *dvc, *dmu, *part;
    float4 *lstat;
    float *dal;
    void *dQ, *dK, *dV;
    float *dalpha;
};
int bwd_tiles(int L);
hipError_t launch_backward(const BwdArgs &a, ca_dtype_t dt, hipStream_t st);

// Exact attention (decoder / cross-attention branch): Q [S, L, 64], K, V
// [S / G, Nk, 64] (grouped heads as in kv_slice); qvalid [S / H, L], kvalid
// [S / H, Nk] nullable.
hipError_t launch_exact_attention(const void *Q, const void *K, const void *V, int S, int L,
                                  int Nk, bool causal, ca_dtype_t dt, const uint8_t *qvalid,
                                  const uint8_t *kvalid, int H, int G, void *out, hipStream_t st);

bool fused_supported(int L, int Kc);
hipError_t launch_fused_forward(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                                int iters, int radius, float alpha, const Variant &var,
                                ca_dtype_t dt, const uint8_t *valid, int H, int G, void *out,
                                int32_t *assign, hipStream_t st);

// C[z] = A . Bt[z]^T for z < count (bf16 bits, fp32 accumulation). a_heads:
// A is [B, H, L, 64] read as [B*L, 64 H]; c_heads: C[z] is written as
// [B, H, L, 64] from [B*L, 64 H]. N and K multiples of 64.
hipError_t launch_gemm_nt(const uint16_t *A, const uint16_t *const *Bt, uint16_t *const *C,
                          int count, int M, int N, int K, bool a_heads, bool c_heads, int L, int H,
                          hipStream_t st);
// dst[z] = src[z]^T for z < count; src [R, Cc], R and Cc multiples of 64.
hipError_t launch_transpose_bf16(const uint16_t *const *src, uint16_t *const *dst, int count,
                                 int R, int Cc, hipStream_t st);

}  // namespace ca
