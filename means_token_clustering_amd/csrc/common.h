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

}  // namespace ca
