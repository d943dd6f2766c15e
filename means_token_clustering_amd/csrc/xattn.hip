// Centroid cross-attention on the fp16 matrix cores (staged path, any L):
//   Vc_k = sum_j softmax_j(mu_k . k_j / sqrt(d)) v_j over all L keys
// (model card "Hooshaai/distilbert-sst2-cluster-attention", Architecture
// Overview figure, Softmax(mu K^T / 8) V with d = 64; "ClusterFormer" spec 3).
//
// Work split: one workgroup (8 waves) per (slice, range of 128 keys). The
// range's K and V rows are staged once as fp16 h/m planes; the centroids
// then pass through in groups of 16, each group in the single-launch
// forward's pattern: wave w scores key tile w against the group (three
// partial products per 32-deep chunk), the softmax maximum and sum are
// reduced across the waves through LDS, the probabilities go to LDS as fp16
// h/m planes [centroid][key], and waves 0-3 form V^T P^T for dimension tile
// w. With one range per slice the result is written directly; otherwise
// each range stores (max, sum, unnormalised row) in the layout of the
// scalar kernel, and xattn_combine_kernel merges the ranges in range order.
// Maxima are kept in natural-log units there (base-2 maxima times ln 2).
//
// Scaling as in the forward: K, V and the centroids by one power of two per
// tensor and workgroup; the factors are undone on the fp32 results.
//
// Key-padding mask (optional; ClusterAttention listing on the
// "Hooshaai/svd-sst2-roberta-cluster" page, forward, bidirectional branch):
// a padded key takes the logit -10000.
#include "xattn_body.h"

namespace ca {

template <typename T, bool MASKED, bool K64, bool FULLR>
__global__ __launch_bounds__(kThreads, 4) void xattn_mfma_kernel(
    const float *__restrict__ mu, const T *__restrict__ Kx, const T *__restrict__ Vx, int L,
    int Kc, int nsplit, const uint8_t *__restrict__ valid, int H, int G,
    float *__restrict__ vcent, float *__restrict__ part, float *__restrict__ stats) {
    __shared__ __align__(16) unsigned char smem[K64 ? kX64Lds : kXLdsM];
    const int split = blockIdx.x % nsplit;
    const long s = blockIdx.x / nsplit;
    xattn_range<T, MASKED, K64, FULLR>(mu + s * (long)Kc * kD, Kx, Vx, L, Kc, nsplit, valid, H,
                                       G, vcent, part, stats, smem, threadIdx.x, s, split);
}

// Merge key ranges in range order: M = max m_r, out = sum e^(m_r-M) acc_r /
// sum e^(m_r-M) l_r. One workgroup per centroid row, lane j = dimension j:
// wave q folds ranges q, q + 4, ... (eight loads in flight per lane) into
// (M_q, num_q, den_q), and wave 0 merges the four records in wave order.
__global__ __launch_bounds__(256) void xattn_combine_kernel(const float *__restrict__ part,
                                                            int nsplit, int Kc,
                                                            float *__restrict__ vcent,
                                                            float *__restrict__ stats) {
    __shared__ float rec[4][kD + 2];
    const int q = threadIdx.x >> 6, j = threadIdx.x & 63;
    const long sk = blockIdx.x;       // s * Kc + k
    const long s = sk / Kc, k = sk % Kc;
    const float *p0 = part + (s * nsplit * (long)Kc + k) * kXPartStride;
    const long rs = (long)Kc * kXPartStride;   // from one range to the next
    // one pass over the wave's ranges (r = q, q + 4, ...), eight loads of each
    // kind in flight, with a running maximum: a single pass up to 32 ranges
    float Mq = -__builtin_inff(), num = 0.f, den = 0.f;
    for (int r0 = q; r0 < nsplit; r0 += 32) {
        float m8[8], a8[8], l8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = r0 + 4 * u;
            const float *pp = p0 + (r < nsplit ? r : q) * rs;
            m8[u] = r < nsplit ? pp[kD] : -__builtin_inff();
            a8[u] = pp[j];
            l8[u] = pp[kD + 1];
        }
        float Mn = Mq;   // finite: range r0 exists
#pragma unroll
        for (int u = 0; u < 8; ++u) Mn = fmaxf(Mn, m8[u]);
        const float f = exp_f32(Mq - Mn);   // 0 on the first pass
        num *= f;
        den *= f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float w = exp_f32(m8[u] - Mn);   // 0 past the last range
            num = fmaf(w, a8[u], num);
            den = fmaf(w, l8[u], den);
        }
        Mq = Mn;
    }
    rec[q][j] = num;
    if (j == 0) {
        rec[q][kD] = Mq;
        rec[q][kD + 1] = den;
    }
    __syncthreads();
    if (q != 0) return;
    float M = rec[0][kD];
#pragma unroll
    for (int u = 1; u < 4; ++u) M = fmaxf(M, rec[u][kD]);
    float n = 0.f, d = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float f = exp_f32(rec[u][kD] - M);   // exp(-inf) = 0 for a wave without ranges
        n = fmaf(f, rec[u][j], n);
        d = fmaf(f, rec[u][kD + 1], d);
    }
    vcent[sk * kD + j] = n / d;
    if (stats && j == 0) { stats[2 * sk] = M; stats[2 * sk + 1] = d; }
}

static hipError_t launch_xattn_combine(const float *partials, long S, int nsplit, int Kc,
                                       float *vcent, float *stats, hipStream_t st) {
    hipLaunchKernelGGL(xattn_combine_kernel, dim3((unsigned)(S * Kc)), dim3(256), 0, st, partials,
                       nsplit, Kc, vcent, stats);
    return hipGetLastError();
}

int xattn_splits(int L) { return (L + 127) / 128; }

template <typename T>
static hipError_t xattn_mfma_dispatch(const float *mu, const void *K, const void *V, int S, int L,
                                      int Kc, const uint8_t *valid, int H, int G, float *vcent,
                                      float *partials, float *stats, bool combine,
                                      hipStream_t st) {
    const int nsplit = xattn_splits(L);
    const dim3 grid((unsigned)((long)S * nsplit)), block(kThreads);
    const T *k = static_cast<const T *>(K), *v = static_cast<const T *>(V);
#define CA_XA_LAUNCH(M, K64, F)                                                               \
    hipLaunchKernelGGL((xattn_mfma_kernel<T, M, K64, F>), grid, block, 0, st, mu, k, v, L, Kc, \
                       nsplit, valid, H, G, vcent, partials, stats)
#define CA_XA_LAUNCH_F(M, K64)                                                                \
    do {                                                                                      \
        if (L % 128 == 0) CA_XA_LAUNCH(M, K64, true); else CA_XA_LAUNCH(M, K64, false);       \
    } while (0)
    const bool k64 = Kc > 48 && Kc <= 64;
    if (valid) {
        if (k64) CA_XA_LAUNCH_F(true, true); else CA_XA_LAUNCH_F(true, false);
    } else {
        if (k64) CA_XA_LAUNCH_F(false, true); else CA_XA_LAUNCH_F(false, false);
    }
#undef CA_XA_LAUNCH_F
#undef CA_XA_LAUNCH
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || nsplit == 1 || !combine) return err;
    return launch_xattn_combine(partials, S, nsplit, Kc, vcent, stats, st);
}

hipError_t launch_centroid_xattn(const float *mu, const void *K, const void *V, int S, int L,
                                 int Kc, ca_dtype_t dt, const uint8_t *valid, int H, int G,
                                 float *vcent, float *partials, hipStream_t st, float *stats,
                                 bool combine) {
    if (dt == CA_BF16)
        return xattn_mfma_dispatch<bf16_t>(mu, K, V, S, L, Kc, valid, H, G, vcent, partials,
                                           stats, combine, st);
    return xattn_mfma_dispatch<float>(mu, K, V, S, L, Kc, valid, H, G, vcent, partials, stats,
                                      combine, st);
}

}  // namespace ca
