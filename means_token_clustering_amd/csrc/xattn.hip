// Centroid cross-attention (staged path, any L):
//   Vc_k = sum_j softmax_j(mu_k . k_j / sqrt(d)) v_j over all L keys
// (model card "Hooshaai/distilbert-sst2-cluster-attention", Architecture
// Overview figure, Softmax(mu K^T / 8) V with d = 64; "ClusterFormer" spec 3).
//
// Work split: the keys of a slice are cut into `nsplit` contiguous ranges
// (a multiple of 64 keys each); one workgroup per (slice, range, group of 16
// centroids) streams its keys through LDS in 64-row K/V tiles with an online
// (running max) softmax, 16 lanes per centroid. With one range the result is
// written directly; otherwise each range stores (max, sum, acc) and a
// combine kernel merges the ranges in range order (deterministic).
//
// Key-padding mask (optional; ClusterAttention listing on the
// "Hooshaai/svd-sst2-roberta-cluster" page, forward, bidirectional branch):
// a key with valid[b * L + j] == 0 takes the logit -10000 (b = s / H).
//
// stats (optional, [S, Kc, 2]): each row's largest scaled logit m and
// sum_j exp(logit_j - m), which the backward pass uses to rebuild the
// probabilities.
#include "launch.h"

namespace ca {

constexpr int kKeyTile = 64;
constexpr int kXPad = kD + 1;
constexpr int kChunk = 16;               // centroids per pass
constexpr int kPartStride = kD + 2;      // acc[64], max, sum

int xattn_splits(long S, int L) {
    // enough (slice, range) workgroups to fill the chip (about 1024), at
    // most one range per 64-key tile and 64 ranges per slice
    const long tiles = (L + kKeyTile - 1) / kKeyTile;
    const long want = (1024 + S - 1) / S;
    long split = tiles < want ? tiles : want;
    return (int)(split < 64 ? split : 64);
}

static int keys_per_split(int L, int nsplit) {
    const int tiles = (L + kKeyTile - 1) / kKeyTile;
    const int tps = (tiles + nsplit - 1) / nsplit;
    return tps * kKeyTile;
}

template <typename T>
__global__ __launch_bounds__(256) void centroid_xattn_kernel(
    const float *__restrict__ mu, const T *__restrict__ Kx, const T *__restrict__ Vx, int L,
    int Kc, int nsplit, int kps, const uint8_t *__restrict__ valid, int H, int G,
    float *__restrict__ vcent, float *__restrict__ part, float *__restrict__ stats) {
    __shared__ float sm_k[kKeyTile * kXPad];
    __shared__ float sm_v[kKeyTile * kXPad];
    __shared__ float sm_mu[kChunk * kXPad];
    __shared__ float sm_p[kChunk * kKeyTile];
    __shared__ uint8_t sm_ok[kKeyTile];

    const int tid = threadIdx.x;
    const int nchunk = (Kc + kChunk - 1) / kChunk;
    const int chunk = blockIdx.x % nchunk;
    const int split = (blockIdx.x / nchunk) % nsplit;
    const long s = blockIdx.x / nchunk / nsplit;
    const int j0 = split * kps;
    const int j1 = min(L, j0 + kps);
    const long skv = kv_slice(s, H, G);
    const T *Ks = Kx + skv * (long)L * kD;
    const T *Vs = Vx + skv * (long)L * kD;
    const int cl = tid >> 4, t = tid & 15;
    const float scale = 1.0f / sqrtf((float)kD);

    {
        const int c0 = chunk * kChunk;
        const int ck = min(kChunk, Kc - c0);
        __syncthreads();
        for (int e = tid; e < ck * (kD / 4); e += 256) {
            const int k = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
            float4 v = load4<float>(mu + (s * Kc + c0 + k) * kD + c4);
            float *dst = sm_mu + k * kXPad + c4;
            dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
        }
        float m = -__builtin_inff(), l = 0.f;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int jt = j0; jt < j1; jt += kKeyTile) {
            const int nk = min(kKeyTile, j1 - jt);
            __syncthreads();
            for (int e = tid; e < nk * (kD / 4); e += 256) {
                const int r = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
                float4 kv = load4<T>(Ks + (long)(jt + r) * kD + c4);
                float4 vv = load4<T>(Vs + (long)(jt + r) * kD + c4);
                float *dk = sm_k + r * kXPad + c4;
                float *dv = sm_v + r * kXPad + c4;
                dk[0] = kv.x; dk[1] = kv.y; dk[2] = kv.z; dk[3] = kv.w;
                dv[0] = vv.x; dv[1] = vv.y; dv[2] = vv.z; dv[3] = vv.w;
            }
            for (int r = tid; r < nk; r += 256)
                sm_ok[r] = valid == nullptr || valid[(s / H) * L + jt + r] != 0;
            __syncthreads();
            float sc[4];
            float mt = -__builtin_inff();
            const float *mr = sm_mu + cl * kXPad;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int key = t + 16 * u;
                if (key < nk && cl < ck) {
                    const float *kr = sm_k + key * kXPad;
                    const float dot = dot64(mr, kr);
                    sc[u] = sm_ok[key] ? dot * scale : -10000.f;
                } else {
                    sc[u] = -__builtin_inff();
                }
                mt = fmaxf(mt, sc[u]);
            }
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
            const float mn = fmaxf(m, mt);
            const float corr = (m == -__builtin_inff()) ? 0.f : exp_f32(m - mn);
            float ls = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float p = (sc[u] == -__builtin_inff()) ? 0.f : exp_f32(sc[u] - mn);
                sm_p[cl * kKeyTile + t + 16 * u] = p;
                ls += p;
            }
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) ls += __shfl_xor(ls, off);
            l = l * corr + ls;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] *= corr;
            m = mn;
            __syncthreads();
            const float *pr = sm_p + cl * kKeyTile;
            for (int key = 0; key < nk; ++key) {
                const float p = pr[key];
                const float *vr = sm_v + key * kXPad + 4 * t;
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = fmaf(p, vr[q], acc[q]);
            }
        }
        if (cl < ck) {
            const long k = s * Kc + c0 + cl;
            if (nsplit == 1) {
                const float inv = 1.0f / l;
#pragma unroll
                for (int q = 0; q < 4; ++q) vcent[k * kD + 4 * t + q] = acc[q] * inv;
                if (stats && t == 0) { stats[2 * k] = m; stats[2 * k + 1] = l; }
            } else {
                float *pp = part + ((s * nsplit + split) * (long)Kc + c0 + cl) * kPartStride;
#pragma unroll
                for (int q = 0; q < 4; ++q) pp[4 * t + q] = acc[q];
                if (t == 0) { pp[kD] = m; pp[kD + 1] = l; }
            }
        }
    }
}

// Merge key ranges in range order: M = max m_r, out = sum e^(m_r-M) acc_r /
// sum e^(m_r-M) l_r.
__global__ __launch_bounds__(256) void xattn_combine_kernel(const float *__restrict__ part,
                                                            int nsplit, int Kc, long total,
                                                            float *__restrict__ vcent,
                                                            float *__restrict__ stats) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const long sk = e / kD;           // s * Kc + k
    const int j = (int)(e % kD);
    const long s = sk / Kc, k = sk % Kc;
    float M = -__builtin_inff();
    for (int r = 0; r < nsplit; ++r)
        M = fmaxf(M, part[((s * nsplit + r) * Kc + k) * kPartStride + kD]);
    float num = 0.f, den = 0.f;
    for (int r = 0; r < nsplit; ++r) {
        const float *pp = part + ((s * nsplit + r) * Kc + k) * kPartStride;
        const float w = exp_f32(pp[kD] - M);
        num = fmaf(w, pp[j], num);
        den = fmaf(w, pp[kD + 1], den);
    }
    vcent[e] = num / den;
    if (stats && j == 0) { stats[2 * sk] = M; stats[2 * sk + 1] = den; }
}

template <typename T>
static hipError_t xattn_dispatch(const float *mu, const void *K, const void *V, int S, int L,
                                 int Kc, const uint8_t *valid, int H, int G, float *vcent,
                                 float *partials, float *stats, hipStream_t st) {
    const int nsplit = xattn_splits(S, L);
    const int kps = keys_per_split(L, nsplit);
    const int used = (L + kps - 1) / kps;   // ranges that hold keys
    const int nchunk = (Kc + kChunk - 1) / kChunk;
    const dim3 grid((unsigned)((long)S * used * nchunk)), block(256);
    hipLaunchKernelGGL(centroid_xattn_kernel<T>, grid, block, 0, st, mu,
                       static_cast<const T *>(K), static_cast<const T *>(V), L, Kc, used, kps,
                       valid, H, G, vcent, partials, stats);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || used == 1) return err;
    const long total = (long)S * Kc * kD;
    hipLaunchKernelGGL(xattn_combine_kernel, dim3((unsigned)((total + 255) / 256)), block, 0, st,
                       partials, used, Kc, total, vcent, stats);
    return hipGetLastError();
}

hipError_t launch_centroid_xattn(const float *mu, const void *K, const void *V, int S, int L,
                                 int Kc, ca_dtype_t dt, const uint8_t *valid, int H, int G,
                                 float *vcent, float *partials, hipStream_t st, float *stats) {
    if (dt == CA_BF16)
        return xattn_dispatch<bf16_t>(mu, K, V, S, L, Kc, valid, H, G, vcent, partials, stats,
                                      st);
    return xattn_dispatch<float>(mu, K, V, S, L, Kc, valid, H, G, vcent, partials, stats, st);
}

}  // namespace ca
