// Local sliding-window attention with the fused gather + convex-fusion
// epilogue (staged path, any L).
//
// Branch: model card "Hooshaai/distilbert-sst2-cluster-attention",
// Architecture Overview figure (LocalAttn(Q, K, V, W=32), then
// O = (1 - alpha) V^gathered + alpha O^local with V^gathered_i = Vc_{c_i});
// "ClusterFormer" spec 3 (band-masked attention) and 4 (2W+1 band). Window
// reading used throughout the library: key j belongs to query i iff
// |i - j| <= r, clipped to [0, L), with r = floor(W/2) (r = W in the
// ClusterAttention listing's band).
//
// Work split: one workgroup per 64-query tile; the tile's keys
// [i0 - r, i0 + 63 + r] stream through LDS in 64-row K/V tiles (the halo).
// Four lanes share a query, each holding 16 of its 64 dims: partial dot
// products meet through two butterfly adds that every lane performs in the
// same order, so all four see the same score. Scores of one key tile go to
// LDS, then an online softmax folds the tile in.
//
// Key-padding mask (optional; ClusterAttention listing on the
// "Hooshaai/svd-sst2-roberta-cluster" page, forward, bidirectional branch):
// a key with valid[b * L + j] == 0 takes the logit -10000 inside the window,
// and the fused output row of a padded query is zero (b = s / H).
//
// Soft gather (the same listing's forward): with mu given, the gathered
// context of query i is sum_k softmax_k(q_i . mu_k / sqrt(d)) vcent_k,
// folded in 64-centroid chunks staged through LDS with an online softmax.
#include "launch.h"

namespace ca {

constexpr int kQTile = 64;
constexpr int kLTile = 64;
constexpr int kLPad = kD + 1;   // LDS stride of the per-query score rows
constexpr int kLRow = kD;       // LDS stride of K/V rows (a whole wave reads one row)

template <typename T, bool FUSE, bool SOFT>
__global__ __launch_bounds__(256) void local_window_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx, int L, int r,
    int ntile, const float *__restrict__ vcent, const int32_t *__restrict__ assign, int Kc,
    float alpha, const uint8_t *__restrict__ valid, int H, int G, T *__restrict__ out,
    float *__restrict__ oloc, const float *__restrict__ mu) {
    __shared__ __align__(16) float sm_k[kLTile * kLRow];
    __shared__ __align__(16) float sm_v[kLTile * kLRow];
    __shared__ float sm_s[kQTile * kLPad];
    __shared__ uint8_t sm_ok[kLTile];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x % ntile;
    const long s = blockIdx.x / ntile;
    const long base = s * (long)L * kD;
    const long kvbase = kv_slice(s, H, G) * (long)L * kD;
    const int i0 = tile * kQTile;
    const int nq = min(kQTile, L - i0);
    const int qi = tid >> 2, g = tid & 3;
    const int i = i0 + qi;
    const bool active = qi < nq;
    // window of this query and of the whole tile (64-bit: r may be huge)
    const int lo = (int)max(0L, (long)i - r);
    const int hi = (int)min((long)L - 1, (long)i + r);
    const int tlo = (int)max(0L, (long)i0 - r);
    const int thi = (int)min((long)L, (long)i0 + nq + r);   // exclusive
    const float scale = 1.0f / sqrtf((float)kD);

    float qr[16];
    if (active) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float4 v = load4<T>(Q + base + (long)i * kD + 16 * g + 4 * c);
            qr[4 * c] = v.x * scale; qr[4 * c + 1] = v.y * scale;
            qr[4 * c + 2] = v.z * scale; qr[4 * c + 3] = v.w * scale;
        }
    } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) qr[c] = 0.f;
    }
    float m = -__builtin_inff(), l = 0.f;
    float acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = 0.f;

    for (int jt = tlo; jt < thi; jt += kLTile) {
        const int nk = min(kLTile, thi - jt);
        __syncthreads();
        for (int e = tid; e < nk * (kD / 4); e += 256) {
            const int rr = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
            float4 kv = load4<T>(Kx + kvbase + (long)(jt + rr) * kD + c4);
            float4 vv = load4<T>(Vx + kvbase + (long)(jt + rr) * kD + c4);
            float *dk = sm_k + rr * kLRow + c4;
            float *dv = sm_v + rr * kLRow + c4;
            dk[0] = kv.x; dk[1] = kv.y; dk[2] = kv.z; dk[3] = kv.w;
            dv[0] = vv.x; dv[1] = vv.y; dv[2] = vv.z; dv[3] = vv.w;
        }
        for (int rr = tid; rr < nk; rr += 256)
            sm_ok[rr] = valid == nullptr || valid[(s / H) * L + jt + rr] != 0;
        __syncthreads();
        // keys of this tile inside this query's window
        const int a = active ? max(lo, jt) - jt : 0;
        const int b = active ? min(hi, jt + nk - 1) - jt : -1;   // inclusive
        // the four lanes of a query share a and b, so the shuffles below
        // stay within converged groups; loop bounds of the wave are the
        // union of its queries' ranges
        const int wa = wave_min_i32(a < b + 1 ? a : kLTile);
        const int wb = wave_max_i32(b);
        float mt = -__builtin_inff();
        for (int key = wa; key <= wb; ++key) {
            const float *kr = sm_k + key * kLRow + 16 * g;
            float sc = quad_sum(dot16(qr, kr));
            if (!sm_ok[key]) sc = -10000.f;
            if (key >= a && key <= b) {
                mt = fmaxf(mt, sc);
                if (g == 0) sm_s[qi * kLPad + key] = sc;
            }
        }
        __syncthreads();
        if (b >= a) {
            const float mn = fmaxf(m, mt);
            const float corr = (m == -__builtin_inff()) ? 0.f : exp_f32(m - mn);
            l *= corr;
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[c] *= corr;
            for (int key = a; key <= b; ++key) {
                const float p = exp_f32(sm_s[qi * kLPad + key] - mn);
                l += p;
                const float *vr = sm_v + key * kLRow + 16 * g;
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[c] = fmaf(p, vr[c], acc[c]);
            }
            m = mn;
        }
    }
    float gsoft[16];
    if (SOFT) {
        // centroids and their contexts in chunks of 64 rows (sm_k, sm_v)
        float m2 = -__builtin_inff(), l2 = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) gsoft[c] = 0.f;
        for (int k0 = 0; k0 < Kc; k0 += kLTile) {
            const int nk = min(kLTile, Kc - k0);
            __syncthreads();
            for (int e = tid; e < nk * (kD / 4); e += 256) {
                const int rr = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
                const float4 mv = load4<float>(mu + (s * Kc + k0 + rr) * kD + c4);
                const float4 gv = load4<float>(vcent + (s * Kc + k0 + rr) * kD + c4);
                float *dm = sm_k + rr * kLRow + c4;
                float *dg = sm_v + rr * kLRow + c4;
                dm[0] = mv.x; dm[1] = mv.y; dm[2] = mv.z; dm[3] = mv.w;
                dg[0] = gv.x; dg[1] = gv.y; dg[2] = gv.z; dg[3] = gv.w;
            }
            __syncthreads();
            float mt = -__builtin_inff();
            for (int k = 0; k < nk; ++k) {   // every lane runs every k: shuffles converge
                const float *mr = sm_k + k * kLRow + 16 * g;
                const float sc = quad_sum(dot16(qr, mr));
                mt = fmaxf(mt, sc);
                if (g == 0) sm_s[qi * kLPad + k] = sc;
            }
            __syncthreads();
            const float mn = fmaxf(m2, mt);
            const float corr = (m2 == -__builtin_inff()) ? 0.f : exp_f32(m2 - mn);
            l2 *= corr;
#pragma unroll
            for (int c = 0; c < 16; ++c) gsoft[c] *= corr;
            for (int k = 0; k < nk; ++k) {
                const float p = exp_f32(sm_s[qi * kLPad + k] - mn);
                l2 += p;
                const float *gr = sm_v + k * kLRow + 16 * g;
#pragma unroll
                for (int c = 0; c < 16; ++c) gsoft[c] = fmaf(p, gr[c], gsoft[c]);
            }
            m2 = mn;
        }
        const float iz = 1.0f / l2;
#pragma unroll
        for (int c = 0; c < 16; ++c) gsoft[c] *= iz;
    }
    if (!active) return;
    const float inv = 1.0f / l;
    const long o = base + (long)i * kD + 16 * g;
    if (FUSE) {
        const int c = SOFT ? 0 : assign[s * L + i];
        const float *gv = SOFT ? gsoft : vcent + (s * Kc + c) * kD + 16 * g;
        const bool keep = valid == nullptr || valid[(s / H) * L + i] != 0;
        const float wg = keep ? 1.0f - alpha : 0.f;
        const float wl = keep ? alpha : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 v;
            v.x = wg * gv[4 * q + 0] + wl * (acc[4 * q + 0] * inv);
            v.y = wg * gv[4 * q + 1] + wl * (acc[4 * q + 1] * inv);
            v.z = wg * gv[4 * q + 2] + wl * (acc[4 * q + 2] * inv);
            v.w = wg * gv[4 * q + 3] + wl * (acc[4 * q + 3] * inv);
            store4<T>(out + o + 4 * q, v);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 v = make_float4(acc[4 * q] * inv, acc[4 * q + 1] * inv, acc[4 * q + 2] * inv,
                                   acc[4 * q + 3] * inv);
            store4<float>(oloc + o + 4 * q, v);
        }
    }
}

// out = (1 - alpha) vcent[assign] + alpha oloc, one thread per 4 elements.
template <typename T>
__global__ __launch_bounds__(256) void gather_fuse_kernel(const float *__restrict__ vcent,
                                                          const int32_t *__restrict__ assign,
                                                          const float *__restrict__ oloc,
                                                          int L, int Kc, float alpha, long total4,
                                                          T *__restrict__ out) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= total4) return;
    const long row = e / (kD / 4);       // s * L + i
    const int c4 = (int)(e % (kD / 4)) * 4;
    const long s = row / L;
    const int c = min(max(assign[row], 0), Kc - 1);   // clamp a caller's bad index
    const float4 gv = load4<float>(vcent + (s * Kc + c) * kD + c4);
    const float4 lv = load4<float>(oloc + row * kD + c4);
    const float wg = 1.0f - alpha;
    float4 v;
    v.x = wg * gv.x + alpha * lv.x;
    v.y = wg * gv.y + alpha * lv.y;
    v.z = wg * gv.z + alpha * lv.z;
    v.w = wg * gv.w + alpha * lv.w;
    store4<T>(out + row * kD + c4, v);
}

template <typename T>
static hipError_t local_dispatch(const void *Q, const void *K, const void *V, int S, int L, int r,
                                 const float *vcent, const int32_t *assign, int Kc, float alpha,
                                 const uint8_t *valid, int H, int G, void *out, float *oloc,
                                 const float *mu, hipStream_t st) {
    const int ntile = (L + kQTile - 1) / kQTile;
    const dim3 grid((unsigned)((long)S * ntile)), block(256);
    const T *q = static_cast<const T *>(Q);
    const T *k = static_cast<const T *>(K);
    const T *v = static_cast<const T *>(V);
    if (oloc == nullptr && mu != nullptr)
        hipLaunchKernelGGL((local_window_kernel<T, true, true>), grid, block, 0, st, q, k, v, L, r,
                           ntile, vcent, assign, Kc, alpha, valid, H, G, static_cast<T *>(out),
                           oloc, mu);
    else if (oloc == nullptr)
        hipLaunchKernelGGL((local_window_kernel<T, true, false>), grid, block, 0, st, q, k, v, L, r,
                           ntile, vcent, assign, Kc, alpha, valid, H, G, static_cast<T *>(out),
                           oloc, mu);
    else
        hipLaunchKernelGGL((local_window_kernel<T, false, false>), grid, block, 0, st, q, k, v, L,
                           r, ntile, vcent, assign, Kc, alpha, valid, H, G, static_cast<T *>(out),
                           oloc, mu);
    return hipGetLastError();
}

hipError_t launch_local_window(const void *Q, const void *K, const void *V, int S, int L, int r,
                               ca_dtype_t dt, const float *vcent, const int32_t *assign, int Kc,
                               float alpha, const uint8_t *valid, int H, int G, void *out,
                               float *oloc, hipStream_t st, const float *mu) {
    if (dt == CA_BF16)
        return local_dispatch<bf16_t>(Q, K, V, S, L, r, vcent, assign, Kc, alpha, valid, H, G,
                                      out, oloc, mu, st);
    return local_dispatch<float>(Q, K, V, S, L, r, vcent, assign, Kc, alpha, valid, H, G, out,
                                 oloc, mu, st);
}

hipError_t launch_gather_fuse(const float *vcent, const int32_t *assign, const float *oloc, int S,
                              int L, int Kc, float alpha, ca_dtype_t dt, void *out,
                              hipStream_t st) {
    const long total4 = (long)S * L * (kD / 4);
    const dim3 grid((unsigned)((total4 + 255) / 256)), block(256);
    if (dt == CA_BF16)
        hipLaunchKernelGGL(gather_fuse_kernel<bf16_t>, grid, block, 0, st, vcent, assign, oloc, L,
                           Kc, alpha, total4, static_cast<bf16_t *>(out));
    else
        hipLaunchKernelGGL(gather_fuse_kernel<float>, grid, block, 0, st, vcent, assign, oloc, L,
                           Kc, alpha, total4, static_cast<float *>(out));
    return hipGetLastError();
}

}  // namespace ca
