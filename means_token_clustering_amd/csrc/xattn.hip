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
#include "launch.h"
#include "mfma_split.h"

namespace ca {
namespace {

constexpr int kXOffK = 0;
constexpr int kXOffV = 2 * kPlane;
constexpr int kXOffMu = 4 * kPlane;                  // [16][64] h, m
constexpr int kXOffP = kXOffMu + 2 * kPlaneMu;       // [16][128] h, m
constexpr int kXOffXm = kXOffP + 2 * kPlaneRow;      // [16][8] per-wave maxima
constexpr int kXOffXl = kXOffXm + kFK * 8 * 4;       // [16][8] per-wave sums
constexpr int kXOffMax = kXOffXl + kFK * 8 * 4;      // [8][4] tensor maxima, mask words
constexpr int kXLdsM = kXOffMax + 8 * 4 * 4;
static_assert(kXLdsM <= 81920, "two workgroups per CU");

}  // namespace

template <typename T, bool MASKED>
__global__ __launch_bounds__(kThreads, 4) void xattn_mfma_kernel(
    const float *__restrict__ mu, const T *__restrict__ Kx, const T *__restrict__ Vx, int L,
    int Kc, int nsplit, const uint8_t *__restrict__ valid, int H, int G,
    float *__restrict__ vcent, float *__restrict__ part, float *__restrict__ stats) {
    __shared__ __align__(16) unsigned char smem[kXLdsM];
    uint16_t *sK = reinterpret_cast<uint16_t *>(smem + kXOffK);
    uint16_t *sV = reinterpret_cast<uint16_t *>(smem + kXOffV);
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kXOffMu);
    uint16_t *sP = reinterpret_cast<uint16_t *>(smem + kXOffP);
    float *sXm = reinterpret_cast<float *>(smem + kXOffXm);
    float *sXl = reinterpret_cast<float *>(smem + kXOffXl);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kXOffMax);
    const u8 *pK = smem + kXOffK, *pV = smem + kXOffV, *pMu = smem + kXOffMu, *pP = smem + kXOffP;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int split = blockIdx.x % nsplit;
    const long s = blockIdx.x / nsplit;
    const int j0 = 128 * split;                    // first key of the range
    const int nk = min(128, L - j0);
    const long kvrow = kv_slice(s, H, G) * (long)L + j0;
    const LaneOffs lo = lane_offsets(l16, g);
    const int trq0 = 1024 * g + (lo.tr0 ^ (32 * (w & 3)));
    const int trq1 = 1024 * g + (lo.tr4 ^ (32 * (w & 3)));

    // ------------------------------------------------------------ K, V planes
    float kraw[2][8], vraw[2][8];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;   // row it / 8, dims 8 (it % 8) ..
        load_row8<T, false>(Kx + kvrow * kD, it >> 3, nk, (it & 7) * 8, kraw[n]);
        load_row8<T, false>(Vx + kvrow * kD, it >> 3, nk, (it & 7) * 8, vraw[n]);
    }
    float mm = 0.f;   // largest |mu| of the slice
    for (int e = tid; e < Kc * (kD / 4); e += kThreads) {
        const float4 v = load4<float>(mu + s * (long)Kc * kD + 4 * e);
        mm = fmaxf(mm, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    {
        const uint32_t bk = wave_max_u(__float_as_uint(absmax8(kraw[1], absmax8(kraw[0], 0.f))));
        const uint32_t bv = wave_max_u(__float_as_uint(absmax8(vraw[1], absmax8(vraw[0], 0.f))));
        const uint32_t bm = wave_max_u(__float_as_uint(mm));
        if (lane == 0) {
            sMax[4 * w] = bk;
            sMax[4 * w + 1] = bv;
            sMax[4 * w + 2] = bm;
        }
    }
    if (MASKED && w < 2) {   // keys j0 + 64w .. of the range, words 2w and 2w+1
        const int j = 64 * w + lane;
        const uint64_t bits = __ballot(j < nk && valid[(s / H) * (long)L + j0 + j] != 0);
        if (lane == 0) {
            sMax[4 * (2 * w) + 3] = (uint32_t)bits;
            sMax[4 * (2 * w + 1) + 3] = (uint32_t)(bits >> 32);
        }
    }
    __syncthreads();
    uint32_t mk = 0, mv = 0, mmu = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) {
        mk = max(mk, sMax[4 * ww]);
        mv = max(mv, sMax[4 * ww + 1]);
        mmu = max(mmu, sMax[4 * ww + 2]);
    }
    KeyBits kb;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        kb.w[k] = MASKED ? (uint32_t)__builtin_amdgcn_readfirstlane((int)sMax[4 * k + 3]) : ~0u;
    const int sk = scale_shift(mk, kKVLimit), sv = scale_shift(mv, kKVLimit);
    const int smu = scale_shift(mmu, kQLimit);
    {
        const float fk = __builtin_ldexpf(1.f, -sk), fv = __builtin_ldexpf(1.f, -sv);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int it = tid + kThreads * n;
            float x[8], y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] = kraw[n][i] * fk;
                y[i] = vraw[n][i] * fv;
            }
            const Sp8 kp = split8(x), vp = split8(y);
            const int o = off64(it >> 3, (it & 7) * 8);
            st16(sK + o, kp.h);
            st16(sK + kPlaneE + o, kp.m);
            st16(sV + o, vp.h);
            st16(sV + kPlaneE + o, vp.m);
        }
    }
    const float sscale2 = __builtin_ldexpf(0.125f, smu + sk) * 1.4426950408889634f;
    const float fmu = __builtin_ldexpf(1.f, -smu), vunscale = __builtin_ldexpf(1.f, sv);
    const int nch = (nk + 31) >> 5;

    // ------------------------------------------------------------ groups of 16 centroids
    for (int k0 = 0; k0 < Kc; k0 += kFK) {
        if (tid < 128) {   // centroid row k0 + tid / 8, dims 8 (tid % 8) ..
            const int r = tid >> 3, c = (tid & 7) * 8;
            float x[8];
            if (k0 + r < Kc) {
                load8<float>(mu + (s * Kc + k0 + r) * kD + c, x);
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] *= fmu;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = 0.f;
            }
            const Sp8 mp = split8(x);
            const int o = off64(r, c);
            st16(sMu + o, mp.h);
            st16(sMu + kPlaneMuE + o, mp.m);
        }
        __syncthreads();
        // scores of key tile w: a[rr] = k_{16w+4g+rr} . mu_{k0+l16} (scaled units)
        float sx[4];
        {
            const Sp8 ka = frag_at(pK, kPlane, 2048 * w + lo.rl64), ma = frag_at(pMu, kPlaneMu, lo.rl64);
            const Sp8 kc = frag_at(pK, kPlane, 2048 * w + (lo.rl64 ^ 64)), mc = frag_at(pMu, kPlaneMu, lo.rl64 ^ 64);
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t a = mma3(ka, ma, kZero4);
            a = mma3(kc, mc, a);
            const uint32_t nib = MASKED ? kb.tile(w) >> (4 * g) : 0xfu;
            float mloc = -__builtin_inff();
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = 16 * w + 4 * g + rr;
                const float v = (!MASKED || ((nib >> rr) & 1u)) ? a[rr] * sscale2 : kPadLogit2;
                sx[rr] = key < nk ? v : -__builtin_inff();
                mloc = fmaxf(mloc, sx[rr]);
            }
            mloc = col_max(mloc);
            if (g == 0) sXm[l16 * 8 + w] = mloc;
        }
        __syncthreads();
        float M;
        {
            const float4 m0 = *reinterpret_cast<const float4 *>(sXm + l16 * 8);
            const float4 m1 = *reinterpret_cast<const float4 *>(sXm + l16 * 8 + 4);
            M = fmaxf(fmaxf(fmaxf(m0.x, m0.y), fmaxf(m0.z, m0.w)),
                      fmaxf(fmaxf(m1.x, m1.y), fmaxf(m1.z, m1.w)));
            float p[4], ls = 0.f;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                p[rr] = __builtin_amdgcn_exp2f(sx[rr] - M);   // exp2(-inf) = 0
                ls += p[rr];
            }
            ls = col_sum(ls);
            const Sp4 ps = split4(p[0], p[1], p[2], p[3]);
            const int o = off128(l16, 16 * w + 4 * g);   // P[centroid l16][keys 16w + 4g ..]
            st8(sP + o, ps.h);
            st8(sP + kPlaneRowE + o, ps.m);
            if (g == 0) sXl[l16 * 8 + w] = ls;
        }
        __syncthreads();
        if (w < 4) {   // V^cent^T[dim 16w + 4g + rr][centroid l16] = sum over keys of V^T P^T
            f32x4_t a2[2] = {kZero4, kZero4};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c < nch) {
                    const Sp8 vf = colfrag8_at(pV, 4096 * c + trq0, 4096 * c + trq1);
                    const Sp8 pf = frag_at(pP, kPlaneRow, lo.rl128 ^ (64 * c));
                    a2[c & 1] = mma3(vf, pf, a2[c & 1]);
                }
            }
            const f32x4_t a = a2[0] + a2[1];
            const float4 l0 = *reinterpret_cast<const float4 *>(sXl + l16 * 8);
            const float4 l1 = *reinterpret_cast<const float4 *>(sXl + l16 * 8 + 4);
            const float den = ((((((l0.x + l0.y) + l0.z) + l0.w) + l1.x) + l1.y) + l1.z) + l1.w;
            const int k = k0 + l16;
            if (k < Kc) {
                const long row = s * Kc + k;
                const float mnat = M * 0.6931471805599453f;   // base-2 maximum in natural units
                if (nsplit == 1) {
                    const float f = vunscale / den;
                    *reinterpret_cast<float4 *>(vcent + row * kD + 16 * w + 4 * g) =
                        make_float4(a[0] * f, a[1] * f, a[2] * f, a[3] * f);
                    if (stats && w == 0 && g == 0) {
                        stats[2 * row] = mnat;
                        stats[2 * row + 1] = den;
                    }
                } else {
                    float *pp = part + ((s * nsplit + split) * (long)Kc + k) * kXPartStride;
                    *reinterpret_cast<float4 *>(pp + 16 * w + 4 * g) =
                        make_float4(a[0] * vunscale, a[1] * vunscale, a[2] * vunscale,
                                    a[3] * vunscale);
                    if (w == 0 && g == 0) {
                        pp[kD] = mnat;
                        pp[kD + 1] = den;
                    }
                }
            }
        }
    }
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
    if (valid)
        hipLaunchKernelGGL((xattn_mfma_kernel<T, true>), grid, block, 0, st, mu, k, v, L, Kc,
                           nsplit, valid, H, G, vcent, partials, stats);
    else
        hipLaunchKernelGGL((xattn_mfma_kernel<T, false>), grid, block, 0, st, mu, k, v, L, Kc,
                           nsplit, valid, H, G, vcent, partials, stats);
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
