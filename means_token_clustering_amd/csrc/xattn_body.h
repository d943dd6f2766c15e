// The centroid cross-attention of one 128-key range on the fp16 matrix cores
// (its LDS layout and xattn_range), shared by xattn_mfma_kernel and the
// clustering launch that forms the key ranges after the Lloyd iterations
// (kmeans_slice.hip). The operation and the arithmetic are described in
// xattn.hip.
#pragma once
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
// all 64 centroids at once (K64): the tensor maxima, then the centroid
// planes [64][64] h, m, then the softmax statistics [64][8] share the region
// after V; the P planes [64][128] h, m take the K region once the scores
// are formed
constexpr int kX64MuPlane = 64 * kD * 2;               // one fp16 plane [64][64]
constexpr int kX64PPlane = 64 * kFL * 2;               // one fp16 plane [64][128]
constexpr int kX64Lds = kXOffMu + 2 * kX64MuPlane;
static_assert(2 * kX64PPlane <= kXOffV && kX64Lds <= 81920, "two workgroups per CU");

}  // namespace

// K64: Kc in 49 .. 64, every centroid in one pass (fewer barriers, the four
// groups' score chains independent, V^T P^T on all eight waves); the same
// arithmetic in the same order as the group-by-group pass. FULLR: L is a
// multiple of 128, so every range holds 128 keys (no bounds tests).
// One key range (split) of slice s by 512 threads (tid) with kXLdsM bytes of
// LDS at smem (kX64Lds with K64); mu_s: the slice's Kc fp32 centroid rows
// (global memory or LDS). Every call passes the same sequence of workgroup
// barriers, so two halves of a 1,024-thread workgroup may run two ranges.
template <typename T, bool MASKED, bool K64, bool FULLR>
__device__ __forceinline__ void xattn_range(
    const float *__restrict__ mu_s, const T *__restrict__ Kx, const T *__restrict__ Vx, int L, int Kc,
    int nsplit, const uint8_t *__restrict__ valid, int H, int G, float *__restrict__ vcent,
    float *__restrict__ part, float *__restrict__ stats, unsigned char *smem, int tid, long s,
    int split) {
    uint16_t *sK = reinterpret_cast<uint16_t *>(smem + kXOffK);
    uint16_t *sV = reinterpret_cast<uint16_t *>(smem + kXOffV);
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kXOffMu);
    uint16_t *sP = reinterpret_cast<uint16_t *>(smem + kXOffP);
    float *sXm = reinterpret_cast<float *>(smem + kXOffXm);
    float *sXl = reinterpret_cast<float *>(smem + kXOffXl);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + (K64 ? kXOffMu : kXOffMax));
    const u8 *pK = smem + kXOffK, *pV = smem + kXOffV, *pMu = smem + kXOffMu, *pP = smem + kXOffP;

    constexpr bool kZ = bf16_storage<T>();   // Q (K, V) planes with zero m parts
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int j0 = 128 * split;                    // first key of the range
    const int nk = FULLR ? 128 : min(128, L - j0);
    const long kvrow = kv_slice(s, H, G) * (long)L + j0;
    const LaneOffs lo = lane_offsets(l16, g);
    const int trq0 = 1024 * g + (lo.tr0 ^ (32 * (w & 3)));
    const int trq1 = 1024 * g + (lo.tr4 ^ (32 * (w & 3)));

    // ------------------------------------------------------------ K, V planes
    float kraw[2][8], vraw[2][8];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;   // row it / 8, dims 8 (it % 8) ..
        load_row8<T, FULLR>(Kx + kvrow * kD, it >> 3, nk, (it & 7) * 8, kraw[n]);
        load_row8<T, FULLR>(Vx + kvrow * kD, it >> 3, nk, (it & 7) * 8, vraw[n]);
    }
    // the slice's first 64 centroid rows: row tid / 8, dims 8 (tid % 8) ..
    // (zeros past Kc), requested with K and V so that every group of 16
    // takes its planes from registers
    float mraw[8];
    {
        const int r = tid >> 3, c = (tid & 7) * 8;
        if (r < Kc) {
            load8<float>(mu_s + r * kD + c, mraw);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) mraw[i] = 0.f;
        }
    }
    float mm = absmax8(mraw, 0.f);   // largest |mu| of the slice
    for (int e = kThreads * 2 + tid; e < Kc * (kD / 4); e += kThreads) {
        const float4 v = load4<float>(mu_s + 4 * e);
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
            if (!kZ) st16(sK + kPlaneE + o, kp.m);   // zero for bf16 storage, never read
            st16(sV + o, vp.h);
            if (!kZ) st16(sV + kPlaneE + o, vp.m);   // zero for bf16 storage, never read
        }
    }
    const float sscale2 = __builtin_ldexpf(0.125f, smu + sk) * 1.4426950408889634f;
    const float fmu = __builtin_ldexpf(1.f, -smu), vunscale = __builtin_ldexpf(1.f, sv);
    const int nch = (nk + 31) >> 5;

    if constexpr (K64) {
        __syncthreads();   // K and V planes written; every wave has read the maxima
        {   // centroid row tid / 8, dims 8 (tid % 8) .. (zero rows past Kc)
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = mraw[i] * fmu;
            const Sp8 mp = split8(x);
            const int o = off64(tid >> 3, (tid & 7) * 8);
            st16(sMu + o, mp.h);
            st16(sMu + kX64MuPlane / 2 + o, mp.m);
        }
        __syncthreads();
        // scores of key tile w against the four groups: a[kg][rr] =
        // k_{16w+4g+rr} . mu_{16kg+l16} (scaled units), base-2 logits
        float sx[4][4], M[4];
        {
            const Sp8 ka = frag_at(pK, kPlane, 2048 * w + lo.rl64);
            const Sp8 kc = frag_at(pK, kPlane, 2048 * w + (lo.rl64 ^ 64));
            f32x4_t a[4];
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) {
                const Sp8 ma = frag_at(pMu, kX64MuPlane, 2048 * kg + lo.rl64);
                const Sp8 mc = frag_at(pMu, kX64MuPlane, 2048 * kg + (lo.rl64 ^ 64));
                a[kg] = mma3z<kZ, false>(ka, ma, kZero4);
                a[kg] = mma3z<kZ, false>(kc, mc, a[kg]);
            }
            const uint32_t nib = MASKED ? kb.tile(w) >> (4 * g) : 0xfu;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) {
                float mloc = -__builtin_inff();
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int key = 16 * w + 4 * g + rr;
                    const float v = (!MASKED || ((nib >> rr) & 1u)) ? a[kg][rr] * sscale2 : kPadLogit2;
                    sx[kg][rr] = key < nk ? v : -__builtin_inff();
                    mloc = fmaxf(mloc, sx[kg][rr]);
                }
                M[kg] = col_max(mloc);
            }
        }
        __syncthreads();   // the K and centroid planes are dead
        float *sYm = reinterpret_cast<float *>(smem + kXOffMu);   // [64][8] per-wave maxima
        float *sYl = sYm + 64 * 8;                                // [64][8] per-wave sums
        if (g == 0) {
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) sYm[(16 * kg + l16) * 8 + w] = M[kg];
        }
        __syncthreads();
        uint16_t *sP64 = reinterpret_cast<uint16_t *>(smem);   // in the K region
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
            const float4 m0 = *reinterpret_cast<const float4 *>(sYm + (16 * kg + l16) * 8);
            const float4 m1 = *reinterpret_cast<const float4 *>(sYm + (16 * kg + l16) * 8 + 4);
            M[kg] = fmaxf(fmaxf(fmaxf(m0.x, m0.y), fmaxf(m0.z, m0.w)),
                          fmaxf(fmaxf(m1.x, m1.y), fmaxf(m1.z, m1.w)));
            float p[4], ls = 0.f;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                p[rr] = __builtin_amdgcn_exp2f(sx[kg][rr] - M[kg]);   // exp2(-inf) = 0
                ls += p[rr];
            }
            ls = col_sum(ls);
            const Sp4 ps = split4(p[0], p[1], p[2], p[3]);
            const int o = off128(16 * kg + l16, 16 * w + 4 * g);   // P[centroid][keys 16w + 4g ..]
            st8(sP64 + o, ps.h);
            st8(sP64 + kX64PPlane / 2 + o, ps.m);
            if (g == 0) sYl[(16 * kg + l16) * 8 + w] = ls;
        }
        __syncthreads();
        // V^cent^T[dim 16 dt + 4g + rr][centroid 16 kg + l16] for dimension
        // tile dt = w % 4 and groups w / 4, w / 4 + 2
        const int dt = w & 3, kq = w >> 2;
        f32x4_t aA[2] = {kZero4, kZero4}, aB[2] = {kZero4, kZero4};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (c < nch) {
                const Sp8 vf = colfrag8_at(pV, 4096 * c + trq0, 4096 * c + trq1);
                const Sp8 pa = frag_at(smem, kX64PPlane, 4096 * kq + (lo.rl128 ^ (64 * c)));
                const Sp8 pb = frag_at(smem, kX64PPlane, 4096 * (kq + 2) + (lo.rl128 ^ (64 * c)));
                aA[c & 1] = mma3z<kZ, false>(vf, pa, aA[c & 1]);
                aB[c & 1] = mma3z<kZ, false>(vf, pb, aB[c & 1]);
            }
        }
        auto store = [&](int kg, f32x4_t a) {
            const float4 l0 = *reinterpret_cast<const float4 *>(sYl + (16 * kg + l16) * 8);
            const float4 l1 = *reinterpret_cast<const float4 *>(sYl + (16 * kg + l16) * 8 + 4);
            const float den = ((((((l0.x + l0.y) + l0.z) + l0.w) + l1.x) + l1.y) + l1.z) + l1.w;
            const int k = 16 * kg + l16;
            if (k >= Kc) return;
            const long row = s * Kc + k;
            const float mnat = M[kg] * 0.6931471805599453f;   // base-2 maximum in natural units
            if (nsplit == 1) {
                const float f = vunscale / den;
                *reinterpret_cast<float4 *>(vcent + row * kD + 16 * dt + 4 * g) =
                    make_float4(a[0] * f, a[1] * f, a[2] * f, a[3] * f);
                if (stats && dt == 0 && g == 0) {
                    stats[2 * row] = mnat;
                    stats[2 * row + 1] = den;
                }
            } else {
                float *pp = part + ((s * nsplit + split) * (long)Kc + k) * kXPartStride;
                *reinterpret_cast<float4 *>(pp + 16 * dt + 4 * g) =
                    make_float4(a[0] * vunscale, a[1] * vunscale, a[2] * vunscale, a[3] * vunscale);
                if (dt == 0 && g == 0) {
                    pp[kD] = mnat;
                    pp[kD + 1] = den;
                }
            }
        };
        store(kq, aA[0] + aA[1]);
        store(kq + 2, aB[0] + aB[1]);
        return;
    }

    // ------------------------------------------------------------ groups of 16 centroids
    for (int k0 = 0; k0 < Kc; k0 += kFK) {
        if (k0 < 64 && (tid >> 7) == (k0 >> 4)) {   // rows k0 .. k0 + 15 from registers
            const int r = (tid >> 3) - k0, c = (tid & 7) * 8;
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = mraw[i] * fmu;
            const Sp8 mp = split8(x);
            const int o = off64(r, c);
            st16(sMu + o, mp.h);
            st16(sMu + kPlaneMuE + o, mp.m);
        } else if (k0 >= 64 && tid < 128) {   // centroid row k0 + tid / 8, dims 8 (tid % 8) ..
            const int r = tid >> 3, c = (tid & 7) * 8;
            float x[8];
            if (k0 + r < Kc) {
                load8<float>(mu_s + (k0 + r) * kD + c, x);
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
            f32x4_t a = mma3z<kZ, false>(ka, ma, kZero4);
            a = mma3z<kZ, false>(kc, mc, a);
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
                    a2[c & 1] = mma3z<kZ, false>(vf, pf, a2[c & 1]);
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


}  // namespace ca
