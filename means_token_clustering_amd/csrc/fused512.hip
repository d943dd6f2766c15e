// Single-launch cluster attention forward for 128 < L <= 512 tokens, K <= 16,
// window radius r <= 16, no key-padding mask: one workgroup of 16 waves per
// slice runs Lloyd's k-means, the centroid cross-attention, the local window
// branch and the gather + convex fusion, reading Q, K, V from HBM once each
// (K and V once more for the window's halo rows) and writing the output and
// the assignment.
//
// Method: model card "Hooshaai/distilbert-sst2-cluster-attention",
// Architecture Overview figure and Mathematical Formulation 1; "ClusterFormer"
// spec (svd-sst2-roberta-cluster page) 2.1 and 3. Conventions as in the other
// kernels: ties to the lowest cluster, empty cluster -> zero vector, window
// |i - j| <= r, scale 1/sqrt(d).
//
// Phases (wave w owns token tiles w and w + 16; the arithmetic is the
// single-launch forward's: fp16 h/m split planes, three partial products,
// base-2 softmax, power-of-two range scaling):
//   1. Lloyd's iterations as in kmeans_slice_kernel, with Q planes of 512
//      rows in LDS and the final centroids kept as planes.
//   2. Centroid attention over key chunks of 128: waves 0-7 and 8-15 each
//      take one chunk at a time (K, V planes with their own scales), the
//      forward's scores / softmax statistics / V^T P^T per chunk, and each
//      context wave folds its chunks into a running (max, sum, row); the two
//      halves meet in a fixed order.
//   3. Local window over two passes of 256 queries: the pass's rows with a
//      16-row halo (at most 288) as K, V planes, the forward's narrow window
//      routine per query tile, then the gather of (1 - alpha) V^cent_{c_i}
//      and the fused row stores.
#include <atomic>

#include "launch.h"
#include "mfma_split.h"

namespace ca {
namespace {

constexpr int kGL = 512;                          // max tokens
constexpr int kGThreads = 1024;                   // 16 waves
constexpr int kGPlaneQ = kGL * kD * 2;            // fp16 plane [512][64]
constexpr int kGRows3 = 288;                      // phase 3: 256 queries + two 16-row halos
constexpr int kGPlane3 = kGRows3 * kD * 2;        // fp16 plane [288][64]
constexpr int kGMuXCols = 32;
// region R (phases reuse it)
constexpr int kGOffPart = 2 * kGPlaneQ;           // phase 1: update partials after the Q planes
constexpr int kGOffP = 2 * 4 * kPlane;            // phase 2: P planes after two chunks of K, V planes
constexpr int kGR = 4 * kGPlane3;                 // 147,456 B
static_assert(kGOffPart + 3 * 4 * 64 * 5 * 4 <= kGR, "phase 1 fits");
static_assert(kGOffP + 2 * 2 * kPlaneRow <= kGR, "phase 2 fits");
// outside R
constexpr int kGOffMu = kGR;                              // [16][64] h, m
constexpr int kGOffMuX = kGOffMu + 2 * kPlaneMu;          // [16][32] fp16
constexpr int kGOffC = kGOffMuX + kFK * kGMuXCols * 2;    // [512] assignments
constexpr int kGOffVc = kGOffC + kGL * 4;                 // [16][64] fp32 (1 - alpha) V^cent
constexpr int kGOffXm = kGOffVc + kFK * kD * 4;           // [2][16][8]
constexpr int kGOffXl = kGOffXm + 2 * kFK * 8 * 4;        // [2][16][8]
constexpr int kGOffMax = kGOffXl + 2 * kFK * 8 * 4;       // [16][4]
constexpr int kGLds = kGOffMax + 16 * 4 * 4;
static_assert(kGLds <= 163840, "one workgroup per CU");

}  // namespace

// HIST: hist receives the assignment of every Lloyd iteration, [iters, S, L]
// (S = the grid size).
// FULL: L is 512 (no bounds tests in the clustering and the centroid attention;
// the window passes keep theirs, which the register budget needs).
template <typename T, bool HIST, bool FULL>
__global__ __launch_bounds__(kGThreads, 1) void cluster_attn_fused512_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx, int L, int Kc,
    int iters, int rad, float alpha, int init_step, int H, int G, T *__restrict__ out,
    int32_t *__restrict__ assign, int32_t *__restrict__ hist) {
    __shared__ __align__(16) unsigned char smem[kGLds];
    uint16_t *sQ = reinterpret_cast<uint16_t *>(smem);
    float *sPart = reinterpret_cast<float *>(smem + kGOffPart);
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kGOffMu);
    uint16_t *sMuX = reinterpret_cast<uint16_t *>(smem + kGOffMuX);
    int *sC = reinterpret_cast<int *>(smem + kGOffC);
    float *sVc = reinterpret_cast<float *>(smem + kGOffVc);
    float *sXm = reinterpret_cast<float *>(smem + kGOffXm);
    float *sXl = reinterpret_cast<float *>(smem + kGOffXl);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kGOffMax);
    const u8 *pQ = smem, *pMu = smem + kGOffMu, *pMuX = smem + kGOffMuX;

    const int tid = threadIdx.x;
    constexpr bool kZ = bf16_storage<T>();   // Q (K, V) planes with zero m parts
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const long s = blockIdx.x;
    const long base = s * (long)L * kD;
    const long kvbase = kv_slice(s, H, G) * (long)L * kD;
    const T *Qs = Q + base;
    const int NT = (L + 15) >> 4;
    const LaneOffs lo = lane_offsets(l16, g);
    const int trv = 1024 * (g >> 1) + ((g & 1) ? lo.tr4 : lo.tr0);

    // ============================================================ 1. clustering
    float qraw[2][2][8];   // [tile u: w + 16u][c][i]
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c)
            load_row8<T, FULL>(Qs, 16 * (w + 16 * u) + l16, L, 32 * c + 8 * g, qraw[u][c]);
    // the initial centroids' rows mu_k = Q[init_row(k)] (threads tid < 128:
    // row tid / 8, dims 8 (tid % 8) ..), requested with the Q rows
    float m0[8];
    {
        const int r = tid >> 3, c8 = (tid & 7) * 8;
        if (tid < 128 && r < Kc) {
            load8<T>(Qs + (long)init_row(r, L, Kc, init_step) * kD + c8, m0);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) m0[i] = 0.f;
        }
    }
    {
        float m = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) m = absmax8(qraw[u][1], absmax8(qraw[u][0], m));
        const uint32_t b = wave_max_u(__float_as_uint(m));
        if (lane == 0) sMax[4 * w] = b;
    }
    __syncthreads();
    int sq;
    {
        uint32_t m = 0;
#pragma unroll
        for (int ww = 0; ww < 16; ++ww) m = max(m, sMax[4 * ww]);
        sq = scale_shift(m, kQLimit);
    }
    const float fq = __builtin_ldexpf(1.f, -sq);
    Sp8 qf[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = qraw[u][c][i] * fq;
            qf[u][c] = split8<true>(x);
            const int o = (2048 * (w + 16 * u) + (lo.rl64 ^ (64 * c))) / 2;
            st16(sQ + o, qf[u][c].h);
            if (!kZ) st16(sQ + kGPlaneQ / 2 + o, qf[u][c].m);   // zero for bf16 storage, never read
        }
    if (tid < 128) {   // mu_k = Q[init_row(k)]; rows >= Kc: zero with a -inf part
        const int r = tid >> 3, c8 = (tid & 7) * 8;
        float x[8], n2 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = m0[i] * fq;
            n2 = fmaf(x[i], x[i], n2);
        }
        const Sp8 mp = split8(x);
        const int o = off64(r, c8);
        st16(sMu + o, mp.h);
        st16(sMu + kPlaneMuE + o, mp.m);
        n2 += __shfl_xor(n2, 1);
        n2 += __shfl_xor(n2, 2);
        n2 += __shfl_xor(n2, 4);
        const int c0 = (tid & 7) * 4;
        uint32_t h = 0, m = 0;
        if (r < Kc && c0 == 0) split2(-0.5f * n2, 0.f, h, m);
        uint32_t v0 = 0;
        if (c0 == 0) v0 = r < Kc ? ((h & 0xffffu) | ((m & 0xffffu) << 16)) : (uint32_t)kNegInfH;
        *reinterpret_cast<u32x2_t *>(sMuX + r * kGMuXCols + c0) = u32x2_t{v0, 0u};
    }
    __syncthreads();
    {
        const u32x4_t ones_g0 =
            g == 0 ? u32x4_t{kOneH2, kOneH2, kOneH2, kOneH2} : u32x4_t{0u, 0u, 0u, 0u};
        const u32x4_t ones = {kOneH2, kOneH2, kOneH2, kOneH2};
        const int dt = w & 3, qd = w >> 2;
        const int trq0 = 1024 * g + (lo.tr0 ^ (32 * dt)), trq1 = 1024 * g + (lo.tr4 ^ (32 * dt));
        for (int t = 1; t <= iters; ++t) {
            {
                const u32x4_t mx = ldb16(pMuX, 64 * l16 + 16 * g);
                const Sp8 mu0 = frag_at(pMu, kPlaneMu, lo.rl64), mu1 = frag_at(pMu, kPlaneMu, lo.rl64 ^ 64);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int tile = w + 16 * u;
                    if (FULL || tile < NT) {
                        f32x4_t a = mma(mx, ones_g0, kZero4);
                        a = mma3z<false, kZ>(mu0, qf[u][0], a);
                        a = mma3z<false, kZ>(mu1, qf[u][1], a);
                        float best = a[0];
                        int bk = 4 * g;
#pragma unroll
                        for (int rr = 1; rr < 4; ++rr) {
                            const bool up = a[rr] > best;
                            best = up ? a[rr] : best;
                            bk = up ? 4 * g + rr : bk;
                        }
                        bk = col_argmax(best, bk);
                        const int tok = 16 * tile + l16;
                        if (g == 0 && (FULL || tok < L)) {
                            sC[tok] = bk;
                            if (t == iters && assign) assign[s * L + tok] = bk;
                            if (HIST) hist[((long)(t - 1) * gridDim.x + s) * L + tok] = bk;
                        }
                    }
                }
            }
            __syncthreads();
            f32x4_t sh = kZero4, sm = kZero4, cnt = kZero4;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int cc = 4 * qd + c;
                if (FULL || 32 * cc < L) {
                    const int t0 = 32 * cc + 8 * g;
                    const int4 ca = *reinterpret_cast<const int4 *>(sC + t0);
                    const int4 cb = *reinterpret_cast<const int4 *>(sC + t0 + 4);
                    const int cv[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
                    uint32_t pk[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo16 =
                            ((FULL || t0 + 2 * e < L) && cv[2 * e] == l16) ? 0x3c00u : 0u;
                        const uint32_t hi16 =
                            ((FULL || t0 + 2 * e + 1 < L) && cv[2 * e + 1] == l16) ? 0x3c00u : 0u;
                        pk[e] = lo16 | (hi16 << 16);
                    }
                    const u32x4_t oh = {pk[0], pk[1], pk[2], pk[3]};
                    const Sp8 qt = colfrag8_at<kGPlaneQ>(pQ, 4096 * cc + trq0, 4096 * cc + trq1);
                    if (!kZ) sm = mma(qt.m, oh, sm);
                    sh = mma(qt.h, oh, sh);
                    cnt = mma(ones, oh, cnt);
                }
            }
            if (qd > 0) {
                float *pp = sPart + (((qd - 1) * 4 + dt) * 64 + lane) * 5;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) pp[rr] = sm[rr] + sh[rr];
                pp[4] = cnt[0];
            }
            __syncthreads();
            if (qd == 0) {
                float v[4], n = cnt[0];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = sm[rr] + sh[rr];
#pragma unroll
                for (int q2 = 0; q2 < 3; ++q2) {
                    const float *pp = sPart + ((q2 * 4 + dt) * 64 + lane) * 5;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) v[rr] += pp[rr];
                    n += pp[4];
                }
                const float inv = 1.0f / fmaxf(n, 1.f);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] *= inv;
                const Sp4 mu4 = split4(v[0], v[1], v[2], v[3]);
                float n2p = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) n2p = fmaf(v[rr], v[rr], n2p);
                n2p = col_sum(n2p);
                if (l16 < Kc) {
                    const int o = off64(l16, 16 * dt + 4 * g);
                    st8(sMu + o, mu4.h);
                    st8(sMu + kPlaneMuE + o, mu4.m);
                    if (g == 0) {
                        uint32_t h, m;
                        split2(-0.5f * n2p, 0.f, h, m);
                        sMuX[l16 * kGMuXCols + 2 * dt] = (uint16_t)(h & 0xffffu);
                        sMuX[l16 * kGMuXCols + 2 * dt + 1] = (uint16_t)(m & 0xffffu);
                    }
                }
            }
            __syncthreads();
        }
    }

    // ============================================================ 2. centroid attention
    // half hf = w / 8 takes chunks hf and hf + 2 (keys 128 ch ..); wave w % 8
    // scores key tile w % 8 of its chunk; waves with w % 8 < 4 form the
    // context for dimension tile w % 8 and keep the running (max, sum, row)
    {
        // key chunk loads of this wave's half (keys 128 ch ..); each round's
        // successor is requested as soon as the round's planes are written
        const int hf = w >> 3, tl = tid & 511, wl = w & 7;
        float kraw[2][8], vraw[2][8];
        auto load_chunk = [&](int ch) {
            const int j0 = 128 * ch, nk = FULL ? 128 : min(128, L - j0);
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int it = tl + 512 * n;
                load_row8<T, FULL>(Kx + kvbase + (long)j0 * kD, it >> 3, nk, (it & 7) * 8, kraw[n]);
                load_row8<T, FULL>(Vx + kvbase + (long)j0 * kD, it >> 3, nk, (it & 7) * 8, vraw[n]);
            }
        };
        load_chunk(hf);   // L > 128: both halves have a first chunk
        u8 *pK = smem + 4 * kPlane * hf, *pV = pK + 2 * kPlane;
        uint16_t *cK = reinterpret_cast<uint16_t *>(pK), *cV = reinterpret_cast<uint16_t *>(pV);
        uint16_t *cP = reinterpret_cast<uint16_t *>(smem + kGOffP + 2 * kPlaneRow * hf);
        const u8 *pP = reinterpret_cast<const u8 *>(cP);
        float *xm = sXm + hf * kFK * 8, *xl = sXl + hf * kFK * 8;
        const int trc0 = 1024 * g + (lo.tr0 ^ (32 * (wl & 3)));
        const int trc1 = 1024 * g + (lo.tr4 ^ (32 * (wl & 3)));
        float Mr = -__builtin_inff(), lr = 0.f;
        f32x4_t ar = kZero4;
        for (int r = 0; r < 2; ++r) {
            const int ch = 2 * r + hf;
            const int j0 = 128 * ch;
            const bool on = FULL || j0 < L;         // uniform over the half
            const int nk = FULL ? 128 : on ? min(128, L - j0) : 0;
            if (on) {   // kraw, vraw hold chunk ch (requested earlier)
                const uint32_t bk = wave_max_u(__float_as_uint(absmax8(kraw[1], absmax8(kraw[0], 0.f))));
                const uint32_t bv = wave_max_u(__float_as_uint(absmax8(vraw[1], absmax8(vraw[0], 0.f))));
                if (lane == 0) {
                    sMax[4 * w + 1] = bk;
                    sMax[4 * w + 2] = bv;
                }
            }
            __syncthreads();
            int sk = 0, sv = 0;
            if (on) {
                uint32_t mk = 0, mv = 0;
#pragma unroll
                for (int ww = 0; ww < 8; ++ww) {
                    mk = max(mk, sMax[4 * (8 * hf + ww) + 1]);
                    mv = max(mv, sMax[4 * (8 * hf + ww) + 2]);
                }
                sk = scale_shift(mk, kKVLimit);
                sv = scale_shift(mv, kKVLimit);
                const float fk = __builtin_ldexpf(1.f, -sk), fv = __builtin_ldexpf(1.f, -sv);
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int it = tl + 512 * n;
                    float x[8], y[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        x[i] = kraw[n][i] * fk;
                        y[i] = vraw[n][i] * fv;
                    }
                    const Sp8 kp = split8(x), vp = split8(y);
                    const int o = off64(it >> 3, (it & 7) * 8);
                    st16(cK + o, kp.h);
                    if (!kZ) st16(cK + kPlaneE + o, kp.m);   // zero for bf16 storage, never read
                    st16(cV + o, vp.h);
                    if (!kZ) st16(cV + kPlaneE + o, vp.m);   // zero for bf16 storage, never read
                }
                if (r == 0 && (FULL || 128 * (ch + 2) < L)) load_chunk(ch + 2);   // the next round's chunk
            }
            __syncthreads();
            const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;
            float sx[4];
            if (on) {
                const Sp8 ka = frag_at(pK, kPlane, 2048 * wl + lo.rl64), ma = frag_at(pMu, kPlaneMu, lo.rl64);
                const Sp8 kc = frag_at(pK, kPlane, 2048 * wl + (lo.rl64 ^ 64)), mc = frag_at(pMu, kPlaneMu, lo.rl64 ^ 64);
                __builtin_amdgcn_sched_barrier(0);
                f32x4_t a = mma3z<kZ, false>(ka, ma, kZero4);
                a = mma3z<kZ, false>(kc, mc, a);
                float mloc = -__builtin_inff();
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int key = 16 * wl + 4 * g + rr;
                    sx[rr] = FULL || key < nk ? a[rr] * sscale2 : -__builtin_inff();
                    mloc = fmaxf(mloc, sx[rr]);
                }
                mloc = col_max(mloc);
                if (g == 0) xm[l16 * 8 + wl] = mloc;
            }
            __syncthreads();
            float M = -__builtin_inff();
            if (on) {
                const float4 m0 = *reinterpret_cast<const float4 *>(xm + l16 * 8);
                const float4 m1 = *reinterpret_cast<const float4 *>(xm + l16 * 8 + 4);
                M = fmaxf(fmaxf(fmaxf(m0.x, m0.y), fmaxf(m0.z, m0.w)),
                          fmaxf(fmaxf(m1.x, m1.y), fmaxf(m1.z, m1.w)));
                float p[4], ls = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    p[rr] = __builtin_amdgcn_exp2f(sx[rr] - M);
                    ls += p[rr];
                }
                ls = col_sum(ls);
                const Sp4 ps = split4(p[0], p[1], p[2], p[3]);
                const int o = off128(l16, 16 * wl + 4 * g);
                st8(cP + o, ps.h);
                st8(cP + kPlaneRowE + o, ps.m);
                if (g == 0) xl[l16 * 8 + wl] = ls;
            }
            __syncthreads();
            if (on && wl < 4) {
                const int nch = (nk + 31) >> 5;
                f32x4_t a2[2] = {kZero4, kZero4};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (FULL || c < nch) {
                        const Sp8 vf = colfrag8_at(pV, 4096 * c + trc0, 4096 * c + trc1);
                        const Sp8 pf = frag_at(pP, kPlaneRow, lo.rl128 ^ (64 * c));
                        a2[c & 1] = mma3z<kZ, false>(vf, pf, a2[c & 1]);
                    }
                }
                const float4 l0 = *reinterpret_cast<const float4 *>(xl + l16 * 8);
                const float4 l1 = *reinterpret_cast<const float4 *>(xl + l16 * 8 + 4);
                const float den = ((((((l0.x + l0.y) + l0.z) + l0.w) + l1.x) + l1.y) + l1.z) + l1.w;
                const float vu = __builtin_ldexpf(1.f, sv);
                const f32x4_t ac = (a2[0] + a2[1]) * vu;   // real units, max M
                if (r == 0) {
                    Mr = M;
                    lr = den;
                    ar = ac;
                } else {   // fold chunk 2 + hf into the running record of chunk hf
                    const float Mn = fmaxf(Mr, M);
                    const float fa = __builtin_amdgcn_exp2f(Mr - Mn), fb = __builtin_amdgcn_exp2f(M - Mn);
                    lr = lr * fa + den * fb;
                    ar = ar * fa + ac * fb;
                    Mr = Mn;
                }
            }
            __syncthreads();   // the chunk planes are rewritten next round
        }
        // the two halves meet in a fixed order: half 0, then half 1
        float *xch = reinterpret_cast<float *>(smem + kGOffP);   // [4 dim tiles][64 lanes][6]
        if (hf == 1 && wl < 4) {
            float *e = xch + (wl * 64 + lane) * 6;
            e[0] = Mr; e[1] = lr; e[2] = ar[0]; e[3] = ar[1]; e[4] = ar[2]; e[5] = ar[3];
        }
        __syncthreads();
        if (hf == 0 && wl < 4) {
            const float *e = xch + (wl * 64 + lane) * 6;
            const float M1 = e[0];
            const float Mn = fmaxf(Mr, M1);
            const float fa = __builtin_amdgcn_exp2f(Mr - Mn);
            const float fb = M1 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M1 - Mn);
            const float den = lr * fa + e[1] * fb;
            const float f = (1.0f - alpha) / den;
            float v[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) v[rr] = (ar[rr] * fa + e[2 + rr] * fb) * f;
            *reinterpret_cast<float4 *>(sVc + l16 * kD + 16 * wl + 4 * g) =
                make_float4(v[0], v[1], v[2], v[3]);
        }
        __syncthreads();
    }

    // ============================================================ 3. local window + output
    {
        uint16_t *tK = reinterpret_cast<uint16_t *>(smem), *tV = tK + kGPlane3;   // h, m pairs
        const u8 *pK3 = smem, *pV3 = smem + 2 * kGPlane3;
        constexpr int kItems = (kGRows3 * kD / 8 + kGThreads - 1) / kGThreads;   // 3
        KeyBits kb;
#pragma unroll
        for (int k = 0; k < 4; ++k) kb.w[k] = ~0u;
        for (int p = 0; p < 2; ++p) {
            const int q0 = 256 * p;                 // first query of the pass
            if (q0 >= L) break;                     // uniform
            const int r0 = p == 0 ? 0 : q0 - 16;    // first staged row
            const int Lp = min(L, q0 + 272) - r0;   // staged rows holding keys
            const int NTp = (Lp + 15) >> 4;
            float kraw[kItems][8], vraw[kItems][8];
#pragma unroll
            for (int n = 0; n < kItems; ++n) {
                const int it = tid + kGThreads * n;
                if (it < kGRows3 * kD / 8) {
                    load_row8<T, false>(Kx + kvbase + (long)r0 * kD, it >> 3, Lp, (it & 7) * 8, kraw[n]);
                    load_row8<T, false>(Vx + kvbase + (long)r0 * kD, it >> 3, Lp, (it & 7) * 8, vraw[n]);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) kraw[n][i] = vraw[n][i] = 0.f;
                }
            }
            {
                float mk = 0.f, mv = 0.f;
#pragma unroll
                for (int n = 0; n < kItems; ++n) {
                    mk = absmax8(kraw[n], mk);
                    mv = absmax8(vraw[n], mv);
                }
                const uint32_t bk = wave_max_u(__float_as_uint(mk));
                const uint32_t bv = wave_max_u(__float_as_uint(mv));
                if (lane == 0) {
                    sMax[4 * w + 1] = bk;
                    sMax[4 * w + 2] = bv;
                }
            }
            __syncthreads();
            uint32_t mk = 0, mv = 0;
#pragma unroll
            for (int ww = 0; ww < 16; ++ww) {
                mk = max(mk, sMax[4 * ww + 1]);
                mv = max(mv, sMax[4 * ww + 2]);
            }
            const int sk = scale_shift(mk, kKVLimit), sv = scale_shift(mv, kKVLimit);
            // the wave's query rows of this pass, requested before the planes
            // are built so that their latency passes during that work
            const int tile = 16 * p + w;   // the wave's query tile of this pass
            float qx[2][8];
#pragma unroll
            for (int c = 0; c < 2; ++c) load_row8<T, false>(Qs, 16 * tile + l16, L, 32 * c + 8 * g, qx[c]);
            {
                const float fk = __builtin_ldexpf(1.f, -sk), fv = __builtin_ldexpf(1.f, -sv);
#pragma unroll
                for (int n = 0; n < kItems; ++n) {
                    const int it = tid + kGThreads * n;
                    if (it < kGRows3 * kD / 8) {
                        float x[8], y[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            x[i] = kraw[n][i] * fk;
                            y[i] = vraw[n][i] * fv;
                        }
                        const Sp8 kp = split8(x), vp = split8(y);
                        const int o = off64(it >> 3, (it & 7) * 8);
                        st16(tK + o, kp.h);
                        if (!kZ) st16(tK + kGPlane3 / 2 + o, kp.m);   // zero for bf16 storage, never read
                        st16(tV + o, vp.h);
                        if (!kZ) st16(tV + kGPlane3 / 2 + o, vp.m);   // zero for bf16 storage, never read
                    }
                }
            }
            __syncthreads();
            if (tile < NT) {
                const int qt = (16 * tile - r0) >> 4;
                const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;
                // the tile's Q fragments again (cheaper than keeping them live
                // through the centroid attention): the same values as in phase 1
                Sp8 qp[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) qx[c][i] *= fq;
                    qp[c] = split8<true>(qx[c]);
                }
                f32x4_t o[4];
                float lsum;
                local_narrow<false, false, KeyBits, kGPlane3, kZ>(pK3, pV3, qp, qt, NTp, Lp, rad,
                                                            sscale2, l16, g, lo.rl64, trv, kb, o,
                                                            lsum);
                const int tok = 16 * tile + l16;
                if (tok < L) {
                    const float f = alpha * __builtin_ldexpf(1.f, sv) * __builtin_amdgcn_rcpf(lsum);
                    const float *vc = sVc + sC[tok] * kD;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {   // o[j][rr] = Oloc^T[dim 16j + 4g + rr][query tok]
                        const int d0 = 16 * j + 4 * g;
                        const float4 c4 = *reinterpret_cast<const float4 *>(vc + d0);
                        store4<T>(out + base + (long)tok * kD + d0,
                                  make_float4(fmaf(o[j][0], f, c4.x), fmaf(o[j][1], f, c4.y),
                                              fmaf(o[j][2], f, c4.z), fmaf(o[j][3], f, c4.w)));
                    }
                }
            }
            __syncthreads();   // the planes are rewritten by the next pass
        }
    }
}

// Split form (SPLIT, bf16 storage): a grid of 2 S workgroups, S at most half
// the CUs, so that all of them are resident at once (one per CU).
//   Workgroup s < S (clustering) runs phase 1 for slice s, publishes the
//   final centroid planes and its Q scale and raises the slice's flag to
//   2e + 1 (e: the launch number), runs round 0 of phase 2 (key chunks 0 and
//   1), publishes that round's record (maximum, sum, row of each context lane)
//   and the assignment, and raises the flag to 2e + 2.
//   Workgroup S + s (window) runs phase 3 for slice s on a CU the single launch
//   would leave idle, each pass with its own Q scale, and keeps the window
//   rows in LDS as fp16; after the first flag it runs round 1 of phase 2 (key
//   chunks 2 and 3) with the published centroids, after the second it merges
//   the two records in chunk order into (1 - alpha) V^cent and writes the
//   fused rows. Measured, bf16 L = 512, 96 slices: 25.9 us per forward
//   against 27.9 us for the staged launches (same box); per workgroup, the
//   clustering publishes its centroids at 10.4 us and its record at 15.5 us,
//   the window workgroup ends its passes at 13.3 us and its round at 17.3 us
//   and writes the last rows at 20.3 us.
// Each value that crosses workgroups is written with a device-scope atomic
// store and read with a device-scope atomic load (coherent across the XCDs'
// L2 caches); a writer waits for its stores to complete before the barrier
// that precedes its flag store, a reader loads only after it saw the flag, so
// no cache write-back or invalidate is needed. A wait is bounded: past
// kSpinLimit polls it records the launch in the ring's error word and the
// window workgroup writes NaN rows, so that the failure cannot pass unnoticed.
// words of one slice's published values: the final centroid planes (h, m), the
// record of key chunks 0 and 1 ([4 dim tiles][64 lanes][M, l, row 0..3]), c
constexpr int kPubMu = 0;
constexpr int kPubPart = kPubMu + 2 * kPlaneMu / 4;
constexpr int kPubC = kPubPart + 4 * 64 * 6;
constexpr int kPubSq = kPubC + kGL;          // the clustering's Q scale shift
constexpr int kPubStride = kPubSq + 64;      // (rounded up to 256 bytes)
constexpr int kSpinLimit = 1 << 18;          // polls of a flag before giving up (about 0.3 s)

// Flags of the split form, owned by the library (zero when the code object is
// loaded, one copy per device): launch number e (per device, from 1, never
// reused) uses ring e % kRings; the clustering workgroup of slice s sets word
// s of that ring to 2e + 1 once its centroids are published and to 2e + 2 once
// its record and the assignment are, and a wait that gives up stores e in the
// ring's error word. Values left by earlier launches of the ring are at most
// 2 (e - kRings) + 2, so no reset is needed between launches, and launches in
// flight at the same time use different rings unless kRings of them overlap.
constexpr int kRings = 64;
constexpr int kMaxSplitSlices = 512;
__device__ unsigned long long g_split_flags[kRings * kMaxSplitSlices];
__device__ unsigned long long g_split_err[kRings];
__device__ __forceinline__ unsigned long long *split_flag(unsigned long long e, long s) {
    return g_split_flags + (e % kRings) * kMaxSplitSlices + s;
}
__device__ __forceinline__ unsigned long long *split_err(unsigned long long e) {
    return g_split_err + e % kRings;
}
static_assert(2 * kPlaneMu / 4 == kGThreads, "one centroid-plane word per thread");

// device-scope atomic load of a published word (coherent across the XCDs)
__device__ __forceinline__ uint32_t ld_pub(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 polls *flag until it holds at least v (bounded: past kSpinLimit
// polls it stores the launch number e in the ring's error word and stops
// waiting); the workgroup then passes a barrier.
__device__ __forceinline__ void wait_flag(unsigned long long *flag, unsigned long long v,
                                          unsigned long long e) {
    if (threadIdx.x == 0) {
        int polls = 0;
        while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < v) {
            __builtin_amdgcn_s_sleep(1);
            if (++polls > kSpinLimit) {
                __hip_atomic_store(split_err(e), e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// LDS block (2 KB, lane-major 16-byte chunks) holding wave w's window rows of
// pass p as fp16 while the split form's window workgroup runs the rest: bytes
// [48K, 64K) and [112K, 128K) for pass 0 (unwritten by the second pass and by
// the centroid attention), [16K, 32K) and [80K, 96K) for pass 1 (unwritten by
// the centroid attention), waves 0-7 in the first range, 8-15 in the second.
__device__ __forceinline__ u32x4_t *stash_at(unsigned char *smem, int p, int w) {
    const int base = (p == 0 ? 48 : 16) * 1024 + (w < 8 ? 0 : 64 * 1024) + 2048 * (w & 7);
    return reinterpret_cast<u32x4_t *>(smem + base);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
// o[j][rr] * il (rounded to nearest fp16) of this lane
__device__ __forceinline__ void stash_put(u32x4_t *blk, const f32x4_t *o, float il) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const f32x4_t a = o[2 * c] * il, b = o[2 * c + 1] * il;
        blk[64 * c + lane] = u32x4_t{pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]),
                                     pack_f16x2(b[0], b[1]), pack_f16x2(b[2], b[3])};
    }
}
__device__ __forceinline__ void stash_get(const u32x4_t *blk, float *y) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const u32x4_t v = blk[64 * c + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[8 * c + 2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[i] & 0xffffu));
            y[8 * c + 2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[i] >> 16));
        }
    }
}

// The split form's kernel: the single launch's phases as routines (phase 3 over
// a range of window passes, phase 2 over a range of key-chunk rounds) run by
// the two kinds of workgroup. Its steps that only the split form takes are
// marked by SPLIT (always true here): the single launch above keeps its own
// copy of the phases, which the compiler schedules better on their own
// (same-box A/B at 192 slices: 33.2 against 34.7 us once both forms shared one
// kernel). HIST and FULL as above.
template <typename T, bool HIST, bool FULL, bool SPLIT>
__global__ __launch_bounds__(kGThreads, 1) void cluster_attn_fused512_split_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx, int L, int Kc,
    int iters, int rad, float alpha, int init_step, int H, int G, T *__restrict__ out,
    int32_t *__restrict__ assign, int32_t *__restrict__ hist, int S, uint32_t *__restrict__ pub,
    unsigned long long epoch) {
    __shared__ __align__(16) unsigned char smem[kGLds];
    uint16_t *sQ = reinterpret_cast<uint16_t *>(smem);
    float *sPart = reinterpret_cast<float *>(smem + kGOffPart);
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kGOffMu);
    uint16_t *sMuX = reinterpret_cast<uint16_t *>(smem + kGOffMuX);
    int *sC = reinterpret_cast<int *>(smem + kGOffC);
    float *sVc = reinterpret_cast<float *>(smem + kGOffVc);
    float *sXm = reinterpret_cast<float *>(smem + kGOffXm);
    float *sXl = reinterpret_cast<float *>(smem + kGOffXl);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kGOffMax);
    const u8 *pQ = smem, *pMu = smem + kGOffMu, *pMuX = smem + kGOffMuX;

    const int tid = threadIdx.x;
    constexpr bool kZ = bf16_storage<T>();   // Q (K, V) planes with zero m parts
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const bool win = SPLIT && (int)blockIdx.x >= S;   // window workgroup of the split form
    const long s = win ? (long)blockIdx.x - S : (long)blockIdx.x;
    const long base = s * (long)L * kD;
    const long kvbase = kv_slice(s, H, G) * (long)L * kD;
    const T *Qs = Q + base;
    const int NT = (L + 15) >> 4;
    const LaneOffs lo = lane_offsets(l16, g);
    const int trv = 1024 * (g >> 1) + ((g & 1) ? lo.tr4 : lo.tr0);

    // Phase 3 (below) as a routine of the slice's Q scale shift: the single
    // launch runs it after phase 2, a window workgroup of the split form alone.
    // phase 2's key chunk rows of this thread (rows it / 8, it = tid % 512 + 512 n,
    // of chunk ch, dims 8 (it % 8) ..): declared here so that the split form's
    // window workgroup can request its first chunk before it waits
    float ckraw[2][8], cvraw[2][8];
    auto load_chunk = [&](int ch) {
        const int j0 = 128 * ch, nk = FULL ? 128 : min(128, L - j0), tl = tid & 511;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int it = tl + 512 * n;
            load_row8<T, FULL>(Kx + kvbase + (long)j0 * kD, it >> 3, nk, (it & 7) * 8, ckraw[n]);
            load_row8<T, FULL>(Vx + kvbase + (long)j0 * kD, it >> 3, nk, (it & 7) * 8, cvraw[n]);
        }
    };
    float wfac0 = 0.f, wfac1 = 0.f;   // split form: alpha 2^sv of each window pass
    auto phase3 = [&](const int sq, const float fq) {
    {
        uint16_t *tK = reinterpret_cast<uint16_t *>(smem), *tV = tK + kGPlane3;   // h, m pairs
        const u8 *pK3 = smem, *pV3 = smem + 2 * kGPlane3;
        constexpr int kItems = (kGRows3 * kD / 8 + kGThreads - 1) / kGThreads;   // 3
        KeyBits kb;
#pragma unroll
        for (int k = 0; k < 4; ++k) kb.w[k] = ~0u;
        // split form: each pass's window rows O^loc / l (scaled units of V)
        // wait for the gather as fp16 in LDS that neither the second pass nor
        // the centroid attention writes (bf16 storage leaves their m planes
        // unused; stash_at), their factor alpha 2^sv in wfac0 / wfac1; the second
        // pass's rows are stored once its planes are dead
        static_assert(!SPLIT || bf16_storage<T>(), "the split form keeps results in the m planes");
        f32x4_t o1[4] = {kZero4, kZero4, kZero4, kZero4};
        float il1 = 0.f;
        // one window pass (p = 0: queries 0 .. 255, 1: 256 ..); false when L has no such queries
        // split form: the second pass's K and V rows, requested during the
        // first pass's window products and kept as raw bf16 (16 bytes per item)
        u32x4_t kpre[kItems], vpre[kItems], qpre[2];
        // the wave's query rows (token tile 16 p + w, 8 bf16 at columns
        // 32 c + 8 g) as raw bf16; rows past the slice read the last row
        auto load_qraw = [&](const int p, u32x4_t *qr) {
            const int row = 16 * (16 * p + w) + l16, rc = row < L ? row : L - 1;
#pragma unroll
            for (int c = 0; c < 2; ++c)
                qr[c] = *reinterpret_cast<const u32x4_t *>(Qs + (long)rc * kD + 32 * c + 8 * g);
        };
        auto prefetch1 = [&]() {
            const int r0 = 240, Lp = min(L, 528) - r0;
#pragma unroll
            for (int n = 0; n < kItems; ++n) {
                const int it = tid + kGThreads * n;
                const int row = it >> 3, rc = row < Lp ? row : Lp - 1;
                const long off = kvbase + (long)(r0 + rc) * kD + (it & 7) * 8;
                kpre[n] = *reinterpret_cast<const u32x4_t *>(Kx + off);
                vpre[n] = *reinterpret_cast<const u32x4_t *>(Vx + off);
            }
        };
        auto pass = [&](const int p) -> bool {
            const int q0 = 256 * p;                 // first query of the pass
            if (q0 >= L) return false;              // uniform
            const int r0 = p == 0 ? 0 : q0 - 16;    // first staged row
            const int Lp = min(L, q0 + 272) - r0;   // staged rows holding keys
            const int NTp = (Lp + 15) >> 4;
            float kraw[kItems][8], vraw[kItems][8];
#pragma unroll
            for (int n = 0; n < kItems; ++n) {
                const int it = tid + kGThreads * n;
                if (it < kGRows3 * kD / 8) {
                    if (SPLIT && p == 1) {   // prefetched: rows past the slice become zeros
                        const bool in = (it >> 3) < Lp;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t ku = in ? kpre[n][i] : 0u, vu = in ? vpre[n][i] : 0u;
                            kraw[n][2 * i] = __uint_as_float(ku << 16);
                            kraw[n][2 * i + 1] = __uint_as_float(ku & 0xffff0000u);
                            vraw[n][2 * i] = __uint_as_float(vu << 16);
                            vraw[n][2 * i + 1] = __uint_as_float(vu & 0xffff0000u);
                        }
                    } else {
                        load_row8<T, false>(Kx + kvbase + (long)r0 * kD, it >> 3, Lp, (it & 7) * 8, kraw[n]);
                        load_row8<T, false>(Vx + kvbase + (long)r0 * kD, it >> 3, Lp, (it & 7) * 8, vraw[n]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) kraw[n][i] = vraw[n][i] = 0.f;
                }
            }
            const int tile = 16 * p + w;   // the wave's query tile of this pass
            // split form: the pass's own Q scale (its 256 query rows), so that
            // the window workgroup needs nothing of phase 1; a power of two
            // either way, which leaves the products unchanged. Its query rows
            // stay in registers as raw bf16 (the second pass's were requested
            // during the first pass's products).
            uint32_t bq = 0u;
            u32x4_t qr[2] = {u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}};
            if (SPLIT) {
                if (p == 0) load_qraw(0, qr);
                else { qr[0] = qpre[0]; qr[1] = qpre[1]; }
                const bool in = 16 * tile + l16 < L;
                float m = 0.f;
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        qr[c][i] = in ? qr[c][i] : 0u;
                        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(qr[c][i] << 16)),
                                           fabsf(__uint_as_float(qr[c][i] & 0xffff0000u))));
                    }
                bq = __float_as_uint(m);
            }
            {
                float mk = 0.f, mv = 0.f;
#pragma unroll
                for (int n = 0; n < kItems; ++n) {
                    mk = absmax8(kraw[n], mk);
                    mv = absmax8(vraw[n], mv);
                }
                const uint32_t bk = wave_max_u(__float_as_uint(mk));
                const uint32_t bv = wave_max_u(__float_as_uint(mv));
                if (SPLIT) bq = wave_max_u(bq);
                if (lane == 0) {
                    if (SPLIT) sMax[4 * w] = bq;
                    sMax[4 * w + 1] = bk;
                    sMax[4 * w + 2] = bv;
                }
            }
            __syncthreads();
            uint32_t mk = 0, mv = 0, mq = 0;
#pragma unroll
            for (int ww = 0; ww < 16; ++ww) {
                mk = max(mk, sMax[4 * ww + 1]);
                mv = max(mv, sMax[4 * ww + 2]);
                if (SPLIT) mq = max(mq, sMax[4 * ww]);
            }
            const int sk = scale_shift(mk, kKVLimit), sv = scale_shift(mv, kKVLimit);
            const int sqp = SPLIT ? scale_shift(mq, kQLimit) : sq;
            const float fqp = SPLIT ? __builtin_ldexpf(1.f, -sqp) : fq;
            (p == 0 ? wfac0 : wfac1) = alpha * __builtin_ldexpf(1.f, sv);   // uniform
            // the wave's query rows of this pass, requested before the planes
            // are built so that their latency passes during that work
            float qx[2][8];
            if (SPLIT) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        qx[c][2 * i] = __uint_as_float(qr[c][i] << 16);
                        qx[c][2 * i + 1] = __uint_as_float(qr[c][i] & 0xffff0000u);
                    }
            } else {
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    load_row8<T, false>(Qs, 16 * tile + l16, L, 32 * c + 8 * g, qx[c]);
            }
            {
                const float fk = __builtin_ldexpf(1.f, -sk), fv = __builtin_ldexpf(1.f, -sv);
#pragma unroll
                for (int n = 0; n < kItems; ++n) {
                    const int it = tid + kGThreads * n;
                    if (it < kGRows3 * kD / 8) {
                        float x[8], y[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            x[i] = kraw[n][i] * fk;
                            y[i] = vraw[n][i] * fv;
                        }
                        const Sp8 kp = split8(x), vp = split8(y);
                        const int o = off64(it >> 3, (it & 7) * 8);
                        st16(tK + o, kp.h);
                        if (!kZ) st16(tK + kGPlane3 / 2 + o, kp.m);   // zero for bf16 storage, never read
                        st16(tV + o, vp.h);
                        if (!kZ) st16(tV + kGPlane3 / 2 + o, vp.m);   // zero for bf16 storage, never read
                    }
                }
            }
            __syncthreads();
            if (SPLIT && p == 0 && L > 256) prefetch1();
            if (tile < NT) {
                const int qt = (16 * tile - r0) >> 4;
                const float sscale2 = __builtin_ldexpf(0.125f, sqp + sk) * 1.4426950408889634f;
                // the tile's Q fragments again (cheaper than keeping them live
                // through the centroid attention): the same values as in phase 1
                Sp8 qp[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) qx[c][i] *= fqp;
                    qp[c] = split8<true>(qx[c]);
                }
                f32x4_t o[4];
                float lsum;
                local_narrow<false, false, KeyBits, kGPlane3, kZ>(pK3, pV3, qp, qt, NTp, Lp, rad,
                                                            sscale2, l16, g, lo.rl64, trv, kb, o,
                                                            lsum);
                const int tok = 16 * tile + l16;
                if (SPLIT) {
                    if (p == 0) {
                        stash_put(stash_at(smem, 0, w), o, __builtin_amdgcn_rcpf(lsum));
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) o1[j] = o[j];
                        il1 = __builtin_amdgcn_rcpf(lsum);
                    }
                } else if (tok < L) {
                    const float f = alpha * __builtin_ldexpf(1.f, sv) * __builtin_amdgcn_rcpf(lsum);
                    const float *vc = sVc + sC[tok] * kD;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {   // o[j][rr] = Oloc^T[dim 16j + 4g + rr][query tok]
                        const int d0 = 16 * j + 4 * g;
                        const float4 c4 = *reinterpret_cast<const float4 *>(vc + d0);
                        store4<T>(out + base + (long)tok * kD + d0,
                                  make_float4(fmaf(o[j][0], f, c4.x), fmaf(o[j][1], f, c4.y),
                                              fmaf(o[j][2], f, c4.z), fmaf(o[j][3], f, c4.w)));
                    }
                }
            }
            // the second pass's query rows, in flight while the waves meet;
            // after the second pass, the rows of key chunk 2 + hf (phase 2's
            // round 1), in flight while the workgroup waits for the centroids
            if (SPLIT && p == 0 && L > 256) load_qraw(1, qpre);
            if (SPLIT && p == 1 && (FULL || 128 * (2 + (w >> 3)) < L)) load_chunk(2 + (w >> 3));
            __syncthreads();   // the planes are rewritten by the next pass
            return true;
        };
        // the split form runs the passes as separate copies (p known to the
        // compiler), so that the first pass's registers hold nothing of the second's
        if (SPLIT) {
            if (pass(0)) pass(1);
        } else {
            for (int p = 0; p < 2; ++p)
                if (!pass(p)) break;
        }
        if (SPLIT && 16 * (16 + w) < L) stash_put(stash_at(smem, 1, w), o1, il1);
    }
    };
    // ============================================================ 2. centroid attention
    // Rounds r0 .. r1 - 1 of it: in round r, half hf = w / 8 takes key chunk
    // 2 r + hf (keys 128 ch ..; the single launch runs rounds 0 and 1); wave
    // w % 8 scores key tile w % 8 of its chunk; waves with w % 8 < 4 form the
    // context for dimension tile w % 8 and keep the running (max, sum, row).
    // The halves meet in a fixed order (half 0, then half 1), leaving in the
    // context waves of half 0 the record of every chunk taken: maximum Mo,
    // sum lo2 and unnormalised row ao in real base-2 units (-inf, 0, 0 when
    // there was none).
    // pre: the first round's chunk rows are already requested (load_chunk)
    auto phase2 = [&](const int sq, const int r0, const int r1, const bool pre, float &Mo,
                      float &lo2, f32x4_t &ao) {
        // key chunk loads of this wave's half (keys 128 ch ..); each round's
        // successor is requested as soon as the round's planes are written
        const int hf = w >> 3, tl = tid & 511, wl = w & 7;
        float (&kraw)[2][8] = ckraw, (&vraw)[2][8] = cvraw;
        if (!pre && (FULL || 128 * (2 * r0 + hf) < L)) load_chunk(2 * r0 + hf);
        u8 *pK = smem + 4 * kPlane * hf, *pV = pK + 2 * kPlane;
        uint16_t *cK = reinterpret_cast<uint16_t *>(pK), *cV = reinterpret_cast<uint16_t *>(pV);
        uint16_t *cP = reinterpret_cast<uint16_t *>(smem + kGOffP + 2 * kPlaneRow * hf);
        const u8 *pP = reinterpret_cast<const u8 *>(cP);
        float *xm = sXm + hf * kFK * 8, *xl = sXl + hf * kFK * 8;
        const int trc0 = 1024 * g + (lo.tr0 ^ (32 * (wl & 3)));
        const int trc1 = 1024 * g + (lo.tr4 ^ (32 * (wl & 3)));
        float Mr = -__builtin_inff(), lr = 0.f;
        f32x4_t ar = kZero4;
        for (int r = r0; r < r1; ++r) {
            const int ch = 2 * r + hf;
            const int j0 = 128 * ch;
            const bool on = FULL || j0 < L;         // uniform over the half
            const int nk = FULL ? 128 : on ? min(128, L - j0) : 0;
            if (on) {   // kraw, vraw hold chunk ch (requested earlier)
                const uint32_t bk = wave_max_u(__float_as_uint(absmax8(kraw[1], absmax8(kraw[0], 0.f))));
                const uint32_t bv = wave_max_u(__float_as_uint(absmax8(vraw[1], absmax8(vraw[0], 0.f))));
                if (lane == 0) {
                    sMax[4 * w + 1] = bk;
                    sMax[4 * w + 2] = bv;
                }
            }
            __syncthreads();
            int sk = 0, sv = 0;
            if (on) {
                uint32_t mk = 0, mv = 0;
#pragma unroll
                for (int ww = 0; ww < 8; ++ww) {
                    mk = max(mk, sMax[4 * (8 * hf + ww) + 1]);
                    mv = max(mv, sMax[4 * (8 * hf + ww) + 2]);
                }
                sk = scale_shift(mk, kKVLimit);
                sv = scale_shift(mv, kKVLimit);
                const float fk = __builtin_ldexpf(1.f, -sk), fv = __builtin_ldexpf(1.f, -sv);
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int it = tl + 512 * n;
                    float x[8], y[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        x[i] = kraw[n][i] * fk;
                        y[i] = vraw[n][i] * fv;
                    }
                    const Sp8 kp = split8(x), vp = split8(y);
                    const int o = off64(it >> 3, (it & 7) * 8);
                    st16(cK + o, kp.h);
                    if (!kZ) st16(cK + kPlaneE + o, kp.m);   // zero for bf16 storage, never read
                    st16(cV + o, vp.h);
                    if (!kZ) st16(cV + kPlaneE + o, vp.m);   // zero for bf16 storage, never read
                }
                if (r + 1 < r1 && (FULL || 128 * (ch + 2) < L)) load_chunk(ch + 2);   // the next round's chunk
            }
            __syncthreads();
            const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;
            float sx[4];
            if (on) {
                const Sp8 ka = frag_at(pK, kPlane, 2048 * wl + lo.rl64), ma = frag_at(pMu, kPlaneMu, lo.rl64);
                const Sp8 kc = frag_at(pK, kPlane, 2048 * wl + (lo.rl64 ^ 64)), mc = frag_at(pMu, kPlaneMu, lo.rl64 ^ 64);
                __builtin_amdgcn_sched_barrier(0);
                f32x4_t a = mma3z<kZ, false>(ka, ma, kZero4);
                a = mma3z<kZ, false>(kc, mc, a);
                float mloc = -__builtin_inff();
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int key = 16 * wl + 4 * g + rr;
                    sx[rr] = FULL || key < nk ? a[rr] * sscale2 : -__builtin_inff();
                    mloc = fmaxf(mloc, sx[rr]);
                }
                mloc = col_max(mloc);
                if (g == 0) xm[l16 * 8 + wl] = mloc;
            }
            __syncthreads();
            float M = -__builtin_inff();
            if (on) {
                const float4 m0 = *reinterpret_cast<const float4 *>(xm + l16 * 8);
                const float4 m1 = *reinterpret_cast<const float4 *>(xm + l16 * 8 + 4);
                M = fmaxf(fmaxf(fmaxf(m0.x, m0.y), fmaxf(m0.z, m0.w)),
                          fmaxf(fmaxf(m1.x, m1.y), fmaxf(m1.z, m1.w)));
                float p[4], ls = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    p[rr] = __builtin_amdgcn_exp2f(sx[rr] - M);
                    ls += p[rr];
                }
                ls = col_sum(ls);
                const Sp4 ps = split4(p[0], p[1], p[2], p[3]);
                const int o = off128(l16, 16 * wl + 4 * g);
                st8(cP + o, ps.h);
                st8(cP + kPlaneRowE + o, ps.m);
                if (g == 0) xl[l16 * 8 + wl] = ls;
            }
            __syncthreads();
            if (on && wl < 4) {
                const int nch = (nk + 31) >> 5;
                f32x4_t a2[2] = {kZero4, kZero4};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (FULL || c < nch) {
                        const Sp8 vf = colfrag8_at(pV, 4096 * c + trc0, 4096 * c + trc1);
                        const Sp8 pf = frag_at(pP, kPlaneRow, lo.rl128 ^ (64 * c));
                        a2[c & 1] = mma3z<kZ, false>(vf, pf, a2[c & 1]);
                    }
                }
                const float4 l0 = *reinterpret_cast<const float4 *>(xl + l16 * 8);
                const float4 l1 = *reinterpret_cast<const float4 *>(xl + l16 * 8 + 4);
                const float den = ((((((l0.x + l0.y) + l0.z) + l0.w) + l1.x) + l1.y) + l1.z) + l1.w;
                const float vu = __builtin_ldexpf(1.f, sv);
                const f32x4_t ac = (a2[0] + a2[1]) * vu;   // real units, max M
                if (r == r0) {
                    Mr = M;
                    lr = den;
                    ar = ac;
                } else {   // fold chunk 2 + hf into the running record of chunk hf
                    const float Mn = fmaxf(Mr, M);
                    const float fa = __builtin_amdgcn_exp2f(Mr - Mn), fb = __builtin_amdgcn_exp2f(M - Mn);
                    lr = lr * fa + den * fb;
                    ar = ar * fa + ac * fb;
                    Mr = Mn;
                }
            }
            __syncthreads();   // the chunk planes are rewritten next round
        }
        // the two halves meet in a fixed order: half 0, then half 1
        float *xch = reinterpret_cast<float *>(smem + kGOffP);   // [4 dim tiles][64 lanes][6]
        if (hf == 1 && wl < 4) {
            float *e = xch + (wl * 64 + lane) * 6;
            e[0] = Mr; e[1] = lr; e[2] = ar[0]; e[3] = ar[1]; e[4] = ar[2]; e[5] = ar[3];
        }
        __syncthreads();
        Mo = -__builtin_inff();
        lo2 = 0.f;
        ao = kZero4;
        if (hf == 0 && wl < 4) {
            const float *e = xch + (wl * 64 + lane) * 6;
            const float M1 = e[0];
            const float Mn = fmaxf(Mr, M1);
            if (Mn != -__builtin_inff()) {
                const float fa = Mr == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(Mr - Mn);
                const float fb = M1 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M1 - Mn);
                Mo = Mn;
                lo2 = lr * fa + e[1] * fb;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) ao[rr] = ar[rr] * fa + e[2 + rr] * fb;
            }
        }
        __syncthreads();   // xch is rewritten next
    };

    if (win) {
        // window workgroup: both window passes (each with its own Q scale) ...
        phase3(0, 1.f);
        // ... then the clustering workgroup's final centroids, Q scale and
        // assignment (flag value 2 epoch + 1) and key chunks 2 and 3 of the
        // centroid attention with them
        const uint32_t *pv = pub + s * kPubStride;
        unsigned long long *flag = split_flag(epoch, s);
        wait_flag(flag, 2 * epoch + 1, epoch);
        reinterpret_cast<uint32_t *>(sMu)[tid] = ld_pub(pv + kPubMu + tid);   // 2 kPlaneMu bytes
        if (tid < L) sC[tid] = (int)ld_pub(pv + kPubC + tid);
        const int sqc = (int)ld_pub(pv + kPubSq);
        __syncthreads();
        const int hf = w >> 3, wl = w & 7;
        float Mh, lh;
        f32x4_t ah;
        phase2(sqc, 1, 2, L > 256, Mh, lh, ah);
        // its record of chunks 0 and 1 (flag value 2 epoch + 2); the records
        // meet in chunk order, then (1 - alpha) V^cent
        wait_flag(flag, 2 * epoch + 2, epoch);
        if (hf == 0 && wl < 4) {
            const uint32_t *e = pv + kPubPart + (wl * 64 + lane) * 6;
            float rec[6];
#pragma unroll
            for (int i = 0; i < 6; ++i) rec[i] = __uint_as_float(ld_pub(e + i));
            const float Mn = fmaxf(rec[0], Mh);   // chunk 0 makes it finite
            const float fa = rec[0] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(rec[0] - Mn);
            const float fb = Mh == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(Mh - Mn);
            const float f = (1.0f - alpha) / (rec[1] * fa + lh * fb);
            float v[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) v[rr] = (rec[2 + rr] * fa + ah[rr] * fb) * f;
            *reinterpret_cast<float4 *>(sVc + l16 * kD + 16 * wl + 4 * g) =
                make_float4(v[0], v[1], v[2], v[3]);
        }
        __syncthreads();
        // the gather and the fused rows of both passes; a wait that gave up
        // leaves no valid V^cent: NaN rows, so that it cannot pass unnoticed
        const bool bad = __hip_atomic_load(split_err(epoch), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == epoch;
        const float qnan = __builtin_nanf("");
        // each wave's 16 rows go through a 2 KB LDS tile (16-byte chunks
        // XOR-swizzled by the row; bytes [0, 16K) and [64K, 80K), which phase 2
        // no longer needs) so that every store writes 64 x 16 bytes of whole rows
        u8 *stg = smem + (w < 8 ? 0 : 64 * 1024) + 2048 * (w & 7);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int tile = 16 * p + w;
            if (16 * tile >= L) continue;   // uniform over the wave
            const int tok = 16 * tile + l16;
            if (tok < L) {
                float y[16];
                stash_get(stash_at(smem, p, w), y);
                const float f = p == 0 ? wfac0 : wfac1;
                const float *vc = sVc + sC[tok] * kD;
#pragma unroll
                for (int j = 0; j < 4; ++j) {   // y[4j + rr] = Oloc^T[dim 16j + 4g + rr][query tok] / l
                    const int d0 = 16 * j + 4 * g;
                    const float4 c4 = *reinterpret_cast<const float4 *>(vc + d0);
                    float v0 = fmaf(y[4 * j], f, c4.x), v1 = fmaf(y[4 * j + 1], f, c4.y);
                    float v2 = fmaf(y[4 * j + 2], f, c4.z), v3 = fmaf(y[4 * j + 3], f, c4.w);
                    if (bad) v0 = v1 = v2 = v3 = qnan;
                    const int byte = 2 * d0;   // within the 128-byte row
                    *reinterpret_cast<u32x2_t *>(stg + 128 * l16 + (((byte >> 4) ^ (l16 & 7)) << 4) +
                                                 (byte & 15)) =
                        u32x2_t{(uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16),
                                (uint32_t)f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16)};
                }
            }
            __builtin_amdgcn_wave_barrier();
            u8 *dst = reinterpret_cast<u8 *>(out + base + (long)16 * tile * kD);
#pragma unroll
            for (int i = 0; i < 2; ++i) {   // 128 chunks of 16 bytes, 8 per row
                const int flat = 64 * i + lane, row = flat >> 3, c = flat & 7;
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stg + 128 * row + ((c ^ (row & 7)) << 4));
                if (16 * tile + row < L)
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst + 16 * flat));
            }
            __builtin_amdgcn_wave_barrier();   // the tile is rewritten by the next pass
        }
        return;
    }

    int sq;     // the slice's Q scale shift
    float fq;   // 2^-sq
    // ============================================================ 1. clustering
    float qraw[2][2][8];   // [tile u: w + 16u][c][i]
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c)
            load_row8<T, FULL>(Qs, 16 * (w + 16 * u) + l16, L, 32 * c + 8 * g, qraw[u][c]);
    // the initial centroids' rows mu_k = Q[init_row(k)] (threads tid < 128:
    // row tid / 8, dims 8 (tid % 8) ..), requested with the Q rows
    float m0[8];
    {
        const int r = tid >> 3, c8 = (tid & 7) * 8;
        if (tid < 128 && r < Kc) {
            load8<T>(Qs + (long)init_row(r, L, Kc, init_step) * kD + c8, m0);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) m0[i] = 0.f;
        }
    }
    {
        float m = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) m = absmax8(qraw[u][1], absmax8(qraw[u][0], m));
        const uint32_t b = wave_max_u(__float_as_uint(m));
        if (lane == 0) sMax[4 * w] = b;
    }
    __syncthreads();
    {
        uint32_t m = 0;
#pragma unroll
        for (int ww = 0; ww < 16; ++ww) m = max(m, sMax[4 * ww]);
        sq = scale_shift(m, kQLimit);
    }
    fq = __builtin_ldexpf(1.f, -sq);
    Sp8 qf[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = qraw[u][c][i] * fq;
            qf[u][c] = split8<true>(x);
            const int o = (2048 * (w + 16 * u) + (lo.rl64 ^ (64 * c))) / 2;
            st16(sQ + o, qf[u][c].h);
            if (!kZ) st16(sQ + kGPlaneQ / 2 + o, qf[u][c].m);   // zero for bf16 storage, never read
        }
    if (tid < 128) {   // mu_k = Q[init_row(k)]; rows >= Kc: zero with a -inf part
        const int r = tid >> 3, c8 = (tid & 7) * 8;
        float x[8], n2 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = m0[i] * fq;
            n2 = fmaf(x[i], x[i], n2);
        }
        const Sp8 mp = split8(x);
        const int o = off64(r, c8);
        st16(sMu + o, mp.h);
        st16(sMu + kPlaneMuE + o, mp.m);
        n2 += __shfl_xor(n2, 1);
        n2 += __shfl_xor(n2, 2);
        n2 += __shfl_xor(n2, 4);
        const int c0 = (tid & 7) * 4;
        uint32_t h = 0, m = 0;
        if (r < Kc && c0 == 0) split2(-0.5f * n2, 0.f, h, m);
        uint32_t v0 = 0;
        if (c0 == 0) v0 = r < Kc ? ((h & 0xffffu) | ((m & 0xffffu) << 16)) : (uint32_t)kNegInfH;
        *reinterpret_cast<u32x2_t *>(sMuX + r * kGMuXCols + c0) = u32x2_t{v0, 0u};
    }
    __syncthreads();
    {
        const u32x4_t ones_g0 =
            g == 0 ? u32x4_t{kOneH2, kOneH2, kOneH2, kOneH2} : u32x4_t{0u, 0u, 0u, 0u};
        const u32x4_t ones = {kOneH2, kOneH2, kOneH2, kOneH2};
        const int dt = w & 3, qd = w >> 2;
        const int trq0 = 1024 * g + (lo.tr0 ^ (32 * dt)), trq1 = 1024 * g + (lo.tr4 ^ (32 * dt));
        for (int t = 1; t <= iters; ++t) {
            {
                const u32x4_t mx = ldb16(pMuX, 64 * l16 + 16 * g);
                const Sp8 mu0 = frag_at(pMu, kPlaneMu, lo.rl64), mu1 = frag_at(pMu, kPlaneMu, lo.rl64 ^ 64);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int tile = w + 16 * u;
                    if (FULL || tile < NT) {
                        f32x4_t a = mma(mx, ones_g0, kZero4);
                        a = mma3z<false, kZ>(mu0, qf[u][0], a);
                        a = mma3z<false, kZ>(mu1, qf[u][1], a);
                        float best = a[0];
                        int bk = 4 * g;
#pragma unroll
                        for (int rr = 1; rr < 4; ++rr) {
                            const bool up = a[rr] > best;
                            best = up ? a[rr] : best;
                            bk = up ? 4 * g + rr : bk;
                        }
                        bk = col_argmax(best, bk);
                        const int tok = 16 * tile + l16;
                        if (g == 0 && (FULL || tok < L)) {
                            sC[tok] = bk;
                            if (t == iters && assign) assign[s * L + tok] = bk;
                            if (HIST) hist[((long)(t - 1) * (SPLIT ? S : gridDim.x) + s) * L + tok] = bk;
                        }
                    }
                }
            }
            // the rows of key chunk w / 8 (phase 2's round 0), in flight
            // during the last update
            if (t == iters) load_chunk(w >> 3);
            __syncthreads();
            f32x4_t sh = kZero4, sm = kZero4, cnt = kZero4;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int cc = 4 * qd + c;
                if (FULL || 32 * cc < L) {
                    const int t0 = 32 * cc + 8 * g;
                    const int4 ca = *reinterpret_cast<const int4 *>(sC + t0);
                    const int4 cb = *reinterpret_cast<const int4 *>(sC + t0 + 4);
                    const int cv[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
                    uint32_t pk[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo16 =
                            ((FULL || t0 + 2 * e < L) && cv[2 * e] == l16) ? 0x3c00u : 0u;
                        const uint32_t hi16 =
                            ((FULL || t0 + 2 * e + 1 < L) && cv[2 * e + 1] == l16) ? 0x3c00u : 0u;
                        pk[e] = lo16 | (hi16 << 16);
                    }
                    const u32x4_t oh = {pk[0], pk[1], pk[2], pk[3]};
                    const Sp8 qt = colfrag8_at<kGPlaneQ>(pQ, 4096 * cc + trq0, 4096 * cc + trq1);
                    if (!kZ) sm = mma(qt.m, oh, sm);
                    sh = mma(qt.h, oh, sh);
                    cnt = mma(ones, oh, cnt);
                }
            }
            if (qd > 0) {
                float *pp = sPart + (((qd - 1) * 4 + dt) * 64 + lane) * 5;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) pp[rr] = sm[rr] + sh[rr];
                pp[4] = cnt[0];
            }
            __syncthreads();
            if (qd == 0) {
                float v[4], n = cnt[0];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = sm[rr] + sh[rr];
#pragma unroll
                for (int q2 = 0; q2 < 3; ++q2) {
                    const float *pp = sPart + ((q2 * 4 + dt) * 64 + lane) * 5;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) v[rr] += pp[rr];
                    n += pp[4];
                }
                const float inv = 1.0f / fmaxf(n, 1.f);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] *= inv;
                const Sp4 mu4 = split4(v[0], v[1], v[2], v[3]);
                float n2p = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) n2p = fmaf(v[rr], v[rr], n2p);
                n2p = col_sum(n2p);
                if (l16 < Kc) {
                    const int o = off64(l16, 16 * dt + 4 * g);
                    st8(sMu + o, mu4.h);
                    st8(sMu + kPlaneMuE + o, mu4.m);
                    if (g == 0) {
                        uint32_t h, m;
                        split2(-0.5f * n2p, 0.f, h, m);
                        sMuX[l16 * kGMuXCols + 2 * dt] = (uint16_t)(h & 0xffffu);
                        sMuX[l16 * kGMuXCols + 2 * dt + 1] = (uint16_t)(m & 0xffffu);
                    }
                }
            }
            __syncthreads();
        }
    }

    const int hf = w >> 3, wl = w & 7;   // the halves and context waves of phase 2
    // clustering workgroup: the final centroid planes, Q scale and
    // assignment for the window workgroup (flag value 2 epoch + 1) ...
    uint32_t *pv = pub + s * kPubStride;
    unsigned long long *flag = split_flag(epoch, s);
    __hip_atomic_store(pv + kPubMu + tid, reinterpret_cast<const uint32_t *>(sMu)[tid],
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // 2 kPlaneMu bytes
    if (tid == 0)
        __hip_atomic_store(pv + kPubSq, (uint32_t)sq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < L)
        __hip_atomic_store(pv + kPubC + tid, (uint32_t)sC[tid], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // every store complete ...
    __syncthreads();
    if (tid == 0)   // ... before the flag goes up
        __hip_atomic_store(flag, 2 * epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // ... then its own half (key chunks 0 and 1), whose record goes out next
    // (flag value 2 epoch + 2)
    float Mh, lh;
    f32x4_t ah;
    phase2(sq, 0, 1, true, Mh, lh, ah);
    if (hf == 0 && wl < 4) {
        uint32_t *e = pv + kPubPart + (wl * 64 + lane) * 6;
        const float rec[6] = {Mh, lh, ah[0], ah[1], ah[2], ah[3]};
#pragma unroll
        for (int i = 0; i < 6; ++i)
            __hip_atomic_store(e + i, __float_as_uint(rec[i]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
        __hip_atomic_store(flag, 2 * epoch + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Clears the flags of launch e's ring for S slices (before a launch that a
// graph records, whose replays repeat the same launch number).
__global__ void fused512_clear_flags_kernel(unsigned long long e, int S) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < S) *split_flag(e, i) = 0ull;
    if (i == 0) *split_err(e) = 0ull;
}

// launch numbers of the split form, per device
constexpr int kMaxDevices = 64;
std::atomic<unsigned long long> g_split_launches[kMaxDevices];

bool fused512_supported(int L, int Kc, int r) {
    return L > 128 && L <= kGL && Kc >= 1 && Kc <= kFK && r >= 0 && r <= 16;
}

size_t fused512_split_workspace_bytes(long S) {
    return ((sizeof(uint32_t) * (size_t)S * kPubStride + 255) / 256) * 256;
}

int fused512_split_max_slices() { return kMaxSplitSlices; }

hipError_t launch_fused512(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                           int iters, int r, float alpha, int init_step, ca_dtype_t dt, int H,
                           int G, void *out, int32_t *assign, hipStream_t st, int32_t *hist,
                           void *split_ws) {
    uint32_t *pub = nullptr;
    unsigned long long epoch = 0;
    const bool split = split_ws != nullptr;
    if (split) {
        if (S > kMaxSplitSlices || dt != CA_BF16) return hipErrorInvalidValue;
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        pub = static_cast<uint32_t *>(split_ws);
        epoch = g_split_launches[dev].fetch_add(1, std::memory_order_relaxed) + 1;
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(st, &cap);
        if (e != hipSuccess) return e;
        if (cap != hipStreamCaptureStatusNone)
            hipLaunchKernelGGL(fused512_clear_flags_kernel, dim3((unsigned)((S + 255) / 256)),
                               dim3(256), 0, st, epoch, S);
    }
    const dim3 grid((unsigned)(split ? 2 * S : S)), block(kGThreads);
#define CA_F512_ARGS(TT)                                                                         \
    static_cast<const TT *>(Q), static_cast<const TT *>(K), static_cast<const TT *>(V), L, Kc,   \
        iters, r, alpha, init_step, H, G, static_cast<TT *>(out), assign, hist
#define CA_F512_ONE(TT, HH, F)                                                                   \
    hipLaunchKernelGGL((cluster_attn_fused512_kernel<TT, HH, F>), grid, block, 0, st,            \
                       CA_F512_ARGS(TT))
#define CA_F512_SPLIT(HH, F)                                                                     \
    hipLaunchKernelGGL((cluster_attn_fused512_split_kernel<bf16_t, HH, F, true>), grid, block, 0, \
                       st, CA_F512_ARGS(bf16_t), S, pub, epoch)
    const bool full = L == kGL;
    if (dt == CA_BF16) {
        if (split) {
            if (hist) {
                if (full) CA_F512_SPLIT(true, true); else CA_F512_SPLIT(true, false);
            } else {
                if (full) CA_F512_SPLIT(false, true); else CA_F512_SPLIT(false, false);
            }
        } else if (hist) {
            if (full) CA_F512_ONE(bf16_t, true, true); else CA_F512_ONE(bf16_t, true, false);
        } else {
            if (full) CA_F512_ONE(bf16_t, false, true); else CA_F512_ONE(bf16_t, false, false);
        }
    } else {   // the split form is for bf16 storage only
        if (split) return hipErrorInvalidValue;
        if (hist) {
            if (full) CA_F512_ONE(float, true, true); else CA_F512_ONE(float, true, false);
        } else {
            if (full) CA_F512_ONE(float, false, true); else CA_F512_ONE(float, false, false);
        }
    }
#undef CA_F512_SPLIT
#undef CA_F512_ONE
#undef CA_F512_ARGS
    return hipGetLastError();
}

}  // namespace ca
