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

bool fused512_supported(int L, int Kc, int r) {
    return L > 128 && L <= kGL && Kc >= 1 && Kc <= kFK && r >= 0 && r <= 16;
}

hipError_t launch_fused512(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                           int iters, int r, float alpha, int init_step, ca_dtype_t dt, int H,
                           int G, void *out, int32_t *assign, hipStream_t st, int32_t *hist) {
    const dim3 grid((unsigned)S), block(kGThreads);
#define CA_F512_LAUNCH(TT, HH, F)                                                                \
    hipLaunchKernelGGL((cluster_attn_fused512_kernel<TT, HH, F>), grid, block, 0, st,            \
                       static_cast<const TT *>(Q), static_cast<const TT *>(K),                   \
                       static_cast<const TT *>(V), L, Kc, iters, r, alpha, init_step, H, G,      \
                       static_cast<TT *>(out), assign, hist)
#define CA_F512_LAUNCH_F(TT, HH)                                                                 \
    do {                                                                                         \
        if (L == kGL) CA_F512_LAUNCH(TT, HH, true); else CA_F512_LAUNCH(TT, HH, false);          \
    } while (0)
    if (dt == CA_BF16) {
        if (hist) CA_F512_LAUNCH_F(bf16_t, true); else CA_F512_LAUNCH_F(bf16_t, false);
    } else {
        if (hist) CA_F512_LAUNCH_F(float, true); else CA_F512_LAUNCH_F(float, false);
    }
#undef CA_F512_LAUNCH_F
#undef CA_F512_LAUNCH
    return hipGetLastError();
}

}  // namespace ca
