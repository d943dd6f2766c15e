// All Lloyd iterations of one slice in one launch, for L <= 512 and K <= 16
// (staged path): the assignment after the last iteration and the final
// centroids, on the fp16 matrix cores.
//
// Steps: model card "Hooshaai/distilbert-sst2-cluster-attention",
// Mathematical Formulation 1, and the "ClusterFormer" spec
// (svd-sst2-roberta-cluster page) 2.1: mu^(0)_k = Q[init_row(k)], then for
// t = 1..I: c_i = argmin_k ||q_i - mu_k||^2 (ties to the lowest index) and
// mu_k = sum_{c_i = k} q_i / max(1, n_k) (an empty cluster becomes zero).
//
// Work split: one workgroup of 16 waves per slice; wave w owns token tiles w
// and w + 16. Q lives in LDS as fp16 h/m planes of 512 rows for the whole
// launch and in registers as the waves' B fragments. Distances are the
// single-launch forward's chain (mu . q - ||mu||^2/2 with the norm parts in
// a 32-deep chunk). The update is a product with the one-hot matrix, whose
// fragments each lane builds in registers from the assignments in LDS
// (exact 0/1 weights): wave w sums dimension tile w % 4 over the token
// quarter w / 4, and the waves of quarter 0 add the other quarters in order,
// divide, split the new centroids into their planes and form the norm parts,
// as the single-launch forward does. Q is scaled by one power of two per
// slice (the centroids, means of its rows, follow); the centroids are scaled
// back exactly when stored.
#include "local_mfma_body.h"
#include "xattn_body.h"

namespace ca {
namespace {

constexpr int kSL = 512;                          // max tokens
constexpr int kSThreads = 1024;                   // 16 waves
constexpr int kSPlane = kSL * kD * 2;             // one fp16 plane [512][64]
constexpr int kSMuXCols = 32;
constexpr int kSOffQ = 0;                         // Q planes h, m
constexpr int kSOffMu = 2 * kSPlane;              // [16][64] h, m
constexpr int kSOffMuX = kSOffMu + 2 * kPlaneMu;  // [16][32] fp16 norm parts
constexpr int kSOffC = kSOffMuX + kFK * kSMuXCols * 2;   // [512] assignments
constexpr int kSOffPart = kSOffC + kSL * 4;       // [3 quarters][4 dim tiles][64 lanes][5]
constexpr int kSOffMax = kSOffPart + 3 * 4 * 64 * 5 * 4;
constexpr int kSLds = kSOffMax + 16 * 4;
static_assert(kSLds <= 163840, "one workgroup per CU");

}  // namespace

// HIST: hist receives c^(t) of every iteration t at hist[(t - 1) * S + s][L]
// (S slices in all). FULL: L is 512 (no bounds tests).
template <typename T, bool HIST, bool FULL>
__device__ __forceinline__ void kmeans_slice_body(const T *__restrict__ Q, int L, int Kc,
                                                  int iters, int init_step,
                                                  int32_t *__restrict__ assign,
                                                  float *__restrict__ mu_out, long s, int tid,
                                                  unsigned char *smem,
                                                  int32_t *__restrict__ hist, long S,
                                                  float *mu_tab = nullptr) {
    uint16_t *sQ = reinterpret_cast<uint16_t *>(smem + kSOffQ);
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kSOffMu);
    uint16_t *sMuX = reinterpret_cast<uint16_t *>(smem + kSOffMuX);
    int *sC = reinterpret_cast<int *>(smem + kSOffC);
    float *sPart = reinterpret_cast<float *>(smem + kSOffPart);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kSOffMax);
    const u8 *pQ = smem + kSOffQ, *pMu = smem + kSOffMu, *pMuX = smem + kSOffMuX;

    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    constexpr bool kZ = bf16_storage<T>();   // Q (K, V) planes with zero m parts
    const T *Qs = Q + s * (long)L * kD;
    const int NT = (L + 15) >> 4;
    const LaneOffs lo = lane_offsets(l16, g);

    // ------------------------------------------------------------ Q
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
        if (lane == 0) sMax[w] = b;
    }
    __syncthreads();
    int sq;
    {
        uint32_t m = 0;
#pragma unroll
        for (int ww = 0; ww < 16; ++ww) m = max(m, sMax[ww]);
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
            if (!kZ) st16(sQ + kSPlane / 2 + o, qf[u][c].m);   // zero for bf16 storage, never read
        }
    // initial centroids mu_k = Q[init_row(k)] (rows >= Kc: zero, -inf part)
    if (tid < 128) {
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
        *reinterpret_cast<u32x2_t *>(sMuX + r * kSMuXCols + c0) = u32x2_t{v0, 0u};
    }
    __syncthreads();

    const u32x4_t ones_g0 =
        g == 0 ? u32x4_t{kOneH2, kOneH2, kOneH2, kOneH2} : u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t ones = {kOneH2, kOneH2, kOneH2, kOneH2};
    const int dt = w & 3, qd = w >> 2;   // update: dimension tile, token quarter
    const int trq0 = 1024 * g + (lo.tr0 ^ (32 * dt)), trq1 = 1024 * g + (lo.tr4 ^ (32 * dt));
    for (int t = 1; t <= iters; ++t) {
        // ---------------------------------------------------- assignment
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
                        if (t == iters) assign[s * L + tok] = bk;
                        if (HIST) hist[((long)(t - 1) * S + s) * L + tok] = bk;
                    }
                }
            }
        }
        __syncthreads();
        // ---------------------------------------------------- update
        // this wave: dims 16 dt + 4g + rr of cluster l16 over tokens 128 qd ..
        f32x4_t sh = kZero4, sm = kZero4, cnt = kZero4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int cc = 4 * qd + c;   // 32-token chunk
            if (FULL || 32 * cc < L) {
                // one-hot B fragment: tokens 32cc + 8g .. +7 for cluster l16
                const int t0 = 32 * cc + 8 * g;
                const int4 ca = *reinterpret_cast<const int4 *>(sC + t0);
                const int4 cb = *reinterpret_cast<const int4 *>(sC + t0 + 4);
                const int cv[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
                uint32_t pk[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo16 = ((FULL || t0 + 2 * e < L) && cv[2 * e] == l16) ? 0x3c00u : 0u;
                    const uint32_t hi16 =
                        ((FULL || t0 + 2 * e + 1 < L) && cv[2 * e + 1] == l16) ? 0x3c00u : 0u;
                    pk[e] = lo16 | (hi16 << 16);
                }
                const u32x4_t oh = {pk[0], pk[1], pk[2], pk[3]};
                const Sp8 qt = colfrag8_at<kSPlane>(pQ, 4096 * cc + trq0, 4096 * cc + trq1);
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
            if (t == iters) {
                if (l16 < Kc) {
                    const float back = __builtin_ldexpf(1.f, sq);
                    const float4 f4 = make_float4(v[0] * back, v[1] * back, v[2] * back, v[3] * back);
                    *reinterpret_cast<float4 *>(mu_out + (s * Kc + l16) * kD + 16 * dt + 4 * g) = f4;
                    // the same rows for a centroid attention in this workgroup
                    if (mu_tab) *reinterpret_cast<float4 *>(mu_tab + l16 * kD + 16 * dt + 4 * g) = f4;
                }
            } else {
                const Sp4 mu4 = split4(v[0], v[1], v[2], v[3]);
                float n2p = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) n2p = fmaf(v[rr], v[rr], n2p);
                n2p = col_sum(n2p);   // over the 16 dims of tile dt
                if (l16 < Kc) {
                    const int o = off64(l16, 16 * dt + 4 * g);
                    st8(sMu + o, mu4.h);
                    st8(sMu + kPlaneMuE + o, mu4.m);
                    if (g == 0) {
                        uint32_t h, m;
                        split2(-0.5f * n2p, 0.f, h, m);
                        sMuX[l16 * kSMuXCols + 2 * dt] = (uint16_t)(h & 0xffffu);
                        sMuX[l16 * kSMuXCols + 2 * dt + 1] = (uint16_t)(m & 0xffffu);
                    }
                }
            }
        }
        __syncthreads();
    }
}

template <typename T, bool HIST, bool FULL>
__global__ __launch_bounds__(kSThreads, 1) void kmeans_slice_kernel(
    const T *__restrict__ Q, int L, int Kc, int iters, int init_step,
    int32_t *__restrict__ assign, float *__restrict__ mu_out, int32_t *__restrict__ hist) {
    __shared__ __align__(16) unsigned char smem[kSLds];
    kmeans_slice_body<T, HIST, FULL>(Q, L, Kc, iters, init_step, assign, mu_out, blockIdx.x,
                               threadIdx.x, smem, hist, gridDim.x);
}

// The clustering of S slices (workgroups 0 .. S-1) and, beside it, the window
// branch of every 128-query block (two blocks per later workgroup, one per
// half of its 16 waves, each with its own 80 KB of LDS), which stores
// alpha O^loc for a later gather: the window needs no clustering result.
constexpr int kKWLds = kSLds > 2 * kMLds ? kSLds : 2 * kMLds;
static_assert(kKWLds <= 163840, "one workgroup per CU");

template <typename T, bool MASKED_IN, bool HIST>
__global__ __launch_bounds__(kSThreads, 1) void kmeans_window_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx, int L, int Kc,
    int iters, int init_step, int32_t *__restrict__ assign_out, float *__restrict__ mu_out, int S,
    int rad, int nblk, float alpha, const uint8_t *__restrict__ valid_in, int H, int G,
    float *__restrict__ oloc, int32_t *__restrict__ hist) {
    __shared__ __align__(16) unsigned char smem[kKWLds];
    if ((int)blockIdx.x < S) {
        kmeans_slice_body<T, HIST, false>(Q, L, Kc, iters, init_step, assign_out, mu_out, blockIdx.x,
                                   threadIdx.x, smem, hist, S);
        return;
    }
    // window blocks: alpha O^loc only (no gather; padded query rows zero)
    const int half = threadIdx.x >> 9;   // uniform per wave
    local_window_block<T, MASKED_IN, true, false>(Q, Kx, Vx, L, rad, nblk, nullptr, nullptr, Kc,
                                                  alpha, valid_in, H, G, nullptr, nullptr, 0, oloc,
                                           smem + half * kMLds, threadIdx.x & (kThreads - 1),
                                           2 * (blockIdx.x - S) + half);
}

bool kmeans_window_supported(long S, int L, int Kc, int r) {
    return kmeans_slice_supported(L, Kc) && local_mfma_supported(r) &&
           (S * ((L + 127) / 128)) % 2 == 0;
}

hipError_t launch_kmeans_window(const void *Q, const void *K, const void *V, int S, int L,
                                int Kc, int iters, ca_dtype_t dt, int32_t *assign, float *mu,
                                int init_step, int r, float alpha, const uint8_t *valid, int H,
                                int G, float *oloc, hipStream_t st, int32_t *hist) {
    const int nblk = (L + 127) / 128;
    if (!kmeans_window_supported(S, L, Kc, r)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(S + (long)S * nblk / 2)), block(kSThreads);
#define CA_KW_LAUNCH(TT, M, HH)                                                                  \
    hipLaunchKernelGGL((kmeans_window_kernel<TT, M, HH>), grid, block, 0, st,                    \
                       static_cast<const TT *>(Q), static_cast<const TT *>(K),                   \
                       static_cast<const TT *>(V), L, Kc, iters, init_step, assign, mu, S, r,    \
                       nblk, alpha, valid, H, G, oloc, hist)
#define CA_KW_LAUNCH_H(TT, M)                                                                    \
    do {                                                                                         \
        if (hist) CA_KW_LAUNCH(TT, M, true); else CA_KW_LAUNCH(TT, M, false);                    \
    } while (0)
    if (dt == CA_BF16) {
        if (valid) CA_KW_LAUNCH_H(bf16_t, true); else CA_KW_LAUNCH_H(bf16_t, false);
    } else {
        if (valid) CA_KW_LAUNCH_H(float, true); else CA_KW_LAUNCH_H(float, false);
    }
#undef CA_KW_LAUNCH_H
#undef CA_KW_LAUNCH
    return hipGetLastError();
}

// The clustering of S slices followed, in the same launch, by their centroid
// attention over four 128-key ranges: two workgroups per slice both run the
// clustering (the same arithmetic, so the same assignments and centroids,
// which both store), keep the final centroids in LDS, and then each half of
// a workgroup's waves forms one key range's partial (workgroup s: ranges 0
// and 1, workgroup S + s: ranges 2 and 3), merged later in range order by
// the window kernel. The clustering's LDS is dead by then; the table of
// centroids lies past both halves' attention LDS.
constexpr int kKXTab = 2 * kXLdsM;                          // [16][64] fp32 centroids
constexpr int kKXLds = kKXTab + kFK * kD * 4;
static_assert(kSLds <= kKXTab && kKXLds <= 163840, "one workgroup per CU");

template <typename T, bool HIST, bool FULL>
__global__ __launch_bounds__(kSThreads, 1) void kmeans_xattn_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx, int L, int Kc,
    int iters, int init_step, int H, int G, int32_t *__restrict__ assign,
    float *__restrict__ mu_out, float *__restrict__ xpart, int32_t *__restrict__ hist, int S) {
    __shared__ __align__(16) unsigned char smem[kKXLds];
    const int part = (int)blockIdx.x >= S ? 1 : 0;
    const long s = (long)blockIdx.x - (long)part * S;
    float *tab = reinterpret_cast<float *>(smem + kKXTab);
    kmeans_slice_body<T, HIST, FULL>(Q, L, Kc, iters, init_step, assign, mu_out, s, threadIdx.x,
                                     smem, hist, S, tab);
    __syncthreads();   // the centroids are in the table; the clustering's LDS is free
    const int half = threadIdx.x >> 9;   // uniform per wave
    xattn_range<T, false, false, FULL>(tab, Kx, Vx, L, Kc, 4, nullptr, H, G, nullptr, xpart,
                                       nullptr, smem + half * kXLdsM, threadIdx.x & (kThreads - 1),
                                       s, 2 * part + half);
}

bool kmeans_xattn_supported(long S, int L, int Kc, int cus) {
    return kmeans_slice_supported(L, Kc) && xattn_splits(L) == 4 && 2 * S <= cus;
}

hipError_t launch_kmeans_xattn(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                               int iters, ca_dtype_t dt, int32_t *assign, float *mu,
                               int init_step, int H, int G, float *xpart, hipStream_t st,
                               int32_t *hist) {
    if (!kmeans_slice_supported(L, Kc) || xattn_splits(L) != 4) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(2 * S)), block(kSThreads);
#define CA_KX_LAUNCH(TT, HH, F)                                                                  \
    hipLaunchKernelGGL((kmeans_xattn_kernel<TT, HH, F>), grid, block, 0, st,                     \
                       static_cast<const TT *>(Q), static_cast<const TT *>(K),                   \
                       static_cast<const TT *>(V), L, Kc, iters, init_step, H, G, assign, mu,    \
                       xpart, hist, S)
#define CA_KX_LAUNCH_F(TT, HH)                                                                   \
    do {                                                                                         \
        if (L == kSL) CA_KX_LAUNCH(TT, HH, true); else CA_KX_LAUNCH(TT, HH, false);              \
    } while (0)
    if (dt == CA_BF16) {
        if (hist) CA_KX_LAUNCH_F(bf16_t, true); else CA_KX_LAUNCH_F(bf16_t, false);
    } else {
        if (hist) CA_KX_LAUNCH_F(float, true); else CA_KX_LAUNCH_F(float, false);
    }
#undef CA_KX_LAUNCH_F
#undef CA_KX_LAUNCH
    return hipGetLastError();
}

bool kmeans_slice_supported(int L, int Kc) { return L >= 1 && L <= kSL && Kc >= 1 && Kc <= kFK; }

hipError_t launch_kmeans_slice(const void *Q, int S, int L, int Kc, int iters, ca_dtype_t dt,
                               int32_t *assign, float *mu, int init_step, hipStream_t st,
                               int32_t *hist) {
    const dim3 grid((unsigned)S), block(kSThreads);
#define CA_KS_LAUNCH(TT, HH, F)                                                                  \
    hipLaunchKernelGGL((kmeans_slice_kernel<TT, HH, F>), grid, block, 0, st,                     \
                       static_cast<const TT *>(Q), L, Kc, iters, init_step, assign, mu, hist)
#define CA_KS_LAUNCH_F(TT, HH)                                                                   \
    do {                                                                                         \
        if (L == kSL) CA_KS_LAUNCH(TT, HH, true); else CA_KS_LAUNCH(TT, HH, false);              \
    } while (0)
    if (dt == CA_BF16) {
        if (hist) CA_KS_LAUNCH_F(bf16_t, true); else CA_KS_LAUNCH_F(bf16_t, false);
    } else {
        if (hist) CA_KS_LAUNCH_F(float, true); else CA_KS_LAUNCH_F(float, false);
    }
#undef CA_KS_LAUNCH_F
#undef CA_KS_LAUNCH
    return hipGetLastError();
}

}  // namespace ca
