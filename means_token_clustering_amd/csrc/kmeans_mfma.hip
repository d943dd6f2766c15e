// One Lloyd step (assignment + per-block cluster sums) on the fp16 matrix
// cores for the staged path (any L, K <= 64).
//
// Step: model card "Hooshaai/distilbert-sst2-cluster-attention",
// Mathematical Formulation 1, and the "ClusterFormer" spec
// (svd-sst2-roberta-cluster page) 2.1: c_i = argmin_k ||q_i - mu_k||^2, then
// mu_k = sum_{c_i = k} q_i / max(1, n_k). Here the score of cluster k for
// token i is mu_k . q_i - ||mu_k||^2 / 2 (the largest is the nearest); ties
// go to the lowest index.
//
// Work split: one workgroup (8 waves) per 128-token block of a slice; wave w
// owns token tile w, as in the single-launch forward. The centroids sit in
// LDS as fp16 h/m planes of up to 64 rows with their -||mu||^2/2 parts; each
// group of 16 clusters costs one chain of seven products per wave, and the
// running best over the groups keeps the earlier group on equal scores. The
// block's cluster sums and sizes are one-hot products of the same planes
// (Q^T times the [cluster][token] one-hot matrix, exact 0/1 weights), stored
// per block; centroid_reduce_kernel adds the blocks in a fixed order, or, for
// few blocks, the next step's workgroups add them themselves.
// Q and the centroids are scaled by one power of two per block (the largest
// |q| or |mu|), which leaves every comparison unchanged; the sums are scaled
// back exactly.
#include "launch.h"
#include "mfma_split.h"

namespace ca {
namespace {

constexpr int kKM = 64;                        // max clusters
constexpr int kKMuPlane = kKM * kD * 2;        // fp16 plane [64][64]
constexpr int kKOhPlane = kKM * kFL * 2;       // fp16 one-hot [64][128]
constexpr int kKMuXCols = 32;                  // [64][32] fp16: -||mu||^2/2 parts
constexpr int kKOffQ = 0;                      // Q planes [128][64] h, m
constexpr int kKOffMu = 2 * kPlane;
constexpr int kKOffOH = kKOffMu + 2 * kKMuPlane;
constexpr int kKOffMuX = kKOffOH + kKOhPlane;
constexpr int kKOffMax = kKOffMuX + kKM * kKMuXCols * 2;
constexpr int kKLds = kKOffMax + 8 * 4 * 4;
static_assert(kKLds <= 81920, "two workgroups per CU");

}  // namespace

template <typename T, bool INIT>
__global__ __launch_bounds__(kThreads, 4) void kmeans_mfma_kernel(
    const T *__restrict__ Q, const float *__restrict__ mu, int L, int Kc, int nblk,
    int32_t *__restrict__ assign, float *__restrict__ part_sum, int32_t *__restrict__ part_cnt,
    int init_step, float *__restrict__ mu_init, const float *__restrict__ prev_sum,
    const int32_t *__restrict__ prev_cnt) {
    __shared__ __align__(16) unsigned char smem[kKLds];
    uint16_t *sQ = reinterpret_cast<uint16_t *>(smem + kKOffQ);
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kKOffMu);
    uint16_t *sOH = reinterpret_cast<uint16_t *>(smem + kKOffOH);
    uint16_t *sMuX = reinterpret_cast<uint16_t *>(smem + kKOffMuX);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kKOffMax);
    const u8 *pQ = smem + kKOffQ, *pMu = smem + kKOffMu, *pOH = smem + kKOffOH,
             *pMuX = smem + kKOffMuX;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int blk = blockIdx.x % nblk;
    const long s = blockIdx.x / nblk;
    const T *Qs = Q + s * (long)L * kD;
    const int i0 = 128 * blk;
    const int Lb = min(128, L - i0);               // tokens of the block
    const int tok = 16 * w + l16;                  // the lane's token in the block
    const int NG = (Kc + 15) >> 4;                 // groups of 16 clusters
    const LaneOffs lo = lane_offsets(l16, g);

    // the wave's Q rows (dims 32c + 8g ..), zeros past the block
    float qraw[2][8];
#pragma unroll
    for (int c = 0; c < 2; ++c) load_row8<T, false>(Qs + (long)i0 * kD, tok, Lb, 32 * c + 8 * g, qraw[c]);
    // centroid row tid / 8, dims 8 (tid % 8) .. (zeros for rows >= Kc)
    const int mrow = tid >> 3, mcol = (tid & 7) * 8;
    float mraw[8];
    if (mrow < Kc) {
        if (INIT) {
            const long row = init_row(mrow, L, Kc, init_step);
            load8<T>(Qs + row * kD + mcol, mraw);
            if (mu_init && blk == 0) {
                *reinterpret_cast<float4 *>(mu_init + (s * Kc + mrow) * kD + mcol) =
                    make_float4(mraw[0], mraw[1], mraw[2], mraw[3]);
                *reinterpret_cast<float4 *>(mu_init + (s * Kc + mrow) * kD + mcol + 4) =
                    make_float4(mraw[4], mraw[5], mraw[6], mraw[7]);
            }
        } else if (prev_sum) {
            // the previous step's block sums of this slice, added in block
            // order, over max(1, n) (the update of centroid_reduce_kernel)
            float x[8];
            int n = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) mraw[i] = 0.f;
            for (int b2 = 0; b2 < nblk; ++b2) {
                const long pr = (s * nblk + b2) * (long)Kc + mrow;
                load8<float>(prev_sum + pr * kD + mcol, x);
#pragma unroll
                for (int i = 0; i < 8; ++i) mraw[i] += x[i];
                n += prev_cnt[pr];
            }
            const float dn = (float)(n > 1 ? n : 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) mraw[i] /= dn;
        } else {
            load8<float>(mu + (s * Kc + mrow) * kD + mcol, mraw);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) mraw[i] = 0.f;
    }
    {
        const float mq = absmax8(qraw[1], absmax8(qraw[0], absmax8(mraw, 0.f)));
        const uint32_t b = wave_max_u(__float_as_uint(mq));
        if (lane == 0) sMax[w] = b;
    }
    // one-hot matrix cleared (16 KB: 32 bytes per thread)
    reinterpret_cast<u32x4_t *>(sOH)[2 * tid] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t *>(sOH)[2 * tid + 1] = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();
    int sq;
    {
        uint32_t m = 0;
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) m = max(m, sMax[ww]);
        sq = scale_shift(m, kQLimit);
    }
    const float fq = __builtin_ldexpf(1.f, -sq);

    // Q planes + the wave's fragments; centroid planes and norm parts
    Sp8 qf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = qraw[c][i] * fq;
        qf[c] = split8(x);
        const int o = (2048 * w + (lo.rl64 ^ (64 * c))) / 2;   // row tok, cols 32c + 8g
        st16(sQ + o, qf[c].h);
        st16(sQ + kPlaneE + o, qf[c].m);
    }
    {
        float x[8], n2 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = mraw[i] * fq;
            n2 = fmaf(x[i], x[i], n2);
        }
        const Sp8 mp = split8(x);
        const int o = off64(mrow, mcol);
        st16(sMu + o, mp.h);
        st16(sMu + kKMuPlane / 2 + o, mp.m);
        // the row's eight lanes (tid % 8) add their parts in a fixed order
        n2 += __shfl_xor(n2, 1);
        n2 += __shfl_xor(n2, 2);
        n2 += __shfl_xor(n2, 4);
        // row mrow of the parts: (h, m) of -||mu||^2/2 in columns 0, 1; zero
        // elsewhere; -inf for clusters >= Kc so that they are never chosen
        const int c0 = (tid & 7) * 4;   // four columns per lane
        uint32_t h = 0, m = 0;
        if (mrow < Kc && c0 == 0) split2(-0.5f * n2, 0.f, h, m);
        uint32_t v0 = 0, v1 = 0;
        if (c0 == 0) {
            v0 = mrow < Kc ? ((h & 0xffffu) | ((m & 0xffffu) << 16)) : (uint32_t)kNegInfH;
        }
        *reinterpret_cast<u32x2_t *>(sMuX + mrow * kKMuXCols + c0) = u32x2_t{v0, v1};
    }
    __syncthreads();

    // ------------------------------------------------------------ assignment
    const bool tok_in = tok < Lb;
    {
        const u32x4_t ones_g0 =
            g == 0 ? u32x4_t{kOneH2, kOneH2, kOneH2, kOneH2} : u32x4_t{0u, 0u, 0u, 0u};
        float run = -__builtin_inff();
        int rk = 0;
        for (int kg = 0; kg < NG; ++kg) {
            const u32x4_t mx = ldb16(pMuX, 64 * (16 * kg + l16) + 16 * g);
            const Sp8 mu0 = frag_at(pMu, kKMuPlane, 2048 * kg + lo.rl64);
            const Sp8 mu1 = frag_at(pMu, kKMuPlane, 2048 * kg + (lo.rl64 ^ 64));
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t a = mma(mx, ones_g0, kZero4);
            a = mma3(mu0, qf[0], a);
            a = mma3(mu1, qf[1], a);
            float best = a[0];
            int bk = 16 * kg + 4 * g;
#pragma unroll
            for (int rr = 1; rr < 4; ++rr) {
                const bool up = a[rr] > best;
                best = up ? a[rr] : best;
                bk = up ? 16 * kg + 4 * g + rr : bk;
            }
            // (score, index) maximum over the column; lowest index on ties
            uint32_t x0, x1, i0a, i1a;
            pair16(__float_as_uint(best), x0, x1);
            pair16((uint32_t)bk, i0a, i1a);
            bool up = __uint_as_float(x1) > __uint_as_float(x0);
            best = up ? __uint_as_float(x1) : __uint_as_float(x0);
            bk = up ? (int)i1a : (int)i0a;
            pair32(__float_as_uint(best), x0, x1);
            pair32((uint32_t)bk, i0a, i1a);
            up = __uint_as_float(x1) > __uint_as_float(x0);
            best = up ? __uint_as_float(x1) : __uint_as_float(x0);
            bk = up ? (int)i1a : (int)i0a;
            if (kg == 0 || best > run) {
                run = best;
                rk = bk;
            }
        }
        if (g == 0 && tok_in) {
            assign[s * L + i0 + tok] = rk;
            sOH[off128(rk, tok)] = 0x3c00;   // fp16 1.0
        }
    }
    if (part_sum == nullptr) return;
    __syncthreads();

    // ------------------------------------------------------------ cluster sums
    // tile u = (dimension tile dt = u % 4, cluster group kg = u / 4): sums of
    // dims 16 dt + 4g + rr for cluster 16 kg + l16, and its size
    const long pb = (s * nblk + blk) * (long)Kc;
    const float back = __builtin_ldexpf(1.f, sq);
    const u32x4_t ones = {kOneH2, kOneH2, kOneH2, kOneH2};
    const int nch = (Lb + 31) >> 5;
    for (int u = w; u < 4 * NG; u += 8) {
        const int dt = u & 3, kg = u >> 2;
        const int trq0 = 1024 * g + (lo.tr0 ^ (32 * dt)), trq1 = 1024 * g + (lo.tr4 ^ (32 * dt));
        f32x4_t sh = kZero4, sm = kZero4, cnt = kZero4;
        for (int c = 0; c < nch; ++c) {
            const u32x4_t oh = ldb16(pOH, 4096 * kg + (lo.rl128 ^ (64 * c)));
            const Sp8 qt = colfrag8_at(pQ, 4096 * c + trq0, 4096 * c + trq1);
            sm = mma(qt.m, oh, sm);
            sh = mma(qt.h, oh, sh);
            if (dt == 0) cnt = mma(ones, oh, cnt);
        }
        const int k = 16 * kg + l16;
        if (k < Kc) {
            *reinterpret_cast<float4 *>(part_sum + (pb + k) * kD + 16 * dt + 4 * g) =
                make_float4((sm[0] + sh[0]) * back, (sm[1] + sh[1]) * back,
                            (sm[2] + sh[2]) * back, (sm[3] + sh[3]) * back);
            if (dt == 0 && g == 0) part_cnt[pb + k] = (int32_t)cnt[0];
        }
    }
}

bool kmeans_mfma_supported(int Kc) { return Kc >= 1 && Kc <= kKM; }
int kmeans_mfma_blocks(int L) { return (L + 127) / 128; }

template <typename T>
static hipError_t kmeans_mfma_dispatch(const void *Q, const float *mu, int S, int L, int Kc,
                                       int32_t *assign, float *part_sum, int32_t *part_cnt,
                                       hipStream_t st, int init_step, float *mu_init,
                                       const float *prev_sum, const int32_t *prev_cnt) {
    const int nblk = kmeans_mfma_blocks(L);
    const dim3 grid((unsigned)((long)S * nblk)), block(kThreads);
    const T *q = static_cast<const T *>(Q);
    if (mu == nullptr)
        hipLaunchKernelGGL((kmeans_mfma_kernel<T, true>), grid, block, 0, st, q, mu, L, Kc, nblk,
                           assign, part_sum, part_cnt, init_step, mu_init, prev_sum, prev_cnt);
    else
        hipLaunchKernelGGL((kmeans_mfma_kernel<T, false>), grid, block, 0, st, q, mu, L, Kc, nblk,
                           assign, part_sum, part_cnt, init_step, mu_init, prev_sum, prev_cnt);
    return hipGetLastError();
}

hipError_t launch_kmeans_mfma(const void *Q, const float *mu, int S, int L, int Kc,
                              ca_dtype_t dt, int32_t *assign, float *part_sum, int32_t *part_cnt,
                              hipStream_t st, int init_step, float *mu_init,
                              const float *prev_sum, const int32_t *prev_cnt) {
    if (dt == CA_BF16)
        return kmeans_mfma_dispatch<bf16_t>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st,
                                            init_step, mu_init, prev_sum, prev_cnt);
    return kmeans_mfma_dispatch<float>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st,
                                       init_step, mu_init, prev_sum, prev_cnt);
}

}  // namespace ca
