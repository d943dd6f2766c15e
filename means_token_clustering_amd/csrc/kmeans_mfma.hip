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
// Work split: one workgroup (8 waves) per run of up to nsub consecutive
// 128-token blocks of a slice (nsub = 1 when the blocks fill the chip at most
// two deep); wave w owns token tile w of each block, as in the single-launch
// forward. The workgroup takes its blocks in order, requesting the next
// block's Q rows while it scores the current one, and keeps the run's cluster
// sums in fp32 registers (block sums added in block order), so a run of nsub
// blocks writes one partial instead of nsub. The centroids sit in
// LDS as fp16 h/m planes of up to 64 rows with their -||mu||^2/2 parts; each
// group of 16 clusters costs one chain of seven products per wave (five for
// bf16 storage), and the running best over the groups keeps the earlier
// group on equal scores. The
// block's cluster sums and sizes are one-hot products of the same planes
// (Q^T times the [cluster][token] one-hot matrix, exact 0/1 weights), stored
// per run; centroid_reduce_kernel adds the runs in a fixed order, or, for
// few blocks, the next step's workgroups add them themselves.
// Q and the centroids are scaled by one power of two per block (the largest
// |q| or |mu|), or, in the steps after the first of a run launch, per run
// (the run's largest |q| recorded by the first step), which leaves every
// comparison unchanged; the sums are scaled back exactly.
#include <type_traits>

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

// SCORES: instead of the assignment, write every score mu_k . q_i -
// ||mu_k||^2 / 2 in unscaled units to scores [S, L, Kc] (no partials).
// RUN: runs of nsub blocks per workgroup; else one block (nsub is 1).
// qmax (RUN, nullable): the run's largest |q| (float bits), [S, runs]; the
// first step (INIT) writes it, and with FIXED a later step takes it: one
// scale for the whole run (with the centroids' maximum), the centroid planes
// built once, no per-block maximum. Each block's own scale gives the same
// products (power-of-two scaling is exact), so only fp16 subnormals differ.
// K64: all four groups of 16 clusters are present (Kc > 48). The groups'
// score chains are then independent products and one (score, index) maximum
// runs over the lane's 16 clusters before the column, and the two sum tiles
// of a wave (same dimension tile, cluster groups kg and kg + 2) share their Q
// fragments; every result is the one of the group-by-group form. FB: L is
// a multiple of 128, so every block holds 128 tokens (no bounds tests).
template <typename T, bool INIT, bool SCORES, bool RUN, bool FIXED, bool K64, bool FB>
__global__ __launch_bounds__(kThreads, 4) void kmeans_mfma_kernel(
    const T *__restrict__ Q, const float *__restrict__ mu, int L, int Kc, int nblk, int nsub,
    int32_t *__restrict__ assign, float *__restrict__ part_sum, int32_t *__restrict__ part_cnt,
    int init_step, float *__restrict__ mu_init, const float *__restrict__ prev_sum,
    const int32_t *__restrict__ prev_cnt, float *__restrict__ scores,
    uint32_t *__restrict__ qmax) {
    static_assert(!FIXED || (RUN && !INIT && !SCORES), "a fixed run scale is for later steps");
    static_assert(!K64 || !SCORES, "the score dump takes the group-by-group form");
    __shared__ __align__(16) unsigned char smem[kKLds];
    uint16_t *sQ = reinterpret_cast<uint16_t *>(smem + kKOffQ);
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kKOffMu);
    uint16_t *sOH = reinterpret_cast<uint16_t *>(smem + kKOffOH);
    uint16_t *sMuX = reinterpret_cast<uint16_t *>(smem + kKOffMuX);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kKOffMax);
    const u8 *pQ = smem + kKOffQ, *pMu = smem + kKOffMu, *pOH = smem + kKOffOH,
             *pMuX = smem + kKOffMuX;

    const int tid = threadIdx.x;
    constexpr bool kZ = bf16_storage<T>();   // Q (K, V) planes with zero m parts
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    // runs of nsub blocks; the slices' shorter last runs come after all the
    // full runs, so that they are the workgroups of a second round
    const unsigned nfull = (unsigned)(nblk / nsub), npart = (unsigned)((nblk + nsub - 1) / nsub);
    const unsigned nfw = gridDim.x / npart * nfull;   // workgroups of full runs
    unsigned s32, part;
    if (!RUN) {
        s32 = blockIdx.x / (unsigned)nblk;
        part = blockIdx.x - s32 * (unsigned)nblk;
    } else if (blockIdx.x < nfw) {
        s32 = blockIdx.x / nfull;
        part = blockIdx.x - s32 * nfull;
    } else {
        s32 = blockIdx.x - nfw;
        part = nfull;
    }
    const long s = s32;
    const int b0 = RUN ? (int)part * nsub : (int)part;
    const int b1 = RUN ? min(nblk, b0 + nsub) : b0 + 1;
    const T *Qs = Q + s * (long)L * kD;
    const int tok = 16 * w + l16;                  // the lane's token in a block
    const int NG = K64 ? 4 : (Kc + 15) >> 4;       // groups of 16 clusters
    const LaneOffs lo = lane_offsets(l16, g);

    // the wave's Q rows of the first block (dims 32c + 8g ..), zeros past it
    float qraw[2][8];
    {
        const int Lb0 = FB ? 128 : min(128, L - 128 * b0);
#pragma unroll
        for (int c = 0; c < 2; ++c)
            load_row8<T, FB>(Qs + (long)(128 * b0) * kD, tok, Lb0, 32 * c + 8 * g, qraw[c]);
    }
    // centroid row tid / 8, dims 8 (tid % 8) .. (zeros for rows >= Kc)
    const int mrow = tid >> 3, mcol = (tid & 7) * 8;
    float mraw[8];
    if (mrow < Kc) {
        if (INIT) {
            const long row = init_row(mrow, L, Kc, init_step);
            load8<T>(Qs + row * kD + mcol, mraw);
            if (mu_init && part == 0) {
                *reinterpret_cast<float4 *>(mu_init + (s * Kc + mrow) * kD + mcol) =
                    make_float4(mraw[0], mraw[1], mraw[2], mraw[3]);
                *reinterpret_cast<float4 *>(mu_init + (s * Kc + mrow) * kD + mcol + 4) =
                    make_float4(mraw[4], mraw[5], mraw[6], mraw[7]);
            }
        } else if (prev_sum) {
            // the previous step's run sums of this slice, added in run order,
            // over max(1, n) (the update of centroid_reduce_kernel)
            float x[8];
            int n = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) mraw[i] = 0.f;
            for (int b2 = 0; b2 < (int)npart; ++b2) {
                const long pr = (s * (long)npart + b2) * (long)Kc + mrow;
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
    const float mmax = absmax8(mraw, 0.f);
    {   // the centroids' largest magnitude, published by the first barrier below
        const uint32_t b = wave_max_u(__float_as_uint(mmax));
        if (lane == 0) sMax[8 + w] = b;
    }
    // centroid planes and -||mu||^2/2 parts at scale 2^-sq
    auto mu_planes = [&](float fq) {
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
    };
    int sq = 0;
    float fq = 1.f;
    if constexpr (FIXED) {
        __syncthreads();
        uint32_t m = qmax[s * (long)npart + part];
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) m = max(m, sMax[8 + ww]);
        sq = scale_shift(m, kQLimit);
        fq = __builtin_ldexpf(1.f, -sq);
        mu_planes(fq);
        // one-hot matrix cleared once: afterwards each token's lane resets
        // the one entry it set (its own column) before setting the next
        reinterpret_cast<u32x4_t *>(sOH)[2 * tid] = u32x4_t{0u, 0u, 0u, 0u};
        reinterpret_cast<u32x4_t *>(sOH)[2 * tid + 1] = u32x4_t{0u, 0u, 0u, 0u};
        __syncthreads();
    }
    uint32_t runq = 0;   // the run's largest |q| so far (INIT with qmax)
    int set_k = -1;      // FIXED: the cluster of this lane's one-hot entry (-1: none)

    // the run's cluster sums: tile u = w + 8 j (dimension tile u % 4, cluster
    // group u / 4), four dims per lane, and the tile's cluster sizes
    float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float accn[2] = {0.f, 0.f};

    for (int blk = b0; blk < b1; ++blk) {
    const int i0 = 128 * blk;
    const int Lb = FB ? 128 : min(128, L - i0);    // tokens of the block
    if constexpr (!FIXED) {
        const float mq = absmax8(qraw[1], absmax8(qraw[0], 0.f));
        const uint32_t b = wave_max_u(__float_as_uint(mq));
        if (lane == 0) sMax[w] = b;
    }
    if constexpr (FIXED) {
        // the previous block's entry of this lane's column (every wave has
        // read the matrix: the last barrier followed the sums)
        if (set_k >= 0) sOH[off128(set_k, tok)] = 0;
        set_k = -1;
    } else {
        // one-hot matrix cleared (16 KB: 32 bytes per thread)
        reinterpret_cast<u32x4_t *>(sOH)[2 * tid] = u32x4_t{0u, 0u, 0u, 0u};
        reinterpret_cast<u32x4_t *>(sOH)[2 * tid + 1] = u32x4_t{0u, 0u, 0u, 0u};
        __syncthreads();
        uint32_t mq = 0, m = 0;
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) {
            mq = max(mq, sMax[ww]);
            m = max(m, sMax[8 + ww]);
        }
        runq = max(runq, mq);
        sq = scale_shift(max(m, mq), kQLimit);
        fq = __builtin_ldexpf(1.f, -sq);
    }

    // Q planes + the wave's fragments; centroid planes and norm parts
    Sp8 qf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = qraw[c][i] * fq;
        qf[c] = split8<true>(x);
        const int o = (2048 * w + (lo.rl64 ^ (64 * c))) / 2;   // row tok, cols 32c + 8g
        st16(sQ + o, qf[c].h);
        if (!kZ) st16(sQ + kPlaneE + o, qf[c].m);   // zero for bf16 storage, never read
    }
    // FIXED: the centroid planes are already published and the assignment
    // reads only registers and them, so the Q planes go out with the one-hot
    // matrix at the next barrier
    if constexpr (!FIXED) {
        mu_planes(fq);
        __syncthreads();
    }
    // the next block's Q rows, in flight while this block is scored
    if (blk + 1 < b1) {
        const int Ln = FB ? 128 : min(128, L - i0 - 128);
#pragma unroll
        for (int c = 0; c < 2; ++c)
            load_row8<T, FB>(Qs + (long)(i0 + 128) * kD, tok, Ln, 32 * c + 8 * g, qraw[c]);
    }

    // ------------------------------------------------------------ assignment
    const bool tok_in = tok < Lb;
    {
        const u32x4_t ones_g0 =
            g == 0 ? u32x4_t{kOneH2, kOneH2, kOneH2, kOneH2} : u32x4_t{0u, 0u, 0u, 0u};
        float run = -__builtin_inff();
        int rk = 0;
        if constexpr (K64) {
            // four independent chains, then the lane's best of its clusters
            // 16 kg + 4 g + rr in index order (strictly larger replaces)
            f32x4_t a[4];
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) {
                const u32x4_t mx = ldb16(pMuX, 64 * (16 * kg + l16) + 16 * g);
                const Sp8 mu0 = frag_at(pMu, kKMuPlane, 2048 * kg + lo.rl64);
                const Sp8 mu1 = frag_at(pMu, kKMuPlane, 2048 * kg + (lo.rl64 ^ 64));
                a[kg] = mma(mx, ones_g0, kZero4);
                a[kg] = mma3z<false, kZ>(mu0, qf[0], a[kg]);
                a[kg] = mma3z<false, kZ>(mu1, qf[1], a[kg]);
            }
            float best = a[0][0];
            int bk = 4 * g;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg)
#pragma unroll
                for (int rr = kg == 0 ? 1 : 0; rr < 4; ++rr) {
                    const bool up = a[kg][rr] > best;
                    best = up ? a[kg][rr] : best;
                    bk = up ? 16 * kg + 4 * g + rr : bk;
                }
            // over the column's four lane groups: the larger score, the lower
            // index on equal scores
            uint32_t x0, x1, i0a, i1a;
            pair16(__float_as_uint(best), x0, x1);
            pair16((uint32_t)bk, i0a, i1a);
            bool up = __uint_as_float(x1) > __uint_as_float(x0) ||
                      (__uint_as_float(x1) == __uint_as_float(x0) && i1a < i0a);
            best = up ? __uint_as_float(x1) : __uint_as_float(x0);
            bk = up ? (int)i1a : (int)i0a;
            pair32(__float_as_uint(best), x0, x1);
            pair32((uint32_t)bk, i0a, i1a);
            up = __uint_as_float(x1) > __uint_as_float(x0) ||
                 (__uint_as_float(x1) == __uint_as_float(x0) && i1a < i0a);
            rk = up ? (int)i1a : (int)i0a;
        }
        for (int kg = 0; !K64 && kg < NG; ++kg) {
            const u32x4_t mx = ldb16(pMuX, 64 * (16 * kg + l16) + 16 * g);
            const Sp8 mu0 = frag_at(pMu, kKMuPlane, 2048 * kg + lo.rl64);
            const Sp8 mu1 = frag_at(pMu, kKMuPlane, 2048 * kg + (lo.rl64 ^ 64));
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t a = mma(mx, ones_g0, kZero4);
            a = mma3z<false, kZ>(mu0, qf[0], a);
            a = mma3z<false, kZ>(mu1, qf[1], a);
            if (SCORES) {   // both operands carry 2^-sq: the score carries 2^-2sq
                const float up2 = __builtin_ldexpf(1.f, 2 * sq);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int k = 16 * kg + 4 * g + rr;
                    if (tok_in && k < Kc) scores[(s * L + i0 + tok) * (long)Kc + k] = a[rr] * up2;
                }
                continue;
            }
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
        if (!SCORES && g == 0 && tok_in) {
            assign[s * L + i0 + tok] = rk;
            sOH[off128(rk, tok)] = 0x3c00;   // fp16 1.0
            if (FIXED) set_k = rk;
        }
    }
    if (!SCORES && part_sum != nullptr) {
    __syncthreads();

    // ------------------------------------------------------------ cluster sums
    // tile u = (dimension tile dt = u % 4, cluster group kg = u / 4): sums of
    // dims 16 dt + 4g + rr for cluster 16 kg + l16, and its size
    const float back = __builtin_ldexpf(1.f, sq);
    const u32x4_t ones = {kOneH2, kOneH2, kOneH2, kOneH2};
    if constexpr (K64) {
        // tiles u = w and w + 8 together: dimension tile w % 4, cluster
        // groups w / 4 and w / 4 + 2, one Q fragment per chunk for both
        const int dt = w & 3, kg = w >> 2;
        const int trq0 = 1024 * g + (lo.tr0 ^ (32 * dt)), trq1 = 1024 * g + (lo.tr4 ^ (32 * dt));
        f32x4_t sh0 = kZero4, sm0 = kZero4, cn0 = kZero4, sh1 = kZero4, sm1 = kZero4, cn1 = kZero4;
        auto chunk2 = [&](int c) {
            const Sp8 qt = colfrag8_at(pQ, 4096 * c + trq0, 4096 * c + trq1);
            const u32x4_t oh0 = ldb16(pOH, 4096 * kg + (lo.rl128 ^ (64 * c)));
            const u32x4_t oh1 = ldb16(pOH, 4096 * (kg + 2) + (lo.rl128 ^ (64 * c)));
            if (!kZ) {
                sm0 = mma(qt.m, oh0, sm0);
                sm1 = mma(qt.m, oh1, sm1);
            }
            sh0 = mma(qt.h, oh0, sh0);
            sh1 = mma(qt.h, oh1, sh1);
            if (dt == 0) {
                cn0 = mma(ones, oh0, cn0);
                cn1 = mma(ones, oh1, cn1);
            }
        };
        if constexpr (RUN) {
#pragma unroll
            for (int c = 0; c < 4; ++c) chunk2(c);
        } else {
            const int nch = (Lb + 31) >> 5;
            for (int c = 0; c < nch; ++c) chunk2(c);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            acc[0][rr] += (sm0[rr] + sh0[rr]) * back;
            acc[1][rr] += (sm1[rr] + sh1[rr]) * back;
        }
        accn[0] += cn0[0];
        accn[1] += cn1[0];
    }
#pragma unroll
    for (int j = 0; !K64 && j < 2; ++j) {
        const int u = w + 8 * j;
        if (u >= 4 * NG) break;
        const int dt = u & 3, kg = u >> 2;
        const int trq0 = 1024 * g + (lo.tr0 ^ (32 * dt)), trq1 = 1024 * g + (lo.tr4 ^ (32 * dt));
        // the chunks of 32 tokens: in a run all four (past the block's tokens
        // the Q planes and the one-hot rows are zero, so those products add
        // exact zeros), unrolled; a single block stops at its last chunk
        f32x4_t sh = kZero4, sm = kZero4, cnt = kZero4;
        auto chunk = [&](int c) {
            const u32x4_t oh = ldb16(pOH, 4096 * kg + (lo.rl128 ^ (64 * c)));
            const Sp8 qt = colfrag8_at(pQ, 4096 * c + trq0, 4096 * c + trq1);
            if (!kZ) sm = mma(qt.m, oh, sm);
            sh = mma(qt.h, oh, sh);
            if (dt == 0) cnt = mma(ones, oh, cnt);
        };
        if constexpr (RUN) {
#pragma unroll
            for (int c = 0; c < 4; ++c) chunk(c);
        } else {
            const int nch = (Lb + 31) >> 5;
            for (int c = 0; c < nch; ++c) chunk(c);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[j][rr] += (sm[rr] + sh[rr]) * back;
        accn[j] += cnt[0];
    }
    }
    if (blk + 1 < b1) __syncthreads();   // the planes and the one-hot matrix are rewritten
    }   // blocks of the run
    if (INIT && RUN && qmax != nullptr && tid == 0) qmax[s * (long)npart + part] = runq;
    if (SCORES || part_sum == nullptr) return;

    // the run's sums and sizes
    const long pb = (s * (long)npart + part) * (long)Kc;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int u = w + 8 * j;
        if (u >= 4 * NG) break;
        const int dt = u & 3, k = 16 * (u >> 2) + l16;
        if (k < Kc) {
            *reinterpret_cast<float4 *>(part_sum + (pb + k) * kD + 16 * dt + 4 * g) =
                make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
            if (dt == 0 && g == 0) part_cnt[pb + k] = (int32_t)accn[j];
        }
    }
}

bool kmeans_mfma_supported(int Kc) { return Kc >= 1 && Kc <= kKM; }
int kmeans_mfma_blocks(int L) { return (L + 127) / 128; }

// Blocks per workgroup: one while the blocks fill the compute units at most
// two deep (every workgroup resident in the first round), else runs of
// kRunBlocks, which leaves about one run per compute unit for long slices.
constexpr int kRunBlocks = 3;
int kmeans_mfma_run(long S, int L, int cus) {
    const int nblk = kmeans_mfma_blocks(L);
    if (S * nblk <= 2L * cus) return 1;
    return nblk < kRunBlocks ? nblk : kRunBlocks;
}
int kmeans_mfma_parts(int L, int nsub) { return (kmeans_mfma_blocks(L) + nsub - 1) / nsub; }

template <typename T>
static hipError_t kmeans_mfma_dispatch(const void *Q, const float *mu, int S, int L, int Kc,
                                       int32_t *assign, float *part_sum, int32_t *part_cnt,
                                       hipStream_t st, int init_step, float *mu_init,
                                       const float *prev_sum, const int32_t *prev_cnt,
                                       int nsub, uint32_t *qmax) {
    const int nblk = kmeans_mfma_blocks(L);
    const dim3 grid((unsigned)((long)S * kmeans_mfma_parts(L, nsub))), block(kThreads);
    const T *q = static_cast<const T *>(Q);
    float *const no_scores = nullptr;
    uint32_t *const qm = nsub > 1 ? qmax : nullptr;
    auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, q, mu, L, Kc, nblk, nsub, assign, part_sum,
                           part_cnt, init_step, mu_init, prev_sum, prev_cnt, no_scores, qm);
    };
    // runs of blocks over slices of whole blocks drop the bounds tests
    const bool fb = nsub > 1 && L % 128 == 0;
    auto pick = [&](auto k64) {
        constexpr bool K = decltype(k64)::value;
        if (mu == nullptr) {
            if (fb) launch(kmeans_mfma_kernel<T, true, false, true, false, K, true>);
            else if (nsub > 1) launch(kmeans_mfma_kernel<T, true, false, true, false, K, false>);
            else launch(kmeans_mfma_kernel<T, true, false, false, false, K, false>);
        } else {
            if (nsub > 1 && qm && !prev_sum) {
                if (fb) launch(kmeans_mfma_kernel<T, false, false, true, true, K, true>);
                else launch(kmeans_mfma_kernel<T, false, false, true, true, K, false>);
            } else if (nsub > 1) {
                launch(kmeans_mfma_kernel<T, false, false, true, false, K, false>);
            } else {
                launch(kmeans_mfma_kernel<T, false, false, false, false, K, false>);
            }
        }
    };
    if (Kc > 48) pick(std::true_type{});
    else pick(std::false_type{});
    return hipGetLastError();
}

template <typename T>
static hipError_t kmeans_scores_dispatch(const void *Q, const float *mu, int S, int L, int Kc,
                                         float *scores, hipStream_t st) {
    const int nblk = kmeans_mfma_blocks(L);
    const dim3 grid((unsigned)((long)S * nblk)), block(kThreads);
    hipLaunchKernelGGL((kmeans_mfma_kernel<T, false, true, false, false, false, false>), grid, block, 0, st,
                       static_cast<const T *>(Q), mu, L, Kc, nblk, 1, (int32_t *)nullptr,
                       (float *)nullptr, (int32_t *)nullptr, 0, (float *)nullptr,
                       (const float *)nullptr, (const int32_t *)nullptr, scores,
                       (uint32_t *)nullptr);
    return hipGetLastError();
}

hipError_t launch_kmeans_scores(const void *Q, const float *mu, int S, int L, int Kc,
                                ca_dtype_t dt, float *scores, hipStream_t st) {
    if (dt == CA_BF16) return kmeans_scores_dispatch<bf16_t>(Q, mu, S, L, Kc, scores, st);
    return kmeans_scores_dispatch<float>(Q, mu, S, L, Kc, scores, st);
}

hipError_t launch_kmeans_mfma(const void *Q, const float *mu, int S, int L, int Kc,
                              ca_dtype_t dt, int32_t *assign, float *part_sum, int32_t *part_cnt,
                              hipStream_t st, int init_step, float *mu_init,
                              const float *prev_sum, const int32_t *prev_cnt, int nsub,
                              uint32_t *qmax) {
    if (nsub < 1) return hipErrorInvalidValue;
    if (dt == CA_BF16)
        return kmeans_mfma_dispatch<bf16_t>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st,
                                            init_step, mu_init, prev_sum, prev_cnt, nsub, qmax);
    return kmeans_mfma_dispatch<float>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st,
                                       init_step, mu_init, prev_sum, prev_cnt, nsub, qmax);
}

}  // namespace ca
