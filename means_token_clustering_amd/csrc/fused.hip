// Single-launch cluster attention forward for short sequences (L <= 128,
// K <= 16, d = 64). One workgroup (512 threads, 8 waves) runs the whole path
// of one (b, h) slice on chip - Lloyd's k-means, centroid cross-attention,
// the local window branch and the gather + convex fusion - and touches HBM
// only to read Q, K, V once and to write the output and the assignment. At
// most 128 VGPRs per lane and 80,768 bytes of LDS let two slices share a CU,
// so one slice's loads and barriers overlap the other's arithmetic.
//
// Method: model card "Hooshaai/distilbert-sst2-cluster-attention",
// Architecture Overview figure and Mathematical Formulation 1; "ClusterFormer"
// spec (svd-sst2-roberta-cluster page) 2.1 and 3. Conventions as in the
// staged kernels: ties to the lowest cluster, empty cluster -> zero vector,
// window |i - j| <= radius (floor(W/2) by default), scale 1/sqrt(d); the
// listing-compatible variants (initial rows, kept empty clusters, soft
// gather) are selected per launch.
//
// Arithmetic. Every contraction runs on the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16, fp32 accumulation). Each operand
// tensor of a slice is first scaled by a power of two 2^-s (exact, only when
// its largest magnitude is outside [2^-3, 2^5) for Q or [2^-3, 2^15) for K
// and V, and then into the top binade of that range); each
// scaled fp32 value x is then split into two fp16 parts x = h + m + e (h = x
// rounded toward zero to fp16, m = the remainder x - h rounded to nearest
// fp16), which leaves |e| <= 2^-21 |x| (2^-25 absolute below the fp16 normal
// range). A product a.b accumulates h.h, h.m and m.h: the dropped terms are
// below 2^-19 |a||b| per element pair. Products with an exact 0/1
// operand (one-hot cluster sums, counts) are exact up to fp32 accumulation.
// The scale factors are undone on the fp32 results (scores, outputs);
// distances stay in the scaled units of Q, which leaves every comparison
// unchanged.
//
// Distances. The score of cluster k for token i is mu_k . q_i - ||mu_k||^2/2
// (the largest score is the nearest centroid). The -||mu_k||^2/2 term rides in
// the same MFMA chain as an extra 32-deep chunk: row k of that chunk holds the
// fp16 split parts of four partial sums over 16 dimensions each, and the
// query side holds ones, so the matrix core adds them.
//
// Layouts (confirmed on gfx950): for 16x16x32, lane l holds A[l%16][8(l/16)+i]
// and B[8(l/16)+i][l%16], i = 0..7; the 16x16 result has lane l, register r
// at D[4(l/16)+r][l%16]. Write
// l16 = l%16 and g = l/16. ds_read_b64_tr_b16: within each group of 16 lanes,
// if lane j points at 4 consecutive 16-bit values X_j[0..3], lane i receives
// X_{4e + i/4}[i%4] for e = 0..3; pointing lane j at row r0 + j/4, column
// c0 + 4(j%4) of a row-major plane therefore hands lane i the column c0 + i,
// rows r0 .. r0+3: a transposed MFMA operand straight from LDS.
//
// Work split per slice (tile = 16 tokens, NT = ceil(L/16) <= 8): wave w owns
// token tile w (distances, local branch, output rows) and key tile w
// (centroid-key scores); waves 0-3 also own dimension tile w (cluster sums and
// the centroid context). Q, K, V live in LDS as fp16 h/m planes [128][64]
// with 16-byte chunks XOR-swizzled by the row; V takes the place of Q once
// the clustering is done.
#include "launch.h"
#include "mfma_split.h"

namespace ca {
namespace {

// LDS map (bytes)
constexpr int kMuXCols = 32;                  // [16][32] fp16: -||mu||^2/2 parts
constexpr int kVcRow = 68;                    // fp32 V^cent row stride
constexpr int kOffK = 0;
constexpr int kOffQV = kOffK + 2 * kPlane;    // Q planes, then V planes
constexpr int kOffMu = kOffQV + 2 * kPlane;
constexpr int kOffOH = kOffMu + 2 * kPlaneMu;
constexpr int kOffP = kOffMu;                 // P planes reuse mu + one-hot
constexpr int kOffMuX = kOffOH + kPlaneRow;
constexpr int kOffVc = kOffMuX + kFK * kMuXCols * 2;
constexpr int kOffC = kOffVc + kFK * kVcRow * 4;
constexpr int kOffXm = kOffC + kFL * 4;
constexpr int kOffXl = kOffXm + kFK * 8 * 4;
constexpr int kOffMax = kOffXl + kFK * 8 * 4;
constexpr int kLdsTotal = kOffMax + 8 * 4 * 4;
static_assert(2 * kPlaneRow == 2 * kPlaneMu + kPlaneRow, "P planes fill mu + one-hot exactly");
static_assert(kLdsTotal <= 81920, "two workgroups per CU");

}  // namespace

// Tokens that start a cluster: bit t set iff token t is the initial centroid
// of some cluster k < Kc (one bit per token, L <= 128). The initial rows
// increase with k, so token t starts cluster k = number of set bits below t.
struct InitMask {
    uint32_t w[4];
};

// MASKED: valid is the key-padding mask [S / H, L] (nonzero = real token);
// padded keys take the logit -10000 in both softmaxes, and the output rows of
// padded queries are zero.
// EXT: the listing's variants below are switched by the runtime flags
// (without EXT both are off and compiled out), and hist (nullable) receives
// the assignment of every Lloyd iteration, [iters, S, L]. soft: the gathered context
// of token i is sum_k softmax_k(q_i . mu_k / sqrt(d)) V^cent_k over the
// final centroids instead of V^cent_{c_i}. keep_empty: an empty cluster
// keeps its previous centroid instead of becoming the zero vector. (Both are
// rules of the ClusterAttention listing on the "Hooshaai/svd-sst2-roberta-
// cluster" page, its k-means routine and forward.)
template <typename T, bool FULL, bool NARROW, bool MASKED, bool EXT>
__global__ __launch_bounds__(kThreads, 4) void cluster_attn_fused_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx, int S, int L,
    int Kc, int iters, int radius, float alpha, const uint8_t *__restrict__ valid, int H, int G,
    T *__restrict__ out, int32_t *__restrict__ assign_out, InitMask init, int keep_empty,
    int soft, int32_t *__restrict__ hist, int solo_lo, int solo_hi) {
    __shared__ __align__(16) unsigned char smem[kLdsTotal];
    uint16_t *sK = reinterpret_cast<uint16_t *>(smem + kOffK);
    uint16_t *sQV = reinterpret_cast<uint16_t *>(smem + kOffQV);
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kOffMu);
    uint16_t *sOH = reinterpret_cast<uint16_t *>(smem + kOffOH);
    uint16_t *sP = reinterpret_cast<uint16_t *>(smem + kOffP);
    uint16_t *sMuX = reinterpret_cast<uint16_t *>(smem + kOffMuX);
    float *sVc = reinterpret_cast<float *>(smem + kOffVc);
    int *sC = reinterpret_cast<int *>(smem + kOffC);
    float *sXm = reinterpret_cast<float *>(smem + kOffXm);
    float *sXl = reinterpret_cast<float *>(smem + kOffXl);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kOffMax);

    const int tid = threadIdx.x;
    constexpr bool kZ = bf16_storage<T>();   // Q, K, V planes with zero m parts
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const bool keep_old = EXT && keep_empty != 0, soft_g = EXT && soft != 0;   // uniform
    const long slice = blockIdx.x;
    if (slice >= S) return;
    // A workgroup that has its CU to itself starts about 2 us late, so that
    // the loads of the CUs holding two slices, which set the launch time, are
    // served first (the launcher names these workgroups; none when the slices
    // fit the CUs one each or fill them twice).
    if ((int)blockIdx.x >= solo_lo && (int)blockIdx.x < solo_hi) __builtin_amdgcn_s_sleep(64);
    const int NT = FULL ? 8 : (L + 15) >> 4;
    const int tok = 16 * w + l16;
    const long base = slice * (long)L * kD;
    const long kvbase = kv_slice(slice, H, G) * (long)L * kD;   // K and V (grouped heads)
    const LaneOffs lo = lane_offsets(l16, g);
    const u8 *pK = smem + kOffK, *pQV = smem + kOffQV, *pMu = smem + kOffMu, *pOH = smem + kOffOH,
             *pP = smem + kOffP, *pMuX = smem + kOffMuX;
    // transposed reads of rows 32c + 8g (+4) .. of columns 16w + l16 (cluster
    // sums and centroid context of dimension tile w): byte 4096 c + trq[h]
    const int trq0 = 1024 * g + (lo.tr0 ^ (32 * (w & 3)));
    const int trq1 = 1024 * g + (lo.tr4 ^ (32 * (w & 3)));
    // ... of rows 16 kt + 4g .. of columns 16j + l16 (local branch): byte 2048 kt + (trv ^ 32j)
    const int trv = 1024 * (g >> 1) + ((g & 1) ? lo.tr4 : lo.tr0);

    // ------------------------------------------------------------ fetch Q
    // Q rows of token tile w (dims 32c + 8g ..). K and V are requested only
    // once the Q planes are written, so that every slice's Q arrives first and
    // the K and V traffic overlaps the clustering, which needs Q only.
    float qraw[2][8], kraw[2][8], vraw[2][8];
#pragma unroll
    for (int c = 0; c < 2; ++c) load_row8<T, FULL>(Q + base, tok, L, 32 * c + 8 * g, qraw[c]);
    // waves 0 and 1: the key-padding mask of tokens 64w .. 64w+63 (one byte each)
    bool tok_ok = false;
    if (MASKED && w < 2) {
        const int t = 64 * w + lane;
        tok_ok = t < L && valid[(slice / H) * (long)L + t] != 0;
    }
    {   // largest |q| of the slice (bit patterns of |x| order like the values)
        const uint32_t bq = wave_max_u(__float_as_uint(absmax8(qraw[1], absmax8(qraw[0], 0.f))));
        if (lane == 0) sMax[w * 4 + 0] = bq;
    }

    // ------------------------------------------------------------ split Q
    // Q planes + the register fragments qf of token tile w, and the strided
    // initial centroids mu_k = Q[floor(k L / Kc)] with their -||mu||^2/2
    // parts; first without scaling (the usual case), redone below if Q is
    // outside the range the fp16 split takes as is.
    Sp8 qf[2];
    int kinit;
    bool owner;
    {
        const int wd = __builtin_amdgcn_readfirstlane(w) >> 1;   // word of tok = 16w + l16
        const uint32_t word = init.w[wd];
        int below = 0;
        for (int i = 0; i < wd; ++i) below += __builtin_popcount(init.w[i]);
        const int bit = tok & 31;
        owner = (word >> bit) & 1u;
        kinit = below + __builtin_popcount(word & ((1u << bit) - 1u));
    }
    auto split_q = [&](float fq, bool scaled) {
        float n2 = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] = scaled ? qraw[c][i] * fq : qraw[c][i];
                n2 = fmaf(x[i], x[i], n2);
            }
            qf[c] = split8<true>(x);
            const int o = (2048 * w + (lo.rl64 ^ (64 * c))) / 2;   // row tok, cols 32c + 8g
            st16(sQV + o, qf[c].h);
            if (!kZ) st16(sQV + kPlaneE + o, qf[c].m);   // zero for bf16 storage, never read
            if (owner) {
                const int om = off64(kinit, 32 * c + 8 * g);
                st16(sMu + om, qf[c].h);
                st16(sMu + kPlaneMuE + om, qf[c].m);
            }
        }
        if (owner) {
            uint32_t h, m;
            split2(-0.5f * n2, 0.f, h, m);
            sMuX[kinit * kMuXCols + 2 * g] = (uint16_t)(h & 0xffffu);
            sMuX[kinit * kMuXCols + 2 * g + 1] = (uint16_t)(m & 0xffffu);
        }
    };
    split_q(1.f, false);
    // one-hot matrix cleared; clusters >= Kc: zero centroid rows and a -inf
    // score part, so they are never chosen; unused columns of the parts zero
    reinterpret_cast<u32x2_t *>(sOH)[tid] = u32x2_t{0u, 0u};
    for (int e = tid; e < kFK * kMuXCols; e += kThreads) {
        const int kk = e / kMuXCols, j = e % kMuXCols;
        if (kk >= Kc) sMuX[e] = j == 0 ? kNegInfH : (uint16_t)0;
        else if (j >= 8) sMuX[e] = 0;
    }
    for (int e = tid; e < (kFK - Kc) * kD; e += kThreads) {
        const int kk = Kc + e / kD, dd = e % kD;
        sMu[off64(kk, dd)] = 0;
        sMu[kPlaneMuE + off64(kk, dd)] = 0;
    }
    if (MASKED && w < 2) {   // mask words 2w, 2w+1 into the spare slot of the maxima
        const uint64_t bits = __ballot(tok_ok);
        if (lane == 0) {
            sMax[4 * (2 * w) + 3] = (uint32_t)bits;
            sMax[4 * (2 * w + 1) + 3] = (uint32_t)(bits >> 32);
        }
    }
    __syncthreads();
    KeyBits kb;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        kb.w[k] = MASKED ? (uint32_t)__builtin_amdgcn_readfirstlane((int)sMax[4 * k + 3]) : ~0u;

    int sq;
    {
        uint32_t mq = 0;
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) mq = max(mq, sMax[4 * ww]);
        sq = scale_shift(mq, kQLimit);
    }
    if (sq != 0) {   // uniform over the workgroup; reload rather than keep
#pragma unroll
        for (int c = 0; c < 2; ++c) load_row8<T, FULL>(Q + base, tok, L, 32 * c + 8 * g, qraw[c]);
        split_q(__builtin_ldexpf(1.f, -sq), true);
        __syncthreads();
    }

    // ------------------------------------------------------------ fetch K, V
    // items (row it/8, dims 8 (it%8) ..), it = tid and tid + 512; consumed
    // after the clustering. K is requested now and V at the start of the
    // third iteration (or the last, if fewer), so that the address units of
    // the CU never queue every load of both at once (measured fastest).
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;
        load_row8<T, FULL>(Kx + kvbase, it >> 3, L, (it & 7) * 8, kraw[n]);
    }
    const int tv = iters >= 3 ? 3 : iters;   // iteration that requests V
    // iteration at whose start the K planes are written (into the K region,
    // which the clustering does not use), from the maximum published at the
    // end of the iteration before; 0: after the clustering (one iteration)
    const int tk = iters >= 2 ? 2 : 0;
    int sk = 0;
    // K planes: the items of this thread (rows it/8, dims 8 (it%8) ..,
    // it = tid, tid + 512), range-scaled by 2^-sk
    auto k_planes = [&]() {
        uint32_t mk = 0;
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) mk = max(mk, sMax[4 * ww + 1]);
        sk = scale_shift(mk, kKVLimit);
        if (__builtin_expect(sk != 0, 0)) {   // uniform; rare
            const float fk = __builtin_ldexpf(1.f, -sk);
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int i = 0; i < 8; ++i) kraw[n][i] *= fk;
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int it = tid + kThreads * n;
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = kraw[n][i];
            const Sp8 kp = split8(x);
            const int o = off64(it >> 3, (it & 7) * 8);
            st16(sK + o, kp.h);
            if (!kZ) st16(sK + kPlaneE + o, kp.m);   // zero for bf16 storage, never read
        }
    };

    // ------------------------------------------------------------ Lloyd
    const u32x4_t ones_g0 = g == 0 ? u32x4_t{kOneH2, kOneH2, kOneH2, kOneH2} : u32x4_t{0u, 0u, 0u, 0u};
    int cprev = -1;
    for (int t = 1; t <= iters; ++t) {
        if (t == tk) k_planes();
        if (t == tv) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int it = tid + kThreads * n;
                load_row8<T, FULL>(Vx + kvbase, it >> 3, L, (it & 7) * 8, vraw[n]);
            }
        }
        if (FULL || w < NT) {
            // a[r] = mu_k . q_tok - ||mu_k||^2 / 2, k = 4g + r (scaled units of Q)
            const u32x4_t mx = ldb16(pMuX, 64 * l16 + 16 * g);
            const Sp8 mu0 = frag_at(pMu, kPlaneMu, lo.rl64), mu1 = frag_at(pMu, kPlaneMu, lo.rl64 ^ 64);
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t a = mma(mx, ones_g0, kZero4);
            a = mma3z<false, kZ>(mu0, qf[0], a);
            a = mma3z<false, kZ>(mu1, qf[1], a);
            float best = a[0];
            int bk = 4 * g;
#pragma unroll
            for (int rr = 1; rr < 4; ++rr) {
                const bool up = a[rr] > best;
                best = up ? a[rr] : best;
                bk = up ? 4 * g + rr : bk;
            }
            bk = col_argmax(best, bk);
            if (g == 0 && (FULL || tok < L)) {
                if (bk != cprev) {
                    if (cprev >= 0) sOH[off128(cprev, tok)] = 0;
                    sOH[off128(bk, tok)] = 0x3c00;   // fp16 1.0
                    cprev = bk;
                }
                if (t == iters) sC[tok] = bk;
                // c^(t) of every iteration, slot t - 1 (EXT only)
                if (EXT && hist) hist[((long)(t - 1) * S + slice) * L + tok] = bk;
            }
        }
        __syncthreads();
        if (w < 4) {
            // (Q^T one-hot)[dim 16w + 4g + rr][cluster l16] and the sizes n_l16
            f32x4_t sh = kZero4, sm = kZero4, cnt = kZero4;
            const u32x4_t ones = {kOneH2, kOneH2, kOneH2, kOneH2};
            const int nch = (NT + 1) >> 1;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c < nch) {
                    const u32x4_t oh = ldb16(pOH, lo.rl128 ^ (64 * c));
                    const Sp8 qt = colfrag8_at(pQV, 4096 * c + trq0, 4096 * c + trq1);
                    if (!kZ) sm = mma(qt.m, oh, sm);
                    sh = mma(qt.h, oh, sh);
                    cnt = mma(ones, oh, cnt);
                }
            }
            const float inv = __builtin_amdgcn_rcpf(fmaxf(cnt[0], 1.f));
            const int o = off64(l16, 16 * w + 4 * g);
            float v[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) v[rr] = (sm[rr] + sh[rr]) * inv;
            if (keep_old && cnt[0] == 0.f) {   // empty: the stored centroid stays
                const u32x2_t oh = *reinterpret_cast<const u32x2_t *>(sMu + o);
                const u32x2_t om = *reinterpret_cast<const u32x2_t *>(sMu + kPlaneMuE + o);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = half_at(oh, rr) + half_at(om, rr);
            }
            const Sp4 mu4 = split4(v[0], v[1], v[2], v[3]);
            // With kept centroids the norm is taken of the stored vector
            // itself, by this code only, so that a kept centroid and a fresh
            // mean with the same stored value score every token alike (an
            // exact tie then goes to the lower index, as it should).
            float n2p = 0.f;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float x = keep_old ? half_at(mu4.h, rr) + half_at(mu4.m, rr) : v[rr];
                n2p = fmaf(x, x, n2p);
            }
            n2p = col_sum(n2p);   // over the 16 dims of tile w
            if (l16 < Kc) {
                st8(sMu + o, mu4.h);
                st8(sMu + kPlaneMuE + o, mu4.m);
                if (g == 0) {
                    uint32_t h, m;
                    split2(-0.5f * n2p, 0.f, h, m);
                    sMuX[l16 * kMuXCols + 2 * w] = (uint16_t)(h & 0xffffu);
                    sMuX[l16 * kMuXCols + 2 * w + 1] = (uint16_t)(m & 0xffffu);
                }
            }
        }
        if (t == (tk > 0 ? tk - 1 : iters)) {   // largest |k| of the slice, published by the barrier below
            const uint32_t bk = wave_max_u(__float_as_uint(absmax8(kraw[1], absmax8(kraw[0], 0.f))));
            if (lane == 0) sMax[w * 4 + 1] = bk;
        }
        __syncthreads();
    }
    if (tk == 0) {   // one iteration: the K planes now, published with the V maximum
        k_planes();
    }

    // ------------------------------------------------------------ after the clustering
    // (V, requested last, gets its maximum after the scores and its planes
    // after the barrier that follows, in the place of the Q planes)
    const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;   // log2(e)/sqrt(64)
    // soft gather: softmax over the final centroids of token tok, clusters
    // 4g .. 4g+3 (the B operand of the gather product below, normalised)
    Sp4 psoft;
    if (soft_g && (FULL || w < NT)) {
        const Sp8 mu0 = frag_at(pMu, kPlaneMu, lo.rl64), mu1 = frag_at(pMu, kPlaneMu, lo.rl64 ^ 64);
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t a = mma3z<false, kZ>(mu0, qf[0], kZero4);   // a[rr] = mu_{4g+rr} . q_tok (scaled units)
        a = mma3z<false, kZ>(mu1, qf[1], a);
        const float s2 = __builtin_ldexpf(0.125f, 2 * sq) * 1.4426950408889634f;
        float x[4], mx = -__builtin_inff();
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            x[rr] = 4 * g + rr < Kc ? a[rr] * s2 : -__builtin_inff();
            mx = fmaxf(mx, x[rr]);
        }
        mx = col_max(mx);
        float z = 0.f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            x[rr] = __builtin_amdgcn_exp2f(x[rr] - mx);
            z += x[rr];
        }
        const float iz = 1.0f / col_sum(z);
        psoft = split4<true>(x[0] * iz, x[1] * iz, x[2] * iz, x[3] * iz);
    }
    uint16_t *sV = sQV;   // Q planes are dead
    if (tk == 0) __syncthreads();   // the K planes written after the clustering

    // ------------------------------------------------------------ centroid-key scores
    float sx[4];
    {
        float mloc = -__builtin_inff();
        if (FULL || w < NT) {
            const Sp8 k0 = frag_at(pK, kPlane, 2048 * w + lo.rl64), m0 = frag_at(pMu, kPlaneMu, lo.rl64);
            const Sp8 k1 = frag_at(pK, kPlane, 2048 * w + (lo.rl64 ^ 64)), m1 = frag_at(pMu, kPlaneMu, lo.rl64 ^ 64);
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t a = mma3z<kZ, false>(k0, m0, kZero4);
            a = mma3z<kZ, false>(k1, m1, a);
            const uint32_t nib = MASKED ? kb.tile(w) >> (4 * g) : 0xfu;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = 16 * w + 4 * g + rr;   // a[rr] = k_key . mu_l16
                const float sv = (!MASKED || ((nib >> rr) & 1u)) ? a[rr] * sscale2 : kPadLogit2;
                sx[rr] = (FULL || key < L) ? sv : -__builtin_inff();
                mloc = fmaxf(mloc, sx[rr]);
            }
            mloc = col_max(mloc);
        } else {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sx[rr] = -__builtin_inff();
        }
        if (g == 0) sXm[l16 * 8 + w] = mloc;
    }
    {   // largest |v| of the slice (V arrives last: after the scores)
        const uint32_t bv = wave_max_u(__float_as_uint(absmax8(vraw[1], absmax8(vraw[0], 0.f))));
        if (lane == 0) sMax[w * 4 + 2] = bv;
    }
    __syncthreads();   // V maxima and the score maxima published
    // V planes (first read after the next barrier)
    int sv;
    {
        uint32_t mv = 0;
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) mv = max(mv, sMax[4 * ww + 2]);
        sv = scale_shift(mv, kKVLimit);
    }
    const float vunscale = __builtin_ldexpf(1.f, sv);
    if (__builtin_expect(sv != 0, 0)) {   // uniform; rare
        const float fv = __builtin_ldexpf(1.f, -sv);
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int i = 0; i < 8; ++i) vraw[n][i] *= fv;
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = vraw[n][i];
        const Sp8 vp = split8(x);
        const int o = off64(it >> 3, (it & 7) * 8);
        st16(sV + o, vp.h);
        if (!kZ) st16(sV + kPlaneE + o, vp.m);   // zero for bf16 storage, never read
    }
    // mu and the one-hot matrix are dead from here on (P reuses them): every
    // wave read mu for its scores before the barrier above
    {
        const float4 m0 = *reinterpret_cast<const float4 *>(sXm + l16 * 8);
        const float4 m1 = *reinterpret_cast<const float4 *>(sXm + l16 * 8 + 4);
        const float Mx = fmaxf(fmaxf(fmaxf(m0.x, m0.y), fmaxf(m0.z, m0.w)),
                               fmaxf(fmaxf(m1.x, m1.y), fmaxf(m1.z, m1.w)));
        float p[4];
        float ls = 0.f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            p[rr] = __builtin_amdgcn_exp2f(sx[rr] - Mx);   // exp2(-inf) = 0
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

    // ------------------------------------------------------------ centroid context (waves 0-3)
    if (w < 4) {
        // V^cent^T[dim 16w + 4g + rr][centroid l16] = sum over keys of V^T P^T
        const int nch = (NT + 1) >> 1;
        Sp8 vf[4], pf[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (FULL || c < nch) {
                vf[c] = colfrag8_at(pQV, 4096 * c + trq0, 4096 * c + trq1);
                pf[c] = frag_at(pP, kPlaneRow, lo.rl128 ^ (64 * c));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t a2[2] = {kZero4, kZero4};   // even and odd key chunks
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (FULL || c < nch) a2[c & 1] = mma3z<kZ, false>(vf[c], pf[c], a2[c & 1]);
        const f32x4_t a = a2[0] + a2[1];
        const float4 l0 = *reinterpret_cast<const float4 *>(sXl + l16 * 8);
        const float4 l1 = *reinterpret_cast<const float4 *>(sXl + l16 * 8 + 4);
        const float den = ((((((l0.x + l0.y) + l0.z) + l0.w) + l1.x) + l1.y) + l1.z) + l1.w;
        // (1 - alpha) V^cent; kept in the scaled units of V for the soft
        // gather, whose fp16 operands need them
        const float f = (1.0f - alpha) * (soft_g ? 1.f : vunscale) * __builtin_amdgcn_rcpf(den);
        *reinterpret_cast<float4 *>(sVc + l16 * kVcRow + 16 * w + 4 * g) =
            make_float4(a[0] * f, a[1] * f, a[2] * f, a[3] * f);
    }

    // ------------------------------------------------------------ local window branch
    f32x4_t o[4];   // set below for every wave that uses it
    float lsum;
    if (FULL || w < NT) {
        const int rad = radius < L ? radius : L;
        if (NARROW)
            local_narrow<FULL, MASKED, KeyBits, kPlane, kZ>(pK, pQV, qf, w, NT, L, rad, sscale2,
                                                            l16, g, lo.rl64, trv, kb, o, lsum);
        else
            local_wide<FULL, MASKED, false, kZ>(pK, pQV, qf, w, NT, L, rad, sscale2, l16, g,
                                                lo.rl64, trv, kb, o, lsum);
    }
    __syncthreads();

    // ------------------------------------------------------------ gather + fusion
    // The fused rows of token tile w go through a wave-private LDS tile (in
    // the dead K planes; 16 rows, 16-byte chunks XOR-swizzled by the row) so
    // that every store instruction writes whole rows: 64 lanes x 16 bytes of
    // consecutive memory.
    {
        constexpr int kRowB = kD * (int)sizeof(T);   // bytes per output row
        constexpr int kCpr = kRowB / 16;             // 16-byte chunks per row
        u8 *stg = smem + kOffK + w * 16 * kRowB;
        if (FULL || w < NT) {
            const float f = alpha * vunscale * __builtin_amdgcn_rcpf(lsum);
            const float *vc = sVc + sC[tok] * kVcRow;
            const bool keep = !MASKED || ((kb.tile(w) >> l16) & 1u);   // padded query: zero row
#pragma unroll
            for (int j = 0; j < 4; ++j) {   // o[j][rr] = Oloc^T[dim 16j + 4g + rr][query tok]
                const int d0 = 16 * j + 4 * g;
                float4 c4;
                if (soft_g) {
                    // G^T[dim 16j + 4g + rr][token tok] = sum_k V^cent^T[dim][k] p[k][tok]:
                    // A[dim 16j + l16][k = 4g + i] from the fp32 rows of V^cent
                    const float *vk = sVc + 4 * g * kVcRow + 16 * j + l16;
                    const Sp4 va = split4<true>(vk[0], vk[kVcRow], vk[2 * kVcRow], vk[3 * kVcRow]);
                    const f32x4_t gs = mma3_16(va, psoft, kZero4);
                    c4 = make_float4(gs[0] * vunscale, gs[1] * vunscale, gs[2] * vunscale,
                                     gs[3] * vunscale);
                } else {
                    c4 = *reinterpret_cast<const float4 *>(vc + d0);
                }
                float v0 = fmaf(o[j][0], f, c4.x), v1 = fmaf(o[j][1], f, c4.y);
                float v2 = fmaf(o[j][2], f, c4.z), v3 = fmaf(o[j][3], f, c4.w);
                if (MASKED && !keep) v0 = v1 = v2 = v3 = 0.f;
                const int byte = d0 * (int)sizeof(T);   // within the row
                u8 *p = stg + l16 * kRowB + ((((byte >> 4) ^ (l16 & (kCpr - 1)))) << 4) + (byte & 15);
                if (sizeof(T) == 4) {
                    *reinterpret_cast<f32x4_t *>(p) = f32x4_t{v0, v1, v2, v3};
                } else {
                    *reinterpret_cast<u32x2_t *>(p) =
                        u32x2_t{(uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16),
                                (uint32_t)f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16)};
                }
            }
            __builtin_amdgcn_wave_barrier();
            u8 *dst = reinterpret_cast<u8 *>(out + base + (long)16 * w * kD);
#pragma unroll
            for (int i = 0; i < kCpr / 4; ++i) {   // 64 chunks = 64 / kCpr rows per store
                const int flat = 64 * i + lane;
                const int row = flat / kCpr, c = flat % kCpr;
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(
                    stg + row * kRowB + (((c ^ (row & (kCpr - 1)))) << 4));
                if (FULL || 16 * w + row < L)
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst + flat * 16));
            }
        }
    }
    if (assign_out && tid < L) __builtin_nontemporal_store(sC[tid], assign_out + slice * L + tid);
}

// Exact attention of one slice (the decoder / cross-attention branch of the
// ClusterAttention listing on the "Hooshaai/svd-sst2-roberta-cluster" page)
// for L = Nk <= 128: the forward kernel's loads, range scaling, fp16 split
// planes and wide local window, with the window [0, qi] (CAUSAL) or every key,
// and no clustering. Padded keys take the -10000 logit; padded query rows are
// zero. With CAUSAL the future keys are excluded rather than filled, which is
// the same result whenever every real query has a real key at or before it
// (the host routes other masks to the staged kernel).
constexpr int kXOffV = 2 * kPlane;                 // K planes, then V planes
constexpr int kXOffMax = kXOffV + 2 * kPlane;
constexpr int kXLds = kXOffMax + 8 * 4 * 4;

template <typename T, bool FULL, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(kThreads, 4) void exact_fused_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx, int S, int L,
    const uint8_t *__restrict__ qvalid, const uint8_t *__restrict__ kvalid, int H, int G,
    T *__restrict__ out, int solo_lo, int solo_hi) {
    __shared__ __align__(16) unsigned char smem[kXLds];
    uint16_t *sK = reinterpret_cast<uint16_t *>(smem);
    uint16_t *sV = reinterpret_cast<uint16_t *>(smem + kXOffV);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kXOffMax);
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const long slice = blockIdx.x;
    if (slice >= S) return;
    // a workgroup alone on its CU starts about 2 us late (as in the forward)
    if ((int)blockIdx.x >= solo_lo && (int)blockIdx.x < solo_hi) __builtin_amdgcn_s_sleep(64);
    const int NT = FULL ? 8 : (L + 15) >> 4;
    const int tok = 16 * w + l16;
    const long base = slice * (long)L * kD;
    const long kvbase = kv_slice(slice, H, G) * (long)L * kD;
    const long brow = (slice / H) * (long)L;
    const LaneOffs lo = lane_offsets(l16, g);
    const int trv = 1024 * (g >> 1) + ((g & 1) ? lo.tr4 : lo.tr0);

    float qraw[2][8], kraw[2][8], vraw[2][8];
#pragma unroll
    for (int c = 0; c < 2; ++c) load_row8<T, FULL>(Q + base, tok, L, 32 * c + 8 * g, qraw[c]);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;
        load_row8<T, FULL>(Kx + kvbase, it >> 3, L, (it & 7) * 8, kraw[n]);
        load_row8<T, FULL>(Vx + kvbase, it >> 3, L, (it & 7) * 8, vraw[n]);
    }
    bool tok_ok = false;
    if (MASKED && w < 2) {
        const int t = 64 * w + lane;
        tok_ok = t < L && (kvalid == nullptr || kvalid[brow + t] != 0);
    }
    {
        const uint32_t bq = wave_max_u(__float_as_uint(absmax8(qraw[1], absmax8(qraw[0], 0.f))));
        const uint32_t bk = wave_max_u(__float_as_uint(absmax8(kraw[1], absmax8(kraw[0], 0.f))));
        const uint32_t bv = wave_max_u(__float_as_uint(absmax8(vraw[1], absmax8(vraw[0], 0.f))));
        if (lane == 0) {
            sMax[4 * w] = bq;
            sMax[4 * w + 1] = bk;
            sMax[4 * w + 2] = bv;
        }
    }
    if (MASKED && w < 2) {   // key mask words 2w, 2w+1 into the spare slots
        const uint64_t bits = __ballot(tok_ok);
        if (lane == 0) {
            sMax[4 * (2 * w) + 3] = (uint32_t)bits;
            sMax[4 * (2 * w + 1) + 3] = (uint32_t)(bits >> 32);
        }
    }
    __syncthreads();
    KeyBits kb;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        kb.w[k] = MASKED ? (uint32_t)__builtin_amdgcn_readfirstlane((int)sMax[4 * k + 3]) : ~0u;
    uint32_t mq = 0, mk = 0, mv = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) {
        mq = max(mq, sMax[4 * ww]);
        mk = max(mk, sMax[4 * ww + 1]);
        mv = max(mv, sMax[4 * ww + 2]);
    }
    const int sq = scale_shift(mq, kQLimit), sk = scale_shift(mk, kKVLimit);
    const int sv = scale_shift(mv, kKVLimit);
    const float fq = __builtin_ldexpf(1.f, -sq), fk = __builtin_ldexpf(1.f, -sk);
    const float fv = __builtin_ldexpf(1.f, -sv);
    Sp8 qf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = qraw[c][i] * fq;   // exact power-of-two scaling
        qf[c] = split8<true>(x);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;
        const int o = off64(it >> 3, (it & 7) * 8);
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = kraw[n][i] * fk;
        const Sp8 kp = split8(x);
        st16(sK + o, kp.h);
        st16(sK + kPlaneE + o, kp.m);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = vraw[n][i] * fv;
        const Sp8 vp = split8(x);
        st16(sV + o, vp.h);
        st16(sV + kPlaneE + o, vp.m);
    }
    __syncthreads();
    const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;
    f32x4_t o[4];
    float lsum = 1.f;
    if (FULL || w < NT)
        local_wide<FULL, MASKED, CAUSAL>(smem, smem + kXOffV, qf, w, NT, L, L, sscale2, l16, g,
                                         lo.rl64, trv, kb, o, lsum);
    __syncthreads();   // K planes are dead: they stage the output rows
    constexpr int kRowB = kD * (int)sizeof(T);
    constexpr int kCpr = kRowB / 16;
    u8 *stg = smem + w * 16 * kRowB;
    if (FULL || w < NT) {
        const bool keep = !MASKED || qvalid == nullptr || tok >= L || qvalid[brow + tok] != 0;
        const float f = keep ? __builtin_ldexpf(1.f, sv) * __builtin_amdgcn_rcpf(lsum) : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int byte = (16 * j + 4 * g) * (int)sizeof(T);
            u8 *p = stg + l16 * kRowB + ((((byte >> 4) ^ (l16 & (kCpr - 1)))) << 4) + (byte & 15);
            const float v0 = o[j][0] * f, v1 = o[j][1] * f, v2 = o[j][2] * f, v3 = o[j][3] * f;
            if (sizeof(T) == 4) {
                *reinterpret_cast<f32x4_t *>(p) = f32x4_t{v0, v1, v2, v3};
            } else {
                *reinterpret_cast<u32x2_t *>(p) =
                    u32x2_t{(uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16),
                            (uint32_t)f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16)};
            }
        }
        __builtin_amdgcn_wave_barrier();
        u8 *dst = reinterpret_cast<u8 *>(out + base + (long)16 * w * kD);
#pragma unroll
        for (int i = 0; i < kCpr / 4; ++i) {
            const int flat = 64 * i + lane;
            const int row = flat / kCpr, c = flat % kCpr;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(
                stg + row * kRowB + (((c ^ (row & (kCpr - 1)))) << 4));
            if (FULL || 16 * w + row < L)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst + flat * 16));
        }
    }
}

bool exact_fused_supported(int L, int Nk) { return L == Nk && L >= 1 && L <= kFL; }

template <typename T, bool CAUSAL, bool MASKED>
static hipError_t exact_fused_launch_t(const void *Q, const void *K, const void *V, int S, int L,
                                       const uint8_t *qvalid, const uint8_t *kvalid, int H, int G,
                                       void *out, hipStream_t st, int cus) {
    const T *q = static_cast<const T *>(Q), *k = static_cast<const T *>(K);
    // two workgroups fit a CU: with cus < S < 2 cus, workgroups S - cus ..
    // cus - 1 run alone
    const int solo_lo = cus > 0 && S > cus && S < 2 * cus ? S - cus : 0;
    const int solo_hi = solo_lo > 0 ? cus : 0;
    const T *v = static_cast<const T *>(V);
    if (L == kFL)
        hipLaunchKernelGGL((exact_fused_kernel<T, true, CAUSAL, MASKED>), dim3((unsigned)S),
                           dim3(kThreads), 0, st, q, k, v, S, L, qvalid, kvalid, H, G,
                           static_cast<T *>(out), solo_lo, solo_hi);
    else
        hipLaunchKernelGGL((exact_fused_kernel<T, false, CAUSAL, MASKED>), dim3((unsigned)S),
                           dim3(kThreads), 0, st, q, k, v, S, L, qvalid, kvalid, H, G,
                           static_cast<T *>(out), solo_lo, solo_hi);
    return hipGetLastError();
}

template <typename T>
static hipError_t exact_fused_dispatch(const void *Q, const void *K, const void *V, int S, int L,
                                       bool causal, const uint8_t *qvalid, const uint8_t *kvalid,
                                       int H, int G, void *out, hipStream_t st, int cus) {
    const bool masked = qvalid != nullptr || kvalid != nullptr;
    if (causal)
        return masked ? exact_fused_launch_t<T, true, true>(Q, K, V, S, L, qvalid, kvalid, H, G, out, st, cus)
                      : exact_fused_launch_t<T, true, false>(Q, K, V, S, L, qvalid, kvalid, H, G, out, st, cus);
    return masked ? exact_fused_launch_t<T, false, true>(Q, K, V, S, L, qvalid, kvalid, H, G, out, st, cus)
                  : exact_fused_launch_t<T, false, false>(Q, K, V, S, L, qvalid, kvalid, H, G, out, st, cus);
}

hipError_t launch_exact_fused(const void *Q, const void *K, const void *V, int S, int L,
                              bool causal, ca_dtype_t dt, const uint8_t *qvalid,
                              const uint8_t *kvalid, int H, int G, void *out, hipStream_t st,
                              int cus) {
    if (dt == CA_BF16)
        return exact_fused_dispatch<bf16_t>(Q, K, V, S, L, causal, qvalid, kvalid, H, G, out, st,
                                            cus);
    return exact_fused_dispatch<float>(Q, K, V, S, L, causal, qvalid, kvalid, H, G, out, st, cus);
}

bool fused_supported(int L, int Kc) { return L >= 1 && L <= kFL && Kc >= 1 && Kc <= kFK; }

// Arguments of one launch, fixed on the host.
struct FusedArgs {
    const void *Q, *K, *V;
    int S, L, Kc, iters, radius;
    float alpha;
    const uint8_t *valid;
    int H, G;
    void *out;
    int32_t *assign;
    InitMask init;
    int keep_empty, soft;
    int32_t *hist;
    int solo_lo, solo_hi;   // workgroups alone on their CU: [solo_lo, solo_hi)
};

template <typename T, bool FULL, bool NARROW, bool MASKED, bool EXT>
static hipError_t fused_launch_t(const FusedArgs &a, hipStream_t st) {
    auto kern = cluster_attn_fused_kernel<T, FULL, NARROW, MASKED, EXT>;
    hipLaunchKernelGGL(kern, dim3((unsigned)a.S), dim3(kThreads), 0, st,
                       static_cast<const T *>(a.Q), static_cast<const T *>(a.K),
                       static_cast<const T *>(a.V), a.S, a.L, a.Kc, a.iters, a.radius, a.alpha,
                       a.valid, a.H, a.G, static_cast<T *>(a.out), a.assign, a.init,
                       a.keep_empty, a.soft, a.hist, a.solo_lo, a.solo_hi);
    return hipGetLastError();
}

template <typename T, bool MASKED, bool EXT>
static hipError_t fused_launch_m(const FusedArgs &a, hipStream_t st) {
    const bool full = a.L == kFL;
    const bool narrow = a.radius <= 16;
    if (full && narrow) return fused_launch_t<T, true, true, MASKED, EXT>(a, st);
    if (full) return fused_launch_t<T, true, false, MASKED, EXT>(a, st);
    if (narrow) return fused_launch_t<T, false, true, MASKED, EXT>(a, st);
    return fused_launch_t<T, false, false, MASKED, EXT>(a, st);
}

template <typename T>
static hipError_t fused_launch(const FusedArgs &a, hipStream_t st) {
    const bool ext = a.keep_empty || a.soft || a.hist;
    if (a.valid)
        return ext ? fused_launch_m<T, true, true>(a, st) : fused_launch_m<T, true, false>(a, st);
    return ext ? fused_launch_m<T, false, true>(a, st) : fused_launch_m<T, false, false>(a, st);
}

hipError_t launch_fused_forward(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                                int iters, int radius, float alpha, const Variant &var,
                                ca_dtype_t dt, const uint8_t *valid, int H, int G, void *out,
                                int32_t *assign, hipStream_t st, int32_t *hist, int cus) {
    FusedArgs a{Q, K, V, S, L, Kc, iters, radius, alpha, valid, H, G, out, assign, InitMask{},
                var.keep_empty ? 1 : 0, var.soft ? 1 : 0, hist, 0, 0};
    // Two workgroups fit a CU. With cus < S < 2 cus the dispatcher places
    // workgroups 0 .. cus-1 one per CU and the rest beside workgroups
    // 0 .. S-cus-1, so workgroups S-cus .. cus-1 run alone (measured, 384
    // slices on 256 CUs: 14.5 -> 14.0 us with these delayed).
    if (cus > 0 && S > cus && S < 2 * cus) {
        a.solo_lo = S - cus;
        a.solo_hi = cus;
    }
    for (int k = 0; k < Kc; ++k) {
        const int t = init_row(k, L, Kc, var.init_step);
        a.init.w[t >> 5] |= 1u << (t & 31);
    }
    if (dt == CA_BF16) return fused_launch<bf16_t>(a, st);
    return fused_launch<float>(a, st);
}

}  // namespace ca
