// Local-branch backward of one slice in one launch (L <= 128, one query head
// per K/V head): the band part of the backward pass on the fp16 matrix cores,
// with the forward kernel's split planes and fragment readers.
//
// Per slice the local branch is O^loc = P V with P = softmax over the window
// |i - j| <= r of q_i . k_j / 8 (a padded key's logit is -10000). For the
// loss sum(dO * O) with O = keep ((1 - alpha) V^cent_c + alpha O^loc) and
// g = keep dO, its gradients are (the softmax rule dS = P (dP - D)):
//   dP_ij = alpha g_i . v_j,  D_i = alpha g_i . O^loc_i,
//   dS_ij = P_ij (dP_ij - D_i) / 8   (0 for a padded key: constant logit),
//   dQ_i += sum_j dS_ij k_j,  dK_j += sum_i dS_ij q_i,  dV_j += alpha sum_i P_ij g_i.
// The centroid branch's shares (dK_c, dV_c in fp32, dmu with the counts, the
// slice's centroid term of dalpha) come from bwd_centroid_fused_kernel below
// and are added here: dQ_i += dmu_{c_i} / n_{c_i}; dalpha of the slice is
// sum keep dO . O^loc minus sum_k G_k . V^cent_k.
//
// Two passes over the band, each the mirror of the other:
//   query pass (wave w owns query tile w; K and V planes in LDS, its Q and g
//     rows as B fragments): the forward's wide window gives O^loc and the
//     softmax statistics; a second sweep recomputes S^T and dP^T tile pairs
//     and accumulates dQ^T = K^T dS^T, exactly like P V;
//   key pass (wave w owns key tile w; Q and g planes in LDS, its K and V rows
//     as B fragments): S and dP in [query][key] orientation, probabilities
//     from the query statistics of the first pass, dK^T = Q^T dS and
//     dV^T = g^T P.
// Scaling: Q and K are scaled by powers of two as in the forward; V and g to
// magnitudes below 2^4, so that dP (64 products) and dS stay below 2^14 and
// fit the fp16 split; the factors are undone on the fp32 results.
#include "launch.h"
#include "mfma_split.h"

namespace ca {
namespace {

constexpr int kBVLimit = 4;                   // scaled |v|, |g| < 2^4
constexpr int kBOffB = 2 * kPlane;            // V planes, later g planes
constexpr int kBOffStat = 4 * kPlane;         // per query: max, 1/sum, D, dalpha share
constexpr int kBOffMax = kBOffStat + kFL * 16;
constexpr int kBLds = kBOffMax + 8 * 8 * 4;

}  // namespace

template <typename T, bool FULL, bool MASKED>
__global__ __launch_bounds__(kThreads, 4) void bwd_local_fused_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx,
    const T *__restrict__ dO, const int32_t *__restrict__ assign,
    const uint8_t *__restrict__ valid, const float *__restrict__ dalc,
    const float *__restrict__ dmu, const int32_t *__restrict__ counts,
    const float *__restrict__ dKc, const float *__restrict__ dVc, int S, int L, int Kc,
    int radius, float alpha, int H, T *__restrict__ dQ, T *__restrict__ dK, T *__restrict__ dV,
    float *__restrict__ dal, int solo_lo, int solo_hi) {
    __shared__ __align__(16) unsigned char smem[kBLds];
    uint16_t *sA = reinterpret_cast<uint16_t *>(smem);            // K, then Q planes
    uint16_t *sB = reinterpret_cast<uint16_t *>(smem + kBOffB);   // V, then g planes
    float4 *sStat = reinterpret_cast<float4 *>(smem + kBOffStat);
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kBOffMax);   // [8 waves][8]
    const u8 *pA = smem, *pB = smem + kBOffB;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const long slice = blockIdx.x;
    if (slice >= S) return;
    // a workgroup alone on its CU starts about 2 us late, so that the loads of
    // the CUs holding two slices are served first (the launcher names these
    // workgroups)
    if ((int)blockIdx.x >= solo_lo && (int)blockIdx.x < solo_hi) __builtin_amdgcn_s_sleep(64);
    const int NT = FULL ? 8 : (L + 15) >> 4;
    const bool tile_on = FULL || w < NT;
    const int tok = 16 * w + l16;                // query (first pass) and key (second) of the lane
    const bool tok_in = FULL || tok < L;
    const long base = slice * (long)L * kD;
    const long brow = (slice / H) * (long)L;
    const LaneOffs lo = lane_offsets(l16, g);
    const int trv = 1024 * (g >> 1) + ((g & 1) ? lo.tr4 : lo.tr0);
    const int nr = (radius + 15) >> 4;           // tiles on each side of a tile's window

    // ------------------------------------------------------------ loads
    // Q and K first: their planes and fragments are formed while V and dO
    // are still arriving
    float qraw[2][8], graw[2][8], kraw[2][8], vraw[2][8];
#pragma unroll
    for (int c = 0; c < 2; ++c) load_row8<T, FULL>(Q + base, tok, L, 32 * c + 8 * g, qraw[c]);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;
        load_row8<T, FULL>(Kx + base, it >> 3, L, (it & 7) * 8, kraw[n]);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;
        load_row8<T, FULL>(Vx + base, it >> 3, L, (it & 7) * 8, vraw[n]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) load_row8<T, FULL>(dO + base, tok, L, 32 * c + 8 * g, graw[c]);
    const bool tok_keep = !MASKED || !tok_in || valid[brow + tok] != 0;
    {
        const uint32_t bq = wave_max_u(__float_as_uint(absmax8(qraw[1], absmax8(qraw[0], 0.f))));
        const uint32_t bk = wave_max_u(__float_as_uint(absmax8(kraw[1], absmax8(kraw[0], 0.f))));
        if (lane == 0) {
            sMax[8 * w] = bq;
            sMax[8 * w + 1] = bk;
        }
    }
    if (MASKED && w < 2) {   // key mask of tokens 64w .. 64w+63, words 2w and 2w+1
        const int t = 64 * w + lane;
        const uint64_t bits = __ballot(t < L && valid[brow + t] != 0);
        if (lane == 0) {
            sMax[8 * (2 * w) + 4] = (uint32_t)bits;
            sMax[8 * (2 * w + 1) + 4] = (uint32_t)(bits >> 32);
        }
    }
    __syncthreads();
    KeyBits kb;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        kb.w[k] = MASKED ? (uint32_t)__builtin_amdgcn_readfirstlane((int)sMax[8 * k + 4]) : ~0u;
    uint32_t mq = 0, mk = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) {
        mq = max(mq, sMax[8 * ww]);
        mk = max(mk, sMax[8 * ww + 1]);
    }
    const int sq = scale_shift(mq, kQLimit), sk = scale_shift(mk, kKVLimit);
    const float fq = __builtin_ldexpf(1.f, -sq), fk = __builtin_ldexpf(1.f, -sk);
    Sp8 qf[2], gf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = qraw[c][i] * fq;
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
        st16(sA + o, kp.h);
        st16(sA + kPlaneE + o, kp.m);
    }
    // V and dO (slots 2 and 3 of the maxima are free)
    if (!tok_keep) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) graw[c][i] = 0.f;
    }
    {
        const uint32_t bv = wave_max_u(__float_as_uint(absmax8(vraw[1], absmax8(vraw[0], 0.f))));
        const uint32_t bg = wave_max_u(__float_as_uint(absmax8(graw[1], absmax8(graw[0], 0.f))));
        if (lane == 0) {
            sMax[8 * w + 2] = bv;
            sMax[8 * w + 3] = bg;
        }
    }
    __syncthreads();
    uint32_t mv = 0, mg = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) {
        mv = max(mv, sMax[8 * ww + 2]);
        mg = max(mg, sMax[8 * ww + 3]);
    }
    const int sv = scale_shift(mv, kBVLimit), sg = scale_shift(mg, kBVLimit);
    const float fv = __builtin_ldexpf(1.f, -sv), fg = __builtin_ldexpf(1.f, -sg);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = graw[c][i] * fg;
        gf[c] = split8<true>(y);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;
        const int o = off64(it >> 3, (it & 7) * 8);
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = vraw[n][i] * fv;
        const Sp8 vp = split8(x);
        st16(sB + o, vp.h);
        st16(sB + kPlaneE + o, vp.m);
    }
    __syncthreads();
    const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;
    const float du_scale = __builtin_ldexpf(1.f, -(sg + sv));   // real D -> units of dP

    // ------------------------------------------------------------ query pass
    if (tile_on) {
        f32x4_t o[4];
        float lsum = 1.f, M = 0.f;
        local_wide<FULL, MASKED>(pA, pB, qf, w, NT, L, radius, sscale2, l16, g, lo.rl64, trv, kb,
                                 o, lsum, &M);
        const float invl = 1.0f / lsum;
        // D = alpha g . O^loc from O^loc and g in the same lane layout (dims
        // 16j + 4g .. +3 of query tok); g . O^loc is also the local term of
        // dalpha
        float dpart = 0.f;
        const int c = tok_in ? min(max(assign[slice * L + tok], 0), Kc - 1) : 0;
        if (tok_in && tok_keep) {
            const float olf = __builtin_ldexpf(1.f, sv) * invl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 16 * j + 4 * g;
                const float4 g4 = load4<T>(dO + base + (long)tok * kD + d0);
                const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) dpart = fmaf(gg[rr], o[j][rr] * olf, dpart);
            }
        }
        const float A = col_sum(dpart);
        const float D = alpha * A;
        if (g == 0 && tok_in) sStat[tok] = make_float4(M, invl, D, A);
        // second sweep: dQ^T = K^T dS^T over the window's key tile pairs
        const float Du = D * du_scale;
        const int kt_lo = w - nr < 0 ? 0 : w - nr;
        const int kt_hi = w + nr < NT - 1 ? w + nr : NT - 1;
        f32x4_t dq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) dq[j] = kZero4;
        for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
            const bool two = kt + 1 <= kt_hi;
            float ds[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ktt = two ? kt + h : kt;
                const Sp8 k0 = frag_at(pA, kPlane, 2048 * ktt + lo.rl64);
                const Sp8 k1 = frag_at(pA, kPlane, 2048 * ktt + (lo.rl64 ^ 64));
                const Sp8 v0 = frag_at(pB, kPlane, 2048 * ktt + lo.rl64);
                const Sp8 v1 = frag_at(pB, kPlane, 2048 * ktt + (lo.rl64 ^ 64));
                f32x4_t a = mma3(k0, qf[0], kZero4);
                a = mma3(k1, qf[1], a);
                f32x4_t a2 = mma3(v0, gf[0], kZero4);
                a2 = mma3(v1, gf[1], a2);
                const uint32_t nib = MASKED ? kb.tile(ktt) >> (4 * g) : 0xfu;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int key = 16 * ktt + 4 * g + rr;
                    const int dist = key > tok ? key - tok : tok - key;
                    const bool in = (FULL || key < L) && dist <= radius && (h == 0 || two);
                    const bool kok = !MASKED || ((nib >> rr) & 1u);
                    const float s2 = kok ? a[rr] * sscale2 : kPadLogit2;
                    const float p = in ? __builtin_amdgcn_exp2f(s2 - M) * invl : 0.f;
                    ds[4 * h + rr] = (in && kok) ? p * (alpha * a2[rr] - Du) : 0.f;
                }
            }
            const Sp8 dsp = split8<true>(ds);
            const int b0 = 2048 * kt + trv, b1 = two ? b0 + 2048 : b0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dq[j] = mma3(colfrag8_at(pA, b0 ^ (32 * j), b1 ^ (32 * j)), dsp, dq[j]);
        }
        if (tok_in) {
            const float f = __builtin_ldexpf(0.125f, sg + sv + sk);
            const int n = counts[slice * Kc + c];
            const float invn = 1.0f / (float)(n > 1 ? n : 1);
            const float *dm = dmu + (slice * Kc + c) * kD;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 16 * j + 4 * g;
                const float4 m4 = load4<float>(dm + d0);
                store4<T>(dQ + base + (long)tok * kD + d0,
                          make_float4(fmaf(dq[j][0], f, m4.x * invn), fmaf(dq[j][1], f, m4.y * invn),
                                      fmaf(dq[j][2], f, m4.z * invn), fmaf(dq[j][3], f, m4.w * invn)));
            }
        }
    }
    __syncthreads();
    // own key tile's K and V rows as B fragments, before the planes change
    Sp8 kf[2], vf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        kf[c] = frag_at(pA, kPlane, 2048 * w + (lo.rl64 ^ (64 * c)));
        vf[c] = frag_at(pB, kPlane, 2048 * w + (lo.rl64 ^ (64 * c)));
    }
    __syncthreads();
    // Q and g planes from the query pass's own fragments (each wave's tile
    // rows, already scaled and split; zero rows past L and for padded queries)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int o = (2048 * w + (lo.rl64 ^ (64 * c))) / 2;   // row tok, cols 32c + 8g
        st16(sA + o, qf[c].h);
        st16(sA + kPlaneE + o, qf[c].m);
        st16(sB + o, gf[c].h);
        st16(sB + kPlaneE + o, gf[c].m);
    }
    __syncthreads();

    // ------------------------------------------------------------ key pass
    if (tile_on) {
        const bool kok = !MASKED || ((kb.tile(w) >> l16) & 1u);   // the lane's own key
        const int qt_lo = w - nr < 0 ? 0 : w - nr;
        const int qt_hi = w + nr < NT - 1 ? w + nr : NT - 1;
        f32x4_t dk[4], dv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) dk[j] = dv[j] = kZero4;
        for (int qt = qt_lo; qt <= qt_hi; qt += 2) {
            const bool two = qt + 1 <= qt_hi;
            float ds[8], pp[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int qtt = two ? qt + h : qt;
                const Sp8 q0 = frag_at(pA, kPlane, 2048 * qtt + lo.rl64);
                const Sp8 q1 = frag_at(pA, kPlane, 2048 * qtt + (lo.rl64 ^ 64));
                const Sp8 g0 = frag_at(pB, kPlane, 2048 * qtt + lo.rl64);
                const Sp8 g1 = frag_at(pB, kPlane, 2048 * qtt + (lo.rl64 ^ 64));
                f32x4_t a = mma3(q0, kf[0], kZero4);    // [query 4g + rr][key l16]
                a = mma3(q1, kf[1], a);
                f32x4_t a2 = mma3(g0, vf[0], kZero4);
                a2 = mma3(g1, vf[1], a2);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int qi = 16 * qtt + 4 * g + rr;
                    const int dist = qi > tok ? qi - tok : tok - qi;
                    const bool in = (FULL || qi < L) && tok_in && dist <= radius && (h == 0 || two);
                    const float4 st = sStat[in ? qi : 0];
                    const float s2 = kok ? a[rr] * sscale2 : kPadLogit2;
                    const float p = in ? __builtin_amdgcn_exp2f(s2 - st.x) * st.y : 0.f;
                    pp[4 * h + rr] = p;
                    ds[4 * h + rr] = (in && kok) ? p * (alpha * a2[rr] - st.z * du_scale) : 0.f;
                }
            }
            const Sp8 dsp = split8<true>(ds), ppp = split8<true>(pp);
            const int b0 = 2048 * qt + trv, b1 = two ? b0 + 2048 : b0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dk[j] = mma3(colfrag8_at(pA, b0 ^ (32 * j), b1 ^ (32 * j)), dsp, dk[j]);
                dv[j] = mma3(colfrag8_at(pB, b0 ^ (32 * j), b1 ^ (32 * j)), ppp, dv[j]);
            }
        }
        if (tok_in) {
            const float fkk = __builtin_ldexpf(0.125f, sg + sv + sq);
            const float fvv = alpha * __builtin_ldexpf(1.f, sg);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 16 * j + 4 * g;
                const long r0 = base + (long)tok * kD + d0;
                const float4 ck = load4<float>(dKc + r0), cv = load4<float>(dVc + r0);
                store4<T>(dK + r0, make_float4(fmaf(dk[j][0], fkk, ck.x), fmaf(dk[j][1], fkk, ck.y),
                                               fmaf(dk[j][2], fkk, ck.z), fmaf(dk[j][3], fkk, ck.w)));
                store4<T>(dV + r0, make_float4(fmaf(dv[j][0], fvv, cv.x), fmaf(dv[j][1], fvv, cv.y),
                                               fmaf(dv[j][2], fvv, cv.z), fmaf(dv[j][3], fvv, cv.w)));
            }
        }
    }
    if (tid == 0) {   // the slice's dalpha: local terms in token order minus the centroid term
        float t = 0.f;
        for (int i = 0; i < L; ++i) t += sStat[i].w;
        dal[slice] = t - dalc[slice];
    }
}

// ---------------------------------------------------------------- centroid branch
// The centroid branch's backward of one slice in one launch (L <= 128,
// K <= 16): the means mu and the cluster sums G_k = sum_{c_i = k} g_i from the
// one-hot products of the forward's update step, the centroid softmax
// P_c = softmax_j(mu_k . k_j / 8) (a padded key's logit -10000) with its
// statistics reduced across the waves, V^cent = P_c V only through
// GV_k = G_k . V^cent_k, and then
//   D_k = (1 - alpha) GV_k,  dP_kj = (1 - alpha) G_k . v_j,
//   dS_kj = P_kj (dP_kj - D_k) / 8   (0 for a padded key),
//   dK_j = sum_k dS_kj mu_k,  dV_j = (1 - alpha) sum_k P_kj G_k   (fp32 shares),
//   dmu_k = sum_j dS_kj k_j,  counts n_k,  and sum_k GV_k (the slice's
//   centroid term of dalpha, subtracted by the local kernel).
// Wave w owns key tile w: S_c, dP_c and dS_c sit in registers in [cluster
// 4g + r][key l16] orientation, which is the B operand of the 16-deep
// products with mu^T and G_k^T. V^cent and dmu come from [cluster][key]
// planes in LDS with the forward's centroid-context product.
namespace {
constexpr int kCOffMu = 4 * kPlane;                 // mu planes [16][64]
constexpr int kCOffGk = kCOffMu + 2 * kPlaneMu;     // G_k planes [16][64]
constexpr int kCOffR = kCOffGk + 2 * kPlaneMu;      // [16][128] planes: one-hot, P_c, dS_c
constexpr int kCLds = kCOffR + 2 * kPlaneRow;
static_assert(kCLds <= 81920, "two workgroups per CU");

// max / sum over the 16 lanes of a row (DPP rotations); lane 0 of the row
// holds a value that the caller publishes
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false)));
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false)));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
    return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
}
// A fragment of a [16][64] plane pair transposed for a 16-deep product:
// lane (l16, g) gets rows 4g .. 4g+3 of column 16j + l16
__device__ __forceinline__ Sp4 colfrag4_mu(const uint16_t *pl, int j, int l16, int g) {
    uint16_t h[4], m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int o = off64(4 * g + i, 16 * j + l16);
        h[i] = pl[o];
        m[i] = pl[kPlaneMuE + o];
    }
    return Sp4{u32x2_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)},
               u32x2_t{(uint32_t)m[0] | ((uint32_t)m[1] << 16), (uint32_t)m[2] | ((uint32_t)m[3] << 16)}};
}
}  // namespace

template <typename T, bool FULL, bool MASKED>
__global__ __launch_bounds__(kThreads, 4) void bwd_centroid_fused_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx,
    const T *__restrict__ dO, const int32_t *__restrict__ assign,
    const uint8_t *__restrict__ valid, int S, int L, int Kc, float alpha, int H,
    float *__restrict__ dKc, float *__restrict__ dVc, float *__restrict__ dmu,
    int32_t *__restrict__ counts, float *__restrict__ dalc, int solo_lo, int solo_hi) {
    __shared__ __align__(16) unsigned char smem[kCLds];
    uint16_t *sA = reinterpret_cast<uint16_t *>(smem);               // Q, then K planes
    uint16_t *sB = reinterpret_cast<uint16_t *>(smem + kBOffB);      // g, then V planes
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kCOffMu);
    uint16_t *sGk = reinterpret_cast<uint16_t *>(smem + kCOffGk);
    uint16_t *sR = reinterpret_cast<uint16_t *>(smem + kCOffR);
    // scratch inside the m plane of R while R holds only the one-hot (h) plane
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kCOffR + kPlaneRow);   // [8][8]
    float *sPart = reinterpret_cast<float *>(smem + kCOffR);                      // [16][8]
    float *sPart2 = sPart + 16 * 8;
    const u8 *pA = smem, *pB = smem + kBOffB, *pMu = smem + kCOffMu, *pGk = smem + kCOffGk,
             *pR = smem + kCOffR;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const long slice = blockIdx.x;
    if (slice >= S) return;
    // a workgroup alone on its CU starts about 2 us late, so that the loads of
    // the CUs holding two slices are served first (the launcher names these
    // workgroups)
    if ((int)blockIdx.x >= solo_lo && (int)blockIdx.x < solo_hi) __builtin_amdgcn_s_sleep(64);
    const int NT = FULL ? 8 : (L + 15) >> 4;
    const int tok = 16 * w + l16;   // the lane's key in the centroid phase
    const bool tok_in = FULL || tok < L;
    const long base = slice * (long)L * kD;
    const long brow = (slice / H) * (long)L;
    const LaneOffs lo = lane_offsets(l16, g);
    const int trq0 = 1024 * g + (lo.tr0 ^ (32 * (w & 3)));
    const int trq1 = 1024 * g + (lo.tr4 ^ (32 * (w & 3)));

    // ------------------------------------------------------------ loads
    // Q and dO now; K and V once the Q and g planes are written, so that
    // they arrive during the mean and cluster-sum products
    float qraw[2][8], graw[2][8], kraw[2][8], vraw[2][8];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n, row = it >> 3, col = (it & 7) * 8;
        load_row8<T, FULL>(Q + base, row, L, col, qraw[n]);
        load_row8<T, FULL>(dO + base, row, L, col, graw[n]);
        if (MASKED && row < L && valid[brow + row] == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) graw[n][i] = 0.f;
        }
    }
    // one-hot plane cleared (h plane of R: 4 KB, 8 bytes per thread)
    reinterpret_cast<u32x2_t *>(sR)[tid] = u32x2_t{0u, 0u};
    {
        const uint32_t bq = wave_max_u(__float_as_uint(absmax8(qraw[1], absmax8(qraw[0], 0.f))));
        const uint32_t bg = wave_max_u(__float_as_uint(absmax8(graw[1], absmax8(graw[0], 0.f))));
        if (lane == 0) {
            sMax[8 * w] = bq;
            sMax[8 * w + 3] = bg;
        }
    }
    if (MASKED && w < 2) {
        const int t = 64 * w + lane;
        const uint64_t bits = __ballot(t < L && valid[brow + t] != 0);
        if (lane == 0) {
            sMax[8 * (2 * w) + 4] = (uint32_t)bits;
            sMax[8 * (2 * w + 1) + 4] = (uint32_t)(bits >> 32);
        }
    }
    __syncthreads();
    KeyBits kb;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        kb.w[k] = MASKED ? (uint32_t)__builtin_amdgcn_readfirstlane((int)sMax[8 * k + 4]) : ~0u;
    uint32_t mq = 0, mg = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) {
        mq = max(mq, sMax[8 * ww]);
        mg = max(mg, sMax[8 * ww + 3]);
    }
    const int sq = scale_shift(mq, kQLimit), sg = scale_shift(mg, kBVLimit);
    const float fq = __builtin_ldexpf(1.f, -sq), fg = __builtin_ldexpf(1.f, -sg);
    __syncthreads();   // maxima and mask words read: the m plane of R is free
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;
        const int o = off64(it >> 3, (it & 7) * 8);
        float x[8], y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = qraw[n][i] * fq;
            y[i] = graw[n][i] * fg;
        }
        const Sp8 qp = split8(x), gp = split8(y);
        st16(sA + o, qp.h);
        st16(sA + kPlaneE + o, qp.m);
        st16(sB + o, gp.h);
        st16(sB + kPlaneE + o, gp.m);
    }
    if (g == 0 && tok_in) {   // one-hot of the given assignment
        const int c = min(max(assign[slice * L + tok], 0), Kc - 1);
        sR[off128(c, tok)] = 0x3c00;   // fp16 1.0
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n, row = it >> 3, col = (it & 7) * 8;
        load_row8<T, FULL>(Kx + base, row, L, col, kraw[n]);
        load_row8<T, FULL>(Vx + base, row, L, col, vraw[n]);
    }
    __syncthreads();

    // ------------------------------------------------------------ mu and G_k
    // waves 0-3: (Q^T one-hot)[dim 16w + 4g + rr][cluster l16] and the counts;
    // waves 4-7: (g^T one-hot) for dims 16(w - 4) + 4g + rr
    int sgk;   // G_k planes hold G_k 2^-sgk (G_k itself in units of 2^sg)
    {
        const u8 *src = w < 4 ? pA : pB;
        f32x4_t sh = kZero4, sm = kZero4, cnt = kZero4;
        const u32x4_t ones = {kOneH2, kOneH2, kOneH2, kOneH2};
        const int nch = (NT + 1) >> 1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (c < nch) {
                const u32x4_t oh = ldb16(pR, lo.rl128 ^ (64 * c));
                const Sp8 qt = colfrag8_at(src, 4096 * c + trq0, 4096 * c + trq1);
                sm = mma(qt.m, oh, sm);
                sh = mma(qt.h, oh, sh);
                cnt = mma(ones, oh, cnt);
            }
        }
        const float scale = w < 4 ? __builtin_amdgcn_rcpf(fmaxf(cnt[0], 1.f)) : 1.f;
        float v[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) v[rr] = (sm[rr] + sh[rr]) * scale;
        const int o = off64(l16, 16 * (w & 3) + 4 * g);
        if (w < 4) {
            const Sp4 p4 = split4(v[0], v[1], v[2], v[3]);
            st8(sMu + o, p4.h);
            st8(sMu + kPlaneMuE + o, p4.m);
            if (w == 0 && g == 0 && l16 < Kc) counts[slice * Kc + l16] = (int32_t)cnt[0];
        } else {
            // a cluster sum can reach L times the largest g: it gets its own
            // power-of-two scale before its planes are written
            const float m4 = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
            const uint32_t bm = wave_max_u(__float_as_uint(m4));
            if (lane == 0) sMax[8 * w + 5] = bm;
        }
        __syncthreads();
        uint32_t mgk = 0;
#pragma unroll
        for (int ww = 4; ww < 8; ++ww) mgk = max(mgk, sMax[8 * ww + 5]);
        sgk = scale_shift(mgk, kBVLimit);
        if (w >= 4) {
            const float f = __builtin_ldexpf(1.f, -sgk);
            const Sp4 p4 = split4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
            st8(sGk + o, p4.h);
            st8(sGk + kPlaneMuE + o, p4.m);
        }
    }
    {   // K and V maxima (slots 1 and 2 are free since the first barrier)
        const uint32_t bk = wave_max_u(__float_as_uint(absmax8(kraw[1], absmax8(kraw[0], 0.f))));
        const uint32_t bv = wave_max_u(__float_as_uint(absmax8(vraw[1], absmax8(vraw[0], 0.f))));
        if (lane == 0) {
            sMax[8 * w + 1] = bk;
            sMax[8 * w + 2] = bv;
        }
    }
    __syncthreads();
    uint32_t mk = 0, mv = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) {
        mk = max(mk, sMax[8 * ww + 1]);
        mv = max(mv, sMax[8 * ww + 2]);
    }
    const int sk = scale_shift(mk, kKVLimit), sv = scale_shift(mv, kBVLimit);
    const float fk = __builtin_ldexpf(1.f, -sk), fv = __builtin_ldexpf(1.f, -sv);
    // K and V planes replace Q and g
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int it = tid + kThreads * n;
        const int o = off64(it >> 3, (it & 7) * 8);
        float x[8], y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = kraw[n][i] * fk;
            y[i] = vraw[n][i] * fv;
        }
        const Sp8 kp = split8(x), vp = split8(y);
        st16(sA + o, kp.h);
        st16(sA + kPlaneE + o, kp.m);
        st16(sB + o, vp.h);
        st16(sB + kPlaneE + o, vp.m);
    }
    __syncthreads();

    // ------------------------------------------------------------ centroid softmax
    const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;
    const Sp8 kf0 = frag_at(pA, kPlane, 2048 * w + lo.rl64);
    const Sp8 kf1 = frag_at(pA, kPlane, 2048 * w + (lo.rl64 ^ 64));
    const Sp8 vf0 = frag_at(pB, kPlane, 2048 * w + lo.rl64);
    const Sp8 vf1 = frag_at(pB, kPlane, 2048 * w + (lo.rl64 ^ 64));
    f32x4_t a = mma3(frag_at(pMu, kPlaneMu, lo.rl64), kf0, kZero4);   // [cluster 4g + r][key l16]
    a = mma3(frag_at(pMu, kPlaneMu, lo.rl64 ^ 64), kf1, a);
    f32x4_t dp = mma3(frag_at(pGk, kPlaneMu, lo.rl64), vf0, kZero4);  // G_k . v_key (scaled)
    dp = mma3(frag_at(pGk, kPlaneMu, lo.rl64 ^ 64), vf1, dp);
    const bool kok = !MASKED || ((kb.tile(w) >> l16) & 1u);
    float s2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool in = tok_in && 4 * g + r < Kc;
        s2[r] = in ? (kok ? a[r] * sscale2 : kPadLogit2) : -__builtin_inff();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float m = row16_max(s2[r]);
        if (l16 == 0) sPart[(4 * g + r) * 8 + w] = m;
    }
    __syncthreads();
    float mc[4], e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float m = -__builtin_inff();
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) m = fmaxf(m, sPart[(4 * g + r) * 8 + ww]);
        mc[r] = m == -__builtin_inff() ? 0.f : m;   // clusters past Kc: no keys
        e[r] = __builtin_amdgcn_exp2f(s2[r] - mc[r]);
        const float z = row16_sum(e[r]);
        if (l16 == 0) sPart2[(4 * g + r) * 8 + w] = z;
    }
    __syncthreads();
    float pc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float z = 0.f;
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) z += sPart2[(4 * g + r) * 8 + ww];
        pc[r] = z > 0.f ? e[r] / z : 0.f;
    }
    __syncthreads();   // scratch read: R takes the P_c planes [cluster][key]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        uint32_t h, m;
        split2(pc[r], 0.f, h, m);
        const int o = off128(4 * g + r, tok);
        sR[o] = (uint16_t)(h & 0xffffu);
        sR[kPlaneRowE + o] = (uint16_t)(m & 0xffffu);
    }
    __syncthreads();
    // GV_k = G_k . V^cent_k: waves 0-3 form V^cent^T[dim 16w + 4g + rr][cluster l16]
    float gvpart = 0.f;
    if (w < 4) {
        const int nch = (NT + 1) >> 1;
        f32x4_t acc = kZero4;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (c < nch)
                acc = mma3(colfrag8_at(pB, 4096 * c + trq0, 4096 * c + trq1),
                           frag_at(pR, kPlaneRow, lo.rl128 ^ (64 * c)), acc);
        const int o = off64(l16, 16 * w + 4 * g);
        const u32x2_t gh = *reinterpret_cast<const u32x2_t *>(sGk + o);
        const u32x2_t gm = *reinterpret_cast<const u32x2_t *>(sGk + kPlaneMuE + o);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) gvpart = fmaf(half_at(gh, rr) + half_at(gm, rr), acc[rr], gvpart);
        gvpart = col_sum(gvpart);   // cluster l16, dims of tile w (scaled units)
    }
    __syncthreads();   // P_c planes read: the scratch returns
    if (w < 4 && g == 0) sPart[l16 * 8 + w] = gvpart;
    __syncthreads();
    const float gvs = __builtin_ldexpf(1.f, sg + sgk + sv);   // scaled G . V -> real
    float dcu[4];   // D_k in units of the scaled products
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int k = 4 * g + r;
        const float gv = sPart[k * 8] + sPart[k * 8 + 1] + sPart[k * 8 + 2] + sPart[k * 8 + 3];
        dcu[r] = (1.0f - alpha) * gv;
    }
    if (tid == 0) {   // the slice's centroid term of dalpha: sum_k G_k . V^cent_k (real)
        float t = 0.f;
        for (int k = 0; k < Kc; ++k)
            t += sPart[k * 8] + sPart[k * 8 + 1] + sPart[k * 8 + 2] + sPart[k * 8 + 3];
        dalc[slice] = t * gvs;
    }
    // dS_c in units of the scaled products; a padded key's logit is a constant
    float dsu[4], pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        dsu[r] = kok ? pc[r] * ((1.0f - alpha) * dp[r] - dcu[r]) : 0.f;
        pv[r] = (1.0f - alpha) * pc[r];
    }
    // dK_c^T = mu^T dS_c and dV_c^T = G_k^T ((1 - alpha) P_c): [dim 16j + 4g + r][key l16]
    {
        const Sp4 dsp = split4<true>(dsu[0], dsu[1], dsu[2], dsu[3]);
        const Sp4 pvp = split4<true>(pv[0], pv[1], pv[2], pv[3]);
        const float fkk = __builtin_ldexpf(0.125f, sg + sgk + sv + sq);
        const float fvv = __builtin_ldexpf(1.f, sg + sgk);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4_t dk = mma3_16(colfrag4_mu(sMu, j, l16, g), dsp, kZero4);
            const f32x4_t dv = mma3_16(colfrag4_mu(sGk, j, l16, g), pvp, kZero4);
            if (tok_in) {
                const long r0 = base + (long)tok * kD + 16 * j + 4 * g;
                *reinterpret_cast<float4 *>(dKc + r0) =
                    make_float4(dk[0] * fkk, dk[1] * fkk, dk[2] * fkk, dk[3] * fkk);
                *reinterpret_cast<float4 *>(dVc + r0) =
                    make_float4(dv[0] * fvv, dv[1] * fvv, dv[2] * fvv, dv[3] * fvv);
            }
        }
    }
    __syncthreads();   // scratch read: R takes the dS_c planes
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        uint32_t h, m;
        split2(dsu[r], 0.f, h, m);
        const int o = off128(4 * g + r, tok);
        sR[o] = (uint16_t)(h & 0xffffu);
        sR[kPlaneRowE + o] = (uint16_t)(m & 0xffffu);
    }
    __syncthreads();
    // dmu^T[dim 16w + 4g + rr][cluster l16] = K^T dS_c^T (waves 0-3)
    if (w < 4) {
        const int nch = (NT + 1) >> 1;
        f32x4_t acc = kZero4;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (c < nch)
                acc = mma3(colfrag8_at(pA, 4096 * c + trq0, 4096 * c + trq1),
                           frag_at(pR, kPlaneRow, lo.rl128 ^ (64 * c)), acc);
        if (l16 < Kc) {
            const float f = __builtin_ldexpf(0.125f, sg + sgk + sv + sk);
            *reinterpret_cast<float4 *>(dmu + (slice * Kc + l16) * kD + 16 * w + 4 * g) =
                make_float4(acc[0] * f, acc[1] * f, acc[2] * f, acc[3] * f);
        }
    }
}

bool bwd_fused_supported(int L, int Kc, int G) {
    return G == 1 && L >= 1 && L <= kFL && Kc >= 1 && Kc <= kFK;
}

template <typename T, bool FULL, bool MASKED>
static hipError_t bwd_fused_launch_t(const BwdArgs &a, hipStream_t st) {
    const T *q = static_cast<const T *>(a.Q), *k = static_cast<const T *>(a.K);
    const T *v = static_cast<const T *>(a.V), *go = static_cast<const T *>(a.dO);
    const int S = a.B * a.H;
    float *dalc = reinterpret_cast<float *>(a.lstat);   // one float per slice
    int32_t *counts = const_cast<int32_t *>(a.counts);
    hipLaunchKernelGGL((bwd_centroid_fused_kernel<T, FULL, MASKED>), dim3((unsigned)S),
                       dim3(kThreads), 0, st, q, k, v, go, a.assign, a.valid, S, a.L, a.Kc, a.alpha,
                       a.H, a.dkc, a.dvl, a.dmu, counts, dalc, a.solo_lo, a.solo_hi);
    hipLaunchKernelGGL((bwd_local_fused_kernel<T, FULL, MASKED>), dim3((unsigned)S),
                       dim3(kThreads), 0, st, q, k, v, go, a.assign, a.valid, dalc, a.dmu,
                       a.counts, a.dkc, a.dvl, S, a.L, a.Kc, a.r, a.alpha, a.H,
                       static_cast<T *>(a.dQ), static_cast<T *>(a.dK), static_cast<T *>(a.dV),
                       a.dal, a.solo_lo, a.solo_hi);
    return hipGetLastError();
}

template <typename T>
static hipError_t bwd_fused_dispatch(const BwdArgs &a, hipStream_t st) {
    if (a.L == kFL)
        return a.valid ? bwd_fused_launch_t<T, true, true>(a, st)
                       : bwd_fused_launch_t<T, true, false>(a, st);
    return a.valid ? bwd_fused_launch_t<T, false, true>(a, st)
                   : bwd_fused_launch_t<T, false, false>(a, st);
}

hipError_t launch_backward_fused(const BwdArgs &a, ca_dtype_t dt, hipStream_t st) {
    if (dt == CA_BF16) return bwd_fused_dispatch<bf16_t>(a, st);
    return bwd_fused_dispatch<float>(a, st);
}

}  // namespace ca
