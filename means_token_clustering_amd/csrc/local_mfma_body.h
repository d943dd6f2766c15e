// The window branch on the fp16 matrix cores for one 128-query block (its
// LDS layout and local_window_block), shared by local_mfma_kernel and the
// clustering launch that runs the window blocks beside the Lloyd iterations
// (kmeans_slice.hip).
#pragma once
#include <type_traits>
#include "launch.h"
#include "mfma_split.h"

namespace ca {
namespace {

constexpr int kMRows = 160;                  // 16 halo + 128 + 16 halo key rows
constexpr int kMPlane = kMRows * kD * 2;     // bytes of one fp16 plane
constexpr int kMPlaneE = kMPlane / 2;
constexpr int kMOffV = 2 * kMPlane;
constexpr int kMLds = 4 * kMPlane;           // 81,920 B: two workgroups per CU
constexpr int kMChunks = kMRows * kD / 8;    // 8-element chunks per staged tensor
constexpr int kMItems = (kMChunks + kThreads - 1) / kThreads;
constexpr int kTabRows = 16;                 // V^cent table in LDS for Kc <= 16
constexpr int kTabStride = kD + 4;           // floats per table row (bank spread)

}  // namespace

// One 128-query block of the window branch on the fp16 matrix cores, run by
// local_mfma_kernel (local_mfma.hip, where the branch and its arithmetic are
// described) and by the clustering launch that runs the window blocks beside
// the Lloyd iterations (kmeans_slice.hip). smem: kMLds bytes of LDS of this
// block; tid: 0 .. 511; bid: slice * nblk + block. OLOC: store alpha O^loc as
// fp32 rows to oloc (zero rows for padded queries) instead of the fused
// output (1 - alpha) V^cent_{c_i} + alpha O^loc to out; vcent, assign, out
// and xpart are then unused. MASKED: valid is the key-padding mask [S / H,
// L]. XPART: xpart (2 .. kXMergeInLocal key-range partials, nsplit of them)
// replaces vcent.
template <typename T, bool MASKED, bool OLOC, bool XPART>
__device__ __forceinline__ void local_window_block(
    const T *Q, const T *Kx, const T *Vx, int L, int rad, int nblk, const float *vcent,
    const int32_t *assign, int Kc, float alpha, const uint8_t *valid, int H, int G, T *out,
    const float *xpart, int nsplit, float *oloc, unsigned char *smem, int tid, unsigned bid) {
    uint16_t *sK = reinterpret_cast<uint16_t *>(smem);
    uint16_t *sV = reinterpret_cast<uint16_t *>(smem + kMOffV);
    // per-wave maxima [8][4] and the five key-mask words, in the last 256
    // bytes of the V m plane until the planes are written
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kMLds - 256);
    const u8 *pK = smem, *pV = smem + kMOffV;

    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int blk = bid % nblk;
    const long s = bid / nblk;
    const long brow = (s / H) * (long)L;
    const long base = s * (long)L * kD;
    const long kvbase = kv_slice(s, H, G) * (long)L * kD;
    const int i0 = 128 * blk;                      // first query of the block
    const int t0 = blk == 0 ? 0 : 8 * blk - 1;     // first staged key tile
    const int r0 = 16 * t0;                        // ... and row
    const int Lp = min(L, i0 + 144) - r0;          // staged rows that hold keys
    const int NTp = (Lp + 15) >> 4;
    const int qt = 8 * blk - t0 + w;               // the wave's query tile among the staged rows
    const int tok = i0 + 16 * w + l16;             // the lane's query
    const bool wave_on = i0 + 16 * w < L;
    const LaneOffs lo = lane_offsets(l16, g);
    const int trv = 1024 * (g >> 1) + ((g & 1) ? lo.tr4 : lo.tr0);

    float qraw[2][8], kraw[kMItems][8], vraw[kMItems][8];
#pragma unroll
    for (int c = 0; c < 2; ++c) load_row8<T, false>(Q + base, tok, L, 32 * c + 8 * g, qraw[c]);
    const T *Ks = Kx + kvbase + (long)r0 * kD, *Vs = Vx + kvbase + (long)r0 * kD;
#pragma unroll
    for (int n = 0; n < kMItems; ++n) {
        const int it = tid + kThreads * n;   // row it / 8, dims 8 (it % 8) ..
        if (it < kMChunks) {
            load_row8<T, false>(Ks, it >> 3, Lp, (it & 7) * 8, kraw[n]);
            load_row8<T, false>(Vs, it >> 3, Lp, (it & 7) * 8, vraw[n]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) kraw[n][i] = vraw[n][i] = 0.f;
        }
    }
    // V^cent rows of the slice, requested with the inputs (Kc <= 16): thread
    // t holds row t / 32, dims 2 (t % 32) .. of the table; with xpart the rows
    // are merged from the key-range partials (range order, as the combine)
    const bool table = !OLOC && Kc <= kTabRows;
    const int tk = tid >> 5, td = 2 * (tid & 31);
    float2 tpa[kXMergeInLocal], tpml[kXMergeInLocal];
    if (table && tk < Kc) {
        if (XPART) {
            const float *p0 = xpart + (s * nsplit * (long)Kc + tk) * kXPartStride;
#pragma unroll
            for (int r = 0; r < kXMergeInLocal; ++r) {
                const float *pr = p0 + (r < nsplit ? r : 0) * (long)Kc * kXPartStride;
                tpml[r] = *reinterpret_cast<const float2 *>(pr + kD);
                tpa[r] = *reinterpret_cast<const float2 *>(pr + td);
            }
        } else {
            tpa[0] = *reinterpret_cast<const float2 *>(vcent + (s * Kc + tk) * kD + td);
        }
    }
    const int cpre = !OLOC && tok < L ? assign[s * L + tok] : 0;
    {
        float mk = 0.f, mv = 0.f;
#pragma unroll
        for (int n = 0; n < kMItems; ++n) {
            mk = absmax8(kraw[n], mk);
            mv = absmax8(vraw[n], mv);
        }
        const uint32_t bq = wave_max_u(__float_as_uint(absmax8(qraw[1], absmax8(qraw[0], 0.f))));
        const uint32_t bk = wave_max_u(__float_as_uint(mk));
        const uint32_t bv = wave_max_u(__float_as_uint(mv));
        if (lane == 0) {
            sMax[4 * w] = bq;
            sMax[4 * w + 1] = bk;
            sMax[4 * w + 2] = bv;
        }
    }
    if (MASKED && w < 3) {   // key mask of staged rows 64w .. 64w+63
        const int row = 64 * w + lane;
        const uint64_t bits = __ballot(row < Lp && valid[brow + r0 + row] != 0);
        if (lane == 0) {
            sMax[32 + 2 * w] = (uint32_t)bits;
            if (w < 2) sMax[32 + 2 * w + 1] = (uint32_t)(bits >> 32);
        }
    }
    __syncthreads();
    uint32_t mq = 0, mk = 0, mv = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) {
        mq = max(mq, sMax[4 * ww]);
        mk = max(mk, sMax[4 * ww + 1]);
        mv = max(mv, sMax[4 * ww + 2]);
    }
    KeyBits160 kb;
#pragma unroll
    for (int k = 0; k < 5; ++k)
        kb.w[k] = MASKED ? (uint32_t)__builtin_amdgcn_readfirstlane((int)sMax[32 + k]) : ~0u;
    const int sq = scale_shift(mq, kQLimit), sk = scale_shift(mk, kKVLimit);
    const int sv = scale_shift(mv, kKVLimit);
    __syncthreads();   // the maxima are read: the planes may cover them

    Sp8 qf[2];
    {
        const float fq = __builtin_ldexpf(1.f, -sq);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = qraw[c][i] * fq;
            qf[c] = split8<true>(x);
        }
    }
    {
        const float fk = __builtin_ldexpf(1.f, -sk), fv = __builtin_ldexpf(1.f, -sv);
#pragma unroll
        for (int n = 0; n < kMItems; ++n) {
            const int it = tid + kThreads * n;
            if (it < kMChunks) {
                float x[8], y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[i] = kraw[n][i] * fk;
                    y[i] = vraw[n][i] * fv;
                }
                const Sp8 kp = split8(x), vp = split8(y);
                const int o = off64(it >> 3, (it & 7) * 8);
                st16(sK + o, kp.h);
                if (!bf16_storage<T>()) st16(sK + kMPlaneE + o, kp.m);   // zero for bf16 storage, never read
                st16(sV + o, vp.h);
                if (!bf16_storage<T>()) st16(sV + kMPlaneE + o, vp.m);   // zero for bf16 storage, never read
            }
        }
    }
    float2 tab = {0.f, 0.f};
    if (table && tk < Kc) {
        if (XPART) {
            float M = tpml[0].x;
#pragma unroll
            for (int r = 1; r < kXMergeInLocal; ++r) M = r < nsplit ? fmaxf(M, tpml[r].x) : M;
            float e[kXMergeInLocal], den = 0.f, n0 = 0.f, n1 = 0.f;
#pragma unroll
            for (int r = 0; r < kXMergeInLocal; ++r) {
                e[r] = r < nsplit ? exp_f32(tpml[r].x - M) : 0.f;
                den = fmaf(e[r], tpml[r].y, den);
            }
            const float inv = 1.0f / den;
#pragma unroll
            for (int r = 0; r < kXMergeInLocal; ++r) {
                n0 = fmaf(e[r], tpa[r].x, n0);
                n1 = fmaf(e[r], tpa[r].y, n1);
            }
            tab = make_float2(n0 * inv, n1 * inv);
        } else {
            tab = tpa[0];
        }
    }
    __syncthreads();

    f32x4_t o[4];
    float lsum = 1.f;
    if (wave_on) {
        const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;
        local_narrow<false, MASKED, KeyBits160, kMPlane, bf16_storage<T>()>(
            pK, pV, qf, qt, NTp, Lp, rad, sscale2, l16, g, lo.rl64, trv, kb, o, lsum);
    }
    __syncthreads();   // the K planes become the output staging area, the V
                       // planes the V^cent table
    const float *sTab = reinterpret_cast<const float *>(smem + kMOffV);
    if (table) {
        if (tk < Kc)
            *reinterpret_cast<float2 *>(smem + kMOffV + 4 * (tk * kTabStride + td)) = tab;
        __syncthreads();
    }

    // fused rows of the wave's tile through a wave-private LDS tile (16 rows,
    // 16-byte chunks XOR-swizzled by the row), then whole-row stores
    if (!wave_on) return;
    using OT = typename std::conditional<OLOC, float, T>::type;   // stored row type
    constexpr int kRowB = kD * (int)sizeof(OT);
    constexpr int kCpr = kRowB / 16;
    u8 *stg = smem + w * 16 * kRowB;
    {
        const bool tok_in = tok < L;
        const float f = alpha * __builtin_ldexpf(1.f, sv) * __builtin_amdgcn_rcpf(lsum);
        const int c = tok_in ? min(max(cpre, 0), Kc - 1) : 0;
        const bool keep = tok_in && (!MASKED || valid[brow + tok] != 0);
        const float wg = 1.0f - alpha;
        float4 cv[4];   // V^cent_c, dims 16j + 4g .. (zero: alpha O^loc alone)
        if (OLOC) {
#pragma unroll
            for (int j = 0; j < 4; ++j) cv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        } else if (table) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                cv[j] = *reinterpret_cast<const float4 *>(sTab + c * kTabStride + 16 * j + 4 * g);
        } else if (XPART) {
            // merge the key-range partials of row (s, c) in range order:
            // V^cent = sum_r e^(m_r - M) acc_r / sum_r e^(m_r - M) l_r
            const float *p0 = xpart + (s * nsplit * (long)Kc + c) * kXPartStride;
            const long rs = (long)Kc * kXPartStride;
            float m[kXMergeInLocal], l[kXMergeInLocal];
            float2 a[kXMergeInLocal][4][2];
#pragma unroll
            for (int r = 0; r < kXMergeInLocal; ++r) {
                const float *pr = p0 + (r < nsplit ? r : 0) * rs;
                const float2 ml = *reinterpret_cast<const float2 *>(pr + kD);
                m[r] = r < nsplit ? ml.x : -__builtin_inff();
                l[r] = ml.y;
#pragma unroll
                for (int j = 0; j < 4; ++j) {   // 8-byte aligned: the stride is 66 floats
                    a[r][j][0] = *reinterpret_cast<const float2 *>(pr + 16 * j + 4 * g);
                    a[r][j][1] = *reinterpret_cast<const float2 *>(pr + 16 * j + 4 * g + 2);
                }
            }
            float M = m[0];
#pragma unroll
            for (int r = 1; r < kXMergeInLocal; ++r) M = fmaxf(M, m[r]);
            float e[kXMergeInLocal], den = 0.f;
#pragma unroll
            for (int r = 0; r < kXMergeInLocal; ++r) {
                e[r] = r < nsplit ? exp_f32(m[r] - M) : 0.f;
                den = fmaf(e[r], l[r], den);
            }
            const float inv = 1.0f / den;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float n0 = 0.f, n1 = 0.f, n2 = 0.f, n3 = 0.f;
#pragma unroll
                for (int r = 0; r < kXMergeInLocal; ++r) {
                    n0 = fmaf(e[r], a[r][j][0].x, n0);
                    n1 = fmaf(e[r], a[r][j][0].y, n1);
                    n2 = fmaf(e[r], a[r][j][1].x, n2);
                    n3 = fmaf(e[r], a[r][j][1].y, n3);
                }
                cv[j] = make_float4(n0 * inv, n1 * inv, n2 * inv, n3 * inv);
            }
        } else {
            const float *vc = vcent + (s * Kc + c) * kD;
#pragma unroll
            for (int j = 0; j < 4; ++j) cv[j] = load4<float>(vc + 16 * j + 4 * g);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // o[j][rr] = Oloc^T[dim 16j + 4g + rr][query tok]
            const int d0 = 16 * j + 4 * g;
            const float4 c4 = cv[j];
            float v0 = fmaf(o[j][0], f, wg * c4.x), v1 = fmaf(o[j][1], f, wg * c4.y);
            float v2 = fmaf(o[j][2], f, wg * c4.z), v3 = fmaf(o[j][3], f, wg * c4.w);
            if (!keep) v0 = v1 = v2 = v3 = 0.f;
            const int byte = d0 * (int)sizeof(OT);
            u8 *p = stg + l16 * kRowB + ((((byte >> 4) ^ (l16 & (kCpr - 1)))) << 4) + (byte & 15);
            if (sizeof(OT) == 4) {
                *reinterpret_cast<f32x4_t *>(p) = f32x4_t{v0, v1, v2, v3};
            } else {
                *reinterpret_cast<u32x2_t *>(p) =
                    u32x2_t{(uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16),
                            (uint32_t)f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16)};
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    u8 *dst = OLOC ? reinterpret_cast<u8 *>(oloc + base + (long)(i0 + 16 * w) * kD)
                   : reinterpret_cast<u8 *>(out + base + (long)(i0 + 16 * w) * kD);
    const int nrow = min(16, L - (i0 + 16 * w));
#pragma unroll
    for (int i = 0; i < kCpr / 4; ++i) {   // 64 chunks = 64 / kCpr rows per store
        const int flat = 64 * i + lane;
        const int row = flat / kCpr, ch = flat % kCpr;
        const u32x4_t v =
            *reinterpret_cast<const u32x4_t *>(stg + row * kRowB + (((ch ^ (row & (kCpr - 1)))) << 4));
        if (row < nrow) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst + flat * 16));
    }
}

}  // namespace ca
