// Single-launch cluster attention forward for short sequences (L <= 128,
// K <= 16, d = 64). Each workgroup (512 threads, 8 waves) runs the whole path
// of one (b, h) slice on chip - Lloyd's k-means, centroid cross-attention,
// the local window branch and the gather + convex fusion - and touches HBM
// only to read Q, K, V once and to write the output and the assignment.
//
// Method: model card "Hooshaai/distilbert-sst2-cluster-attention",
// Architecture Overview figure and Mathematical Formulation 1; "ClusterFormer"
// spec (svd-sst2-roberta-cluster page) 2.1 and 3. Conventions as in the
// staged kernels: ties to the lowest cluster, empty cluster -> zero vector,
// window |i - j| <= floor(W/2), scale 1/sqrt(d).
//
// Arithmetic: every contraction runs on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16 / 16x16x16) with fp32 accumulation. Each fp32
// operand x is split exactly into three bf16 parts x = h + m + l (truncation:
// h keeps the top 8 significand bits, m the next 8, l the last 8), and a
// product a.b is accumulated from the six partial products whose weight is
// at least 2^-16 of the leading one (l.h, h.l, m.m, m.h, h.m, h.h), which
// leaves a relative error of order 2^-24, i.e. fp32 grade. The one-hot
// products (centroid sums and counts) need three and one (exact 0/1 side).
//
// Layouts (confirmed on gfx950): for 16x16x32, lane l holds A[l%16][8(l/16)+i]
// and B[8(l/16)+i][l%16], i = 0..7; the 16x16 result has lane l, register r
// at D[4(l/16)+r][l%16]. 16x16x16 is the same with 4 values per lane.
//
// Work split per slice (token tile = 16 tokens, NT = ceil(L/16) <= 8):
//   wave w owns token tile w: its Q fragments stay in registers for the
//   distance products and the local-window scores; waves 0-3 own dim tile w
//   of the centroid sums (one-hot^T Q) and keep Q in that layout too;
//   K and V live in LDS as split planes (V transposed) for all waves.
#include "common.h"

namespace ca {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kFL = 128;              // max tokens
constexpr int kFK = 16;               // max clusters
constexpr int kThreads = 512;         // 8 waves
constexpr int kKRow = 72;             // K / centroid plane row stride in bf16 (64 + 8)
constexpr int kVRow = 136;            // V^T plane row stride in bf16 (128 + 8)
constexpr int kKPlane = kFL * kKRow;  // bf16 elements per K plane
constexpr int kVPlane = kD * kVRow;   // bf16 elements per V^T plane
constexpr int kMuPlane = kFK * kKRow; // bf16 elements per centroid plane
constexpr int kMuRow = 68;            // fp32 row stride of mu and vcent
constexpr int kPartW = kD * kFK;      // fp32 partial V^cent per wave

constexpr size_t kLdsK = sizeof(uint16_t) * 3 * kKPlane;
constexpr size_t kLdsV = sizeof(uint16_t) * 3 * kVPlane;
constexpr size_t kLdsMuP = sizeof(uint16_t) * 3 * kMuPlane;
constexpr size_t kLdsMu = sizeof(float) * kFK * kMuRow;
constexpr size_t kLdsPart = sizeof(float) * 8 * kPartW;
// wave maxima [16][8], wave sums [16][8], ||mu||^2 partials [4][16], assignment [128]
constexpr size_t kLdsSmall = sizeof(float) * (2 * kFK * 8 + 4 * kFK) + sizeof(int) * kFL;
constexpr size_t kLdsTotal = kLdsK + kLdsV + kLdsMuP + 2 * kLdsMu + kLdsPart + kLdsSmall;
static_assert(kLdsTotal <= 160 * 1024, "LDS budget");

struct Split8 {  // 8 values as three bf16x8 planes (pairs packed low-first)
    u32x4_t h, m, l;
};
struct Split4 {  // 4 values as three bf16x4 planes
    u32x2_t h, m, l;
};

__device__ __forceinline__ uint32_t pack_hi(uint32_t lo_elem, uint32_t hi_elem) {
    return (lo_elem >> 16) | (hi_elem & 0xffff0000u);
}

// Exact split of two floats: x = h + m + l, each part a bf16 (truncation).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &h, uint32_t &m, uint32_t &l) {
    const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
    h = pack_hi(u0, u1);
    const float r0 = x0 - __uint_as_float(u0 & 0xffff0000u);
    const float r1 = x1 - __uint_as_float(u1 & 0xffff0000u);
    const uint32_t v0 = __float_as_uint(r0), v1 = __float_as_uint(r1);
    m = pack_hi(v0, v1);
    const float s0 = r0 - __uint_as_float(v0 & 0xffff0000u);
    const float s1 = r1 - __uint_as_float(v1 & 0xffff0000u);
    l = pack_hi(__float_as_uint(s0), __float_as_uint(s1));
}

__device__ __forceinline__ Split8 split8(const float *x) {
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(x[2 * i], x[2 * i + 1], h[i], m[i], l[i]);
    Split8 s;
    s.h = u32x4_t{h[0], h[1], h[2], h[3]};
    s.m = u32x4_t{m[0], m[1], m[2], m[3]};
    s.l = u32x4_t{l[0], l[1], l[2], l[3]};
    return s;
}

__device__ __forceinline__ Split4 split4(const float *x) {
    uint32_t h[2], m[2], l[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) split2(x[2 * i], x[2 * i + 1], h[i], m[i], l[i]);
    Split4 s;
    s.h = u32x2_t{h[0], h[1]};
    s.m = u32x2_t{m[0], m[1]};
    s.l = u32x2_t{l[0], l[1]};
    return s;
}

__device__ __forceinline__ f32x4_t mma32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mma16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// c += a . b to fp32 grade (six partial products, smallest first)
__device__ __forceinline__ f32x4_t mma32x6(const Split8 &a, const Split8 &b, f32x4_t c) {
    c = mma32(a.l, b.h, c);
    c = mma32(a.h, b.l, c);
    c = mma32(a.m, b.m, c);
    c = mma32(a.m, b.h, c);
    c = mma32(a.h, b.m, c);
    c = mma32(a.h, b.h, c);
    return c;
}

__device__ __forceinline__ f32x4_t mma16x6(const Split4 &a, const Split4 &b, f32x4_t c) {
    c = mma16(a.l, b.h, c);
    c = mma16(a.h, b.l, c);
    c = mma16(a.m, b.m, c);
    c = mma16(a.m, b.h, c);
    c = mma16(a.h, b.m, c);
    c = mma16(a.h, b.h, c);
    return c;
}

__device__ __forceinline__ f32x4_t add4(f32x4_t a, f32x4_t b) {
    return f32x4_t{a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
}

// ---- cross-lane helpers (no LDS traffic)
// Combine lane l with lane l^32 (resp. l^16): both lanes receive the two
// values, the lower lane's first, in the same order.
__device__ __forceinline__ void pair32(float v, float &lo, float &hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair16(float v, float &lo, float &hi) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32i(int v, int &lo, int &hi) {
    const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    lo = (int)r[0];
    hi = (int)r[1];
}
__device__ __forceinline__ void pair16i(int v, int &lo, int &hi) {
    const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    lo = (int)r[0];
    hi = (int)r[1];
}

// sum / max over the four lane groups g of a column (lanes l16, l16+16, ...);
// every lane of the column gets the same bits
__device__ __forceinline__ float col_sum(float v) {
    float a, b;
    pair16(v, a, b);
    v = a + b;
    pair32(v, a, b);
    return a + b;
}
__device__ __forceinline__ float col_max(float v) {
    float a, b;
    pair16(v, a, b);
    v = fmaxf(a, b);
    pair32(v, a, b);
    return fmaxf(a, b);
}

// lexicographic (value, index) minimum over the four lane groups of a column
__device__ __forceinline__ void col_argmin(float &best, int &bk) {
    float a, b;
    int ia, ib;
    pair16(best, a, b);
    pair16i(bk, ia, ib);
    if (lex_less(b, ib, a, ia)) { a = b; ia = ib; }
    pair32(a, best, b);
    pair32i(ia, bk, ib);
    if (lex_less(b, ib, best, bk)) { best = b; bk = ib; }
}

// DPP move within a row of 16 lanes
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;   // row_ror:4
constexpr int kDppRor8 = 0x128;   // row_ror:8

// sum over the 16 lanes of a row; lane l16 == 0 holds a fixed-order total
__device__ __forceinline__ float row_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppRor4>(v);
    v += dpp<kDppRor8>(v);
    return v;
}

// ---- storage access
template <typename T>
__device__ __forceinline__ void load8(const T *p, float *x) {
    const float4 a = load4<T>(p), b = load4<T>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <typename T>
__device__ __forceinline__ float load1(const T *p);
template <>
__device__ __forceinline__ float load1<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load1<bf16_t>(const bf16_t *p) { return bf16_to_f32(p->bits); }

// 8 consecutive elements of row `row` (zeros when row >= L)
template <typename T, bool FULL>
__device__ __forceinline__ void load_row8(const T *base, int row, int L, int col, float *x) {
    if (FULL) {
        load8<T>(base + (long)row * kD + col, x);
    } else {
        const int rc = row < L ? row : L - 1;
        load8<T>(base + (long)rc * kD + col, x);
        if (row >= L) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
    }
}

// rows r0..r0+7 of column `col` (zeros for rows >= L)
template <typename T, bool FULL>
__device__ __forceinline__ void load_col8(const T *base, int r0, int L, int col, float *x) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = r0 + i;
        if (FULL) {
            x[i] = load1<T>(base + (long)row * kD + col);
        } else {
            const int rc = row < L ? row : L - 1;
            const float v = load1<T>(base + (long)rc * kD + col);
            x[i] = row < L ? v : 0.f;
        }
    }
}

__device__ __forceinline__ u32x4_t lds_u32x4(const uint16_t *p) {
    return *reinterpret_cast<const u32x4_t *>(p);
}
__device__ __forceinline__ u32x2_t lds_u32x2(const uint16_t *p) {
    return *reinterpret_cast<const u32x2_t *>(p);
}
__device__ __forceinline__ void put_split8(uint16_t *dst, int plane, const Split8 &s) {
    *reinterpret_cast<u32x4_t *>(dst) = s.h;
    *reinterpret_cast<u32x4_t *>(dst + plane) = s.m;
    *reinterpret_cast<u32x4_t *>(dst + 2 * plane) = s.l;
}

// K fragment (rows = keys 16*kt + l16, dims 32c + 8g ..)
__device__ __forceinline__ Split8 k_frag(const uint16_t *sK, int kt, int c, int l16, int g) {
    const uint16_t *p = sK + (16 * kt + l16) * kKRow + 32 * c + 8 * g;
    Split8 s;
    s.h = lds_u32x4(p);
    s.m = lds_u32x4(p + kKPlane);
    s.l = lds_u32x4(p + 2 * kKPlane);
    return s;
}

// centroid fragment (rows = centroids l16, dims 32c + 8g ..)
__device__ __forceinline__ Split8 mu_frag(const uint16_t *sMuP, int c, int l16, int g) {
    const uint16_t *p = sMuP + l16 * kKRow + 32 * c + 8 * g;
    Split8 s;
    s.h = lds_u32x4(p);
    s.m = lds_u32x4(p + kMuPlane);
    s.l = lds_u32x4(p + 2 * kMuPlane);
    return s;
}

// V^T fragment for 16x16x16 (rows = dims 16j + l16, keys 16kt + 4g + i)
__device__ __forceinline__ Split4 v_frag_tile(const uint16_t *sV, int j, int kt, int l16, int g) {
    const uint16_t *p = sV + (16 * j + l16) * kVRow + 16 * kt + 4 * g;
    Split4 s;
    s.h = lds_u32x2(p);
    s.m = lds_u32x2(p + kVPlane);
    s.l = lds_u32x2(p + 2 * kVPlane);
    return s;
}

// V^T fragment over key tiles ka, kb for 16x16x32 in the order the score
// tiles hold them: lane group g takes keys 16ka + 4g + (0..3), 16kb + 4g + (0..3)
__device__ __forceinline__ Split8 v_frag_two(const uint16_t *sV, int j, int ka, int kb, int l16,
                                             int g) {
    const uint16_t *pa = sV + (16 * j + l16) * kVRow + 16 * ka + 4 * g;
    const uint16_t *pb = sV + (16 * j + l16) * kVRow + 16 * kb + 4 * g;
    Split8 s;
    u32x2_t a, b;
    a = lds_u32x2(pa);               b = lds_u32x2(pb);
    s.h = u32x4_t{a.x, a.y, b.x, b.y};
    a = lds_u32x2(pa + kVPlane);     b = lds_u32x2(pb + kVPlane);
    s.m = u32x4_t{a.x, a.y, b.x, b.y};
    a = lds_u32x2(pa + 2 * kVPlane); b = lds_u32x2(pb + 2 * kVPlane);
    s.l = u32x4_t{a.x, a.y, b.x, b.y};
    return s;
}

// store the split of two adjacent dims (d, d+1) of centroid k
__device__ __forceinline__ void put_mu_pair(uint16_t *sMuP, int k, int d, float x0, float x1) {
    uint32_t h, m, l;
    split2(x0, x1, h, m, l);
    uint16_t *p = sMuP + k * kKRow + d;
    *reinterpret_cast<uint32_t *>(p) = h;
    *reinterpret_cast<uint32_t *>(p + kMuPlane) = m;
    *reinterpret_cast<uint32_t *>(p + 2 * kMuPlane) = l;
}

// Raw (unsplit) inputs of one slice held by one thread between the fetch and
// the split: K items (row, 8-dim chunk) and V items (dim, 8-key group) -
// waves 0-3 take one of each, waves 4-7 three - the thread's Q row chunk
// pair, and for waves 0-3 the Q column block of the centroid sums.
struct Raw {
    float k[3][8];
    float v[3][8];
    float q[2][8];
    float qc[4][8];
};

template <typename T, bool FULL>
__device__ __forceinline__ void fetch_slice(const T *Q, const T *Kx, const T *Vx, long slice,
                                            int L, int tid, int w, int l16, int g, Raw &raw) {
    const long base = slice * (long)L * kD;
    const T *Qs = Q + base;
    const T *Ks = Kx + base;
    const T *Vs = Vx + base;
    const int nitems = w < 4 ? 1 : 3;
#pragma unroll
    for (int n = 0; n < 3; ++n) {
        if (n < nitems) {
            const int it = tid + 256 * n;
            load_row8<T, FULL>(Ks, it >> 3, L, (it & 7) * 8, raw.k[n]);
            load_col8<T, FULL>(Vs, (it >> 6) * 8, L, it & 63, raw.v[n]);
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) load_row8<T, FULL>(Qs, 16 * w + l16, L, 32 * c + 8 * g, raw.q[c]);
    if (w < 4) {
#pragma unroll
        for (int c = 0; c < 4; ++c) load_col8<T, FULL>(Qs, 32 * c + 8 * g, L, 16 * w + l16, raw.qc[c]);
    }
}

}  // namespace

template <typename T, bool FULL, bool NARROW>
__global__ __launch_bounds__(kThreads, 1) void cluster_attn_fused_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx, int S, int L,
    int Kc, int iters, int radius, float alpha, T *__restrict__ out,
    int32_t *__restrict__ assign_out) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t *sK = reinterpret_cast<uint16_t *>(smem);
    uint16_t *sV = reinterpret_cast<uint16_t *>(smem + kLdsK);
    uint16_t *sMuP = reinterpret_cast<uint16_t *>(smem + kLdsK + kLdsV);
    float *sMu = reinterpret_cast<float *>(smem + kLdsK + kLdsV + kLdsMuP);
    float *sVc = sMu + kFK * kMuRow;
    float *sPart = sVc + kFK * kMuRow;           // [8][kPartW]
    float *sXm = sPart + 8 * kPartW;             // [16][8] wave maxima
    float *sXl = sXm + 8 * kFK;                  // [16][8] wave sums
    float *sN2 = sXl + 8 * kFK;                  // [4][16] partial ||mu_k||^2
    int *sC = reinterpret_cast<int *>(sN2 + 4 * kFK);   // [128]

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int NT = FULL ? 8 : (L + 15) >> 4;
    const int tok = 16 * w + l16;
    const float scale = 0.125f;   // 1/sqrt(64), exact
    const int nitems = w < 4 ? 1 : 3;

    // the token this lane owns starts centroid k = ceil(tok Kc / L) when
    // floor(k L / Kc) == tok (the strided initial rows are distinct)
    int init_k = -1;
    {
        const int k = (tok * Kc + L - 1) / L;
        if (tok < L && k < Kc && (k * L) / Kc == tok) init_k = k;
    }

    const long slice = blockIdx.x;
    if (slice < S) {
        Raw raw;
        fetch_slice<T, FULL>(Q, Kx, Vx, slice, L, tid, w, l16, g, raw);
        // ------------- split this slice's inputs: K, V planes in LDS, Q in registers
#pragma unroll
        for (int n = 0; n < 3; ++n) {
            if (n < nitems) {
                const int it = tid + 256 * n;
                put_split8(sK + (it >> 3) * kKRow + (it & 7) * 8, kKPlane, split8(raw.k[n]));
                put_split8(sV + (it & 63) * kVRow + (it >> 6) * 8, kVPlane, split8(raw.v[n]));
            }
        }
        Split8 qf[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) qf[c] = split8(raw.q[c]);
        Split8 qc[4];
        if (w < 4) {
#pragma unroll
            for (int c = 0; c < 4; ++c) qc[c] = split8(raw.qc[c]);
        }
        // strided initial centroids mu_k = Q[floor(k L / Kc)] from the owning lanes
        if (init_k >= 0) {
            float n2 = 0.f;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int d0 = 32 * c + 8 * g;
                put_split8(sMuP + init_k * kKRow + d0, kMuPlane, qf[c]);
                float *m = sMu + init_k * kMuRow + d0;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    m[i] = raw.q[c][i];
                    n2 = fmaf(raw.q[c][i], raw.q[c][i], n2);
                }
            }
            sN2[g * kFK + init_k] = n2;
        }
        // centroids beyond Kc stay zero (never chosen)
        for (int e = tid; e < (kFK - Kc) * kD; e += kThreads) {
            const int k = Kc + e / kD, dd = e % kD;
            sMu[k * kMuRow + dd] = 0.f;
            sMuP[k * kKRow + dd] = 0;
            sMuP[kMuPlane + k * kKRow + dd] = 0;
            sMuP[2 * kMuPlane + k * kKRow + dd] = 0;
            if (dd < 4) sN2[dd * kFK + k] = 0.f;
        }
        if (!FULL && tid < kFL && tid >= L) sC[tid] = -1;   // padded tokens join no cluster
        __syncthreads();

        // ------------- Lloyd iterations
        for (int t = 1; t <= iters; ++t) {
            if (w < NT) {
                // acc[r] = mu_{4g+r} . q_tok - ||mu_{4g+r}||^2 / 2 (exact halving)
                f32x4_t a0, a1 = {0.f, 0.f, 0.f, 0.f};
                {
                    const float4 p0 = *reinterpret_cast<const float4 *>(sN2 + 0 * kFK + 4 * g);
                    const float4 p1 = *reinterpret_cast<const float4 *>(sN2 + 1 * kFK + 4 * g);
                    const float4 p2 = *reinterpret_cast<const float4 *>(sN2 + 2 * kFK + 4 * g);
                    const float4 p3 = *reinterpret_cast<const float4 *>(sN2 + 3 * kFK + 4 * g);
                    a0[0] = -0.5f * (((p0.x + p1.x) + p2.x) + p3.x);
                    a0[1] = -0.5f * (((p0.y + p1.y) + p2.y) + p3.y);
                    a0[2] = -0.5f * (((p0.z + p1.z) + p2.z) + p3.z);
                    a0[3] = -0.5f * (((p0.w + p1.w) + p2.w) + p3.w);
                }
                a0 = mma32x6(mu_frag(sMuP, 0, l16, g), qf[0], a0);
                a1 = mma32x6(mu_frag(sMuP, 1, l16, g), qf[1], a1);
                // D = ||mu||^2 - 2 mu.q = -2 (a0 + a1)
                float best = __builtin_inff();
                int bk = 0x7fffffff;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int k = 4 * g + r;
                    const float D = k < Kc ? -2.f * (a0[r] + a1[r]) : __builtin_inff();
                    if (lex_less(D, k, best, bk)) { best = D; bk = k; }
                }
                col_argmin(best, bk);
                if (bk >= Kc) bk = 0;   // only if every distance was NaN
                if (g == 0 && (FULL || tok < L)) sC[tok] = bk;
            }
            __syncthreads();
            if (w < 4) {
                // (one-hot^T Q)[centroid 4g+r][dim 16w + l16] and the cluster sizes
                f32x4_t sl = {0.f, 0.f, 0.f, 0.f}, sm = sl, sh = sl, cnt = sl;
                const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int4 ca = *reinterpret_cast<const int4 *>(sC + 32 * c + 8 * g);
                    const int4 cb = *reinterpret_cast<const int4 *>(sC + 32 * c + 8 * g + 4);
                    u32x4_t oh;
                    oh.x = (ca.x == l16 ? 0x3f80u : 0u) | (ca.y == l16 ? 0x3f800000u : 0u);
                    oh.y = (ca.z == l16 ? 0x3f80u : 0u) | (ca.w == l16 ? 0x3f800000u : 0u);
                    oh.z = (cb.x == l16 ? 0x3f80u : 0u) | (cb.y == l16 ? 0x3f800000u : 0u);
                    oh.w = (cb.z == l16 ? 0x3f80u : 0u) | (cb.w == l16 ? 0x3f800000u : 0u);
                    sl = mma32(oh, qc[c].l, sl);
                    sm = mma32(oh, qc[c].m, sm);
                    sh = mma32(oh, qc[c].h, sh);
                    cnt = mma32(oh, ones, cnt);
                }
                float v[4], n2p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = ((sl[r] + sm[r]) + sh[r]) / fmaxf(cnt[r], 1.f);
                    sMu[(4 * g + r) * kMuRow + 16 * w + l16] = v[r];
                    n2p[r] = row_sum(v[r] * v[r]);
                }
                if (l16 == 0)
                    *reinterpret_cast<float4 *>(sN2 + w * kFK + 4 * g) =
                        make_float4(n2p[0], n2p[1], n2p[2], n2p[3]);
                // split planes: lanes l16 and l16^1 hold adjacent dims; the even
                // lane stores centroids 4g, 4g+1, the odd lane 4g+2, 4g+3
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = dpp<kDppXor1>(v[r]);
                const int d = 16 * w + (l16 & ~1);
                if ((l16 & 1) == 0) {
                    put_mu_pair(sMuP, 4 * g + 0, d, v[0], o[0]);
                    put_mu_pair(sMuP, 4 * g + 1, d, v[1], o[1]);
                } else {
                    put_mu_pair(sMuP, 4 * g + 2, d, o[2], v[2]);
                    put_mu_pair(sMuP, 4 * g + 3, d, o[3], v[3]);
                }
            }
            __syncthreads();
        }

        // ------------- centroid cross-attention (wave w: key tile w)
        float sx[4];
        float mloc = -__builtin_inff();
        if (w < NT) {
            f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
            a0 = mma32x6(k_frag(sK, w, 0, l16, g), mu_frag(sMuP, 0, l16, g), a0);
            a1 = mma32x6(k_frag(sK, w, 1, l16, g), mu_frag(sMuP, 1, l16, g), a1);
            // a[r] = k_{16w+4g+r} . mu_{l16}
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = 16 * w + 4 * g + r;
                sx[r] = (FULL || key < L) ? (a0[r] + a1[r]) * scale : -__builtin_inff();
                mloc = fmaxf(mloc, sx[r]);
            }
            mloc = col_max(mloc);
        }
        if (g == 0) sXm[l16 * 8 + w] = mloc;
        __syncthreads();
        float M;
        {
            const float4 m0 = *reinterpret_cast<const float4 *>(sXm + l16 * 8);
            const float4 m1 = *reinterpret_cast<const float4 *>(sXm + l16 * 8 + 4);
            M = fmaxf(fmaxf(fmaxf(m0.x, m0.y), fmaxf(m0.z, m0.w)),
                      fmaxf(fmaxf(m1.x, m1.y), fmaxf(m1.z, m1.w)));
        }
        if (w < NT) {
            float p[4];
            float ls = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = sx[r] == -__builtin_inff() ? 0.f : exp_f32(sx[r] - M);
                ls += p[r];
            }
            ls = col_sum(ls);
            const Split4 pf = split4(p);
            float *part = sPart + w * kPartW;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma16x6(v_frag_tile(sV, j, w, l16, g), pf, acc);
                // acc[r] = partial Vc[centroid l16][dim 16j + 4g + r]
#pragma unroll
                for (int r = 0; r < 4; ++r) part[(16 * j + 4 * g + r) * kFK + l16] = acc[r];
            }
            if (g == 0) sXl[l16 * 8 + w] = ls;
        } else if (g == 0) {
            sXl[l16 * 8 + w] = 0.f;
        }
        __syncthreads();
        for (int e = tid; e < kFK * kD; e += kThreads) {
            const int k = e & 15, dim = e >> 4;
            float num = 0.f;
            for (int ww = 0; ww < NT; ++ww) num += sPart[ww * kPartW + dim * kFK + k];
            const float4 l0 = *reinterpret_cast<const float4 *>(sXl + k * 8);
            const float4 l1 = *reinterpret_cast<const float4 *>(sXl + k * 8 + 4);
            const float den = ((((((l0.x + l0.y) + l0.z) + l0.w) + l1.x) + l1.y) + l1.z) + l1.w;
            sVc[k * kMuRow + dim] = num / den;
        }
        __syncthreads();

        // ------------- local window branch + gather + fusion (wave w: query tile w)
        if (w < NT) {
            const int qi = tok;
            const int r = radius < L ? radius : L;
            f32x4_t o[4], o2[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = o2[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            float lsum;
            if (NARROW) {
                // radius <= 16: the tile's keys lie in tiles w-1, w, w+1
                const int kt0 = w > 0 ? w - 1 : 0;
                const int kt2 = w + 1 < NT ? w + 1 : NT - 1;
                const int ntile = kt2 - kt0 + 1;          // 1, 2 or 3
                float sc[3][4];
                float m = -__builtin_inff();
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    const int kt = kt0 + q;
                    if (q < ntile) {
                        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
                        a0 = mma32x6(k_frag(sK, kt, 0, l16, g), qf[0], a0);
                        a1 = mma32x6(k_frag(sK, kt, 1, l16, g), qf[1], a1);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int key = 16 * kt + 4 * g + rr;
                            const int dist = key > qi ? key - qi : qi - key;
                            const bool in = (FULL || key < L) && dist <= r;
                            sc[q][rr] = in ? (a0[rr] + a1[rr]) * scale : -__builtin_inff();
                            m = fmaxf(m, sc[q][rr]);
                        }
                    } else {
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) sc[q][rr] = -__builtin_inff();
                    }
                }
                m = col_max(m);
                float ls = 0.f;
#pragma unroll
                for (int q = 0; q < 3; ++q) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const float pp = sc[q][rr] == -__builtin_inff() ? 0.f : exp_f32(sc[q][rr] - m);
                        sc[q][rr] = pp;
                        ls += pp;
                    }
                }
                lsum = col_sum(ls);
                {   // tiles (kt0, kt0+1); the second may not exist (then p = 0)
                    const float pv[8] = {sc[0][0], sc[0][1], sc[0][2], sc[0][3],
                                         sc[1][0], sc[1][1], sc[1][2], sc[1][3]};
                    const Split8 pf = split8(pv);
                    const int kb = ntile > 1 ? kt0 + 1 : kt0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = mma32x6(v_frag_two(sV, j, kt0, kb, l16, g), pf, o[j]);
                }
                if (ntile == 3) {   // tile kt0+2 with an empty partner (p = 0)
                    const float pv[8] = {sc[2][0], sc[2][1], sc[2][2], sc[2][3], 0.f, 0.f, 0.f, 0.f};
                    const Split8 pf = split8(pv);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        o2[j] = mma32x6(v_frag_two(sV, j, kt0 + 2, kt0 + 2, l16, g), pf, o2[j]);
                }
            } else {
                const int lo_key = 16 * w - r;                 // window of the whole tile
                const int hi_key = 16 * w + 15 + r;
                const int kt_lo = lo_key < 0 ? 0 : (lo_key >> 4);
                const int kt_hi = (hi_key >> 4) < NT - 1 ? (hi_key >> 4) : NT - 1;
                float sc[8][4];
                float m = -__builtin_inff();
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) {
                    if (kt >= kt_lo && kt <= kt_hi) {
                        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
                        a0 = mma32x6(k_frag(sK, kt, 0, l16, g), qf[0], a0);
                        a1 = mma32x6(k_frag(sK, kt, 1, l16, g), qf[1], a1);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int key = 16 * kt + 4 * g + rr;
                            const int dist = key > qi ? key - qi : qi - key;
                            const bool in = (FULL || key < L) && dist <= r;
                            sc[kt][rr] = in ? (a0[rr] + a1[rr]) * scale : -__builtin_inff();
                            m = fmaxf(m, sc[kt][rr]);
                        }
                    } else {
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) sc[kt][rr] = -__builtin_inff();
                    }
                }
                m = col_max(m);
                float ls = 0.f;
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const float pp = sc[kt][rr] == -__builtin_inff() ? 0.f : exp_f32(sc[kt][rr] - m);
                        sc[kt][rr] = pp;
                        ls += pp;
                    }
                }
                lsum = col_sum(ls);
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    if (2 * ch + 1 >= kt_lo && 2 * ch <= kt_hi) {
                        const float pv[8] = {sc[2 * ch][0], sc[2 * ch][1], sc[2 * ch][2],
                                             sc[2 * ch][3], sc[2 * ch + 1][0], sc[2 * ch + 1][1],
                                             sc[2 * ch + 1][2], sc[2 * ch + 1][3]};
                        const Split8 pf = split8(pv);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            if (ch & 1)
                                o2[j] = mma32x6(v_frag_two(sV, j, 2 * ch, 2 * ch + 1, l16, g), pf, o2[j]);
                            else
                                o[j] = mma32x6(v_frag_two(sV, j, 2 * ch, 2 * ch + 1, l16, g), pf, o[j]);
                        }
                    }
                }
            }
            // o + o2 = sum p v[dim 16j + 4g + rr] for query qi
            if (FULL || qi < L) {
                const float inv = 1.0f / lsum;
                const int cq = sC[qi];
                const float wg = 1.0f - alpha;
                const float *vc = sVc + cq * kMuRow;
                T *dst = out + slice * (long)L * kD + (long)qi * kD;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = 16 * j + 4 * g;
                    const f32x4_t ol = add4(o[j], o2[j]);
                    float4 v;
                    v.x = wg * vc[d0 + 0] + alpha * (ol[0] * inv);
                    v.y = wg * vc[d0 + 1] + alpha * (ol[1] * inv);
                    v.z = wg * vc[d0 + 2] + alpha * (ol[2] * inv);
                    v.w = wg * vc[d0 + 3] + alpha * (ol[3] * inv);
                    store4<T>(dst + d0, v);
                }
            }
        }
        if (assign_out) {
            for (int i = tid; i < L; i += kThreads) assign_out[slice * L + i] = sC[i];
        }
    }
}

bool fused_supported(int L, int Kc) { return L >= 1 && L <= kFL && Kc >= 1 && Kc <= kFK; }

template <typename T, bool FULL, bool NARROW>
static hipError_t fused_launch_t(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                                 int iters, int radius, float alpha, void *out, int32_t *assign,
                                 hipStream_t st) {
    auto kern = cluster_attn_fused_kernel<T, FULL, NARROW>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsTotal);
    if (e != hipSuccess) return e;
    // one workgroup per slice (the LDS footprint admits one per CU)
    const int grid = S;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), kLdsTotal, st,
                       static_cast<const T *>(Q), static_cast<const T *>(K),
                       static_cast<const T *>(V), S, L, Kc, iters, radius, alpha,
                       static_cast<T *>(out), assign);
    return hipGetLastError();
}

template <typename T>
static hipError_t fused_launch(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                               int iters, int W, float alpha, void *out, int32_t *assign,
                               hipStream_t st) {
    const int radius = W / 2;
    const bool full = L == kFL;
    const bool narrow = radius <= 16;
    if (full && narrow)
        return fused_launch_t<T, true, true>(Q, K, V, S, L, Kc, iters, radius, alpha, out, assign, st);
    if (full)
        return fused_launch_t<T, true, false>(Q, K, V, S, L, Kc, iters, radius, alpha, out, assign, st);
    if (narrow)
        return fused_launch_t<T, false, true>(Q, K, V, S, L, Kc, iters, radius, alpha, out, assign, st);
    return fused_launch_t<T, false, false>(Q, K, V, S, L, Kc, iters, radius, alpha, out, assign, st);
}

hipError_t launch_fused_forward(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                                int iters, int W, float alpha, ca_dtype_t dt, void *out,
                                int32_t *assign, hipStream_t st) {
    if (dt == CA_BF16)
        return fused_launch<bf16_t>(Q, K, V, S, L, Kc, iters, W, alpha, out, assign, st);
    return fused_launch<float>(Q, K, V, S, L, Kc, iters, W, alpha, out, assign, st);
}

}  // namespace ca
