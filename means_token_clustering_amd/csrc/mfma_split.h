// Single-slice building blocks on the fp16 matrix cores (gfx950), shared by
// the single-launch kernels (forward, exact attention, backward): the fp16
// h/m split of fp32 values, the three-product MFMA chains, cross-lane column
// reductions, power-of-two range scaling, XOR-swizzled fp16 planes of a
// [128][64] slice with their fragment readers (rows and ds_read_b64_tr_b16
// transposes), the key-padding bit masks and the two local-window routines.
// The arithmetic and the lane layouts are described where the forward kernel
// (fused.hip) starts.
#pragma once

#include "common.h"

namespace ca {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kFL = 128;              // max tokens
constexpr int kFK = 16;               // max clusters
constexpr int kThreads = 512;         // 8 waves
constexpr int kQLimit = 5;            // scaled |q| < 2^5 keeps 16 q^2 in fp16 range
constexpr int kKVLimit = 15;          // scaled |k|, |v| < 2^15

// fp16 plane sizes of one slice (bytes, elements)
constexpr int kPlane = kFL * kD * 2;          // one fp16 plane [128][64]
constexpr int kPlaneE = kPlane / 2;           // ... in elements
constexpr int kPlaneMu = kFK * kD * 2;        // one fp16 plane [16][64]
constexpr int kPlaneMuE = kPlaneMu / 2;
constexpr int kPlaneRow = kFK * kFL * 2;      // one fp16 plane [16][128] (one-hot, P)
constexpr int kPlaneRowE = kPlaneRow / 2;

constexpr uint32_t kOneH2 = 0x3c003c00u;      // two fp16 1.0
constexpr uint16_t kNegInfH = 0xfc00u;        // fp16 -inf

struct Sp8 {  // 8 values as two fp16 planes (pairs packed low-first)
    u32x4_t h, m;
};
struct Sp4 {  // 4 values as two fp16 planes
    u32x2_t h, m;
};

// x0, x1 -> packed fp16 pairs h and m with x = h + m + e: h rounded toward
// zero, m = x - h (exact inside the mixed-precision fma) rounded to nearest
// into the low / high half of m.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &h, uint32_t &m) {
    h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x0));
    asm("v_fma_mixhi_f16 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "+v"(r) : "v"(h), "v"(x1));
    m = r;
}

// A matrix instruction that reads a vector-ALU result from registers needs
// wait states after the write; the compiler inserts them only after writes it
// can see, not after asm. mfma_ready passes a whole split group through one
// asm that names every register of the group as an in-out operand and holds
// s_nop 4 (five wait states): data dependence places it after the last write
// of any part of the group and every matrix read after it, and any copy the
// compiler makes afterwards is a visible vector-ALU write that it guards
// itself. Only groups that reach a matrix instruction from registers need it;
// groups stored to LDS are read back by LDS loads.
__device__ __forceinline__ void mfma_ready(u32x4_t &h, u32x4_t &m) {
    asm("s_nop 4" : "+v"(h), "+v"(m));
}
__device__ __forceinline__ void mfma_ready(u32x2_t &h, u32x2_t &m) {
    asm("s_nop 4" : "+v"(h), "+v"(m));
}

// MFMA = true: the group feeds matrix instructions from registers (mfma_ready).
template <bool MFMA = false>
__device__ __forceinline__ Sp8 split8(const float *x) {
    uint32_t h[4], m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(x[2 * i], x[2 * i + 1], h[i], m[i]);
    Sp8 r{u32x4_t{h[0], h[1], h[2], h[3]}, u32x4_t{m[0], m[1], m[2], m[3]}};
    if (MFMA) mfma_ready(r.h, r.m);
    return r;
}
template <bool MFMA = false>
__device__ __forceinline__ Sp4 split4(float x0, float x1, float x2, float x3) {
    uint32_t h0, m0, h1, m1;
    split2(x0, x1, h0, m0);
    split2(x2, x3, h1, m1);
    Sp4 r{u32x2_t{h0, h1}, u32x2_t{m0, m1}};
    if (MFMA) mfma_ready(r.h, r.m);
    return r;
}

// fp16 value i (0..3) of a packed pair of pairs, widened
__device__ __forceinline__ float half_at(u32x2_t p, int i) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p[i >> 1] >> (16 * (i & 1))));
}

__device__ __forceinline__ f32x4_t mma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
// c += a . b from the three leading partial products (smallest first)
__device__ __forceinline__ f32x4_t mma3(const Sp8 &a, const Sp8 &b, f32x4_t c) {
    c = mma(a.m, b.h, c);
    c = mma(a.h, b.m, c);
    return mma(a.h, b.h, c);
}
// The same with the products of a's (ZA) or b's (ZB) m plane left out, for
// operands split from bf16 storage. A bf16 value carries 8 significant bits,
// so once scaled by a power of two into fp16's normal range it is an fp16
// value: its h part is exact and its m part zero, and the left-out products
// would add exact zeros (same result, same order of the remaining ones). Only
// values that scale below fp16's smallest normal (2^-14; the scaled maxima
// lie in [2^4, 2^15)) lose m parts below the subnormal step 2^-24.
template <bool ZA, bool ZB>
__device__ __forceinline__ f32x4_t mma3z(const Sp8 &a, const Sp8 &b, f32x4_t c) {
    if (!ZA) c = mma(a.m, b.h, c);
    if (!ZB) c = mma(a.h, b.m, c);
    return mma(a.h, b.h, c);
}
// whether a storage type is bf16 (its split planes have zero m parts)
template <typename T>
constexpr bool bf16_storage() { return sizeof(T) == 2; }
// the same on 16-deep operands (v_mfma_f32_16x16x16_f16: lane l holds
// A[l%16][4(l/16)+i] and B[4(l/16)+i][l%16], i = 0..3; D as for 16x16x32)
__device__ __forceinline__ f32x4_t mma16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma3_16(const Sp4 &a, const Sp4 &b, f32x4_t c) {
    c = mma16(a.m, b.h, c);
    c = mma16(a.h, b.m, c);
    return mma16(a.h, b.h, c);
}

constexpr f32x4_t kZero4 = {0.f, 0.f, 0.f, 0.f};

// ---- cross-lane helpers (no LDS traffic)
// lanes l and l^32 (resp. l^16) both receive (lower lane value, upper lane value)
__device__ __forceinline__ void pair32(uint32_t v, uint32_t &lo, uint32_t &hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    lo = r[0];
    hi = r[1];
}
__device__ __forceinline__ void pair16(uint32_t v, uint32_t &lo, uint32_t &hi) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    lo = r[0];
    hi = r[1];
}
// sum / max over the four lane groups g of a column; every lane of the
// column gets the same bits
__device__ __forceinline__ float col_sum(float v) {
    uint32_t a, b;
    pair16(__float_as_uint(v), a, b);
    v = __uint_as_float(a) + __uint_as_float(b);
    pair32(__float_as_uint(v), a, b);
    return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float col_max(float v) {
    uint32_t a, b;
    pair16(__float_as_uint(v), a, b);
    v = fmaxf(__uint_as_float(a), __uint_as_float(b));
    pair32(__float_as_uint(v), a, b);
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
// (score, index) maximum over the four lane groups of a column. Lane group g
// holds indices 4g .. 4g+3, so taking the upper half only when it is strictly
// larger keeps the lowest index among equal scores.
__device__ __forceinline__ int col_argmax(float best, int bk) {
    uint32_t a, b, ia, ib;
    pair16(__float_as_uint(best), a, b);
    pair16((uint32_t)bk, ia, ib);
    bool up = __uint_as_float(b) > __uint_as_float(a);
    best = up ? __uint_as_float(b) : __uint_as_float(a);
    bk = up ? (int)ib : (int)ia;
    pair32(__float_as_uint(best), a, b);
    pair32((uint32_t)bk, ia, ib);
    up = __uint_as_float(b) > __uint_as_float(a);
    return up ? (int)ib : (int)ia;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
    v = max(v, dpp_u<0xB1>(v));    // quad_perm [1,0,3,2]
    v = max(v, dpp_u<0x4E>(v));    // quad_perm [2,3,0,1]
    v = max(v, dpp_u<0x124>(v));   // row_ror:4
    v = max(v, dpp_u<0x128>(v));   // row_ror:8
    uint32_t a, b;
    pair16(v, a, b);
    v = max(a, b);
    pair32(v, a, b);
    return max(a, b);
}

// ---- storage access
template <typename T>
__device__ __forceinline__ void load8(const T *p, float *x) {
    const float4 a = load4<T>(p), b = load4<T>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// 8 consecutive elements of row `row` (zeros when row >= L). For bf16 storage
// the zeros are selects: a branch around them makes the compiler wait for each
// 16-byte load before it issues the next one (measured: the 512-token single
// launch 37.3 against 40.2 us at 192 slices). For fp32 the branch stays (the
// selects measured slower in the long-slice staged kernels: 148.0 against
// 140.5 us).
template <typename T, bool FULL>
__device__ __forceinline__ void load_row8(const T *base, int row, int L, int col, float *x) {
    if (FULL) {
        load8<T>(base + (long)row * kD + col, x);
    } else if (sizeof(T) == 2) {
        const bool in = row < L;
        load8<T>(base + (long)(in ? row : L - 1) * kD + col, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = in ? x[i] : 0.f;
    } else {
        const int rc = row < L ? row : L - 1;
        load8<T>(base + (long)rc * kD + col, x);
        if (row >= L) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
    }
}
__device__ __forceinline__ float absmax8(const float *x, float m) {
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
    return m;
}
// Power-of-two shift s for a tensor whose largest magnitude has bits
// `maxbits`: 0 when that maximum lies in [2^-3, 2^limit), where the fp16 split
// keeps every element above 2^-14 to 2^-20 relative and the rest to 2^-21 of
// the maximum; otherwise s brings the maximum into [2^(limit-1), 2^limit)
// (at most 2^100 up). Zero or subnormal maxima need no scaling.
__device__ __forceinline__ int scale_shift(uint32_t maxbits, int limit) {
    if (maxbits < 0x00800000u) return 0;
    const int e = (int)(maxbits >> 23) - 127;   // 2^e <= max < 2^(e+1)
    if (e >= -3 && e < limit) return 0;
    const int s = e + 1 - limit;
    return s < -100 ? -100 : s;
}

// ---- swizzled fp16 planes (element offsets). 64-wide rows: 8 chunks of 8
// elements, chunk index XOR (row & 7); 128-wide rows: 16 chunks, XOR (row & 15).
__device__ __forceinline__ int off64(int row, int col) {
    return row * 64 + ((((col >> 3) ^ (row & 7))) << 3) + (col & 7);
}
__device__ __forceinline__ int off128(int row, int col) {
    return row * 128 + ((((col >> 3) ^ (row & 15))) << 3) + (col & 7);
}
__device__ __forceinline__ u32x4_t ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4_t *>(p); }
__device__ __forceinline__ void st16(uint16_t *p, u32x4_t v) { *reinterpret_cast<u32x4_t *>(p) = v; }
__device__ __forceinline__ void st8(uint16_t *p, u32x2_t v) { *reinterpret_cast<u32x2_t *>(p) = v; }

// Per-lane parts of the swizzled plane offsets, in bytes, so that every
// fragment read is one XOR (or none) plus an immediate offset (element
// offsets above, times two):
//   off64(R + l16, 32c + 8g)            -> 128 R + (rl64 ^ 64c)        (R % 16 == 0)
//   off128(l16, 32c + 8g)               -> rl128 ^ 64c
//   off64(B + l16/4, 16j + 4(l16%4))    -> 128 (B & ~7) + (tr(B & 4) ^ 32j)
struct LaneOffs {
    int rl64, rl128, tr0, tr4;
};
__device__ __forceinline__ LaneOffs lane_offsets(int l16, int g) {
    LaneOffs o;
    o.rl64 = 2 * (l16 * 64 + 8 * (g ^ (l16 & 3)) + 32 * ((l16 >> 2) & 1));
    o.rl128 = 2 * (l16 * 128 + 32 * (l16 >> 2) + 8 * (g ^ (l16 & 3)));
    const int b = (l16 >> 1) & 1;
    int sw = l16 >> 2;   // row & 7 for B % 8 == 0
    o.tr0 = 2 * ((l16 >> 2) * 64 + 8 * (b ^ (sw & 1)) + 4 * (l16 & 1) + 16 * ((sw >> 1) & 3));
    sw += 4;             // B % 8 == 4
    o.tr4 = 2 * (256 + (l16 >> 2) * 64 + 8 * (b ^ (sw & 1)) + 4 * (l16 & 1) + 16 * ((sw >> 1) & 3));
    return o;
}
typedef unsigned char u8;
__device__ __forceinline__ u32x4_t ldb16(const u8 *base, int off) {
    return *reinterpret_cast<const u32x4_t *>(base + off);
}
// 16-byte row fragment of a plane pair (planes `plane` bytes apart) at byte offset off
__device__ __forceinline__ Sp8 frag_at(const u8 *base, int plane, int off) {
    return Sp8{ldb16(base, off), ldb16(base, off + plane)};
}
// transposed 4-deep read (ds_read_b64_tr_b16) at byte offset off: with off
// from the tr(.) form above, lane l16 receives rows B .. B+3 of column
// 16j + l16
__device__ __forceinline__ u32x2_t tr_at(const u8 *base, int off) {
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)((__attribute__((address_space(3))) u8 *)(base + off)));
    return __builtin_bit_cast(u32x2_t, v);
}
// 8-deep transposed fragment of a [rows][64] plane pair (planes PLANE bytes
// apart; [128][64] by default) from two row groups
template <int PLANE = kPlane>
__device__ __forceinline__ Sp8 colfrag8_at(const u8 *base, int o0, int o1) {
    const u32x2_t h0 = tr_at(base, o0), h1 = tr_at(base, o1);
    const u32x2_t m0 = tr_at(base, o0 + PLANE), m1 = tr_at(base, o1 + PLANE);
    return Sp8{u32x4_t{h0[0], h0[1], h1[0], h1[1]}, u32x4_t{m0[0], m0[1], m1[0], m1[1]}};
}

// Key-padding mask of a slice, one bit per token (bit t of word t / 32); all
// bits set when the launch has no mask. A padded key's logit is -10000 in
// natural units (ClusterAttention listing on the "Hooshaai/svd-sst2-roberta-
// cluster" page, forward, bidirectional branch), -10000 log2(e) in the base-2
// units used here.
struct KeyBits {
    uint32_t w[4];
    // the 16 bits of key tile t (t uniform over the wave)
    __device__ __forceinline__ uint32_t tile(int t) const {
        const int k = t >> 1;
        const uint32_t x = k == 0 ? w[0] : (k == 1 ? w[1] : (k == 2 ? w[2] : w[3]));
        return (x >> (16 * (t & 1))) & 0xffffu;
    }
};
constexpr float kPadLogit2 = -14426.950408889634f;

// The same for up to 160 keys (a 128-query block with a 16-key halo on each
// side), keys counted from the first staged row.
struct KeyBits160 {
    uint32_t w[5];
    __device__ __forceinline__ uint32_t tile(int t) const {
        const int k = t >> 1;
        const uint32_t x =
            k == 0 ? w[0] : (k == 1 ? w[1] : (k == 2 ? w[2] : (k == 3 ? w[3] : w[4])));
        return (x >> (16 * (t & 1))) & 0xffffu;
    }
};

// Local window of radius <= 16 for query tile qt: scores against key tiles
// qt-1, qt, qt+1 (others are outside every window of the tile), base-2
// softmax, then O^T = V^T P^T: the pair (qt-1, qt) as one 32-deep product and
// tile qt+1 as a 16-deep one. Tiles outside [0, NT) get probability 0; their
// K and V reads are moved onto tile qt (finite values times zero). Every LDS
// read of a stage is issued before its first product, and the products of
// independent tiles alternate, so that neither the LDS latency nor the
// matrix-core latency is exposed per product. PLANE: byte distance of the
// h and m planes (rows of the planes: NT tiles of 16, L valid; KB: the key
// mask of those rows). Z: Q, K and V come from bf16 storage (mma3z).
template <bool FULL, bool MASKED, typename KB = KeyBits, int PLANE = kPlane, bool Z = false>
__device__ __forceinline__ void local_narrow(const u8 *pK, const u8 *pV, const Sp8 *qf,
                                             int qt, int NT, int L, int rad, float sscale2,
                                             int l16, int g, int rl64, int trv, const KB &kb,
                                             f32x4_t *o, float &lsum) {
    bool valid[3];
    Sp8 kfr[3][2];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const int kt = qt + d - 1;
        valid[d] = kt >= 0 && kt < NT;
        const int kb = 2048 * (valid[d] ? kt : qt);
#pragma unroll
        for (int c = 0; c < 2; ++c) kfr[d][c] = frag_at(pK, PLANE, kb + (rl64 ^ (64 * c)));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t sc[3] = {kZero4, kZero4, kZero4};
#pragma unroll
    for (int c = 0; c < 2; ++c) {   // the three mma3 chains, interleaved
        if (!Z) {
#pragma unroll
            for (int d = 0; d < 3; ++d) sc[d] = mma(kfr[d][c].m, qf[c].h, sc[d]);
#pragma unroll
            for (int d = 0; d < 3; ++d) sc[d] = mma(kfr[d][c].h, qf[c].m, sc[d]);
        }
#pragma unroll
        for (int d = 0; d < 3; ++d) sc[d] = mma(kfr[d][c].h, qf[c].h, sc[d]);
    }
    float s[3][4];
    float m = -__builtin_inff();
    // key - query = 16 (d - 1) + rel0 + rr for key tile qt + d - 1; tile qt-1
    // is in the window where key - query >= -rad, tile qt+1 where it is <= rad,
    // and all of tile qt once rad >= 15
    const int rel0 = 4 * g - l16;
    const int lo0 = rel0 - 16 + rad, hi2 = rel0 + 16 - rad;
    const bool whole1 = rad >= 15;
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const int kt = qt + d - 1;
        const uint32_t nib = MASKED ? kb.tile(valid[d] ? kt : qt) >> (4 * g) : 0xfu;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {   // sc[d][rr] = k_{16kt+4g+rr} . q_{16qt+l16}
            bool in;
            if (d == 0) in = valid[0] && lo0 >= -rr;
            else if (d == 2) in = valid[2] && hi2 <= -rr;
            else in = whole1 || (rel0 + rr <= rad && -(rel0 + rr) <= rad);
            if (!FULL) in = in && 16 * kt + 4 * g + rr < L;
            const float sv = (!MASKED || ((nib >> rr) & 1u)) ? sc[d][rr] * sscale2 : kPadLogit2;
            s[d][rr] = in ? sv : -__builtin_inff();
            m = fmaxf(m, s[d][rr]);
        }
    }
    m = col_max(m);   // finite: every query sees itself
#pragma unroll
    for (int d = 0; d < 3; ++d)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) s[d][rr] = __builtin_amdgcn_exp2f(s[d][rr] - m);   // exp2(-inf) = 0
    float ls = s[0][0];
#pragma unroll
    for (int e = 1; e < 12; ++e) ls += s[e >> 2][e & 3];
    lsum = col_sum(ls);
    const float pa[8] = {s[0][0], s[0][1], s[0][2], s[0][3], s[1][0], s[1][1], s[1][2], s[1][3]};
    const Sp8 pA = split8<true>(pa);
    const float pb[8] = {s[2][0], s[2][1], s[2][2], s[2][3], 0.f, 0.f, 0.f, 0.f};
    const Sp8 pB = split8<true>(pb);
    // V^T rows 16kt + 4g .. +3 of columns 16j + l16 start at byte 2048 kt + (trv ^ 32j);
    // the zero-weight half of the second product reads a fourth tile (any
    // finite values do; a distinct tile avoids register copies)
    const int b1 = 2048 * qt + trv;
    const int b0 = valid[0] ? b1 - 2048 : b1;
    const int b2 = valid[2] ? b1 + 2048 : b1;
    const int b3 = qt + 2 < NT ? b1 + 4096 : (qt >= 2 ? b1 - 4096 : b1);
    // two column tiles j per stage: 16 transposed reads, then 12 products
#pragma unroll
    for (int jj = 0; jj < 4; jj += 2) {
        Sp8 va[2], vb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int j = jj + u;
            va[u] = colfrag8_at<PLANE>(pV, b0 ^ (32 * j), b1 ^ (32 * j));
            vb[u] = colfrag8_at<PLANE>(pV, b2 ^ (32 * j), b3 ^ (32 * j));
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t acc[2] = {kZero4, kZero4};
        if (!Z) {
#pragma unroll
            for (int u = 0; u < 2; ++u) acc[u] = mma(va[u].m, pA.h, acc[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[u] = mma(va[u].h, pA.m, acc[u]);
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[u] = mma(va[u].h, pA.h, acc[u]);
        if (!Z) {
#pragma unroll
            for (int u = 0; u < 2; ++u) acc[u] = mma(vb[u].m, pB.h, acc[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[u] = mma(vb[u].h, pB.m, acc[u]);
#pragma unroll
        for (int u = 0; u < 2; ++u) o[jj + u] = mma(vb[u].h, pB.h, acc[u]);
    }
}

// Local window of any radius: key tiles in [qt - ceil(r/16), qt + ceil(r/16)]
// two at a time with a running maximum (online softmax) and 32-deep P V
// products; a missing second tile gets zero weights on repeated V rows.
// CAUSAL: the window is keys 0 .. qi instead (rad unused). mfinal (if not
// null) receives the final running maximum of the column's base-2 logits.
// Z: Q, K and V come from bf16 storage (mma3z).
template <bool FULL, bool MASKED, bool CAUSAL = false, bool Z = false>
__device__ __forceinline__ void local_wide(const u8 *pK, const u8 *pV, const Sp8 *qf,
                                           int qt, int NT, int L, int rad, float sscale2,
                                           int l16, int g, int rl64, int trv, const KeyBits &kb,
                                           f32x4_t *o, float &lsum, float *mfinal = nullptr) {
    const int qi = 16 * qt + l16;
    const int lo_key = CAUSAL ? 0 : 16 * qt - rad, hi_key = CAUSAL ? 16 * qt + 15 : 16 * qt + 15 + rad;
    const int kt_lo = lo_key < 0 ? 0 : (lo_key >> 4);
    const int kt_hi = (hi_key >> 4) < NT - 1 ? (hi_key >> 4) : NT - 1;
    float M = -__builtin_inff(), ls = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = kZero4;
    for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
        const bool two = kt + 1 <= kt_hi;
        float s[8];
        float mt = -__builtin_inff();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ktt = two ? kt + h : kt;
            f32x4_t a = mma3z<Z, Z>(frag_at(pK, kPlane, 2048 * ktt + rl64), qf[0], kZero4);
            a = mma3z<Z, Z>(frag_at(pK, kPlane, 2048 * ktt + (rl64 ^ 64)), qf[1], a);
            const uint32_t nib = MASKED ? kb.tile(ktt) >> (4 * g) : 0xfu;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = 16 * ktt + 4 * g + rr;
                const int dist = key > qi ? key - qi : qi - key;
                const bool in = (FULL || key < L) && (CAUSAL ? key <= qi : dist <= rad) &&
                                (h == 0 || two);
                const float sv = (!MASKED || ((nib >> rr) & 1u)) ? a[rr] * sscale2 : kPadLogit2;
                s[4 * h + rr] = in ? sv : -__builtin_inff();
                mt = fmaxf(mt, s[4 * h + rr]);
            }
        }
        mt = col_max(mt);
        const float Mn = fmaxf(M, mt);
        const float Ms = Mn == -__builtin_inff() ? 0.f : Mn;   // nothing seen yet
        const float f = __builtin_amdgcn_exp2f(M - Ms);
        M = Mn;
        ls *= f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] = __builtin_amdgcn_exp2f(s[i] - Ms);
            ls += s[i];
        }
        const Sp8 p = split8<true>(s);
        const int b0 = 2048 * kt + trv, b1 = two ? b0 + 2048 : b0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = mma3z<Z, false>(colfrag8_at(pV, b0 ^ (32 * j), b1 ^ (32 * j)), p, o[j] * f);
    }
    lsum = col_sum(ls);
    if (mfinal) *mfinal = M;
}

}  // namespace
}  // namespace ca
