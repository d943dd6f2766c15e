// bf16 projection GEMMs of the full attention layer (model card
// "Hooshaai/distilbert-sst2-cluster-attention", Architecture Overview: the
// multi-head projections of X and the output projection Y = O W_O;
// "ClusterFormer" spec on the "Hooshaai/svd-sst2-roberta-cluster" page,
// section 3, first and last rows of the tensor trace).
//
// C = A . B on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulation, one round-to-nearest-even at the store). The weight operand
// comes in either layout, chosen at compile time:
//   KN : W [K, N] row-major, the [in, out] layout of the layer's weights. Its
//        tile is kept in LDS as stored ([k][n]) and the matrix-core operand is
//        read with ds_read_b64_tr_b16, which hands each lane 4 consecutive k
//        of one column n; no transposed copy of W is ever made.
//   BT : Bt [N, K] row-major (C = A . Bt^T), read with plain 16-byte rows.
// Up to four weights of the same shape (Q, K and V) form one launch as the
// column blocks of one [K, count * N] product. A rows are plain row-major
// [M, K] or the heads of a [B, H, L, 64] tensor merged on the fly (row b*L + l,
// column 64 h + j); C rows are plain [M, N] or split into heads on the fly
// ([B, H, L, 64], head h = columns 64 h ..).
//
// Work split. Each wave owns a 64 x 96 block of C (4 x 6 matrix-core blocks
// of 16 x 16, 96 accumulator registers); a workgroup of WM x WN waves owns a
// (64 WM) x (96 WN) tile. Two shapes:
//   4 x 3 waves, 256 x 288 tiles, one workgroup per CU, 3 stages:
//     [8192 x 768] x [768 x 2304] is 256 tiles, one per CU, and each CU takes
//     in 544 rows of operands per k instead of the 960 of three 128 x 192
//     tiles (operand delivery into a CU runs at 64 B per clock).
//   2 x 2 waves, 128 x 192 tiles, 2 stages, three workgroups per CU (other
//     shapes); with at most one tile per CU (the output projection
//     [8192 x 768] x [768 x 768]) two k groups of 2 x 2 waves, each taking
//     every other 32-deep k step, their sums added in LDS at the end: 17.4
//     against 18.6 us with one group (three groups 17.8, three stages 19.3).
// Measured on [8192 x 768] x [768 x 2304] (same box, A rotating past the
// caches): 34.9 us for the 256 x 288 tiles, 35.9 us for 128 x 192 tiles with
// three workgroups per CU, 38-46 us with 2 workgroups per CU or 128 x 288
// tiles, 38.9 us with 32 x 32 x 16 blocks; the library GEMM behind torch's
// matmul took 41.9-44.9 us on the same product.
// The tiles of a 32-deep k step go from global memory straight into LDS
// (global_load_lds_dwordx4: no registers, no LDS store instructions), a ring
// of S stages (S - 1 steps ahead). The matrix core computes the transposed
// product (weight rows first), so each lane ends with 4 consecutive output
// columns per block; each wave's block leaves through LDS so that every
// global store writes 16 bytes of a row. Tile numbers are spread so that the
// workgroups on one XCD (workgroup id mod 8) share rows of A.
//
// LDS layouts (bank-conflict free for the reads below):
//   A and Bt tiles: rows of 32 bf16 (4 chunks of 16 B), chunk c of row r at
//     chunk c ^ ((r >> 1) & 3).
//   W tile ([32 k][96 WN n]): rows of 192 WN bytes; the 8-byte unit u of row
//     r at unit u ^ 4 (r & 3) when the row length is a multiple of 128 B
//     (WN even), u ^ 4 ((r >> 1) & 1) when it is an odd multiple of 64 B
//     (16-byte chunks stay whole). A transposed read has lane 4e + q of each
//     16-lane group at row r0 + e, columns c0 + 4q .. c0 + 4q + 3.
//   Output staging: 64 rows of 200 B per wave (96 bf16 + 8 B pad).
#include "launch.h"

namespace ca {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 32;                  // k step of one LDS stage
constexpr int kWaveM = 64, kWaveN = 96;  // C block of one wave
constexpr int kWRow = 2 * kWaveN + 8;    // bytes per staged output row of a wave

struct GemmArgs {
    const uint16_t *A;
    const uint16_t *B[4];   // per weight z: W [K, N] (KN) or Bt [N, K] (BT)
    uint16_t *C[4];
    int M, N, K;            // N: columns of one weight
    int count;              // weights
    int L, H;               // head geometry of the merged / split modes
    int tiles_m, tiles_n;   // tiles_n over all count * N columns
};

// Shape of one launch: WM x WN waves per k group, KS k groups, S stages. With
// KS > 1 a stage holds KS consecutive 32-deep k tiles and wave group g
// multiplies tile g of each stage; the groups' sums meet in LDS at the end,
// folded from the last group down (group 0 ends with g0 + (g1 + (g2 ..))).
template <int WM, int WN, int S, int KS>
struct Cfg {
    static constexpr int kWavesT = WM * WN;                  // waves per k group
    static constexpr int kWaves = kWavesT * KS, kThreads = 64 * kWaves;
    static constexpr int kTM = kWaveM * WM, kTN = kWaveN * WN;
    static constexpr int kATile = kTM * kBK, kBTile = kTN * kBK;   // elements
    static constexpr int kTile1 = kATile + kBTile;           // one k tile
    static constexpr int kStage = KS * kTile1;
    static constexpr int kAInst = kATile * 2 / 1024;   // 1 KB direct loads per k tile
    static constexpr int kInst1 = kTile1 * 2 / 1024;
    static constexpr int kInst = KS * kInst1;
    static constexpr int kMaxPerWave = (kInst + kWaves - 1) / kWaves;
    static constexpr int kCpr = kTN / 8;                // 16-byte chunks of a W tile row
    static constexpr int kStgElems = kWavesT * 64 * kWRow / 2;
    static constexpr int kRedElems = KS > 1 ? kWavesT * 64 * 96 * 2 : 0;   // fp32 sums of a group
    static constexpr int kLdsElems =
        S * kStage > kStgElems ? (S * kStage > kRedElems ? S * kStage : kRedElems)
                               : (kStgElems > kRedElems ? kStgElems : kRedElems);
    static_assert(kATile * 2 % 1024 == 0 && kTile1 * 2 % 1024 == 0, "whole 1 KB loads");
    static_assert(kLdsElems * 2 <= 160 * 1024, "LDS");
    static_assert((S - 2) * kMaxPerWave <= 12, "wait counts");
};

// element offset of 16-byte chunk c (0..3) of row r of a [rows][32] tile
__device__ __forceinline__ int swz(int r, int c) { return r * kBK + ((c ^ ((r >> 1) & 3)) << 3); }
// XOR applied to the 8-byte unit index of row r of the W tile
template <int WN>
__device__ __forceinline__ int wx(int r) { return WN % 2 == 0 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

__device__ __forceinline__ u32x2_t tr_read(const uint16_t *base, int byte) {
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)((__attribute__((address_space(3))) unsigned char *)(
            reinterpret_cast<const unsigned char *>(base) + byte)));
    return __builtin_bit_cast(u32x2_t, v);
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes bytes 16 l .. 16 l + 15 after the wave-uniform LDS byte address
// lds. Written as inline assembly so that the compiler, which does not see
// these writes, adds no waits of its own before the LDS reads of the other
// stages; the kernel waits for them explicitly (s_waitcnt vmcnt). M0 carries
// the LDS address; nothing else in the kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const uint16_t *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(lds), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n) for a wave-uniform n <= 12
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
        case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    }
}

// Workgroup barrier without a memory fence: every wave has already waited
// for what the barrier publishes (its direct loads of the stage, its LDS
// reads of the previous tile).
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }

// waves per SIMD the register budget has to allow
template <int WM, int WN, int S, int KS>
constexpr int occupancy() { return KS > 1 ? 2 : (WM * WN >= 12 ? 3 : (S == 2 ? 3 : 2)); }

template <int WM, int WN, int S, int KS, bool AHEADS, bool CHEADS, bool KN>
__global__ __launch_bounds__((64 * WM * WN * KS), (occupancy<WM, WN, S, KS>())) void gemm_bf16_kernel(GemmArgs p) {
    using G = Cfg<WM, WN, S, KS>;
    __shared__ __align__(16) uint16_t smem[G::kLdsElems];
    // tile numbering: consecutive numbers share the A rows; workgroup ids
    // that differ by a multiple of 8 (one XCD) get consecutive numbers
    const int T = p.tiles_m * p.tiles_n;
    int bid = blockIdx.x;
    if (T % 8 == 0) bid = (bid & 7) * (T >> 3) + (bid >> 3);
    const int mt = bid / p.tiles_n, nt = bid - mt * p.tiles_n;
    const int m0 = mt * G::kTM, n0 = nt * G::kTN;   // n0 over all count * N columns
    const int ncols = p.count * p.N;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int ks = w / G::kWavesT, wt = w - ks * G::kWavesT;   // k group, wave in the group
    const int wm = wt / WN, wn = wt - wm * WN;
    const int wu = __builtin_amdgcn_readfirstlane(w);

    // Direct loads of one stage: load i (1 KB: the A rows, then the weight
    // tile) is issued by wave i % waves. Each lane fetches the global chunk
    // that belongs at its LDS position under the swizzle; rows and columns
    // past the matrix are clamped into range (they only feed results that
    // are never stored).
    const uint16_t *src[G::kMaxPerWave];
    long step[G::kMaxPerWave];   // source advance per k step (weight loads)
    bool is_a[G::kMaxPerWave];
    int kj[G::kMaxPerWave];      // k tile of the stage the load fills
    int nl = 0;                  // loads of this wave per stage (wave-uniform)
#pragma unroll
    for (int t = 0; t < G::kMaxPerWave; ++t) {
        const int i = wu + G::kWaves * t;
        src[t] = p.A;
        step[t] = 0;
        is_a[t] = false;
        kj[t] = 0;
        if (i >= G::kInst) continue;
        ++nl;
        kj[t] = i / G::kInst1;
        const int i1 = i - kj[t] * G::kInst1;   // load within the k tile
        if (i1 < G::kAInst) {
            const int pos = i1 * 64 + lane;   // 16-byte chunk of the A tile
            const int row = pos >> 2, lc = (pos & 3) ^ ((row >> 1) & 3);
            const int m = min(m0 + row, p.M - 1);
            if (AHEADS) {
                const int b = m / p.L, l = m - b * p.L;
                src[t] = p.A + ((long)b * p.H * p.L + l) * kD + 8 * lc;
            } else {
                src[t] = p.A + (long)m * p.K + 8 * lc;
            }
            is_a[t] = true;
        } else {
            const int pos = (i1 - G::kAInst) * 64 + lane;   // chunk of the weight tile
            if (KN) {   // [32 k][kCpr chunks of n]
                const int row = pos / G::kCpr, pc = pos - row * G::kCpr;
                const int lc = pc ^ (wx<WN>(row) >> 1);
                const int ng = min(n0 + 8 * lc, ncols - 8);
                const int z = ng / p.N, n = ng - z * p.N;
                src[t] = p.B[z] + (long)row * p.N + n;
                step[t] = (long)kBK * p.N;
            } else {    // [kTN n][4 chunks of k], one weight
                const int row = pos >> 2, lc = (pos & 3) ^ ((row >> 1) & 3);
                const int n = min(n0 + row, p.N - 1);
                src[t] = p.B[0] + (long)n * p.K + 8 * lc;
                step[t] = kBK;
            }
        }
    }
    const int nk = p.K / kBK / KS;   // stages of KS k tiles
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)smem;
    auto issue = [&](int kt) {
        const uint32_t s = lds0 + 2 * G::kStage * (kt % S);   // byte address of the stage
#pragma unroll
        for (int t = 0; t < G::kMaxPerWave; ++t) {
            const int i = wu + G::kWaves * t;
            const int kk = KS * kt + kj[t];   // 32-deep k step of this load
            // A advance: 32 columns per step; in head layout 2 steps per head
            const long aoff =
                AHEADS ? (long)(kk >> 1) * p.L * kD + 32 * (kk & 1) : (long)kk * kBK;
            if (i < G::kInst)
                load_lds16(src[t] + (is_a[t] ? aoff : (long)kk * step[t]), s + 1024 * i);
        }
    };

    f32x4_t acc[4][6];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 6; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // transposed W reads: lane 4e + q of group g at row 8g + e (+ 4),
    // columns 96 wn + 16 j + 4q (unit 24 wn + 4 j + q); rows 8g + e and
    // 8g + e + 4 take the same XOR
    const int e = l16 >> 2, qq = l16 & 3;
    const int wrow = 8 * g + e, wxor = wx<WN>(wrow);
    auto products = [&](const uint16_t *sA) {
        const uint16_t *sB = sA + G::kATile;
        u32x4_t xf[4], wf[6];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xf[i] = *reinterpret_cast<const u32x4_t *>(sA + swz(kWaveM * wm + 16 * i + l16, g));
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            if (KN) {
                const int u = 24 * wn + 4 * j + qq;
                const int byte = wrow * (2 * G::kTN) + ((u ^ wxor) << 3);
                const u32x2_t lo = tr_read(sB, byte), hi = tr_read(sB, byte + 4 * 2 * G::kTN);
                wf[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
            } else {
                wf[j] = *reinterpret_cast<const u32x4_t *>(sB + swz(kWaveN * wn + 16 * j + l16, g));
            }
        }
        // the matrix-core phase at raised priority: a wave that has its
        // fragments issues its products ahead of waves still reading LDS
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 6; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, wf[j]), __builtin_bit_cast(bf16x8_t, xf[i]),
                    acc[i][j], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
    };

    // Tile kt sits in stage kt % S. Each wave waits for its own direct loads
    // of tile kt (loads complete in order, so those of the later tiles may
    // stay in flight); the barrier then publishes every wave's share and ends
    // the reads of tile kt - 1, whose stage receives tile kt + S - 1.
    for (int kt = 0; kt < S - 1 && kt < nk; ++kt) issue(kt);
    for (int kt = 0; kt < nk; ++kt) {
        const int later = min(S - 2, nk - 1 - kt);   // tiles issued after kt
        wait_vm(later * nl);
        bar();
        if (kt + S - 1 < nk) issue(kt + S - 1);
        products(smem + G::kStage * (kt % S) + G::kTile1 * ks);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this tile's LDS reads are done
    }
    bar();   // every wave is done reading the stages
    if constexpr (KS > 1) {
        // from the last k group down: group k2 leaves its sums in LDS, group
        // k2 - 1 adds them; group 0 then writes the block
        f32x4_t *red = reinterpret_cast<f32x4_t *>(smem);
#pragma unroll
        for (int k2 = KS - 1; k2 > 0; --k2) {
            if (ks == k2) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 6; ++j) red[(wt * 24 + 6 * i + j) * 64 + lane] = acc[i][j];
            }
            __syncthreads();
            if (ks == k2 - 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 6; ++j) acc[i][j] += red[(wt * 24 + 6 * i + j) * 64 + lane];
            }
            __syncthreads();   // the next fold or the staging reuses the region
        }
        if (ks > 0) return;
    }

    // acc[i][j][r] = C[m0 + 64 wm + 16 i + l16][n0 + 96 wn + 16 j + 4 g + r]:
    // wave w stages its 64 x 96 block as bf16 rows, then writes 16-byte
    // chunks of whole row segments
    unsigned char *cs = reinterpret_cast<unsigned char *>(smem) + 64 * kWRow * wt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + l16;
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            const int col = 16 * j + 4 * g;
            const bf16x4_t v = {(__bf16)acc[i][j][0], (__bf16)acc[i][j][1], (__bf16)acc[i][j][2],
                                (__bf16)acc[i][j][3]};   // round to nearest even
            *reinterpret_cast<bf16x4_t *>(cs + row * kWRow + 2 * col) = v;
        }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < 12; ++q) {
        const int idx = lane + 64 * q;
        const int row = idx / 12, chunk = idx - row * 12;
        const int m = m0 + kWaveM * wm + row, ng = n0 + kWaveN * wn + 8 * chunk;
        if (m >= p.M || ng >= ncols) continue;
        const int z = ng / p.N, n = ng - z * p.N;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(cs + row * kWRow + 16 * chunk);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(cs + row * kWRow + 16 * chunk + 8);
        uint16_t *dst;
        if (CHEADS) {
            const int b = m / p.L, l = m - b * p.L;
            dst = p.C[z] + (((long)b * p.H + (n >> 6)) * p.L + l) * kD + (n & 63);
        } else {
            dst = p.C[z] + (long)m * p.N + n;
        }
        *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
}

template <int WM, int WN, int S, bool AHEADS, bool CHEADS, bool KN, int KS = 1>
hipError_t launch_cfg(const GemmArgs &a0, hipStream_t st) {
    using G = Cfg<WM, WN, S, KS>;
    GemmArgs a = a0;
    a.tiles_m = (a.M + G::kTM - 1) / G::kTM;
    a.tiles_n = (a.count * a.N + G::kTN - 1) / G::kTN;
    const long T = (long)a.tiles_m * a.tiles_n;
    if (T >= (1L << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, S, KS, AHEADS, CHEADS, KN>), dim3((unsigned)T),
                       dim3(G::kThreads), 0, st, a);
    return hipGetLastError();
}

constexpr int kSmallKS = 2, kSmallS = 2;   // k groups and stages of the one-tile-per-CU 128 x 192 shape

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t *A, const uint16_t *const *B, uint16_t *const *C,
                            int count, int M, int N, int K, bool w_kn, bool a_heads, bool c_heads,
                            int L, int H, int cus, hipStream_t st) {
    if (count < 1 || count > 4 || M < 1 || N < 64 || N % 64 != 0 || K < 64 || K % 64 != 0)
        return hipErrorInvalidValue;
    if ((long)N * K >= (1L << 31) || (long)count * N >= (1L << 30) || (a_heads && c_heads))
        return hipErrorInvalidValue;
    if (!w_kn && (a_heads || c_heads || count != 1)) return hipErrorInvalidValue;
    GemmArgs a{};
    a.A = A;
    for (int i = 0; i < count; ++i) {
        a.B[i] = B[i];
        a.C[i] = C[i];
    }
    a.M = M;
    a.N = N;
    a.K = K;
    a.count = count;
    a.L = L;
    a.H = H;
    // one 256 x 288 tile per CU when the columns split evenly and the tiles
    // fill the CUs; 128 x 192 tiles otherwise
    const int total_n = count * N;
    const long big = (long)((M + 255) / 256) * (total_n / 288);
    if (w_kn && total_n % 288 == 0 && big >= cus) {
        if (a_heads) return launch_cfg<4, 3, 3, true, false, true>(a, st);
        if (c_heads) return launch_cfg<4, 3, 3, false, true, true>(a, st);
        return launch_cfg<4, 3, 3, false, false, true>(a, st);
    }
    // 128 x 192 tiles; at most one per CU (and an even number of k steps):
    // two k groups of four waves
    const long small = (long)((M + 127) / 128) * ((total_n + 191) / 192);
    if (small <= cus && (K / kBK) % kSmallKS == 0) {
        if (!w_kn) return launch_cfg<2, 2, kSmallS, false, false, false, kSmallKS>(a, st);
        if (a_heads) return launch_cfg<2, 2, kSmallS, true, false, true, kSmallKS>(a, st);
        if (c_heads) return launch_cfg<2, 2, kSmallS, false, true, true, kSmallKS>(a, st);
        return launch_cfg<2, 2, kSmallS, false, false, true, kSmallKS>(a, st);
    }
    if (!w_kn) return launch_cfg<2, 2, 2, false, false, false>(a, st);
    if (a_heads) return launch_cfg<2, 2, 2, true, false, true>(a, st);
    if (c_heads) return launch_cfg<2, 2, 2, false, true, true>(a, st);
    return launch_cfg<2, 2, 2, false, false, true>(a, st);
}

}  // namespace ca
