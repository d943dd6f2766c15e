// bf16 projection GEMMs of the full attention layer (model card
// "Hooshaai/distilbert-sst2-cluster-attention", Architecture Overview: the
// multi-head projections of X and the output projection Y = O W_O;
// "ClusterFormer" spec on the "Hooshaai/svd-sst2-roberta-cluster" page,
// section 3, first and last rows of the tensor trace).
//
// C = A . Bt^T on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulation, one round-to-nearest-even at the store). Both operands are
// read with the contraction index fastest, which is what the matrix cores
// consume, so a weight stored [in, out] is first transposed once per call.
//
// Operand modes, chosen at compile time:
//   A rows      : plain row-major [M, K], or the heads of a [B, H, L, 64]
//                 tensor merged on the fly (row b*L + l, column 64 h + j).
//   C rows      : plain row-major [M, N], or split into heads on the fly
//                 ([B, H, L, 64], head h = columns 64 h .. 64 h + 63).
//
// Tiling: 128 x 128 output tile per workgroup of 4 waves (64 x 64 each),
// 64-deep k steps, A and Bt tiles double-buffered in LDS as XOR-swizzled
// rows of 8 sixteen-byte chunks. Within each 64-row group of the Bt tile,
// row 16a + 4j + r is stored at LDS row 16j + 4a + r, so that the 16 x 16
// result blocks j = 0..3 of a wave leave each lane with 16 consecutive output
// columns (two 16-byte stores per row).
#include "launch.h"

namespace ca {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kTile = kBM * kBK;   // elements of one operand tile (kBM == kBN)

struct GemmArgs {
    const uint16_t *A;
    const uint16_t *Bt[4];
    uint16_t *C[4];
    int M, N, K;
    int L, H;   // head geometry of the merged / split modes
};

__device__ __forceinline__ int swz(int row, int chunk) {   // element offset of a 16-B chunk
    return row * kBK + ((chunk ^ (row & 7)) << 3);
}
__device__ __forceinline__ u32x4_t lds16(const uint16_t *p) { return *reinterpret_cast<const u32x4_t *>(p); }

// Bt tile row (within its 64-row group) -> LDS row: swap the 16-row and 4-row fields
__device__ __forceinline__ int bt_row(int row) {
    const int a = (row >> 4) & 3, j = (row >> 2) & 3;
    return (row & ~63) | (j << 4) | (a << 2) | (row & 3);
}

template <bool AHEADS, bool CHEADS>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_nt_kernel(GemmArgs p) {
    __shared__ __align__(16) uint16_t sA[2][kTile];
    __shared__ __align__(16) uint16_t sB[2][kTile];
    const int z = blockIdx.z;
    const uint16_t *__restrict__ Bt = p.Bt[z];
    uint16_t *__restrict__ C = p.C[z];
    const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int wm = w >> 1, wn = w & 1;
    const int chunk = tid & 7;

    // per-thread global rows (clamped into range; rows past M or N only feed
    // results that are never stored) and their LDS destinations
    long abase[4], bbase[4];
    int aoff[4], boff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = (tid >> 3) + 32 * q;
        int m = m0 + row;
        m = m < p.M ? m : p.M - 1;
        if (AHEADS) {
            const int b = m / p.L, l = m - b * p.L;
            abase[q] = ((long)b * p.H * p.L + l) * kD + 8 * chunk;
        } else {
            abase[q] = (long)m * p.K + 8 * chunk;
        }
        int n = n0 + row;
        n = n < p.N ? n : p.N - 1;
        bbase[q] = (long)n * p.K + 8 * chunk;
        aoff[q] = swz(row, chunk);
        boff[q] = swz(bt_row(row), chunk);
    }
    const long astep = AHEADS ? (long)p.L * kD : kBK;   // A advance per k step

    const int nk = p.K / kBK;
    // two register stages: tile t is loaded into stage t % 2 two steps before
    // its products and stored to LDS buffer t % 2 one step before
    u32x4_t ra[2][4], rb[2][4];
    auto gload = [&](int kt, int sl) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ra[sl][q] = *reinterpret_cast<const u32x4_t *>(p.A + abase[q] + kt * astep);
            rb[sl][q] = *reinterpret_cast<const u32x4_t *>(Bt + bbase[q] + (long)kt * kBK);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<u32x4_t *>(&sA[buf][aoff[q]]) = ra[buf][q];
            *reinterpret_cast<u32x4_t *>(&sB[buf][boff[q]]) = rb[buf][q];
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto products = [&](int buf) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4_t af[4], bf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) af[j] = lds16(&sB[buf][swz(64 * wn + 16 * j + l16, 4 * c + g)]);
#pragma unroll
            for (int i = 0; i < 4; ++i) bf[i] = lds16(&sA[buf][swz(64 * wm + 16 * i + l16, 4 * c + g)]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, af[j]), __builtin_bit_cast(bf16x8_t, bf[i]),
                        acc[i][j], 0, 0, 0);
        }
    };
    // one k step on LDS buffer b (= kt % 2): request tile kt + 2, multiply
    // tile kt, store tile kt + 1
    auto step = [&](int kt, int b) {
        if (kt + 2 < nk) gload(kt + 2, b);
        products(b);
        if (kt + 1 < nk) sstore(b ^ 1);
        __syncthreads();
    };

    gload(0, 0);
    sstore(0);
    if (nk > 1) gload(1, 1);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, 0);
        if (kt + 1 < nk) step(kt + 1, 1);
    }

    // acc[i][j][r] = C[m0 + 64 wm + 16 i + l16][n0 + 64 wn + 16 g + 4 j + r]
    const int nb = n0 + 64 * wn + 16 * g;
    if (nb >= p.N) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + 64 * wm + 16 * i + l16;
        if (m >= p.M) continue;
        uint32_t pk[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pk[2 * j] = (uint32_t)f32_to_bf16(acc[i][j][0]) | ((uint32_t)f32_to_bf16(acc[i][j][1]) << 16);
            pk[2 * j + 1] = (uint32_t)f32_to_bf16(acc[i][j][2]) | ((uint32_t)f32_to_bf16(acc[i][j][3]) << 16);
        }
        uint16_t *dst;
        if (CHEADS) {
            const int b = m / p.L, l = m - b * p.L, h = nb >> 6;
            dst = C + (((long)b * p.H + h) * p.L + l) * kD + (nb & 63);
        } else {
            dst = C + (long)m * p.N + nb;
        }
        reinterpret_cast<u32x4_t *>(dst)[0] = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
        reinterpret_cast<u32x4_t *>(dst)[1] = u32x4_t{pk[4], pk[5], pk[6], pk[7]};
    }
}

// W [R, Cc] -> Wt [Cc, R] (bf16 bits), 64 x 64 tiles through LDS; blockIdx.z
// selects one of up to four matrices of the same shape
struct TransposeArgs {
    const uint16_t *src[4];
    uint16_t *dst[4];
    int R, Cc;
};

__global__ __launch_bounds__(256) void transpose_bf16_kernel(TransposeArgs p) {
    __shared__ uint16_t t[64][66];
    const uint16_t *__restrict__ src = p.src[blockIdx.z];
    uint16_t *__restrict__ dst = p.dst[blockIdx.z];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = (tid >> 3) + 32 * q, ch = tid & 7;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(src + (long)(r0 + row) * p.Cc + c0 + 8 * ch);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            t[8 * ch + 2 * e][row] = (uint16_t)(v[e] & 0xffffu);
            t[8 * ch + 2 * e + 1][row] = (uint16_t)(v[e] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int col = (tid >> 3) + 32 * q, ch = tid & 7;
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w4[e] = (uint32_t)t[col][8 * ch + 2 * e] | ((uint32_t)t[col][8 * ch + 2 * e + 1] << 16);
        *reinterpret_cast<u32x4_t *>(dst + (long)(c0 + col) * p.R + r0 + 8 * ch) =
            u32x4_t{w4[0], w4[1], w4[2], w4[3]};
    }
}

}  // namespace

hipError_t launch_transpose_bf16(const uint16_t *const *src, uint16_t *const *dst, int count,
                                 int R, int Cc, hipStream_t st) {
    TransposeArgs a{};
    for (int i = 0; i < count; ++i) {
        a.src[i] = src[i];
        a.dst[i] = dst[i];
    }
    a.R = R;
    a.Cc = Cc;
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3(Cc / 64, R / 64, count), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm_nt(const uint16_t *A, const uint16_t *const *Bt, uint16_t *const *C,
                          int count, int M, int N, int K, bool a_heads, bool c_heads, int L, int H,
                          hipStream_t st) {
    GemmArgs a{};
    a.A = A;
    for (int i = 0; i < count; ++i) {
        a.Bt[i] = Bt[i];
        a.C[i] = C[i];
    }
    a.M = M;
    a.N = N;
    a.K = K;
    a.L = L;
    a.H = H;
    const dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM, count);
    if (a_heads && c_heads) return hipErrorInvalidValue;
    if (a_heads)
        hipLaunchKernelGGL((gemm_nt_kernel<true, false>), grid, dim3(kGemmThreads), 0, st, a);
    else if (c_heads)
        hipLaunchKernelGGL((gemm_nt_kernel<false, true>), grid, dim3(kGemmThreads), 0, st, a);
    else
        hipLaunchKernelGGL((gemm_nt_kernel<false, false>), grid, dim3(kGemmThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace ca
