// Lloyd's k-means steps on per-head queries (staged path, any L).
//
// Assignment and update follow the model card "Hooshaai/distilbert-sst2-
// cluster-attention", Mathematical Formulation 1, and the "ClusterFormer"
// spec (svd-sst2-roberta-cluster page) 2.1: c_i = argmin_k ||q_i - mu_k||^2
// (expanded as ||mu_k||^2 - 2 q_i . mu_k; ||q_i||^2 is common to all k and
// dropped), then mu_k = sum_{c_i = k} q_i / max(1, n_k).
//
// Work split: one workgroup per 64-token tile of one slice. The tile's
// queries and all centroids sit in LDS; four lanes share a token and each
// scans every fourth centroid, then the four candidates meet in a
// lexicographic (distance, index) minimum so ties go to the lowest index.
// The same workgroup emits its tile's per-cluster partial sums in token
// order; a second kernel adds the tiles' partials in tile order. No float
// atomics anywhere, so the result is bitwise reproducible.
#include <map>
#include <mutex>
#include <utility>

#include "launch.h"

namespace ca {

constexpr int kTile = 64;      // tokens per workgroup
constexpr int kPad = kD + 1;   // LDS row stride (breaks bank conflicts)

int kmeans_tiles(int L) { return (L + kTile - 1) / kTile; }

// MODE: 0 = assign only, 1 = assign and emit partials, 2 = partials of a
// given assignment (read from `assign`). INIT: centroids are the initial
// rows of Q (init_row: floor(k L / Kc), or k * init_step in the listing's
// variant) instead of `mu`; the first tile of each slice then also writes
// them to mu_init when that is not null.
template <typename T, bool INIT, int MODE>
__global__ __launch_bounds__(256) void kmeans_assign_kernel(
    const T *__restrict__ Q, const float *__restrict__ mu, int L, int Kc, int ntile,
    int32_t *__restrict__ assign, float *__restrict__ part_sum, int32_t *__restrict__ part_cnt,
    int init_step, float *__restrict__ mu_init) {
    extern __shared__ float smem[];
    float *sm_mu = smem;                    // [Kc][kPad]
    float *sm_mn = sm_mu + Kc * kPad;       // [Kc]
    float *sm_q = sm_mn + Kc;               // [kTile][kPad]
    int *sm_c = reinterpret_cast<int *>(sm_q + kTile * kPad);  // [kTile]
    float *sm_p = reinterpret_cast<float *>(sm_c + kTile);     // [Kc][kD]
    int *sm_n = reinterpret_cast<int *>(sm_p + Kc * kD);        // [Kc]

    const int tid = threadIdx.x;
    const int tile = blockIdx.x % ntile;
    const long s = blockIdx.x / ntile;
    const T *Qs = Q + s * (long)L * kD;
    const int i0 = tile * kTile;
    const int nt = min(kTile, L - i0);

    if (MODE != 2) {
        for (int e = tid; e < Kc * (kD / 4); e += 256) {
            const int k = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
            float4 v;
            if (INIT) {
                const long row = init_row(k, L, Kc, init_step);
                v = load4<T>(Qs + row * kD + c4);
                if (mu_init && tile == 0)
                    *reinterpret_cast<float4 *>(mu_init + (s * Kc + k) * kD + c4) = v;
            } else {
                v = load4<float>(mu + (s * Kc + k) * kD + c4);
            }
            float *dst = sm_mu + k * kPad + c4;
            dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
        }
    }
    for (int e = tid; e < nt * (kD / 4); e += 256) {
        const int i = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
        float4 v = load4<T>(Qs + (long)(i0 + i) * kD + c4);
        float *dst = sm_q + i * kPad + c4;
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
    if (MODE == 2) {
        // a given assignment outside [0, Kc) is clamped into it
        for (int i = tid; i < nt; i += 256) sm_c[i] = min(max(assign[s * L + i0 + i], 0), Kc - 1);
    } else {
        __syncthreads();
        for (int k = tid; k < Kc; k += 256) {
            const float *m = sm_mu + k * kPad;
            float a = 0.f;
            for (int j = 0; j < kD; ++j) a = fmaf(m[j], m[j], a);
            sm_mn[k] = a;
        }
        __syncthreads();

        const int t = tid >> 2, g = tid & 3;
        float best = __builtin_inff();
        int bk = 0x7fffffff;
        if (t < nt) {
            const float *q = sm_q + t * kPad;
            for (int k = g; k < Kc; k += 4) {
                const float *m = sm_mu + k * kPad;
                const float dot = dot64(q, m);
                const float D = fmaf(-2.f, dot, sm_mn[k]);
                if (lex_less(D, k, best, bk)) { best = D; bk = k; }
            }
        }
#pragma unroll
        for (int off = 1; off < 4; off <<= 1) {
            const float ob = __shfl_xor(best, off);
            const int ok = __shfl_xor(bk, off);
            if (lex_less(ob, ok, best, bk)) { best = ob; bk = ok; }
        }
        if (bk >= Kc) bk = 0;  // only if every distance was NaN
        if (t < nt && g == 0) {
            sm_c[t] = bk;
            assign[s * L + i0 + t] = bk;
        }
    }
    if (MODE == 0) return;

    // Per-tile partial sums. Cell (k, j) belongs to lane j of wave k % 4, so
    // each cell is updated by one thread, in token order.
    const int j = tid & (kD - 1), w = tid >> 6;
    for (int k = w; k < Kc; k += 4) {
        sm_p[k * kD + j] = 0.f;
        if (j == 0) sm_n[k] = 0;
    }
    __syncthreads();
    for (int i = 0; i < nt; ++i) {
        const int k = sm_c[i];
        if ((k & 3) == w) {
            sm_p[k * kD + j] += sm_q[i * kPad + j];
            if (j == 0) sm_n[k] += 1;
        }
    }
    __syncthreads();
    const long base = (s * ntile + tile) * (long)Kc;
    for (int e = tid; e < Kc * kD; e += 256) part_sum[base * kD + e] = sm_p[e];
    for (int k = tid; k < Kc; k += 256) part_cnt[base + k] = sm_n[k];
}

// mu[s,k,:] = (sum over the blocks) / max(1, n); counts optional.
// keep_empty (the listing's rule): a cluster with n = 0 leaves mu[s,k,:] as
// it was. One workgroup per centroid row, lane j = dimension j: wave q adds
// blocks q, q + 4, ... (eight loads in flight per lane), and wave 0 adds the
// four sums in wave order.
__global__ __launch_bounds__(256) void centroid_reduce_kernel(
    const float *__restrict__ part_sum, const int32_t *__restrict__ part_cnt, int nblk, int Kc,
    float *__restrict__ mu, int32_t *__restrict__ counts, int keep_empty) {
    __shared__ float rec[4][kD];
    __shared__ int rcnt[4];
    const int q = threadIdx.x >> 6, j = threadIdx.x & 63;
    const long sk = blockIdx.x;   // s * Kc + k
    const long s = sk / Kc, k = sk % Kc;
    const long per = (long)Kc * kD;
    const float *p0 = part_sum + s * nblk * per + k * kD + j;
    const int32_t *c0 = part_cnt + s * nblk * (long)Kc + k;
    float acc = 0.f;
    int n = 0;
    for (int b0 = q; b0 < nblk; b0 += 32) {
        float a8[8];
        int n8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int b = b0 + 4 * u;
            a8[u] = b < nblk ? p0[b * per] : 0.f;
            n8[u] = b < nblk ? c0[(long)b * Kc] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            acc += a8[u];
            n += n8[u];
        }
    }
    rec[q][j] = acc;
    if (j == 0) rcnt[q] = n;
    __syncthreads();
    if (q != 0) return;
    const float tot = ((rec[0][j] + rec[1][j]) + rec[2][j]) + rec[3][j];
    const int nt = rcnt[0] + rcnt[1] + rcnt[2] + rcnt[3];
    if (!(keep_empty && nt == 0)) mu[sk * kD + j] = tot / (float)(nt > 1 ? nt : 1);
    if (counts && j == 0) counts[sk] = nt;
}

static size_t assign_lds_bytes(int Kc, bool partials) {
    size_t b = sizeof(float) * ((size_t)Kc * kPad + Kc + kTile * kPad) + sizeof(int) * kTile;
    if (partials) b += sizeof(float) * (size_t)Kc * kD + sizeof(int) * Kc;
    return b;
}

template <typename T, bool INIT, int MODE>
static hipError_t assign_launch(const void *Q, const float *mu, int S, int L, int Kc,
                                int32_t *assign, float *part_sum, int32_t *part_cnt,
                                hipStream_t st, int init_step = 0, float *mu_init = nullptr) {
    auto kern = kmeans_assign_kernel<T, INIT, MODE>;
    const size_t lds = assign_lds_bytes(Kc, MODE != 0);
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(kern), (int)lds);
    if (e != hipSuccess) return e;
    const int ntile = kmeans_tiles(L);
    hipLaunchKernelGGL(kern, dim3((unsigned)((long)S * ntile)), dim3(256), lds, st,
                       static_cast<const T *>(Q), mu, L, Kc, ntile, assign, part_sum, part_cnt,
                       init_step, mu_init);
    return hipGetLastError();
}

template <typename T>
static hipError_t assign_dispatch(const void *Q, const float *mu, int S, int L, int Kc,
                                  int32_t *assign, float *part_sum, int32_t *part_cnt,
                                  hipStream_t st, int init_step, float *mu_init) {
    const bool partials = part_sum != nullptr;
    if (mu == nullptr)
        return partials ? assign_launch<T, true, 1>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st,
                                                    init_step, mu_init)
                        : assign_launch<T, true, 0>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st,
                                                    init_step, mu_init);
    return partials ? assign_launch<T, false, 1>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st)
                    : assign_launch<T, false, 0>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st);
}

hipError_t launch_kmeans_assign(const void *Q, const float *mu, int S, int L, int Kc,
                                ca_dtype_t dt, int32_t *assign, float *part_sum,
                                int32_t *part_cnt, hipStream_t st, int init_step,
                                float *mu_init) {
    if (dt == CA_BF16)
        return assign_dispatch<bf16_t>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st, init_step,
                                       mu_init);
    return assign_dispatch<float>(Q, mu, S, L, Kc, assign, part_sum, part_cnt, st, init_step,
                                  mu_init);
}

hipError_t launch_centroid_partials(const void *Q, const int32_t *assign, int S, int L, int Kc,
                                    ca_dtype_t dt, float *part_sum, int32_t *part_cnt,
                                    hipStream_t st) {
    int32_t *c = const_cast<int32_t *>(assign);   // read-only in this mode
    if (dt == CA_BF16)
        return assign_launch<bf16_t, false, 2>(Q, nullptr, S, L, Kc, c, part_sum, part_cnt, st);
    return assign_launch<float, false, 2>(Q, nullptr, S, L, Kc, c, part_sum, part_cnt, st);
}

hipError_t launch_centroid_reduce(const float *part_sum, const int32_t *part_cnt, int nblk,
                                  int S, int Kc, float *mu, int32_t *counts, hipStream_t st,
                                  bool keep_empty) {
    hipLaunchKernelGGL(centroid_reduce_kernel, dim3((unsigned)((long)S * Kc)), dim3(256), 0, st,
                       part_sum, part_cnt, nblk, Kc, mu, counts, keep_empty ? 1 : 0);
    return hipGetLastError();
}

hipError_t ensure_dynamic_lds(const void *fn, int bytes) {
    static std::mutex lock;
    static std::map<std::pair<const void *, int>, int> limits;   // (kernel, device) -> bytes
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> guard(lock);
    int &have = limits[{fn, dev}];
    if (have >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) have = bytes;
    return e;
}

}  // namespace ca
