// Exact attention of the decoder and cross-attention branch (any L, Nk).
//
// The ClusterAttention listing on the "Hooshaai/svd-sst2-roberta-cluster"
// page sends causal decoders and cross-attention to exact attention instead
// of clustering ("Architectural Support" section; forward, decoder branch):
//   O_i = sum_j softmax_j(s_ij) v_j over all Nk keys,
//   s_ij = q_i . k_j / 8, or -10000 where key j is padded or (causal) j > i,
// and the row of a padded query is zero. The -10000 is a fill, not an
// exclusion: a causal row whose keys j <= i are all padded is uniform over all
// Nk keys, future ones included.
//
// Work split: one workgroup per 64-query tile; four lanes per query (16 dims
// each, partial dot products joined by DPP quad sums); key tiles of 64 rows
// stream through LDS with an online softmax, as in the local window kernel.
// A causal tile stops at its last query; a second pass over the later keys
// runs only if some query of the tile saw padded keys alone (every later
// key then weighs exactly as much as those).
#include "launch.h"

namespace ca {

constexpr int kEQ = 64;         // queries per workgroup
constexpr int kEK = 64;         // keys per LDS tile
constexpr int kERow = kD;       // K/V row stride (a whole wave reads one row)
constexpr int kEPad = kD + 1;   // score rows (lanes read different rows)

template <typename T, bool CAUSAL>
__global__ __launch_bounds__(256) void exact_attn_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx, int L, int Nk,
    int ntile, const uint8_t *__restrict__ qvalid, const uint8_t *__restrict__ kvalid, int H,
    int G, T *__restrict__ out) {
    __shared__ __align__(16) float sm_k[kEK * kERow];
    __shared__ __align__(16) float sm_v[kEK * kERow];
    __shared__ float sm_s[kEQ * kEPad];
    __shared__ uint8_t sm_ok[kEK];
    __shared__ int sm_any;

    const int tid = threadIdx.x;
    const int tile = blockIdx.x % ntile;
    const long s = blockIdx.x / ntile;
    const long b = s / H;
    const long base = s * (long)L * kD;
    const long kvbase = kv_slice(s, H, G) * (long)Nk * kD;
    const int i0 = tile * kEQ, nq = min(kEQ, L - i0);
    const int qi = tid >> 2, g = tid & 3;
    const int i = i0 + qi;
    const bool active = qi < nq;
    const float scale = 1.0f / sqrtf((float)kD);

    float qr[16];
    if (active) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float4 v = load4<T>(Q + base + (long)i * kD + 16 * g + 4 * c);
            qr[4 * c] = v.x * scale; qr[4 * c + 1] = v.y * scale;
            qr[4 * c + 2] = v.z * scale; qr[4 * c + 3] = v.w * scale;
        }
    } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) qr[c] = 0.f;
    }
    float m = -__builtin_inff(), l = 0.f, acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = 0.f;

    // keys [lo, hi] of this row (inclusive, absolute), key tiles [t0, t1)
    // of the workgroup; fill: every key of the pass takes the -10000 logit
    auto pass = [&](int lo, int hi, int t0, int t1, bool fill) {
        for (int jt = t0; jt < t1; jt += kEK) {
            const int nk = min(kEK, t1 - jt);
            __syncthreads();
            for (int e = tid; e < nk * (kD / 4); e += 256) {
                const int rr = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
                *reinterpret_cast<float4 *>(sm_k + rr * kERow + c4) =
                    load4<T>(Kx + kvbase + (long)(jt + rr) * kD + c4);
                *reinterpret_cast<float4 *>(sm_v + rr * kERow + c4) =
                    load4<T>(Vx + kvbase + (long)(jt + rr) * kD + c4);
            }
            for (int rr = tid; rr < nk; rr += 256)
                sm_ok[rr] = !fill && (kvalid == nullptr || kvalid[b * Nk + jt + rr] != 0);
            __syncthreads();
            const int a = max(lo, jt) - jt;
            const int bb = min(hi, jt + nk - 1) - jt;   // a > bb: none
            const int wa = wave_min_i32(a <= bb ? a : kEK);
            const int wb = wave_max_i32(a <= bb ? bb : -1);
            float mt = -__builtin_inff();
            for (int key = wa; key <= wb; ++key) {
                const float *kr = sm_k + key * kERow + 16 * g;
                float sc = quad_sum(dot16(qr, kr));
                if (!sm_ok[key]) sc = -10000.f;
                if (key >= a && key <= bb) {
                    mt = fmaxf(mt, sc);
                    if (g == 0) sm_s[qi * kEPad + key] = sc;
                }
            }
            __syncthreads();
            if (a <= bb) {
                const float mn = fmaxf(m, mt);
                const float corr = (m == -__builtin_inff()) ? 0.f : exp_f32(m - mn);
                l *= corr;
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[c] *= corr;
                for (int key = a; key <= bb; ++key) {
                    const float p = exp_f32(sm_s[qi * kEPad + key] - mn);
                    l += p;
                    const float *vr = sm_v + key * kERow + 16 * g;
#pragma unroll
                    for (int c = 0; c < 16; ++c) acc[c] = fmaf(p, vr[c], acc[c]);
                }
                m = mn;
            }
        }
    };

    const int hi = active ? (CAUSAL ? min(i, Nk - 1) : Nk - 1) : -1;
    const int t1 = CAUSAL ? min(Nk, i0 + nq) : Nk;
    pass(0, hi, 0, t1, false);
    if (CAUSAL && t1 < Nk) {
        // rows that met padded keys alone: the later keys carry the same
        // -10000 logit, so they enter the softmax too
        const bool only_pad = active && m == -10000.f && hi < Nk - 1;
        if (tid == 0) sm_any = 0;
        __syncthreads();
        if (only_pad) sm_any = 1;
        __syncthreads();
        // every such row has hi = i >= i0, so its later keys start in tile i0
        if (sm_any) pass(only_pad ? hi + 1 : Nk, Nk - 1, i0, Nk, true);
    }
    if (!active) return;
    const bool keep = qvalid == nullptr || qvalid[b * L + i] != 0;
    const float inv = keep ? 1.0f / l : 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        store4<T>(out + base + (long)i * kD + 16 * g + 4 * c,
                  make_float4(acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv,
                              acc[4 * c + 3] * inv));
}

template <typename T>
static hipError_t exact_dispatch(const void *Q, const void *K, const void *V, int S, int L, int Nk,
                                 bool causal, const uint8_t *qvalid, const uint8_t *kvalid, int H,
                                 int G, void *out, hipStream_t st) {
    const int ntile = (L + kEQ - 1) / kEQ;
    const dim3 grid((unsigned)((long)S * ntile)), block(256);
    const T *q = static_cast<const T *>(Q), *k = static_cast<const T *>(K);
    const T *v = static_cast<const T *>(V);
    if (causal)
        hipLaunchKernelGGL((exact_attn_kernel<T, true>), grid, block, 0, st, q, k, v, L, Nk, ntile,
                           qvalid, kvalid, H, G, static_cast<T *>(out));
    else
        hipLaunchKernelGGL((exact_attn_kernel<T, false>), grid, block, 0, st, q, k, v, L, Nk,
                           ntile, qvalid, kvalid, H, G, static_cast<T *>(out));
    return hipGetLastError();
}

hipError_t launch_exact_attention(const void *Q, const void *K, const void *V, int S, int L,
                                  int Nk, bool causal, ca_dtype_t dt, const uint8_t *qvalid,
                                  const uint8_t *kvalid, int H, int G, void *out,
                                  hipStream_t st) {
    if (dt == CA_BF16)
        return exact_dispatch<bf16_t>(Q, K, V, S, L, Nk, causal, qvalid, kvalid, H, G, out, st);
    return exact_dispatch<float>(Q, K, V, S, L, Nk, causal, qvalid, kvalid, H, G, out, st);
}

}  // namespace ca
