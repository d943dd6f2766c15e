// Backward pass of cluster attention (any L): gradients of sum(dO * O) with
// respect to Q, K, V and alpha, with the final assignment c held fixed.
//
// Why c is fixed: the assignment is a piecewise-constant argmin; the pages
// fine-tune through the clustering (the svd-sst2-roberta-cluster page calls
// the k-means differentiable in its "Architectural Support" section; the
// model card's benchmark table has a "Post-KD Recovery" column), so the
// gradient flows through everything else:
//   mu_k   = sum_{c_i = k} q_i / n_k                  (d mu_k / d q_i = 1 / n_k)
//   Pc_kj  = softmax_j(mu_k . k_j / 8),  Vc = Pc V    (model card pipeline figure)
//   Pl_ij  = softmax_{|i-j| <= r}(q_i . k_j / 8),  Ol = Pl V
//   O_i    = keep_i ((1 - alpha) Vc_{c_i} + alpha Ol_i)
// and the softmax rule dS = P (dP - rowsum(P dP)) for both branches. A padded
// key's logit is the constant -10000: it passes no gradient to q or k.
//
// Launch sequence (host side in api.hip): the centroid update and the
// centroid attention with its row statistics are the forward's own kernels;
// then
//   1. bwd_cluster_sum_kernel + bwd_partial_reduce_kernel:
//        dVc_k = (1 - alpha) sum_{c_i = k} keep_i dO_i  (token order per tile,
//        tile order across tiles: deterministic, no float atomics);
//   2. bwd_query_stats_kernel: per query tile, the local softmax statistics
//        (max, sum), Ol_i, D_i = dOl_i . Ol_i with dOl_i = alpha keep_i dO_i,
//        and the tile's share of dalpha = sum keep dO . (Ol - Vc_c);
//   3. bwd_key_kernel: per (K/V slice, 64-key tile), over the query heads
//        that share the K/V head: dK_j and dV_j from both branches, written
//        once (each key row has one owner), and per-tile partial sums of
//        dmu_k = sum_j dSc_kj k_j / 8;
//   4. bwd_partial_reduce_kernel: dmu in tile order;
//   5. bwd_query_kernel: per query tile, dQ_i = sum_j dSl_ij k_j / 8 +
//        dmu_{c_i} / n_{c_i};
//   6. bwd_sum_kernel: dalpha in a fixed order.
// Arithmetic is fp32 (the storage dtype is read and written); four lanes
// share a row, each holding 16 of its 64 dims, and meet through two
// butterfly adds, as in the forward's staged kernels.
#include "launch.h"

namespace ca {

constexpr int kBT = 64;          // rows per tile
constexpr int kBPad = kD + 1;    // LDS stride of rows that lanes read at different rows
constexpr int kRow = kD;         // LDS stride of rows that a whole wave reads at once
constexpr int kBChunk = 32;      // centroids per pass of the key kernel

template <typename T>
__device__ __forceinline__ void load16(const T *p, float *x) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float4 v = load4<T>(p + 4 * c);
        x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
    }
}

template <typename T>
__device__ __forceinline__ void store16(T *p, const float *x) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
        store4<T>(p + 4 * c, make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]));
}

__device__ __forceinline__ bool token_ok(const uint8_t *valid, long b, int L, int i) {
    return valid == nullptr || valid[b * L + i] != 0;
}

// ---------------------------------------------------------------- 1. dVc partials
// part[s, tile, k, :] = sum over the tile's tokens i with c_i = k of keep_i dO_i
// (cell (k, t) is updated by lane t of wave k % 4 only, in token order).
template <typename T>
__global__ __launch_bounds__(256) void bwd_cluster_sum_kernel(
    const T *__restrict__ dO, const int32_t *__restrict__ assign, const uint8_t *__restrict__ valid,
    int L, int Kc, int H, int ntile, float *__restrict__ part) {
    extern __shared__ float smem[];
    float *sm_g = smem;                                   // [kBT][kBPad]
    float *sm_p = sm_g + kBT * kBPad;                     // [Kc][kD]
    int *sm_c = reinterpret_cast<int *>(sm_p + Kc * kD);  // [kBT]
    const int tid = threadIdx.x;
    const int tile = blockIdx.x % ntile;
    const long s = blockIdx.x / ntile;
    const int i0 = tile * kBT, nt = min(kBT, L - i0);
    for (int e = tid; e < nt * (kD / 4); e += 256) {
        const int i = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
        const bool keep = token_ok(valid, s / H, L, i0 + i);
        const float4 v = load4<T>(dO + (s * L + i0 + i) * (long)kD + c4);
        float *dst = sm_g + i * kBPad + c4;
        dst[0] = keep ? v.x : 0.f; dst[1] = keep ? v.y : 0.f;
        dst[2] = keep ? v.z : 0.f; dst[3] = keep ? v.w : 0.f;
    }
    for (int i = tid; i < nt; i += 256) sm_c[i] = min(max(assign[s * L + i0 + i], 0), Kc - 1);
    const int t = tid & (kD - 1), w = tid >> 6;
    for (int k = w; k < Kc; k += 4) sm_p[k * kD + t] = 0.f;
    __syncthreads();
    for (int i = 0; i < nt; ++i) {
        const int k = sm_c[i];
        if ((k & 3) == w) sm_p[k * kD + t] += sm_g[i * kBPad + t];
    }
    __syncthreads();
    float *dst = part + (s * ntile + tile) * (long)Kc * kD;
    for (int e = tid; e < Kc * kD; e += 256) dst[e] = sm_p[e];
}

// out[s, k, :] = scale * sum over tiles (in tile order) of part[s, tile, k, :]
__global__ __launch_bounds__(256) void bwd_partial_reduce_kernel(
    const float *__restrict__ part, int ntile, int Kc, long total, float scale,
    float *__restrict__ out) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const long per = (long)Kc * kD;
    const long s = e / per, r = e % per;
    float acc = 0.f;
    for (int b = 0; b < ntile; ++b) acc += part[(s * ntile + b) * per + r];
    out[e] = acc * scale;
}

// ---------------------------------------------------------------- 2. query statistics
// lstat[s, i] = (max logit, sum exp(logit - max), D_i, 0) of query i's
// window; dal[s * ntile + tile] = the tile's share of dalpha.
template <typename T>
__global__ __launch_bounds__(256) void bwd_query_stats_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx,
    const T *__restrict__ dO, const int32_t *__restrict__ assign, const float *__restrict__ vcent,
    const uint8_t *__restrict__ valid, int L, int r, int ntile, int Kc, float alpha, int H, int G,
    float4 *__restrict__ lstat, float *__restrict__ dal) {
    __shared__ __align__(16) float sm_k[kBT * kRow];
    __shared__ __align__(16) float sm_v[kBT * kRow];
    __shared__ float sm_s[kBT * kBPad];
    __shared__ uint8_t sm_ok[kBT];
    __shared__ float sm_red[kBT];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x % ntile;
    const long s = blockIdx.x / ntile;
    const long base = s * (long)L * kD;
    const long kvbase = kv_slice(s, H, G) * (long)L * kD;
    const int i0 = tile * kBT, nq = min(kBT, L - i0);
    const int qi = tid >> 2, g = tid & 3;
    const int i = i0 + qi;
    const bool active = qi < nq;
    const int lo = (int)max(0L, (long)i - r), hi = (int)min((long)L - 1, (long)i + r);
    const int tlo = (int)max(0L, (long)i0 - r);
    const int thi = (int)min((long)L, (long)i0 + nq + r);
    const float scale = 1.0f / sqrtf((float)kD);

    float qr[16];
    if (active) {
        load16(Q + base + (long)i * kD + 16 * g, qr);
#pragma unroll
        for (int c = 0; c < 16; ++c) qr[c] *= scale;
    } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) qr[c] = 0.f;
    }
    float m = -__builtin_inff(), l = 0.f, acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = 0.f;
    for (int jt = tlo; jt < thi; jt += kBT) {
        const int nk = min(kBT, thi - jt);
        __syncthreads();
        for (int e = tid; e < nk * (kD / 4); e += 256) {
            const int rr = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
            const float4 kv = load4<T>(Kx + kvbase + (long)(jt + rr) * kD + c4);
            const float4 vv = load4<T>(Vx + kvbase + (long)(jt + rr) * kD + c4);
            float *dk = sm_k + rr * kRow + c4;
            float *dv = sm_v + rr * kRow + c4;
            dk[0] = kv.x; dk[1] = kv.y; dk[2] = kv.z; dk[3] = kv.w;
            dv[0] = vv.x; dv[1] = vv.y; dv[2] = vv.z; dv[3] = vv.w;
        }
        for (int rr = tid; rr < nk; rr += 256) sm_ok[rr] = token_ok(valid, s / H, L, jt + rr);
        __syncthreads();
        const int a = active ? max(lo, jt) - jt : 0;
        const int b = active ? min(hi, jt + nk - 1) - jt : -1;
        const int wa = wave_min_i32(a < b + 1 ? a : kBT);
        const int wb = wave_max_i32(b);
        float mt = -__builtin_inff();
        for (int key = wa; key <= wb; ++key) {
            const float *kr = sm_k + key * kRow + 16 * g;
            float sc = quad_sum(dot16(qr, kr));
            if (!sm_ok[key]) sc = -10000.f;
            if (key >= a && key <= b) {
                mt = fmaxf(mt, sc);
                if (g == 0) sm_s[qi * kBPad + key] = sc;
            }
        }
        __syncthreads();
        if (b >= a) {
            const float mn = fmaxf(m, mt);
            const float corr = (m == -__builtin_inff()) ? 0.f : exp_f32(m - mn);
            l *= corr;
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[c] *= corr;
            for (int key = a; key <= b; ++key) {
                const float p = exp_f32(sm_s[qi * kBPad + key] - mn);
                l += p;
                const float *vr = sm_v + key * kRow + 16 * g;
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[c] = fmaf(p, vr[c], acc[c]);
            }
            m = mn;
        }
    }
    float dpart = 0.f, apart = 0.f;
    if (active) {
        const bool keep = token_ok(valid, s / H, L, i);
        float go[16];
        load16(dO + base + (long)i * kD + 16 * g, go);
        const int c = min(max(assign[s * L + i], 0), Kc - 1);
        const float *vc = vcent + (s * Kc + c) * kD + 16 * g;
        const float inv = 1.0f / l;
        if (keep) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float ol = acc[e] * inv;
                dpart = fmaf(alpha * go[e], ol, dpart);
                apart = fmaf(go[e], ol - vc[e], apart);
            }
        }
    }
    const float D = quad_sum(dpart);
    const float A = quad_sum(apart);
    if (active && g == 0) lstat[s * L + i] = make_float4(m, l, D, 0.f);
    if (g == 0) sm_red[qi] = active ? A : 0.f;
    __syncthreads();
    if (tid == 0) {
        float t = 0.f;
        for (int q = 0; q < kBT; ++q) t += sm_red[q];
        dal[s * ntile + tile] = t;
    }
}

// ---------------------------------------------------------------- 3. key side
// One workgroup per (K/V slice, 64-key tile); lane group j (four lanes) owns
// key j0 + j. For each query head sharing the K/V slice: the centroid branch
// (all clusters, in chunks of 32) and the local branch (every query whose
// window holds a key of the tile). dmu_part[s, tile, k, :] receives the
// tile's sum_j dSc_kj k_j / 8 for query slice s. Without LOCAL only the
// centroid branch runs and dK, dV (of type TO) hold its share alone.
template <typename T, bool LOCAL, typename TO>
__global__ __launch_bounds__(256) void bwd_key_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx,
    const T *__restrict__ dO, const float *__restrict__ mu, const float *__restrict__ vcent,
    const float *__restrict__ cstat, const float *__restrict__ dvc,
    const float4 *__restrict__ lstat, const uint8_t *__restrict__ valid, int L, int r, int ntile,
    int Kc, float alpha, int H, int G, TO *__restrict__ dK, TO *__restrict__ dV,
    float *__restrict__ dmu_part) {
    __shared__ __align__(16) float sm_k[kBT * kRow];       // this tile's keys (for dmu)
    __shared__ __align__(16) float sm_a[kBT * kRow];       // mu chunk, then query rows
    __shared__ __align__(16) float sm_b[kBT * kRow];       // dVc chunk, then alpha keep dO rows
    __shared__ __align__(16) float sm_ds[kBChunk * kBT];   // dSc of the chunk [k][j]
    __shared__ float sm_st[kBT * 4];          // (m, l, D) per centroid or query
    __shared__ uint8_t sm_kok[kBT];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x % ntile;
    const long skv = blockIdx.x / ntile;
    const int Hkv = H / G;
    const long bb = skv / Hkv;                 // batch row
    const long s0 = bb * H + (skv % Hkv) * G;  // first query slice of the group
    const long kvbase = skv * (long)L * kD;
    const int j0 = tile * kBT, nk = min(kBT, L - j0);
    const int jl = tid >> 2, g = tid & 3;
    const int j = j0 + jl;
    const bool active = jl < nk;
    const float scale = 1.0f / sqrtf((float)kD);

    float kr[16], vr[16], gk[16], gv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) gk[c] = gv[c] = kr[c] = vr[c] = 0.f;
    if (active) {
        load16(Kx + kvbase + (long)j * kD + 16 * g, kr);
        load16(Vx + kvbase + (long)j * kD + 16 * g, vr);
    }
    for (int e = tid; e < nk * (kD / 4); e += 256) {
        const int rr = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
        const float4 kv = load4<T>(Kx + kvbase + (long)(j0 + rr) * kD + c4);
        float *dk = sm_k + rr * kRow + c4;
        dk[0] = kv.x; dk[1] = kv.y; dk[2] = kv.z; dk[3] = kv.w;
    }
    for (int rr = tid; rr < nk; rr += 256) sm_kok[rr] = token_ok(valid, bb, L, j0 + rr);
    const bool kok = active && token_ok(valid, bb, L, j);
    // queries whose window meets the tile
    const int qlo = (int)max(0L, (long)j0 - r);
    const int qhi = (int)min((long)L, (long)j0 + nk + r);   // exclusive

    for (int gi = 0; gi < G; ++gi) {
        const long s = s0 + gi;
        const long base = s * (long)L * kD;
        // ------------------------------------------ centroid branch
        for (int c0 = 0; c0 < Kc; c0 += kBChunk) {
            const int ck = min(kBChunk, Kc - c0);
            __syncthreads();
            for (int e = tid; e < ck * (kD / 4); e += 256) {
                const int k = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
                const float4 mv = load4<float>(mu + (s * Kc + c0 + k) * kD + c4);
                const float4 dv = load4<float>(dvc + (s * Kc + c0 + k) * kD + c4);
                float *da = sm_a + k * kRow + c4;
                float *db = sm_b + k * kRow + c4;
                da[0] = mv.x; da[1] = mv.y; da[2] = mv.z; da[3] = mv.w;
                db[0] = dv.x; db[1] = dv.y; db[2] = dv.z; db[3] = dv.w;
            }
            // D_k = dVc_k . Vc_k, eight lanes per centroid
            {
                const int k = tid >> 3, part = tid & 7;
                float dd = 0.f;
                if (k < ck) {
                    const float *vc = vcent + (s * Kc + c0 + k) * kD + 8 * part;
                    const float *gc = dvc + (s * Kc + c0 + k) * kD + 8 * part;
#pragma unroll
                    for (int e = 0; e < 8; ++e) dd = fmaf(gc[e], vc[e], dd);
                }
                dd = quad_sum(dd);
                dd += __shfl_xor(dd, 4);
                if (k < ck && part == 0) {
                    sm_st[4 * k] = cstat[2 * (s * Kc + c0 + k)];
                    sm_st[4 * k + 1] = 1.0f / cstat[2 * (s * Kc + c0 + k) + 1];
                    sm_st[4 * k + 2] = dd;
                }
            }
            __syncthreads();
            for (int k = 0; k < ck; ++k) {
                const float *mr = sm_a + k * kRow + 16 * g;
                const float *gr = sm_b + k * kRow + 16 * g;
                const float dot = quad_sum(dot16(mr, kr));   // every lane, before any select
                const float dp = quad_sum(dot16(gr, vr));
                const float sc = kok ? dot * scale : -10000.f;
                const float p = active ? exp_f32(sc - sm_st[4 * k]) * sm_st[4 * k + 1] : 0.f;
                const float ds = kok ? p * (dp - sm_st[4 * k + 2]) * scale : 0.f;
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    gk[c] = fmaf(ds, mr[c], gk[c]);
                    gv[c] = fmaf(p, gr[c], gv[c]);
                }
                if (g == 0) sm_ds[k * kBT + jl] = ds;   // 0 for keys past the tile
            }
            __syncthreads();
            // dmu partial of the chunk: [k][t] = sum_j ds[k][j] k_j[t]. Lane t
            // of wave kw sums clusters kw, kw + 4, ...: one read of K feeds all
            // of them, and the wave reads each ds row four keys at a time
            // (ds is 0 for keys past the tile).
            {
                const int t = tid & (kD - 1), kw = tid >> 6;
                float acc[kBChunk / 4];
#pragma unroll
                for (int u = 0; u < kBChunk / 4; ++u) acc[u] = 0.f;
                for (int q = 0; q < nk; q += 4) {
                    float kq[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) kq[i] = q + i < nk ? sm_k[(q + i) * kRow + t] : 0.f;
#pragma unroll
                    for (int u = 0; u < kBChunk / 4; ++u) {
                        if (kw + 4 * u < ck) {
                            const float4 d4 =
                                *reinterpret_cast<const float4 *>(sm_ds + (kw + 4 * u) * kBT + q);
                            acc[u] = fmaf(d4.w, kq[3], fmaf(d4.z, kq[2],
                                          fmaf(d4.y, kq[1], fmaf(d4.x, kq[0], acc[u]))));
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < kBChunk / 4; ++u)
                    if (kw + 4 * u < ck)
                        dmu_part[((s * ntile + tile) * (long)Kc + c0 + kw + 4 * u) * kD + t] = acc[u];
            }
        }
        // ------------------------------------------ local branch
        for (int it = qlo; LOCAL && it < qhi; it += kBT) {
            const int nq = min(kBT, qhi - it);
            __syncthreads();
            for (int e = tid; e < nq * (kD / 4); e += 256) {
                const int rr = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
                const bool keep = token_ok(valid, bb, L, it + rr);
                const float4 qv = load4<T>(Q + base + (long)(it + rr) * kD + c4);
                const float4 gv4 = load4<T>(dO + base + (long)(it + rr) * kD + c4);
                const float w = keep ? alpha : 0.f;
                float *da = sm_a + rr * kRow + c4;
                float *db = sm_b + rr * kRow + c4;
                da[0] = qv.x; da[1] = qv.y; da[2] = qv.z; da[3] = qv.w;
                db[0] = w * gv4.x; db[1] = w * gv4.y; db[2] = w * gv4.z; db[3] = w * gv4.w;
            }
            for (int rr = tid; rr < nq; rr += 256) {
                const float4 st = lstat[s * L + it + rr];
                sm_st[4 * rr] = st.x;
                sm_st[4 * rr + 1] = 1.0f / st.y;
                sm_st[4 * rr + 2] = st.z;
            }
            __syncthreads();
            // queries of this tile inside key j's window, |i - j| <= r
            const int a = active ? (int)max(0L, (long)j - r) - it : 0;
            const int b = active ? (int)min((long)it + nq - 1, (long)j + r) - it : -1;
            const int aa = max(a, 0);
            const int wa = wave_min_i32(aa < b + 1 ? aa : kBT);
            const int wb = wave_max_i32(b);
            for (int q = wa; q <= wb; ++q) {
                const float *qr = sm_a + q * kRow + 16 * g;
                const float *gr = sm_b + q * kRow + 16 * g;
                const float dot = quad_sum(dot16(qr, kr));
                const float dp = quad_sum(dot16(gr, vr));
                const float sc = kok ? dot * scale : -10000.f;
                if (q >= aa && q <= b) {
                    const float p = exp_f32(sc - sm_st[4 * q]) * sm_st[4 * q + 1];
                    const float ds = kok ? p * (dp - sm_st[4 * q + 2]) * scale : 0.f;
#pragma unroll
                    for (int c = 0; c < 16; ++c) {
                        gk[c] = fmaf(ds, qr[c], gk[c]);
                        gv[c] = fmaf(p, gr[c], gv[c]);
                    }
                }
            }
        }
    }
    if (active) {
        store16(dK + kvbase + (long)j * kD + 16 * g, gk);
        store16(dV + kvbase + (long)j * kD + 16 * g, gv);
    }
}

// ---------------------------------------------------------------- 5. query side
template <typename T>
__global__ __launch_bounds__(256) void bwd_query_kernel(
    const T *__restrict__ Q, const T *__restrict__ Kx, const T *__restrict__ Vx,
    const T *__restrict__ dO, const int32_t *__restrict__ assign, const float *__restrict__ dmu,
    const int32_t *__restrict__ counts, const float4 *__restrict__ lstat,
    const uint8_t *__restrict__ valid, int L, int r, int ntile, int Kc, float alpha, int H, int G,
    T *__restrict__ dQ) {
    __shared__ __align__(16) float sm_k[kBT * kRow];
    __shared__ __align__(16) float sm_v[kBT * kRow];
    __shared__ uint8_t sm_ok[kBT];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x % ntile;
    const long s = blockIdx.x / ntile;
    const long base = s * (long)L * kD;
    const long kvbase = kv_slice(s, H, G) * (long)L * kD;
    const int i0 = tile * kBT, nq = min(kBT, L - i0);
    const int qi = tid >> 2, g = tid & 3;
    const int i = i0 + qi;
    const bool active = qi < nq;
    const int lo = (int)max(0L, (long)i - r), hi = (int)min((long)L - 1, (long)i + r);
    const int tlo = (int)max(0L, (long)i0 - r);
    const int thi = (int)min((long)L, (long)i0 + nq + r);
    const float scale = 1.0f / sqrtf((float)kD);

    float qr[16], gr[16], dq[16];
    float m = 0.f, l = 1.f, D = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) qr[c] = gr[c] = dq[c] = 0.f;
    if (active) {
        load16(Q + base + (long)i * kD + 16 * g, qr);
        load16(dO + base + (long)i * kD + 16 * g, gr);
        const float w = token_ok(valid, s / H, L, i) ? alpha : 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            qr[c] *= scale;
            gr[c] *= w;
        }
        const float4 st = lstat[s * L + i];
        m = st.x; l = st.y; D = st.z;
    }
    const float inv = 1.0f / l;
    for (int jt = tlo; jt < thi; jt += kBT) {
        const int nk = min(kBT, thi - jt);
        __syncthreads();
        for (int e = tid; e < nk * (kD / 4); e += 256) {
            const int rr = e / (kD / 4), c4 = (e % (kD / 4)) * 4;
            const float4 kv = load4<T>(Kx + kvbase + (long)(jt + rr) * kD + c4);
            const float4 vv = load4<T>(Vx + kvbase + (long)(jt + rr) * kD + c4);
            float *dk = sm_k + rr * kRow + c4;
            float *dv = sm_v + rr * kRow + c4;
            dk[0] = kv.x; dk[1] = kv.y; dk[2] = kv.z; dk[3] = kv.w;
            dv[0] = vv.x; dv[1] = vv.y; dv[2] = vv.z; dv[3] = vv.w;
        }
        for (int rr = tid; rr < nk; rr += 256) sm_ok[rr] = token_ok(valid, s / H, L, jt + rr);
        __syncthreads();
        const int a = active ? max(lo, jt) - jt : 0;
        const int b = active ? min(hi, jt + nk - 1) - jt : -1;
        const int wa = wave_min_i32(a < b + 1 ? a : kBT);
        const int wb = wave_max_i32(b);
        for (int key = wa; key <= wb; ++key) {
            const float *kk = sm_k + key * kRow + 16 * g;
            const float *vv = sm_v + key * kRow + 16 * g;
            const float sc = quad_sum(dot16(qr, kk));
            const float dp = quad_sum(dot16(gr, vv));
            if (key >= a && key <= b && sm_ok[key]) {
                const float p = exp_f32(sc - m) * inv;
                const float ds = p * (dp - D) * scale;
#pragma unroll
                for (int c = 0; c < 16; ++c) dq[c] = fmaf(ds, kk[c], dq[c]);
            }
        }
    }
    if (!active) return;
    const int c = min(max(assign[s * L + i], 0), Kc - 1);
    const int n = counts[s * Kc + c];
    const float invn = 1.0f / (float)(n > 1 ? n : 1);
    const float *dm = dmu + (s * Kc + c) * kD + 16 * g;
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[e] = fmaf(dm[e], invn, dq[e]);
    store16(dQ + base + (long)i * kD + 16 * g, dq);
}

// ---------------------------------------------------------------- 6. dalpha
__global__ __launch_bounds__(256) void bwd_sum_kernel(const float *__restrict__ part, long n,
                                                      float *__restrict__ out) {
    __shared__ float red[256];
    float acc = 0.f;
    for (long e = threadIdx.x; e < n; e += 256) acc += part[e];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0];
}

// ---------------------------------------------------------------- host side
int bwd_tiles(int L) { return (L + kBT - 1) / kBT; }

template <typename T>
static hipError_t bwd_dispatch(const BwdArgs &a, hipStream_t st) {
    const int ntile = bwd_tiles(a.L);
    const int G = a.H / a.Hkv;
    const long S = (long)a.B * a.H, Skv = (long)a.B * a.Hkv;
    const T *Q = static_cast<const T *>(a.Q), *K = static_cast<const T *>(a.K);
    const T *V = static_cast<const T *>(a.V), *dO = static_cast<const T *>(a.dO);
    const dim3 block(256);
    // 1. dVc
    const size_t lds = sizeof(float) * ((size_t)kBT * kBPad + (size_t)a.Kc * kD) + sizeof(int) * kBT;
    hipError_t e =
        ensure_dynamic_lds(reinterpret_cast<const void *>(bwd_cluster_sum_kernel<T>), (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_cluster_sum_kernel<T>, dim3((unsigned)(S * ntile)), block, lds, st, dO,
                       a.assign, a.valid, a.L, a.Kc, a.H, ntile, a.part);
    const long total = S * a.Kc * kD;
    const dim3 rgrid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(bwd_partial_reduce_kernel, rgrid, block, 0, st, a.part, ntile, a.Kc, total,
                       1.0f - a.alpha, a.dvc);
    // 2. local statistics, dalpha shares
    hipLaunchKernelGGL(bwd_query_stats_kernel<T>, dim3((unsigned)(S * ntile)), block, 0, st, Q, K,
                       V, dO, a.assign, a.vcent, a.valid, a.L, a.r, ntile, a.Kc, a.alpha, a.H, G,
                       a.lstat, a.dal);
    // 3. key side (dK, dV; dmu partials in a.part)
    hipLaunchKernelGGL((bwd_key_kernel<T, true, T>), dim3((unsigned)(Skv * ntile)), block, 0, st, Q, K, V, dO,
                       a.mu, a.vcent, a.cstat, a.dvc, a.lstat, a.valid, a.L, a.r, ntile, a.Kc,
                       a.alpha, a.H, G, static_cast<T *>(a.dK), static_cast<T *>(a.dV), a.part);
    // 4. dmu
    hipLaunchKernelGGL(bwd_partial_reduce_kernel, rgrid, block, 0, st, a.part, ntile, a.Kc, total,
                       1.0f, a.dmu);
    // 5. dQ
    hipLaunchKernelGGL(bwd_query_kernel<T>, dim3((unsigned)(S * ntile)), block, 0, st, Q, K, V, dO,
                       a.assign, a.dmu, a.counts, a.lstat, a.valid, a.L, a.r, ntile, a.Kc, a.alpha,
                       a.H, G, static_cast<T *>(a.dQ));
    // 6. dalpha
    if (a.dalpha)
        hipLaunchKernelGGL(bwd_sum_kernel, dim3(1), block, 0, st, a.dal, S * ntile, a.dalpha);
    return hipGetLastError();
}

hipError_t launch_bwd_sum(const float *part, long n, float *out, hipStream_t st) {
    if (!out) return hipSuccess;
    hipLaunchKernelGGL(bwd_sum_kernel, dim3(1), dim3(256), 0, st, part, n, out);
    return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs &a, ca_dtype_t dt, hipStream_t st) {
    if (dt == CA_BF16) return bwd_dispatch<bf16_t>(a, st);
    return bwd_dispatch<float>(a, st);
}

}  // namespace ca
