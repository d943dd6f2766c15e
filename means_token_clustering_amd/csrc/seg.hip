// Single-launch cluster attention forward for long slices: each slice is split
// into NS segments of at most 480 tokens, one workgroup of 16 waves per
// segment, all workgroups of the launch resident at once (one per compute
// unit). K <= 64 clusters, window radius <= 16, no key-padding mask and none
// of the listing variants.
//
// Method: model card "Hooshaai/distilbert-sst2-cluster-attention",
// Architecture Overview figure and Mathematical Formulation 1; "ClusterFormer"
// spec (svd-sst2-roberta-cluster page) 2.1 and 3: mu^(0)_k = Q[floor(k L / K)];
// for t = 1..I, c_i = argmin_k ||q_i - mu_k||^2 (lowest k on ties) and mu_k =
// sum_{c_i = k} q_i / max(1, n_k) (empty -> zero vector); V^cent_k =
// softmax_j(mu_k . k_j / sqrt(d)) over all keys, times V; O_i = (1 - alpha)
// V^cent_{c_i} + alpha sum_{|i - j| <= r} softmax_j(q_i . k_j / sqrt(d)) v_j.
//
// Phases of workgroup (s, j), which owns tokens [j T, j T + T) of slice s:
//   0. Its Q rows go to LDS as fp16 h/m planes (they stay for all Lloyd
//      iterations) and to the waves' registers as B fragments; the largest
//      |q| of the segment meets the others' at the first slice barrier, so
//      that every segment scales Q by the same power of two (the centroids,
//      means of Q rows, then fit the same range).
//   1. Per Lloyd iteration: the distance chain of the other single-launch
//      kernels for up to four 16-cluster groups (running best over the
//      groups, lowest index on ties), then the segment's cluster sums as
//      one-hot products (fragments built in registers from the assignments)
//      written to the workspace, a slice barrier, and the update: either
//      every workgroup adds the NS segment sums in segment order (NS <= 4),
//      or workgroup j adds them for clusters k = j mod NS and, after a second
//      barrier, every workgroup reads the new centroids. Both give every
//      workgroup the same fp32 centroids, hence the same planes.
//   2. Centroid attention over the segment's keys in chunks of 128 (K, V
//      planes per chunk), a running (max, sum, row) per centroid row, written
//      as the segment's partial; after a barrier the NS partials merge in
//      segment order (one- or two-level as the update), giving
//      (1 - alpha) V^cent in an LDS table.
//   3. The window branch for the segment's queries in passes of up to 256
//      (halo keys read from the neighbouring segments' rows), the gather from
//      the table and the fused row stores.
// The slice barriers count arrivals in a workspace word per slice (each on
// its own 256-byte line) that a small kernel zeroes before the launch. Every
// value that crosses workgroups (segment maxima, sums, attention partials,
// reduced rows) is written and read only with device-scope atomic stores and
// loads, which are coherent across the XCDs' separate L2 caches; a writer's
// stores complete (s_waitcnt vmcnt(0)) before its arrival is counted, and
// readers load only after the count is reached. No plain global data crosses
// workgroups, so no L2 write-back or invalidate is needed (a fenced barrier
// measured 3-13 us here, this one about 1 us). Every wait is bounded, so the
// launch ends even if the co-residency it relies on were not given (the host
// only launches grids of at most one workgroup per compute unit).
//
// Arithmetic as in the other single-launch kernels (power-of-two range
// scaling, the fp16 h/m split, three partial products, base-2 softmax).
#include "launch.h"
#include "mfma_split.h"

namespace ca {
namespace {

constexpr int kSegMax = 480;                      // tokens per workgroup
constexpr int kSegTiles = kSegMax / 16;           // 30
constexpr int kSegThreads = 1024;                 // 16 waves
constexpr int kSegK = 64;                         // max clusters
constexpr int kSQPlane = kSegMax * kD * 2;        // fp16 plane [480][64]
constexpr int kSMuPlane = kSegK * kD * 2;         // fp16 plane [64][64]
constexpr int kSMuXCols = 32;                     // [64][32] fp16: -||mu||^2/2 parts
constexpr int kSRows3 = 288;                      // phase 3: 256 queries + two halos
constexpr int kS3Plane = kSRows3 * kD * 2;        // fp16 plane [288][64]
// LDS map (bytes); region R at 0 is reused by the phases
constexpr int kSOffMu = 2 * kSQPlane;                     // 122,880: [64][64] h, m
constexpr int kSOffMuX = kSOffMu + 2 * kSMuPlane;         // [64][32] fp16
constexpr int kSOffComb = kSOffMuX + kSegK * kSMuXCols * 2;   // spare (segment-sum scratch)
constexpr int kSOffC = kSOffComb + 3 * 4 * 64 * 5 * 4;    // [480] assignments (bytes, K <= 64)
constexpr int kSOffMax = kSOffC + kSegMax;                // [16][4] words
constexpr int kSLds = kSOffMax + 16 * 4 * 4;
// phase 2 inside R: chunk K planes [0, 2 kPlane), V planes [2 kPlane, 4 kPlane),
// P planes (four groups) then the per-wave row maxima and sums
constexpr int kSOffP = 4 * kPlane;
constexpr int kSOffXm = kSOffP + 4 * 2 * kPlaneRow;
constexpr int kSOffXl = kSOffXm + kSegK * 8 * 4;
static_assert(kSOffXl + kSegK * 8 * 4 <= kSOffMu, "phase 2 fits below the centroid planes");
static_assert(4 * kS3Plane + kFK * 2 * kD * 4 <= kSOffComb + 3 * 4 * 64 * 5 * 4,
              "phase 3 planes and a 32-row table fit below the assignments");
static_assert(4 * (kS3Plane - 16 * kD * 2) + kSegK * kD * 4 <= kSOffC,
              "phase 3 planes of 272 rows and a 64-row table fit below the assignments");
static_assert(kSLds <= 163840, "one workgroup per CU");
// segment-sum scratch in [kSOffMu, kSOffC), 64 lanes x 5 floats per entry:
// NG <= 2: 3 parts x 4 dim tiles x 2 groups; NG >= 3: 1 part x 8 (group pair,
// dim tile) slots x 2 groups
static_assert(3 * 4 * 2 * 64 * 5 * 4 <= kSOffC - kSOffMu, "segment-sum scratch fits (NG <= 2)");
static_assert(1 * 8 * 2 * 64 * 5 * 4 <= kSOffC - kSOffMu, "segment-sum scratch fits (NG >= 3)");

constexpr int kSpinLimit = 1 << 18;   // polls of one barrier wait before giving up (about 0.3 s)
constexpr int kBarStride = 64;        // words from one slice's counter to the next (256 B)

// device-scope atomic store / load of one value that crosses workgroups
__device__ __forceinline__ void st_shared(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_shared(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One barrier of slice s: every device-scope atomic store (st_shared) made by
// the slice's workgroups before it is visible to their device-scope atomic
// loads (ld_shared) after it. Each wave first waits for its own stores to
// complete (what a release amounts to for atomic-only data); thread 0 then
// counts the workgroup's arrival in bar (zero at launch) and polls it: the
// b-th barrier (b = 1, 2, ...) is passed once it holds b * ns. A wait that
// exceeds kSpinLimit polls (about 7 ms) sets *err and returns.
__device__ __forceinline__ void slice_barrier(uint32_t *bar, int b, int ns, uint32_t *err) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t target = (uint32_t)b * (uint32_t)ns;
        int polls = 0;
        while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(1);
            if (++polls > kSpinLimit) {
                __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// (score, index) maximum over the four lane groups of a column, lowest index
// among equal scores; both the score and the index are returned.
__device__ __forceinline__ void col_argmax2(float &best, int &bk) {
    uint32_t a, b, ia, ib;
    pair16(__float_as_uint(best), a, b);
    pair16((uint32_t)bk, ia, ib);
    bool up = __uint_as_float(b) > __uint_as_float(a);
    best = up ? __uint_as_float(b) : __uint_as_float(a);
    bk = up ? (int)ib : (int)ia;
    pair32(__float_as_uint(best), a, b);
    pair32((uint32_t)bk, ia, ib);
    up = __uint_as_float(b) > __uint_as_float(a);
    best = up ? __uint_as_float(b) : __uint_as_float(a);
    bk = up ? (int)ib : (int)ia;
}

}  // namespace

// Arguments of one launch (host-filled).
struct SegArgs {
    const void *Q, *K, *V;
    int L, Kc, iters, rad;
    float alpha;
    int init_step, H, G;
    void *out;
    int32_t *assign, *hist;
    long S;
    int ns, seg;            // segments per slice, tokens per segment (multiple of 16)
    int two_level;          // update and merge through owner workgroups
    float *part;            // [2][S][ns][Kc][kXPartStride] segment sums / attention partials
    float *rows;            // [S][Kc][64] reduced rows (two-level)
    uint32_t *bar;          // [S + 1][kBarStride]: arrival counters (zeroed before the launch), error word
};

__global__ void seg_zero_kernel(uint32_t *words, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) words[i] = 0u;
}

template <typename T, bool HIST>
__global__ __launch_bounds__(kSegThreads, 1) void cluster_attn_seg_kernel(SegArgs a) {
    __shared__ __align__(16) unsigned char smem[kSLds];
    uint16_t *sQ = reinterpret_cast<uint16_t *>(smem);
    uint16_t *sMu = reinterpret_cast<uint16_t *>(smem + kSOffMu);
    uint16_t *sMuX = reinterpret_cast<uint16_t *>(smem + kSOffMuX);
    uint8_t *sC = smem + kSOffC;
    uint32_t *sMax = reinterpret_cast<uint32_t *>(smem + kSOffMax);
    const u8 *pQ = smem, *pMu = smem + kSOffMu, *pMuX = smem + kSOffMuX;

    const T *Q = static_cast<const T *>(a.Q);
    const T *Kx = static_cast<const T *>(a.K);
    const T *Vx = static_cast<const T *>(a.V);
    const int L = a.L, Kc = a.Kc, ns = a.ns, T_ = a.seg;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const long s = blockIdx.x / ns;
    const int j = blockIdx.x % ns;
    const int seg0 = j * T_;                          // first token of the segment
    const int Ls = max(0, min(T_, L - seg0));          // tokens of the segment
    const int NTs = (Ls + 15) >> 4;                    // its tiles
    const int NG = (Kc + 15) >> 4;                     // groups of 16 clusters
    const long base = s * (long)L * kD;
    const long kvbase = kv_slice(s, a.H, a.G) * (long)L * kD;
    const T *Qs = Q + base;
    uint32_t *bar = a.bar + s * kBarStride;
    uint32_t *err = a.bar + a.S * kBarStride;
    const LaneOffs lo = lane_offsets(l16, g);
    int nbar = 0;   // slice barriers passed

    // the part buffer of parity p: [S][ns][Kc][kXPartStride]
    auto part_at = [&](int p, int seg, int k) -> float * {
        return a.part + ((((long)p * a.S + s) * ns + seg) * (long)Kc + k) * kXPartStride;
    };

    // ============================================================ 0. Q
    float qraw[2][2][8];   // tiles w and w + 16 of the segment
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c)
            load_row8<T, false>(Qs + (long)seg0 * kD, 16 * (w + 16 * u) + l16, Ls, 32 * c + 8 * g,
                                qraw[u][c]);
    {
        float m = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) m = absmax8(qraw[u][1], absmax8(qraw[u][0], m));
        const uint32_t b = wave_max_u(__float_as_uint(m));
        if (lane == 0) sMax[w] = b;
    }
    __syncthreads();
    if (tid == 0) {   // the segment's largest |q| (bits) for the others
        uint32_t m = 0;
#pragma unroll
        for (int ww = 0; ww < 16; ++ww) m = max(m, sMax[ww]);
        __hip_atomic_store(reinterpret_cast<uint32_t *>(part_at(0, j, 0)), m, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);   // buffer 0: iteration 1 writes buffer 1
    }
    slice_barrier(bar, ++nbar, ns, err);
    int sq;
    {
        uint32_t m = 0;
        for (int j0 = 0; j0 < ns; j0 += 8) {   // eight loads in flight
            uint32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = __hip_atomic_load(reinterpret_cast<uint32_t *>(part_at(0, min(j0 + u, ns - 1), 0)),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < 8; ++u) m = max(m, v[u]);
        }
        sq = scale_shift(m, kQLimit);
    }
    const float fq = __builtin_ldexpf(1.f, -sq);
    // Q planes (zeros past the segment's tokens); the distance step reads its
    // B fragments back from them, which frees the registers for the loop
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = qraw[u][c][i] * fq;
            const Sp8 qp = split8(x);
            if (w + 16 * u < kSegTiles) {
                const int o = (2048 * (w + 16 * u) + (lo.rl64 ^ (64 * c))) / 2;
                st16(sQ + o, qp.h);
                st16(sQ + kSQPlane / 2 + o, qp.m);
            }
        }

    // centroid rows -> planes and norm parts (rows >= Kc: zero with a -inf part);
    // thread t: row t / 16, dims 4 (t % 16) ..; x already in scaled units
    auto store_mu = [&](const float *x4) {
        const int r = tid >> 4, c4 = 4 * (tid & 15);
        float x[4] = {x4[0], x4[1], x4[2], x4[3]};
        if (r >= Kc) x[0] = x[1] = x[2] = x[3] = 0.f;
        const Sp4 mp = split4(x[0], x[1], x[2], x[3]);
        const int o = off64(r, c4);
        st8(sMu + o, mp.h);
        st8(sMu + kSMuPlane / 2 + o, mp.m);
        float n2 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) n2 = fmaf(x[i], x[i], n2);
        n2 += __shfl_xor(n2, 1);
        n2 += __shfl_xor(n2, 2);
        n2 += __shfl_xor(n2, 4);
        n2 += __shfl_xor(n2, 8);
        uint32_t v = 0;
        if ((tid & 15) == 0) {
            uint32_t h = 0, m = 0;
            if (r < Kc) split2(-0.5f * n2, 0.f, h, m);
            v = r < Kc ? ((h & 0xffffu) | ((m & 0xffffu) << 16)) : (uint32_t)kNegInfH;
        }
        *reinterpret_cast<uint32_t *>(sMuX + r * kSMuXCols + 2 * (tid & 15)) = v;
    };
    {   // mu^(0) = Q[init_row(k)]
        const int r = tid >> 4, c4 = 4 * (tid & 15);
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (r < Kc) {
            const float4 v = load4<T>(Qs + (long)init_row(r, L, Kc, a.init_step) * kD + c4);
            x[0] = v.x * fq; x[1] = v.y * fq; x[2] = v.z * fq; x[3] = v.w * fq;
        }
        store_mu(x);
    }
    __syncthreads();

    // ============================================================ 1. Lloyd
    const u32x4_t ones_g0 =
        g == 0 ? u32x4_t{kOneH2, kOneH2, kOneH2, kOneH2} : u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t ones = {kOneH2, kOneH2, kOneH2, kOneH2};
    // segment-sum work split: wave w takes dimension tile dt = w & 3 and
    // reads each Q^T fragment and each assignment word of its chunks once for
    // several cluster groups: for NG <= 2 all groups over chunk part w >> 2 of
    // four, for NG >= 3 groups 2 (w >> 3) and 2 (w >> 3) + 1 over chunk part
    // (w >> 2) & 1 of two; the parts meet in a fixed order through LDS.
    const int dt = w & 3;
    const bool wide = NG >= 3;
    const int nparts = wide ? 2 : 4;
    const int part = wide ? (w >> 2) & 1 : w >> 2;
    const int kg0 = wide ? 2 * (w >> 3) : 0;           // first group of the wave
    const int ngw = wide ? min(2, NG - kg0) : NG;      // its groups (0 .. 2)
    float *sPart = reinterpret_cast<float *>(smem + kSOffMu);   // dead between assign and update
    const int trq0 = 1024 * g + (lo.tr0 ^ (32 * dt)), trq1 = 1024 * g + (lo.tr4 ^ (32 * dt));
    const int NCH = (Ls + 31) >> 5;
    const float back = __builtin_ldexpf(1.f, sq);
    for (int t = 1; t <= a.iters; ++t) {
        // ---------------------------------------------------- assignment
        {
            // the wave's tiles w and w + 16; each group's centroid fragments
            // are read once for both
            const bool on1 = w + 16 < NTs;
            float run[2] = {-__builtin_inff(), -__builtin_inff()};
            int rk[2] = {0, 0};
            if (w < NTs) {
                Sp8 qf[2][2];   // the tiles' Q fragments, from the planes
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        qf[u][c] = frag_at(pQ, kSQPlane, 2048 * (u == 1 && on1 ? w + 16 : w) +
                                                             (lo.rl64 ^ (64 * c)));
                for (int kg = 0; kg < NG; ++kg) {
                    const u32x4_t mx = ldb16(pMuX, 64 * (16 * kg + l16) + 16 * g);
                    const Sp8 mu0 = frag_at(pMu, kSMuPlane, 2048 * kg + lo.rl64);
                    const Sp8 mu1 = frag_at(pMu, kSMuPlane, 2048 * kg + (lo.rl64 ^ 64));
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        if (u == 1 && !on1) break;
                        f32x4_t sc = mma(mx, ones_g0, kZero4);
                        sc = mma3(mu0, qf[u][0], sc);
                        sc = mma3(mu1, qf[u][1], sc);
                        float best = sc[0];
                        int bk = 16 * kg + 4 * g;
#pragma unroll
                        for (int rr = 1; rr < 4; ++rr) {
                            const bool up = sc[rr] > best;
                            best = up ? sc[rr] : best;
                            bk = up ? 16 * kg + 4 * g + rr : bk;
                        }
                        col_argmax2(best, bk);
                        if (kg == 0 || best > run[u]) {   // an earlier group keeps equal scores
                            run[u] = best;
                            rk[u] = bk;
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tok = 16 * (w + 16 * u) + l16;
                if (g == 0 && tok < Ls) {
                    sC[tok] = (uint8_t)rk[u];
                    const long gi = s * (long)L + seg0 + tok;
                    if (t == a.iters && a.assign) a.assign[gi] = rk[u];
                    if (HIST) a.hist[(long)(t - 1) * a.S * L + gi] = rk[u];
                }
            }
        }
        __syncthreads();
        // ---------------------------------------------------- segment sums
        // acc[u]: sums of dims 16 dt + 4 g + rr of cluster 16 (kg0 + u) + l16
        // (the h and m parts accumulate in one chain); cnt[u]: its size
        f32x4_t acc[2] = {kZero4, kZero4}, cnt[2] = {kZero4, kZero4};
        for (int cc = part; cc < NCH; cc += nparts) {
            const int t0 = 32 * cc + 8 * g;
            const uint2 cw = *reinterpret_cast<const uint2 *>(sC + t0);
            const Sp8 qt = colfrag8_at<kSQPlane>(pQ, 4096 * cc + trq0, 4096 * cc + trq1);
            int cv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cv[e] = t0 + e < Ls ? (int)((cw.x >> (8 * e)) & 0xff) : -1;
                cv[4 + e] = t0 + 4 + e < Ls ? (int)((cw.y >> (8 * e)) & 0xff) : -1;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u < ngw) {
                    const int kcl = 16 * (kg0 + u) + l16;   // this lane's cluster
                    uint32_t pk[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pk[e] = (cv[2 * e] == kcl ? 0x3c00u : 0u) |
                                ((cv[2 * e + 1] == kcl ? 0x3c00u : 0u) << 16);
                    const u32x4_t oh = {pk[0], pk[1], pk[2], pk[3]};
                    acc[u] = mma(qt.m, oh, acc[u]);
                    acc[u] = mma(qt.h, oh, acc[u]);
                    if (dt == 0) cnt[u] = mma(ones, oh, cnt[u]);
                }
            }
        }
        // parts 1 .. nparts - 1 leave (sums, size) per group; part 0 adds them in order
        const int nslots = wide ? 8 : 4;
        const int slot = wide ? (w >> 3) * 4 + dt : dt;   // waves sharing groups and dt
        if (part > 0) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u < ngw) {
                    float *pp = sPart + ((((part - 1) * nslots + slot) * 2 + u) * 64 + lane) * 5;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) pp[rr] = acc[u][rr];
                    pp[4] = cnt[u][0];
                }
            }
        }
        __syncthreads();
        const int pb = t & 1;   // part buffer of this iteration
        if (part == 0) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u < ngw) {
                    float v[4], n = cnt[u][0];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) v[rr] = acc[u][rr];
                    for (int q2 = 1; q2 < nparts; ++q2) {
                        const float *pp = sPart + ((((q2 - 1) * nslots + slot) * 2 + u) * 64 + lane) * 5;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) v[rr] += pp[rr];
                        n += pp[4];
                    }
                    const int k = 16 * (kg0 + u) + l16;
                    if (k < Kc) {
                        float *pp = part_at(pb, j, k);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            st_shared(pp + 16 * dt + 4 * g + rr, v[rr] * back);
                        if (dt == 0 && g == 0) st_shared(pp + kD, n);
                    }
                }
            }
        }
        __syncthreads();   // the part scratch is read before the planes are rewritten
        slice_barrier(bar, ++nbar, ns, err);
        // ---------------------------------------------------- update
        if (!a.two_level) {
            // every workgroup: the ns segment sums in segment order
            const int r = tid >> 4, c4 = 4 * (tid & 15);
            float x[4] = {0.f, 0.f, 0.f, 0.f};
            if (r < Kc) {
                float n = 0.f, v[4][5];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {   // ns <= 4 here: every load in flight
                    const float *pp = part_at(pb, min(jj, ns - 1), r);
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[jj][i] = ld_shared(pp + c4 + i);
                    v[jj][4] = ld_shared(pp + kD);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {   // segment order
                    if (jj < ns) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) x[i] += v[jj][i];
                        n += v[jj][4];
                    }
                }
                const float dn = fmaxf(n, 1.f);
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = x[i] / dn * fq;
            }
            store_mu(x);
        } else {
            // owner workgroups: clusters k = j, j + ns, ... (at most 16 rows)
            {
                const int rr = tid >> 6, d = tid & 63;
                const int k = j + ns * rr;
                if (k < Kc) {
                    float sum = 0.f, n = 0.f;
                    for (int j0 = 0; j0 < ns; j0 += 8) {   // eight segments in flight
                        float v[8], c[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const float *pp = part_at(pb, min(j0 + u, ns - 1), k);
                            v[u] = ld_shared(pp + d);
                            c[u] = ld_shared(pp + kD);
                        }
#pragma unroll
                        for (int u = 0; u < 8; ++u) {   // segment order
                            if (j0 + u < ns) {
                                sum += v[u];
                                n += c[u];
                            }
                        }
                    }
                    st_shared(a.rows + (s * Kc + k) * kD + d, sum / fmaxf(n, 1.f));
                }
            }
            slice_barrier(bar, ++nbar, ns, err);
            const int r = tid >> 4, c4 = 4 * (tid & 15);
            float x[4] = {0.f, 0.f, 0.f, 0.f};
            if (r < Kc) {
                const float *pr = a.rows + (s * Kc + r) * kD + c4;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = ld_shared(pr + i) * fq;
            }
            store_mu(x);
        }
        __syncthreads();
    }

    // ============================================================ 2. centroid attention
    // over the segment's keys in chunks of 128; wave w scores key tile w % 8
    // against groups w / 8 and w / 8 + 2; PV unit (dim tile w & 3, group w >> 2)
    // keeps the running (max, sum, row) of its 16 centroid rows
    const int pbx = (a.iters + 1) & 1;   // the part buffer not read last
    {
        uint16_t *cK = reinterpret_cast<uint16_t *>(smem), *cV = cK + kPlane;   // h, m pairs
        const u8 *pK = smem, *pV = smem + 2 * kPlane, *pP = smem + kSOffP;
        float *xm = reinterpret_cast<float *>(smem + kSOffXm);
        float *xl = reinterpret_cast<float *>(smem + kSOffXl);
        const int nchk = (Ls + 127) >> 7;
        const int kt = w & 7;
        const int pdt = w & 3, pkg = w >> 2;   // PV unit
        const bool pv_on = pkg < NG;
        const int trc0 = 1024 * g + (lo.tr0 ^ (32 * pdt)), trc1 = 1024 * g + (lo.tr4 ^ (32 * pdt));
        float kraw[8], vraw[8];
        auto load_chunk = [&](int ch) {   // thread t: row t / 8 of the chunk, dims 8 (t % 8) ..
            const int j0 = seg0 + 128 * ch, nk = min(128, seg0 + Ls - j0);
            load_row8<T, false>(Kx + kvbase + (long)j0 * kD, tid >> 3, nk, (tid & 7) * 8, kraw);
            load_row8<T, false>(Vx + kvbase + (long)j0 * kD, tid >> 3, nk, (tid & 7) * 8, vraw);
        };
        if (nchk > 0) load_chunk(0);
        float Mr = -__builtin_inff(), lr = 0.f;
        f32x4_t ar = kZero4;
        for (int ch = 0; ch < nchk; ++ch) {
            const int nk = min(128, Ls - 128 * ch);
            {
                const uint32_t bk = wave_max_u(__float_as_uint(absmax8(kraw, 0.f)));
                const uint32_t bv = wave_max_u(__float_as_uint(absmax8(vraw, 0.f)));
                if (lane == 0) {
                    sMax[4 * w + 1] = bk;
                    sMax[4 * w + 2] = bv;
                }
            }
            __syncthreads();
            uint32_t mk = 0, mv = 0;
#pragma unroll
            for (int ww = 0; ww < 16; ++ww) {
                mk = max(mk, sMax[4 * ww + 1]);
                mv = max(mv, sMax[4 * ww + 2]);
            }
            const int sk = scale_shift(mk, kKVLimit), sv = scale_shift(mv, kKVLimit);
            {
                const float fk = __builtin_ldexpf(1.f, -sk), fv = __builtin_ldexpf(1.f, -sv);
                float x[8], y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[i] = kraw[i] * fk;
                    y[i] = vraw[i] * fv;
                }
                const Sp8 kp = split8(x), vp = split8(y);
                const int o = off64(tid >> 3, (tid & 7) * 8);
                st16(cK + o, kp.h);
                st16(cK + kPlaneE + o, kp.m);
                st16(cV + o, vp.h);
                st16(cV + kPlaneE + o, vp.m);
            }
            if (ch + 1 < nchk) load_chunk(ch + 1);   // arrives during this chunk
            __syncthreads();
            const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;
            float sx[2][4];
            {
                const Sp8 ka = frag_at(pK, kPlane, 2048 * kt + lo.rl64);
                const Sp8 kc = frag_at(pK, kPlane, 2048 * kt + (lo.rl64 ^ 64));
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int kg = (w >> 3) + 2 * h2;
                    if (kg < NG) {
                        const Sp8 ma = frag_at(pMu, kSMuPlane, 2048 * kg + lo.rl64);
                        const Sp8 mc = frag_at(pMu, kSMuPlane, 2048 * kg + (lo.rl64 ^ 64));
                        f32x4_t sc = mma3(ka, ma, kZero4);
                        sc = mma3(kc, mc, sc);
                        float mloc = -__builtin_inff();
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int key = 16 * kt + 4 * g + rr;
                            sx[h2][rr] = key < nk ? sc[rr] * sscale2 : -__builtin_inff();
                            mloc = fmaxf(mloc, sx[h2][rr]);
                        }
                        mloc = col_max(mloc);
                        if (g == 0) xm[(16 * kg + l16) * 8 + kt] = mloc;
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int kg = (w >> 3) + 2 * h2;
                if (kg < NG) {
                    const int row = 16 * kg + l16;
                    const float4 m0 = *reinterpret_cast<const float4 *>(xm + row * 8);
                    const float4 m1 = *reinterpret_cast<const float4 *>(xm + row * 8 + 4);
                    const float M = fmaxf(fmaxf(fmaxf(m0.x, m0.y), fmaxf(m0.z, m0.w)),
                                          fmaxf(fmaxf(m1.x, m1.y), fmaxf(m1.z, m1.w)));
                    float p[4], ls = 0.f;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        p[rr] = __builtin_amdgcn_exp2f(sx[h2][rr] - M);   // exp2(-inf) = 0
                        ls += p[rr];
                    }
                    ls = col_sum(ls);
                    const Sp4 ps = split4(p[0], p[1], p[2], p[3]);
                    uint16_t *cP = reinterpret_cast<uint16_t *>(smem + kSOffP + kg * 2 * kPlaneRow);
                    const int o = off128(l16, 16 * kt + 4 * g);
                    st8(cP + o, ps.h);
                    st8(cP + kPlaneRowE + o, ps.m);
                    if (g == 0) xl[row * 8 + kt] = ls;
                }
            }
            __syncthreads();
            if (pv_on) {
                const int nc32 = (nk + 31) >> 5;
                const u8 *pPg = pP + pkg * 2 * kPlaneRow;
                f32x4_t a2[2] = {kZero4, kZero4};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (c < nc32) {
                        const Sp8 vf = colfrag8_at(pV, 4096 * c + trc0, 4096 * c + trc1);
                        const Sp8 pf = frag_at(pPg, kPlaneRow, lo.rl128 ^ (64 * c));
                        a2[c & 1] = mma3(vf, pf, a2[c & 1]);
                    }
                }
                const int row = 16 * pkg + l16;
                const float4 m0 = *reinterpret_cast<const float4 *>(xm + row * 8);
                const float4 m1 = *reinterpret_cast<const float4 *>(xm + row * 8 + 4);
                const float M = fmaxf(fmaxf(fmaxf(m0.x, m0.y), fmaxf(m0.z, m0.w)),
                                      fmaxf(fmaxf(m1.x, m1.y), fmaxf(m1.z, m1.w)));
                const float4 l0 = *reinterpret_cast<const float4 *>(xl + row * 8);
                const float4 l1 = *reinterpret_cast<const float4 *>(xl + row * 8 + 4);
                const float den = ((((((l0.x + l0.y) + l0.z) + l0.w) + l1.x) + l1.y) + l1.z) + l1.w;
                const f32x4_t ac = (a2[0] + a2[1]) * __builtin_ldexpf(1.f, sv);   // real units
                if (ch == 0) {
                    Mr = M;
                    lr = den;
                    ar = ac;
                } else {
                    const float Mn = fmaxf(Mr, M);
                    const float fa = __builtin_amdgcn_exp2f(Mr - Mn), fb = __builtin_amdgcn_exp2f(M - Mn);
                    lr = lr * fa + den * fb;
                    ar = ar * fa + ac * fb;
                    Mr = Mn;
                }
            }
            __syncthreads();   // the chunk planes are rewritten next
        }
        // the segment's partial: row (unnormalised), base-2 maximum, sum
        if (pv_on) {
            const int k = 16 * pkg + l16;
            if (k < Kc) {
                float *pp = part_at(pbx, j, k);
                if (nchk == 0) {   // an empty segment: no keys, zero weight
                    Mr = -__builtin_inff();
                    lr = 0.f;
                    ar = kZero4;
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) st_shared(pp + 16 * pdt + 4 * g + rr, ar[rr]);
                if (pdt == 0 && g == 0) {
                    st_shared(pp + kD, Mr);
                    st_shared(pp + kD + 1, lr);
                }
            }
        }
    }
    slice_barrier(bar, ++nbar, ns, err);
    // merge in segment order: V^cent = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j,
    // kept as (1 - alpha) V^cent in the LDS table
    const int pq = Kc > 32 ? 240 : 256;   // queries per pass of phase 3
    const int rows3 = pq + 32;
    float *sTab = reinterpret_cast<float *>(smem + 4 * rows3 * kD * 2);   // after the pass planes
    const float wg = 1.0f - a.alpha;
    auto merge_row = [&](int k, int d0, int nd, float *dst) {   // dims d0 .. d0 + nd - 1
        // pass 1: the largest maximum; pass 2: the weighted sums in segment
        // order; eight segments in flight per batch
        float M = -__builtin_inff();
        for (int j0 = 0; j0 < ns; j0 += 8) {
            float m8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) m8[u] = ld_shared(part_at(pbx, min(j0 + u, ns - 1), k) + kD);
#pragma unroll
            for (int u = 0; u < 8; ++u) M = fmaxf(M, m8[u]);
        }
        float den = 0.f, num[4] = {0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < ns; j0 += 8) {
            float m8[8], l8[8], a8[8][4];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float *pp = part_at(pbx, min(j0 + u, ns - 1), k);
                m8[u] = ld_shared(pp + kD);
                l8[u] = ld_shared(pp + kD + 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) a8[u][i] = i < nd ? ld_shared(pp + d0 + i) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u < ns) {
                    const float e = __builtin_amdgcn_exp2f(m8[u] - M);   // 0: empty segment
                    den = fmaf(e, l8[u], den);
#pragma unroll
                    for (int i = 0; i < 4; ++i) num[i] = fmaf(e, a8[u][i], num[i]);
                }
            }
        }
        const float f = wg / den;
        for (int i = 0; i < nd; ++i) dst[i] = num[i] * f;   // nd <= 4
    };
    if (!a.two_level) {
        const int r = tid >> 4, c4 = 4 * (tid & 15);
        if (r < Kc) {
            float v[4];
            merge_row(r, c4, 4, v);
            *reinterpret_cast<float4 *>(sTab + r * kD + c4) = make_float4(v[0], v[1], v[2], v[3]);
        }
    } else {
        {
            const int rr = tid >> 6, d = tid & 63;
            const int k = j + ns * rr;
            if (k < Kc) {
                float v;
                merge_row(k, d, 1, &v);
                st_shared(a.rows + (s * Kc + k) * kD + d, v);
            }
        }
        slice_barrier(bar, ++nbar, ns, err);
        const int r = tid >> 4, c4 = 4 * (tid & 15);
        if (r < Kc) {
            const float *pr = a.rows + (s * Kc + r) * kD + c4;
            *reinterpret_cast<float4 *>(sTab + r * kD + c4) =
                make_float4(ld_shared(pr), ld_shared(pr + 1), ld_shared(pr + 2), ld_shared(pr + 3));
        }
    }
    __syncthreads();

    // ============================================================ 3. local window + output
    {
        T *out = static_cast<T *>(a.out);
        const int plane3 = rows3 * kD * 2;   // bytes of one plane of this pass size
        uint16_t *tK = reinterpret_cast<uint16_t *>(smem);
        uint16_t *tV = tK + plane3;          // h, m planes of K, then of V
        const u8 *pK3 = smem, *pV3 = smem + 2 * plane3;
        const int trv = 1024 * (g >> 1) + ((g & 1) ? lo.tr4 : lo.tr0);
        constexpr int kItems = (kSRows3 * kD / 8 + kSegThreads - 1) / kSegThreads;   // 3
        KeyBits kb;
#pragma unroll
        for (int k = 0; k < 4; ++k) kb.w[k] = ~0u;
        for (int p = 0; p * pq < Ls; ++p) {
            const int q0 = seg0 + pq * p;                 // first query of the pass
            const int nq = min(pq, seg0 + Ls - q0);       // its queries
            const int r0 = q0 == 0 ? 0 : q0 - 16;         // first staged row
            const int Lp = min(L, q0 + nq + 16) - r0;     // staged rows holding keys
            const int NTp = (Lp + 15) >> 4;
            float kraw[kItems][8], vraw[kItems][8];
#pragma unroll
            for (int n = 0; n < kItems; ++n) {
                const int it = tid + kSegThreads * n;
                if (it < rows3 * kD / 8) {
                    load_row8<T, false>(Kx + kvbase + (long)r0 * kD, it >> 3, Lp, (it & 7) * 8, kraw[n]);
                    load_row8<T, false>(Vx + kvbase + (long)r0 * kD, it >> 3, Lp, (it & 7) * 8, vraw[n]);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) kraw[n][i] = vraw[n][i] = 0.f;
                }
            }
            {
                float mk = 0.f, mv = 0.f;
#pragma unroll
                for (int n = 0; n < kItems; ++n) {
                    mk = absmax8(kraw[n], mk);
                    mv = absmax8(vraw[n], mv);
                }
                const uint32_t bk = wave_max_u(__float_as_uint(mk));
                const uint32_t bv = wave_max_u(__float_as_uint(mv));
                if (lane == 0) {
                    sMax[4 * w + 1] = bk;
                    sMax[4 * w + 2] = bv;
                }
            }
            __syncthreads();
            uint32_t mk = 0, mv = 0;
#pragma unroll
            for (int ww = 0; ww < 16; ++ww) {
                mk = max(mk, sMax[4 * ww + 1]);
                mv = max(mv, sMax[4 * ww + 2]);
            }
            const int sk = scale_shift(mk, kKVLimit), sv = scale_shift(mv, kKVLimit);
            {
                const float fk = __builtin_ldexpf(1.f, -sk), fv = __builtin_ldexpf(1.f, -sv);
#pragma unroll
                for (int n = 0; n < kItems; ++n) {
                    const int it = tid + kSegThreads * n;
                    if (it < rows3 * kD / 8) {
                        float x[8], y[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            x[i] = kraw[n][i] * fk;
                            y[i] = vraw[n][i] * fv;
                        }
                        const Sp8 kp = split8(x), vp = split8(y);
                        const int o = off64(it >> 3, (it & 7) * 8);
                        st16(tK + o, kp.h);
                        st16(tK + plane3 / 2 + o, kp.m);
                        st16(tV + o, vp.h);
                        st16(tV + plane3 / 2 + o, vp.m);
                    }
                }
            }
            __syncthreads();
            if (16 * w < nq) {   // the wave's query tile of this pass
                const int qt = (q0 + 16 * w - r0) >> 4;
                const float sscale2 = __builtin_ldexpf(0.125f, sq + sk) * 1.4426950408889634f;
                // the tile's Q fragments again (the values of phase 0)
                Sp8 qp[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float x[8];
                    load_row8<T, false>(Qs, q0 + 16 * w + l16, L, 32 * c + 8 * g, x);
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i] *= fq;
                    qp[c] = split8<true>(x);
                }
                f32x4_t o[4];
                float lsum;
                if (rows3 == kSRows3)
                    local_narrow<false, false, KeyBits, kS3Plane>(pK3, pV3, qp, qt, NTp, Lp,
                                                                  a.rad, sscale2, l16, g, lo.rl64,
                                                                  trv, kb, o, lsum);
                else
                    local_narrow<false, false, KeyBits, kS3Plane - 16 * kD * 2>(
                        pK3, pV3, qp, qt, NTp, Lp, a.rad, sscale2, l16, g, lo.rl64, trv, kb, o,
                        lsum);
                const int tok = q0 + 16 * w + l16;   // absolute
                if (tok < seg0 + Ls) {
                    const float f = a.alpha * __builtin_ldexpf(1.f, sv) * __builtin_amdgcn_rcpf(lsum);
                    const float *vc = sTab + sC[tok - seg0] * kD;
#pragma unroll
                    for (int jd = 0; jd < 4; ++jd) {   // o[jd][rr] = Oloc^T[dim 16jd + 4g + rr][query tok]
                        const int d0 = 16 * jd + 4 * g;
                        const float4 c4 = *reinterpret_cast<const float4 *>(vc + d0);
                        store4<T>(out + base + (long)tok * kD + d0,
                                  make_float4(fmaf(o[jd][0], f, c4.x), fmaf(o[jd][1], f, c4.y),
                                              fmaf(o[jd][2], f, c4.z), fmaf(o[jd][3], f, c4.w)));
                    }
                }
            }
            __syncthreads();   // the pass planes are rewritten next
        }
    }
    // A slice barrier that gave up (only possible while other work holds CUs
    // this launch needs, for longer than the spin limit) leaves wrong sums
    // behind: a workgroup that sees the error word then turns its rows into
    // NaN and its assignments into -1, so the failure cannot pass unnoticed.
    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        T *out = static_cast<T *>(a.out);
        const float qnan = __builtin_nanf("");
        for (int e = tid; e < Ls * (kD / 4); e += kSegThreads)
            store4<T>(out + base + (long)(seg0 + e / (kD / 4)) * kD + 4 * (e % (kD / 4)),
                      make_float4(qnan, qnan, qnan, qnan));
        if (a.assign)
            for (int e = tid; e < Ls; e += kSegThreads) a.assign[s * (long)L + seg0 + e] = -1;
    }
}

// Segments per slice for the launch (0: the shape does not take it): one
// workgroup per CU for all S x ns workgroups, at most kSegMax tokens each.
int seg_count(long S, int L, int Kc, int r, int cus) {
    if (Kc < 1 || Kc > kSegK || r < 0 || r > 16 || L < 2 || cus < 1 || S > cus) return 0;
    const long ns_max = cus / S;                         // co-resident limit
    const long ns_min = (L + kSegMax - 1) / kSegMax;     // LDS limit
    const long ns_tiles = (L + 15) / 16;                 // at least one tile each
    long ns = ns_max < ns_tiles ? ns_max : ns_tiles;
    if (ns < ns_min || ns < 2) return 0;
    // segments of a multiple of 16 tokens; no segment left empty
    const long seg = 16 * (((L + ns - 1) / ns + 15) / 16);
    ns = (L + seg - 1) / seg;
    if (ns < 2 || seg > kSegMax) return 0;
    return (int)ns;
}

int seg_tokens(int L, int ns) { return 16 * (((L + ns - 1) / ns + 15) / 16); }

size_t seg_workspace_bytes(long S, int L, int Kc, int ns) {
    (void)L;
    const size_t part = sizeof(float) * 2 * (size_t)S * ns * Kc * kXPartStride;
    const size_t rows = sizeof(float) * (size_t)S * Kc * kD;
    const size_t bar = sizeof(uint32_t) * ((size_t)S + 1) * kBarStride;
    return ((part + 255) / 256 + (rows + 255) / 256 + (bar + 255) / 256) * 256;
}

hipError_t launch_seg(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                      int iters, int r, float alpha, int init_step, ca_dtype_t dt, int H, int G,
                      void *out, int32_t *assign, int ns, void *workspace, hipStream_t st,
                      int32_t *hist) {
    SegArgs a{};
    a.Q = Q; a.K = K; a.V = V;
    a.L = L; a.Kc = Kc; a.iters = iters; a.rad = r; a.alpha = alpha;
    a.init_step = init_step; a.H = H; a.G = G;
    a.out = out; a.assign = assign; a.hist = hist;
    a.S = S; a.ns = ns; a.seg = seg_tokens(L, ns);
    a.two_level = ns > 4;
    char *ws = static_cast<char *>(workspace);
    const size_t part = sizeof(float) * 2 * (size_t)S * ns * Kc * kXPartStride;
    const size_t rows = sizeof(float) * (size_t)S * Kc * kD;
    a.part = reinterpret_cast<float *>(ws);
    a.rows = reinterpret_cast<float *>(ws + (part + 255) / 256 * 256);
    a.bar = reinterpret_cast<uint32_t *>(ws + (part + 255) / 256 * 256 + (rows + 255) / 256 * 256);
    if (a.seg > kSegMax || (long)ns * a.seg < L) return hipErrorInvalidValue;
    const long nw = ((long)S + 1) * kBarStride;
    hipLaunchKernelGGL(seg_zero_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, st, a.bar,
                       nw);
    const dim3 grid((unsigned)((long)S * ns)), block(kSegThreads);
#define CA_SEG_LAUNCH(TT, HH) \
    hipLaunchKernelGGL((cluster_attn_seg_kernel<TT, HH>), grid, block, 0, st, a)
    if (dt == CA_BF16) {
        if (hist) CA_SEG_LAUNCH(bf16_t, true); else CA_SEG_LAUNCH(bf16_t, false);
    } else {
        if (hist) CA_SEG_LAUNCH(float, true); else CA_SEG_LAUNCH(float, false);
    }
#undef CA_SEG_LAUNCH
    return hipGetLastError();
}

}  // namespace ca
