// C ABI of the cluster attention library: argument checks on the host,
// workspace layout, and the launch sequence of each entry point. The
// operation and every convention are stated in include/clusterattn.h.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "launch.h"

namespace {

using namespace ca;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t elem_bytes(ca_dtype_t dt) { return dt == CA_BF16 ? 2 : 4; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int clusters(int nclust, int L) { return nclust < L ? nclust : L; }

struct Span {
    const void *p;
    size_t n;
};

bool any_overlap(const Span *s, int count) {
    for (int i = 0; i < count; ++i)
        for (int j = i + 1; j < count; ++j)
            if (s[i].p && s[j].p && overlap(s[i].p, s[i].n, s[j].p, s[j].n)) return true;
    return false;
}

// Shape checks shared by the whole-forward entry points. Returns CA_OK,
// CA_ERR_INVALID_ARG or CA_ERR_UNSUPPORTED.
ca_status_t check_shape(int B, int H, int L, int d, int nclust, int iters, int W, float alpha,
                        ca_dtype_t dt) {
    if (B < 1 || H < 1 || L < 1 || d < 1 || nclust < 1 || iters < 1 || W < 0)
        return CA_ERR_INVALID_ARG;
    if (!(alpha >= 0.f && alpha <= 1.f)) return CA_ERR_INVALID_ARG;   // also NaN
    if (dt != CA_F32 && dt != CA_BF16) return CA_ERR_INVALID_ARG;
    if ((long long)B * H * L * d > (1LL << 40)) return CA_ERR_INVALID_ARG;
    if ((long long)B * H * L > (1LL << 31) - 1) return CA_ERR_UNSUPPORTED;
    if (d != kD) return CA_ERR_UNSUPPORTED;
    if (clusters(nclust, L) > kMaxClusters) return CA_ERR_UNSUPPORTED;
    return CA_OK;
}

// Workspace of the staged path, carved in this order (each 256-B aligned).
struct StagedLayout {
    size_t mu, assign, part_sum, part_cnt, part_sum2, part_cnt2, vcent, xpart, oloc, qmax, total;
};

// Lloyd steps on the matrix cores pass their block sums straight to the next
// step (two partial buffers, no reduce launch in between) when a slice has
// at most this many 128-token blocks.
constexpr int kChainBlocks = 8;
bool chain_steps(int L, int Kc) {
    return kmeans_mfma_supported(Kc) && kmeans_mfma_blocks(L) <= kChainBlocks;
}

StagedLayout staged_layout(long S, int L, int Kc) {
    StagedLayout w{};
    const long ntile = kmeans_tiles(L);
    const long nsplit = xattn_splits(L);
    const long nchain = chain_steps(L, Kc) ? kmeans_mfma_blocks(L) : 0;
    size_t off = 0;
    w.mu = off;       off += align_up(sizeof(float) * S * Kc * kD);
    w.assign = off;   off += align_up(sizeof(int32_t) * S * L);
    w.part_sum = off; off += align_up(sizeof(float) * S * ntile * Kc * kD);
    w.part_cnt = off; off += align_up(sizeof(int32_t) * S * ntile * Kc);
    w.part_sum2 = off; off += nchain ? align_up(sizeof(float) * S * nchain * Kc * kD) : 0;
    w.part_cnt2 = off; off += nchain ? align_up(sizeof(int32_t) * S * nchain * Kc) : 0;
    w.vcent = off;    off += align_up(sizeof(float) * S * Kc * kD);
    w.xpart = off;    off += nsplit > 1 ? align_up(sizeof(float) * S * nsplit * Kc * (kD + 2)) : 0;
    // alpha O^loc rows when the window runs beside the clustering
    w.oloc = off;     off += kmeans_slice_supported(L, Kc) ? align_up(sizeof(float) * S * L * kD) : 0;
    // the largest |q| of each run of blocks of the matrix-core Lloyd steps
    const long nrun = kmeans_mfma_supported(Kc) && !nchain ? kmeans_mfma_blocks(L) : 0;
    w.qmax = off;     off += nrun ? align_up(sizeof(uint32_t) * S * nrun) : 0;
    w.total = off;
    return w;
}

// Compute units of the current device, looked up once per device (the
// count never changes while the process runs).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < kMaxDevices) {
        const int known = g_cus[dev].load(std::memory_order_relaxed);
        if (known > 0) return known;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev >= 0 && dev < kMaxDevices && cus > 0) g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// The 16-wave single launch for 128 < L <= 512 holds one slice per CU; it
// beats the staged launches when the slices fill between half and all of the
// CUs in one round (measured on MI355X, bf16 L = 512: 43.5 against 50.0 us at
// 144 slices, 47.1 against 60.1 us at 252, but 41.4 against 38.8 us at 96 and
// 83.5 against 79.0 us at 264).
bool fused512_pays(long S) {
    const int cus = device_cus();
    return cus > 0 && 2 * S > cus && S <= cus;
}

// With at most half the CUs' worth of slices, the split form of that launch
// (bf16 storage) runs each slice's window branch on a second workgroup beside
// its clustering, on CUs the single launch would leave idle (measured, bf16
// L = 512, 96 slices: see fused512.hip).
bool fused512_split_pays(long S) {
    const int cus = device_cus();
    return cus > 0 && 2 * S <= cus && S <= fused512_split_max_slices();
}

// The window blocks beside the clustering fill CUs that the clustering
// (one workgroup per slice) leaves idle: taken when the clustering and the
// window workgroups (two 128-query blocks each) fit the CUs in one round
// (measured, bf16 L = 512: 25.9 against 30.7 us at 48 slices; at 96 slices,
// which need 288 workgroups, 36.6 against 35.4 us).
bool window_beside_pays(long S, int L) {
    const int cus = device_cus();
    return cus > 0 && S + S * ((L + 127) / 128) / 2 <= cus;
}

bool use_fused(ca_path_t path, int L, int Kc) {
    if (path == CA_PATH_STAGED) return false;
    return fused_supported(L, Kc);
}

// The launch sequence of one forward call, decided on the host from the shape,
// the variants and the device's CU count.
enum PlanKind {
    kPlanFused,      // cluster_attn_fused_kernel: one launch, L <= 128
    kPlanFused512,   // cluster_attn_fused512_kernel: one launch, 128 < L <= 512
    kPlanF512Split,  // its split form: 2 S workgroups (clustering, window), bf16 storage
    kPlanSeg,        // cluster_attn_seg_kernel: one launch, each slice over ns workgroups
    kPlanBeside,     // kmeans_window_kernel (clustering + window), centroid attention, gather
    kPlanSlice,      // kmeans_slice_kernel, centroid attention, window branch
    kPlanSteps       // one launch per Lloyd step, centroid attention, window branch
};

struct Plan {
    PlanKind kind;
    int ns;                // segments per slice (kPlanSeg)
    bool km_mfma;          // steps on the matrix cores (else the scalar step)
    bool chain;            // steps pass their block sums on (no reduce in between)
    bool mfma_local;       // window branch on the matrix cores (else scalar)
    bool merge_in_local;   // the window kernel merges the key-range partials
    bool slice_xattn;      // kPlanSlice: the clustering launch forms the key ranges too
};

// Returns CA_OK and the plan, or CA_ERR_UNSUPPORTED when CA_PATH_FUSED was
// asked for a shape without a single launch.
ca_status_t make_plan(long S, int L, int Kc, int radius, const Variant &var, bool masked,
                      ca_path_t path, bool bf16, Plan &p) {
    p = Plan{};
    if (path != CA_PATH_SEGMENTED && use_fused(path, L, Kc)) {
        p.kind = kPlanFused;
        return CA_OK;
    }
    const bool plain = !masked && !var.soft && !var.keep_empty;
    // 128 < L <= 512: the 16-wave single launch (forced by CA_PATH_FUSED, by
    // the auto path when it pays)
    const bool f512 = plain && fused512_supported(L, Kc, radius);
    if (path == CA_PATH_FUSED && !f512) return CA_ERR_UNSUPPORTED;
    if (f512 && bf16 && path == CA_PATH_AUTO && fused512_split_pays(S)) {
        p.kind = kPlanF512Split;
        return CA_OK;
    }
    if (f512 && (path == CA_PATH_FUSED || (path == CA_PATH_AUTO && fused512_pays(S)))) {
        p.kind = kPlanFused512;
        return CA_OK;
    }
    // the segmented single launch: only when CA_PATH_SEGMENTED asks for it
    // (on the shapes measured so far the staged launches are faster)
    if (path == CA_PATH_SEGMENTED) {
        const int ns = plain ? seg_count(S, L, Kc, radius, device_cus()) : 0;
        if (ns == 0) return CA_ERR_UNSUPPORTED;
        p.kind = kPlanSeg;
        p.ns = ns;
        return CA_OK;
    }
    const bool one_launch = kmeans_slice_supported(L, Kc) && !var.keep_empty;
    if (one_launch && !var.soft && kmeans_window_supported(S, L, Kc, radius) &&
        window_beside_pays(S, L)) {
        p.kind = kPlanBeside;
        p.merge_in_local = xattn_splits(L) > 1 && xattn_splits(L) <= kXMergeInLocal;
        return CA_OK;
    }
    p.kind = one_launch ? kPlanSlice : kPlanSteps;
    p.km_mfma = kmeans_mfma_supported(Kc);
    // kept empty clusters need every step's centroids in place: no chaining
    p.chain = chain_steps(L, Kc) && !var.keep_empty;
    p.mfma_local = !var.soft && local_mfma_supported(radius);
    // a few key ranges: the window kernel merges them, no combine launch
    p.merge_in_local = p.mfma_local && xattn_splits(L) > 1 && xattn_splits(L) <= kXMergeInLocal;
    // four ranges and the clustering's workgroups doubled within one round:
    // the clustering launch forms the ranges itself (measured, bf16 L = 512,
    // 96 slices: see kmeans_xattn_kernel)
    p.slice_xattn = p.kind == kPlanSlice && !masked && p.merge_in_local &&
                    kmeans_xattn_supported(S, L, Kc, device_cus());
    return CA_OK;
}

const char *plan_name(const Plan &p) {
    switch (p.kind) {
        case kPlanFused: return "fused";
        case kPlanFused512: return "fused512";
        case kPlanF512Split: return "fused512 split (clustering and window workgroups)";
        case kPlanSeg: return "segmented";
        case kPlanBeside:
            return p.merge_in_local ? "staged: kmeans_window, xattn ranges, gather_oloc (merge)"
                                    : "staged: kmeans_window, xattn, gather_oloc";
        case kPlanSlice:
        case kPlanSteps: break;
    }
    // [window: scalar, matrix cores, matrix cores merging the key ranges]
    static const char *const slice_names[3] = {
        "staged: kmeans_slice, xattn, local_scalar", "staged: kmeans_slice, xattn, local_mfma",
        "staged: kmeans_slice, xattn ranges, local_mfma (merge)"};
    // [steps: chained, with reduce launches, scalar][window as above]
    static const char *const step_names[3][3] = {
        {"staged: kmeans_mfma steps (chained), xattn, local_scalar",
         "staged: kmeans_mfma steps (chained), xattn, local_mfma",
         "staged: kmeans_mfma steps (chained), xattn ranges, local_mfma (merge)"},
        {"staged: kmeans_mfma steps + reduce, xattn, local_scalar",
         "staged: kmeans_mfma steps + reduce, xattn, local_mfma",
         "staged: kmeans_mfma steps + reduce, xattn ranges, local_mfma (merge)"},
        {"staged: scalar kmeans steps + reduce, xattn, local_scalar",
         "staged: scalar kmeans steps + reduce, xattn, local_mfma",
         "staged: scalar kmeans steps + reduce, xattn ranges, local_mfma (merge)"}};
    const int loc = !p.mfma_local ? 0 : p.merge_in_local ? 2 : 1;
    if (p.kind == kPlanSlice && p.slice_xattn)
        return "staged: kmeans_slice + xattn ranges, local_mfma (merge)";
    if (p.kind == kPlanSlice) return slice_names[loc];
    return step_names[!p.km_mfma ? 2 : p.chain ? 0 : 1][loc];
}

ca_status_t hip_status(hipError_t e) { return e == hipSuccess ? CA_OK : CA_ERR_HIP; }

#define CA_TRY(expr)                                  \
    do {                                              \
        hipError_t _e = (expr);                       \
        if (_e != hipSuccess) return CA_ERR_HIP;      \
    } while (0)

// valid: key-padding mask [B, L] or nullptr (the unmasked operation); G:
// query heads per K/V head (K and V are [B, H / G, L, d]); flags: CA_FLAG_*;
// hist: nullable [iters, B, H, L] trace of every iteration's assignment.
ca_status_t forward_impl(const void *Q, const void *K, const void *V, const uint8_t *valid, int G,
                         int flags, int B, int H, int L, int d, int nclust, int iters, int W,
                         float alpha, void *out, int32_t *assign_out, ca_dtype_t dt,
                         void *workspace, size_t workspace_bytes, ca_path_t path,
                         hipStream_t stream, int32_t *hist = nullptr) {
    if (flags & ~CA_FLAG_LISTING) return CA_ERR_INVALID_ARG;
    if (flags & CA_FLAG_ALPHA_LOGIT) {   // the listing's sigmoid of its parameter
        if (alpha != alpha) return CA_ERR_INVALID_ARG;
        alpha = (float)(1.0 / (1.0 + exp(-(double)alpha)));
    }
    ca_status_t st = check_shape(B, H, L, d, nclust, iters, W, alpha, dt);
    if (st != CA_OK) return st;
    if (path != CA_PATH_AUTO && path != CA_PATH_FUSED && path != CA_PATH_STAGED &&
        path != CA_PATH_SEGMENTED)
        return CA_ERR_INVALID_ARG;
    if (!Q || !K || !V || !out) return CA_ERR_INVALID_ARG;
    if (G < 1 || H % G != 0) return CA_ERR_INVALID_ARG;
    const long S = (long)B * H;
    const size_t tbytes = (size_t)S * L * d * elem_bytes(dt);
    const size_t kvbytes = tbytes / (size_t)G;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16))
        return CA_ERR_INVALID_ARG;
    if (assign_out && !aligned(assign_out, 4)) return CA_ERR_INVALID_ARG;
    if (overlap(out, tbytes, Q, tbytes) || overlap(out, tbytes, K, kvbytes) ||
        overlap(out, tbytes, V, kvbytes))
        return CA_ERR_INVALID_ARG;
    const size_t abytes = sizeof(int32_t) * (size_t)S * L;
    if (assign_out && (overlap(assign_out, abytes, out, tbytes) ||
                       overlap(assign_out, abytes, Q, tbytes) ||
                       overlap(assign_out, abytes, K, kvbytes) ||
                       overlap(assign_out, abytes, V, kvbytes)))
        return CA_ERR_INVALID_ARG;
    const size_t vbytes = (size_t)B * L;
    if (valid && (overlap(valid, vbytes, out, tbytes) ||
                  (assign_out && overlap(valid, vbytes, assign_out, abytes))))
        return CA_ERR_INVALID_ARG;
    const size_t hbytes = abytes * (size_t)iters;
    if (hist) {
        const Span others[] = {{Q, tbytes}, {K, kvbytes}, {V, kvbytes}, {out, tbytes},
                               {assign_out, abytes}, {valid, vbytes}};
        if (!aligned(hist, 4)) return CA_ERR_INVALID_ARG;
        for (const Span &o : others)
            if (o.p && overlap(hist, hbytes, o.p, o.n)) return CA_ERR_INVALID_ARG;
    }
    const int Kc = clusters(nclust, L);
    Variant var{};
    if (flags & CA_FLAG_INIT_STEP) var.init_step = L / Kc > 1 ? L / Kc : 1;
    var.keep_empty = (flags & CA_FLAG_KEEP_EMPTY) != 0;
    var.soft = (flags & CA_FLAG_SOFT_GATHER) != 0;
    // window radius; the listing's band drops the local branch when W == 0 or
    // W >= L (radius 0 with weight 0 leaves exactly the gathered context)
    int radius = W / 2;
    if (flags & CA_FLAG_BAND) {
        radius = W;
        if (W == 0 || W >= L) {
            radius = 0;
            alpha = 0.f;
        }
    }

    Plan plan;
    st = make_plan(S, L, Kc, radius, var, valid != nullptr, path, dt == CA_BF16, plan);
    if (st != CA_OK) return st;
    if (plan.kind == kPlanFused)
        return hip_status(launch_fused_forward(Q, K, V, (int)S, L, Kc, iters, radius, alpha, var,
                                               dt, valid, H, G, out, assign_out, stream, hist,
                                               device_cus()));
    if (plan.kind == kPlanFused512)
        return hip_status(launch_fused512(Q, K, V, (int)S, L, Kc, iters, radius, alpha,
                                          var.init_step, dt, H, G, out, assign_out, stream,
                                          hist));
    if (plan.kind == kPlanF512Split) {
        const size_t need = fused512_split_workspace_bytes(S);
        if (workspace_bytes < need || !workspace || !aligned(workspace, kAlign))
            return CA_ERR_INVALID_ARG;
        const Span others[] = {{Q, tbytes}, {K, kvbytes}, {V, kvbytes}, {out, tbytes},
                               {assign_out, abytes}, {hist, hbytes}};
        for (const Span &o : others)
            if (o.p && overlap(workspace, need, o.p, o.n)) return CA_ERR_INVALID_ARG;
        return hip_status(launch_fused512(Q, K, V, (int)S, L, Kc, iters, radius, alpha,
                                          var.init_step, dt, H, G, out, assign_out, stream, hist,
                                          workspace));
    }
    if (plan.kind == kPlanSeg) {
        const size_t need = seg_workspace_bytes(S, L, Kc, plan.ns);
        if (workspace_bytes < need || !workspace || !aligned(workspace, kAlign))
            return CA_ERR_INVALID_ARG;
        const Span others[] = {{Q, tbytes}, {K, kvbytes}, {V, kvbytes}, {out, tbytes},
                               {assign_out, abytes}, {hist, hbytes}};
        for (const Span &o : others)
            if (o.p && overlap(workspace, need, o.p, o.n)) return CA_ERR_INVALID_ARG;
        return hip_status(launch_seg(Q, K, V, (int)S, L, Kc, iters, radius, alpha, var.init_step,
                                     dt, H, G, out, assign_out, plan.ns, workspace, stream,
                                     hist));
    }
    const StagedLayout lay = staged_layout(S, L, Kc);
    if (workspace_bytes < lay.total || !workspace) return CA_ERR_INVALID_ARG;
    if (!aligned(workspace, kAlign)) return CA_ERR_INVALID_ARG;
    char *ws = static_cast<char *>(workspace);
    if (overlap(ws, lay.total, out, tbytes) || overlap(ws, lay.total, Q, tbytes) ||
        overlap(ws, lay.total, K, kvbytes) || overlap(ws, lay.total, V, kvbytes) ||
        (assign_out && overlap(ws, lay.total, assign_out, abytes)) ||
        (valid && overlap(ws, lay.total, valid, vbytes)) ||
        (hist && overlap(ws, lay.total, hist, hbytes)))
        return CA_ERR_INVALID_ARG;
    float *mu = reinterpret_cast<float *>(ws + lay.mu);
    int32_t *c = assign_out ? assign_out : reinterpret_cast<int32_t *>(ws + lay.assign);
    float *psum = reinterpret_cast<float *>(ws + lay.part_sum);
    int32_t *pcnt = reinterpret_cast<int32_t *>(ws + lay.part_cnt);
    float *vcent = reinterpret_cast<float *>(ws + lay.vcent);
    float *xpart = reinterpret_cast<float *>(ws + lay.xpart);
    const bool km_mfma = plan.km_mfma;
    const bool chain = plan.chain;
    const int nsub = km_mfma && !chain ? kmeans_mfma_run(S, L, device_cus()) : 1;
    const int nblk = km_mfma ? kmeans_mfma_parts(L, nsub) : kmeans_tiles(L);
    float *ps[2] = {psum, chain ? reinterpret_cast<float *>(ws + lay.part_sum2) : psum};
    int32_t *pc[2] = {pcnt, chain ? reinterpret_cast<int32_t *>(ws + lay.part_cnt2) : pcnt};
    const bool one_launch = plan.kind == kPlanSlice;
    if (plan.kind == kPlanBeside) {
        // clustering and window blocks in one launch, then the centroid
        // attention (its key ranges left unmerged up to kXMergeInLocal) and
        // the gather of (1 - alpha) V^cent_{c_i} onto alpha O^loc
        float *oloc = reinterpret_cast<float *>(ws + lay.oloc);
        const bool merge = plan.merge_in_local;
        CA_TRY(launch_kmeans_window(Q, K, V, (int)S, L, Kc, iters, dt, c, mu, var.init_step,
                                    radius, alpha, valid, H, G, oloc, stream, hist));
        CA_TRY(launch_centroid_xattn(mu, K, V, (int)S, L, Kc, dt, valid, H, G, vcent, xpart,
                                     stream, nullptr, !merge));
        return hip_status(launch_gather_oloc(oloc, c, vcent, merge ? xpart : nullptr, (int)S, L,
                                             Kc, alpha, valid, H, dt, out, stream));
    }
    if (one_launch && plan.slice_xattn)
        CA_TRY(launch_kmeans_xattn(Q, K, V, (int)S, L, Kc, iters, dt, c, mu, var.init_step, H, G,
                                   xpart, stream, hist));
    else if (one_launch)
        CA_TRY(launch_kmeans_slice(Q, (int)S, L, Kc, iters, dt, c, mu, var.init_step, stream,
                                   hist));
    for (int t = 1; !one_launch && t <= iters; ++t) {
        const int cur = chain ? (t - 1) & 1 : 0;
        // a kept empty cluster of the first update needs mu^(0) in place
        const float *mu_in = t == 1 ? nullptr : mu;
        float *mu0 = t == 1 && var.keep_empty ? mu : nullptr;
        // each step's assignment is read by no later step, so the steps
        // before the last write theirs straight into the trace
        int32_t *ct = hist && t < iters ? hist + (size_t)(t - 1) * S * L : c;
        if (km_mfma)
            CA_TRY(launch_kmeans_mfma(Q, mu_in, (int)S, L, Kc, dt, ct, ps[cur], pc[cur], stream,
                                      var.init_step, mu0, chain && t > 1 ? ps[cur ^ 1] : nullptr,
                                      chain && t > 1 ? pc[cur ^ 1] : nullptr, nsub,
                                      nsub > 1 ? reinterpret_cast<uint32_t *>(ws + lay.qmax)
                                               : nullptr));
        else
            CA_TRY(launch_kmeans_assign(Q, mu_in, (int)S, L, Kc, dt, ct, psum, pcnt, stream,
                                        var.init_step, mu0));
        if (!chain || t == iters)
            CA_TRY(launch_centroid_reduce(ps[cur], pc[cur], nblk, (int)S, Kc, mu, nullptr, stream,
                                          var.keep_empty));
    }
    if (hist && !one_launch)
        CA_TRY(hipMemcpyAsync(hist + (size_t)(iters - 1) * S * L, c, abytes,
                              hipMemcpyDeviceToDevice, stream));
    const bool mfma_local = plan.mfma_local;
    const bool merge_in_local = plan.merge_in_local;
    if (!plan.slice_xattn)
        CA_TRY(launch_centroid_xattn(mu, K, V, (int)S, L, Kc, dt, valid, H, G, vcent, xpart,
                                     stream, nullptr, !merge_in_local));
    if (mfma_local)
        return hip_status(launch_local_mfma(Q, K, V, (int)S, L, radius, dt, vcent, c, Kc, alpha,
                                            valid, H, G, out, stream,
                                            merge_in_local ? xpart : nullptr));
    CA_TRY(launch_local_window(Q, K, V, (int)S, L, radius, dt, vcent, c, Kc, alpha, valid, H, G,
                               out, nullptr, stream, var.soft ? mu : nullptr));
    return CA_OK;
}

// Workspace of the backward pass, carved in this order (each 256-B aligned).
struct BwdLayout {
    size_t mu, counts, part, pcnt, vcent, cstat, xpart, dvc, dmu, lstat, dal, dkc, dvl, total;
};

BwdLayout bwd_layout(long S, int L, int Kc) {
    BwdLayout w{};
    const long ntile = bwd_tiles(L) > kmeans_tiles(L) ? bwd_tiles(L) : kmeans_tiles(L);
    const long nsplit = xattn_splits(L);
    size_t off = 0;
    w.mu = off;     off += align_up(sizeof(float) * S * Kc * kD);
    w.counts = off; off += align_up(sizeof(int32_t) * S * Kc);
    w.part = off;   off += align_up(sizeof(float) * S * ntile * Kc * kD);
    w.pcnt = off;   off += align_up(sizeof(int32_t) * S * ntile * Kc);
    w.vcent = off;  off += align_up(sizeof(float) * S * Kc * kD);
    w.cstat = off;  off += align_up(sizeof(float) * S * Kc * 2);
    w.xpart = off;  off += nsplit > 1 ? align_up(sizeof(float) * S * nsplit * Kc * (kD + 2)) : 0;
    w.dvc = off;    off += align_up(sizeof(float) * S * Kc * kD);
    w.dmu = off;    off += align_up(sizeof(float) * S * Kc * kD);
    w.lstat = off;  off += align_up(sizeof(float) * 4 * S * L);
    w.dal = off;    off += align_up(sizeof(float) * S * ntile);
    w.dkc = off;    off += align_up(sizeof(float) * S * L * kD);
    w.dvl = off;    off += align_up(sizeof(float) * S * L * kD);
    w.total = off;
    return w;
}

// Checks shared by the single-step entry points.
ca_status_t check_step(int S, int L, int d, int Kc, ca_dtype_t dt) {
    if (S < 1 || L < 1 || d < 1 || Kc < 1) return CA_ERR_INVALID_ARG;
    if (dt != CA_F32 && dt != CA_BF16) return CA_ERR_INVALID_ARG;
    if ((long long)S * L > (1LL << 31) - 1) return CA_ERR_UNSUPPORTED;
    if (d != kD || Kc > kMaxClusters) return CA_ERR_UNSUPPORTED;
    return CA_OK;
}

// Workspace of the full layer, carved in this order (each 256-B aligned):
// Q/K/V ([3, B, H, L, 64]; unused when the caller passes qkv_out), the
// attention output O ([B, H, L, 64]) and the cluster attention workspace of
// the bf16 [B, H, L, 64] problem.
struct LayerLayout {
    size_t qkv, o, attn, attn_bytes, total;
};

LayerLayout layer_layout(int B, int L, int Dm, int H, int nclust) {
    LayerLayout w{};
    const size_t tok = (size_t)B * L;
    size_t off = 0;
    w.qkv = off;  off += align_up(sizeof(uint16_t) * 3 * tok * Dm);
    w.o = off;    off += align_up(sizeof(uint16_t) * tok * Dm);
    w.attn = off;
    w.attn_bytes = align_up(cluster_attn_workspace_size_ex(B, H, L, kD, nclust, CA_BF16,
                                                           CA_PATH_AUTO));
    off += w.attn_bytes;
    w.total = off;
    return w;
}

ca_status_t check_layer(int B, int L, int Dm, int H, int d, int nclust, int iters, int W,
                        float alpha) {
    if (Dm < 1) return CA_ERR_INVALID_ARG;
    ca_status_t st = check_shape(B, H, L, d, nclust, iters, W, alpha, CA_BF16);
    if (st != CA_OK) return st;
    if ((long long)B * L * Dm > (1LL << 40)) return CA_ERR_INVALID_ARG;
    if ((long long)Dm != (long long)H * d) return CA_ERR_UNSUPPORTED;
    return CA_OK;
}


}  // namespace

extern "C" {

const char *ca_status_string(ca_status_t s) {
    switch (s) {
        case CA_OK: return "ok";
        case CA_ERR_INVALID_ARG: return "invalid argument";
        case CA_ERR_UNSUPPORTED: return "unsupported shape or type";
        case CA_ERR_HIP: return "HIP launch error";
        case CA_ERR_SCRATCH_TOO_SMALL:
            return "the call needs more workspace than the allocation-free entry point holds";
    }
    return "unknown status";
}

int ca_version(void) { return 200; }

size_t cluster_attn_workspace_size_ex(int B, int H, int L, int d, int nclust, ca_dtype_t dt,
                                      ca_path_t path) {
    if (check_shape(B, H, L, d, nclust, 1, 0, 0.f, dt) != CA_OK) return 0;
    const int Kc = clusters(nclust, L);
    const long S = (long)B * H;
    if (path == CA_PATH_FUSED || (path == CA_PATH_AUTO && use_fused(path, L, Kc))) return 0;
    if (path == CA_PATH_SEGMENTED) {
        const int ns = seg_count(S, L, Kc, 0, device_cus());
        return ns > 0 ? seg_workspace_bytes(S, L, Kc, ns) : 0;
    }
    // the auto path's split form needs less than the staged launches, but
    // take the larger of the two so the size never depends on the CU count
    const size_t staged = staged_layout(S, L, Kc).total;
    const size_t split = fused512_split_workspace_bytes(S);
    return staged > split ? staged : split;
}

const char *cluster_attn_plan(int B, int H, int L, int nclust, int W, int flags, int masked,
                              ca_path_t path) {
    return cluster_attn_plan_dt(B, H, L, nclust, W, flags, masked, path, CA_F32);
}

const char *cluster_attn_plan_dt(int B, int H, int L, int nclust, int W, int flags, int masked,
                                 ca_path_t path, ca_dtype_t dt) {
    if (check_shape(B, H, L, kD, nclust, 1, W, 0.f, dt) != CA_OK) return nullptr;
    if ((flags & ~CA_FLAG_LISTING) ||
        (path != CA_PATH_AUTO && path != CA_PATH_FUSED && path != CA_PATH_STAGED &&
         path != CA_PATH_SEGMENTED))
        return nullptr;
    const int Kc = clusters(nclust, L);
    Variant var{};
    if (flags & CA_FLAG_INIT_STEP) var.init_step = L / Kc > 1 ? L / Kc : 1;
    var.keep_empty = (flags & CA_FLAG_KEEP_EMPTY) != 0;
    var.soft = (flags & CA_FLAG_SOFT_GATHER) != 0;
    int radius = W / 2;
    if (flags & CA_FLAG_BAND) radius = (W == 0 || W >= L) ? 0 : W;
    Plan p;
    if (make_plan((long)B * H, L, Kc, radius, var, masked != 0, path, dt == CA_BF16, p) != CA_OK)
        return nullptr;
    return plan_name(p);
}

size_t cluster_attn_workspace_size(int B, int H, int L, int d, int nclust, ca_dtype_t dt) {
    return cluster_attn_workspace_size_ex(B, H, L, d, nclust, dt, CA_PATH_AUTO);
}

ca_status_t cluster_attn_forward(const void *Q, const void *K, const void *V, int B, int H, int L,
                                 int d, int nclust, int iters, int W, float alpha, void *out,
                                 int32_t *assign_out, ca_dtype_t dt, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    return forward_impl(Q, K, V, nullptr, 1, 0, B, H, L, d, nclust, iters, W, alpha, out,
                        assign_out, dt, workspace, workspace_bytes, CA_PATH_AUTO, stream);
}

ca_status_t cluster_attn_forward_ex(const void *Q, const void *K, const void *V, int B, int H,
                                    int L, int d, int nclust, int iters, int W, float alpha,
                                    void *out, int32_t *assign_out, ca_dtype_t dt,
                                    void *workspace, size_t workspace_bytes, ca_path_t path,
                                    hipStream_t stream) {
    return forward_impl(Q, K, V, nullptr, 1, 0, B, H, L, d, nclust, iters, W, alpha, out,
                        assign_out, dt, workspace, workspace_bytes, path, stream);
}

ca_status_t cluster_attn_forward_masked(const void *Q, const void *K, const void *V,
                                        const uint8_t *valid, int B, int H, int L, int d,
                                        int nclust, int iters, int W, float alpha, void *out,
                                        int32_t *assign_out, ca_dtype_t dt, void *workspace,
                                        size_t workspace_bytes, ca_path_t path,
                                        hipStream_t stream) {
    if (!valid) return CA_ERR_INVALID_ARG;
    return forward_impl(Q, K, V, valid, 1, 0, B, H, L, d, nclust, iters, W, alpha, out, assign_out,
                        dt, workspace, workspace_bytes, path, stream);
}

ca_status_t cluster_attn_forward_opts(const void *Q, const void *K, const void *V, int B, int H,
                                      int L, int d, int nclust, int iters, int W, float alpha,
                                      const ca_options_t *opts, void *out, int32_t *assign_out,
                                      ca_dtype_t dt, void *workspace, size_t workspace_bytes,
                                      ca_path_t path, hipStream_t stream) {
    const uint8_t *valid = opts ? opts->valid : nullptr;
    const int flags = opts ? opts->flags : 0;
    int32_t *hist = opts ? opts->assign_hist : nullptr;
    int G = 1;
    if (opts) {
        if (opts->kv_heads < 0) return CA_ERR_INVALID_ARG;
        if (opts->kv_heads > 0) {
            if (H < 1 || opts->kv_heads > H || H % opts->kv_heads != 0) return CA_ERR_INVALID_ARG;
            G = H / opts->kv_heads;
        }
    }
    return forward_impl(Q, K, V, valid, G, flags, B, H, L, d, nclust, iters, W, alpha, out,
                        assign_out, dt, workspace, workspace_bytes, path, stream, hist);
}

size_t cluster_attn_backward_workspace_size(int B, int H, int kv_heads, int L, int d,
                                            int nclust, ca_dtype_t dt) {
    if (check_shape(B, H, L, d, nclust, 1, 0, 0.f, dt) != CA_OK) return 0;
    if (kv_heads < 0 || kv_heads > H || (kv_heads > 0 && H % kv_heads != 0)) return 0;
    return bwd_layout((long)B * H, L, clusters(nclust, L)).total;
}

ca_status_t cluster_attn_backward(const void *Q, const void *K, const void *V, const void *dO,
                                  const int32_t *assign, const uint8_t *valid, int B, int H,
                                  int kv_heads, int L, int d, int nclust, int W, float alpha,
                                  void *dQ, void *dK, void *dV, float *dalpha, ca_dtype_t dt,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    ca_status_t st = check_shape(B, H, L, d, nclust, 1, W, alpha, dt);
    if (st != CA_OK) return st;
    if (kv_heads < 0 || kv_heads > H || (kv_heads > 0 && H % kv_heads != 0))
        return CA_ERR_INVALID_ARG;
    const int Hkv = kv_heads > 0 ? kv_heads : H;
    if (!Q || !K || !V || !dO || !assign || !dQ || !dK || !dV || !workspace)
        return CA_ERR_INVALID_ARG;
    const void *p16[] = {Q, K, V, dO, dQ, dK, dV};
    for (const void *p : p16)
        if (!aligned(p, 16)) return CA_ERR_INVALID_ARG;
    if (!aligned(assign, 4) || (dalpha && !aligned(dalpha, 4)) || !aligned(workspace, kAlign))
        return CA_ERR_INVALID_ARG;
    const long S = (long)B * H;
    const int Kc = clusters(nclust, L);
    const BwdLayout lay = bwd_layout(S, L, Kc);
    if (workspace_bytes < lay.total) return CA_ERR_INVALID_ARG;
    const size_t tb = (size_t)S * L * d * elem_bytes(dt), kvb = tb / (size_t)(H / Hkv);
    const Span outs[] = {{dQ, tb}, {dK, kvb}, {dV, kvb}, {dalpha, sizeof(float)},
                         {workspace, lay.total}};
    if (any_overlap(outs, 5)) return CA_ERR_INVALID_ARG;
    const Span ins[] = {{Q, tb}, {K, kvb}, {V, kvb}, {dO, tb}, {assign, sizeof(int32_t) * S * L},
                        {valid, (size_t)B * L}};
    for (const Span &o : outs)
        for (const Span &i : ins)
            if (o.p && i.p && overlap(o.p, o.n, i.p, i.n)) return CA_ERR_INVALID_ARG;

    char *ws = static_cast<char *>(workspace);
    float *mu = reinterpret_cast<float *>(ws + lay.mu);
    int32_t *counts = reinterpret_cast<int32_t *>(ws + lay.counts);
    float *part = reinterpret_cast<float *>(ws + lay.part);
    int32_t *pcnt = reinterpret_cast<int32_t *>(ws + lay.pcnt);
    float *vcent = reinterpret_cast<float *>(ws + lay.vcent);
    float *cstat = reinterpret_cast<float *>(ws + lay.cstat);
    float *xpart = reinterpret_cast<float *>(ws + lay.xpart);
    BwdArgs a{};
    a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.assign = assign; a.valid = valid;
    a.B = B; a.H = H; a.Hkv = Hkv; a.L = L; a.Kc = Kc; a.r = W / 2; a.alpha = alpha;
    a.mu = mu; a.counts = counts; a.vcent = vcent; a.cstat = cstat;
    a.dvc = reinterpret_cast<float *>(ws + lay.dvc);
    a.dmu = reinterpret_cast<float *>(ws + lay.dmu);
    a.part = part;
    a.lstat = reinterpret_cast<float4 *>(ws + lay.lstat);
    a.dal = reinterpret_cast<float *>(ws + lay.dal);
    a.dQ = dQ; a.dK = dK; a.dV = dV; a.dalpha = dalpha;
    a.dkc = reinterpret_cast<float *>(ws + lay.dkc);
    a.dvl = reinterpret_cast<float *>(ws + lay.dvl);
    if (bwd_fused_supported(L, Kc, H / Hkv)) {   // two launches per slice, then dalpha
        // measured, 384 slices on 256 CUs: 56.6 -> 54.3 us with the solo
        // workgroups delayed (same-box A/B)
        const int cus = device_cus();
        if (cus > 0 && S > cus && S < 2 * cus) {
            a.solo_lo = (int)(S - cus);
            a.solo_hi = cus;
        }
        CA_TRY(launch_backward_fused(a, dt, stream));
        return hip_status(launch_bwd_sum(a.dal, S, dalpha, stream));
    }
    // staged: the forward's final means and centroid attention from the given
    // assignment, then the backward kernels
    CA_TRY(launch_centroid_partials(Q, assign, (int)S, L, Kc, dt, part, pcnt, stream));
    CA_TRY(launch_centroid_reduce(part, pcnt, kmeans_tiles(L), (int)S, Kc, mu, counts, stream));
    CA_TRY(launch_centroid_xattn(mu, K, V, (int)S, L, Kc, dt, valid, H, H / Hkv, vcent, xpart,
                                 stream, cstat));
    return hip_status(launch_backward(a, dt, stream));
}

ca_status_t cluster_attn_exact_forward(const void *Q, const void *K, const void *V,
                                       const uint8_t *q_valid, const uint8_t *k_valid, int B,
                                       int H, int kv_heads, int L, int Nk, int d, int causal,
                                       void *out, ca_dtype_t dt, hipStream_t stream) {
    if (B < 1 || H < 1 || L < 1 || Nk < 1 || d < 1) return CA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return CA_ERR_INVALID_ARG;
    if (dt != CA_F32 && dt != CA_BF16) return CA_ERR_INVALID_ARG;
    if (kv_heads < 0 || kv_heads > H || (kv_heads > 0 && H % kv_heads != 0))
        return CA_ERR_INVALID_ARG;
    if ((long long)B * H * L * d > (1LL << 40) || (long long)B * H * Nk * d > (1LL << 40))
        return CA_ERR_INVALID_ARG;
    if ((long long)B * H * L > (1LL << 31) - 1 || (long long)B * H * Nk > (1LL << 31) - 1)
        return CA_ERR_UNSUPPORTED;
    if (d != kD) return CA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !out) return CA_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16))
        return CA_ERR_INVALID_ARG;
    const int Hkv = kv_heads > 0 ? kv_heads : H;
    const size_t e = elem_bytes(dt);
    const size_t qb = (size_t)B * H * L * d * e, kb = (size_t)B * Hkv * Nk * d * e;
    const Span ins[] = {{Q, qb}, {K, kb}, {V, kb}, {q_valid, (size_t)B * L},
                        {k_valid, (size_t)B * Nk}};
    for (const Span &i : ins)
        if (i.p && overlap(out, qb, i.p, i.n)) return CA_ERR_INVALID_ARG;
    // single launch when the future-key exclusion equals the listing's fill
    if (exact_fused_supported(L, Nk) && (!causal || !k_valid || k_valid == q_valid))
        return hip_status(launch_exact_fused(Q, K, V, B * H, L, causal != 0, dt, q_valid, k_valid,
                                             H, H / Hkv, out, stream, device_cus()));
    return hip_status(launch_exact_attention(Q, K, V, B * H, L, Nk, causal != 0, dt, q_valid,
                                             k_valid, H, H / Hkv, out, stream));
}

ca_status_t ca_kmeans_assign(const void *Q, const float *mu, int S, int L, int d, int Kc,
                             ca_dtype_t dt, int32_t *assign, hipStream_t stream) {
    ca_status_t st = check_step(S, L, d, Kc, dt);
    if (st != CA_OK) return st;
    if (!Q || !assign) return CA_ERR_INVALID_ARG;
    if (!mu && Kc > L) return CA_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || (mu && !aligned(mu, 16)) || !aligned(assign, 4))
        return CA_ERR_INVALID_ARG;
    return hip_status(launch_kmeans_assign(Q, mu, S, L, Kc, dt, assign, nullptr, nullptr, stream));
}

ca_status_t ca_kmeans_scores(const void *Q, const float *mu, int S, int L, int d, int Kc,
                             ca_dtype_t dt, float *scores, hipStream_t stream) {
    ca_status_t st = check_step(S, L, d, Kc, dt);
    if (st != CA_OK) return st;
    if (!kmeans_mfma_supported(Kc)) return CA_ERR_UNSUPPORTED;
    if (!Q || !mu || !scores) return CA_ERR_INVALID_ARG;
    if ((long long)S * L * Kc > (1LL << 40)) return CA_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(mu, 16) || !aligned(scores, 4)) return CA_ERR_INVALID_ARG;
    const size_t sb = sizeof(float) * (size_t)S * L * Kc;
    if (overlap(scores, sb, Q, (size_t)S * L * d * elem_bytes(dt)) ||
        overlap(scores, sb, mu, sizeof(float) * (size_t)S * Kc * d))
        return CA_ERR_INVALID_ARG;
    return hip_status(launch_kmeans_scores(Q, mu, S, L, Kc, dt, scores, stream));
}

size_t ca_centroid_update_workspace_size(int S, int L, int d, int Kc) {
    if (check_step(S, L, d, Kc, CA_F32) != CA_OK) return 0;
    const size_t n = (size_t)S * kmeans_tiles(L) * Kc;
    return align_up(sizeof(float) * n * kD) + align_up(sizeof(int32_t) * n);
}

ca_status_t ca_centroid_update(const void *Q, const int32_t *assign, int S, int L, int d, int Kc,
                               ca_dtype_t dt, float *mu, int32_t *counts, void *workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    ca_status_t st = check_step(S, L, d, Kc, dt);
    if (st != CA_OK) return st;
    if (!Q || !assign || !mu || !workspace) return CA_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(mu, 16) || !aligned(assign, 4) ||
        (counts && !aligned(counts, 4)) || !aligned(workspace, kAlign))
        return CA_ERR_INVALID_ARG;
    if (workspace_bytes < ca_centroid_update_workspace_size(S, L, d, Kc)) return CA_ERR_INVALID_ARG;
    // per-tile partial sums of the given assignment, then the tile-order sum
    const size_t n = (size_t)S * kmeans_tiles(L) * Kc;
    char *ws = static_cast<char *>(workspace);
    float *psum = reinterpret_cast<float *>(ws);
    int32_t *pcnt = reinterpret_cast<int32_t *>(ws + align_up(sizeof(float) * n * kD));
    CA_TRY(launch_centroid_partials(Q, assign, S, L, Kc, dt, psum, pcnt, stream));
    return hip_status(launch_centroid_reduce(psum, pcnt, kmeans_tiles(L), S, Kc, mu, counts, stream));
}

size_t ca_centroid_xattn_workspace_size(int S, int L, int d, int Kc) {
    if (check_step(S, L, d, Kc, CA_F32) != CA_OK) return 0;
    const int nsplit = xattn_splits(L);
    return nsplit > 1 ? align_up(sizeof(float) * (size_t)S * nsplit * Kc * (kD + 2)) : 0;
}

ca_status_t ca_centroid_xattn(const float *mu, const void *K, const void *V, int S, int L, int d,
                              int Kc, ca_dtype_t dt, float *vcent, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    ca_status_t st = check_step(S, L, d, Kc, dt);
    if (st != CA_OK) return st;
    if (!mu || !K || !V || !vcent) return CA_ERR_INVALID_ARG;
    if (!aligned(mu, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(vcent, 16))
        return CA_ERR_INVALID_ARG;
    const size_t need = ca_centroid_xattn_workspace_size(S, L, d, Kc);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)))
        return CA_ERR_INVALID_ARG;
    return hip_status(launch_centroid_xattn(mu, K, V, S, L, Kc, dt, nullptr, 1, 1, vcent,
                                            static_cast<float *>(workspace), stream));
}

ca_status_t ca_local_window_attn(const void *Q, const void *K, const void *V, int S, int L, int d,
                                 int W, ca_dtype_t dt, float *oloc, hipStream_t stream) {
    ca_status_t st = check_step(S, L, d, 1, dt);
    if (st != CA_OK) return st;
    if (W < 0 || !Q || !K || !V || !oloc) return CA_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(oloc, 16))
        return CA_ERR_INVALID_ARG;
    return hip_status(launch_local_window(Q, K, V, S, L, W / 2, dt, nullptr, nullptr, 1, 1.f,
                                          nullptr, 1, 1, nullptr, oloc, stream));
}

ca_status_t ca_gather_fuse(const float *vcent, const int32_t *assign, const float *oloc, int S,
                           int L, int d, int Kc, float alpha, ca_dtype_t dt, void *out,
                           hipStream_t stream) {
    ca_status_t st = check_step(S, L, d, Kc, dt);
    if (st != CA_OK) return st;
    if (!(alpha >= 0.f && alpha <= 1.f)) return CA_ERR_INVALID_ARG;
    if (!vcent || !assign || !oloc || !out) return CA_ERR_INVALID_ARG;
    if (!aligned(vcent, 16) || !aligned(oloc, 16) || !aligned(out, 16) || !aligned(assign, 4))
        return CA_ERR_INVALID_ARG;
    return hip_status(launch_gather_fuse(vcent, assign, oloc, S, L, Kc, alpha, dt, out, stream));
}

size_t cluster_attn_layer_workspace_size(int B, int L, int Dm, int H, int d, int nclust) {
    if (check_layer(B, L, Dm, H, d, nclust, 1, 0, 0.f) != CA_OK) return 0;
    return layer_layout(B, L, Dm, H, nclust).total;
}

ca_status_t cluster_attn_layer_forward(const void *X, const void *Wq, const void *Wk,
                                       const void *Wv, const void *Wo, int B, int L, int Dm,
                                       int H, int d, int nclust, int iters, int W, float alpha,
                                       void *Y, int32_t *assign_out, void *qkv_out,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    ca_status_t st = check_layer(B, L, Dm, H, d, nclust, iters, W, alpha);
    if (st != CA_OK) return st;
    if (!X || !Wq || !Wk || !Wv || !Wo || !Y || !workspace) return CA_ERR_INVALID_ARG;
    const void *ptrs16[] = {X, Wq, Wk, Wv, Wo, Y, qkv_out};
    for (const void *q : ptrs16)
        if (q && !aligned(q, 16)) return CA_ERR_INVALID_ARG;
    if (assign_out && !aligned(assign_out, 4)) return CA_ERR_INVALID_ARG;
    if (!aligned(workspace, kAlign)) return CA_ERR_INVALID_ARG;
    const LayerLayout lay = layer_layout(B, L, Dm, H, nclust);
    if (workspace_bytes < lay.total) return CA_ERR_INVALID_ARG;
    const size_t tok = (size_t)B * L;
    const size_t act = sizeof(uint16_t) * tok * Dm, wbytes = sizeof(uint16_t) * (size_t)Dm * Dm;
    // outputs and workspace must not overlap each other or the inputs
    const Span outs[] = {{Y, act}, {assign_out, sizeof(int32_t) * tok * H},
                         {qkv_out, 3 * act}, {workspace, lay.total}};
    if (any_overlap(outs, 4)) return CA_ERR_INVALID_ARG;
    const Span ins[] = {{X, act}, {Wq, wbytes}, {Wk, wbytes}, {Wv, wbytes}, {Wo, wbytes}};
    for (const Span &o : outs)
        for (const Span &i : ins)
            if (o.p && overlap(o.p, o.n, i.p, i.n)) return CA_ERR_INVALID_ARG;

    char *ws = static_cast<char *>(workspace);
    uint16_t *qkv = qkv_out ? static_cast<uint16_t *>(qkv_out)
                            : reinterpret_cast<uint16_t *>(ws + lay.qkv);
    uint16_t *heads[3] = {qkv, qkv + tok * Dm, qkv + 2 * tok * Dm};
    uint16_t *O = reinterpret_cast<uint16_t *>(ws + lay.o);
    // the weights are read in their [in, out] layout
    const uint16_t *wqkv[3] = {static_cast<const uint16_t *>(Wq), static_cast<const uint16_t *>(Wk),
                               static_cast<const uint16_t *>(Wv)};
    CA_TRY(launch_gemm_bf16(static_cast<const uint16_t *>(X), wqkv, heads, 3, (int)tok, Dm, Dm,
                            true, false, true, L, H, device_cus(), stream));
    st = forward_impl(heads[0], heads[1], heads[2], nullptr, 1, 0, B, H, L, d, nclust, iters, W,
                      alpha, O, assign_out, CA_BF16, ws + lay.attn, lay.attn_bytes, CA_PATH_AUTO,
                      stream);
    if (st != CA_OK) return st;
    const uint16_t *wo[1] = {static_cast<const uint16_t *>(Wo)};
    uint16_t *yv[1] = {static_cast<uint16_t *>(Y)};
    return hip_status(
        launch_gemm_bf16(O, wo, yv, 1, (int)tok, Dm, Dm, true, true, false, L, H, device_cus(),
                         stream));
}

static ca_status_t gemm_entry(const void *A, const void *B, int M, int N, int Kd, void *C,
                              bool w_kn, hipStream_t stream) {
    if (!A || !B || !C || M < 1 || N < 1 || Kd < 1) return CA_ERR_INVALID_ARG;
    if ((long long)M * Kd > (1LL << 40) || (long long)N * Kd > (1LL << 40) ||
        (long long)M * N > (1LL << 40))
        return CA_ERR_INVALID_ARG;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16)) return CA_ERR_INVALID_ARG;
    const size_t ca = sizeof(uint16_t) * (size_t)M * Kd, cb = sizeof(uint16_t) * (size_t)N * Kd,
                 cc = sizeof(uint16_t) * (size_t)M * N;
    if (overlap(C, cc, A, ca) || overlap(C, cc, B, cb)) return CA_ERR_INVALID_ARG;
    if (N % 64 != 0 || Kd % 64 != 0 || M > (1 << 30) || (long long)N * Kd >= (1LL << 31))
        return CA_ERR_UNSUPPORTED;
    const uint16_t *b[1] = {static_cast<const uint16_t *>(B)};
    uint16_t *c[1] = {static_cast<uint16_t *>(C)};
    return hip_status(launch_gemm_bf16(static_cast<const uint16_t *>(A), b, c, 1, M, N, Kd, w_kn,
                                       false, false, 1, 1, device_cus(), stream));
}

ca_status_t ca_gemm_bf16(const void *A, const void *Bt, int M, int N, int Kd, void *C,
                         hipStream_t stream) {
    return gemm_entry(A, Bt, M, N, Kd, C, false, stream);
}

ca_status_t ca_gemm_bf16_kn(const void *A, const void *W, int M, int N, int Kd, void *C,
                            hipStream_t stream) {
    return gemm_entry(A, W, M, N, Kd, C, true, stream);
}

}  // extern "C"
