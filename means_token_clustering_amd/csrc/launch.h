// Host-side launch helpers of the cluster attention library: each is
// defined in one .hip file and declared here so that the C-ABI translation
// unit (api.hip) can call it. Device helpers live in common.h.
#pragma once

#include "staged.h"

// Host-side launch helpers live in the .hip files; declared here so the
// C-ABI translation unit can call them.
namespace ca {

// Listing-compatible variants of the clustering and the gather (the
// ClusterAttention listing on the "Hooshaai/svd-sst2-roberta-cluster" page,
// its k-means routine and forward).
struct Variant {
    int init_step;     // 0: initial rows floor(k L / Kc); > 0: rows k * init_step
    bool keep_empty;   // an empty cluster keeps its previous centroid (else zero)
    bool soft;         // gather sum_k softmax_k(q . mu_k / sqrt(d)) V^cent_k
};

// Row of Q that initialises cluster k (increasing in k, below L for Kc <= L).
__host__ __device__ inline int init_row(int k, int L, int Kc, int init_step) {
    return init_step > 0 ? k * init_step : (int)(((long)k * L) / Kc);
}

// Lets kernel fn launch with `bytes` of dynamic LDS on the current device:
// hipFuncSetAttribute runs only when the device has not yet been given a limit
// at least that large for fn (once per kernel and device in practice).
hipError_t ensure_dynamic_lds(const void *fn, int bytes);

// mu == nullptr: the centroids are the initial rows of Q (init_row with
// init_step); mu_init, if not null, then receives them.
hipError_t launch_kmeans_assign(const void *Q, const float *mu, int S, int L, int Kc,
                                ca_dtype_t dt, int32_t *assign, float *part_sum,
                                int32_t *part_cnt, hipStream_t st, int init_step = 0,
                                float *mu_init = nullptr);
hipError_t launch_centroid_partials(const void *Q, const int32_t *assign, int S, int L, int Kc,
                                    ca_dtype_t dt, float *part_sum, int32_t *part_cnt,
                                    hipStream_t st);
int kmeans_tiles(int L);
// keep_empty: an empty cluster leaves its row of mu as it was
hipError_t launch_centroid_reduce(const float *part_sum, const int32_t *part_cnt, int nblk,
                                  int S, int Kc, float *mu, int32_t *counts, hipStream_t st,
                                  bool keep_empty = false);

// One Lloyd step on the matrix cores (kmeans_mfma.hip) for K <= 64: the
// assignment and the cluster sums / sizes of each run of nsub 128-token
// blocks, laid out as launch_kmeans_assign's partials with
// kmeans_mfma_parts(L, nsub) runs per slice; part_sum == nullptr: assignment
// only. With prev_sum / prev_cnt (the previous step's partials, same nsub)
// the centroids are formed from them in run order instead of being read
// from mu. kmeans_mfma_run picks nsub for S slices on cus compute units.
// qmax (nsub > 1, nullable; [S, runs] words): the first step (mu == nullptr)
// writes each run's largest |q|, and a later step given it scales the whole
// run at once.
bool kmeans_mfma_supported(int Kc);
int kmeans_mfma_blocks(int L);
int kmeans_mfma_run(long S, int L, int cus);
int kmeans_mfma_parts(int L, int nsub);
hipError_t launch_kmeans_mfma(const void *Q, const float *mu, int S, int L, int Kc,
                              ca_dtype_t dt, int32_t *assign, float *part_sum, int32_t *part_cnt,
                              hipStream_t st, int init_step = 0, float *mu_init = nullptr,
                              const float *prev_sum = nullptr, const int32_t *prev_cnt = nullptr,
                              int nsub = 1, uint32_t *qmax = nullptr);

// Scores mu_k . q_i - ||mu_k||^2 / 2 of the matrix-core step (Kc <= 64) in
// unscaled units, [S, L, Kc]: the distances the step compares.
hipError_t launch_kmeans_scores(const void *Q, const float *mu, int S, int L, int Kc,
                                ca_dtype_t dt, float *scores, hipStream_t st);

// The whole forward in one launch per slice for 128 < L <= 512, K <= 16,
// radius <= 16, without a key-padding mask (fused512.hip); assign nullable.
// split_ws (256-byte aligned, fused512_split_workspace_bytes(S) bytes): the
// split form, a second workgroup per slice running the window branch beside
// the clustering (2 S workgroups, one per CU: only for 2 S <= the CU count),
// preceded by a small launch that clears its flags.
bool fused512_supported(int L, int Kc, int r);
size_t fused512_split_workspace_bytes(long S);
int fused512_split_max_slices();   // largest S of the split form
hipError_t launch_fused512(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                           int iters, int r, float alpha, int init_step, ca_dtype_t dt, int H,
                           int G, void *out, int32_t *assign, hipStream_t st,
                           int32_t *hist = nullptr, void *split_ws = nullptr);

// The whole forward in one launch with each slice split over ns co-resident
// workgroups of at most 480 tokens (seg.hip): K <= 64, radius <= 16, no mask
// or listing variants. seg_count: ns for this shape on a device with `cus`
// compute units (0: not supported); the launch needs seg_workspace_bytes of
// workspace (256-byte aligned).
int seg_count(long S, int L, int Kc, int r, int cus);
size_t seg_workspace_bytes(long S, int L, int Kc, int ns);
hipError_t launch_seg(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                      int iters, int r, float alpha, int init_step, ca_dtype_t dt, int H, int G,
                      void *out, int32_t *assign, int ns, void *workspace, hipStream_t st,
                      int32_t *hist = nullptr);

// All Lloyd iterations of each slice in one launch (kmeans_slice.hip) for
// L <= 512, K <= 16: the last assignment and the final centroids mu [S, K, 64].
bool kmeans_slice_supported(int L, int Kc);
hipError_t launch_kmeans_slice(const void *Q, int S, int L, int Kc, int iters, ca_dtype_t dt,
                               int32_t *assign, float *mu, int init_step, hipStream_t st,
                               int32_t *hist = nullptr);
// The same clustering followed by the centroid attention's four key-range
// partials (xpart, unmasked) in one launch of 2 S workgroups, for 384 < L <=
// 512 and 2 S <= cus (every workgroup resident at once).
bool kmeans_xattn_supported(long S, int L, int Kc, int cus);
hipError_t launch_kmeans_xattn(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                               int iters, ca_dtype_t dt, int32_t *assign, float *mu,
                               int init_step, int H, int G, float *xpart, hipStream_t st,
                               int32_t *hist = nullptr);

// key ranges per slice of the centroid cross-attention (partials when > 1)
int xattn_splits(int L);
// one range partial: acc[64] (unnormalised context), largest logit (natural-log
// units), sum of exp(logit - largest); [S, nsplit, Kc] of them
constexpr int kXPartStride = 64 + 2;
// ranges whose partials the window kernel merges itself (no combine launch)
constexpr int kXMergeInLocal = 4;
// valid: key-padding mask [B, L] (nonzero = real token) or nullptr; slice s
// belongs to batch row s / H. G: query heads per K/V head (see kv_slice).
// stats (nullable, [S, Kc, 2]): per row the largest scaled logit and the sum
// of exp(logit - largest). combine = false leaves more than one range as
// partials only (vcent untouched), for launch_local_mfma to merge.
hipError_t launch_centroid_xattn(const float *mu, const void *K, const void *V, int S, int L,
                                 int Kc, ca_dtype_t dt, const uint8_t *valid, int H, int G,
                                 float *vcent, float *partials, hipStream_t st,
                                 float *stats = nullptr, bool combine = true);

// Window |i - j| <= r. With oloc == nullptr the gather + fusion epilogue
// writes out; mu != nullptr selects the soft gather over the centroids mu.
hipError_t launch_local_window(const void *Q, const void *K, const void *V, int S, int L, int r,
                               ca_dtype_t dt, const float *vcent, const int32_t *assign, int Kc,
                               float alpha, const uint8_t *valid, int H, int G, void *out,
                               float *oloc, hipStream_t st, const float *mu = nullptr);
// The same window branch with the fused epilogue on the matrix cores
// (local_mfma.hip), for radius r <= 16 and the hard gather. With xpart set
// (xattn_splits(L) ranges, 2 .. kXMergeInLocal), the gathered row is merged
// from the unmerged range partials instead of read from vcent.
bool local_mfma_supported(int r);
hipError_t launch_local_mfma(const void *Q, const void *K, const void *V, int S, int L, int r,
                             ca_dtype_t dt, const float *vcent, const int32_t *assign, int Kc,
                             float alpha, const uint8_t *valid, int H, int G, void *out,
                             hipStream_t st, const float *xpart = nullptr);
// The clustering (kmeans_slice) with the window blocks of the same slices
// beside it in one launch (every slice's block count times S even): the
// window blocks store alpha O^loc as fp32 [S, L, 64] rows in oloc (zero for
// padded queries when valid is set), and
// launch_gather_oloc forms out = (1 - alpha) V^cent_{c_i} + that row (with
// xpart: V^cent merged from 2 .. kXMergeInLocal key-range partials).
bool kmeans_window_supported(long S, int L, int Kc, int r);
hipError_t launch_kmeans_window(const void *Q, const void *K, const void *V, int S, int L,
                                int Kc, int iters, ca_dtype_t dt, int32_t *assign, float *mu,
                                int init_step, int r, float alpha, const uint8_t *valid, int H,
                                int G, float *oloc, hipStream_t st, int32_t *hist = nullptr);
hipError_t launch_gather_oloc(const float *oloc, const int32_t *assign, const float *vcent,
                              const float *xpart, int S, int L, int Kc, float alpha,
                              const uint8_t *valid, int H, ca_dtype_t dt, void *out,
                              hipStream_t st);
hipError_t launch_gather_fuse(const float *vcent, const int32_t *assign, const float *oloc, int S,
                              int L, int Kc, float alpha, ca_dtype_t dt, void *out,
                              hipStream_t st);

// Backward pass (backward.hip): buffers and sizes of one launch sequence.
// Q, dO, dQ [B, H, L, 64]; K, V, dK, dV [B, Hkv, L, 64] (storage dtype);
// assign [B, H, L]; the rest fp32 workspace: mu, vcent, dvc, dmu [S, Kc, 64],
// counts [S, Kc], cstat [S, Kc, 2] (row max and sum of the centroid
// softmax), part [S, tiles, Kc, 64], lstat [S, L] (max, sum, D, 0 of the
// local softmax), dal [S * tiles]; dalpha (nullable) one float.
struct BwdArgs {
    const void *Q, *K, *V, *dO;
    const int32_t *assign;
    const uint8_t *valid;
    int B, H, Hkv, L, Kc, r;
    float alpha;
    const float *mu;
    const int32_t *counts;
    const float *vcent, *cstat;
    float *dvc, *dmu, *part;
    float4 *lstat;
    float *dal;
    void *dQ, *dK, *dV;
    float *dalpha;
    // fp32 [S, L, 64] shares of the centroid branch in dK and dV; nullable
    // (then the staged sequence runs for every shape)
    float *dkc, *dvl;
    // two-launch form: workgroups alone on their CU, [solo_lo, solo_hi) (two
    // workgroups fit a CU; with CUs < S < 2 CUs these are S - CUs .. CUs - 1)
    int solo_lo, solo_hi;
};
int bwd_tiles(int L);
hipError_t launch_backward(const BwdArgs &a, ca_dtype_t dt, hipStream_t st);
// out[0] = sum of part[0 .. n) in a fixed order (nothing when out is null)
hipError_t launch_bwd_sum(const float *part, long n, float *out, hipStream_t st);
// The backward pass in two launches per slice (backward_fused.hip) for
// L <= 128, K <= 16 and one query head per K/V head: the centroid branch
// (dK, dV shares in dkc, dvl; dmu; counts; the centroid term of dalpha in
// lstat's first S floats), then the local branch with the final dQ, dK, dV
// and the slices' dalpha in dal.
bool bwd_fused_supported(int L, int Kc, int G);
hipError_t launch_backward_fused(const BwdArgs &a, ca_dtype_t dt, hipStream_t st);

// Exact attention (decoder / cross-attention branch): Q [S, L, 64], K, V
// [S / G, Nk, 64] (grouped heads as in kv_slice); qvalid [S / H, L], kvalid
// [S / H, Nk] nullable.
hipError_t launch_exact_attention(const void *Q, const void *K, const void *V, int S, int L,
                                  int Nk, bool causal, ca_dtype_t dt, const uint8_t *qvalid,
                                  const uint8_t *kvalid, int H, int G, void *out, hipStream_t st);

// Single-launch exact attention for L = Nk <= 128 (fused.hip); the host sends
// a causal launch here only when every real query has a real key at or
// before it (no key mask, or the query mask itself).
bool exact_fused_supported(int L, int Nk);
hipError_t launch_exact_fused(const void *Q, const void *K, const void *V, int S, int L,
                              bool causal, ca_dtype_t dt, const uint8_t *qvalid,
                              const uint8_t *kvalid, int H, int G, void *out, hipStream_t st,
                              int cus = 0);   // cus: the device's CU count (0: unknown)

bool fused_supported(int L, int Kc);
hipError_t launch_fused_forward(const void *Q, const void *K, const void *V, int S, int L, int Kc,
                                int iters, int radius, float alpha, const Variant &var,
                                ca_dtype_t dt, const uint8_t *valid, int H, int G, void *out,
                                int32_t *assign, hipStream_t st, int32_t *hist = nullptr,
                                int cus = 0);   // cus: the device's CU count (0: unknown)

// C[z] = A . W[z] for z < count (bf16 bits, fp32 accumulation): w_kn, W[z]
// is [K, N] row-major; otherwise B[z] is Bt [N, K] and C = A . Bt^T.
// a_heads: A is [B, H, L, 64] read as [B*L, 64 H]; c_heads: C[z] is written
// as [B, H, L, 64] from [B*L, 64 H] (both only with w_kn). N a multiple of
// 64, K of 64, N*K < 2^31, count <= 4.
// cus: compute units of the device (picks the tile shape).
hipError_t launch_gemm_bf16(const uint16_t *A, const uint16_t *const *B, uint16_t *const *C,
                            int count, int M, int N, int K, bool w_kn, bool a_heads, bool c_heads,
                            int L, int H, int cus, hipStream_t st);

}  // namespace ca
