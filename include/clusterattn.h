/*
 * clusterattn.h - C ABI of the MI355X (gfx950) cluster attention library.
 *
 * The operation (forward pass of Cluster Attention, inference):
 *   model card "Hooshaai/distilbert-sst2-cluster-attention", Architecture
 *   Overview (pipeline figure) and Mathematical Formulation 1; "ClusterFormer"
 *   specification on the "Hooshaai/svd-sst2-roberta-cluster" page, sections
 *   2.1 and 3. Per (batch b, head h) slice, with tokens i = 0..L-1:
 *     K       = min(nclust, L) clusters
 *     mu^(0)  = Q[floor(k L / K)]                       (strided init)
 *     for t = 1..iters:
 *       c_i   = argmin_k ||q_i - mu_k||^2               (lowest k on ties)
 *       mu_k  = sum_{c_i = k} q_i / max(1, n_k)         (empty -> zero vector)
 *     Vc_k    = softmax_j(mu_k . k_j / sqrt(d)) v_j     (all L keys)
 *     Ol_i    = softmax_j(q_i . k_j / sqrt(d)) v_j      (|i - j| <= floor(W/2))
 *     O_i     = (1 - alpha) Vc_{c_i} + alpha Ol_i
 *   The clustering returns (c^(iters), mu^(iters)); no dropout; the key-
 *   padding mask of padded batches is cluster_attn_forward_masked.
 *
 * Conventions shared by every entry point:
 *   - Tensors are device pointers to contiguous row-major arrays. "[B,H,L,d]"
 *     means slice s = b*H + h holds rows s*L .. s*L+L-1 of d elements each.
 *   - Storage dtype CA_F32 (float) or CA_BF16 (uint16 bf16 bits). Results
 *     are fp32-accurate: contractions run on the fp16 matrix cores as three
 *     products of an fp16 split (high and remainder parts) of each fp32
 *     operand with fp32 accumulation; everything else is fp32. A bf16 output
 *     is rounded to nearest-even once, at the store. Centroids, centroid
 *     context and partials are always fp32.
 *   - d must be 64 (CA_ERR_UNSUPPORTED otherwise); K = min(nclust, L) must
 *     be <= 256 (CA_ERR_UNSUPPORTED otherwise).
 *   - Ownership: the caller owns every buffer, including the workspace; the
 *     library never allocates, frees or synchronises. Work is enqueued on
 *     `stream` (0 = the null stream) and runs asynchronously.
 *   - Errors: argument errors are detected on the host before any launch and
 *     leave all outputs untouched (CA_ERR_INVALID_ARG / CA_ERR_UNSUPPORTED).
 *     A failed launch returns CA_ERR_HIP.
 *   - Alignment: tensor pointers must be 16-byte aligned, int32 pointers
 *     4-byte aligned, the workspace 256-byte aligned.
 *   - Determinism: no floating-point atomics; every reduction has a fixed
 *     order, so identical inputs give bitwise identical outputs, and a run
 *     with iters = t reproduces the first t iterations of a longer run.
 *   - Reentrancy: no global mutable state; concurrent calls on different
 *     streams must use different workspaces and outputs.
 */
#ifndef CLUSTERATTN_H
#define CLUSTERATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CA_OK = 0,
    CA_ERR_INVALID_ARG = 1,
    CA_ERR_UNSUPPORTED = 2,
    CA_ERR_HIP = 3,
    CA_ERR_SCRATCH_TOO_SMALL = 4   /* cluster_attn_forward_noalloc only */
} ca_status_t;

typedef enum { CA_F32 = 0, CA_BF16 = 1 } ca_dtype_t;

/* Execution strategy of cluster_attn_forward_ex. AUTO picks the fastest
 * launch sequence for the shape, storage type and CU count (see
 * cluster_attn_forward_ex and cluster_attn_plan_dt). FUSED: one launch, one
 * workgroup per slice, the whole slice on chip. STAGED: one kernel per step,
 * any supported shape. */
typedef enum {
    CA_PATH_AUTO = 0,
    CA_PATH_FUSED = 1,
    CA_PATH_STAGED = 2,
    CA_PATH_SEGMENTED = 3   /* one launch, each slice over several co-resident workgroups */
} ca_path_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *ca_status_string(ca_status_t s);

/* Library version, major*10000 + minor*100 + patch. */
int ca_version(void);

/*
 * Bytes of workspace cluster_attn_forward needs for this shape (0 when the
 * fused path applies). Returns 0 for invalid arguments as well; the forward
 * call reports those.
 */
size_t cluster_attn_workspace_size(int B, int H, int L, int d, int nclust,
                                   ca_dtype_t dt);

/*
 * Cluster attention forward (the whole operation above).
 *   Q, K, V     in   device, [B,H,L,d], dtype dt.
 *   B, H, L, d       all >= 1; d == 64.
 *   nclust           >= 1; clamped to L.
 *   iters            >= 1 Lloyd iterations.
 *   W                >= 0 window width; radius floor(W/2).
 *   alpha            fusion weight, 0 <= alpha <= 1 (NaN rejected).
 *   out         out  device, [B,H,L,d], dtype dt; must not overlap Q, K, V.
 *   assign_out  out  device, [B,H,L] int32 in [0, min(nclust,L)); may be NULL.
 *   workspace        device, >= cluster_attn_workspace_size(...) bytes; may
 *                    be NULL when that size is 0.
 */
ca_status_t cluster_attn_forward(const void *Q, const void *K, const void *V,
                                 int B, int H, int L, int d, int nclust,
                                 int iters, int W, float alpha, void *out,
                                 int32_t *assign_out, ca_dtype_t dt,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Same as cluster_attn_forward with an explicit strategy. CA_PATH_FUSED runs
 * one launch per slice: any supported call with L <= 128 and nclust <= 16, or
 * 128 < L <= 512 with min(nclust, L) <= 16, a window radius <= 16 and neither
 * a key-padding mask nor the kept-centroid or soft-gather variants; on other
 * shapes it returns CA_ERR_UNSUPPORTED. CA_PATH_SEGMENTED runs one launch in
 * which each slice is split into segments of at most 480 tokens, one
 * workgroup each, all resident at once (B * H * segments <= the device's
 * compute units, at least two segments per slice), for min(nclust, L) <= 64,
 * a window radius <= 16 and neither a mask nor a listing variant; otherwise
 * CA_ERR_UNSUPPORTED. Its workgroups wait for one another between steps; a
 * wait longer than about 7 ms (possible only while other work holds the CUs
 * it needs) turns the affected output rows into NaN and their assignments
 * into -1. CA_PATH_AUTO picks the single launch for L <= 128; for
 * longer slices (L <= 512, nclust <= 16, W / 2 <= 16, no mask or listing
 * variant) with bf16 storage and at most half of the compute units' worth
 * of slices, the split form of the 512-token single launch (a second
 * workgroup per slice for the window branch; its bounded waits turn the
 * affected output rows into NaN if they ever give up); the 512-token single
 * launch when the slice count fills between half and all of the compute
 * units; else the staged launches (the segmented launch only when asked
 * for). AUTO, STAGED and SEGMENTED need cluster_attn_workspace_size_ex(...,
 * path) bytes. */
ca_status_t cluster_attn_forward_ex(const void *Q, const void *K, const void *V,
                                    int B, int H, int L, int d, int nclust,
                                    int iters, int W, float alpha, void *out,
                                    int32_t *assign_out, ca_dtype_t dt,
                                    void *workspace, size_t workspace_bytes,
                                    ca_path_t path, hipStream_t stream);

size_t cluster_attn_workspace_size_ex(int B, int H, int L, int d, int nclust,
                                      ca_dtype_t dt, ca_path_t path);

/*
 * Name of the launch sequence that cluster_attn_forward_opts (with the same
 * B, H, L, nclust, W, flags, a mask when masked != 0, and path) takes on the
 * current device, as a static string: "fused" (one launch per slice,
 * L <= 128), "fused512" (one 16-wave launch per slice, 128 < L <= 512), or
 * "staged: ..." naming its clustering, centroid-attention and window
 * launches. NULL when such a call would be rejected. For labelling and
 * tests; the forward decides the same way on its own.
 */
const char *cluster_attn_plan(int B, int H, int L, int nclust, int W, int flags, int masked,
                              ca_path_t path);

/*
 * cluster_attn_plan for the storage type dt (cluster_attn_plan itself answers
 * for CA_F32). With CA_BF16, 128 < L <= 512, nclust <= 16, W / 2 <= 16, no
 * mask or listing variant and B * H slices filling at most half of the CUs,
 * the auto path takes "fused512 split (clustering and window workgroups)":
 * a second workgroup per slice forms the window branch beside the clustering
 * and writes the fused rows once the clustering workgroup has published its
 * centroid context (the rows come out as NaN if that wait ever gave up).
 */
const char *cluster_attn_plan_dt(int B, int H, int L, int nclust, int W, int flags, int masked,
                                 ca_path_t path, ca_dtype_t dt);

/*
 * Cluster attention with a key-padding mask (padded batches): the
 * ClusterAttention listing on the "Hooshaai/svd-sst2-roberta-cluster" page,
 * forward, bidirectional branch (its attention_mask path).
 *   valid       in   device, [B, L] uint8: nonzero = real token, 0 = padding;
 *                    row b serves the H heads of batch element b. NULL is
 *                    CA_ERR_INVALID_ARG (call cluster_attn_forward_ex).
 *   Semantics: a padded key's scaled score is replaced by -10000 in the
 *   centroid-key softmax and inside the local window; the output row of a
 *   padded query is zero; the clustering runs over all L tokens, padded ones
 *   included, and assign_out reports every token.
 *   Every other argument, the workspace size and the paths are those of
 *   cluster_attn_forward_ex; valid must not overlap out, assign_out or the
 *   workspace.
 */
ca_status_t cluster_attn_forward_masked(const void *Q, const void *K, const void *V,
                                        const uint8_t *valid, int B, int H, int L, int d,
                                        int nclust, int iters, int W, float alpha, void *out,
                                        int32_t *assign_out, ca_dtype_t dt,
                                        void *workspace, size_t workspace_bytes,
                                        ca_path_t path, hipStream_t stream);

/*
 * Options of cluster_attn_forward_opts (zero-initialise, then set fields).
 *   valid     key-padding mask as in cluster_attn_forward_masked, or NULL.
 *   kv_heads  heads of K and V: 0 (or H) means H; otherwise H must be a
 *             multiple of kv_heads and the G = H / kv_heads consecutive query
 *             heads h = G*j .. G*j+G-1 share K/V head j (grouped-query
 *             attention, the listing's repeat_kv on the "Hooshaai/svd-sst2-
 *             roberta-cluster" page; K and V are then [B, kv_heads, L, d]).
 *   flags     OR of CA_FLAG_* below, each a rule of the ClusterAttention
 *             listing on the "Hooshaai/svd-sst2-roberta-cluster" page where it
 *             departs from the model card's equations (0 = the equations);
 *             another bit is CA_ERR_INVALID_ARG.
 *   assign_hist  NULL, or device int32 [iters, B, H, L] (4-byte aligned)
 *             receiving the assignment of every Lloyd iteration: slot t-1
 *             holds c^(t), the assignment against mu^(t-1) (model card,
 *             Mathematical Formulation 1; ClusterFormer 2.1, t = 1..iters), so
 *             slot iters-1 equals assign_out. It must not overlap any other
 *             argument buffer. Every path writes it; it changes no other
 *             output. Slot t-1 equals assign_out of the same call with
 *             iters = t (prefix determinism).
 */
typedef struct {
    const uint8_t *valid;
    int kv_heads;
    int flags;
    int32_t *assign_hist;
} ca_options_t;

/* Initial centroids mu_k = Q[k * max(1, floor(L / K))] (the listing's k-means
 * routine) instead of Q[floor(k L / K)]. */
#define CA_FLAG_INIT_STEP 1
/* An empty cluster keeps its previous centroid (the listing's update) instead
 * of becoming the zero vector. */
#define CA_FLAG_KEEP_EMPTY 2
/* Soft gather (the listing's forward): token i takes sum_k softmax_k(q_i .
 * mu_k / sqrt(d)) V^cent_k over the final centroids instead of V^cent_{c_i}
 * (the key-padding mask does not enter this softmax). assign_out still
 * reports the last assignment. */
#define CA_FLAG_SOFT_GATHER 4
/* Band of radius W (|i - j| <= W, the listing's local mask) instead of
 * floor(W / 2); with W == 0 or W >= L there is no local branch and the
 * output is the gathered context alone (alpha is then ignored). */
#define CA_FLAG_BAND 8
/* alpha is the listing's parameter and the weight is its logistic sigmoid
 * 1 / (1 + exp(-alpha)) (any value but NaN; the weight is rounded to float);
 * without this flag alpha is the weight itself, in [0, 1]. */
#define CA_FLAG_ALPHA_LOGIT 16
/* All five: the listing's forward. */
#define CA_FLAG_LISTING 31

/*
 * cluster_attn_forward_ex with options (opts NULL = defaults, which is
 * cluster_attn_forward_ex itself). Workspace size: cluster_attn_workspace_size_ex
 * of the same B, H, L. K and V must not overlap out, assign_out or the
 * workspace; the mask rules are those of cluster_attn_forward_masked.
 */
ca_status_t cluster_attn_forward_opts(const void *Q, const void *K, const void *V, int B,
                                      int H, int L, int d, int nclust, int iters, int W,
                                      float alpha, const ca_options_t *opts, void *out,
                                      int32_t *assign_out, ca_dtype_t dt, void *workspace,
                                      size_t workspace_bytes, ca_path_t path,
                                      hipStream_t stream);

/*
 * Allocation-free variant of cluster_attn_forward_opts, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, results and paths
 * as cluster_attn_forward_opts, without the workspace: a staged call takes
 * its workspace from a device array of CA_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (the single-
 * launch paths need none). The call allocates and frees nothing.
 *   Errors: CA_ERR_SCRATCH_TOO_SMALL, before any launch and with the outputs
 *   untouched, when cluster_attn_workspace_size_ex(B, H, L, d, nclust, dt,
 *   path) exceeds CA_NOALLOC_SCRATCH_BYTES; CA_ERR_HIP if the array's address
 *   cannot be looked up; otherwise the statuses of cluster_attn_forward_opts.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (different streams, or different host threads) race and must
 *   be serialised by the caller. The array keeps the last call's contents;
 *   no call relies on them.
 */
#define CA_NOALLOC_SCRATCH_BYTES (64u << 20)
ca_status_t cluster_attn_forward_noalloc(const void *Q, const void *K, const void *V, int B,
                                         int H, int L, int d, int nclust, int iters, int W,
                                         float alpha, const ca_options_t *opts, void *out,
                                         int32_t *assign_out, ca_dtype_t dt, ca_path_t path,
                                         hipStream_t stream);

/*
 * Backward pass of the forward above (equations' rules, no listing flags):
 * the gradients of sum(dO * O) with the final assignment held fixed. The
 * pages fine-tune through the clustering (the svd-sst2-roberta-cluster page,
 * "Architectural Support": differentiable k-means; the model card's benchmark
 * table, "Post-KD Recovery"); the argmin itself is piecewise constant, so
 * the gradient flows through the final means mu_k = sum_{c_i = k} q_i / n_k
 * (each member receives dmu_k / n_k), both softmaxes, the gather and the
 * fusion. A padded key's -10000 logit is a constant (no gradient to q or k);
 * padded query rows pass no gradient through the output.
 *   Q, dO     in   device, [B, H, L, d], dtype dt (dO: the upstream gradient).
 *   K, V      in   device, [B, kv_heads, L, d] (kv_heads 0 means H).
 *   assign    in   device int32 [B, H, L]: the final assignment that the
 *                  forward wrote to assign_out (values outside [0, K) are
 *                  clamped into it).
 *   valid     in   nullable key-padding mask [B, L] (as in the forward).
 *   nclust, W, alpha: the forward's values (K = min(nclust, L)).
 *   dQ        out  [B, H, L, d]; dK, dV out [B, kv_heads, L, d]; dtype dt
 *                  (fp32 arithmetic, rounded once to bf16 for bf16 storage).
 *                  The G = H / kv_heads query heads of a group add into
 *                  their shared dK, dV.
 *   dalpha    out  nullable device pointer to one float: d/dalpha.
 *   workspace      device, 256-byte aligned, at least
 *                  cluster_attn_backward_workspace_size bytes.
 * Deterministic (fixed summation orders, no float atomics). Outputs and the
 * workspace must not overlap each other or the inputs. d = 64, K <= 256.
 * Errors are caught on the host before any launch.
 */
size_t cluster_attn_backward_workspace_size(int B, int H, int kv_heads, int L, int d,
                                            int nclust, ca_dtype_t dt);
ca_status_t cluster_attn_backward(const void *Q, const void *K, const void *V, const void *dO,
                                  const int32_t *assign, const uint8_t *valid, int B, int H,
                                  int kv_heads, int L, int d, int nclust, int W, float alpha,
                                  void *dQ, void *dK, void *dV, float *dalpha, ca_dtype_t dt,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Exact attention of the decoder and cross-attention branch: the
 * ClusterAttention listing on the "Hooshaai/svd-sst2-roberta-cluster" page
 * sends causal decoders and cross-attention to exact attention instead of
 * clustering ("Architectural Support" section; forward, decoder branch).
 *   out_i = sum_j softmax_j(s_ij) v_j over all Nk keys, s_ij = q_i . k_j /
 *   sqrt(d), replaced by -10000 where key j is padded (k_valid) or, with
 *   causal != 0, where j > i; the row of a padded query (q_valid) is zero.
 *   The -10000 is a fill: a row whose allowed keys are all padded is uniform
 *   over all Nk keys.
 *   Q, out    device, [B, H, L, d], dtype dt.
 *   K, V      device, [B, kv_heads, Nk, d] (kv_heads 0 means H; query head h
 *             reads K/V head h / (H / kv_heads)).
 *   q_valid   nullable device uint8 [B, L]; k_valid nullable [B, Nk];
 *             nonzero = real token (for self-attention pass one mask twice).
 * d = 64. Needs no workspace. out must not overlap the inputs. Errors are
 * caught on the host before any launch.
 */
ca_status_t cluster_attn_exact_forward(const void *Q, const void *K, const void *V,
                                       const uint8_t *q_valid, const uint8_t *k_valid, int B,
                                       int H, int kv_heads, int L, int Nk, int d, int causal,
                                       void *out, ca_dtype_t dt, hipStream_t stream);

/* ---------------------------------------------------------------------
 * Single steps (one kernel each), for callers composing their own loop and
 * for step-by-step checking. S = B*H slices; Kc = number of centroids.
 * --------------------------------------------------------------------- */

/*
 * One assignment step (model card, Mathematical Formulation 1; ClusterFormer
 * 2.1): assign[s,i] = argmin_k ||q_i - mu_k||^2, lowest k on ties, computed
 * as ||mu_k||^2 - 2 q_i . mu_k in fp32.
 *   Q in [S,L,d] dtype dt; mu in fp32 [S,Kc,d] (NULL: use the strided init
 *   rows Q[floor(k L / Kc)], Kc <= L); assign out int32 [S,L].
 */
ca_status_t ca_kmeans_assign(const void *Q, const float *mu, int S, int L,
                             int d, int Kc, ca_dtype_t dt, int32_t *assign,
                             hipStream_t stream);

/*
 * Assignment scores as the matrix-core assignment step evaluates them, for
 * measuring its distance error: scores[s, i, k] = mu_k . q_i - ||mu_k||^2 / 2
 * (fp32, unscaled units), so that ||q_i - mu_k||^2 = ||q_i||^2 - 2 scores[s, i,
 * k]; the step assigns token i to the k with the largest score (lowest k on
 * ties). Same passages as ca_kmeans_assign; the arithmetic is the one every
 * matrix-core clustering kernel uses (power-of-two scaling, fp16 h/m split,
 * three partial products, the -||mu||^2/2 parts in the same chain).
 *   Q in [S,L,d] dtype dt; mu in fp32 [S,Kc,d]; scores out fp32 [S,L,Kc].
 *   Kc <= 64 (CA_ERR_UNSUPPORTED otherwise).
 */
ca_status_t ca_kmeans_scores(const void *Q, const float *mu, int S, int L, int d, int Kc,
                             ca_dtype_t dt, float *scores, hipStream_t stream);

/*
 * One update step (same passages): mu[s,k] = sum_{assign = k} q_i /
 * max(1, n_k), an empty cluster gives the zero vector; counts[s,k] = n_k
 * (counts may be NULL). Deterministic: per-tile partial sums in token order,
 * then a fixed-order sum over tiles.
 *   Q in [S,L,d] dtype dt; assign in int32 [S,L] with values in [0,Kc)
 *   (values outside are clamped into it); mu out fp32 [S,Kc,d]; workspace of
 *   ca_centroid_update_workspace_size(S,L,d,Kc) bytes.
 */
ca_status_t ca_centroid_update(const void *Q, const int32_t *assign, int S,
                               int L, int d, int Kc, ca_dtype_t dt, float *mu,
                               int32_t *counts, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);
size_t ca_centroid_update_workspace_size(int S, int L, int d, int Kc);

/*
 * Centroid cross-attention (model card pipeline figure; ClusterFormer 3):
 * vcent[s,k] = sum_j softmax_j(mu_k . k_j / sqrt(d)) v_j over all L keys.
 *   mu in fp32 [S,Kc,d]; K, V in [S,L,d] dtype dt; vcent out fp32 [S,Kc,d];
 *   workspace of ca_centroid_xattn_workspace_size(S,L,d,Kc) bytes (0 for
 *   L <= 128; otherwise the partials of the 128-key ranges, combined in a
 *   fixed order).
 */
ca_status_t ca_centroid_xattn(const float *mu, const void *K, const void *V,
                              int S, int L, int d, int Kc, ca_dtype_t dt,
                              float *vcent, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);
size_t ca_centroid_xattn_workspace_size(int S, int L, int d, int Kc);

/*
 * Local sliding-window branch (model card pipeline figure; ClusterFormer 3):
 * oloc[s,i] = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j over
 * j in [max(0, i - r), min(L - 1, i + r)], r = floor(W/2).
 *   Q, K, V in [S,L,d] dtype dt; oloc out fp32 [S,L,d].
 */
ca_status_t ca_local_window_attn(const void *Q, const void *K, const void *V,
                                 int S, int L, int d, int W, ca_dtype_t dt,
                                 float *oloc, hipStream_t stream);

/*
 * Gather and convex fusion (model card Architecture Overview item 2):
 * out[s,i] = (1 - alpha) vcent[s, assign[s,i]] + alpha oloc[s,i].
 *   vcent fp32 [S,Kc,d]; assign int32 [S,L] in [0,Kc) (values outside are
 *   clamped into it); oloc fp32 [S,L,d];
 *   out [S,L,d] dtype dt.
 */
ca_status_t ca_gather_fuse(const float *vcent, const int32_t *assign,
                           const float *oloc, int S, int L, int d, int Kc,
                           float alpha, ca_dtype_t dt, void *out,
                           hipStream_t stream);

/* ---------------------------------------------------------------------
 * Full attention layer (model card Architecture Overview: multi-head
 * projections of X, cluster attention, output projection Y = O W_O;
 * ClusterFormer 3, first and last rows of the tensor trace), bf16 storage:
 *   Q = X Wq, K = X Wk, V = X Wv   X [B, L, Dm]; W [Dm, H*d] ([in, out]),
 *                                  no bias; head h is columns h*d .. h*d+d-1;
 *                                  each product accumulated in fp32 and
 *                                  rounded to bf16 (nearest even)
 *   O = cluster attention of (Q, K, V) exactly as cluster_attn_forward with
 *       dt = CA_BF16 (O rounded to bf16)
 *   Y = O_merged Wo                O_merged [B, L, H*d] (heads concatenated),
 *                                  Wo [H*d, Dm], Y [B, L, Dm] rounded to bf16
 * Arguments:
 *   X, Wq, Wk, Wv, Wo  in   device bf16 bits (uint16), 16-byte aligned.
 *   B, L, H >= 1; d == 64 and Dm == H * d (CA_ERR_UNSUPPORTED otherwise);
 *   nclust, iters, W, alpha as in cluster_attn_forward.
 *   Y           out  device bf16 [B, L, Dm].
 *   assign_out  out  device int32 [B, H, L] or NULL.
 *   qkv_out     out  device bf16 [3, B, H, L, d] receiving Q, K, V, or NULL.
 *   workspace        device, cluster_attn_layer_workspace_size(...) bytes,
 *                    256-byte aligned; it holds Q, K, V (when qkv_out is
 *                    NULL), O and the attention workspace.
 *   Outputs and workspace must not overlap each other or the inputs.
 *   Launches: one GEMM for Q, K and V together (weights read in their
 *   [in, out] layout), the cluster attention launches, one GEMM for Y.
 * --------------------------------------------------------------------- */
size_t cluster_attn_layer_workspace_size(int B, int L, int Dm, int H, int d,
                                         int nclust);

ca_status_t cluster_attn_layer_forward(const void *X, const void *Wq,
                                       const void *Wk, const void *Wv,
                                       const void *Wo, int B, int L, int Dm,
                                       int H, int d, int nclust, int iters,
                                       int W, float alpha, void *Y,
                                       int32_t *assign_out, void *qkv_out,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * The layer's bf16 GEMM on its own: C[M, N] = A[M, Kd] . Bt[N, Kd]^T, i.e.
 * C[m][n] = sum_k A[m][k] Bt[n][k] (Bt in the [out, in] layout of a linear
 * layer's weight), fp32 accumulation, one round-to-nearest-even to bf16.
 *   A, Bt in, C out: device bf16 bits, row-major, 16-byte aligned; C must
 *   not overlap A or Bt. M, N, Kd >= 1 (CA_ERR_INVALID_ARG otherwise); N and
 *   Kd multiples of 64 and N * Kd < 2^31 (CA_ERR_UNSUPPORTED otherwise);
 *   any M.
 */
ca_status_t ca_gemm_bf16(const void *A, const void *Bt, int M, int N, int Kd,
                         void *C, hipStream_t stream);

/*
 * The same GEMM with the weight in the [in, out] layout the layer's
 * projections take (Architecture Overview of the model card: Q = X W_Q, ...):
 * C[M, N] = A[M, Kd] . W[Kd, N], C[m][n] = sum_k A[m][k] W[k][n]. Arguments,
 * alignment, precision and errors as for ca_gemm_bf16, with W [Kd, N]
 * row-major in place of Bt.
 */
ca_status_t ca_gemm_bf16_kn(const void *A, const void *W, int M, int N, int Kd,
                            void *C, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CLUSTERATTN_H */
