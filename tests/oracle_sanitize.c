/*
 * Driver that runs every entry point of oracle/oracle.c on small and edge
 * shapes, built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitize.py (host code only, no GPU). It checks memory
 * safety and undefined behaviour of the oracle, not its values: the values are
 * pinned by tests/test_oracle.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ora_num_clusters(int nclust, int L);
void ora_init_centroids(const double *Q, long S, int L, int d, int K, double *mu);
void ora_init_centroids_step(const double *Q, long S, int L, int d, int K, double *mu);
void ora_assign(const double *Q, const double *mu, long S, int L, int d, int K, int32_t *c,
                double *dbest, double *gap, double *qn2);
void ora_update(const double *Q, const int32_t *c, long S, int L, int d, int K,
                const double *prev, double *mu, int32_t *counts);
void ora_objective(const double *Q, const double *mu, const int32_t *c, long S, int L, int d,
                   int K, double *J);
void ora_centroid_xattn(const double *mu, const double *Kt, const double *V, long S, int L,
                        int d, int K, const int32_t *valid, double *vcent, double *psum);
void ora_local_attn(const double *Q, const double *Kt, const double *V, long S, int L, int d,
                    int W, const int32_t *valid, double *oloc, double *psum);
void ora_fuse(const double *vcent, const int32_t *c, const double *oloc, long S, int L, int d,
              int K, double alpha, const int32_t *valid, const double *G, double *out);
void ora_soft_gather(const double *Q, const double *mu, const double *vcent, long S, int L,
                     int d, int K, double *G);
int ora_forward(const double *Q, const double *Kt, const double *V, int B, int H, int L, int d,
                int nclust, int iters, int W, double alpha, const int32_t *valid, int flags,
                double *out, int32_t *assign, double *mu_hist, int32_t *c_hist,
                double *gap_hist, double *J, double *Jp, double *qn2, double *vcent_out,
                double *oloc_out);
void ora_forward_from_assign(const double *Q, const double *Kt, const double *V, long S, int L,
                             int d, int K, const int32_t *c, int W, double alpha,
                             const int32_t *valid, int flags, const double *mu_in, double *out,
                             double *mu_out, double *vcent_out, double *oloc_out);
void ora_backward(const double *Q, const double *Kt, const double *V, const double *dO, long S,
                  int L, int d, int K, const int32_t *c, int W, double alpha,
                  const int32_t *valid, double *dQ, double *dK, double *dV, double *dalpha);
void ora_exact_attention(const double *Q, const double *Kt, const double *V, long S, int L,
                         int Nk, int d, int causal, const int32_t *qvalid, const int32_t *kvalid,
                         double *out);
void ora_matmul(const double *A, const double *Bm, long M, long P, long N, double *C);
double ora_round_bf16(double x);
void ora_round_bf16_array(double *x, long n);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

/* xorshift64* uniform in [-1, 1) (inputs only; no method arithmetic) */
static double urand(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    const uint64_t x = rng_state * 0x2545f4914f6cdd1dull;
    return (double)(x >> 11) / (double)(1ull << 52) - 1.0;
}

/* exact-size heap arrays so that any overrun is reported */
static double *darr(long n) {
    double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) p[i] = urand();
    return p;
}

static int32_t *iarr(long n) {
    return (int32_t *)calloc((size_t)(n > 0 ? n : 1), sizeof(int32_t));
}

static int32_t *mask(long S, int L, int keep_first) {
    int32_t *v = iarr(S * L);
    for (long s = 0; s < S; ++s)
        for (int i = 0; i < L; ++i) v[s * L + i] = (i < keep_first || urand() > 0.3) ? 1 : 0;
    return v;
}

static double checksum(const double *p, long n) {
    double t = 0.0;
    for (long i = 0; i < n; ++i) t += fabs(p[i]);
    return t;
}

static int run_case(int B, int H, int L, int d, int nclust, int iters, int W, double alpha,
                    int flags, int masked) {
    const long S = (long)B * H;
    const int K = ora_num_clusters(nclust, L);
    double *Q = darr(S * L * d), *Kt = darr(S * L * d), *V = darr(S * L * d);
    double *dO = darr(S * L * d);
    int32_t *valid = masked ? mask(S, L, 1) : NULL;
    double *out = darr(S * L * d), *mu_hist = darr((iters + 1) * S * K * d);
    int32_t *assign = iarr(S * L), *c_hist = iarr(iters * S * L);
    double *gap = darr(iters * S * L), *J = darr(iters * S), *Jp = darr(iters * S);
    double *qn2 = darr(S * L), *vc = darr(S * K * d), *ol = darr(S * L * d);
    const int rk = ora_forward(Q, Kt, V, B, H, L, d, nclust, iters, W, alpha, valid, flags, out,
                               assign, mu_hist, c_hist, gap, J, Jp, qn2, vc, ol);
    if (rk != K) {
        fprintf(stderr, "ora_forward returned %d, expected %d\n", rk, K);
        return 1;
    }
    for (long i = 0; i < S * L; ++i)
        if (assign[i] < 0 || assign[i] >= K) {
            fprintf(stderr, "assignment out of range\n");
            return 1;
        }
    /* the untraced call and the steps one by one */
    double *out2 = darr(S * L * d);
    ora_forward(Q, Kt, V, B, H, L, d, nclust, iters, W, alpha, valid, flags, out2, assign, NULL,
                NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    double *mu = darr(S * K * d), *mu2 = darr(S * K * d), *db = darr(S * L);
    int32_t *counts = iarr(S * K);
    ora_init_centroids(Q, S, L, d, K, mu);
    ora_init_centroids_step(Q, S, L, d, K, mu2);
    ora_assign(Q, mu, S, L, d, K, assign, db, gap, qn2);
    ora_update(Q, assign, S, L, d, K, NULL, mu2, counts);
    ora_update(Q, assign, S, L, d, K, mu, mu2, counts);
    ora_objective(Q, mu2, assign, S, L, d, K, J);
    double *psum = darr(S * L), *G = darr(S * L * d);
    ora_centroid_xattn(mu2, Kt, V, S, L, d, K, valid, vc, psum);
    ora_local_attn(Q, Kt, V, S, L, d, W, valid, ol, psum);
    ora_soft_gather(Q, mu2, vc, S, L, d, K, G);
    ora_fuse(vc, assign, ol, S, L, d, K, alpha, valid, NULL, out);
    ora_fuse(vc, assign, ol, S, L, d, K, alpha, valid, G, out);
    ora_forward_from_assign(Q, Kt, V, S, L, d, K, assign, W, alpha, valid, flags, NULL, out, mu,
                            vc, ol);
    ora_forward_from_assign(Q, Kt, V, S, L, d, K, assign, W, alpha, valid, flags, mu2, out, NULL,
                            NULL, NULL);
    double *dQ = darr(S * L * d), *dK = darr(S * L * d), *dV = darr(S * L * d), da = 0.0;
    ora_backward(Q, Kt, V, dO, S, L, d, K, assign, W, alpha, valid, dQ, dK, dV, &da);
    ora_backward(Q, Kt, V, dO, S, L, d, K, assign, W, alpha, NULL, dQ, dK, dV, &da);
    ora_exact_attention(Q, Kt, V, S, L, L, d, 1, valid, valid, out2);
    ora_exact_attention(Q, Kt, V, S, L, L, d, 0, NULL, valid, out2);
    if (L > 1) ora_exact_attention(Q, Kt, V, S, L - 1, L, d, 0, NULL, NULL, out2);
    const double cs = checksum(out, S * L * d) + checksum(dQ, S * L * d) + fabs(da);
    free(Q); free(Kt); free(V); free(dO); free(valid); free(out); free(mu_hist); free(assign);
    free(c_hist); free(gap); free(J); free(Jp); free(qn2); free(vc); free(ol); free(out2);
    free(mu); free(mu2); free(db); free(counts); free(psum); free(G); free(dQ); free(dK);
    free(dV);
    if (!isfinite(cs)) {
        fprintf(stderr, "non-finite result B=%d H=%d L=%d\n", B, H, L);
        return 1;
    }
    return 0;
}

int main(void) {
    /* B, H, L, d, nclust, iters, W, alpha, flags, masked */
    static const struct {
        int B, H, L, d, nclust, iters, W;
        double alpha;
        int flags, masked;
    } cases[] = {
        {1, 2, 128, 64, 16, 3, 32, 0.5, 0, 0},   /* the tiny workload's shape */
        {1, 1, 1, 64, 16, 2, 32, 0.5, 0, 0},     /* one token, K > L */
        {2, 3, 37, 16, 5, 2, 33, 0.3, 0, 1},     /* ragged, masked */
        {1, 2, 10, 8, 4, 3, 0, 0.0, 1, 0},       /* W = 0, K does not divide L, step init */
        {1, 2, 40, 8, 40, 2, 200, 1.0, 2, 1},    /* K = L, window past both ends, kept */
        {1, 1, 64, 16, 1, 4, 7, 0.5, 4, 0},      /* one cluster, odd W, soft gather */
        {2, 1, 50, 8, 6, 3, 60, 0.5, 8, 1},      /* band W >= L: no local branch */
        {1, 2, 33, 8, 3, 2, 5, 0.25, 31, 1},     /* every listing flag */
    };
    int bad = 0;
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i)
        bad |= run_case(cases[i].B, cases[i].H, cases[i].L, cases[i].d, cases[i].nclust,
                        cases[i].iters, cases[i].W, cases[i].alpha, cases[i].flags,
                        cases[i].masked);
    double A[6] = {1, 2, 3, 4, 5, 6}, Bm[6] = {1, 0, 0, 1, 1, 1}, C[4];
    ora_matmul(A, Bm, 2, 3, 2, C);
    double r[4] = {1.0 + 1.0 / 256, -3.5e-40, 65504.0, 0.0};
    ora_round_bf16_array(r, 4);
    bad |= ora_round_bf16(1.0) != 1.0;
    if (bad) return 1;
    printf("oracle sanitizer run ok\n");
    return 0;
}
