/*
 * TreeWY CPU oracle -- TEST INFRASTRUCTURE, not part of the product.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load this
 * library.  It shares no code, header or helper with the GPU path.
 *
 * What it computes is the plain definition of speculative verification on a gated
 * delta rule layer, from "TreeWY: Speculative Verification for Gated DeltaNet Hybrids"
 * (arXiv 2608.20961):
 *
 *   - Eq. (1), §1 "Background":  S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *     o_t = S_t q_t, with S in R^{dv x dk}.
 *   - §3 "Verifying a draft": in a draft tree, the state before node t is the state
 *     of t's parent; node t's output is the recurrence chained along its own
 *     root-to-node path (nodes are numbered so that parents come first).
 *   - §3 "Key rewrite": the pseudo-value of node t is b_t (v_t - a_t S_parent k_t);
 *     the oracle records it while replaying.
 *   - §3 "Reconstruct on commit": after node a is accepted, the next committed state
 *     is the state at a.  Here that state is obtained by replaying Eq. (1) along a's
 *     path; nothing is accepted (a = -1) leaves S0 untouched.
 *
 * Everything is computed in double precision from float inputs widened exactly.
 * No solve, no closed form and no reordering beyond the token-by-token replay.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_OK = 0, OR_EINVAL = 1, OR_ETREE = 3, OR_EACCEPT = 4 };

/* Tree bookkeeping for one draft tree (§3 "Verifying a draft"):
 * parent[t] must lie in [-1, t-1]; depth(t) = 1 + depth(parent(t)) with depth(S0) = 0;
 * anc[t] has bit i set for every ancestor i of t, t itself included (needs N <= 64). */
int oracle_index_tree(int N, const int32_t* parent, int32_t* depth, uint64_t* anc)
{
    if (N < 1 || N > 64 || !parent) return OR_EINVAL;
    for (int t = 0; t < N; ++t) {
        int p = parent[t];
        if (p < -1 || p >= t) return OR_ETREE;
        int d = (p < 0) ? 1 : depth[p] + 1;
        uint64_t m = (p < 0) ? 0 : anc[p];
        depth[t] = d;
        anc[t] = m | ((uint64_t)1 << t);
    }
    return OR_OK;
}

/* Root-to-t path of node t, written root first; returns its length. */
static int path_to(int t, const int32_t* parent, int* path)
{
    int n = 0;
    for (int j = t; j >= 0; j = parent[j]) ++n;
    int i = n;
    for (int j = t; j >= 0; j = parent[j]) path[--i] = j;
    return n;
}

/* One step of Eq. (1) applied in place to S (dv x dk, row-major).
 * u receives S_before k (length dv). */
static void gdn_step(int dk, int dv, double* S, double* u,
                     const double* k, const double* v, double a, double b)
{
    for (int r = 0; r < dv; ++r) {
        double s = 0.0;
        for (int c = 0; c < dk; ++c) s += S[r * dk + c] * k[c];
        u[r] = s;
    }
    /* S <- a (S - b (S k) k^T) + b v k^T */
    for (int r = 0; r < dv; ++r)
        for (int c = 0; c < dk; ++c)
            S[r * dk + c] = a * (S[r * dk + c] - b * u[r] * k[c]) + b * v[r] * k[c];
}

/*
 * One (sequence, head): per-node outputs O[t] = S_t q_t, pseudo-values U[t],
 * cumulative decays gamma[t] = product of a_j over j on t's path, and, when
 * S_new is given, the state after replaying the path of node `accepted`.
 *
 * Shapes (row-major): S0 dv x dk; q, k N x dk; v N x dv; alpha, beta N;
 * O, U N x dv; gamma N; S_new dv x dk.
 */
int oracle_head(int N, int dk, int dv, const double* S0, const double* q,
                const double* k, const double* v, const double* alpha,
                const double* beta, const int32_t* parent, int accepted,
                double* O, double* U, double* gamma, double* S_new)
{
    if (N < 1 || N > 64 || dk < 1 || dv < 1) return OR_EINVAL;
    int32_t depth[64];
    uint64_t anc[64];
    int rc = oracle_index_tree(N, parent, depth, anc);
    if (rc) return rc;
    if (S_new && (accepted < -1 || accepted >= N)) return OR_EACCEPT;

    double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    int path[64];
    if (!S || !u) { free(S); free(u); return OR_EINVAL; }

    for (int t = 0; t < N; ++t) {
        memcpy(S, S0, sizeof(double) * (size_t)dv * dk);
        int n = path_to(t, parent, path);
        double g = 1.0;
        for (int s = 0; s < n; ++s) {
            int j = path[s];
            gdn_step(dk, dv, S, u, k + (size_t)j * dk, v + (size_t)j * dv, alpha[j], beta[j]);
            if (j == t)  /* S_parent k_t was in u; pseudo-value of §3 "Key rewrite" */
                for (int r = 0; r < dv; ++r)
                    U[(size_t)t * dv + r] = beta[t] * (v[(size_t)t * dv + r] - alpha[t] * u[r]);
            g *= alpha[j];
        }
        gamma[t] = g;
        for (int r = 0; r < dv; ++r) {
            double s = 0.0;
            for (int c = 0; c < dk; ++c) s += S[r * dk + c] * q[(size_t)t * dk + c];
            O[(size_t)t * dv + r] = s;
        }
    }

    if (S_new) {
        memcpy(S_new, S0, sizeof(double) * (size_t)dv * dk);
        if (accepted >= 0) {
            int n = path_to(accepted, parent, path);
            for (int s = 0; s < n; ++s) {
                int j = path[s];
                gdn_step(dk, dv, S_new, u, k + (size_t)j * dk, v + (size_t)j * dv, alpha[j], beta[j]);
            }
        }
    }
    free(S);
    free(u);
    return OR_OK;
}

/*
 * Batched driver over the device layouts: S0 [B,H,dv,dk]; q, k [B,N,H,dk];
 * v [B,N,H,dv]; alpha, beta [B,N,H]; parent [B,N]; accepted [B] (nullable).
 * sel lists nsel (b, h) pairs to compute (NULL: all B*H heads in (b, h) order).
 * Outputs are per selected head: O, U [nsel,N,dv]; gamma [nsel,N];
 * S_new [nsel,dv,dk] (nullable).  Returns the first error met, else OR_OK.
 * Heads are independent and run on `nthreads` OpenMP threads.
 */
int oracle_batch(int B, int H, int N, int dk, int dv, const float* S0,
                 const float* q, const float* k, const float* v,
                 const float* alpha, const float* beta, const int32_t* parent,
                 const int32_t* accepted, int nsel, const int32_t* sel,
                 double* O, double* U, double* gamma, double* S_new, int nthreads)
{
    if (B < 1 || H < 1 || N < 1 || N > 64 || dk < 1 || dv < 1) return OR_EINVAL;
    int total = sel ? nsel : B * H;
    int err = OR_OK;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int s = 0; s < total; ++s) {
        int b = sel ? sel[2 * s] : s / H;
        int h = sel ? sel[2 * s + 1] : s % H;
        if (b < 0 || b >= B || h < 0 || h >= H) {
#pragma omp critical
            { if (!err) err = OR_EINVAL; }
            continue;
        }
        size_t sd = (size_t)dv * dk;
        double* S0d = (double*)malloc(sizeof(double) * sd);
        double* qd = (double*)malloc(sizeof(double) * (size_t)N * dk);
        double* kd = (double*)malloc(sizeof(double) * (size_t)N * dk);
        double* vd = (double*)malloc(sizeof(double) * (size_t)N * dv);
        double ad[64], bd[64];
        const float* s0 = S0 + ((size_t)b * H + h) * sd;
        for (size_t i = 0; i < sd; ++i) S0d[i] = s0[i];
        for (int t = 0; t < N; ++t) {
            size_t row = ((size_t)b * N + t) * H + h;
            for (int c = 0; c < dk; ++c) {
                qd[(size_t)t * dk + c] = q[row * dk + c];
                kd[(size_t)t * dk + c] = k[row * dk + c];
            }
            for (int r = 0; r < dv; ++r) vd[(size_t)t * dv + r] = v[row * dv + r];
            ad[t] = alpha[row];
            bd[t] = beta[row];
        }
        int a = accepted ? accepted[b] : -1;
        int rc = oracle_head(N, dk, dv, S0d, qd, kd, vd, ad, bd, parent + (size_t)b * N, a,
                             O + (size_t)s * N * dv, U + (size_t)s * N * dv,
                             gamma + (size_t)s * N, S_new ? S_new + (size_t)s * sd : NULL);
        if (rc) {
#pragma omp critical
            { if (!err) err = rc; }
        }
        free(S0d); free(qd); free(kd); free(vd);
    }
    return err;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
