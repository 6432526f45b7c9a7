/*
 * oracle/recurrence.c -- token-by-token fp64 reference of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP path is
 * checked against.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load it.  It shares no code, header or constant with
 * the GPU library, and the GPU library never calls it.
 *
 * Sources (page title, then section):
 *   [KDA]  "TileLang 实战：KDA 从零到一–Kimi Delta Attention"
 *          opening equation and section 3.1 (reference A): the per-token
 *          update S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *          o_t = S_t q_t, with S in R^{dv x dk}; g = log a (section 0).
 *          Diag(a_t) sits between S_{t-1} and the Householder factor.
 *   [SD]   "TileLang 实战：KDA 从零到一--标量衰减"
 *          section 1.1: S_t = alpha S_{t-1} + v_t k_t^T, o_t = S_t q_t
 *          (scalar decay, no delta term); section 1.0 lets alpha vary per token.
 *   [GDN]  "Gated DeltaNet", section "DeltaNet 与
 *          Gated Delta Rule": decay the entry state first, then the rank-one
 *          residual write along k.  The scalar-gate case of [KDA]'s update.
 *
 * Orientation: the state is kept exactly as the pages write it, S in
 * R^{dv x dk} (value index = row, key index = column).  h0 and hT are in the
 * same orientation here: [B, H, Dv, Dk].  (The GPU library stores the
 * transpose; tests convert explicitly.)
 *
 * Everything is double precision.  Inputs are given as double arrays; the
 * callers upcast the exact bf16 / fp32 values the GPU receives.
 *
 * Layouts: q, k [B,T,H,Dk]; v, o [B,T,H,Dv]; g [B,T,H,Dk] (kind 0) or
 * [B,T,H] (kinds 1, 2); beta [B,T,H] (ignored for kind 2).
 *
 * kind 0 = KDA (per-channel gate), 1 = GDN (scalar gate), 2 = scalar-decay
 * linear attention without the delta term.
 *
 * The (b, h) chains are independent, so they are spread over threads; inside
 * a chain the tokens are processed strictly in order, one full update each.
 */
#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int kind, B, T, H, Dk, Dv;
    const double *q, *k, *v, *g, *beta, *h0;
    double *o, *hT;
    atomic_int next;
    atomic_int failed;
} oracle_job;

static void run_chain(oracle_job* J, int b, int h)
{
    const int Dk = J->Dk, Dv = J->Dv, T = J->T, H = J->H;
    double* S = (double*)malloc(sizeof(double) * (size_t)Dv * Dk);
    double* a = (double*)malloc(sizeof(double) * (size_t)Dk);
    double* Sk = (double*)malloc(sizeof(double) * (size_t)Dv);
    if (!S || !a || !Sk) {
        atomic_store(&J->failed, 1);
        free(S); free(a); free(Sk);
        return;
    }
    const size_t sh = ((size_t)b * H + h) * (size_t)Dv * Dk;
    if (J->h0)
        memcpy(S, J->h0 + sh, sizeof(double) * (size_t)Dv * Dk);
    else
        memset(S, 0, sizeof(double) * (size_t)Dv * Dk);

    for (int t = 0; t < T; ++t) {
        const size_t row = ((size_t)b * T + t) * H + h;   /* token-head index */
        const double* qt = J->q + row * Dk;
        const double* kt = J->k + row * Dk;
        const double* vt = J->v + row * Dv;
        double* ot = J->o + row * Dv;

        /* gate a_t = exp(g_t): per channel for KDA, one scalar otherwise */
        if (J->kind == 0) {
            for (int j = 0; j < Dk; ++j) a[j] = exp(J->g[row * Dk + j]);
        } else {
            const double s = exp(J->g[row]);
            for (int j = 0; j < Dk; ++j) a[j] = s;
        }

        if (J->kind == 2) {
            /* [SD] 1.1: S_t = alpha_t S_{t-1} + v_t k_t^T */
            for (int i = 0; i < Dv; ++i)
                for (int j = 0; j < Dk; ++j)
                    S[(size_t)i * Dk + j] = a[j] * S[(size_t)i * Dk + j] + vt[i] * kt[j];
        } else {
            const double bt = J->beta[row];
            /* X = S_{t-1} Diag(a_t): column j scaled by a_j */
            for (int i = 0; i < Dv; ++i)
                for (int j = 0; j < Dk; ++j)
                    S[(size_t)i * Dk + j] *= a[j];
            /* X (I - beta k k^T) = X - beta (X k) k^T */
            for (int i = 0; i < Dv; ++i) {
                double acc = 0.0;
                for (int j = 0; j < Dk; ++j) acc += S[(size_t)i * Dk + j] * kt[j];
                Sk[i] = acc;
            }
            for (int i = 0; i < Dv; ++i)
                for (int j = 0; j < Dk; ++j)
                    S[(size_t)i * Dk + j] -= bt * Sk[i] * kt[j];
            /* + beta v k^T */
            for (int i = 0; i < Dv; ++i)
                for (int j = 0; j < Dk; ++j)
                    S[(size_t)i * Dk + j] += bt * vt[i] * kt[j];
        }
        /* o_t = S_t q_t */
        for (int i = 0; i < Dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < Dk; ++j) acc += S[(size_t)i * Dk + j] * qt[j];
            ot[i] = acc;
        }
    }
    if (J->hT) memcpy(J->hT + sh, S, sizeof(double) * (size_t)Dv * Dk);
    free(S); free(a); free(Sk);
}

static void* worker(void* arg)
{
    oracle_job* J = (oracle_job*)arg;
    const int n = J->B * J->H;
    for (;;) {
        const int i = atomic_fetch_add(&J->next, 1);
        if (i >= n) break;
        run_chain(J, i / J->H, i % J->H);
    }
    return NULL;
}

/*
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 * nthreads <= 0 means one thread per online CPU (capped at the chain count).
 */
int oracle_forward(int kind, const double* q, const double* k, const double* v,
                   const double* g, const double* beta, const double* h0,
                   double* o, double* hT, int B, int T, int H, int Dk, int Dv,
                   int nthreads)
{
    if (kind < 0 || kind > 2 || B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (!o || (T > 0 && (!q || !k || !v || !g))) return -1;
    if (kind != 2 && T > 0 && !beta) return -1;
    oracle_job J;
    J.kind = kind; J.B = B; J.T = T; J.H = H; J.Dk = Dk; J.Dv = Dv;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0;
    J.o = o; J.hT = hT;
    atomic_init(&J.next, 0);
    atomic_init(&J.failed, 0);
    const int chains = B * H;
    if (chains == 0) return 0;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > chains) nthreads = chains;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -2;
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
        ++started;
    }
    worker(&J);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    free(th);
    return atomic_load(&J.failed) ? -2 : 0;
}

/* Threads the oracle would use for nthreads <= 0 (reported by the benchmark). */
int oracle_default_threads(void) { return (int)sysconf(_SC_NPROCESSORS_ONLN); }
