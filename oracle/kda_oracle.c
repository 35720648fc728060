/*
 * kda_oracle.c -- plain fp64 CPU oracle for the KDA (per-channel gate)
 * variant of the ReplaySSM ring spec-verify.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
 * baseline of the benchmark, never by the library; it shares no code,
 * header or table with the HIP path.
 *
 * The KDA layer differs from the GDN layer in one place: its gate is a
 * vector over the key channels, so the state decays column by column
 * (PR #36821 summary: the KDA spec ring keeps g as [slots, HV, L, K] fp32,
 * "per-K KDA gate", beside raw k, raw v and a scalar beta per value head).
 * Definitions, for value head hv and key channel c:
 *   gate     g_c  = -exp(A_log[hv]) * softplus(a_c + dt_bias[hv][c]),
 *            beta = sigmoid(b)                  (per-channel form of the GDN
 *                                                gate: a reading, the pages
 *                                                print no KDA gate formula)
 *   step     S[:, c] <- e^{g_c} S[:, c];  u = S k_hat;  S <- S + beta (v - u) k_hat^T
 *   output   o_t = scale * S_t q_hat_t, for every window position
 * The ring, cursors, history replay, exact fold and ring write follow the
 * GDN oracle (gdn_oracle.c) with g widened to K values per record.
 *
 * All state is fp64; activations arrive widened exactly from their storage
 * dtype.  (row, value head) pairs are split across pthreads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int B, T, H, HV, K, V, L, max_spec, num_slots;
    double scale, softplus_threshold, eps;
} kda_shape;

/* Layouts (row-major):
 *   S      [num_slots][HV][V][K]
 *   rawk   [num_slots][H][L][K]     rawv [num_slots][HV][L][V]
 *   rg     [num_slots][HV][L][K]    rb   [num_slots][HV][L]
 *   wp, base, flush [num_slots]     slot [B]
 *   q, k   [B*T][H][K]   v [B*T][HV][V]   a [B*T][HV][K]   b [B*T][HV]
 *   A_log  [HV]          dt_bias [HV][K]
 *   o      [B*T][HV][V]
 */
typedef struct {
    kda_shape sh;
    double *S, *rawk, *rawv, *rg, *rb;
    const int32_t *wp, *base, *flush, *slot;
    const double *q, *k, *v, *a, *b;
    const double *A_log, *dt_bias;
    double *o;
    int fold_flagged, only_flagged;
} kda_args;

static double kda_softplus(double x, double threshold)
{
    return x > threshold ? x : log1p(exp(x));
}

/* g [K] and beta of one token and value head. */
void kda_gate(const double *a, double b, double A_log, const double *dt_bias, int K,
              double threshold, double *g, double *beta)
{
    for (int c = 0; c < K; c++)
        g[c] = -exp(A_log) * kda_softplus(a[c] + dt_bias[c], threshold);
    *beta = 1.0 / (1.0 + exp(-b));
}

static double kda_rnorm(const double *x, int n, double eps)
{
    double ss = 0.0;
    for (int i = 0; i < n; i++)
        ss += x[i] * x[i];
    return 1.0 / sqrt(ss + eps);
}

/* One step on a V x K state: column c decays by e^{g_c}, then the delta
 * rule with the normalised raw key. */
void kda_step(double *S, int V, int K, const double *k_raw, const double *v, const double *g,
              double beta, double eps)
{
    double rn = kda_rnorm(k_raw, K, eps);
    for (int r = 0; r < V; r++) {
        double *row = S + (size_t)r * K;
        double u = 0.0;
        for (int c = 0; c < K; c++)
            row[c] *= exp(g[c]);
        for (int c = 0; c < K; c++)
            u += row[c] * (k_raw[c] * rn);
        double d = beta * (v[r] - u);
        for (int c = 0; c < K; c++)
            row[c] += d * (k_raw[c] * rn);
    }
}

void kda_readout(const double *S, int V, int K, const double *q_raw, double scale, double eps,
                 double *o)
{
    double rn = kda_rnorm(q_raw, K, eps);
    for (int r = 0; r < V; r++) {
        double acc = 0.0;
        for (int c = 0; c < K; c++)
            acc += S[(size_t)r * K + c] * (q_raw[c] * rn);
        o[r] = scale * acc;
    }
}

static int kda_clamp_wp(int wp, const kda_shape *sh)
{
    int hi = sh->L - sh->T;
    return wp < 0 ? 0 : (wp > hi ? hi : wp);
}

static int kda_phys(int base, int logical, int L)
{
    return (base + logical) & (L - 1);
}

static int kda_valid_slot(int s, const kda_shape *sh)
{
    return s >= 0 && s < sh->num_slots;
}

/* Committed records 0..n-1 of slot s applied to the state of value head hv. */
static void kda_replay(const kda_args *A, double *Sw, int s, int hv, int n)
{
    const kda_shape *sh = &A->sh;
    int h = hv / (sh->HV / sh->H);
    for (int j = 0; j < n; j++) {
        int p = kda_phys(A->base[s], j, sh->L);
        size_t gi = ((size_t)s * sh->HV + hv) * sh->L + p;
        kda_step(Sw, sh->V, sh->K, A->rawk + (((size_t)s * sh->H + h) * sh->L + p) * sh->K,
                 A->rawv + gi * sh->V, A->rg + gi * sh->K, A->rb[gi], sh->eps);
    }
}

static void kda_verify_pair(const kda_args *A, int row, int hv, double *Sw, double *gw)
{
    const kda_shape *sh = &A->sh;
    int s = A->slot[row];
    if (!kda_valid_slot(s, sh))
        return;
    int h = hv / (sh->HV / sh->H);
    size_t VK = (size_t)sh->V * sh->K;
    double *S0 = A->S + ((size_t)s * sh->HV + hv) * VK;
    int wp = kda_clamp_wp(A->wp[s], sh);
    int flagged = A->flush[s] != 0;
    if (flagged && A->fold_flagged)
        kda_replay(A, S0, s, hv, wp);           /* exact fold into the checkpoint */
    int hist = flagged ? 0 : wp;
    memcpy(Sw, S0, VK * sizeof(double));
    kda_replay(A, Sw, s, hv, hist);             /* committed history, not stored */
    for (int t = 0; t < sh->T; t++) {
        size_t tok = (size_t)row * sh->T + t;
        double beta;
        kda_gate(A->a + (tok * sh->HV + hv) * sh->K, A->b[tok * sh->HV + hv], A->A_log[hv],
                 A->dt_bias + (size_t)hv * sh->K, sh->K, sh->softplus_threshold, gw, &beta);
        kda_step(Sw, sh->V, sh->K, A->k + (tok * sh->H + h) * sh->K,
                 A->v + (tok * sh->HV + hv) * sh->V, gw, beta, sh->eps);
        kda_readout(Sw, sh->V, sh->K, A->q + (tok * sh->H + h) * sh->K, sh->scale, sh->eps,
                    A->o + (tok * sh->HV + hv) * sh->V);
    }
}

static void kda_fold_pair(const kda_args *A, int row, int hv, double *Sw, double *gw)
{
    (void)Sw;
    (void)gw;
    const kda_shape *sh = &A->sh;
    int s = A->slot[row];
    if (!kda_valid_slot(s, sh))
        return;
    if (A->only_flagged && A->flush[s] == 0)
        return;
    double *S0 = A->S + ((size_t)s * sh->HV + hv) * (size_t)sh->V * sh->K;
    kda_replay(A, S0, s, hv, kda_clamp_wp(A->wp[s], sh));
}

typedef void (*kda_pair_fn)(const kda_args *, int, int, double *, double *);

typedef struct {
    const kda_args *A;
    kda_pair_fn fn;
    int tid, nthreads;
} kda_ctx;

static void *kda_worker(void *p)
{
    kda_ctx *w = (kda_ctx *)p;
    const kda_args *A = w->A;
    double *Sw = (double *)malloc((size_t)A->sh.V * A->sh.K * sizeof(double));
    double *gw = (double *)malloc((size_t)A->sh.K * sizeof(double));
    for (int i = w->tid; i < A->sh.B * A->sh.HV; i += w->nthreads)
        w->fn(A, i / A->sh.HV, i % A->sh.HV, Sw, gw);
    free(Sw);
    free(gw);
    return NULL;
}

static void kda_run(const kda_args *A, kda_pair_fn fn, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    kda_ctx *ctx = (kda_ctx *)malloc(sizeof(kda_ctx) * nthreads);
    for (int i = 0; i < nthreads; i++) {
        ctx[i].A = A;
        ctx[i].fn = fn;
        ctx[i].tid = i;
        ctx[i].nthreads = nthreads;
        pthread_create(&th[i], NULL, kda_worker, &ctx[i]);
    }
    for (int i = 0; i < nthreads; i++)
        pthread_join(th[i], NULL);
    free(th);
    free(ctx);
}

/* The window's raw records at logical positions wp + t: rawk once per
 * qk-head, rawv, the K-channel gate and beta once per value head. */
static void kda_write_window(const kda_args *A)
{
    const kda_shape *sh = &A->sh;
    for (int row = 0; row < sh->B; row++) {
        int s = A->slot[row];
        if (!kda_valid_slot(s, sh))
            continue;
        int wp = kda_clamp_wp(A->wp[s], sh);
        for (int t = 0; t < sh->T; t++) {
            int p = kda_phys(A->base[s], wp + t, sh->L);
            size_t tok = (size_t)row * sh->T + t;
            for (int h = 0; h < sh->H; h++)
                memcpy(A->rawk + (((size_t)s * sh->H + h) * sh->L + p) * sh->K,
                       A->k + (tok * sh->H + h) * sh->K, sh->K * sizeof(double));
            for (int hv = 0; hv < sh->HV; hv++) {
                size_t gi = ((size_t)s * sh->HV + hv) * sh->L + p;
                memcpy(A->rawv + gi * sh->V, A->v + (tok * sh->HV + hv) * sh->V,
                       sh->V * sizeof(double));
                kda_gate(A->a + (tok * sh->HV + hv) * sh->K, A->b[tok * sh->HV + hv],
                         A->A_log[hv], A->dt_bias + (size_t)hv * sh->K, sh->K,
                         sh->softplus_threshold, A->rg + gi * sh->K, &A->rb[gi]);
            }
        }
    }
}

void kda_verify(kda_args *A, int write_ring, int nthreads)
{
    kda_run(A, kda_verify_pair, nthreads);
    if (write_ring)
        kda_write_window(A);
}

void kda_write_ring(kda_args *A)
{
    kda_write_window(A);
}

void kda_fold(kda_args *A, int nthreads)
{
    kda_run(A, kda_fold_pair, nthreads);
}

size_t kda_args_size(void) { return sizeof(kda_args); }
