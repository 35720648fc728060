/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the GDN ReplaySSM ring spec-verify.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or table with the HIP path.
 *
 * What it computes is the plain definition, not the closed form:
 *
 *   gating   g = -exp(A_log) * softplus(a + dt_bias),  beta = sigmoid(b)
 *            (PR #33102 report, test anchor 3: the fused gating reference and
 *             the fp32 sigmoid; replayssm(B)SpecDecode App. A.1 parameter table)
 *   l2 norm  x_hat = x / sqrt(sum x^2 + eps), applied to q and k inside the
 *            kernel (App. A.1 constexpr USE_QK_L2NORM_IN_KERNEL)
 *   step     S <- e^g S ;  u = S k_hat ;  S <- S + beta (v - u) k_hat^T
 *            (the gated delta rule; replayssm(B)SpecDecode §12.1 and §12.6:
 *             the corrected delta d = beta (v - e^g S k) is the rank-1 factor)
 *   output   o_t = scale * S_t q_hat_t for every window position, including
 *            the ones later rejected (replayssm(B)SpecDecode §5.1)
 *
 * The committed state of a slot is the checkpoint folded with the committed
 * records 0..write_pos-1 of its ring, record j living at physical position
 * (cache_base + j) & (L-1) (replayssm(B)SpecDecode §10.1-10.2).  A verify
 * replays those records from the frozen checkpoint, then the window tokens,
 * and never writes the checkpoint (§4.1).  A slot flagged is_flush is first
 * folded into its checkpoint exactly, record by record, and then verified with
 * an empty history (§8.1, §9.1; PR #28695 summary: the closed-loop exact fold).
 * The window's raw records (k, v bits, g, beta) are written to the ring at
 * logical positions write_pos + t (§10.1, phys_spec); this never changes the
 * outputs (PR #33102 report, anchor 1).
 *
 * Conventions shared with the library's documented behaviour: rows whose slot
 * is outside [0, num_slots) are padding and are skipped; write_pos is clamped
 * to [0, L-T] before use (a no-op under the ring invariant of §8.2).
 *
 * All state is fp64.  Activations arrive already widened exactly from their
 * storage dtype.  Work over (row, value head) pairs is split across pthreads;
 * pairs are independent, so threading does not change any arithmetic.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int B, T, H, HV, K, V, L, max_spec, num_slots;
    double scale, softplus_threshold, eps;
} orc_shape;

/* Arrays of one layer.  Layouts (row-major):
 *   S      [num_slots][HV][V][K]          checkpoint, updated only by folds
 *   rawk   [num_slots][H][L][K]           ring: raw keys
 *   rawv   [num_slots][HV][L][V]          ring: raw values
 *   rg, rb [num_slots][HV][L]             ring: gate g and beta
 *   wp, base, flush [num_slots]           cursors (int32)
 *   slot   [B]                            slot of each row
 *   q, k   [B*T][H][K]; v [B*T][HV][V]; a, b [B*T][HV]   window, token = row*T+t
 *   o      [B*T][HV][V]
 *   snap   [B][T][HV][V][K]
 *   dwin   [B*T][HV][V]                   window corrected deltas (optional)
 *   rd     [num_slots][HV][L][V]          ring: corrected deltas (optional)
 */
typedef struct {
    orc_shape sh;
    double *S;
    double *rawk, *rawv, *rg, *rb;
    const int32_t *wp, *base, *flush, *slot;
    const double *q, *k, *v, *a, *b;
    const double *A_log, *dt_bias;
    double *o, *snap;
    int fold_flagged;     /* verify: fold flagged rows first            */
    int only_flagged;     /* fold: skip rows whose slot is not flagged  */
    const int32_t *pair_row, *pair_hv;   /* optional (row, hv) subset   */
    int n_pairs;
    double *dwin;         /* verify: corrected delta of each window step */
    double *rd;           /* ring write: corrected deltas (needs dwin)    */
} orc_args;

/* ---------------------------------------------------------------- helpers */

static double softplus(double x, double threshold)
{
    return x > threshold ? x : log1p(exp(x));
}

void orc_gate(double a, double b, double A_log, double dt_bias, double threshold,
              double *g, double *beta)
{
    *g = -exp(A_log) * softplus(a + dt_bias, threshold);
    *beta = 1.0 / (1.0 + exp(-b));
}

double orc_rnorm(const double *x, int n, double eps)
{
    double ss = 0.0;
    for (int i = 0; i < n; i++)
        ss += x[i] * x[i];
    return 1.0 / sqrt(ss + eps);
}

/* One gated delta-rule step on a V x K state, with the raw key normalised.
 * d_out (optional, length V) receives the corrected delta of each state row,
 * d = beta (v - e^g S k_hat): the rank-1 factor the step adds along k_hat
 * (replayssm(B)SpecDecode §1.1 table and §12.6, the d ring of the first
 * generation). */
void orc_step_d(double *S, int V, int K, const double *k_raw, const double *v,
                double g, double beta, double eps, double *d_out)
{
    double rn = orc_rnorm(k_raw, K, eps);
    double decay = exp(g);
    for (int r = 0; r < V; r++) {
        double *row = S + (size_t)r * K;
        double u = 0.0;
        for (int c = 0; c < K; c++)
            row[c] *= decay;
        for (int c = 0; c < K; c++)
            u += row[c] * (k_raw[c] * rn);
        double d = beta * (v[r] - u);
        if (d_out)
            d_out[r] = d;
        for (int c = 0; c < K; c++)
            row[c] += d * (k_raw[c] * rn);
    }
}

void orc_step(double *S, int V, int K, const double *k_raw, const double *v,
              double g, double beta, double eps)
{
    orc_step_d(S, V, K, k_raw, v, g, beta, eps, NULL);
}

/* o[r] = scale * sum_c S[r][c] * q_hat[c] */
void orc_readout(const double *S, int V, int K, const double *q_raw, double scale,
                 double eps, double *o)
{
    double rn = orc_rnorm(q_raw, K, eps);
    for (int r = 0; r < V; r++) {
        double acc = 0.0;
        for (int c = 0; c < K; c++)
            acc += S[(size_t)r * K + c] * (q_raw[c] * rn);
        o[r] = scale * acc;
    }
}

static int clamp_wp(int wp, const orc_shape *sh)
{
    int hi = sh->L - sh->T;
    return wp < 0 ? 0 : (wp > hi ? hi : wp);
}

static int phys_pos(int base, int logical, int L)
{
    return (base + logical) & (L - 1);
}

static int valid_slot(int s, const orc_shape *sh)
{
    return s >= 0 && s < sh->num_slots;
}

/* Apply committed records 0..n-1 of slot s (value head hv) to state Sw. */
static void replay_records(const orc_args *A, double *Sw, int s, int hv, int n)
{
    const orc_shape *sh = &A->sh;
    int h = hv / (sh->HV / sh->H);
    for (int j = 0; j < n; j++) {
        int p = phys_pos(A->base[s], j, sh->L);
        const double *kr = A->rawk + (((size_t)s * sh->H + h) * sh->L + p) * sh->K;
        const double *vr = A->rawv + (((size_t)s * sh->HV + hv) * sh->L + p) * sh->V;
        size_t gi = ((size_t)s * sh->HV + hv) * sh->L + p;
        orc_step(Sw, sh->V, sh->K, kr, vr, A->rg[gi], A->rb[gi], sh->eps);
    }
}

/* -------------------------------------------------------------- per pair */

static void verify_pair(const orc_args *A, int row, int hv, double *Sw)
{
    const orc_shape *sh = &A->sh;
    int s = A->slot[row];
    if (!valid_slot(s, sh))
        return;
    int h = hv / (sh->HV / sh->H);
    size_t VK = (size_t)sh->V * sh->K;
    double *S0 = A->S + ((size_t)s * sh->HV + hv) * VK;
    int wp = clamp_wp(A->wp[s], sh);
    int flagged = A->flush[s] != 0;

    if (flagged && A->fold_flagged)
        replay_records(A, S0, s, hv, wp);     /* exact fold into the checkpoint */

    int hist = flagged ? 0 : wp;
    memcpy(Sw, S0, VK * sizeof(double));
    replay_records(A, Sw, s, hv, hist);      /* committed history, not stored */

    for (int t = 0; t < sh->T; t++) {
        size_t tok = (size_t)row * sh->T + t;
        double g, beta;
        orc_gate(A->a[tok * sh->HV + hv], A->b[tok * sh->HV + hv], A->A_log[hv],
                 A->dt_bias[hv], sh->softplus_threshold, &g, &beta);
        const double *kt = A->k + (tok * sh->H + h) * sh->K;
        const double *vt = A->v + (tok * sh->HV + hv) * sh->V;
        const double *qt = A->q + (tok * sh->H + h) * sh->K;
        orc_step_d(Sw, sh->V, sh->K, kt, vt, g, beta, sh->eps,
                   A->dwin ? A->dwin + (tok * sh->HV + hv) * sh->V : NULL);
        orc_readout(Sw, sh->V, sh->K, qt, sh->scale, sh->eps,
                    A->o + (tok * sh->HV + hv) * sh->V);
    }
}

static void fold_pair(const orc_args *A, int row, int hv, double *Sw)
{
    (void)Sw;
    const orc_shape *sh = &A->sh;
    int s = A->slot[row];
    if (!valid_slot(s, sh))
        return;
    if (A->only_flagged && A->flush[s] == 0)
        return;
    double *S0 = A->S + ((size_t)s * sh->HV + hv) * (size_t)sh->V * sh->K;
    replay_records(A, S0, s, hv, clamp_wp(A->wp[s], sh));
}

static void snapshot_pair(const orc_args *A, int row, int hv, double *Sw)
{
    const orc_shape *sh = &A->sh;
    int s = A->slot[row];
    if (!valid_slot(s, sh))
        return;
    int h = hv / (sh->HV / sh->H);
    size_t VK = (size_t)sh->V * sh->K;
    memcpy(Sw, A->S + ((size_t)s * sh->HV + hv) * VK, VK * sizeof(double));
    for (int t = 0; t < sh->T; t++) {
        size_t tok = (size_t)row * sh->T + t;
        double g, beta;
        orc_gate(A->a[tok * sh->HV + hv], A->b[tok * sh->HV + hv], A->A_log[hv],
                 A->dt_bias[hv], sh->softplus_threshold, &g, &beta);
        orc_step(Sw, sh->V, sh->K, A->k + (tok * sh->H + h) * sh->K,
                 A->v + (tok * sh->HV + hv) * sh->V, g, beta, sh->eps);
        memcpy(A->snap + (((size_t)row * sh->T + t) * sh->HV + hv) * VK, Sw,
               VK * sizeof(double));
        orc_readout(Sw, sh->V, sh->K, A->q + (tok * sh->H + h) * sh->K, sh->scale,
                    sh->eps, A->o + (tok * sh->HV + hv) * sh->V);
    }
}

/* Deltas of the committed history, recorded in one pass: the state is
 * stepped from the checkpoint through records 0..write_pos-1 and each step's
 * corrected delta goes to the d ring at the record's physical position.  A
 * one-token d-cache verify of record j replays the same j records from the
 * same checkpoint before forming that delta, so a ring filled by such
 * verifies holds these values. */
static void fill_dring_pair(const orc_args *A, int row, int hv, double *Sw)
{
    const orc_shape *sh = &A->sh;
    int s = A->slot[row];
    if (!valid_slot(s, sh))
        return;
    int h = hv / (sh->HV / sh->H);
    size_t VK = (size_t)sh->V * sh->K;
    memcpy(Sw, A->S + ((size_t)s * sh->HV + hv) * VK, VK * sizeof(double));
    int n = clamp_wp(A->wp[s], sh);
    for (int j = 0; j < n; j++) {
        int p = phys_pos(A->base[s], j, sh->L);
        const double *kr = A->rawk + (((size_t)s * sh->H + h) * sh->L + p) * sh->K;
        const double *vr = A->rawv + (((size_t)s * sh->HV + hv) * sh->L + p) * sh->V;
        size_t gi = ((size_t)s * sh->HV + hv) * sh->L + p;
        orc_step_d(Sw, sh->V, sh->K, kr, vr, A->rg[gi], A->rb[gi], sh->eps,
                   A->rd + gi * sh->V);
    }
}

/* --------------------------------------------------------------- threads */

typedef void (*pair_fn)(const orc_args *, int, int, double *);

typedef struct {
    const orc_args *A;
    pair_fn fn;
    int tid, nthreads;
} worker_ctx;

static void *worker(void *p)
{
    worker_ctx *w = (worker_ctx *)p;
    const orc_args *A = w->A;
    int total = A->n_pairs > 0 ? A->n_pairs : A->sh.B * A->sh.HV;
    double *Sw = (double *)malloc((size_t)A->sh.V * A->sh.K * sizeof(double));
    for (int i = w->tid; i < total; i += w->nthreads) {
        int row, hv;
        if (A->n_pairs > 0) {
            row = A->pair_row[i];
            hv = A->pair_hv[i];
        } else {
            row = i / A->sh.HV;
            hv = i % A->sh.HV;
        }
        w->fn(A, row, hv, Sw);
    }
    free(Sw);
    return NULL;
}

static void run_pairs(const orc_args *A, pair_fn fn, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    worker_ctx *ctx = (worker_ctx *)malloc(sizeof(worker_ctx) * nthreads);
    for (int i = 0; i < nthreads; i++) {
        ctx[i].A = A;
        ctx[i].fn = fn;
        ctx[i].tid = i;
        ctx[i].nthreads = nthreads;
        pthread_create(&th[i], NULL, worker, &ctx[i]);
    }
    for (int i = 0; i < nthreads; i++)
        pthread_join(th[i], NULL);
    free(th);
    free(ctx);
}

/* Ring write of the window's raw records at logical positions wp + t.
 * rawk is written once per qk-head, g/beta once per value head. */
static void write_window_records(const orc_args *A)
{
    const orc_shape *sh = &A->sh;
    for (int row = 0; row < sh->B; row++) {
        int s = A->slot[row];
        if (!valid_slot(s, sh))
            continue;
        int wp = clamp_wp(A->wp[s], sh);
        for (int t = 0; t < sh->T; t++) {
            int p = phys_pos(A->base[s], wp + t, sh->L);
            size_t tok = (size_t)row * sh->T + t;
            for (int h = 0; h < sh->H; h++)
                memcpy(A->rawk + (((size_t)s * sh->H + h) * sh->L + p) * sh->K,
                       A->k + (tok * sh->H + h) * sh->K, sh->K * sizeof(double));
            for (int hv = 0; hv < sh->HV; hv++) {
                memcpy(A->rawv + (((size_t)s * sh->HV + hv) * sh->L + p) * sh->V,
                       A->v + (tok * sh->HV + hv) * sh->V, sh->V * sizeof(double));
                double g, beta;
                orc_gate(A->a[tok * sh->HV + hv], A->b[tok * sh->HV + hv], A->A_log[hv],
                         A->dt_bias[hv], sh->softplus_threshold, &g, &beta);
                size_t gi = ((size_t)s * sh->HV + hv) * sh->L + p;
                A->rg[gi] = g;
                A->rb[gi] = beta;
                if (A->rd && A->dwin)
                    memcpy(A->rd + gi * sh->V, A->dwin + (tok * sh->HV + hv) * sh->V,
                           sh->V * sizeof(double));
            }
        }
    }
}

/* ----------------------------------------------------------- entry points */

/* Verify: outputs for every window position; folds flagged rows first when
 * fold_flagged; then (write_ring) records the window in the ring.  With dwin
 * set it also returns each window step's corrected delta, and with rd set the
 * ring write records those deltas beside the raw records (the d-cache ring).   The ring
 * write happens after every pair has read its history, which is equivalent
 * because history and window positions never overlap under the invariant. */
void orc_verify(orc_args *A, int write_ring, int nthreads)
{
    run_pairs(A, verify_pair, nthreads);
    if (write_ring)
        write_window_records(A);
}

/* Ring write alone: record the window's raw records (used to pre-fill rings). */
void orc_write_ring(orc_args *A)
{
    write_window_records(A);
}

void orc_fold(orc_args *A, int nthreads)
{
    run_pairs(A, fold_pair, nthreads);
}

void orc_fill_dring(orc_args *A, int nthreads)
{
    run_pairs(A, fill_dring_pair, nthreads);
}

void orc_snapshot(orc_args *A, int write_ring, int nthreads)
{
    run_pairs(A, snapshot_pair, nthreads);
    if (write_ring)
        write_window_records(A);
}

size_t orc_args_size(void) { return sizeof(orc_args); }
size_t orc_shape_size(void) { return sizeof(orc_shape); }
