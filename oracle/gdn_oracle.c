/*
 * gdn_oracle.c -- plain fp64 CPU oracle of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It includes no header of
 * the GPU path, shares no helper, table or constant with it, and the GPU path
 * never calls it.
 *
 * What it computes, for every independent unit u = (sequence, head), in IEEE
 * double precision and strictly token by token (no chunking, no blocking).
 * The definition is the per-token update of the Qiita article by Nyysyyan on
 * the Linear Attention lineage, section "Gated-DeltaNet":
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,    o_t = S_t q_t
 *
 * Multiplying out the first term, alpha S (I - beta k k^T) = S~ - beta (S~ k) k^T
 * with S~ = alpha S, so one token is evaluated as
 *
 *     S~    = alpha_t S                         (alpha_t = exp(log_alpha_t); 1 when NULL)
 *     e     = beta_t (v_t - S~ k_t)             one value per row of S
 *     S     = S~ + e k_t^T
 *     o_t   = S q_t                             the state AFTER token t's write
 *
 * which is the same expression with its products grouped per row; no term is
 * dropped or reordered beyond that.  The post "linear-attention" on kkkzoz.top
 * (section "Gated DeltaNet") states the same update, and
 * LinearAttention系列解读(六)：DeltaNet的Chunkwise Form推导, section 3 (recursive
 * form), is its alpha = 1 case (DeltaNet).
 *
 * State orientation: S is [Dv][Dk] row-major, o = S q (both pages read the
 * state as S q with S of shape [Dv, Dk]).
 *
 * A second mode (no_erase != 0) drops the prediction term,
 * S = a S + beta v k^T: the Mamba2 update of the same Qiita article (section
 * "Mamba2") with a write strength beta.  The tests pin it against that
 * section's closed form, and it is the definition the no-erase chunk kernels
 * are checked against.
 *
 * Per-channel gate (gate_vec != 0).  log_alpha then holds one value per key
 * channel, [B][T][H][Dk], and the gate of token t is the diagonal matrix
 * D_t = diag(exp(log_alpha_t)) acting on the key side of the state:
 *     S~ = S D_t   (column c of S scaled by alpha_t[c])
 * in place of S~ = alpha_t S; the rest of the token is unchanged, so the two
 * modes read
 *     S_t = S_{t-1} D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T      (erase)
 *     S_t = S_{t-1} D_t + beta_t v_t k_t^T                             (no erase)
 * LinearAttention系列解读(六)：DeltaNet的Chunkwise Form推导, section 1 (引言),
 * names this vector-gated GLA: its transition is a diagonal matrix that scales
 * each state element independently, by an amount fixed by the gate alone.
 * The no-erase form is that GLA with a write strength beta.  With every
 * channel of alpha_t equal it is exactly the scalar gate (the same doubles).
 *
 * Layouts (all dense, row-major):
 *   q, k        [B][T][H][Dk]         v, O   [B][T][H][Dv]
 *   log_alpha   [B][T][H] or NULL ([B][T][H][Dk] with gate_vec)   beta [B][T][H]
 *   S0, S_T     [N][H][Dv][Dk]; S0 may be NULL (zero state)
 *   cu_seqlens  [N+1] or NULL.  NULL: N = B sequences of length T each.
 *               Otherwise B == 1 and sequence n is tokens cu[n] .. cu[n+1]-1.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *q, *k, *v, *log_alpha, *beta, *S0;
    const int64_t *cu;
    int64_t B, T, H, Dk, Dv, N;
    double *O, *S_T;
    int no_erase, gate_vec;
    int64_t next_unit;          /* shared work counter, guarded by mu */
    pthread_mutex_t mu;
} job_t;

/* S: [Dv][Dk] state scratch; ga: [Dk] gate scratch (the gate of each key
 * channel for the current token) */
static void run_unit(const job_t *j, int64_t u, double *S, double *ga) {
    const int64_t n = u / j->H, h = u % j->H;
    const int64_t Dk = j->Dk, Dv = j->Dv, H = j->H;
    int64_t b, t0, t1;
    if (j->cu) { b = 0; t0 = j->cu[n]; t1 = j->cu[n + 1]; }
    else       { b = n; t0 = 0;        t1 = j->T; }

    const int64_t sz = Dv * Dk;
    if (j->S0) memcpy(S, j->S0 + u * sz, (size_t)sz * sizeof(double));
    else       memset(S, 0, (size_t)sz * sizeof(double));

    for (int64_t t = t0; t < t1; ++t) {
        const int64_t x = (b * j->T + t) * H + h;          /* (b, t, h) flat index */
        const double *kt = j->k + x * Dk, *qt = j->q + x * Dk, *vt = j->v + x * Dv;
        if (j->log_alpha && j->gate_vec) {
            for (int64_t c = 0; c < Dk; ++c) ga[c] = exp(j->log_alpha[x * Dk + c]);
        } else {
            const double a = j->log_alpha ? exp(j->log_alpha[x]) : 1.0;
            for (int64_t c = 0; c < Dk; ++c) ga[c] = a;
        }
        const double be = j->beta[x];
        for (int64_t r = 0; r < Dv; ++r) {
            double *row = S + r * Dk;
            double p = 0.0;
            for (int64_t c = 0; c < Dk; ++c) { row[c] *= ga[c]; p += row[c] * kt[c]; }
            const double e = j->no_erase ? be * vt[r] : be * (vt[r] - p);
            for (int64_t c = 0; c < Dk; ++c) row[c] += e * kt[c];
        }
        double *ot = j->O + x * Dv;
        for (int64_t r = 0; r < Dv; ++r) {
            const double *row = S + r * Dk;
            double o = 0.0;
            for (int64_t c = 0; c < Dk; ++c) o += row[c] * qt[c];
            ot[r] = o;
        }
    }
    if (j->S_T) memcpy(j->S_T + u * sz, S, (size_t)sz * sizeof(double));
}

static void *worker(void *arg) {
    job_t *j = (job_t *)arg;
    double *S = (double *)malloc((size_t)(j->Dv * j->Dk + j->Dk) * sizeof(double));
    if (!S) return (void *)1;
    for (;;) {
        pthread_mutex_lock(&j->mu);
        const int64_t u = j->next_unit++;
        pthread_mutex_unlock(&j->mu);
        if (u >= j->N * j->H) break;
        run_unit(j, u, S, S + j->Dv * j->Dk);
    }
    free(S);
    return NULL;
}

/* Runs the recurrence over all units.  Returns the number of threads used
 * (>= 1), or a negative value on a bad argument / allocation failure.
 * n_threads <= 0 means one per online core, capped at the unit count.
 * gate_vec != 0: log_alpha is [B][T][H][Dk] (one gate per key channel). */
int gdn_oracle_forward(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta, const double *S0,
                       const int64_t *cu_seqlens, int64_t n_seqs,
                       int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                       double *O, double *S_T, int n_threads, int no_erase, int gate_vec) {
    if (!q || !k || !v || !beta || !O) return -1;
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return -2;
    if (cu_seqlens && (B != 1 || n_seqs < 1)) return -3;
    job_t j;
    j.q = q; j.k = k; j.v = v; j.log_alpha = log_alpha; j.beta = beta; j.S0 = S0;
    j.cu = cu_seqlens; j.B = B; j.T = T; j.H = H; j.Dk = Dk; j.Dv = Dv;
    j.N = cu_seqlens ? n_seqs : B;
    j.O = O; j.S_T = S_T; j.no_erase = no_erase; j.gate_vec = gate_vec; j.next_unit = 0;
    pthread_mutex_init(&j.mu, NULL);

    int64_t units = j.N * H;
    long cores = sysconf(_SC_NPROCESSORS_ONLN);
    int nt = n_threads > 0 ? n_threads : (int)(cores > 0 ? cores : 1);
    if (nt > units) nt = (int)units;
    if (nt < 1) nt = 1;

    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) { pthread_mutex_destroy(&j.mu); return -4; }
    int started = 0, failed = 0;
    for (int i = 0; i < nt; ++i) {
        if (pthread_create(&th[i], NULL, worker, &j) != 0) break;
        ++started;
    }
    if (started == 0) failed |= (worker(&j) != NULL);   /* no thread: run inline */
    for (int i = 0; i < started; ++i) {
        void *rv = NULL;
        pthread_join(th[i], &rv);
        failed |= (rv != NULL);
    }
    free(th);
    pthread_mutex_destroy(&j.mu);
    if (failed) return -4;
    return started > 0 ? started : 1;
}
