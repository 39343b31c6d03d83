/*
 * gdr_oracle.c -- fp64 CPU oracle for the gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. The GPU library never links it,
 * includes it or calls it, and it shares no code with the GPU library.
 *
 * What it computes: the plain token-by-token definition of the recurrence, in
 * double precision, one token at a time, in the order the pages give:
 *
 *   alpha = exp(g_t)                     scalar or one value per key channel
 *   e     = beta_t * k_t   or  b_t (.) k_t      erase / read key
 *   z     = beta_t * v_t   or  w_t (.) v_t      gated write value
 *   Sbar  = Diag(alpha) S                forget first
 *   u     = z - Sbar^T e                 predict, then correct
 *   S     = Sbar + k u^T                 write
 *   o_t   = scale * S^T q_t              read after the write
 *
 * Sources (page titles; cited below by the short name in brackets):
 *   [family]  "Uma análise das variantes de atenção linear da família DeltaNet"
 *             -- sections "Gated DeltaNet: esquecer primeiro o estado inteiro"
 *             (forget, predict, correct, write), "Kimi Delta Attention:
 *             atenuação por canal" (per-channel decay, read after write,
 *             d_k^-1/2 read scale), its subsection "Transição
 *             diagonal-mais-baixo-posto" (g = log alpha <= 0, the transposed
 *             d_k x d_v layout).
 *   [gdn2]    "Resumo Técnico: Gated DeltaNet-2" -- section "Regra Delta
 *             Portão-2" (update S_t = (I - k (b.k)^T) D S + k (w.v)^T, with
 *             e = b.k, z = w.v; b = w = beta*1 gives KDA, scalar alpha gives
 *             Gated DeltaNet) and "Perspectiva de Atualização de Pesos
 *             Rápidos" (the read of the decayed memory along e is corrected
 *             toward z).
 *   [lesson]  "Gated DeltaNet: o mixer em 48 das 64 camadas" -- section
 *             "Conceito" (16 QK heads serve 48 V heads, three each).
 *
 * Layout (all row-major, contiguous): q, k [B,T,Hqk,dk]; v, o [B,T,Hv,dv];
 * beta [B,T,Hv]; g [B,T,Hv] (scalar decay) or [B,T,Hv,dk] (per channel);
 * b [B,T,Hv,dk]; w [B,T,Hv,dv]; S0, ST [B,Hv,dk,dv] with row i = key
 * channel i, column j = value channel j, so the read is S^T q.
 * V head h reads QK head h / (Hv / Hqk): each QK head serves a contiguous
 * group of V heads (the pages do not say which; this is the reading taken).
 *
 * Value columns evolve independently (the transition multiplies S on the
 * left), so work is split over (sequence, V head, block of value columns)
 * tasks on a pool of threads. Each task runs the token loop above on its own
 * columns only; no arithmetic is reordered across tokens.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

enum { DECAY_NONE = 0, DECAY_SCALAR = 1, DECAY_CHANNEL = 2 };

typedef struct {
    int B, T, Hqk, Hv, dk, dv;
    const double *q, *k, *v, *g, *beta, *bg, *wg, *S0;
    int decay;
    double scale;
    double *o, *ST;
    const int *heads; /* V heads to compute */
    int n_heads;
    int col0, col1, colblk; /* value columns [col0, col1) in blocks of colblk */
    int n_colblk;
    long n_tasks;
    long next; /* next task index, taken under the lock */
    pthread_mutex_t lock;
    int err;
} job_t;

/* One (b, h, column block) task: the token loop of the recurrence. */
static int run_task(const job_t *J, int b, int h, int c0, int c1) {
    const int dk = J->dk, dv = J->dv, T = J->T;
    const int nc = c1 - c0;
    const int group = J->Hv / J->Hqk;
    const int hq = h / group;
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * nc);
    double *alpha = (double *)malloc(sizeof(double) * dk);
    double *e = (double *)malloc(sizeof(double) * dk);
    double *z = (double *)malloc(sizeof(double) * nc);
    double *u = (double *)malloc(sizeof(double) * nc);
    if (!S || !alpha || !e || !z || !u) {
        free(S); free(alpha); free(e); free(z); free(u);
        return -1;
    }

    /* S <- S_0 (zero when absent). */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nc; ++j)
            S[(size_t)i * nc + j] =
                J->S0 ? J->S0[(((size_t)b * J->Hv + h) * dk + i) * dv + c0 + j] : 0.0;

    for (int t = 0; t < T; ++t) {
        const size_t bt = (size_t)b * T + t;
        const double *qt = J->q + (bt * J->Hqk + hq) * dk;
        const double *kt = J->k + (bt * J->Hqk + hq) * dk;
        const double *vt = J->v + (bt * J->Hv + h) * dv;

        /* alpha_t = exp(g_t): [family] "Transição diagonal-mais-baixo-posto". */
        for (int i = 0; i < dk; ++i) {
            if (J->decay == DECAY_NONE)
                alpha[i] = 1.0;
            else if (J->decay == DECAY_SCALAR)
                alpha[i] = exp(J->g[bt * J->Hv + h]);
            else
                alpha[i] = exp(J->g[(bt * J->Hv + h) * dk + i]);
        }

        /* e and z: beta-tied (GDN, KDA) or decoupled gates ([gdn2] "Regra Delta Portão-2"). */
        if (J->beta) {
            const double bt_ = J->beta[bt * J->Hv + h];
            for (int i = 0; i < dk; ++i) e[i] = bt_ * kt[i];
            for (int j = 0; j < nc; ++j) z[j] = bt_ * vt[c0 + j];
        } else {
            const double *bb = J->bg + (bt * J->Hv + h) * dk;
            const double *ww = J->wg + (bt * J->Hv + h) * dv;
            for (int i = 0; i < dk; ++i) e[i] = bb[i] * kt[i];
            for (int j = 0; j < nc; ++j) z[j] = ww[c0 + j] * vt[c0 + j];
        }

        /* Forget: Sbar = Diag(alpha) S. */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < nc; ++j) S[(size_t)i * nc + j] *= alpha[i];

        /* Predict and correct: u = z - Sbar^T e. */
        for (int j = 0; j < nc; ++j) {
            double r = 0.0;
            for (int i = 0; i < dk; ++i) r += S[(size_t)i * nc + j] * e[i];
            u[j] = z[j] - r;
        }

        /* Write: S = Sbar + k u^T. */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < nc; ++j) S[(size_t)i * nc + j] += kt[i] * u[j];

        /* Read after write: o_t = scale * S^T q_t. */
        double *ot = J->o + (bt * J->Hv + h) * dv;
        for (int j = 0; j < nc; ++j) {
            double r = 0.0;
            for (int i = 0; i < dk; ++i) r += S[(size_t)i * nc + j] * qt[i];
            ot[c0 + j] = J->scale * r;
        }
    }

    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nc; ++j)
            J->ST[(((size_t)b * J->Hv + h) * dk + i) * dv + c0 + j] = S[(size_t)i * nc + j];

    free(S); free(alpha); free(e); free(z); free(u);
    return 0;
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        long task = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (task >= J->n_tasks) break;
        const int cb = (int)(task % J->n_colblk);
        const long bh = task / J->n_colblk;
        const int hi = (int)(bh % J->n_heads);
        const int b = (int)(bh / J->n_heads);
        const int c0 = J->col0 + cb * J->colblk;
        int c1 = c0 + J->colblk;
        if (c1 > J->col1) c1 = J->col1;
        if (run_task(J, b, J->heads[hi], c0, c1) != 0) {
            pthread_mutex_lock(&J->lock);
            J->err = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

/*
 * Run the recurrence. Returns 0 on success, -1 on a bad argument, -2 when out
 * of host memory. heads == NULL computes every V head; otherwise only the
 * n_heads listed ones (the other heads' entries of o and ST are not written).
 * Only value columns [col0, col1) are computed. beta != NULL selects the tied
 * gate (e = beta k, z = beta v) and then bg, wg must be NULL; beta == NULL
 * needs both bg and wg. g may be NULL only with decay == 0.
 */
int gdr_oracle_recurrent(int B, int T, int Hqk, int Hv, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *g, int decay, const double *beta,
                         const double *bg, const double *wg, double scale,
                         const double *S0, double *o, double *ST,
                         const int *heads, int n_heads, int col0, int col1,
                         int nthreads) {
    if (B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0) return -1;
    if (Hv % Hqk != 0) return -1;
    if (!q || !k || !v || !o || !ST) return -1;
    if (decay < DECAY_NONE || decay > DECAY_CHANNEL) return -1;
    if ((decay != DECAY_NONE) != (g != NULL)) return -1;
    if (beta ? (bg || wg) : (!bg || !wg)) return -1;
    if (col0 < 0 || col1 > dv || col0 >= col1) return -1;

    int *all = NULL;
    if (!heads) {
        all = (int *)malloc(sizeof(int) * Hv);
        if (!all) return -2;
        for (int h = 0; h < Hv; ++h) all[h] = h;
        heads = all;
        n_heads = Hv;
    }
    for (int i = 0; i < n_heads; ++i)
        if (heads[i] < 0 || heads[i] >= Hv) { free(all); return -1; }

    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.Hqk = Hqk; J.Hv = Hv; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.bg = bg; J.wg = wg;
    J.S0 = S0; J.decay = decay; J.scale = scale; J.o = o; J.ST = ST;
    J.heads = heads; J.n_heads = n_heads;
    J.col0 = col0; J.col1 = col1;
    J.colblk = 16;
    J.n_colblk = (col1 - col0 + J.colblk - 1) / J.colblk;
    J.n_tasks = (long)B * n_heads * J.n_colblk;
    pthread_mutex_init(&J.lock, NULL);

    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads == 1 || J.n_tasks <= 1) {
        worker(&J);
    } else {
        pthread_t th[256];
        int started = 0;
        for (int i = 0; i < nthreads; ++i)
            if (pthread_create(&th[i], NULL, worker, &J) == 0) ++started;
        if (started == 0) worker(&J);
        for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    }
    pthread_mutex_destroy(&J.lock);
    free(all);
    return J.err ? -2 : 0;
}
