/*
 * wkv7_oracle.c -- plain fp64 CPU definition of the RWKV-7 WKV7 recurrence,
 * forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the HIP library; the HIP library never calls it.
 *
 * What it computes (rwkv-mlx page, section "Metal kernel architecture",
 * forward block; the per-element form is the plain reading of that block):
 * every head keeps a D x D state S (row i runs with v and y, column j with
 * r, w, k, a, b).  For each token t, in order:
 *
 *   F1  if t is a multiple of 32: ckpt[t/32] = S   (state entering the chunk)
 *   F2  sa[i]   = sum_j S[i][j] * a_t[j]                (S before the update)
 *   F3  S[i][j] = w_t[j]*S[i][j] + v_t[i]*k_t[j] + sa[i]*b_t[j]
 *   F4  y_t[i]  = sum_j S[i][j] * r_t[j]                (S after the update)
 *
 * and hT = S after the last token.  The RWKV-LM README page warns that the
 * decayed-state update needs at least fp32 because w may sit very near 1;
 * this oracle goes further and uses fp64 throughout.
 *
 * Backward (same page, section "Metal kernel architecture", backward block:
 * walk the tokens in reverse and produce dr, dw, dk, dv, da, db).  This
 * oracle does not use chunk checkpoints: it keeps every state S_{-1..T-1}
 * of the head in memory (S_{-1} = h0), then with g = dhT (or 0) and for
 * t = T-1 down to 0:
 *
 *   B1  dr_t[j] = sum_i dy_t[i] * S_t[i][j]
 *   B2  g[i][j] += dy_t[i] * r_t[j]
 *   B3  dw_t[j] = sum_i g[i][j] * S_{t-1}[i][j]
 *   B4  dk_t[j] = sum_i g[i][j] * v_t[i]
 *   B5  dv_t[i] = sum_j g[i][j] * k_t[j]
 *   B6  dsa[i]  = sum_j g[i][j] * b_t[j]
 *   B7  db_t[j] = sum_i g[i][j] * sa_t[i]
 *   B8  da_t[j] = sum_i dsa[i] * S_{t-1}[i][j]
 *   B9  g[i][j] = w_t[j]*g[i][j] + dsa[i]*a_t[j]
 *
 * and dh0 = g.  These are the chain rule applied to F2-F4, nothing more.
 *
 * Layouts: r,w,k,v,a,b,y,dy and the six input gradients are (B,T,H,D)
 * row-major; h0, hT, dhT, dh0 are (B,H,D,D) with S[i][j] at i*D+j;
 * ckpt is (B,H,NC,D,D) with NC = ceil(T/32).
 *
 * Heads (b,h) are independent; the only parallelism here is one head per
 * worker thread.  Within a head the arithmetic is in the order written above.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_CHUNK 32

typedef struct {
    int B, T, H, D;
    const double *r, *w, *k, *v, *a, *b, *h0;
    const double *dy, *dhT;
    double *y, *ckpt, *hT;
    double *dr, *dw, *dk, *dv, *da, *db, *dh0;
    int nthreads;
    int is_bwd;
    int status;
} oracle_job;

typedef struct {
    oracle_job *job;
    int tid;
} oracle_worker;

/* offset of element (bb, t, hh, 0) of a (B,T,H,D) tensor */
static size_t tok_off(const oracle_job *J, int bb, int t, int hh)
{
    return (((size_t)bb * J->T + t) * J->H + hh) * (size_t)J->D;
}

/* offset of the (bb, hh) D x D state in a (B,H,D,D) tensor */
static size_t state_off(const oracle_job *J, int bb, int hh)
{
    return ((size_t)bb * J->H + hh) * (size_t)J->D * J->D;
}

/* F2-F4 for one token: S is updated in place, sa and y receive D values. */
static void token_forward(int D, double *S, const double *rt, const double *wt,
                          const double *kt, const double *vt, const double *at,
                          const double *bt, double *sa, double *yt)
{
    for (int i = 0; i < D; ++i) {
        double acc = 0.0;
        for (int j = 0; j < D; ++j) acc += S[i * D + j] * at[j];
        sa[i] = acc;
    }
    for (int i = 0; i < D; ++i)
        for (int j = 0; j < D; ++j)
            S[i * D + j] = wt[j] * S[i * D + j] + vt[i] * kt[j] + sa[i] * bt[j];
    if (yt) {
        for (int i = 0; i < D; ++i) {
            double acc = 0.0;
            for (int j = 0; j < D; ++j) acc += S[i * D + j] * rt[j];
            yt[i] = acc;
        }
    }
}

static int forward_head(oracle_job *J, int bb, int hh)
{
    const int D = J->D, T = J->T;
    const int NC = (T + ORACLE_CHUNK - 1) / ORACLE_CHUNK;
    double *S = (double *)calloc((size_t)D * D, sizeof(double));
    double *sa = (double *)malloc((size_t)D * sizeof(double));
    if (!S || !sa) { free(S); free(sa); return 1; }
    if (J->h0) memcpy(S, J->h0 + state_off(J, bb, hh), (size_t)D * D * sizeof(double));
    for (int t = 0; t < T; ++t) {
        if (J->ckpt && t % ORACLE_CHUNK == 0) {
            size_t off = (((size_t)bb * J->H + hh) * NC + t / ORACLE_CHUNK) * (size_t)D * D;
            memcpy(J->ckpt + off, S, (size_t)D * D * sizeof(double));
        }
        size_t o = tok_off(J, bb, t, hh);
        token_forward(D, S, J->r + o, J->w + o, J->k + o, J->v + o, J->a + o, J->b + o,
                      sa, J->y ? J->y + o : NULL);
    }
    if (J->hT) memcpy(J->hT + state_off(J, bb, hh), S, (size_t)D * D * sizeof(double));
    free(S);
    free(sa);
    return 0;
}

static int backward_head(oracle_job *J, int bb, int hh)
{
    const int D = J->D, T = J->T;
    const size_t DD = (size_t)D * D;
    /* states[t+1] = S_t for t = -1 .. T-1, sa_all[t] = sa_t */
    double *states = (double *)malloc((size_t)(T + 1) * DD * sizeof(double));
    double *sa_all = (double *)malloc((size_t)T * D * sizeof(double));
    double *g = (double *)calloc(DD, sizeof(double));
    double *dsa = (double *)malloc((size_t)D * sizeof(double));
    if (!states || !sa_all || !g || !dsa) {
        free(states); free(sa_all); free(g); free(dsa);
        return 1;
    }
    if (J->h0) memcpy(states, J->h0 + state_off(J, bb, hh), DD * sizeof(double));
    else memset(states, 0, DD * sizeof(double));
    for (int t = 0; t < T; ++t) {
        size_t o = tok_off(J, bb, t, hh);
        memcpy(states + (size_t)(t + 1) * DD, states + (size_t)t * DD, DD * sizeof(double));
        token_forward(D, states + (size_t)(t + 1) * DD, J->r + o, J->w + o, J->k + o,
                      J->v + o, J->a + o, J->b + o, sa_all + (size_t)t * D, NULL);
    }
    if (J->dhT) memcpy(g, J->dhT + state_off(J, bb, hh), DD * sizeof(double));

    for (int t = T - 1; t >= 0; --t) {
        size_t o = tok_off(J, bb, t, hh);
        const double *St = states + (size_t)(t + 1) * DD;   /* S_t     */
        const double *Sp = states + (size_t)t * DD;         /* S_{t-1} */
        const double *sat = sa_all + (size_t)t * D;
        const double *rt = J->r + o, *wt = J->w + o, *kt = J->k + o;
        const double *vt = J->v + o, *at = J->a + o, *bt = J->b + o;
        const double *dyt = J->dy + o;
        double *drt = J->dr + o, *dwt = J->dw + o, *dkt = J->dk + o;
        double *dvt = J->dv + o, *dat = J->da + o, *dbt = J->db + o;

        for (int j = 0; j < D; ++j) {                                   /* B1 */
            double acc = 0.0;
            for (int i = 0; i < D; ++i) acc += dyt[i] * St[i * D + j];
            drt[j] = acc;
        }
        for (int i = 0; i < D; ++i)                                     /* B2 */
            for (int j = 0; j < D; ++j) g[i * D + j] += dyt[i] * rt[j];
        for (int j = 0; j < D; ++j) {                                   /* B3 B4 B7 */
            double aw = 0.0, ak = 0.0, ab = 0.0;
            for (int i = 0; i < D; ++i) {
                aw += g[i * D + j] * Sp[i * D + j];
                ak += g[i * D + j] * vt[i];
                ab += g[i * D + j] * sat[i];
            }
            dwt[j] = aw;
            dkt[j] = ak;
            dbt[j] = ab;
        }
        for (int i = 0; i < D; ++i) {                                   /* B5 B6 */
            double av = 0.0, as = 0.0;
            for (int j = 0; j < D; ++j) {
                av += g[i * D + j] * kt[j];
                as += g[i * D + j] * bt[j];
            }
            dvt[i] = av;
            dsa[i] = as;
        }
        for (int j = 0; j < D; ++j) {                                   /* B8 */
            double acc = 0.0;
            for (int i = 0; i < D; ++i) acc += dsa[i] * Sp[i * D + j];
            dat[j] = acc;
        }
        for (int i = 0; i < D; ++i)                                     /* B9 */
            for (int j = 0; j < D; ++j) g[i * D + j] = wt[j] * g[i * D + j] + dsa[i] * at[j];
    }
    if (J->dh0) memcpy(J->dh0 + state_off(J, bb, hh), g, DD * sizeof(double));
    free(states);
    free(sa_all);
    free(g);
    free(dsa);
    return 0;
}

static void *worker_main(void *arg)
{
    oracle_worker *W = (oracle_worker *)arg;
    oracle_job *J = W->job;
    int nheads = J->B * J->H;
    for (int n = W->tid; n < nheads; n += J->nthreads) {
        int bb = n / J->H, hh = n % J->H;
        int rc = J->is_bwd ? backward_head(J, bb, hh) : forward_head(J, bb, hh);
        if (rc) J->status = rc;   /* any nonzero marks failure; a benign race */
    }
    return NULL;
}

static int run_job(oracle_job *J)
{
    if (J->B <= 0 || J->T <= 0 || J->H <= 0 || J->D <= 0) return 2;
    int nheads = J->B * J->H;
    if (J->nthreads < 1) J->nthreads = 1;
    if (J->nthreads > nheads) J->nthreads = nheads;
    J->status = 0;
    pthread_t *th = (pthread_t *)malloc((size_t)J->nthreads * sizeof(pthread_t));
    oracle_worker *ws = (oracle_worker *)malloc((size_t)J->nthreads * sizeof(oracle_worker));
    if (!th || !ws) { free(th); free(ws); return 1; }
    int started = 0;
    for (int i = 1; i < J->nthreads; ++i) {
        ws[i].job = J;
        ws[i].tid = i;
        if (pthread_create(&th[i], NULL, worker_main, &ws[i]) != 0) { J->status = 3; break; }
        started = i;
    }
    ws[0].job = J;
    ws[0].tid = 0;
    if (J->status == 0) worker_main(&ws[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    free(th);
    free(ws);
    return J->status;
}

/* Forward.  h0, ckpt, hT may be NULL (zero initial state / not wanted).
 * y may be NULL.  Returns 0 on success. */
int oracle_wkv7_fwd(int B, int T, int H, int D,
                    const double *r, const double *w, const double *k,
                    const double *v, const double *a, const double *b,
                    const double *h0, double *y, double *ckpt, double *hT,
                    int nthreads)
{
    oracle_job J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.D = D;
    J.r = r; J.w = w; J.k = k; J.v = v; J.a = a; J.b = b; J.h0 = h0;
    J.y = y; J.ckpt = ckpt; J.hT = hT;
    J.nthreads = nthreads;
    J.is_bwd = 0;
    return run_job(&J);
}

/* Backward.  h0 and dhT may be NULL (zero); dh0 may be NULL.
 * All six input-gradient outputs are required. */
int oracle_wkv7_bwd(int B, int T, int H, int D,
                    const double *r, const double *w, const double *k,
                    const double *v, const double *a, const double *b,
                    const double *h0, const double *dy, const double *dhT,
                    double *dr, double *dw, double *dk, double *dv,
                    double *da, double *db, double *dh0, int nthreads)
{
    if (!dy || !dr || !dw || !dk || !dv || !da || !db) return 2;
    oracle_job J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.D = D;
    J.r = r; J.w = w; J.k = k; J.v = v; J.a = a; J.b = b; J.h0 = h0;
    J.dy = dy; J.dhT = dhT;
    J.dr = dr; J.dw = dw; J.dk = dk; J.dv = dv; J.da = da; J.db = db; J.dh0 = dh0;
    J.nthreads = nthreads;
    J.is_bwd = 1;
    return run_job(&J);
}

/*
 * Time-mix prologue: w, a and b as functions of the layer's raw projections
 * (w_raw, kappa, alpha), one token row of D channels at a time.  The pages
 * print no formula for this step (they name the x070 architecture only); the
 * definitions below are those of the synthetic workloads' w, a and b (a
 * decay through a scaled sigmoid, a unit-norm removal key and a gated
 * replacement key), read as the layer's own arithmetic:
 *
 *   P1  sw[j] = 1 / (1 + exp(-w_raw[j]))
 *   P2  w[j]  = exp(-exp(-1/2) * sw[j])
 *   P3  n     = sqrt(sum_j kappa[j]^2);  kh[j] = kappa[j] / n   (kh = 0 if n = 0)
 *   P4  a[j]  = -kh[j]
 *   P5  sa[j] = 1 / (1 + exp(-alpha[j]));  b[j] = kh[j] * sa[j]
 *
 * Backward, given dw, da, db (the chain rule through P1-P5):
 *
 *   Q1  dw_raw[j] = dw[j] * w[j] * (-exp(-1/2)) * sw[j] * (1 - sw[j])
 *   Q2  g[j]      = -da[j] + db[j] * sa[j]              (gradient w.r.t. kh)
 *   Q3  dalpha[j] = db[j] * kh[j] * sa[j] * (1 - sa[j])
 *   Q4  dkappa[j] = (g[j] - kh[j] * sum_m kh[m] g[m]) / n   (0 if n = 0)
 */
static double logistic(double x) { return 1.0 / (1.0 + exp(-x)); }

int oracle_proj_fwd(long rows, int D, const double *w_raw, const double *kappa,
                    const double *alpha, double *w, double *a, double *b)
{
    if (rows < 0 || D < 1) return 2;
    const double c = exp(-0.5);
    for (long row = 0; row < rows; ++row) {
        const size_t o = (size_t)row * (size_t)D;
        double nn = 0.0;
        for (int j = 0; j < D; ++j) nn += kappa[o + j] * kappa[o + j];
        const double n = sqrt(nn);
        for (int j = 0; j < D; ++j) {
            const double kh = n > 0.0 ? kappa[o + j] / n : 0.0;
            w[o + j] = exp(-c * logistic(w_raw[o + j]));
            a[o + j] = -kh;
            b[o + j] = kh * logistic(alpha[o + j]);
        }
    }
    return 0;
}

int oracle_proj_bwd(long rows, int D, const double *w_raw, const double *kappa,
                    const double *alpha, const double *dw, const double *da,
                    const double *db, double *dw_raw, double *dkappa, double *dalpha)
{
    if (rows < 0 || D < 1) return 2;
    const double c = exp(-0.5);
    for (long row = 0; row < rows; ++row) {
        const size_t o = (size_t)row * (size_t)D;
        double nn = 0.0;
        for (int j = 0; j < D; ++j) nn += kappa[o + j] * kappa[o + j];
        const double n = sqrt(nn);
        double proj = 0.0;   /* sum_m kh[m] g[m] */
        for (int j = 0; j < D; ++j) {
            const double kh = n > 0.0 ? kappa[o + j] / n : 0.0;
            const double sa = logistic(alpha[o + j]);
            proj += kh * (-da[o + j] + db[o + j] * sa);
        }
        for (int j = 0; j < D; ++j) {
            const double sw = logistic(w_raw[o + j]);
            const double wj = exp(-c * sw);
            dw_raw[o + j] = dw[o + j] * wj * (-c) * sw * (1.0 - sw);
            const double kh = n > 0.0 ? kappa[o + j] / n : 0.0;
            const double sa = logistic(alpha[o + j]);
            const double g = -da[o + j] + db[o + j] * sa;
            dalpha[o + j] = db[o + j] * kh * sa * (1.0 - sa);
            dkappa[o + j] = n > 0.0 ? (g - kh * proj) / n : 0.0;
        }
    }
    return 0;
}
