/*
 * gdn2_oracle.c -- fp64 CPU oracle for the Gated DeltaNet-2 recurrent operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product (the HIP
 * library and its Python binding) never calls into it and shares no code,
 * header, table or helper with it.
 *
 * What it computes (source: "Gated DeltaNet-2: decoupling erase and write",
 * iplexlaw.co.kr blog, section "Independent control on two axes"; confirmed by
 * the paper abstract in the OpenAlex record of arXiv:2605.22791): for every
 * (batch, head) pair the state S (dk x dv, key axis = rows) is carried through
 * the tokens one at a time.  For token t, with key channels c and value
 * channels j:
 *
 *   a_c    = exp(log_alpha[t,c])            channel-wise decay on the key axis
 *   e_c    = b[t,c] * k[t,c]                erase gate acts on key channels
 *   z_j    = w[t,j] * v[t,j]                write gate acts on value channels
 *   Sb     = diag(a) S                      decay first
 *   r_j    = sum_c Sb[c,j] e_c              then read through the erased key
 *   S      = Sb + k (z - r)^T               then write along the raw key
 *   o[t,j] = sum_c S[c,j] q[t,c]            the query reads the UPDATED state
 *
 * Nothing is blocked, fused or reordered: this is the per-token rule written
 * out, in double precision.  The backward pass is the exact reverse-mode
 * adjoint of those same per-token steps (loss = sum dO*o + sum dS_final*S_T),
 * walked from t = T-1 down to 0.  The state before each token is recomputed
 * from checkpoints kept every CKPT tokens; that is bookkeeping, not a change of
 * arithmetic.
 *
 * Layouts (all contiguous, row-major):
 *   q, k, log_alpha, b     [B, T, H, dk]
 *   v, w, o                [B, T, H, dv]
 *   S0, S_final            [B, H, dk, dv]
 * Work is split over (batch, head) pairs with POSIX threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define CKPT 64

typedef struct {
    int B, T, H, dk, dv;
    const double *q, *k, *v, *la, *bg, *wg, *S0;
    double *o, *S_final;
    /* backward only */
    const double *dO, *dS_final;
    double *dq, *dk_, *dv_, *dla, *db, *dw, *dS0;
    /* work distribution */
    int next;               /* next (b,h) pair to take */
    pthread_mutex_t lock;
    int failed;
} job_t;

static size_t tok(const job_t *J, int b, int t, int h, int D) {
    return (((size_t)b * J->T + t) * J->H + h) * (size_t)D;
}

/* One step of the rule above: S (dk x dv) is updated in place.  Returns u = z - r
 * in u_out (dv), the decay a (dk) and e (dk) so that the backward can reuse the
 * definitions without re-deriving them. */
static void step(int dk, int dv, const double *q, const double *k, const double *v,
                 const double *la, const double *bg, const double *wg,
                 double *S, double *o, double *a, double *e, double *u) {
    for (int c = 0; c < dk; ++c) {
        a[c] = exp(la[c]);
        e[c] = bg[c] * k[c];
    }
    /* decay first */
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a[c];
    /* read r = Sb^T e, then u = z - r */
    for (int j = 0; j < dv; ++j) {
        double r = 0.0;
        for (int c = 0; c < dk; ++c) r += S[(size_t)c * dv + j] * e[c];
        u[j] = wg[j] * v[j] - r;
    }
    /* write S = Sb + k u^T */
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] += k[c] * u[j];
    /* output reads the updated state */
    if (o) {
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += S[(size_t)c * dv + j] * q[c];
            o[j] = acc;
        }
    }
}

static int take(job_t *J) {
    pthread_mutex_lock(&J->lock);
    int p = J->next < J->B * J->H ? J->next++ : -1;
    pthread_mutex_unlock(&J->lock);
    return p;
}

static void *fwd_worker(void *arg) {
    job_t *J = (job_t *)arg;
    const int dk = J->dk, dv = J->dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *a = (double *)malloc(sizeof(double) * dk);
    double *e = (double *)malloc(sizeof(double) * dk);
    double *u = (double *)malloc(sizeof(double) * dv);
    if (!S || !a || !e || !u) {
        J->failed = 1;
        free(S); free(a); free(e); free(u);
        return NULL;
    }
    int p;
    while ((p = take(J)) >= 0) {
        const int b = p / J->H, h = p % J->H;
        const size_t soff = ((size_t)b * J->H + h) * (size_t)dk * dv;
        if (J->S0) memcpy(S, J->S0 + soff, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);
        for (int t = 0; t < J->T; ++t) {
            const size_t ok = tok(J, b, t, h, dk), ov = tok(J, b, t, h, dv);
            step(dk, dv, J->q + ok, J->k + ok, J->v + ov, J->la + ok, J->bg + ok, J->wg + ov,
                 S, J->o + ov, a, e, u);
        }
        if (J->S_final) memcpy(J->S_final + soff, S, sizeof(double) * (size_t)dk * dv);
    }
    free(S); free(a); free(e); free(u);
    return NULL;
}

/* Reverse-mode adjoint of `step`, token by token.  G holds dL/dS_t on entry
 * (the gradient with respect to the state AFTER token t) and dL/dS_{t-1} on
 * exit.  Sprev is the state before token t (untouched). */
static void back_step(int dk, int dv, const double *q, const double *k, const double *v,
                      const double *la, const double *bg, const double *wg,
                      const double *Sprev, const double *dO, double *G,
                      double *dq, double *dkk, double *dvv, double *dla, double *db, double *dw,
                      double *Snext, double *a, double *e, double *u, double *du, double *de) {
    /* recompute the forward quantities of this token from Sprev */
    memcpy(Snext, Sprev, sizeof(double) * (size_t)dk * dv);
    step(dk, dv, q, k, v, la, bg, wg, Snext, NULL, a, e, u);
    /* o = S_t^T q  ->  dq = S_t dO,  G += q dO^T */
    for (int c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) acc += Snext[(size_t)c * dv + j] * dO[j];
        dq[c] = acc;
        for (int j = 0; j < dv; ++j) G[(size_t)c * dv + j] += q[c] * dO[j];
    }
    /* S_t = Sb + k u^T  ->  dSb = G, dk = G u, du = G^T k */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += G[(size_t)c * dv + j] * k[c];
        du[j] = acc;
    }
    for (int c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) acc += G[(size_t)c * dv + j] * u[j];
        dkk[c] = acc;
    }
    /* u = z - Sb^T e  ->  dz = du, de = -Sb du, dSb -= e du^T ; Sb = diag(a) Sprev */
    for (int c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) acc += a[c] * Sprev[(size_t)c * dv + j] * du[j];
        de[c] = -acc;
    }
    /* z = w * v */
    for (int j = 0; j < dv; ++j) {
        dvv[j] = du[j] * wg[j];
        dw[j] = du[j] * v[j];
    }
    /* e = b * k */
    for (int c = 0; c < dk; ++c) {
        db[c] = de[c] * k[c];
        dkk[c] += de[c] * bg[c];
    }
    /* Sb = diag(a) Sprev, a = exp(la):  dla_c = a_c * sum_j dSb[c,j] Sprev[c,j];
     * dSprev = diag(a) dSb */
    for (int c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
            const double dsb = G[(size_t)c * dv + j] - e[c] * du[j];
            acc += dsb * Sprev[(size_t)c * dv + j];
            G[(size_t)c * dv + j] = a[c] * dsb;
        }
        dla[c] = a[c] * acc;
    }
}

static void *bwd_worker(void *arg) {
    job_t *J = (job_t *)arg;
    const int dk = J->dk, dv = J->dv, T = J->T;
    const size_t SS = (size_t)dk * dv;
    const int nck = (T + CKPT - 1) / CKPT;
    double *ck = (double *)malloc(sizeof(double) * SS * nck);        /* state before each segment */
    double *seg = (double *)malloc(sizeof(double) * SS * (CKPT + 1)); /* states inside one segment */
    double *G = (double *)malloc(sizeof(double) * SS);
    double *Sn = (double *)malloc(sizeof(double) * SS);
    double *a = (double *)malloc(sizeof(double) * dk);
    double *e = (double *)malloc(sizeof(double) * dk);
    double *de = (double *)malloc(sizeof(double) * dk);
    double *u = (double *)malloc(sizeof(double) * dv);
    double *du = (double *)malloc(sizeof(double) * dv);
    if (!ck || !seg || !G || !Sn || !a || !e || !de || !u || !du) {
        J->failed = 1;
        goto done;
    }
    int p;
    while ((p = take(J)) >= 0) {
        const int b = p / J->H, h = p % J->H;
        const size_t soff = ((size_t)b * J->H + h) * SS;
        /* forward pass, keeping the state at the start of every segment */
        double *S = G; /* G is free until the reverse pass starts */
        if (J->S0) memcpy(S, J->S0 + soff, sizeof(double) * SS);
        else memset(S, 0, sizeof(double) * SS);
        for (int t = 0; t < T; ++t) {
            if (t % CKPT == 0) memcpy(ck + (size_t)(t / CKPT) * SS, S, sizeof(double) * SS);
            const size_t ok = tok(J, b, t, h, dk), ov = tok(J, b, t, h, dv);
            step(dk, dv, J->q + ok, J->k + ok, J->v + ov, J->la + ok, J->bg + ok, J->wg + ov,
                 S, NULL, a, e, u);
        }
        /* reverse pass */
        if (J->dS_final) memcpy(G, J->dS_final + soff, sizeof(double) * SS);
        else memset(G, 0, sizeof(double) * SS);
        for (int sgi = nck - 1; sgi >= 0; --sgi) {
            const int t0 = sgi * CKPT;
            const int t1 = t0 + CKPT < T ? t0 + CKPT : T;
            memcpy(seg, ck + (size_t)sgi * SS, sizeof(double) * SS);
            for (int t = t0; t < t1 - 1; ++t) {
                const size_t ok = tok(J, b, t, h, dk), ov = tok(J, b, t, h, dv);
                memcpy(seg + (size_t)(t - t0 + 1) * SS, seg + (size_t)(t - t0) * SS, sizeof(double) * SS);
                step(dk, dv, J->q + ok, J->k + ok, J->v + ov, J->la + ok, J->bg + ok, J->wg + ov,
                     seg + (size_t)(t - t0 + 1) * SS, NULL, a, e, u);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const size_t ok = tok(J, b, t, h, dk), ov = tok(J, b, t, h, dv);
                back_step(dk, dv, J->q + ok, J->k + ok, J->v + ov, J->la + ok, J->bg + ok, J->wg + ov,
                          seg + (size_t)(t - t0) * SS, J->dO + ov, G,
                          J->dq + ok, J->dk_ + ok, J->dv_ + ov, J->dla + ok, J->db + ok, J->dw + ov,
                          Sn, a, e, u, du, de);
            }
        }
        if (J->dS0) memcpy(J->dS0 + soff, G, sizeof(double) * SS);
    }
done:
    free(ck); free(seg); free(G); free(Sn); free(a); free(e); free(de); free(u); free(du);
    return NULL;
}

static int run(job_t *J, void *(*fn)(void *), int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > J->B * J->H) nthreads = J->B * J->H;
    pthread_mutex_init(&J->lock, NULL);
    J->next = 0;
    J->failed = 0;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -1;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, fn, J) == 0) ++started;
    }
    if (started == 0) fn(J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J->lock);
    return J->failed ? -1 : 0;
}

/* Forward: o and (optionally) S_final.  S0 may be NULL (zeros).  Returns 0 on
 * success, -1 on allocation failure or bad sizes. */
int gdn2_oracle_fwd(int B, int T, int H, int dk, int dv,
                    const double *q, const double *k, const double *v,
                    const double *log_alpha, const double *b, const double *w,
                    const double *S0, double *o, double *S_final, int nthreads) {
    if (B < 1 || T < 1 || H < 1 || dk < 1 || dv < 1) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.la = log_alpha; J.bg = b; J.wg = w; J.S0 = S0;
    J.o = o; J.S_final = S_final;
    return run(&J, fwd_worker, nthreads);
}

/* Backward of loss = sum(dO * o) + sum(dS_final * S_final) with respect to
 * q, k, v, log_alpha, b, w and S0.  dS_final and dS0 may be NULL. */
int gdn2_oracle_bwd(int B, int T, int H, int dk, int dv,
                    const double *q, const double *k, const double *v,
                    const double *log_alpha, const double *b, const double *w,
                    const double *S0, const double *dO, const double *dS_final,
                    double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                    double *db, double *dw, double *dS0, int nthreads) {
    if (B < 1 || T < 1 || H < 1 || dk < 1 || dv < 1) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.la = log_alpha; J.bg = b; J.wg = w; J.S0 = S0;
    J.dO = dO; J.dS_final = dS_final;
    J.dq = dq; J.dk_ = dk_out; J.dv_ = dv_out; J.dla = dlog_alpha; J.db = db; J.dw = dw; J.dS0 = dS0;
    return run(&J, bwd_worker, nthreads);
}
