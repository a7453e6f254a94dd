/* Drives the fp64 oracle on small cases (ragged T across the 64-token checkpoints, several
 * threads, optional arguments absent) so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can check its memory accesses and arithmetic.  Exit 0 on success. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int gdn2_oracle_fwd(int B, int T, int H, int dk, int dv, const double *q, const double *k, const double *v,
                    const double *log_alpha, const double *b, const double *w, const double *S0, double *o,
                    double *S_final, int nthreads);
int gdn2_oracle_bwd(int B, int T, int H, int dk, int dv, const double *q, const double *k, const double *v,
                    const double *log_alpha, const double *b, const double *w, const double *S0, const double *dO,
                    const double *dS_final, double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                    double *db, double *dw, double *dS0, int nthreads);

static unsigned long long state = 88172645463325252ull;
static double uni(void) {   /* xorshift64, in [-1, 1) */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 4503599627370496.0 - 1.0;
}

static double *fill(size_t n, double scale, double shift) {
    double *p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = scale * uni() + shift;
    return p;
}

static int run(int B, int T, int H, int dk, int dv, int with_opt, int nthreads) {
    const size_t nk = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv, ns = (size_t)B * H * dk * dv;
    double *q = fill(nk, 0.3, 0), *k = fill(nk, 0.3, 0), *v = fill(nv, 1, 0), *la = fill(nk, 0.05, -0.08);
    double *b = fill(nk, 0.4, 0.5), *w = fill(nv, 0.4, 0.5), *S0 = fill(ns, 0.1, 0), *dO = fill(nv, 1, 0);
    double *dSf = fill(ns, 0.01, 0);
    double *o = malloc(nv * sizeof(double)), *Sf = malloc(ns * sizeof(double));
    double *dq = malloc(nk * sizeof(double)), *dkk = malloc(nk * sizeof(double)), *dvv = malloc(nv * sizeof(double));
    double *dla = malloc(nk * sizeof(double)), *db = malloc(nk * sizeof(double)), *dw = malloc(nv * sizeof(double));
    double *dS0 = malloc(ns * sizeof(double));
    int rc = gdn2_oracle_fwd(B, T, H, dk, dv, q, k, v, la, b, w, with_opt ? S0 : NULL, o, with_opt ? Sf : NULL,
                             nthreads);
    rc |= gdn2_oracle_bwd(B, T, H, dk, dv, q, k, v, la, b, w, with_opt ? S0 : NULL, dO, with_opt ? dSf : NULL, dq,
                          dkk, dvv, dla, db, dw, with_opt ? dS0 : NULL, nthreads);
    double sum = 0;
    for (size_t i = 0; i < nv; ++i) sum += o[i] + dvv[i];
    for (size_t i = 0; i < nk; ++i) sum += dq[i] + dkk[i] + dla[i] + db[i];
    printf("B%d T%d H%d dk%d dv%d opt%d threads%d rc %d checksum %.6e\n", B, T, H, dk, dv, with_opt, nthreads, rc,
           sum);
    int bad = rc != 0 || !isfinite(sum);
    free(q); free(k); free(v); free(la); free(b); free(w); free(S0); free(dO); free(dSf); free(o); free(Sf);
    free(dq); free(dkk); free(dvv); free(dla); free(db); free(dw); free(dS0);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run(1, 1, 1, 8, 8, 1, 1);
    bad |= run(2, 150, 2, 16, 8, 1, 3);
    bad |= run(1, 130, 3, 8, 16, 0, 2);
    bad |= run(1, 64, 1, 32, 32, 1, 1);
    /* invalid sizes are refused */
    bad |= gdn2_oracle_fwd(0, 4, 1, 8, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != -1;
    return bad;
}
