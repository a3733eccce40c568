/* Runs every entry point of oracle/oracle.c on small problems -- dense and
 * block-sparse (with query rows the mask empties), causal or not, GQA, N = 1 and
 * a ragged last block, bad sizes -- for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Outputs must be finite except L = -inf on
 * masked rows. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_fwd(const double *, const double *, const double *, double *, double *, int, int, int, int, int,
               int, const unsigned char *, double);
int oracle_fwd_rows(const double *, const double *, const double *, int, int, int, int, int, int,
                    const unsigned char *, double, int, const int *, const int *, const int *, double *, double *);
int oracle_bwd(const double *, const double *, const double *, const double *, double *, double *, double *,
               double *, int, int, int, int, int, int, const unsigned char *, double);
int oracle_bwd_head(const double *, const double *, const double *, const double *, int, int, int, int, int, int,
                    const unsigned char *, double, int, int, double *, double *, double *, double *, double *);
int oracle_bwd_given(const double *, const double *, const double *, const double *, const double *,
                     const double *, double *, double *, double *, int, int, int, int, int, int,
                     const unsigned char *, double);
int oracle_bwd_given_bf16(const double *, const double *, const double *, const double *, const double *,
                          const double *, double *, double *, double *, int, int, int, int, int, int,
                          const unsigned char *, double);
int oracle_fwd_bf16(const double *, const double *, const double *, double *, double *, int, int, int, int, int,
                    int, const unsigned char *, double);
int oracle_bwd_bf16(const double *, const double *, const double *, const double *, double *, double *, double *,
                    double *, int, int, int, int, int, int, const unsigned char *, double);
int oracle_bwd_bf16_head(const double *, const double *, const double *, const double *, int, int, int, int, int,
                         int, const unsigned char *, double, int, int, double *, double *, double *);

static int failures;

static double *randn(size_t n, unsigned *state) {
    double *x = malloc(n * sizeof *x);
    for (size_t i = 0; i < n; ++i) {
        *state = *state * 1664525u + 1013904223u;
        x[i] = ((double)(*state >> 8) / 16777216.0 - 0.5) * 3.0;
    }
    return x;
}

static void finite(const char *what, const double *x, size_t n, int allow_neg_inf) {
    for (size_t i = 0; i < n; ++i)
        if (!(isfinite(x[i]) || (allow_neg_inf && x[i] == -INFINITY))) {
            fprintf(stderr, "%s[%zu] = %g\n", what, i, x[i]);
            ++failures;
            return;
        }
}

static void run(int B, int Hq, int Hkv, int N, int d, int causal, const unsigned char *bm) {
    unsigned st = (unsigned)(B * 131 + Hq * 17 + N * 7 + d + causal);
    const size_t nq = (size_t)B * Hq * N * d, nk = (size_t)B * Hkv * N * d, nr = (size_t)B * Hq * N;
    double *q = randn(nq, &st), *k = randn(nk, &st), *v = randn(nk, &st), *dO = randn(nq, &st);
    double *o = malloc(nq * sizeof *o), *L = malloc(nr * sizeof *L), *D = malloc(nr * sizeof *D);
    double *dq = malloc(nq * sizeof *dq), *dk = malloc(nk * sizeof *dk), *dv = malloc(nk * sizeof *dv);
    const double scale = 0.4;
    if (oracle_fwd(q, k, v, o, L, B, Hq, Hkv, N, d, causal, bm, scale)) ++failures;
    finite("O", o, nq, 0);
    finite("L", L, nr, 1);
    if (oracle_bwd(q, k, v, dO, dq, dk, dv, D, B, Hq, Hkv, N, d, causal, bm, scale)) ++failures;
    finite("dQ", dq, nq, 0);
    finite("dK", dk, nk, 0);
    finite("dV", dv, nk, 0);
    if (oracle_bwd_given(q, k, v, o, L, dO, dq, dk, dv, B, Hq, Hkv, N, d, causal, bm, scale)) ++failures;
    finite("given dQ", dq, nq, 0);
    if (oracle_bwd_given_bf16(q, k, v, o, L, dO, dq, dk, dv, B, Hq, Hkv, N, d, causal, bm, scale)) ++failures;
    finite("given bf16 dK", dk, nk, 0);
    if (oracle_fwd_bf16(q, k, v, o, L, B, Hq, Hkv, N, d, causal, bm, scale)) ++failures;
    finite("bf16 O", o, nq, 0);
    if (oracle_bwd_bf16(q, k, v, dO, dq, dk, dv, D, B, Hq, Hkv, N, d, causal, bm, scale)) ++failures;
    finite("bf16 dV", dv, nk, 0);
    const int G = Hq / Hkv;
    double *hq = malloc((size_t)G * N * d * sizeof *hq), *hk = malloc((size_t)N * d * sizeof *hk);
    double *hv = malloc((size_t)N * d * sizeof *hv), *hL = malloc((size_t)G * N * sizeof *hL);
    double *hD = malloc((size_t)G * N * sizeof *hD);
    if (oracle_bwd_head(q, k, v, dO, B, Hq, Hkv, N, d, causal, bm, scale, B - 1, Hkv - 1, hq, hk, hv, hL, hD))
        ++failures;
    if (oracle_bwd_bf16_head(q, k, v, dO, B, Hq, Hkv, N, d, causal, bm, scale, 0, 0, hq, hk, hv)) ++failures;
    finite("head dK", hk, (size_t)N * d, 0);
    int rb[2] = {0, B - 1}, rh[2] = {0, Hq - 1}, ri[2] = {0, N - 1};
    double orow[2 * 64], Lrow[2];
    if (d <= 64 && oracle_fwd_rows(q, k, v, B, Hq, Hkv, N, d, causal, bm, scale, 2, rb, rh, ri, orow, Lrow))
        ++failures;
    /* Bad sizes and indices are refused. */
    if (Hkv > 1 && (Hq + 1) % Hkv != 0 && oracle_fwd(q, k, v, o, L, B, Hq + 1, Hkv, N, d, causal, bm, scale) == 0)
        ++failures;   /* Hq not a multiple of Hkv: refused before any access */
    if (oracle_bwd_head(q, k, v, dO, B, Hq, Hkv, N, d, causal, bm, scale, B, 0, hq, hk, hv, hL, hD) == 0) ++failures;
    ri[1] = N;
    if (d <= 64 && oracle_fwd_rows(q, k, v, B, Hq, Hkv, N, d, causal, bm, scale, 2, rb, rh, ri, orow, Lrow) == 0)
        ++failures;
    free(q); free(k); free(v); free(dO); free(o); free(L); free(D); free(dq); free(dk); free(dv);
    free(hq); free(hk); free(hv); free(hL); free(hD);
}

int main(void) {
    /* N = 300: 3 x 3 blocks of 128, the last ragged; query block 1 fully masked. */
    static const unsigned char bm[9] = {1, 0, 1, 0, 0, 0, 1, 1, 1};
    for (int causal = 0; causal < 2; ++causal) {
        run(1, 1, 1, 1, 3, causal, NULL);
        run(2, 4, 2, 33, 16, causal, NULL);
        run(1, 2, 1, 300, 4, causal, bm);
        run(1, 3, 3, 70, 64, causal, NULL);
    }
    if (failures) fprintf(stderr, "%d failure(s)\n", failures);
    else printf("oracle ok\n");
    return failures ? 1 : 0;
}
