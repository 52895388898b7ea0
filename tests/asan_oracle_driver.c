/* Host-only driver that runs the C oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every buffer is allocated at exactly its size, so a read or write past any tensor is reported.
 * It covers batched and packed sequences (empty ones included), both reads, reversed scans,
 * accumulation, absent h0/hT, key-head sharing, and the decode step in place and out of place.
 * Built and run by tests/test_oracle_asan.py; prints "asan driver ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdr_oracle_scan(const double *q, const double *k, const double *v, const double *log_alpha,
                    const double *beta, const double *h0, const int64_t *cu_seqlens, int64_t nseq,
                    int64_t B, int64_t T, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, unsigned flags,
                    double *out, double *hT, int nthreads);
int gdr_oracle_decode(const double *q, const double *k, const double *v, const double *log_alpha,
                      const double *beta, const double *state_in, double *state_out, double *out, int64_t N,
                      int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, unsigned flags, int nthreads);

static double *fill(int64_t n, unsigned seed) {
    double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) {
        seed = seed * 1103515245u + 12345u;
        p[i] = ((double)(seed >> 8) / (double)(1u << 24)) - 0.5;
    }
    return p;
}

static int run_scan(int64_t B, int64_t T, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const int64_t *cu,
                    int64_t nseq, unsigned flags, int with_h0, int with_hT) {
    const int64_t S = cu ? nseq : B;
    double *q = fill(B * Hk * T * dk, 1), *k = fill(B * Hk * T * dk, 2), *v = fill(B * Hv * T * dv, 3);
    double *la = fill(B * Hv * T, 4), *be = fill(B * Hv * T, 5);
    for (int64_t i = 0; i < B * Hv * T; ++i) la[i] = -0.1 * (la[i] + 0.5);
    double *h0 = with_h0 ? fill(S * Hv * dk * dv, 6) : NULL;
    double *out = fill(B * Hv * T * dv, 7);
    double *hT = with_hT ? fill(S * Hv * dk * dv, 8) : NULL;
    const int rc = gdr_oracle_scan(q, k, v, la, be, h0, cu, nseq, B, T, Hk, Hv, dk, dv, flags, out, hT, 2);
    free(q); free(k); free(v); free(la); free(be); free(h0); free(out); free(hT);
    return rc;
}

int main(void) {
    int bad = 0;
    for (unsigned flags = 0; flags < 8; ++flags) {
        bad |= run_scan(2, 70, 1, 2, 8, 4, NULL, 0, flags, 1, 1) != 0;
        bad |= run_scan(1, 33, 2, 4, 4, 8, NULL, 0, flags, 0, 1) != 0;
        bad |= run_scan(3, 5, 1, 1, 4, 4, NULL, 0, flags, 1, 0) != 0;
        int64_t cu[6] = {0, 0, 7, 7, 20, 21};
        int64_t *c = (int64_t *)malloc(sizeof cu);
        for (int i = 0; i < 6; ++i) c[i] = cu[i];
        bad |= run_scan(1, 21, 2, 2, 4, 4, c, 5, flags, 1, 1) != 0;
        bad |= run_scan(1, 21, 1, 3, 8, 4, c, 5, flags, 0, 0) != 0;
        free(c);
    }
    bad |= run_scan(2, 0, 1, 1, 4, 4, NULL, 0, 0, 1, 1) != 0;  /* T = 0 */
    /* decode: out of place and in place, both reads, key heads shared by two value heads */
    for (unsigned flags = 0; flags < 2; ++flags) {
        const int64_t N = 3, Hk = 2, Hv = 4, dk = 8, dv = 4;
        double *q = fill(N * Hk * dk, 11), *k = fill(N * Hk * dk, 12), *v = fill(N * Hv * dv, 13);
        double *la = fill(N * Hv, 14), *be = fill(N * Hv, 15);
        double *s = fill(N * Hv * dk * dv, 16), *s2 = fill(N * Hv * dk * dv, 17), *o = fill(N * Hv * dv, 18);
        bad |= gdr_oracle_decode(q, k, v, la, be, s, s2, o, N, Hk, Hv, dk, dv, flags, 2) != 0;
        bad |= gdr_oracle_decode(q, k, v, la, be, s, s, o, N, Hk, Hv, dk, dv, flags, 2) != 0;
        free(q); free(k); free(v); free(la); free(be); free(s); free(s2); free(o);
    }
    /* argument checks return -1 without touching memory */
    bad |= gdr_oracle_scan(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 1, 1, 1, 1, 1, 1, 0, NULL, NULL, 1) != -1;
    if (bad) {
        printf("asan driver: a call returned an unexpected status\n");
        return 1;
    }
    printf("asan driver ok\n");
    return 0;
}
