/* Runs every function of the fp64 oracle on small packed workloads (empty, one-token and
 * ragged sequences, one and several threads) with buffers allocated to their exact sizes.
 * Built with -fsanitize=address,undefined: a read or write past a buffer, a use of freed
 * memory, a signed overflow or a misaligned access ends the run with a report. Prints a
 * checksum of the results so the work cannot be skipped. */
#include <stdio.h>
#include <stdlib.h>

#include "gdn_oracle.h"

static unsigned long long rng = 88172645463325252ull;
static double rnd(void) {   /* xorshift64, uniform in (-1, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / (double)(1ull << 52) - 1.0;
}
static double* arr(long n) {
    double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) p[i] = rnd();
    return p;
}
static double sum(const double* p, long n) {
    double s = 0.0;
    for (long i = 0; i < n; ++i) s += p[i];
    return s;
}

static double run(const int* lens, int nseq, int H, int dk, int dv, int nthreads) {
    int* cu = (int*)malloc(sizeof(int) * (nseq + 1));
    cu[0] = 0;
    for (int s = 0; s < nseq; ++s) cu[s + 1] = cu[s] + lens[s];
    const long ntok = cu[nseq];
    const int K = 4, C = H * (2 * dk + dv);
    double check = 0.0;

    double *x = arr(ntok * C), *w = arr((long)C * K), *u = arr(ntok * C);
    double *hin = arr((long)nseq * (K - 1) * C), *hout = arr((long)nseq * (K - 1) * C);
    gdn_oracle_short_conv(x, w, K, cu, nseq, C, u);
    check += sum(u, ntok * C);
    gdn_oracle_short_conv_hist(x, w, K, cu, nseq, C, hin, u, hout);
    check += sum(u, ntok * C) + sum(hout, (long)nseq * (K - 1) * C);
    gdn_oracle_short_conv_hist(x, w, K, cu, nseq, C, NULL, u, NULL);
    gdn_oracle_silu(u, ntok * C, x);
    gdn_oracle_l2norm(x, ntok * H, dk, 1e-6, u);
    check += sum(u, ntok * H * dk);

    double *a_raw = arr(ntok * H), *b_raw = arr(ntok * H), *A_log = arr(H), *dt = arr(H);
    double *g = arr(ntok * H), *alpha = arr(ntok * H), *beta = arr(ntok * H);
    gdn_oracle_gates(a_raw, b_raw, A_log, dt, ntok, H, g, alpha, beta);
    check += sum(alpha, ntok * H) + sum(beta, ntok * H);

    double *q = arr(ntok * H * dk), *k = arr(ntok * H * dk), *v = arr(ntok * H * dv);
    gdn_oracle_l2norm(q, ntok * H, dk, 1e-6, q);
    gdn_oracle_l2norm(k, ntok * H, dk, 1e-6, k);
    const long ns = (long)nseq * H * dk * dv;
    double *S0 = arr(ns), *ST = arr(ns), *y = arr(ntok * H * dv);
    for (int closed = 0; closed < 2; ++closed) {
        if (gdn_oracle_recurrence(q, k, v, alpha, beta, S0, cu, nseq, H, dk, dv, closed, y, ST,
                                  nthreads) != 0) return 1e300;
        check += sum(y, ntok * H * dv) + sum(ST, ns);
    }
    if (gdn_oracle_recurrence(q, k, v, alpha, beta, NULL, cu, nseq, H, dk, dv, 0, y, ST,
                              nthreads) != 0) return 1e300;
    double* ak = arr(ntok * H * dk);
    for (long i = 0; i < ntok * H * dk; ++i) ak[i] = 0.5 + 0.5 * (ak[i] * ak[i]);
    if (gdn_oracle_kda_recurrence(q, k, v, ak, beta, S0, cu, nseq, H, dk, dv, y, ST, nthreads) != 0)
        return 1e300;
    check += sum(y, ntok * H * dv);

    double *dy = arr(ntok * H * dv), *dST = arr(ns);
    double *dq = arr(ntok * H * dk), *dkk = arr(ntok * H * dk), *dvv = arr(ntok * H * dv);
    double *da = arr(ntok * H), *db = arr(ntok * H), *dS0 = arr(ns);
    if (gdn_oracle_recurrence_backward(q, k, v, alpha, beta, S0, cu, nseq, H, dk, dv, dy, dST, dq,
                                       dkk, dvv, da, db, dS0, nthreads) != 0) return 1e300;
    check += sum(dq, ntok * H * dk) + sum(dS0, ns) + sum(da, ntok * H);
    if (gdn_oracle_recurrence_backward(q, k, v, alpha, beta, NULL, cu, nseq, H, dk, dv, dy, NULL,
                                       dq, dkk, dvv, da, db, NULL, nthreads) != 0) return 1e300;

    double *z = arr(ntok * H * dv), *nw = arr(dv), *o = arr(ntok * H * dv);
    gdn_oracle_output_gate(y, z, nw, ntok * H, dv, 1e-6, o);
    check += sum(o, ntok * H * dv);

    double* bufs[] = {x, w, u, hin, hout, a_raw, b_raw, A_log, dt, g, alpha, beta, q, k, v, S0,
                      ST, y, ak, dy, dST, dq, dkk, dvv, da, db, dS0, z, nw, o};
    for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) free(bufs[i]);
    free(cu);
    return check;
}

int main(void) {
    const int l1[] = {0, 1, 3, 63, 64, 65, 130, 0};
    const int l2[] = {17};
    const int l3[] = {2, 0, 70};
    double c = 0.0;
    c += run(l1, 8, 2, 16, 8, 1);
    c += run(l1, 8, 2, 16, 8, 3);
    c += run(l2, 1, 1, 8, 16, 2);
    c += run(l3, 3, 3, 4, 4, 4);
    if (!(c == c) || c > 1e299) {
        fprintf(stderr, "an oracle call failed\n");
        return 1;
    }
    printf("oracle driver done, checksum %.6e\n", c);
    return 0;
}
