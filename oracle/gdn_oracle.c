/*
 * fp64 CPU oracle for the Gated DeltaNet token mixer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header, table or helper with the HIP library.
 *
 * Source: "On the Design of Qwen3.8-Next Architecture" reading notes,
 * section 2.1.1 (Gated DeltaNet):
 *   - "Gated Delta recurrence", eqs. (1)-(4), and the closed form eq. (5);
 *     the state S in R^{dk x dv} is the transpose of the original GDN
 *     convention, q,k in R^dk, v in R^dv, alpha,beta in (0,1);
 *   - "GDN parameterisation", eqs. (6)-(11): ShortConv -> SiLU -> L2Norm,
 *     beta = sigmoid(.), alpha = exp[-exp(A) softplus(. + b_alpha)],
 *     o = W_o[sigmoid(W_z x) * RMSNorm(y)] with a zero-centred RMSNorm;
 *   - section 3.1 (Muon parameter split): decay and beta projections give one
 *     scalar per head.
 * The design-paper summary page ("Token mixing: GDN plus QSA") adds that the
 * short convolution is causal and depthwise.
 *
 * Everything is plain double arithmetic, token by token, in the pages' order.
 * Sums run in index order. No chunking, blocking or re-association.
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math).
 *
 * Readings where the pages are silent (stated once here, used below):
 *   conv width K and tap order: w[c*K + (K-1)] multiplies the current token,
 *     w[c*K + 0] the oldest; inputs before a sequence start are zero; no bias.
 *   L2Norm(x) = x / sqrt(sum x^2 + eps) over the dk channels of one head-token.
 *   RMSNorm(y) = y / sqrt(mean y^2 + eps) over the dv channels of one
 *     head-token; zero-centred gain (1 + w), w shared by all heads.
 *   The output gate multiplies after the norm; W_o is not part of this oracle.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#include "gdn_oracle.h"

/* ------------------------------------------------------------------ eqs. 6-8 */

/* ShortConv: depthwise causal cross-correlation, zero history at each sequence start.
 * x, u: [ntok, C]; w: [C, K]; cu: [nseq+1] packed sequence offsets. */
void gdn_oracle_short_conv(const double* x, const double* w, int K, const int* cu, int nseq,
                           int C, double* u) {
    for (int s = 0; s < nseq; ++s) {
        for (int t = cu[s]; t < cu[s + 1]; ++t) {
            for (int c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) {
                    int src = t - (K - 1) + j;
                    if (src >= cu[s]) acc += w[(long)c * K + j] * x[(long)src * C + c];
                }
                u[(long)t * C + c] = acc;
            }
        }
    }
}

/* ShortConv with a carried history: the streaming form of the conv above, for a sequence
 * that continues one processed earlier (chunked prefill, decode). The K-1 inputs before the
 * start of sequence s are hist_in[s] ([nseq, K-1, C], row j = the input K-1-j positions
 * before the start, so row K-2 is the newest); hist_in NULL means zero history, which is the
 * conv above. hist_out[s] (nullable) receives the last K-1 inputs of the history followed by
 * the sequence, in the same row order: for a sequence shorter than K-1 its older rows come
 * from hist_in. */
static double conv_input(const double* x, const double* hist_in, const int* cu, int s, int K,
                         int C, long p, int c) {
    if (p >= cu[s]) return x[p * C + c];
    if (!hist_in) return 0.0;
    long j = (K - 1) - (cu[s] - p); /* cu[s] - p in 1..K-1 */
    return hist_in[((long)s * (K - 1) + j) * C + c];
}

void gdn_oracle_short_conv_hist(const double* x, const double* w, int K, const int* cu, int nseq,
                                int C, const double* hist_in, double* u, double* hist_out) {
    for (int s = 0; s < nseq; ++s) {
        for (int t = cu[s]; t < cu[s + 1]; ++t) {
            for (int c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j)
                    acc += w[(long)c * K + j] * conv_input(x, hist_in, cu, s, K, C, t - (K - 1) + j, c);
                u[(long)t * C + c] = acc;
            }
        }
        if (hist_out)
            for (int j = 0; j < K - 1; ++j)
                for (int c = 0; c < C; ++c)
                    hist_out[((long)s * (K - 1) + j) * C + c] =
                        conv_input(x, hist_in, cu, s, K, C, (long)cu[s + 1] - (K - 1) + j, c);
    }
}

/* SiLU(u) = u * sigmoid(u) = u / (1 + exp(-u)) */
void gdn_oracle_silu(const double* u, long n, double* a) {
    for (long i = 0; i < n; ++i) a[i] = u[i] / (1.0 + exp(-u[i]));
}

/* L2Norm over the last axis of [rows, d] */
void gdn_oracle_l2norm(const double* a, long rows, int d, double eps, double* out) {
    for (long r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int c = 0; c < d; ++c) ss += a[r * d + c] * a[r * d + c];
        double inv = 1.0 / sqrt(ss + eps);
        for (int c = 0; c < d; ++c) out[r * d + c] = a[r * d + c] * inv;
    }
}

/* ------------------------------------------------------------------ eqs. 9-10 */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), written so that it neither overflows nor cancels */
static double softplus(double x) { return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/* beta = sigmoid(b_raw); alpha = exp(-exp(A_h) * softplus(a_raw + b_alpha_h)); g = log alpha.
 * a_raw, b_raw, g, alpha, beta: [ntok, H]; A_log, dt_bias: [H] */
void gdn_oracle_gates(const double* a_raw, const double* b_raw, const double* A_log,
                      const double* dt_bias, long ntok, int H, double* g, double* alpha,
                      double* beta) {
    for (long t = 0; t < ntok; ++t) {
        for (int h = 0; h < H; ++h) {
            long i = t * H + h;
            double gi = -exp(A_log[h]) * softplus(a_raw[i] + dt_bias[h]);
            if (g) g[i] = gi;
            if (alpha) alpha[i] = exp(gi);
            if (beta) beta[i] = sigmoid(b_raw[i]);
        }
    }
}

/* ------------------------------------------------------------------ eqs. 1-5 */

typedef struct {
    const double *q, *k, *v, *alpha, *beta, *S0;
    const int* cu;
    int nseq, H, dk, dv;
    int closed_form; /* 0: eqs. 1-4 as written; 1: eq. 5 then eq. 4 */
    double *y, *ST;
    int next; /* work counter over (seq, head) pairs */
    pthread_mutex_t mu;
} rec_job;

static void run_pair(rec_job* J, int s, int h, double* S, double* tmp) {
    const int H = J->H, dk = J->dk, dv = J->dv;
    const long sz = (long)dk * dv;
    if (J->S0)
        memcpy(S, J->S0 + ((long)s * H + h) * sz, sizeof(double) * sz);
    else
        memset(S, 0, sizeof(double) * sz);
    for (int t = J->cu[s]; t < J->cu[s + 1]; ++t) {
        const long row = (long)t * H + h;
        const double* q = J->q + row * dk;
        const double* k = J->k + row * dk;
        const double* v = J->v + row * dv;
        const double a = J->alpha[row], b = J->beta[row];
        if (!J->closed_form) {
            /* eq. 1: S~ = alpha S */
            for (long i = 0; i < sz; ++i) S[i] = a * S[i];
            /* eq. 2: e = v - S~^T k */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * k[i];
                tmp[j] = v[j] - acc;
            }
            /* eq. 3: S = S~ + beta k e^T */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += b * k[i] * tmp[j];
        } else {
            /* eq. 5: S = alpha (I - beta k k^T) S + beta k v^T, with (k^T S) formed first */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += k[i] * S[(long)i * dv + j];
                tmp[j] = acc;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[(long)i * dv + j] =
                        a * (S[(long)i * dv + j] - b * k[i] * tmp[j]) + b * k[i] * v[j];
        }
        /* eq. 4: y = S^T q */
        double* y = J->y + row * dv;
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * q[i];
            y[j] = acc;
        }
    }
    if (J->ST) memcpy(J->ST + ((long)s * H + h) * sz, S, sizeof(double) * sz);
}

static void* rec_worker(void* arg) {
    rec_job* J = (rec_job*)arg;
    double* S = (double*)malloc(sizeof(double) * (size_t)J->dk * J->dv);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)J->dv);
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int p = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (p >= J->nseq * J->H) break;
        run_pair(J, p / J->H, p % J->H, S, tmp);
    }
    free(S);
    free(tmp);
    return NULL;
}

/* Gated delta rule over packed sequences.
 * q,k: [ntok,H,dk]; v,y: [ntok,H,dv]; alpha,beta: [ntok,H];
 * S0 (nullable => zero), ST (nullable): [nseq,H,dk,dv]; cu: [nseq+1].
 * closed_form selects eq. 5 instead of eqs. 1-3. Returns 0 on success. */
int gdn_oracle_recurrence(const double* q, const double* k, const double* v, const double* alpha,
                          const double* beta, const double* S0, const int* cu, int nseq, int H,
                          int dk, int dv, int closed_form, double* y, double* ST, int nthreads) {
    rec_job J;
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.S0 = S0; J.cu = cu;
    J.nseq = nseq; J.H = H; J.dk = dk; J.dv = dv; J.closed_form = closed_form;
    J.y = y; J.ST = ST; J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    int pairs = nseq * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pairs) nthreads = pairs > 0 ? pairs : 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, rec_worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* ------------------------------------------------------------------ per-channel decay */

/* The delta rule with a per-channel (diagonal) decay, as in Kimi Delta Attention, to which the
 * reading notes compare GDN (related work on Kimi K3: a KDA layer whose log-decay has a lower
 * bound). Reading: the scalar alpha of eq. 1 becomes a diagonal over the key channels,
 *   S~ = Diag(alpha_t) S_{t-1};  e = v_t - S~^T k_t;  S_t = S~ + beta_t k_t e^T;  y_t = S_t^T q_t
 * i.e. eqs. 1-4 with row i of the state decayed by alpha_t[i]. alpha: [ntok, H, dk].
 * Other arguments as gdn_oracle_recurrence. */
typedef struct {
    const double *q, *k, *v, *alpha, *beta, *S0;
    const int* cu;
    int nseq, H, dk, dv;
    double *y, *ST;
    int next;
    pthread_mutex_t mu;
} kda_job;

static void kda_pair(kda_job* J, int s, int h, double* S, double* e) {
    const int H = J->H, dk = J->dk, dv = J->dv;
    const long sz = (long)dk * dv;
    if (J->S0) memcpy(S, J->S0 + ((long)s * H + h) * sz, sizeof(double) * sz);
    else memset(S, 0, sizeof(double) * sz);
    for (int t = J->cu[s]; t < J->cu[s + 1]; ++t) {
        const long row = (long)t * H + h;
        const double* q = J->q + row * dk;
        const double* k = J->k + row * dk;
        const double* v = J->v + row * dv;
        const double* al = J->alpha + row * dk;
        const double b = J->beta[row];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(long)i * dv + j] *= al[i];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * k[i];
            e[j] = v[j] - acc;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += b * k[i] * e[j];
        double* y = J->y + row * dv;
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * q[i];
            y[j] = acc;
        }
    }
    if (J->ST) memcpy(J->ST + ((long)s * H + h) * sz, S, sizeof(double) * sz);
}

static void* kda_worker(void* arg) {
    kda_job* J = (kda_job*)arg;
    double* S = (double*)malloc(sizeof(double) * (size_t)J->dk * J->dv);
    double* e = (double*)malloc(sizeof(double) * (size_t)J->dv);
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int p = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (p >= J->nseq * J->H) break;
        kda_pair(J, p / J->H, p % J->H, S, e);
    }
    free(S);
    free(e);
    return NULL;
}

int gdn_oracle_kda_recurrence(const double* q, const double* k, const double* v,
                              const double* alpha, const double* beta, const double* S0,
                              const int* cu, int nseq, int H, int dk, int dv, double* y,
                              double* ST, int nthreads) {
    kda_job J;
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.S0 = S0; J.cu = cu;
    J.nseq = nseq; J.H = H; J.dk = dk; J.dv = dv; J.y = y; J.ST = ST; J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    int pairs = nseq * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pairs) nthreads = pairs > 0 ? pairs : 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, kda_worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* ------------------------------------------------------------------ gradients of eqs. 1-4 */

/* Reverse-mode derivative of the recurrence above (eqs. 1-4 as written), token by token in
 * reverse order: given dL/dy for every token and dL/dS_T, it returns dL/d(q, k, v, alpha,
 * beta, S0). Each token's step is undone in the opposite order of its forward operations:
 *   y = S^T q             -> dq = S dy,  dS += q dy^T
 *   S = S~ + beta k e^T   -> dbeta = k^T dS e,  dk += beta dS e,  de = beta dS^T k,  dS~ = dS
 *   e = v - S~^T k        -> dv = de,  dS~ -= k de^T,  dk -= S~ de
 *   S~ = alpha S_prev     -> dalpha = <dS~, S_prev>,  dS_prev = alpha dS~
 * The state before each token is recomputed from checkpoints taken every CK tokens of the
 * forward pass (the forward is the plain recurrence of eqs. 1-4). */
#define CK 64

typedef struct {
    const double *q, *k, *v, *alpha, *beta, *S0, *dy, *dST;
    const int* cu;
    int nseq, H, dk, dv;
    double *dq, *dk_, *dv_, *dalpha, *dbeta, *dS0;
    int next;
    pthread_mutex_t mu;
} bwd_job;

/* S <- state after token `row` from the state before it (eqs. 1-3); e receives the residual */
static void fwd_token(const bwd_job* J, long row, double* S, double* e) {
    const int dk = J->dk, dv = J->dv;
    const double* k = J->k + row * dk;
    const double* v = J->v + row * dv;
    const double a = J->alpha[row], b = J->beta[row];
    for (long i = 0; i < (long)dk * dv; ++i) S[i] = a * S[i];
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * k[i];
        e[j] = v[j] - acc;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += b * k[i] * e[j];
}

static void bwd_pair(bwd_job* J, int s, int h, double* ckpt, double* prev, double* S, double* dS,
                     double* e, double* de) {
    const int H = J->H, dk = J->dk, dv = J->dv;
    const long sz = (long)dk * dv;
    const int t0 = J->cu[s], t1 = J->cu[s + 1];
    const int nck = (t1 - t0 + CK - 1) / CK;
    /* forward: checkpoints of the state before each CK-token block */
    if (J->S0) memcpy(S, J->S0 + ((long)s * H + h) * sz, sizeof(double) * sz);
    else memset(S, 0, sizeof(double) * sz);
    for (int c = 0; c < nck; ++c) {
        memcpy(ckpt + (long)c * sz, S, sizeof(double) * sz);
        for (int t = t0 + c * CK; t < t0 + (c + 1) * CK && t < t1; ++t)
            fwd_token(J, (long)t * H + h, S, e);
    }
    /* reverse */
    if (J->dST) memcpy(dS, J->dST + ((long)s * H + h) * sz, sizeof(double) * sz);
    else memset(dS, 0, sizeof(double) * sz);
    for (int c = nck - 1; c >= 0; --c) {
        const int ta = t0 + c * CK, tb = (ta + CK < t1) ? ta + CK : t1;
        /* states before each token of the block */
        memcpy(S, ckpt + (long)c * sz, sizeof(double) * sz);
        for (int t = ta; t < tb; ++t) {
            memcpy(prev + (long)(t - ta) * sz, S, sizeof(double) * sz);
            fwd_token(J, (long)t * H + h, S, e);
        }
        for (int t = tb - 1; t >= ta; --t) {
            const long row = (long)t * H + h;
            const double* Sp = prev + (long)(t - ta) * sz;   /* S_{t-1} */
            const double* q = J->q + row * dk;
            const double* k = J->k + row * dk;
            const double* v = J->v + row * dv;
            const double* dy = J->dy + row * dv;
            const double a = J->alpha[row], b = J->beta[row];
            double* dq = J->dq + row * dk;
            double* dkk = J->dk_ + row * dk;
            double* dvv = J->dv_ + row * dv;
            /* recompute S~ = a S_prev (into S), e, and S_t (into S after the write) */
            for (long i = 0; i < sz; ++i) S[i] = a * Sp[i];
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * k[i];
                e[j] = v[j] - acc;
            }
            /* y = S_t^T q with S_t = S~ + b k e^T */
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j)
                    acc += (S[(long)i * dv + j] + b * k[i] * e[j]) * dy[j];
                dq[i] = acc;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) dS[(long)i * dv + j] += q[i] * dy[j];
            /* S_t = S~ + b k e^T */
            double db = 0.0;
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += dS[(long)i * dv + j] * e[j];
                db += k[i] * acc;
                dkk[i] = b * acc;
            }
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += dS[(long)i * dv + j] * k[i];
                de[j] = b * acc;
            }
            /* e = v - S~^T k */
            for (int j = 0; j < dv; ++j) dvv[j] = de[j];
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += S[(long)i * dv + j] * de[j];
                dkk[i] -= acc;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) dS[(long)i * dv + j] -= k[i] * de[j];
            /* S~ = a S_prev */
            double da = 0.0;
            for (long i = 0; i < sz; ++i) da += dS[i] * Sp[i];
            for (long i = 0; i < sz; ++i) dS[i] *= a;
            J->dalpha[row] = da;
            J->dbeta[row] = db;
        }
    }
    if (J->dS0) memcpy(J->dS0 + ((long)s * H + h) * sz, dS, sizeof(double) * sz);
}

static void* bwd_worker(void* arg) {
    bwd_job* J = (bwd_job*)arg;
    const long sz = (long)J->dk * J->dv;
    double* ckpt = NULL;
    int maxck = 1;
    for (int s = 0; s < J->nseq; ++s) {
        int n = (J->cu[s + 1] - J->cu[s] + CK - 1) / CK;
        if (n > maxck) maxck = n;
    }
    ckpt = (double*)malloc(sizeof(double) * (size_t)(sz * maxck));
    double* prev = (double*)malloc(sizeof(double) * (size_t)(sz * CK));
    double* S = (double*)malloc(sizeof(double) * (size_t)sz);
    double* dS = (double*)malloc(sizeof(double) * (size_t)sz);
    double* e = (double*)malloc(sizeof(double) * (size_t)J->dv);
    double* de = (double*)malloc(sizeof(double) * (size_t)J->dv);
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int p = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (p >= J->nseq * J->H) break;
        bwd_pair(J, p / J->H, p % J->H, ckpt, prev, S, dS, e, de);
    }
    free(ckpt); free(prev); free(S); free(dS); free(e); free(de);
    return NULL;
}

/* Gradients of eqs. 1-4 over packed sequences. Inputs as gdn_oracle_recurrence plus
 * dy [ntok,H,dv] and dST [nseq,H,dk,dv] (nullable => zero). Outputs dq, dk [ntok,H,dk],
 * dv [ntok,H,dv], dalpha, dbeta [ntok,H], dS0 [nseq,H,dk,dv] (nullable). Returns 0. */
int gdn_oracle_recurrence_backward(const double* q, const double* k, const double* v,
                                   const double* alpha, const double* beta, const double* S0,
                                   const int* cu, int nseq, int H, int dk, int dv,
                                   const double* dy, const double* dST, double* dq, double* dk_,
                                   double* dv_, double* dalpha, double* dbeta, double* dS0,
                                   int nthreads) {
    bwd_job J;
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.S0 = S0; J.dy = dy; J.dST = dST;
    J.cu = cu; J.nseq = nseq; J.H = H; J.dk = dk; J.dv = dv;
    J.dq = dq; J.dk_ = dk_; J.dv_ = dv_; J.dalpha = dalpha; J.dbeta = dbeta; J.dS0 = dS0;
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    int pairs = nseq * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pairs) nthreads = pairs > 0 ? pairs : 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, bwd_worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* ------------------------------------------------------------------ eq. 11 (without W_o) */

/* o = sigmoid(z) * RMSNorm(y) with zero-centred gain: RMSNorm(y) = (1 + w) * y / sqrt(mean y^2 + eps).
 * y, z, o: [rows, dv]; w: [dv] */
void gdn_oracle_output_gate(const double* y, const double* z, const double* w, long rows, int dv,
                            double eps, double* o) {
    for (long r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int j = 0; j < dv; ++j) ss += y[r * dv + j] * y[r * dv + j];
        double inv = 1.0 / sqrt(ss / dv + eps);
        for (int j = 0; j < dv; ++j)
            o[r * dv + j] = sigmoid(z[r * dv + j]) * ((1.0 + w[j]) * (y[r * dv + j] * inv));
    }
}
