/* fp64 CPU oracle for the Gated DeltaNet token mixer: TEST INFRASTRUCTURE ONLY.
 * Declarations of gdn_oracle.c; see that file for the passages each function follows. */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

void gdn_oracle_short_conv(const double* x, const double* w, int K, const int* cu, int nseq,
                           int C, double* u);
void gdn_oracle_short_conv_hist(const double* x, const double* w, int K, const int* cu, int nseq,
                                int C, const double* hist_in, double* u, double* hist_out);
void gdn_oracle_silu(const double* u, long n, double* a);
void gdn_oracle_l2norm(const double* a, long rows, int d, double eps, double* out);
void gdn_oracle_gates(const double* a_raw, const double* b_raw, const double* A_log,
                      const double* dt_bias, long ntok, int H, double* g, double* alpha,
                      double* beta);
int gdn_oracle_recurrence(const double* q, const double* k, const double* v, const double* alpha,
                          const double* beta, const double* S0, const int* cu, int nseq, int H,
                          int dk, int dv, int closed_form, double* y, double* ST, int nthreads);
int gdn_oracle_kda_recurrence(const double* q, const double* k, const double* v,
                              const double* alpha, const double* beta, const double* S0,
                              const int* cu, int nseq, int H, int dk, int dv, double* y,
                              double* ST, int nthreads);
int gdn_oracle_recurrence_backward(const double* q, const double* k, const double* v,
                                   const double* alpha, const double* beta, const double* S0,
                                   const int* cu, int nseq, int H, int dk, int dv,
                                   const double* dy, const double* dST, double* dq, double* dk_,
                                   double* dv_, double* dalpha, double* dbeta, double* dS0,
                                   int nthreads);
void gdn_oracle_output_gate(const double* y, const double* z, const double* w, long rows, int dv,
                            double eps, double* o);

#ifdef __cplusplus
}
#endif
#endif
