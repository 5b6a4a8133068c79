/*
 * gdn.h - C ABI of the MI355X (gfx950) Gated DeltaNet token-mixer library (libgdn.so).
 *
 * The operations are those of the Gated DeltaNet layer in the reading notes of
 * "On the Design of Qwen3.8-Next Architecture" (arXiv 2608.30320), section 2.1.1:
 *   eqs. (1)-(4) the gated delta rule, eq. (5) its closed form,
 *   eqs. (6)-(8) q,k = L2Norm(SiLU(ShortConv(.))), v = SiLU(ShortConv(.)),
 *   eqs. (9)-(10) beta = sigmoid(.), alpha = exp[-exp(A) softplus(. + b_alpha)],
 *   eq. (11) o = W_o[sigmoid(W_z x) * RMSNorm(y)] with a zero-centred RMSNorm.
 * Per head: q, k in R^dk, v in R^dv, state S in R^{dk x dv} (rows over dk, columns
 * over dv: the transpose of the original GDN convention), y = S^T q. The decay and
 * write-strength gates are one scalar per (token, head) (section 3.1 of the same notes).
 * The projections W_q, W_k, W_v, W_alpha, W_beta, W_z, W_o are dense GEMMs of the
 * surrounding model and are not part of this library: its inputs are the projected
 * streams.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the library never
 *     allocates, frees or retains device memory and keeps no mutable global state, with
 *     one exception: gdn_chunk_prefill_noalloc uses a scratch array of the library's own
 *     (below).
 *   - Layouts are dense, row-major and token-major over packed sequences:
 *       q, k [ntok, H, dk]; v, y, z, o [ntok, H, dv]; g, beta, a_raw, b_raw [ntok, H];
 *       states [num_seqs, H, dk, dv] (fp32); per-head vectors [H]; norm weight [dv].
 *   - bf16 tensors hold IEEE bfloat16 bit patterns (round-to-nearest-even on output).
 *   - Pointers to vector data (x*, q, k, v, y, z, o, conv taps, states, workspace) must be
 *     16-byte aligned; scalar arrays (g, beta, a_raw, b_raw, A_log, dt_bias, norm weight,
 *     cu_seqlens) 4-byte aligned. dk, dv in {64, 128}. H >= 1.
 *   - Every array a call touches has at most 2^31 - 1 elements: ntok * H * max(dk, dv) for
 *     token arrays (N * T * H * max(dk, dv) in decode), num_seqs * H * dk * dv for states,
 *     num_seqs * 3 * H * (2 dk + dv) for conv histories. Larger calls return GDN_ERR_SHAPE.
 *   - Arrays indexed by token (or, in decode, by sequence: the decode states and conv
 *     histories included) may be NULL when that count (ntok, or N) is 0: nothing reads or
 *     writes them then. Per-head and per-channel arrays (conv taps, A_log, dt_bias, norm
 *     weight) and the workspace stay required.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call is
 *     asynchronous on it: it validates its arguments on the host, enqueues its kernels
 *     and returns. Device faults surface when the caller synchronises.
 *   - On invalid arguments a call returns a non-zero gdn_status, enqueues nothing and
 *     records a message readable with gdn_last_error() on the calling thread. A failed
 *     launch returns GDN_ERR_HIP with the HIP error text. No C++ exception crosses the ABI.
 *   - Calls are re-entrant and thread-safe; calls on one stream execute in order.
 *   - NaN/Inf inputs are not checked; they propagate into their own (token, head)
 *     slice (and, for the recurrence, into that sequence-head's later outputs and state).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 6

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,      /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,     /* unsupported or inconsistent sizes */
    GDN_ERR_DTYPE = 3,     /* unsupported dtype tag */
    GDN_ERR_SEQLENS = 4,   /* cu_seqlens (host mirror) is not 0 = c0 <= c1 <= ... = ntok */
    GDN_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned */
    GDN_ERR_WORKSPACE = 6, /* workspace missing or smaller than required */
    GDN_ERR_HIP = 7        /* a HIP runtime call failed */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

/* Static text naming a status code. */
const char* gdn_status_string(int status);

/* Message of the last failed call on the calling thread ("" if none). Valid until the
 * next call from the same thread. */
const char* gdn_last_error(void);

/*
 * gdn_preprocess - eqs. (6)-(10): ShortConv -> SiLU -> L2Norm for q and k,
 * ShortConv -> SiLU for v, and the per-head scalar gates.
 *
 *   xq, xk: [ntok, H, dk], xv: [ntok, H, dv] in x_dtype - the projected streams W x.
 *   wq, wk: [H*dk, conv_k], wv: [H*dv, conv_k] fp32 - depthwise causal conv taps; tap
 *       conv_k-1 multiplies the current token, tap 0 the oldest. No bias. Inputs before
 *       each sequence start count as zero (the conv restarts at every sequence).
 *   conv_k must be 4.
 *   a_raw, b_raw: [ntok, H] fp32 - W_alpha x and W_beta x.
 *   A_log, dt_bias: [H] fp32 - A and b_alpha of eq. (10).
 *   cu_seqlens: [num_seqs+1] int32 device offsets, or NULL for num_seqs equal-length
 *       sequences (ntok must then be a multiple of num_seqs).
 *   l2_eps: L2Norm(x) = x / sqrt(sum(x^2) + l2_eps) over the dk channels of one head-token.
 *   q, k, v: outputs in out_dtype, same layouts as xq, xk, xv.
 *   g: [ntok, H] fp32 output, g = log(alpha) = -exp(A_log) * softplus(a_raw + dt_bias).
 *   beta: [ntok, H] fp32 output, beta = sigmoid(b_raw).
 * Gates-only mode: pass xq, xk, xv, wq, wk, wv, q, k, v all NULL; then only g and beta
 * are computed. Passing g, beta, a_raw, b_raw, A_log, dt_bias all NULL skips the gates.
 */
int gdn_preprocess(const void* xq, const void* xk, const void* xv, int x_dtype,
                   const float* wq, const float* wk, const float* wv, int conv_k,
                   const float* a_raw, const float* b_raw, const float* A_log,
                   const float* dt_bias, const int32_t* cu_seqlens, int num_seqs, int ntok,
                   int H, int dk, int dv, float l2_eps, void* q, void* k, void* v,
                   int out_dtype, float* g, float* beta, void* stream);

/*
 * gdn_preprocess_stateful - gdn_preprocess for sequences that continue earlier input
 * (a prompt prefilled in pieces, or decode steps of one or more tokens per sequence).
 * eqs. (6)-(8) apply a causal conv along the whole stream (section 2.1.1 of the notes above;
 * the design-paper summary "设计 LLM 架构", section "Token 混合：GDN 加 QSA", calls the short
 * conv causal and depthwise), so each sequence carries the last conv_k-1 inputs it has seen.
 *
 *   Arguments as gdn_preprocess (the conv inputs and outputs are required), plus:
 *   conv_state_in: [num_seqs, conv_k-1, H*(2*dk+dv)] in x_dtype, or NULL for zero history.
 *       Row j of sequence s holds the input conv_k-1-j positions before its first token
 *       (the last row is the newest); channels are ordered q | k | v, each [H, d] as in
 *       xq, xk, xv.
 *   conv_state_out: same layout, or NULL. Receives, per sequence, the last conv_k-1 inputs
 *       of its history followed by its tokens: the next call's conv_state_in. A sequence
 *       shorter than conv_k-1 (even an empty one) shifts its history by its length.
 *   The two states must not overlap (double-buffer them; GDN_ERR_SHAPE otherwise).
 *   With both NULL the call is gdn_preprocess. Values are copied bit for bit.
 */
int gdn_preprocess_stateful(const void* xq, const void* xk, const void* xv, int x_dtype,
                            const float* wq, const float* wk, const float* wv, int conv_k,
                            const float* a_raw, const float* b_raw, const float* A_log,
                            const float* dt_bias, const int32_t* cu_seqlens, int num_seqs,
                            int ntok, int H, int dk, int dv, float l2_eps, void* q, void* k,
                            void* v, int out_dtype, float* g, float* beta,
                            const void* conv_state_in, void* conv_state_out, void* stream);

/* Bytes of device workspace gdn_chunk_prefill needs for these sizes (may be 0). */
size_t gdn_chunk_prefill_workspace_size(int ntok, int num_seqs, int H, int dk, int dv,
                                        int in_dtype);

/*
 * gdn_chunk_prefill - eqs. (1)-(4) over packed sequences, evaluated chunkwise with
 * C = 64 tokens per chunk (an exact re-association of eq. (5)'s product; chunks restart
 * at every sequence start).
 *
 *   q, k: [ntok, H, dk], v: [ntok, H, dv] in in_dtype (q, k are expected L2-normalised).
 *   g: [ntok, H] fp32 log-decay (alpha = exp(g), g <= 0); beta: [ntok, H] fp32.
 *   initial_state: [num_seqs, H, dk, dv] fp32, or NULL for zero states.
 *   final_state: [num_seqs, H, dk, dv] fp32 output, or NULL (not written). It may be the
 *       same pointer as initial_state (updated in place); otherwise it must not overlap
 *       any input.
 *   cu_seqlens: [num_seqs+1] int32 device offsets, or NULL for equal lengths.
 *   cu_seqlens_host: optional host copy of cu_seqlens; when given it is validated.
 *   y: [ntok, H, dv] output in y_dtype, y_t = S_t^T q_t.
 *   workspace: device scratch of at least gdn_chunk_prefill_workspace_size(...) bytes
 *       (may be NULL when that size is 0); it must not be shared by concurrent calls.
 * in_dtype GDN_F32 runs an all-fp32 chunked path; GDN_BF16 runs bf16 matrix-core
 * products with fp32 accumulation and an fp32 state.
 */
int gdn_chunk_prefill(const void* q, const void* k, const void* v, int in_dtype,
                      const float* g, const float* beta, const float* initial_state,
                      float* final_state, const int32_t* cu_seqlens,
                      const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H, int dk,
                      int dv, void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Size of the library's scratch array behind gdn_chunk_prefill_noalloc (one per GPU). */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * gdn_chunk_prefill_noalloc - gdn_chunk_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It takes the same arguments minus the workspace and computes the same result
 * (the same kernels); in place of the workspace it uses a scratch array of
 * GDN_NOALLOC_SCRATCH_BYTES compiled into the library, one per GPU, which that GPU holds from
 * the first call on it until the process ends. It calls no hipMalloc, hipFree or other
 * allocating routine (the first call on a device only looks the array's address up).
 *   - Sizes whose workspace (gdn_chunk_prefill_workspace_size) exceeds
 *     GDN_NOALLOC_SCRATCH_BYTES return GDN_ERR_WORKSPACE before anything is enqueued
 *     (B = 4, H = 16, T = 4096 needs about 71 MB and fits; H = 32, T = 65536 does not).
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents
 *     (nothing in it needs to start at zero). Calls that overlap in time on one GPU (on
 *     different streams, or from different threads) therefore race and give undefined
 *     results: order them, e.g. on one stream.
 */
int gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v, int in_dtype,
                              const float* g, const float* beta, const float* initial_state,
                              float* final_state, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H,
                              int dk, int dv, void* y, int y_dtype, void* stream);

/* Bytes of device workspace gdn_chunk_backward needs for these sizes. */
size_t gdn_chunk_backward_workspace_size(int ntok, int num_seqs, int H, int dk, int dv);

/*
 * gdn_chunk_backward - gradients of gdn_chunk_prefill for training: given dL/dy and
 * dL/dS_T, the gradients with respect to q, k, v, g (= log alpha), beta and S0 of
 * eqs. (1)-(4) (section 2.1.1; the reading notes' "Kernel 效率" cites backward speedups
 * for chunked GDN kernels, and their section 3.1 trains the decay and beta projections
 * with AdamW). Computed chunkwise (C = 64): a forward sweep stores the state at every chunk
 * start in the workspace, a reverse sweep carries dS back through the chunks and stores it
 * per chunk, and a per-chunk pass forms the gradients.
 *   - in_dtype and dy_dtype GDN_BF16 with dk = dv = 128: products on the bf16 matrix cores
 *     with fp32 accumulation, fp32 operands entering as hi + lo bf16 pairs where the
 *     gradients need them (relative L2 error per (sequence, head) about 1e-3);
 *   - any other combination: fp32 throughout (about 1e-6).
 *
 *   q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, num_seqs, ntok, H, dk, dv:
 *       as gdn_chunk_prefill (the forward's inputs; q, k, v in in_dtype).
 *   dy: [ntok, H, dv] in dy_dtype - dL/dy.
 *   dfinal_state: [num_seqs, H, dk, dv] fp32 dL/dS_T, or NULL (zero).
 *   dq, dk_out: [ntok, H, dk]; dv_out: [ntok, H, dv]; dg, dbeta: [ntok, H]: fp32 outputs.
 *   dinitial_state: [num_seqs, H, dk, dv] fp32 dL/dS0, or NULL (not written).
 *   workspace: at least gdn_chunk_backward_workspace_size(...) bytes of device scratch.
 *   Results are deterministic (no atomics). All outputs are overwritten.
 */
int gdn_chunk_backward(const void* q, const void* k, const void* v, int in_dtype, const float* g,
                       const float* beta, const float* initial_state, const void* dy,
                       int dy_dtype, const float* dfinal_state, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H, int dk,
                       int dv, float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                       float* dinitial_state, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Bytes of device workspace gdn_kda_chunk_prefill needs for these sizes. */
size_t gdn_kda_chunk_prefill_workspace_size(int ntok, int num_seqs, int H, int dk);

/*
 * gdn_kda_chunk_prefill - the delta rule with a per-channel (diagonal) decay, the variant the
 * reading notes compare GDN with (related work on Kimi K3: Kimi Delta Attention, whose
 * log-decay is lower-bounded). eq. (1)'s scalar alpha_t becomes Diag(alpha_t) over the key
 * channels: row c of the state decays by alpha_t[c] = exp(g[t][h][c]); eqs. (2)-(4) are
 * unchanged. Chunkwise (C = 64) in fp32.
 *
 *   Arguments as gdn_chunk_prefill except g: [ntok, H, dk] fp32 per-channel log-decays
 *   (any g <= 0; the kernels form only exponentials of non-positive differences).
 *   workspace: at least gdn_kda_chunk_prefill_workspace_size(...) bytes.
 */
int gdn_kda_chunk_prefill(const void* q, const void* k, const void* v, int in_dtype,
                          const float* g, const float* beta, const float* initial_state,
                          float* final_state, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H, int dk,
                          int dv, void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Bytes of device workspace gdn_kda_chunk_prefill_bounded needs for these sizes. */
size_t gdn_kda_chunk_prefill_bounded_workspace_size(int ntok, int num_seqs, int H);

/*
 * gdn_kda_chunk_prefill_bounded - the per-channel-decay prefill of gdn_kda_chunk_prefill for
 * log-decays bounded below by -5 (the lower bound of the Kimi Delta Attention gate named
 * in the reading notes' related-work comparison, section "与已归档相关工作的对比"), on the
 * bf16 matrix cores: within 16 tokens the decay spans at most e^80, so the per-channel
 * decays fold into bf16 operands of dense products. fp32 accumulation and an fp32 state.
 *
 *   Arguments as gdn_kda_chunk_prefill, with in_dtype GDN_BF16, dk = dv = 128, and
 *   g: [ntok, H, 128] fp32 log-decays with -5 <= g <= 0, 16-byte aligned. Entries below -5
 *   are outside this path (a 16-token block could then overflow the scaled operands): use
 *   gdn_kda_chunk_prefill for them.
 *   workspace: at least gdn_kda_chunk_prefill_bounded_workspace_size(...) bytes.
 */
int gdn_kda_chunk_prefill_bounded(const void* q, const void* k, const void* v, int in_dtype,
                                  const float* g, const float* beta, const float* initial_state,
                                  float* final_state, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H,
                                  int dk, int dv, void* y, int y_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * gdn_decode_step - one token per sequence through eqs. (1)-(4), state updated in place:
 * S <- alpha S; e = v - S^T k; S <- S + beta k e^T; y = S^T q.
 *
 *   q, k: [N, H, dk], v: [N, H, dv] in in_dtype; g, beta: [N, H] fp32 (alpha = exp(g)).
 *   state: [N, H, dk, dv] fp32, read and overwritten.
 *   y: [N, H, dv] output in y_dtype.
 */
int gdn_decode_step(const void* q, const void* k, const void* v, int in_dtype, const float* g,
                    const float* beta, float* state, int N, int H, int dk, int dv, void* y,
                    int y_dtype, void* stream);

/*
 * gdn_decode_multi - T consecutive tokens per sequence through eqs. (1)-(4), state updated in
 * place: the decode step of multi-token prediction, where one real token and T-1 drafts are
 * verified together. The design-paper summary "设计 LLM 架构" (section "高层设计", output
 * head and MTP) has the MTP module draft tokens for speculative decoding; the reading notes'
 * efficiency analysis (Figure 6) times decode with three extra MTP steps (next_n = 4). The
 * T tokens form one micro-chunk of the chunkwise form of eq. (5), so each state is read
 * once and written once.
 *
 *   q, k: [N, T, H, dk], v: [N, T, H, dv] in in_dtype (token-major: the T tokens of
 *       sequence n are rows n*T .. n*T+T-1 of a packed [N*T, H, d] tensor).
 *   g, beta: [N, T, H] fp32 (alpha = exp(g)).
 *   state: [N, H, dk, dv] fp32, read and overwritten with the state after token T-1.
 *   y: [N, T, H, dv] output in y_dtype; y[n][t] is the output of token t.
 *   step_states: NULL, or [N, T, H, dk, dv] fp32 receiving the state after each token
 *       (step_states[n][T-1] equals the new state), so a caller that accepts only the
 *       first a tokens of a draft restores sequence n from step_states[n][a-1]. Must not
 *       overlap state.
 *   1 <= T <= GDN_DECODE_MAX_TOKENS. T = 1 computes what gdn_decode_step computes.
 */
#define GDN_DECODE_MAX_TOKENS 8
int gdn_decode_multi(const void* q, const void* k, const void* v, int in_dtype, const float* g,
                     const float* beta, float* state, int N, int T, int H, int dk, int dv,
                     void* y, int y_dtype, float* step_states, void* stream);

/*
 * gdn_output_gate - eq. (11) without W_o:
 *   o = sigmoid(z) * (1 + w) * y / sqrt(mean_j(y_j^2) + eps)
 * per (token, head) over the dv channels; w is the zero-centred RMSNorm weight, shared
 * by all heads.
 *
 *   y: [ntok, H, dv] in y_dtype; z: [ntok, H, dv] in z_dtype (W_z x, before the sigmoid);
 *   norm_weight: [dv] fp32; o: [ntok, H, dv] output in o_dtype.
 */
int gdn_output_gate(const void* y, int y_dtype, const void* z, int z_dtype,
                    const float* norm_weight, int ntok, int H, int dv, float eps, void* o,
                    int o_dtype, void* stream);

/* Bytes of device workspace gdn_fused_prefill needs for these sizes (0 for unsupported sizes). */
size_t gdn_fused_prefill_workspace_size(int ntok, int num_seqs, int H, int dk, int dv);

/*
 * gdn_fused_prefill - the token mixer between the projections in one call: eqs. (6)-(10)
 * (conv -> SiLU -> L2Norm, the gates), eqs. (1)-(4) chunkwise, and eq. (11) without W_o,
 * for packed sequences that start from zero conv history (section 2.1.1 of the notes).
 * The conv, SiLU, L2Norm and gates run inside the per-chunk kernel that forms each chunk's
 * (I + A)^{-1} and P, so q and k are written once and read back from cache there, and g and
 * beta never reach memory unless exported; then the scan and the output gate.
 *
 *   xq, xk: [ntok, H, 128], xv: [ntok, H, dv] in x_dtype (the projected streams);
 *   wq, wk, wv, conv_k (= 4), a_raw, b_raw, A_log, dt_bias, l2_eps: as gdn_preprocess;
 *   z: [ntok, H, dv] in z_dtype; norm_weight: [dv] fp32; rms_eps: as gdn_output_gate's eps;
 *   initial_state, final_state, cu_seqlens, cu_seqlens_host, num_seqs: as gdn_chunk_prefill;
 *   o: [ntok, H, dv] output in o_dtype.
 *   q, k, v ([ntok, H, d] bf16), y ([ntok, H, dv] bf16): optional exports of the
 *       intermediates (a backward pass needs q, k, v, g, beta); NULL keeps each in the
 *       workspace. g, beta ([ntok, H] fp32): exported together, or both NULL (not written).
 *   workspace: at least gdn_fused_prefill_workspace_size(...) bytes, not shared by
 *       concurrent calls.
 * dk must be 128 (the bf16 matrix-core path: q, k, v are bf16 between the kernels).
 * q, k, v, g, beta, y and the final state equal gdn_preprocess -> gdn_chunk_prefill with bf16
 * q, k, v, y. With 256 or more (sequence, head) pairs, dv = 128 and no cu_seqlens (equal
 * lengths) the gate of eq. (11) runs inside the scan on the fp32 y (y never leaves the chip
 * unless exported), so o may differ in its last bits from gdn_output_gate applied to the bf16
 * y; otherwise o equals it.
 */
int gdn_fused_prefill(const void* xq, const void* xk, const void* xv, int x_dtype,
                      const float* wq, const float* wk, const float* wv, int conv_k,
                      const float* a_raw, const float* b_raw, const float* A_log,
                      const float* dt_bias, float l2_eps, const void* z, int z_dtype,
                      const float* norm_weight, float rms_eps, const float* initial_state,
                      float* final_state, const int32_t* cu_seqlens,
                      const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H, int dk,
                      int dv, void* o, int o_dtype, void* q, void* k, void* v, float* g,
                      float* beta, void* y, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * gdn_fused_decode - one decode step of the token mixer in one kernel: eqs. (6)-(10) on this
 * step's projected inputs with each sequence's carried conv history, eqs. (1)-(4) for one
 * token (state in place), and eq. (11) without W_o (section 2.1.1 of the notes; the conv is
 * causal and depthwise, design summary "设计 LLM 架构", section "Token 混合：GDN 加 QSA").
 *
 *   xq, xk: [N, H, dk], xv: [N, H, dv] in x_dtype;
 *   wq, wk, wv: [H*d, 4] fp32 conv taps; conv_k must be 4;
 *   conv_state: [N, 3, H*(2*dk+dv)] in x_dtype, in/out: the layout of
 *       gdn_preprocess_stateful's conv states (row 2 the newest input), shifted by this
 *       step's input in place;
 *   a_raw, b_raw: [N, H] fp32; A_log, dt_bias: [H] fp32; l2_eps as gdn_preprocess;
 *   state: [N, H, dk, dv] fp32, in/out;
 *   z: [N, H, dv] in x_dtype; norm_weight: [dv] fp32; rms_eps as gdn_output_gate's eps;
 *   o: [N, H, dv] output in o_dtype; y: optional [N, H, dv] in o_dtype (before the gate).
 * q and k stay fp32 inside the kernel (no bf16 rounding between the steps).
 */
int gdn_fused_decode(const void* xq, const void* xk, const void* xv, int x_dtype,
                     const float* wq, const float* wk, const float* wv, int conv_k,
                     void* conv_state, const float* a_raw, const float* b_raw,
                     const float* A_log, const float* dt_bias, float l2_eps, float* state,
                     const void* z, const float* norm_weight, float rms_eps, int N, int H,
                     int dk, int dv, void* o, int o_dtype, void* y, void* stream);

/*
 * gdn_fused_decode_multi - T consecutive tokens per sequence through the fused decode step in
 * one pass over each state (multi-token prediction verify from the projected streams): the
 * conv over the carried history and the T new inputs, the gates, eqs. (1)-(4) as in
 * gdn_decode_multi, and eq. (11) without W_o per token (sources as gdn_fused_decode and
 * gdn_decode_multi).
 *
 *   xq, xk: [N, T, H, dk], xv, z: [N, T, H, dv] in x_dtype; a_raw, b_raw: [N, T, H] fp32;
 *   wq, wk, wv, conv_k, A_log, dt_bias, l2_eps, norm_weight, rms_eps: as gdn_fused_decode;
 *   conv_state_in: [N, 3, H*(2*dk+dv)] in x_dtype (layout of gdn_preprocess_stateful);
 *   conv_state_out: same layout, the history after the T inputs; it may be conv_state_in
 *       (updated in place) or a buffer that does not overlap it (keeping the old history
 *       lets a caller rebuild the history after the first a accepted tokens);
 *   state: [N, H, dk, dv] fp32, updated in place to the state after all T tokens;
 *   step_states: NULL or [N, T, H, dk, dv] fp32, the state after each token (for rolling
 *       back rejected drafts); must not overlap state;
 *   o: [N, T, H, dv] in o_dtype; y: NULL or [N, T, H, dv] in o_dtype (before the gate).
 *   1 <= T <= GDN_DECODE_MAX_TOKENS.
 */
int gdn_fused_decode_multi(const void* xq, const void* xk, const void* xv, int x_dtype,
                           const float* wq, const float* wk, const float* wv, int conv_k,
                           const void* conv_state_in, void* conv_state_out, const float* a_raw,
                           const float* b_raw, const float* A_log, const float* dt_bias,
                           float l2_eps, float* state, const void* z, const float* norm_weight,
                           float rms_eps, int N, int T, int H, int dk, int dv, void* o,
                           int o_dtype, void* y, float* step_states, void* stream);

/* ---------------------------------------------------------------------------------------
 * Measurement aids (not operations of the layer). They measure, on the device the library
 * runs on, the two ceilings its roofline figures are read against: the HBM bandwidth of the
 * streaming access pattern and the bf16 matrix-core issue rate. Same conventions as above
 * (device pointers owned by the caller, asynchronous on `stream`, gdn_status on invalid
 * arguments).
 *
 * gdn_mb_stream - copies `bytes` bytes from src to dst with 16-byte nontemporal loads and
 *   stores, every byte read once and written once. src == dst is allowed and gives the
 *   in-place read-modify-write stream (the decode state's pattern); otherwise the two
 *   ranges must not overlap (GDN_ERR_SHAPE). bytes must be a multiple of 16 and both
 *   pointers 16-byte aligned.
 *
 * gdn_mb_mfma_bf16 - `workgroups` workgroups of 4 waves; every wave issues `iters` rounds of
 *   four independent v_mfma_f32_32x32x16_bf16 (32768 flops each), so one call performs
 *   workgroups * 4 * iters * 4 * 32768 flops. sink: [workgroups] fp32, one value per
 *   workgroup (a sum of its results, written so the work cannot be elided). workgroups >= 0,
 *   iters >= 1.
 */
int gdn_mb_stream(const void* src, void* dst, size_t bytes, void* stream);
int gdn_mb_mfma_bf16(float* sink, int workgroups, int iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
