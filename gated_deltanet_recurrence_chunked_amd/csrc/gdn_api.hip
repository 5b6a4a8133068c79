// C ABI of libgdn (declared in include/gdn.h): host-side argument validation and dispatch.
// Validation runs entirely on the host before any HIP call, so a rejected call enqueues
// nothing and touches no device state.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/gdn.h"
#include "gdn_launch.h"

static_assert(gdn::kMaxDecodeTokens == GDN_DECODE_MAX_TOKENS, "decode token limit");

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return GDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool valid_dim(int d) { return d == 64 || d == 128; }
bool valid_dtype(int t) { return t == GDN_F32 || t == GDN_BF16; }

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define GDN_REQUIRE(cond, status, ...) \
    do {                               \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

#define GDN_PTR(p)                                                               \
    do {                                                                         \
        GDN_REQUIRE((p) != nullptr, GDN_ERR_NULL, "%s must not be NULL", #p);   \
        GDN_REQUIRE(aligned16(p), GDN_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
    } while (0)

// scalar-per-element arrays (gates, per-head vectors, offsets) only need 4-byte alignment
#define GDN_SPTR(p)                                                              \
    do {                                                                         \
        GDN_REQUIRE((p) != nullptr, GDN_ERR_NULL, "%s must not be NULL", #p);   \
        GDN_REQUIRE(aligned4(p), GDN_ERR_ALIGN, "%s is not 4-byte aligned", #p); \
    } while (0)

// Token-indexed arrays may be NULL when there are no tokens (n == 0): nothing reads them, and
// torch hands out a null pointer for a tensor with no elements.
#define GDN_TPTR(p, n)                  \
    do {                                \
        if ((n) > 0 || (p)) GDN_PTR(p); \
    } while (0)
#define GDN_TSPTR(p, n)                  \
    do {                                 \
        if ((n) > 0 || (p)) GDN_SPTR(p); \
    } while (0)

#define GDN_OPT_PTR(p) \
    GDN_REQUIRE((p) == nullptr || aligned16(p), GDN_ERR_ALIGN, "%s is not 16-byte aligned", #p)

// Every array a call touches holds at most 2^31 - 1 elements (the kernels index within one
// array in 32-bit arithmetic): token arrays rows * H * d, state arrays states * H * dk * dv.
constexpr long long kMaxElems = 2147483647LL;
int check_extents(long long rows, int H, int d, long long states, long long state_elems) {
    GDN_REQUIRE(rows * H * d <= kMaxElems, GDN_ERR_SHAPE,
                "token arrays of %lld rows x H=%d x d=%d exceed 2^31-1 elements", rows, H, d);
    GDN_REQUIRE(states * state_elems <= kMaxElems, GDN_ERR_SHAPE,
                "state arrays of %lld x %lld elements exceed 2^31-1 elements", states, state_elems);
    return GDN_OK;
}
#define GDN_EXTENTS(...)                        \
    do {                                        \
        const int st_ = check_extents(__VA_ARGS__); \
        if (st_) return st_;                    \
    } while (0)

// Checks the packing description shared by preprocess and prefill.
int check_packing(const int32_t* cu_host, bool have_cu, int num_seqs, int ntok) {
    GDN_REQUIRE(num_seqs >= 1, GDN_ERR_SHAPE, "num_seqs must be >= 1 (got %d)", num_seqs);
    GDN_REQUIRE(ntok >= 0, GDN_ERR_SHAPE, "ntok must be >= 0 (got %d)", ntok);
    if (!have_cu)
        GDN_REQUIRE(ntok % num_seqs == 0, GDN_ERR_SHAPE,
                    "without cu_seqlens ntok (%d) must be a multiple of num_seqs (%d)", ntok,
                    num_seqs);
    if (cu_host) {
        GDN_REQUIRE(cu_host[0] == 0, GDN_ERR_SEQLENS, "cu_seqlens[0] must be 0");
        for (int i = 0; i < num_seqs; ++i)
            GDN_REQUIRE(cu_host[i + 1] >= cu_host[i], GDN_ERR_SEQLENS,
                        "cu_seqlens must be non-decreasing (index %d)", i + 1);
        GDN_REQUIRE(cu_host[num_seqs] == ntok, GDN_ERR_SEQLENS,
                    "cu_seqlens[num_seqs] (%d) must equal ntok (%d)", cu_host[num_seqs], ntok);
    }
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(int s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL: return "GDN_ERR_NULL";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE";
        case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE";
        case GDN_ERR_SEQLENS: return "GDN_ERR_SEQLENS";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
        case GDN_ERR_HIP: return "GDN_ERR_HIP";
        default: return "GDN_ERR_UNKNOWN";
    }
}

const char* gdn_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

int preprocess_impl(const void* xq, const void* xk, const void* xv, int x_dtype, const float* wq,
                    const float* wk, const float* wv, int conv_k, const float* a_raw,
                    const float* b_raw, const float* A_log, const float* dt_bias,
                    const int32_t* cu_seqlens, int num_seqs, int ntok, int H, int dk, int dv,
                    float l2_eps, void* q, void* k, void* v, int out_dtype, float* g, float* beta,
                    const void* conv_state_in, void* conv_state_out, void* stream,
                    const char* name) {
    GDN_REQUIRE(valid_dtype(x_dtype) && valid_dtype(out_dtype), GDN_ERR_DTYPE,
                "x_dtype/out_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(H >= 1 && valid_dim(dk) && valid_dim(dv), GDN_ERR_SHAPE,
                "need H >= 1 and dk, dv in {64, 128} (got H=%d dk=%d dv=%d)", H, dk, dv);
    const bool conv = xq || xk || xv || wq || wk || wv || q || k || v;
    const bool gates = a_raw || b_raw || A_log || dt_bias || g || beta;
    GDN_REQUIRE(conv || gates, GDN_ERR_NULL, "nothing to compute: all inputs are NULL");
    if (conv) {
        GDN_TPTR(xq, ntok); GDN_TPTR(xk, ntok); GDN_TPTR(xv, ntok);
        GDN_PTR(wq); GDN_PTR(wk); GDN_PTR(wv);
        GDN_TPTR(q, ntok); GDN_TPTR(k, ntok); GDN_TPTR(v, ntok);
        GDN_REQUIRE(conv_k == 4, GDN_ERR_SHAPE, "conv_k must be 4 (got %d)", conv_k);
        GDN_REQUIRE(l2_eps >= 0.f, GDN_ERR_SHAPE, "l2_eps must be >= 0");
    }
    if (gates) {
        GDN_TSPTR(a_raw, ntok); GDN_TSPTR(b_raw, ntok); GDN_SPTR(A_log); GDN_SPTR(dt_bias);
        GDN_TSPTR(g, ntok); GDN_TSPTR(beta, ntok);
    }
    GDN_REQUIRE(aligned4(cu_seqlens), GDN_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
    int st = check_packing(nullptr, cu_seqlens != nullptr, num_seqs, ntok);
    if (st) return st;
    const int hC = H * (2 * dk + dv);
    GDN_EXTENTS(ntok, H, dk > dv ? dk : dv, num_seqs, 3LL * hC);
    if (conv_state_in || conv_state_out) {
        GDN_REQUIRE(conv, GDN_ERR_NULL, "a conv state needs the conv inputs and outputs");
        GDN_OPT_PTR(conv_state_in);
        GDN_OPT_PTR(conv_state_out);
        const size_t bytes = (size_t)num_seqs * (conv_k - 1) * hC * (x_dtype == GDN_BF16 ? 2 : 4);
        const char* i0 = static_cast<const char*>(conv_state_in);
        const char* o0 = static_cast<const char*>(conv_state_out);
        GDN_REQUIRE(!i0 || !o0 || i0 + bytes <= o0 || o0 + bytes <= i0, GDN_ERR_SHAPE,
                    "conv_state_in and conv_state_out must not overlap");
    }

    gdn::PreprocessArgs a;
    a.x[0] = conv ? xq : nullptr; a.x[1] = conv ? xk : nullptr; a.x[2] = conv ? xv : nullptr;
    a.w[0] = wq; a.w[1] = wk; a.w[2] = wv;
    a.out[0] = q; a.out[1] = k; a.out[2] = v;
    a.d[0] = dk; a.d[1] = dk; a.d[2] = dv;
    a.in_bf16 = x_dtype == GDN_BF16;
    a.out_bf16 = out_dtype == GDN_BF16;
    a.a_raw = gates ? a_raw : nullptr;
    a.b_raw = b_raw; a.A_log = A_log; a.dt_bias = dt_bias; a.g = g; a.beta = beta;
    a.cu = cu_seqlens;
    a.num_seqs = num_seqs; a.ntok = ntok; a.H = H; a.l2_eps = l2_eps;
    a.hin = conv_state_in; a.hout = conv_state_out; a.hC = hC;
    return hip_status(gdn::launch_preprocess(a, static_cast<hipStream_t>(stream)), name);
}

}  // namespace

extern "C" {

int gdn_preprocess(const void* xq, const void* xk, const void* xv, int x_dtype, const float* wq,
                   const float* wk, const float* wv, int conv_k, const float* a_raw,
                   const float* b_raw, const float* A_log, const float* dt_bias,
                   const int32_t* cu_seqlens, int num_seqs, int ntok, int H, int dk, int dv,
                   float l2_eps, void* q, void* k, void* v, int out_dtype, float* g, float* beta,
                   void* stream) {
    return preprocess_impl(xq, xk, xv, x_dtype, wq, wk, wv, conv_k, a_raw, b_raw, A_log, dt_bias,
                           cu_seqlens, num_seqs, ntok, H, dk, dv, l2_eps, q, k, v, out_dtype, g,
                           beta, nullptr, nullptr, stream, "gdn_preprocess");
}

int gdn_preprocess_stateful(const void* xq, const void* xk, const void* xv, int x_dtype,
                            const float* wq, const float* wk, const float* wv, int conv_k,
                            const float* a_raw, const float* b_raw, const float* A_log,
                            const float* dt_bias, const int32_t* cu_seqlens, int num_seqs,
                            int ntok, int H, int dk, int dv, float l2_eps, void* q, void* k,
                            void* v, int out_dtype, float* g, float* beta,
                            const void* conv_state_in, void* conv_state_out, void* stream) {
    return preprocess_impl(xq, xk, xv, x_dtype, wq, wk, wv, conv_k, a_raw, b_raw, A_log, dt_bias,
                           cu_seqlens, num_seqs, ntok, H, dk, dv, l2_eps, q, k, v, out_dtype, g,
                           beta, conv_state_in, conv_state_out, stream, "gdn_preprocess_stateful");
}

// The bf16 path with dk = 128 runs on the matrix cores and keeps per-chunk T and P tiles
// in the workspace; every other combination runs the all-fp32 kernel, which needs none.
static bool use_matrix_path(int in_dtype, int dk) { return in_dtype == GDN_BF16 && dk == 128; }

size_t gdn_chunk_prefill_workspace_size(int ntok, int num_seqs, int H, int dk, int dv, int in_dtype) {
    (void)dv;
    if (ntok < 0 || num_seqs < 1 || H < 1) return 0;
    return use_matrix_path(in_dtype, dk) ? gdn::chunk_bf16_workspace(ntok, num_seqs, H) : 0;
}

}  // extern "C"

namespace {

// gdn_chunk_prefill and its allocation-free variant: validation and dispatch, given the
// workspace (for the variant, the library's scratch array; ws_limit its size, else 0).
int chunk_prefill_impl(const void* q, const void* k, const void* v, int in_dtype, const float* g,
                       const float* beta, const float* initial_state, float* final_state,
                       const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int num_seqs,
                       int ntok, int H, int dk, int dv, void* y, int y_dtype, void* workspace,
                       size_t workspace_bytes, bool noalloc, void* stream, const char* name) {
    GDN_REQUIRE(valid_dtype(in_dtype) && valid_dtype(y_dtype), GDN_ERR_DTYPE,
                "in_dtype/y_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(H >= 1 && valid_dim(dk) && valid_dim(dv), GDN_ERR_SHAPE,
                "need H >= 1 and dk, dv in {64, 128} (got H=%d dk=%d dv=%d)", H, dk, dv);
    GDN_TPTR(q, ntok); GDN_TPTR(k, ntok); GDN_TPTR(v, ntok); GDN_TSPTR(g, ntok);
    GDN_TSPTR(beta, ntok); GDN_TPTR(y, ntok);
    GDN_OPT_PTR(initial_state); GDN_OPT_PTR(final_state);
    GDN_REQUIRE(aligned4(cu_seqlens), GDN_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
    GDN_REQUIRE(cu_seqlens_host == nullptr || cu_seqlens != nullptr, GDN_ERR_NULL,
                "cu_seqlens_host given without the device cu_seqlens");
    int st = check_packing(cu_seqlens_host, cu_seqlens != nullptr, num_seqs, ntok);
    if (st) return st;
    GDN_EXTENTS(ntok, H, dk > dv ? dk : dv, num_seqs, (long long)H * dk * dv);
    const size_t need = gdn_chunk_prefill_workspace_size(ntok, num_seqs, H, dk, dv, in_dtype);
    if (noalloc) {
        GDN_REQUIRE(need <= GDN_NOALLOC_SCRATCH_BYTES, GDN_ERR_WORKSPACE,
                    "%s: these sizes need %zu bytes of workspace, more than the %zu bytes of the "
                    "library's scratch array (use gdn_chunk_prefill with a workspace)",
                    name, need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
        if (need > 0) {
            const hipError_t e = gdn::noalloc_scratch(&workspace);
            if (e != hipSuccess) return hip_status(e, name);
            workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
        }
    }
    GDN_REQUIRE(workspace_bytes >= need && (need == 0 || workspace != nullptr), GDN_ERR_WORKSPACE,
                "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    GDN_OPT_PTR(workspace);

    gdn::ChunkArgs a;
    a.q = q; a.k = k; a.v = v;
    a.in_bf16 = in_dtype == GDN_BF16;
    a.y_bf16 = y_dtype == GDN_BF16;
    a.g = g; a.beta = beta; a.S0 = initial_state; a.ST = final_state;
    a.cu = cu_seqlens;
    a.num_seqs = num_seqs; a.ntok = ntok; a.H = H; a.dk = dk; a.dv = dv;
    a.y = y; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (use_matrix_path(in_dtype, dk)) return hip_status(gdn::launch_chunk_bf16(a, s), name);
    return hip_status(gdn::launch_chunk_fp32(a, s), name);
}

}  // namespace

extern "C" {

int gdn_chunk_prefill(const void* q, const void* k, const void* v, int in_dtype, const float* g,
                      const float* beta, const float* initial_state, float* final_state,
                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int num_seqs,
                      int ntok, int H, int dk, int dv, void* y, int y_dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
    return chunk_prefill_impl(q, k, v, in_dtype, g, beta, initial_state, final_state, cu_seqlens,
                              cu_seqlens_host, num_seqs, ntok, H, dk, dv, y, y_dtype, workspace,
                              workspace_bytes, false, stream, "gdn_chunk_prefill");
}

int gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v, int in_dtype,
                              const float* g, const float* beta, const float* initial_state,
                              float* final_state, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H,
                              int dk, int dv, void* y, int y_dtype, void* stream) {
    return chunk_prefill_impl(q, k, v, in_dtype, g, beta, initial_state, final_state, cu_seqlens,
                              cu_seqlens_host, num_seqs, ntok, H, dk, dv, y, y_dtype, nullptr, 0,
                              true, stream, "gdn_chunk_prefill_noalloc");
}

size_t gdn_chunk_backward_workspace_size(int ntok, int num_seqs, int H, int dk, int dv) {
    if (ntok < 0 || num_seqs < 1 || H < 1 || !valid_dim(dk) || !valid_dim(dv)) return 0;
    return gdn::chunk_bwd_workspace(ntok, num_seqs, H, dk, dv);
}

int gdn_chunk_backward(const void* q, const void* k, const void* v, int in_dtype, const float* g,
                       const float* beta, const float* initial_state, const void* dy,
                       int dy_dtype, const float* dfinal_state, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H, int dk,
                       int dv, float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                       float* dinitial_state, void* workspace, size_t workspace_bytes,
                       void* stream) {
    GDN_REQUIRE(valid_dtype(in_dtype) && valid_dtype(dy_dtype), GDN_ERR_DTYPE,
                "in_dtype/dy_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(H >= 1 && valid_dim(dk) && valid_dim(dv), GDN_ERR_SHAPE,
                "need H >= 1 and dk, dv in {64, 128} (got H=%d dk=%d dv=%d)", H, dk, dv);
    GDN_TPTR(q, ntok); GDN_TPTR(k, ntok); GDN_TPTR(v, ntok); GDN_TSPTR(g, ntok);
    GDN_TSPTR(beta, ntok); GDN_TPTR(dy, ntok);
    GDN_TPTR(dq, ntok); GDN_TPTR(dk_out, ntok); GDN_TPTR(dv_out, ntok); GDN_TSPTR(dg, ntok);
    GDN_TSPTR(dbeta, ntok);
    GDN_OPT_PTR(initial_state); GDN_OPT_PTR(dfinal_state); GDN_OPT_PTR(dinitial_state);
    GDN_REQUIRE(aligned4(cu_seqlens), GDN_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
    GDN_REQUIRE(cu_seqlens_host == nullptr || cu_seqlens != nullptr, GDN_ERR_NULL,
                "cu_seqlens_host given without the device cu_seqlens");
    int st = check_packing(cu_seqlens_host, cu_seqlens != nullptr, num_seqs, ntok);
    if (st) return st;
    GDN_EXTENTS(ntok, H, dk > dv ? dk : dv, num_seqs, (long long)H * dk * dv);
    const size_t need = gdn::chunk_bwd_workspace(ntok, num_seqs, H, dk, dv);
    GDN_REQUIRE(workspace_bytes >= need && workspace != nullptr, GDN_ERR_WORKSPACE,
                "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    GDN_OPT_PTR(workspace);
    gdn::ChunkBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dy = dy;
    a.in_bf16 = in_dtype == GDN_BF16; a.dy_bf16 = dy_dtype == GDN_BF16;
    a.g = g; a.beta = beta; a.S0 = initial_state; a.dST = dfinal_state; a.cu = cu_seqlens;
    a.num_seqs = num_seqs; a.ntok = ntok; a.H = H; a.dk = dk; a.dv = dv;
    a.dq = dq; a.dk_ = dk_out; a.dv_ = dv_out; a.dg = dg; a.dbeta = dbeta;
    a.dS0 = dinitial_state; a.workspace = workspace;
    return hip_status(gdn::launch_chunk_bwd(a, static_cast<hipStream_t>(stream)),
                      "gdn_chunk_backward");
}

size_t gdn_kda_chunk_prefill_workspace_size(int ntok, int num_seqs, int H, int dk) {
    if (ntok < 0 || num_seqs < 1 || H < 1 || !valid_dim(dk)) return 0;
    return gdn::chunk_kda_workspace(ntok, num_seqs, H, dk);
}

int gdn_kda_chunk_prefill(const void* q, const void* k, const void* v, int in_dtype,
                          const float* g, const float* beta, const float* initial_state,
                          float* final_state, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H, int dk,
                          int dv, void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
    GDN_REQUIRE(valid_dtype(in_dtype) && valid_dtype(y_dtype), GDN_ERR_DTYPE,
                "in_dtype/y_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(H >= 1 && valid_dim(dk) && valid_dim(dv), GDN_ERR_SHAPE,
                "need H >= 1 and dk, dv in {64, 128} (got H=%d dk=%d dv=%d)", H, dk, dv);
    GDN_TPTR(q, ntok); GDN_TPTR(k, ntok); GDN_TPTR(v, ntok); GDN_TSPTR(g, ntok);
    GDN_TSPTR(beta, ntok); GDN_TPTR(y, ntok);
    GDN_OPT_PTR(initial_state); GDN_OPT_PTR(final_state);
    GDN_REQUIRE(aligned4(cu_seqlens), GDN_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
    GDN_REQUIRE(cu_seqlens_host == nullptr || cu_seqlens != nullptr, GDN_ERR_NULL,
                "cu_seqlens_host given without the device cu_seqlens");
    int st = check_packing(cu_seqlens_host, cu_seqlens != nullptr, num_seqs, ntok);
    if (st) return st;
    GDN_EXTENTS(ntok, H, dk > dv ? dk : dv, num_seqs, (long long)H * dk * dv);
    const size_t need = gdn::chunk_kda_workspace(ntok, num_seqs, H, dk);
    GDN_REQUIRE(workspace_bytes >= need && workspace != nullptr, GDN_ERR_WORKSPACE,
                "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    GDN_OPT_PTR(workspace);
    gdn::ChunkKdaArgs a;
    a.q = q; a.k = k; a.v = v; a.in_bf16 = in_dtype == GDN_BF16; a.y_bf16 = y_dtype == GDN_BF16;
    a.g = g; a.beta = beta; a.S0 = initial_state; a.ST = final_state; a.cu = cu_seqlens;
    a.num_seqs = num_seqs; a.ntok = ntok; a.H = H; a.dk = dk; a.dv = dv; a.y = y;
    a.workspace = workspace;
    return hip_status(gdn::launch_chunk_kda(a, static_cast<hipStream_t>(stream)),
                      "gdn_kda_chunk_prefill");
}

size_t gdn_kda_chunk_prefill_bounded_workspace_size(int ntok, int num_seqs, int H) {
    if (ntok < 0 || num_seqs < 1 || H < 1) return 0;
    return gdn::kda_bf16_workspace(ntok, num_seqs, H);
}

int gdn_kda_chunk_prefill_bounded(const void* q, const void* k, const void* v, int in_dtype,
                                  const float* g, const float* beta, const float* initial_state,
                                  float* final_state, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H,
                                  int dk, int dv, void* y, int y_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    GDN_REQUIRE(in_dtype == GDN_BF16 && valid_dtype(y_dtype), GDN_ERR_DTYPE,
                "in_dtype must be GDN_BF16 and y_dtype GDN_F32 or GDN_BF16");
    GDN_REQUIRE(H >= 1 && dk == 128 && dv == 128, GDN_ERR_SHAPE,
                "need H >= 1 and dk = dv = 128 (got H=%d dk=%d dv=%d)", H, dk, dv);
    GDN_TPTR(q, ntok); GDN_TPTR(k, ntok); GDN_TPTR(v, ntok); GDN_TPTR(g, ntok);
    GDN_TSPTR(beta, ntok); GDN_TPTR(y, ntok);
    GDN_OPT_PTR(initial_state); GDN_OPT_PTR(final_state);
    GDN_REQUIRE(aligned4(cu_seqlens), GDN_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
    GDN_REQUIRE(cu_seqlens_host == nullptr || cu_seqlens != nullptr, GDN_ERR_NULL,
                "cu_seqlens_host given without the device cu_seqlens");
    int st = check_packing(cu_seqlens_host, cu_seqlens != nullptr, num_seqs, ntok);
    if (st) return st;
    GDN_EXTENTS(ntok, H, dk, num_seqs, (long long)H * dk * dv);
    const size_t need = gdn::kda_bf16_workspace(ntok, num_seqs, H);
    GDN_REQUIRE(workspace_bytes >= need && workspace != nullptr, GDN_ERR_WORKSPACE,
                "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    GDN_OPT_PTR(workspace);
    gdn::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.in_bf16 = 1; a.y_bf16 = y_dtype == GDN_BF16;
    a.g = nullptr; a.beta = beta; a.S0 = initial_state; a.ST = final_state; a.cu = cu_seqlens;
    a.num_seqs = num_seqs; a.ntok = ntok; a.H = H; a.dk = dk; a.dv = dv; a.y = y;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return hip_status(gdn::launch_kda_bf16(a, g, static_cast<hipStream_t>(stream)),
                      "gdn_kda_chunk_prefill_bounded");
}

int gdn_decode_step(const void* q, const void* k, const void* v, int in_dtype, const float* g,
                    const float* beta, float* state, int N, int H, int dk, int dv, void* y,
                    int y_dtype, void* stream) {
    GDN_REQUIRE(valid_dtype(in_dtype) && valid_dtype(y_dtype), GDN_ERR_DTYPE,
                "in_dtype/y_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(N >= 0 && H >= 1 && valid_dim(dk) && valid_dim(dv), GDN_ERR_SHAPE,
                "need N >= 0, H >= 1 and dk, dv in {64, 128} (got N=%d H=%d dk=%d dv=%d)", N, H,
                dk, dv);
    GDN_TPTR(q, N); GDN_TPTR(k, N); GDN_TPTR(v, N); GDN_TSPTR(g, N); GDN_TSPTR(beta, N);
    GDN_TPTR(state, N); GDN_TPTR(y, N);
    GDN_EXTENTS(N, H, dk > dv ? dk : dv, N, (long long)H * dk * dv);
    return hip_status(gdn::launch_decode(q, k, v, in_dtype == GDN_BF16, g, beta, state, N, H, dk,
                                         dv, y, y_dtype == GDN_BF16,
                                         static_cast<hipStream_t>(stream)),
                      "gdn_decode_step");
}

int gdn_decode_multi(const void* q, const void* k, const void* v, int in_dtype, const float* g,
                     const float* beta, float* state, int N, int T, int H, int dk, int dv,
                     void* y, int y_dtype, float* step_states, void* stream) {
    GDN_REQUIRE(valid_dtype(in_dtype) && valid_dtype(y_dtype), GDN_ERR_DTYPE,
                "in_dtype/y_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(N >= 0 && H >= 1 && valid_dim(dk) && valid_dim(dv), GDN_ERR_SHAPE,
                "need N >= 0, H >= 1 and dk, dv in {64, 128} (got N=%d H=%d dk=%d dv=%d)", N, H,
                dk, dv);
    GDN_REQUIRE(T >= 1 && T <= GDN_DECODE_MAX_TOKENS, GDN_ERR_SHAPE,
                "T must be in 1..%d (got %d)", GDN_DECODE_MAX_TOKENS, T);
    GDN_TPTR(q, N); GDN_TPTR(k, N); GDN_TPTR(v, N); GDN_TSPTR(g, N); GDN_TSPTR(beta, N);
    GDN_TPTR(state, N); GDN_TPTR(y, N);
    GDN_OPT_PTR(step_states);
    GDN_EXTENTS((long long)N * T, H, dk > dv ? dk : dv, (long long)N * (step_states ? T : 1),
                (long long)H * dk * dv);
    if (step_states) {
        const char* a0 = reinterpret_cast<const char*>(state);
        const char* b0 = reinterpret_cast<const char*>(step_states);
        const size_t sb = (size_t)N * H * dk * dv * sizeof(float);
        GDN_REQUIRE(a0 + sb <= b0 || b0 + sb * T <= a0, GDN_ERR_SHAPE,
                    "step_states must not overlap state");
    }
    return hip_status(gdn::launch_decode_multi(q, k, v, in_dtype == GDN_BF16, g, beta, state, N, T,
                                               H, dk, dv, y, y_dtype == GDN_BF16, step_states,
                                               static_cast<hipStream_t>(stream)),
                      "gdn_decode_multi");
}

size_t gdn_fused_prefill_workspace_size(int ntok, int num_seqs, int H, int dk, int dv) {
    if (ntok < 0 || num_seqs < 1 || H < 1 || dk != 128 || !valid_dim(dv)) return 0;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t rows = (size_t)ntok * H;
    return up(gdn::chunk_bf16_workspace(ntok, num_seqs, H)) + 2 * up(rows * dk * 2) +
           2 * up(rows * dv * 2) + 2 * up(rows * sizeof(float));
}

int gdn_fused_prefill(const void* xq, const void* xk, const void* xv, int x_dtype, const float* wq,
                      const float* wk, const float* wv, int conv_k, const float* a_raw,
                      const float* b_raw, const float* A_log, const float* dt_bias, float l2_eps,
                      const void* z, int z_dtype, const float* norm_weight, float rms_eps,
                      const float* initial_state, float* final_state, const int32_t* cu_seqlens,
                      const int32_t* cu_seqlens_host, int num_seqs, int ntok, int H, int dk,
                      int dv, void* o, int o_dtype, void* q, void* k, void* v, float* g,
                      float* beta, void* y, void* workspace, size_t workspace_bytes,
                      void* stream) {
    GDN_REQUIRE(valid_dtype(x_dtype) && valid_dtype(z_dtype) && valid_dtype(o_dtype), GDN_ERR_DTYPE,
                "x_dtype/z_dtype/o_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(H >= 1 && dk == 128 && valid_dim(dv), GDN_ERR_SHAPE,
                "need H >= 1, dk = 128 and dv in {64, 128} (got H=%d dk=%d dv=%d)", H, dk, dv);
    GDN_REQUIRE(conv_k == 4, GDN_ERR_SHAPE, "conv_k must be 4 (got %d)", conv_k);
    GDN_REQUIRE(l2_eps >= 0.f && rms_eps >= 0.f, GDN_ERR_SHAPE, "l2_eps and rms_eps must be >= 0");
    GDN_TPTR(xq, ntok); GDN_TPTR(xk, ntok); GDN_TPTR(xv, ntok);
    GDN_PTR(wq); GDN_PTR(wk); GDN_PTR(wv);
    GDN_TSPTR(a_raw, ntok); GDN_TSPTR(b_raw, ntok); GDN_SPTR(A_log); GDN_SPTR(dt_bias);
    GDN_TPTR(z, ntok); GDN_SPTR(norm_weight); GDN_TPTR(o, ntok);
    GDN_OPT_PTR(initial_state); GDN_OPT_PTR(final_state);
    GDN_OPT_PTR(q); GDN_OPT_PTR(k); GDN_OPT_PTR(v); GDN_OPT_PTR(y);
    GDN_REQUIRE(aligned4(g) && aligned4(beta), GDN_ERR_ALIGN, "g/beta are not 4-byte aligned");
    GDN_REQUIRE((g == nullptr) == (beta == nullptr), GDN_ERR_NULL,
                "g and beta are exported together (both or neither)");
    GDN_REQUIRE(aligned4(cu_seqlens), GDN_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
    GDN_REQUIRE(cu_seqlens_host == nullptr || cu_seqlens != nullptr, GDN_ERR_NULL,
                "cu_seqlens_host given without the device cu_seqlens");
    int st = check_packing(cu_seqlens_host, cu_seqlens != nullptr, num_seqs, ntok);
    if (st) return st;
    GDN_EXTENTS(ntok, H, dk > dv ? dk : dv, num_seqs, (long long)H * dk * dv);
    const size_t need = gdn_fused_prefill_workspace_size(ntok, num_seqs, H, dk, dv);
    GDN_REQUIRE(workspace != nullptr && workspace_bytes >= need, GDN_ERR_WORKSPACE,
                "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    GDN_OPT_PTR(workspace);

    // workspace: [prefill tiles | q | k | v | y | g | beta]; exported intermediates replace
    // their slot
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t rows = (size_t)ntok * H;
    char* ws = static_cast<char*>(workspace);
    size_t off = up(gdn::chunk_bf16_workspace(ntok, num_seqs, H));
    void* slot[6];
    const size_t bytes[6] = {rows * dk * 2, rows * dk * 2, rows * dv * 2, rows * dv * 2,
                             rows * sizeof(float), rows * sizeof(float)};
    for (int i = 0; i < 6; ++i) {
        slot[i] = ws + off;
        off += up(bytes[i]);
    }
    void* qb = q ? q : slot[0];
    void* kb = k ? k : slot[1];
    void* vb = v ? v : slot[2];
    void* yb = y ? y : slot[3];
    float* gb = g ? g : static_cast<float*>(slot[4]);
    float* bb = beta ? beta : static_cast<float*>(slot[5]);
    hipStream_t s = static_cast<hipStream_t>(stream);

    // eqs. (6)-(10): the preprocess kernel (bf16 q, k, v), exactly as gdn_preprocess
    gdn::PreprocessArgs p;
    p.x[0] = xq; p.x[1] = xk; p.x[2] = xv;
    p.w[0] = wq; p.w[1] = wk; p.w[2] = wv;
    p.out[0] = qb; p.out[1] = kb; p.out[2] = vb;
    p.d[0] = dk; p.d[1] = dk; p.d[2] = dv;
    p.in_bf16 = x_dtype == GDN_BF16;
    p.out_bf16 = 1;
    p.a_raw = a_raw; p.b_raw = b_raw; p.A_log = A_log; p.dt_bias = dt_bias;
    p.g = gb; p.beta = bb;
    p.cu = cu_seqlens;
    p.num_seqs = num_seqs; p.ntok = ntok; p.H = H; p.l2_eps = l2_eps;
    p.hin = nullptr; p.hout = nullptr; p.hC = 0;
    if (ntok > 0) {
        const hipError_t e = gdn::launch_preprocess(p, s);
        if (e != hipSuccess) return hip_status(e, "gdn_fused_prefill");
    }

    // eqs. (1)-(5) and eq. (11): the chunked prefill with the gate applied to its y (inside
    // the scan when the full-row scan runs)
    gdn::ChunkArgs a;
    a.q = qb; a.k = kb; a.v = vb;
    a.in_bf16 = 1;
    a.y_bf16 = 1;
    a.g = gb; a.beta = bb; a.S0 = initial_state; a.ST = final_state;
    a.cu = cu_seqlens;
    a.num_seqs = num_seqs; a.ntok = ntok; a.H = H; a.dk = dk; a.dv = dv;
    a.y = yb; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    gdn::GateArgs ga;
    ga.z = z; ga.z_bf16 = z_dtype == GDN_BF16;
    ga.w = norm_weight; ga.eps = rms_eps;
    ga.o = o; ga.o_bf16 = o_dtype == GDN_BF16;
    ga.y_export = y;
    return hip_status(gdn::launch_chunk_bf16(a, s, &ga), "gdn_fused_prefill");
}

int gdn_fused_decode(const void* xq, const void* xk, const void* xv, int x_dtype, const float* wq,
                     const float* wk, const float* wv, int conv_k, void* conv_state,
                     const float* a_raw, const float* b_raw, const float* A_log,
                     const float* dt_bias, float l2_eps, float* state, const void* z,
                     const float* norm_weight, float rms_eps, int N, int H, int dk, int dv,
                     void* o, int o_dtype, void* y, void* stream) {
    GDN_REQUIRE(valid_dtype(x_dtype) && valid_dtype(o_dtype), GDN_ERR_DTYPE,
                "x_dtype/o_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(N >= 0 && H >= 1 && valid_dim(dk) && valid_dim(dv), GDN_ERR_SHAPE,
                "need N >= 0, H >= 1 and dk, dv in {64, 128} (got N=%d H=%d dk=%d dv=%d)", N, H,
                dk, dv);
    GDN_REQUIRE(conv_k == 4, GDN_ERR_SHAPE, "conv_k must be 4 (got %d)", conv_k);
    GDN_REQUIRE(l2_eps >= 0.f && rms_eps >= 0.f, GDN_ERR_SHAPE, "l2_eps and rms_eps must be >= 0");
    GDN_TPTR(xq, N); GDN_TPTR(xk, N); GDN_TPTR(xv, N); GDN_PTR(wq); GDN_PTR(wk); GDN_PTR(wv);
    GDN_TPTR(conv_state, N);
    GDN_TSPTR(a_raw, N); GDN_TSPTR(b_raw, N); GDN_SPTR(A_log); GDN_SPTR(dt_bias);
    GDN_TPTR(state, N); GDN_TPTR(z, N); GDN_SPTR(norm_weight); GDN_TPTR(o, N); GDN_OPT_PTR(y);
    GDN_EXTENTS(N, H, dk > dv ? dk : dv, N, (long long)H * dk * dv);
    GDN_EXTENTS(N, 1, 3 * H * (2 * dk + dv), 0, 0);
    gdn::DecodeFusedArgs f;
    f.x[0] = xq; f.x[1] = xk; f.x[2] = xv;
    f.w[0] = wq; f.w[1] = wk; f.w[2] = wv;
    f.conv_state = conv_state;
    f.hC = H * (2 * dk + dv);
    f.a_raw = a_raw; f.b_raw = b_raw; f.A_log = A_log; f.dt_bias = dt_bias;
    f.l2_eps = l2_eps;
    f.state = state; f.z = z; f.norm_w = norm_weight; f.rms_eps = rms_eps;
    f.o = o; f.y = y;
    f.N = N; f.H = H;
    f.in_bf16 = x_dtype == GDN_BF16;
    f.out_bf16 = o_dtype == GDN_BF16;
    return hip_status(gdn::launch_decode_fused(f, dk, dv, static_cast<hipStream_t>(stream)),
                      "gdn_fused_decode");
}

int gdn_fused_decode_multi(const void* xq, const void* xk, const void* xv, int x_dtype,
                           const float* wq, const float* wk, const float* wv, int conv_k,
                           const void* conv_state_in, void* conv_state_out, const float* a_raw,
                           const float* b_raw, const float* A_log, const float* dt_bias,
                           float l2_eps, float* state, const void* z, const float* norm_weight,
                           float rms_eps, int N, int T, int H, int dk, int dv, void* o,
                           int o_dtype, void* y, float* step_states, void* stream) {
    GDN_REQUIRE(valid_dtype(x_dtype) && valid_dtype(o_dtype), GDN_ERR_DTYPE,
                "x_dtype/o_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(N >= 0 && H >= 1 && valid_dim(dk) && valid_dim(dv), GDN_ERR_SHAPE,
                "need N >= 0, H >= 1 and dk, dv in {64, 128} (got N=%d H=%d dk=%d dv=%d)", N, H,
                dk, dv);
    GDN_REQUIRE(T >= 1 && T <= GDN_DECODE_MAX_TOKENS, GDN_ERR_SHAPE,
                "T must be in 1..%d (got %d)", GDN_DECODE_MAX_TOKENS, T);
    GDN_REQUIRE(conv_k == 4, GDN_ERR_SHAPE, "conv_k must be 4 (got %d)", conv_k);
    GDN_REQUIRE(l2_eps >= 0.f && rms_eps >= 0.f, GDN_ERR_SHAPE, "l2_eps and rms_eps must be >= 0");
    GDN_TPTR(xq, N); GDN_TPTR(xk, N); GDN_TPTR(xv, N); GDN_PTR(wq); GDN_PTR(wk); GDN_PTR(wv);
    GDN_TPTR(conv_state_in, N); GDN_TPTR(conv_state_out, N);
    GDN_TSPTR(a_raw, N); GDN_TSPTR(b_raw, N); GDN_SPTR(A_log); GDN_SPTR(dt_bias);
    GDN_TPTR(state, N); GDN_TPTR(z, N); GDN_SPTR(norm_weight); GDN_TPTR(o, N); GDN_OPT_PTR(y);
    GDN_OPT_PTR(step_states);
    GDN_EXTENTS((long long)N * T, H, dk > dv ? dk : dv, (long long)N * (step_states ? T : 1),
                (long long)H * dk * dv);
    GDN_EXTENTS(N, 1, 3 * H * (2 * dk + dv), 0, 0);
    const int hC = H * (2 * dk + dv);
    {
        const size_t hb = (size_t)N * 3 * hC * (x_dtype == GDN_BF16 ? 2 : 4);
        const char* i0 = static_cast<const char*>(conv_state_in);
        const char* o0 = static_cast<const char*>(conv_state_out);
        GDN_REQUIRE(i0 == o0 || i0 + hb <= o0 || o0 + hb <= i0, GDN_ERR_SHAPE,
                    "conv_state_in and conv_state_out must be the same buffer or not overlap");
    }
    if (step_states) {
        const char* a0 = reinterpret_cast<const char*>(state);
        const char* b0 = reinterpret_cast<const char*>(step_states);
        const size_t sb = (size_t)N * H * dk * dv * sizeof(float);
        GDN_REQUIRE(a0 + sb <= b0 || b0 + sb * T <= a0, GDN_ERR_SHAPE,
                    "step_states must not overlap state");
    }
    gdn::DecodeFusedArgs f;
    f.x[0] = xq; f.x[1] = xk; f.x[2] = xv;
    f.w[0] = wq; f.w[1] = wk; f.w[2] = wv;
    f.conv_state = conv_state_out;
    f.hC = hC;
    f.a_raw = a_raw; f.b_raw = b_raw; f.A_log = A_log; f.dt_bias = dt_bias;
    f.l2_eps = l2_eps;
    f.state = state; f.z = z; f.norm_w = norm_weight; f.rms_eps = rms_eps;
    f.o = o; f.y = y;
    f.N = N; f.H = H;
    f.in_bf16 = x_dtype == GDN_BF16;
    f.out_bf16 = o_dtype == GDN_BF16;
    return hip_status(gdn::launch_decode_fused_multi(f, conv_state_in, T, step_states, dk, dv,
                                                     static_cast<hipStream_t>(stream)),
                      "gdn_fused_decode_multi");
}

int gdn_output_gate(const void* y, int y_dtype, const void* z, int z_dtype, const float* norm_weight,
                    int ntok, int H, int dv, float eps, void* o, int o_dtype, void* stream) {
    GDN_REQUIRE(valid_dtype(y_dtype) && valid_dtype(z_dtype) && valid_dtype(o_dtype), GDN_ERR_DTYPE,
                "y_dtype/z_dtype/o_dtype must be GDN_F32 or GDN_BF16");
    GDN_REQUIRE(ntok >= 0 && H >= 1 && valid_dim(dv), GDN_ERR_SHAPE,
                "need ntok >= 0, H >= 1 and dv in {64, 128} (got ntok=%d H=%d dv=%d)", ntok, H, dv);
    GDN_REQUIRE(eps >= 0.f, GDN_ERR_SHAPE, "eps must be >= 0");
    GDN_TPTR(y, ntok); GDN_TPTR(z, ntok); GDN_SPTR(norm_weight); GDN_TPTR(o, ntok);
    GDN_EXTENTS(ntok, H, dv, 0, 0);
    return hip_status(gdn::launch_output_gate(y, y_dtype == GDN_BF16, z, z_dtype == GDN_BF16,
                                              norm_weight, ntok, H, dv, eps, o,
                                              o_dtype == GDN_BF16, static_cast<hipStream_t>(stream)),
                      "gdn_output_gate");
}

int gdn_mb_stream(const void* src, void* dst, size_t bytes, void* stream) {
    GDN_REQUIRE(bytes % 16 == 0, GDN_ERR_SHAPE, "bytes must be a multiple of 16 (got %zu)", bytes);
    if (bytes > 0) {
        GDN_PTR(src);
        GDN_PTR(dst);
        const char* a0 = static_cast<const char*>(src);
        const char* b0 = static_cast<const char*>(dst);
        GDN_REQUIRE(a0 == b0 || a0 + bytes <= b0 || b0 + bytes <= a0, GDN_ERR_SHAPE,
                    "src and dst must be the same buffer or not overlap");
    }
    return hip_status(gdn::launch_mb_stream(src, dst, bytes, static_cast<hipStream_t>(stream)),
                      "gdn_mb_stream");
}

int gdn_mb_mfma_bf16(float* sink, int workgroups, int iters, void* stream) {
    GDN_REQUIRE(workgroups >= 0 && iters >= 1, GDN_ERR_SHAPE,
                "need workgroups >= 0 and iters >= 1 (got %d, %d)", workgroups, iters);
    if (workgroups > 0) GDN_SPTR(sink);
    return hip_status(gdn::launch_mb_mfma(sink, workgroups, iters, static_cast<hipStream_t>(stream)),
                      "gdn_mb_mfma_bf16");
}

}  // extern "C"
