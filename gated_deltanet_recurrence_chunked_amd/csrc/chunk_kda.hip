// Chunkwise delta rule with a per-channel (diagonal) decay on gfx950: the KDA-style variant
// of the Gated DeltaNet recurrence (fp32 vector ALU).
//
// The reading notes of "On the Design of Qwen3.8-Next Architecture" compare GDN with Kimi K3's
// Kimi Delta Attention (related work), whose decay is per channel with a lower-bounded log-decay.
// Reading: eq. (1)'s scalar alpha_t becomes Diag(alpha_t) over the key channels, so row c of the
// state decays by alpha_t[c]. Within a chunk of C = 64 tokens, with Gc[r][c] the running sum of
// g = log(alpha) per channel:
//   A[r,i] = beta_r sum_c k_r[c] k_i[c] e^{Gc[r][c]-Gc[i][c]}  (i < r),  T = (I + A)^{-1}
//   P[r,i] = sum_c q_r[c] k_i[c] e^{Gc[r][c]-Gc[i][c]}          (i <= r)
//   U = T (beta o (V - Kg S)),  Y = Qg S + P U,  S' = e^{Gc[C]} o S + Kc^T U
// with Kg = K o e^{Gc}, Qg = Q o e^{Gc} and Kc = K o e^{Gc[C] - Gc} (every exponent <= 0).
// Two kernels: a per-(chunk, head) prep forms T, P, Kg, Qg, Kc and e^{Gc[C]} into the
// workspace (the pair decays are exponentials of differences, element by element, so no
// factor can overflow); a scan per (sequence, head, 16-column slice of dv) then needs plain
// products only.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;
constexpr int kPT = 512;          // prep threads (one workgroup per CU fits its LDS)
constexpr int kST = 1024;         // scan threads: 16 waves hide the LDS latency of the small products
constexpr int kSL = 16;           // dv columns per scan workgroup

struct KdaLayout {
    size_t T, P, Kg, Qg, Kc, eC, total;
    int max_chunks;
};

KdaLayout kda_layout(int ntok, int num_seqs, int H, int dk) {
    KdaLayout L;
    L.max_chunks = (ntok + kC - 1) / kC + num_seqs;
    const size_t ch = (size_t)L.max_chunks * H;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    L.T = take(ch * kC * kC * sizeof(float));
    L.P = take(ch * kC * kC * sizeof(float));
    L.Kg = take(ch * kC * (size_t)dk * sizeof(float));
    L.Qg = take(ch * kC * (size_t)dk * sizeof(float));
    L.Kc = take(ch * kC * (size_t)dk * sizeof(float));
    L.eC = take(ch * (size_t)dk * sizeof(float));
    L.total = off;
    return L;
}

struct KdaArgs {
    const void *q, *k, *v;
    int in_bf16;
    const float *g, *beta, *S0;   // g: [ntok, H, dk]
    float* ST;
    const int32_t* cu;
    int num_seqs, ntok, H, dk, dv;
    void* y;
    float *T, *P, *Kg, *Qg, *Kc, *eC;
};

__device__ void kda_seq(const KdaArgs& a, int s, int& lo, int& hi, int& cbase) {
    if (a.cu) {
        lo = a.cu[s];
        hi = a.cu[s + 1];
        cbase = 0;
        for (int i = 0; i < s; ++i) cbase += (a.cu[i + 1] - a.cu[i] + kC - 1) / kC;
    } else {
        const int L = a.ntok / a.num_seqs;
        lo = s * L;
        hi = lo + L;
        cbase = s * ((L + kC - 1) / kC);
    }
}

__device__ bool kda_chunk(const KdaArgs& a, int c, int& t0, int& n) {
    int base = 0;
    for (int s = 0; s < a.num_seqs; ++s) {
        int lo, hi, cb;
        kda_seq(a, s, lo, hi, cb);
        const int nc = (hi - lo + kC - 1) / kC;
        if (c < base + nc) {
            t0 = lo + (c - base) * kC;
            n = min(kC, hi - t0);
            return true;
        }
        base += nc;
    }
    return false;
}

template <typename T>
__device__ __forceinline__ float ldx(const void* p, size_t i) {
    return load1(static_cast<const T*>(p) + i);
}

// ------------------------------------------------------------------ prep per chunk-head
template <int DK, typename Tin>
__global__ void __launch_bounds__(kPT) kda_prep_kernel(KdaArgs a) {
    __shared__ float Ks[kC][DK + 1], Qs[kC][DK + 1], Gc[kC][DK + 1];
    __shared__ float A[kC][kC + 1];
    __shared__ float Bt[kC];
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, H = a.H;
    int t0, n;
    if (!kda_chunk(a, c, t0, n)) return;
    for (int e = tid; e < kC * DK; e += kPT) {
        const int r = e / DK, d = e % DK;
        const bool ok = r < n;
        const size_t off = ((size_t)(t0 + r) * H + h) * DK + d;
        Ks[r][d] = ok ? ldx<Tin>(a.k, off) : 0.f;
        Qs[r][d] = ok ? ldx<Tin>(a.q, off) : 0.f;
        Gc[r][d] = ok ? a.g[off] : 0.f;
    }
    if (tid < kC) Bt[tid] = tid < n ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
    __syncthreads();
    if (tid < DK) {   // running sum per channel (tokens past n add zero)
        float acc = 0.f;
        for (int r = 0; r < kC; ++r) {
            acc += Gc[r][tid];
            Gc[r][tid] = acc;
        }
    }
    __syncthreads();
    const size_t ch = (size_t)c * H + h;
    // A (strictly lower) and P (lower with the diagonal): decays per channel and pair
    for (int e = tid; e < kC * kC; e += kPT) {
        const int r = e / kC, i = e % kC;
        float kk = 0.f, qk = 0.f;
        if (i <= r && r < n) {
            for (int d = 0; d < DK; ++d) {
                const float dec = fexp(Gc[r][d] - Gc[i][d]);
                kk += Ks[r][d] * Ks[i][d] * dec;
                qk += Qs[r][d] * Ks[i][d] * dec;
            }
        }
        A[r][i] = i < r ? Bt[r] * kk : 0.f;
        a.P[ch * kC * kC + e] = qk;
    }
    // decayed operands of the scan
    const int last = n - 1;
    for (int e = tid; e < kC * DK; e += kPT) {
        const int r = e / DK, d = e % DK;
        const size_t o = ch * kC * DK + e;
        const bool ok = r < n;
        a.Kg[o] = ok ? Ks[r][d] * fexp(Gc[r][d]) : 0.f;
        a.Qg[o] = ok ? Qs[r][d] * fexp(Gc[r][d]) : 0.f;
        a.Kc[o] = ok ? Ks[r][d] * fexp(Gc[last][d] - Gc[r][d]) : 0.f;
    }
    if (tid < DK) a.eC[ch * DK + tid] = fexp(Gc[last][tid]);
    __syncthreads();
    // T = (I + A)^{-1}, one column per lane, forward substitution unrolled in registers
    if (tid < kC) {
        float x[kC];
#pragma unroll
        for (int r = 0; r < kC; ++r) {
            float acc = r == tid ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= A[r][i] * x[i];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < kC; ++r) a.T[ch * kC * kC + r * kC + tid] = x[r];
    }
}

// ------------------------------------------------------------------ scan per (seq, head, slice)
template <int DK, typename Tin, typename Tout>
__global__ void __launch_bounds__(kST) kda_scan_kernel(KdaArgs a) {
    __shared__ float Kg[kC][DK + 1], Qg[kC][DK + 1], Kc[kC][DK + 1];
    __shared__ float T[kC][kC + 1], P[kC][kC + 1];
    __shared__ float S[DK][kSL];
    __shared__ float R[kC][kSL + 1], U[kC][kSL + 1];
    __shared__ float eC[DK], Bt[kC];
    const int slices = a.dv / kSL;
    const int slice = blockIdx.x % slices;
    const int h = (blockIdx.x / slices) % a.H;
    const int sq = blockIdx.x / (slices * a.H);
    const int j0 = slice * kSL, tid = threadIdx.x, H = a.H, dv = a.dv;
    Tout* y = static_cast<Tout*>(a.y);
    int lo, hi, cbase;
    kda_seq(a, sq, lo, hi, cbase);
    const size_t st_off = ((size_t)sq * H + h) * DK * dv;
    for (int e = tid; e < DK * kSL; e += kST) {
        const int d = e / kSL, j = e % kSL;
        S[d][j] = a.S0 ? a.S0[st_off + (size_t)d * dv + j0 + j] : 0.f;
    }
    for (int t0 = lo, c = cbase; t0 < hi; t0 += kC, ++c) {
        const int n = min(kC, hi - t0);
        const size_t ch = (size_t)c * H + h;
        __syncthreads();
        for (int e = tid; e < kC * DK; e += kST) {
            const size_t o = ch * kC * DK + e;
            Kg[e / DK][e % DK] = a.Kg[o];
            Qg[e / DK][e % DK] = a.Qg[o];
            Kc[e / DK][e % DK] = a.Kc[o];
        }
        for (int e = tid; e < kC * kC; e += kST) {
            T[e / kC][e % kC] = a.T[ch * kC * kC + e];
            P[e / kC][e % kC] = a.P[ch * kC * kC + e];
        }
        if (tid < DK) eC[tid] = a.eC[ch * DK + tid];
        if (tid < kC) Bt[tid] = tid < n ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
        __syncthreads();
        for (int e = tid; e < kC * kSL; e += kST) {   // R = beta o (V - Kg S)
            const int r = e / kSL, j = e % kSL;
            float ks = 0.f;
#pragma unroll 4
            for (int d = 0; d < DK; ++d) ks += Kg[r][d] * S[d][j];
            const float vr = r < n ? ldx<Tin>(a.v, ((size_t)(t0 + r) * H + h) * dv + j0 + j) : 0.f;
            R[r][j] = Bt[r] * (vr - ks);
        }
        __syncthreads();
        for (int e = tid; e < kC * kSL; e += kST) {   // U = T R
            const int r = e / kSL, j = e % kSL;
            float u = 0.f;
            for (int i = 0; i <= r; ++i) u += T[r][i] * R[i][j];
            U[r][j] = u;
        }
        __syncthreads();
        for (int e = tid; e < kC * kSL; e += kST) {   // Y = Qg S + P U
            const int r = e / kSL, j = e % kSL;
            if (r < n) {
                float acc = 0.f;
#pragma unroll 4
                for (int d = 0; d < DK; ++d) acc += Qg[r][d] * S[d][j];
                for (int i = 0; i <= r; ++i) acc += P[r][i] * U[i][j];
                store1(y + ((size_t)(t0 + r) * H + h) * dv + j0 + j, acc);
            }
        }
        __syncthreads();   // Y read S before it moves on
        for (int e = tid; e < DK * kSL; e += kST) {   // S' = e^{Gc[C]} o S + Kc^T U
            const int d = e / kSL, j = e % kSL;
            float acc = 0.f;
            for (int i = 0; i < n; ++i) acc += Kc[i][d] * U[i][j];
            S[d][j] = eC[d] * S[d][j] + acc;
        }
    }
    __syncthreads();
    if (a.ST) {
        for (int e = tid; e < DK * kSL; e += kST) {
            const int d = e / kSL, j = e % kSL;
            a.ST[st_off + (size_t)d * dv + j0 + j] = S[d][j];
        }
    }
}

}  // namespace

size_t chunk_kda_workspace(int ntok, int num_seqs, int H, int dk) {
    return kda_layout(ntok, num_seqs, H, dk).total;
}

hipError_t launch_chunk_kda(const ChunkKdaArgs& c, hipStream_t s) {
    const KdaLayout L = kda_layout(c.ntok, c.num_seqs, c.H, c.dk);
    char* ws = static_cast<char*>(c.workspace);
    KdaArgs a;
    a.q = c.q; a.k = c.k; a.v = c.v; a.in_bf16 = c.in_bf16;
    a.g = c.g; a.beta = c.beta; a.S0 = c.S0; a.ST = c.ST; a.cu = c.cu;
    a.num_seqs = c.num_seqs; a.ntok = c.ntok; a.H = c.H; a.dk = c.dk; a.dv = c.dv;
    a.y = c.y;
    a.T = reinterpret_cast<float*>(ws + L.T);
    a.P = reinterpret_cast<float*>(ws + L.P);
    a.Kg = reinterpret_cast<float*>(ws + L.Kg);
    a.Qg = reinterpret_cast<float*>(ws + L.Qg);
    a.Kc = reinterpret_cast<float*>(ws + L.Kc);
    a.eC = reinterpret_cast<float*>(ws + L.eC);
    const int nchunks = c.cu ? L.max_chunks : c.num_seqs * ((c.ntok / c.num_seqs + kC - 1) / kC);
    const int blocks = c.num_seqs * c.H * (c.dv / kSL);
    if (blocks == 0) return hipSuccess;
#define GDN_KDA(DK, TI, TO)                                                                      \
    do {                                                                                         \
        if (nchunks > 0)                                                                         \
            hipLaunchKernelGGL((kda_prep_kernel<DK, TI>), dim3(nchunks, c.H), dim3(kPT), 0, s, a); \
        hipLaunchKernelGGL((kda_scan_kernel<DK, TI, TO>), dim3(blocks), dim3(kST), 0, s, a);     \
    } while (0)
    if (c.dk == 128) {
        if (c.in_bf16 && c.y_bf16) GDN_KDA(128, uint16_t, uint16_t);
        else if (c.in_bf16) GDN_KDA(128, uint16_t, float);
        else if (c.y_bf16) GDN_KDA(128, float, uint16_t);
        else GDN_KDA(128, float, float);
    } else {
        if (c.in_bf16 && c.y_bf16) GDN_KDA(64, uint16_t, uint16_t);
        else if (c.in_bf16) GDN_KDA(64, uint16_t, float);
        else if (c.y_bf16) GDN_KDA(64, float, uint16_t);
        else GDN_KDA(64, float, float);
    }
#undef GDN_KDA
    return hipGetLastError();
}

}  // namespace gdn
