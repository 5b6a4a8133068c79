// All-fp32 chunkwise gated delta rule on gfx950 (vector ALU; no matrix cores).
//
// Reading notes of "On the Design of Qwen3.8-Next Architecture", section 2.1.1: eqs. (1)-(4)
// token by token are re-associated into chunks of C = 64 tokens by unrolling eq. (5) inside
// a chunk. With G_r the running sum of g = log(alpha) in the chunk, gamma_r = exp(G_r),
//   A[r,i] = beta_r e^{G_r-G_i} (k_r . k_i)  (i < r),     (I + A) U = diag(beta) V - diag(beta gamma) K S
//   Y      = diag(gamma) Q S + (M o Q K^T) U,             M[r,i] = e^{G_r-G_i} (i <= r)
//   S_next = gamma_C S + (diag(gamma_C / gamma) K)^T U
// Columns of S, V, U and Y are independent given (Q, K, beta, G), so each workgroup owns one
// (sequence, head, 32-column slice of dv). This path serves fp32 inputs, whose tolerance is
// beyond bf16 matrix-core products; it favours plain, exact fp32 arithmetic over speed.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kC = 64;            // chunk length
constexpr int kF32Threads = 256;
constexpr int kF32Slice = 32;     // dv columns per workgroup

// Sequence bounds of packed sequence s.
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int num_seqs, int ntok, int s, int& lo,
                                           int& hi) {
    if (cu) {
        lo = cu[s];
        hi = cu[s + 1];
    } else {
        const int L = ntok / num_seqs;
        lo = s * L;
        hi = lo + L;
    }
}

template <int DK, typename Tin, typename Tout>
__global__ void __launch_bounds__(kF32Threads) chunk_fp32_kernel(ChunkArgs p) {
    constexpr int SL = kF32Slice;
    __shared__ float Ks[kC][DK + 1];
    __shared__ float Qs[kC][DK + 1];
    __shared__ float S[DK][SL];
    __shared__ float Vs[kC][SL];
    __shared__ float A[kC][kC + 1];
    __shared__ float P[kC][kC + 1];
    __shared__ float U[kC][SL + 1];
    __shared__ float QSg[kC][SL];
    __shared__ float G[kC], Bt[kC];

    const int slices = p.dv / SL;
    const int slice = blockIdx.x % slices;
    const int h = (blockIdx.x / slices) % p.H;
    const int sq = blockIdx.x / (slices * p.H);
    const int j0 = slice * SL;
    const int tid = threadIdx.x;
    const Tin* q = static_cast<const Tin*>(p.q);
    const Tin* k = static_cast<const Tin*>(p.k);
    const Tin* v = static_cast<const Tin*>(p.v);
    Tout* y = static_cast<Tout*>(p.y);
    const int H = p.H, dv = p.dv;

    int lo, hi;
    seq_bounds(p.cu, p.num_seqs, p.ntok, sq, lo, hi);

    const size_t st_off = ((size_t)sq * H + h) * DK * dv;
    for (int e = tid; e < DK * SL; e += kF32Threads) {
        const int d = e / SL, j = e % SL;
        S[d][j] = p.S0 ? p.S0[st_off + (size_t)d * dv + j0 + j] : 0.f;
    }

    for (int t0 = lo; t0 < hi; t0 += kC) {
        const int n = min(kC, hi - t0);
        __syncthreads();   // previous chunk fully consumed
        for (int e = tid; e < kC * DK; e += kF32Threads) {
            const int r = e / DK, d = e % DK;
            const bool ok = r < n;
            const size_t off = ((size_t)(t0 + r) * H + h) * DK + d;
            Ks[r][d] = ok ? load1(k + off) : 0.f;
            Qs[r][d] = ok ? load1(q + off) : 0.f;
        }
        for (int e = tid; e < kC * SL; e += kF32Threads) {
            const int r = e / SL, j = e % SL;
            Vs[r][j] = r < n ? load1(v + ((size_t)(t0 + r) * H + h) * dv + j0 + j) : 0.f;
        }
        if (tid < kC) {
            const bool ok = tid < n;
            G[tid] = ok ? p.g[(size_t)(t0 + tid) * H + h] : 0.f;
            Bt[tid] = ok ? p.beta[(size_t)(t0 + tid) * H + h] : 0.f;
        }
        __syncthreads();
        if (tid == 0) {   // running sum of the log-decay
            float acc = 0.f;
            for (int r = 0; r < kC; ++r) {
                acc += G[r];
                G[r] = acc;
            }
        }
        __syncthreads();
        // A (strictly lower) and P (lower incl. diagonal)
        for (int e = tid; e < kC * kC; e += kF32Threads) {
            const int r = e / kC, i = e % kC;
            float a = 0.f, pq = 0.f;
            if (i <= r) {
                float kk = 0.f, qk = 0.f;
                for (int d = 0; d < DK; ++d) {
                    kk += Ks[r][d] * Ks[i][d];
                    qk += Qs[r][d] * Ks[i][d];
                }
                const float dec = expf(G[r] - G[i]);
                pq = dec * qk;
                if (i < r) a = Bt[r] * dec * kk;
            }
            A[r][i] = a;
            P[r][i] = pq;
        }
        // right-hand side and the S-part of the output
        for (int e = tid; e < kC * SL; e += kF32Threads) {
            const int r = e / SL, j = e % SL;
            float ks = 0.f, qs = 0.f;
            for (int d = 0; d < DK; ++d) {
                ks += Ks[r][d] * S[d][j];
                qs += Qs[r][d] * S[d][j];
            }
            const float gam = expf(G[r]);
            U[r][j] = Bt[r] * (Vs[r][j] - gam * ks);
            QSg[r][j] = gam * qs;
        }
        __syncthreads();
        // forward substitution (I + A) U = R, one column per thread
        if (tid < SL) {
            for (int r = 1; r < kC; ++r) {
                float acc = U[r][tid];
                for (int i = 0; i < r; ++i) acc -= A[r][i] * U[i][tid];
                U[r][tid] = acc;
            }
        }
        __syncthreads();
        // outputs of the chunk
        for (int e = tid; e < kC * SL; e += kF32Threads) {
            const int r = e / SL, j = e % SL;
            if (r < n) {
                float acc = QSg[r][j];
                for (int i = 0; i <= r; ++i) acc += P[r][i] * U[i][j];
                store1(y + ((size_t)(t0 + r) * H + h) * dv + j0 + j, acc);
            }
        }
        // state to the end of the chunk
        const float gC = G[kC - 1];
        for (int e = tid; e < DK * SL; e += kF32Threads) {
            const int d = e / SL, j = e % SL;
            float acc = 0.f;
            for (int i = 0; i < kC; ++i) acc += expf(gC - G[i]) * Ks[i][d] * U[i][j];
            S[d][j] = expf(gC) * S[d][j] + acc;
        }
    }
    __syncthreads();
    if (p.ST) {
        for (int e = tid; e < DK * SL; e += kF32Threads) {
            const int d = e / SL, j = e % SL;
            p.ST[st_off + (size_t)d * dv + j0 + j] = S[d][j];
        }
    }
}

hipError_t launch_chunk_fp32(const ChunkArgs& a, hipStream_t s) {
    const int blocks = a.num_seqs * a.H * (a.dv / kF32Slice);
    if (blocks == 0) return hipSuccess;
#define GDN_F32(DK, TI, TO) \
    hipLaunchKernelGGL((chunk_fp32_kernel<DK, TI, TO>), dim3(blocks), dim3(kF32Threads), 0, s, a)
    if (a.dk == 128) {
        if (a.in_bf16 && a.y_bf16) GDN_F32(128, uint16_t, uint16_t);
        else if (a.in_bf16) GDN_F32(128, uint16_t, float);
        else if (a.y_bf16) GDN_F32(128, float, uint16_t);
        else GDN_F32(128, float, float);
    } else {
        if (a.in_bf16 && a.y_bf16) GDN_F32(64, uint16_t, uint16_t);
        else if (a.in_bf16) GDN_F32(64, uint16_t, float);
        else if (a.y_bf16) GDN_F32(64, float, uint16_t);
        else GDN_F32(64, float, float);
    }
#undef GDN_F32
    return hipGetLastError();
}

}  // namespace gdn
