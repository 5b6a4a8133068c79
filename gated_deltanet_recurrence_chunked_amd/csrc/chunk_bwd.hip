// Backward pass of the chunkwise gated delta rule on gfx950 (fp32 vector ALU).
//
// Reading notes of "On the Design of Qwen3.8-Next Architecture", section 2.1.1, eqs. (1)-(5):
// the gradients of y and S_T with respect to q, k, v, g = log(alpha), beta and S0. Per chunk of
// C = 64 tokens the forward is (G the running sum of g inside the chunk, gamma = e^G,
// w_r = e^{G_C - G_r}):
//   A[r,i] = beta_r e^{G_r-G_i} k_r.k_i (i < r),  P[r,i] = e^{G_r-G_i} q_r.k_i (i <= r)
//   KS = K S,  R = beta o (V - gamma o KS),  (I + A) U = R,  W = w o U
//   Y = gamma o (Q S) + P U,  S' = gamma_C S + K^T W
// and the backward takes the adjoints of these products in reverse order, chunk by chunk
// from the last, carrying dS (the gradient of the state entering a chunk):
//   dW = K dS',  dU = w o dW + P^T dY,  (I + A)^T dR = dU,  dV = beta o dR,
//   dKS = -(beta gamma) o dR,  dS = gamma_C dS' + Q^T (gamma o dY) + K^T dKS,
//   dA = -(dR U^T) strictly lower,  dP = (dY U^T) lower,
// plus the q, k, beta and gate terms collected below.
//
// Four kernels:
//   ap     per (chunk, head): G, A and P of the chunk (fp32 workspace);
//   states per (sequence, head, 16-column slice of dv): the forward sweep, storing the state at
//          every chunk start;
//   scan   per (sequence, head, slice): the reverse sweep; writes dv and dS0 for its columns
//          and, per chunk, this slice's share of the terms that sum over dv columns
//          (dq, dk partials, dA, dP, and the per-token sums feeding dbeta and dg);
//   finish per (chunk, head): sums the slices' shares and adds the A and P terms.
// Columns of dv are independent in the state recursion (as in the forward), which is what the
// slices use; the terms that mix columns are sums over them, so slice shares add up.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;
constexpr int kBT = 256;          // threads per workgroup
constexpr int kSL = 16;           // dv columns per scan workgroup

struct BwdLayout {
    size_t G, A, P, Sc, part, total;
    int max_chunks;
};

// per-(chunk, head, slice) share: dq part, dk part [64][dk], dA, dP [64][64], and 4 token
// vectors: sum_j dR (V - gamma KS), dgamma, dw, and dgamma_C (one value, in slot 0)
__host__ __device__ inline size_t part_floats(int dk) { return (size_t)2 * kC * dk + 2 * kC * kC + 4 * kC; }

BwdLayout bwd_layout(int ntok, int num_seqs, int H, int dk, int dv) {
    BwdLayout L;
    L.max_chunks = (ntok + kC - 1) / kC + num_seqs;
    const size_t ch = (size_t)L.max_chunks * H;
    const int slices = dv / kSL;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    L.G = take(ch * kC * sizeof(float));
    L.A = take(ch * kC * kC * sizeof(float));
    L.P = take(ch * kC * kC * sizeof(float));
    L.Sc = take(ch * (size_t)dk * dv * sizeof(float));
    L.part = take(ch * slices * part_floats(dk) * sizeof(float));
    L.total = off;
    return L;
}

struct BwdArgs {
    const void *q, *k, *v, *dy;
    int in_bf16, dy_bf16;
    const float *g, *beta, *S0, *dST;
    const int32_t* cu;
    int num_seqs, ntok, H, dk, dv;
    float *dq, *dk_, *dv_, *dg, *dbeta, *dS0;
    float *G, *A, *P, *Sc, *part;
};

// bounds of sequence s and its first chunk's index in the packed chunk numbering
__device__ void seq_info(const BwdArgs& a, int s, int& lo, int& hi, int& cbase) {
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

// (chunk index, head) of a chunk-head workgroup -> sequence and token range; false if the
// packed chunk index is past the last chunk
__device__ bool chunk_info(const BwdArgs& a, int c, int& t0, int& n) {
    int base = 0;
    for (int s = 0; s < a.num_seqs; ++s) {
        int lo, hi;
        if (a.cu) {
            lo = a.cu[s];
            hi = a.cu[s + 1];
        } else {
            const int L = a.ntok / a.num_seqs;
            lo = s * L;
            hi = lo + L;
        }
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
__device__ __forceinline__ float ld(const void* p, size_t i) {
    return load1(static_cast<const T*>(p) + i);
}

// ------------------------------------------------------------------ ap: G, A, P per chunk-head
template <int DK, typename Tin>
__global__ void __launch_bounds__(kBT) bwd_ap_kernel(BwdArgs a) {
    __shared__ float Ks[kC][DK + 1], Qs[kC][DK + 1];
    __shared__ float G[kC], Bt[kC];
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int t0, n;
    if (!chunk_info(a, c, t0, n)) return;
    const int H = a.H;
    for (int e = tid; e < kC * DK; e += kBT) {
        const int r = e / DK, d = e % DK;
        const bool ok = r < n;
        const size_t off = ((size_t)(t0 + r) * H + h) * DK + d;
        Ks[r][d] = ok ? ld<Tin>(a.k, off) : 0.f;
        Qs[r][d] = ok ? ld<Tin>(a.q, off) : 0.f;
    }
    if (tid < kC) {
        G[tid] = tid < n ? a.g[(size_t)(t0 + tid) * H + h] : 0.f;
        Bt[tid] = tid < n ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
        float acc = 0.f;
        for (int r = 0; r < kC; ++r) {
            acc += G[r];
            G[r] = acc;
        }
    }
    __syncthreads();
    const size_t ch = (size_t)c * H + h;
    if (tid < kC) a.G[ch * kC + tid] = G[tid];
    for (int e = tid; e < kC * kC; e += kBT) {
        const int r = e / kC, i = e % kC;
        float av = 0.f, pv = 0.f;
        if (i <= r && r < n) {
            float kk = 0.f, qk = 0.f;
            for (int d = 0; d < DK; ++d) {
                kk += Ks[r][d] * Ks[i][d];
                qk += Qs[r][d] * Ks[i][d];
            }
            const float dec = expf(G[r] - G[i]);
            pv = dec * qk;
            if (i < r) av = Bt[r] * dec * kk;
        }
        a.A[ch * kC * kC + e] = av;
        a.P[ch * kC * kC + e] = pv;
    }
}

// ------------------------------------------------------------------ states: forward sweep
template <int DK, typename Tin>
__global__ void __launch_bounds__(kBT) bwd_states_kernel(BwdArgs a) {
    __shared__ float Ks[kC][DK + 1];
    __shared__ float S[DK][kSL];
    __shared__ float A[kC][kC + 1];
    __shared__ float U[kC][kSL + 1];
    __shared__ float G[kC], Bt[kC];
    const int slices = a.dv / kSL;
    const int slice = blockIdx.x % slices;
    const int h = (blockIdx.x / slices) % a.H;
    const int sq = blockIdx.x / (slices * a.H);
    const int j0 = slice * kSL, tid = threadIdx.x, H = a.H, dv = a.dv;
    int lo, hi, cbase;
    seq_info(a, sq, lo, hi, cbase);
    const size_t st_off = ((size_t)sq * H + h) * DK * dv;
    for (int e = tid; e < DK * kSL; e += kBT) {
        const int d = e / kSL, j = e % kSL;
        S[d][j] = a.S0 ? a.S0[st_off + (size_t)d * dv + j0 + j] : 0.f;
    }
    for (int t0 = lo, c = cbase; t0 < hi; t0 += kC, ++c) {
        const int n = min(kC, hi - t0);
        const size_t ch = (size_t)c * H + h;
        __syncthreads();
        for (int e = tid; e < DK * kSL; e += kBT) {   // the state entering this chunk
            const int d = e / kSL, j = e % kSL;
            a.Sc[ch * DK * dv + (size_t)d * dv + j0 + j] = S[d][j];
        }
        for (int e = tid; e < kC * DK; e += kBT) {
            const int r = e / DK, d = e % DK;
            Ks[r][d] = r < n ? ld<Tin>(a.k, ((size_t)(t0 + r) * H + h) * DK + d) : 0.f;
        }
        for (int e = tid; e < kC * kC; e += kBT) A[e / kC][e % kC] = a.A[ch * kC * kC + e];
        if (tid < kC) {
            G[tid] = a.G[ch * kC + tid];
            Bt[tid] = tid < n ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < kC * kSL; e += kBT) {   // R = beta (V - gamma K S)
            const int r = e / kSL, j = e % kSL;
            float ks = 0.f;
            for (int d = 0; d < DK; ++d) ks += Ks[r][d] * S[d][j];
            const float vr = r < n ? ld<Tin>(a.v, ((size_t)(t0 + r) * H + h) * dv + j0 + j) : 0.f;
            U[r][j] = Bt[r] * (vr - expf(G[r]) * ks);
        }
        __syncthreads();
        if (tid < kSL) {   // (I + A) U = R
            for (int r = 1; r < n; ++r) {
                float acc = U[r][tid];
                for (int i = 0; i < r; ++i) acc -= A[r][i] * U[i][tid];
                U[r][tid] = acc;
            }
        }
        __syncthreads();
        const float gC = G[n - 1];
        for (int e = tid; e < DK * kSL; e += kBT) {   // S' = gamma_C S + K^T (w o U)
            const int d = e / kSL, j = e % kSL;
            float acc = 0.f;
            for (int i = 0; i < n; ++i) acc += expf(gC - G[i]) * Ks[i][d] * U[i][j];
            S[d][j] = expf(gC) * S[d][j] + acc;
        }
    }
}

// ------------------------------------------------------------------ scan: reverse sweep
template <int DK, typename Tin, typename Tdy>
__global__ void __launch_bounds__(kBT) bwd_scan_kernel(BwdArgs a) {
    __shared__ float Ks[kC][DK + 1], Qs[kC][DK + 1];
    __shared__ float S[DK][kSL], dS[DK][kSL];        // state entering the chunk; its gradient after
    __shared__ float Vs[kC][kSL + 1], dY[kC][kSL + 1];
    __shared__ float A[kC][kC + 1], P[kC][kC + 1];
    __shared__ float U[kC][kSL + 1], KS[kC][kSL + 1], dR[kC][kSL + 1];
    __shared__ float G[kC], Bt[kC], gam[kC], w[kC];
    __shared__ float red[kBT];

    const int slices = a.dv / kSL;
    const int slice = blockIdx.x % slices;
    const int h = (blockIdx.x / slices) % a.H;
    const int sq = blockIdx.x / (slices * a.H);
    const int j0 = slice * kSL, tid = threadIdx.x, H = a.H, dv = a.dv;
    int lo, hi, cbase;
    seq_info(a, sq, lo, hi, cbase);
    const int nch = (hi - lo + kC - 1) / kC;
    const size_t st_off = ((size_t)sq * H + h) * DK * dv;
    for (int e = tid; e < DK * kSL; e += kBT) {
        const int d = e / kSL, j = e % kSL;
        dS[d][j] = a.dST ? a.dST[st_off + (size_t)d * dv + j0 + j] : 0.f;
    }
    for (int cc = nch - 1; cc >= 0; --cc) {
        const int t0 = lo + cc * kC, n = min(kC, hi - t0);
        const size_t ch = (size_t)(cbase + cc) * H + h;
        float* part = a.part + (ch * slices + slice) * part_floats(DK);
        float* pdq = part;                         // [64][DK]
        float* pdk = part + kC * DK;               // [64][DK]
        float* pdA = part + 2 * kC * DK;           // [64][64]
        float* pdP = pdA + kC * kC;                // [64][64]
        float* pvec = pdP + kC * kC;               // [4][64]
        __syncthreads();
        for (int e = tid; e < kC * DK; e += kBT) {
            const int r = e / DK, d = e % DK;
            const bool ok = r < n;
            const size_t off = ((size_t)(t0 + r) * H + h) * DK + d;
            Ks[r][d] = ok ? ld<Tin>(a.k, off) : 0.f;
            Qs[r][d] = ok ? ld<Tin>(a.q, off) : 0.f;
        }
        for (int e = tid; e < kC * kSL; e += kBT) {
            const int r = e / kSL, j = e % kSL;
            const bool ok = r < n;
            const size_t off = ((size_t)(t0 + r) * H + h) * dv + j0 + j;
            Vs[r][j] = ok ? ld<Tin>(a.v, off) : 0.f;
            dY[r][j] = ok ? ld<Tdy>(a.dy, off) : 0.f;
        }
        for (int e = tid; e < DK * kSL; e += kBT) {
            const int d = e / kSL, j = e % kSL;
            S[d][j] = a.Sc[ch * DK * dv + (size_t)d * dv + j0 + j];
        }
        for (int e = tid; e < kC * kC; e += kBT) {
            A[e / kC][e % kC] = a.A[ch * kC * kC + e];
            P[e / kC][e % kC] = a.P[ch * kC * kC + e];
        }
        if (tid < kC) G[tid] = a.G[ch * kC + tid];
        __syncthreads();
        if (tid < kC) {
            Bt[tid] = tid < n ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
            gam[tid] = expf(G[tid]);
            w[tid] = tid < n ? expf(G[n - 1] - G[tid]) : 0.f;
        }
        // dgamma_C share: <S, dS'>
        float sdot = 0.f;
        for (int e = tid; e < DK * kSL; e += kBT) sdot += S[e / kSL][e % kSL] * dS[e / kSL][e % kSL];
        red[tid] = sdot;
        __syncthreads();
        // KS = K S and R = beta (V - gamma KS)
        for (int e = tid; e < kC * kSL; e += kBT) {
            const int r = e / kSL, j = e % kSL;
            float ks = 0.f;
            for (int d = 0; d < DK; ++d) ks += Ks[r][d] * S[d][j];
            KS[r][j] = ks;
            U[r][j] = Bt[r] * (Vs[r][j] - gam[r] * ks);
        }
        if (tid == 0) {
            float acc = 0.f;
            for (int i = 0; i < kBT; ++i) acc += red[i];
            pvec[3 * kC] = acc;
        }
        __syncthreads();
        if (tid < kSL) {   // (I + A) U = R
            for (int r = 1; r < n; ++r) {
                float acc = U[r][tid];
                for (int i = 0; i < r; ++i) acc -= A[r][i] * U[i][tid];
                U[r][tid] = acc;
            }
        }
        __syncthreads();
        // dU = w o (K dS') + P^T dY  (into dR, solved in place below)
        for (int e = tid; e < kC * kSL; e += kBT) {
            const int r = e / kSL, j = e % kSL;
            float dw = 0.f;
            for (int d = 0; d < DK; ++d) dw += Ks[r][d] * dS[d][j];
            float pt = 0.f;
            for (int i = r; i < n; ++i) pt += P[i][r] * dY[i][j];
            dR[r][j] = w[r] * dw + pt;
        }
        __syncthreads();
        // per-token sums that need K dS' and QS: dw_r, dgamma (Q S part)
        if (tid < kC) {
            const int r = tid;
            float dwr = 0.f, dg1 = 0.f;
            if (r < n) {
                for (int j = 0; j < kSL; ++j) {
                    float kd = 0.f, qs = 0.f;
                    for (int d = 0; d < DK; ++d) {
                        kd += Ks[r][d] * dS[d][j];
                        qs += Qs[r][d] * S[d][j];
                    }
                    dwr += kd * U[r][j];
                    dg1 += dY[r][j] * qs;
                }
            }
            pvec[2 * kC + r] = dwr;
            pvec[1 * kC + r] = dg1;
        }
        // dk share, first part: W dS'^T (W = w o U), before dS is overwritten
        for (int e = tid; e < kC * DK; e += kBT) {
            const int r = e / DK, d = e % DK;
            float acc = 0.f;
            for (int j = 0; j < kSL; ++j) acc += U[r][j] * dS[d][j];
            pdk[e] = w[r] * acc;
        }
        __syncthreads();
        if (tid < kSL) {   // (I + A)^T dR = dU, from the last token back
            for (int r = n - 2; r >= 0; --r) {
                float acc = dR[r][tid];
                for (int i = r + 1; i < n; ++i) acc -= A[i][r] * dR[i][tid];
                dR[r][tid] = acc;
            }
        }
        __syncthreads();
        // dv (this slice's columns), and the per-token sums of dR
        for (int e = tid; e < kC * kSL; e += kBT) {
            const int r = e / kSL, j = e % kSL;
            if (r < n) a.dv_[((size_t)(t0 + r) * H + h) * dv + j0 + j] = Bt[r] * dR[r][j];
        }
        if (tid < kC) {
            const int r = tid;
            float db = 0.f, dg2 = 0.f;
            for (int j = 0; j < kSL; ++j) {
                db += dR[r][j] * (Vs[r][j] - gam[r] * KS[r][j]);
                dg2 += dR[r][j] * KS[r][j];
            }
            pvec[r] = db;
            pvec[kC + r] -= Bt[r] * dg2;
        }
        // dk share, second part: dKS S^T with dKS = -(beta gamma) o dR; dq share: gamma o (dY S^T)
        for (int e = tid; e < kC * DK; e += kBT) {
            const int r = e / DK, d = e % DK;
            float a1 = 0.f, a2 = 0.f;
            for (int j = 0; j < kSL; ++j) {
                a1 += dR[r][j] * S[d][j];
                a2 += dY[r][j] * S[d][j];
            }
            pdk[e] += -Bt[r] * gam[r] * a1;
            pdq[e] = gam[r] * a2;
        }
        // dA = -(dR U^T) strictly lower, dP = (dY U^T) lower
        for (int e = tid; e < kC * kC; e += kBT) {
            const int r = e / kC, i = e % kC;
            float da = 0.f, dp = 0.f;
            if (i <= r && r < n) {
                for (int j = 0; j < kSL; ++j) {
                    da += dR[r][j] * U[i][j];
                    dp += dY[r][j] * U[i][j];
                }
            }
            pdA[e] = i < r ? -da : 0.f;
            pdP[e] = dp;
        }
        __syncthreads();
        // dS = gamma_C dS' + Q^T (gamma o dY) - K^T ((beta gamma) o dR)
        const float gC = gam[n - 1];
        for (int e = tid; e < DK * kSL; e += kBT) {
            const int d = e / kSL, j = e % kSL;
            float acc = gC * dS[d][j];
            for (int r = 0; r < n; ++r)
                acc += Qs[r][d] * gam[r] * dY[r][j] - Ks[r][d] * Bt[r] * gam[r] * dR[r][j];
            dS[d][j] = acc;   // each element read and written by the same thread
        }
    }
    __syncthreads();
    if (a.dS0) {
        for (int e = tid; e < DK * kSL; e += kBT) {
            const int d = e / kSL, j = e % kSL;
            a.dS0[st_off + (size_t)d * dv + j0 + j] = dS[d][j];
        }
    }
}

// ------------------------------------------------------------------ finish per chunk-head
template <int DK, typename Tin>
__global__ void __launch_bounds__(kBT) bwd_finish_kernel(BwdArgs a) {
    __shared__ float Ks[kC][DK + 1], Qs[kC][DK + 1];
    __shared__ float dAe[kC][kC + 1], dQK[kC][kC + 1];   // dA o e^{D}, dP o e^{D}
    __shared__ float G[kC], Bt[kC], dG[kC], dgam[kC], dw[kC], dbs[kC];
    __shared__ float dgC;
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int t0, n;
    if (!chunk_info(a, c, t0, n)) return;
    const int H = a.H, slices = a.dv / kSL;
    const size_t ch = (size_t)c * H + h;
    for (int e = tid; e < kC * DK; e += kBT) {
        const int r = e / DK, d = e % DK;
        const bool ok = r < n;
        const size_t off = ((size_t)(t0 + r) * H + h) * DK + d;
        Ks[r][d] = ok ? ld<Tin>(a.k, off) : 0.f;
        Qs[r][d] = ok ? ld<Tin>(a.q, off) : 0.f;
    }
    if (tid < kC) {
        G[tid] = a.G[ch * kC + tid];
        Bt[tid] = tid < n ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
        float db = 0.f, dgm = 0.f, dww = 0.f;
        for (int s = 0; s < slices; ++s) {
            const float* pv = a.part + (ch * slices + s) * part_floats(DK) + 2 * kC * DK + 2 * kC * kC;
            db += pv[tid];
            dgm += pv[kC + tid];
            dww += pv[2 * kC + tid];
        }
        dbs[tid] = db;
        dgam[tid] = dgm;
        dw[tid] = dww;
        dG[tid] = 0.f;
    }
    if (tid == 0) {
        float s0 = 0.f;
        for (int s = 0; s < slices; ++s)
            s0 += a.part[(ch * slices + s) * part_floats(DK) + 2 * kC * DK + 2 * kC * kC + 3 * kC];
        dgC = s0;
    }
    __syncthreads();
    // dA, dP summed over slices, times the decay: dAe = dA o e^{D} (strict lower; the k_r.k_i
    // coefficient of A is beta_r dAe), dQK = dP o e^{D} (the q_r.k_i coefficient of P). Their
    // products with A and P feed dG through D = G_r - G_i.
    for (int e = tid; e < kC * kC; e += kBT) {
        const int r = e / kC, i = e % kC;
        float da = 0.f, dp = 0.f;
        for (int s = 0; s < slices; ++s) {
            const float* pp = a.part + (ch * slices + s) * part_floats(DK) + 2 * kC * DK;
            da += pp[e];
            dp += pp[kC * kC + e];
        }
        const float dec = (i <= r && r < n) ? expf(G[r] - G[i]) : 0.f;
        dAe[r][i] = i < r ? da * dec : 0.f;
        dQK[r][i] = dp * dec;
    }
    __syncthreads();
    // dbeta: sum_i dA[r,i] e^{D} k_r.k_i, and dD -> dG rows and columns
    if (tid < kC) {
        const int r = tid;
        float db = 0.f, dgr = 0.f, dgc = 0.f;
        if (r < n) {
            for (int i = 0; i < n; ++i) {
                float kk_ri = 0.f, kk_ir = 0.f, qk_ri = 0.f, qk_ir = 0.f;
                for (int d = 0; d < DK; ++d) {
                    kk_ri += Ks[r][d] * Ks[i][d];
                    qk_ri += Qs[r][d] * Ks[i][d];
                    qk_ir += Qs[i][d] * Ks[r][d];
                }
                kk_ir = kk_ri;
                // row r of dD: dA[r,i] A[r,i] + dP[r,i] P[r,i]
                dgr += Bt[r] * dAe[r][i] * kk_ri + dQK[r][i] * qk_ri;
                // column r of dD (entry [i,r])
                dgc += Bt[i] * dAe[i][r] * kk_ir + dQK[i][r] * qk_ir;
                db += dAe[r][i] * kk_ri;
            }
        }
        dbs[r] += db;
        dG[r] = dgr - dgc + dgam[r] * expf(G[r]) - dw[r] * (r < n ? expf(G[n - 1] - G[r]) : 0.f);
    }
    __syncthreads();
    if (tid == 0) {
        float s = dgC * expf(G[n - 1]);
        for (int r = 0; r < n; ++r) s += dw[r] * expf(G[n - 1] - G[r]);
        dG[n - 1] += s;
        float acc = 0.f;   // dg = reverse running sum of dG
        for (int r = n - 1; r >= 0; --r) {
            acc += dG[r];
            dG[r] = acc;
        }
    }
    __syncthreads();
    if (tid < n) {
        const size_t row = (size_t)(t0 + tid) * H + h;
        a.dg[row] = dG[tid];
        a.dbeta[row] = dbs[tid];
    }
    // dq = sum of shares + dQK K;  dk = sum of shares + (dKK + dKK^T) K + dQK^T Q with
    // dKK[r,i] = beta_r dAe[r,i]
    for (int e = tid; e < kC * DK; e += kBT) {
        const int r = e / DK, d = e % DK;
        if (r >= n) continue;
        float dq = 0.f, dk = 0.f;
        for (int s = 0; s < slices; ++s) {
            const float* pp = a.part + (ch * slices + s) * part_floats(DK);
            dq += pp[e];
            dk += pp[kC * DK + e];
        }
        for (int i = 0; i < n; ++i) {
            dq += dQK[r][i] * Ks[i][d];
            dk += (Bt[r] * dAe[r][i] + Bt[i] * dAe[i][r]) * Ks[i][d] + dQK[i][r] * Qs[i][d];
        }
        const size_t off = ((size_t)(t0 + r) * H + h) * DK + d;
        a.dq[off] = dq;
        a.dk_[off] = dk;
    }
}

}  // namespace

size_t chunk_bwd_workspace(int ntok, int num_seqs, int H, int dk, int dv) {
    return bwd_layout(ntok, num_seqs, H, dk, dv).total;
}

hipError_t launch_chunk_bwd(const ChunkBwdArgs& c, hipStream_t s) {
    const BwdLayout L = bwd_layout(c.ntok, c.num_seqs, c.H, c.dk, c.dv);
    char* ws = static_cast<char*>(c.workspace);
    BwdArgs a;
    a.q = c.q; a.k = c.k; a.v = c.v; a.dy = c.dy;
    a.in_bf16 = c.in_bf16; a.dy_bf16 = c.dy_bf16;
    a.g = c.g; a.beta = c.beta; a.S0 = c.S0; a.dST = c.dST; a.cu = c.cu;
    a.num_seqs = c.num_seqs; a.ntok = c.ntok; a.H = c.H; a.dk = c.dk; a.dv = c.dv;
    a.dq = c.dq; a.dk_ = c.dk_; a.dv_ = c.dv_; a.dg = c.dg; a.dbeta = c.dbeta; a.dS0 = c.dS0;
    a.G = reinterpret_cast<float*>(ws + L.G);
    a.A = reinterpret_cast<float*>(ws + L.A);
    a.P = reinterpret_cast<float*>(ws + L.P);
    a.Sc = reinterpret_cast<float*>(ws + L.Sc);
    a.part = reinterpret_cast<float*>(ws + L.part);
    const int nchunks = c.cu ? L.max_chunks : c.num_seqs * ((c.ntok / c.num_seqs + kC - 1) / kC);
    const int seq_blocks = c.num_seqs * c.H * (c.dv / kSL);
    if (nchunks == 0 || seq_blocks == 0) {
        // no tokens: dS0 = dS_T
        if (c.dS0) {
            const size_t bytes = (size_t)c.num_seqs * c.H * c.dk * c.dv * sizeof(float);
            return c.dST ? hipMemcpyAsync(c.dS0, c.dST, bytes, hipMemcpyDeviceToDevice, s)
                         : hipMemsetAsync(c.dS0, 0, bytes, s);
        }
        return hipSuccess;
    }
#define GDN_BWD(DK, TI, TD)                                                                     \
    do {                                                                                        \
        hipLaunchKernelGGL((bwd_ap_kernel<DK, TI>), dim3(nchunks, c.H), dim3(kBT), 0, s, a);    \
        hipLaunchKernelGGL((bwd_states_kernel<DK, TI>), dim3(seq_blocks), dim3(kBT), 0, s, a);  \
        hipLaunchKernelGGL((bwd_scan_kernel<DK, TI, TD>), dim3(seq_blocks), dim3(kBT), 0, s, a); \
        hipLaunchKernelGGL((bwd_finish_kernel<DK, TI>), dim3(nchunks, c.H), dim3(kBT), 0, s, a); \
    } while (0)
    if (c.dk == 128) {
        if (c.in_bf16 && c.dy_bf16) GDN_BWD(128, uint16_t, uint16_t);
        else if (c.in_bf16) GDN_BWD(128, uint16_t, float);
        else if (c.dy_bf16) GDN_BWD(128, float, uint16_t);
        else GDN_BWD(128, float, float);
    } else {
        if (c.in_bf16 && c.dy_bf16) GDN_BWD(64, uint16_t, uint16_t);
        else if (c.in_bf16) GDN_BWD(64, uint16_t, float);
        else if (c.dy_bf16) GDN_BWD(64, float, uint16_t);
        else GDN_BWD(64, float, float);
    }
#undef GDN_BWD
    return hipGetLastError();
}

}  // namespace gdn
