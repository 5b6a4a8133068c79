// Backward pass of the chunkwise gated delta rule on gfx950 (fp32, products on the matrix core).
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
//   ap     per (chunk, head): G, Ak = e^{D} o KK^T (strictly lower, so A = beta o Ak),
//          P, and T = (I + A)^{-1} (fp32 workspace; the inverse turns both triangular solves
//          of every slice into plain products);
//   states per (sequence, head, 16-column slice of dv): the forward sweep, storing the state at
//          every chunk start;
//   scan   per (sequence, head, slice): the reverse sweep; writes dv and dS0 for its columns
//          and, per chunk, this slice's share of the terms that sum over dv columns
//          (dq, dk partials, dA, dP, and the per-token sums feeding dbeta and dg);
//   finish per (chunk, head): sums the slices' shares and adds the A and P terms.
// Columns of dv are independent in the state recursion (as in the forward), which is what the
// slices use; the terms that mix columns are sums over them, so slice shares add up.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_inverse.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;
constexpr int kBT = 1024;         // threads per workgroup: 16 waves hide the LDS latency of the
                                  // small products every chunk step is made of
constexpr int kFinT = 512;        // threads of the per-chunk-head kernels (one workgroup per CU fits their LDS)
constexpr int kStSL = 32;         // dv columns per forward-sweep workgroup

// dv columns per reverse-sweep workgroup: 32 with bf16 inputs (K and Q then sit in LDS as bf16,
// exactly), 16 with fp32 inputs (their fp32 rows leave no LDS room for wider slices). Fewer,
// wider slices mean fewer shares of the column-summed terms to write and add up.
template <typename Tin> constexpr int scan_cols() { return sizeof(Tin) == 2 ? 32 : 16; }
constexpr int kMinSL = 16;

struct BwdLayout {
    size_t G, Ak, P, T, Sc, part, total;
    int max_chunks;
};

// per-(chunk, head, slice) share: dq part, dk part [64][dk], dA, dP [64][64], and 4 token
// vectors: sum_j dR (V - gamma KS), dgamma, dw, and dgamma_C (one value, in slot 0). The four
// matrices are stored in the 16x16 tile layout of the products that write and read them:
// tile t (row tile rt, column tile ct, t = rt * (columns / 16) + ct), then lane l, then the
// lane's 4 accumulator elements (rows 16 rt + 4 (l / 16) + i, column 16 ct + l % 16), so a lane
// moves one 16-byte piece per tile.
__host__ __device__ inline size_t part_floats(int dk) { return (size_t)2 * kC * dk + 2 * kC * kC + 4 * kC; }

BwdLayout bwd_layout(int ntok, int num_seqs, int H, int dk, int dv) {
    BwdLayout L;
    L.max_chunks = (ntok + kC - 1) / kC + num_seqs;
    const size_t ch = (size_t)L.max_chunks * H;
    const int slices = dv / kMinSL;   // room for the narrowest slicing
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    L.G = take(ch * kC * sizeof(float));
    L.Ak = take(ch * kC * kC * sizeof(float));
    L.P = take(ch * kC * kC * sizeof(float));
    L.T = take(ch * kC * kC * sizeof(float));
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
    int slices;                   // reverse-sweep slices of dv (dv / scan_cols<Tin>())
    float *dq, *dk_, *dv_, *dg, *dbeta, *dS0;
    float *G, *Ak, *P, *T, *Sc, *part;
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

// packed chunk index c -> its token range; false if c is past the last chunk
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

// [64][DK] rows of a token-major [ntok, H, DK] tensor (zero past n) into fp32 LDS rows of stride
// DK+1, one 16-byte global load per unit of 8 (bf16) or 4 (fp32) elements
template <int DK, typename Tin, int NT = kBT>
__device__ __forceinline__ void load_rows(const void* x, int t0, int n, int H, int h, float (*dst)[DK + 1]) {
    constexpr int PER = 16 / sizeof(Tin), UPR = DK / PER;
    const Tin* xp = static_cast<const Tin*>(x);
    for (int u = threadIdx.x; u < kC * UPR; u += NT) {
        const int r = u / UPR, c = (u % UPR) * PER;
        gdn_u32x4 v = {0u, 0u, 0u, 0u};
        if (r < n) v = *reinterpret_cast<const gdn_u32x4*>(xp + ((size_t)(t0 + r) * H + h) * DK + c);
        if constexpr (sizeof(Tin) == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dst[r][c + 2 * i] = __uint_as_float(v[i] << 16);
                dst[r][c + 2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[r][c + i] = __uint_as_float(v[i]);
        }
    }
}

// the same rows kept in their input type (bf16 bits are copied, not widened), row stride RS:
// one 16-byte global load per unit, written to LDS as 4-byte words (RS keeps them 4-aligned)
template <int DK, int RS, typename Tin, int NT>
__device__ __forceinline__ void load_rows_raw(const void* x, int t0, int n, int H, int h, Tin (*dst)[RS]) {
    constexpr int PER = 16 / sizeof(Tin), UPR = DK / PER;
    static_assert((RS * sizeof(Tin)) % 4 == 0, "row stride");
    const Tin* xp = static_cast<const Tin*>(x);
    for (int u = threadIdx.x; u < kC * UPR; u += NT) {
        const int r = u / UPR, c = (u % UPR) * PER;
        gdn_u32x4 v = {0u, 0u, 0u, 0u};
        if (r < n) v = *reinterpret_cast<const gdn_u32x4*>(xp + ((size_t)(t0 + r) * H + h) * DK + c);
        uint32_t* d = reinterpret_cast<uint32_t*>(&dst[r][c]);
        d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    }
}

// a [64][64] fp32 tile of the workspace into LDS rows of stride 65, 16 bytes per global load
template <int NT>
__device__ __forceinline__ void load_tile64(const float* src, float (*dst)[kC + 1]) {
    for (int u = threadIdx.x; u < kC * kC / 4; u += NT) {
        const int r = u / (kC / 4), c = (u % (kC / 4)) * 4;
        const float4 v = reinterpret_cast<const float4*>(src)[u];
        dst[r][c] = v.x; dst[r][c + 1] = v.y; dst[r][c + 2] = v.z; dst[r][c + 3] = v.w;
    }
}

// ------------------------------------------------------------------ ap: G, Ak, P, T per chunk-head
// K and Q stay in their input type in LDS (bf16 is widened exactly as the products read it):
// with bf16 inputs that is 50 KB, so two workgroups share a CU (4 waves per SIMD, which caps
// the registers at 128).
template <int DK, typename Tin>
__global__ void __launch_bounds__(kFinT, 4) bwd_ap_kernel(BwdArgs a) {
    constexpr int KR = DK + (sizeof(Tin) == 2 ? 2 : 1);
    __shared__ Tin Ks[kC][KR], Qs[kC][KR];
    __shared__ float A[kC][kC + 1];
    __shared__ float G[kC], Bt[kC];
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int t0, n;
    if (!chunk_info(a, c, t0, n)) return;
    const int H = a.H;
    load_rows_raw<DK, KR, Tin, kFinT>(a.k, t0, n, H, h, Ks);
    load_rows_raw<DK, KR, Tin, kFinT>(a.q, t0, n, H, h, Qs);
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
    // K K^T and Q K^T on the matrix core, one 16x16 tile per wave (the 10 tiles on or below the
    // diagonal of each), then the decay and the masks per element; tiles above are zero
    const int wave = tid / kWave, lane = tid % kWave, lc = lane & 15, lg = lane >> 4;
    for (int tile = wave; tile < 32; tile += kFinT / kWave) {
        const int kind = tile / 16, rt = (tile % 16) / 4, it = tile % 4;
        const size_t base = ch * kC * kC;
        if (it > rt) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = rt * 16 + 4 * lg + u, i = it * 16 + lc;
                if (kind == 0) {
                    A[r][i] = 0.f;
                    a.Ak[base + r * kC + i] = 0.f;
                } else {
                    a.P[base + r * kC + i] = 0.f;
                }
            }
            continue;
        }
        const Tin* X = kind ? &Qs[rt * 16][0] : &Ks[rt * 16][0];
        const floatx4 acc = mma_f32_tile(X, KR, 1, &Ks[it * 16][0], 1, KR, DK,
                                         floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = rt * 16 + 4 * lg + u, i = it * 16 + lc;
            const float dec = (i <= r && r < n) ? expf(G[r] - G[i]) : 0.f;
            if (kind == 0) {
                const float ak = i < r ? dec * acc[u] : 0.f;
                A[r][i] = Bt[r] * ak;
                a.Ak[base + r * kC + i] = ak;
            } else {
                a.P[base + r * kC + i] = dec * acc[u];
            }
        }
    }
    __syncthreads();
    // T = (I + A)^{-1} by one wave (16x16 diagonal blocks by DPP substitution, then fp32 MFMA
    // levels), in place in LDS, then written out by the whole workgroup
    if (tid < kWave) unit_lower_inverse64<kC + 1, true>(&A[0][0]);
    __syncthreads();
    for (int e = tid; e < kC * kC; e += kFinT) a.T[ch * kC * kC + e] = A[e / kC][e % kC];
}

// ------------------------------------------------------------------ states: forward sweep
// The three products of a chunk step run on the fp32 matrix core, one 16x16 output tile per wave.
template <int DK, typename Tin>
__global__ void __launch_bounds__(kBT) bwd_states_kernel(BwdArgs a) {
    constexpr int SL = kStSL, CT = SL / 16, PR = SL + 1;
    __shared__ float Ks[kC][DK + 1];
    __shared__ float S[DK][PR];
    __shared__ float T[kC][kC + 1];
    __shared__ float R[kC][PR], W[kC][PR];
    __shared__ float gam[kC], w[kC], Bt[kC];
    static_assert((DK / 16) * CT <= kBT / kWave, "one state tile per wave");
    const int slices = a.dv / SL;
    const int slice = blockIdx.x % slices;
    const int h = (blockIdx.x / slices) % a.H;
    const int sq = blockIdx.x / (slices * a.H);
    const int j0 = slice * SL, tid = threadIdx.x, H = a.H, dv = a.dv;
    const int wave = tid / kWave, lane = tid % kWave, lc = lane & 15, lg = lane >> 4;
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    int lo, hi, cbase;
    seq_info(a, sq, lo, hi, cbase);
    const size_t st_off = ((size_t)sq * H + h) * DK * dv;
    for (int e = tid; e < DK * SL; e += kBT) {
        const int d = e / SL, j = e % SL;
        S[d][j] = a.S0 ? a.S0[st_off + (size_t)d * dv + j0 + j] : 0.f;
    }
    // The next chunk's K rows, T, V slice and gate rows are fetched into registers while this
    // chunk computes (16-byte loads; K stays in its input type until it is written to LDS).
    constexpr int KPER = 16 / sizeof(Tin), KUNITS = kC * DK / KPER;
    constexpr int KU = (KUNITS + kBT - 1) / kBT, VE = kC * SL / kBT;
    static_assert(kC * kC / 4 == kBT && VE >= 1, "one T float4 per thread, whole V elements");
    struct Pref {
        gdn_u32x4 k[KU];
        float4 t;
        float v[VE], g, gl, b;
    };
    auto fetch = [&](int t0, int n, size_t ch, Pref& f) __attribute__((always_inline)) {
        const Tin* kp = static_cast<const Tin*>(a.k);
#pragma unroll
        for (int i = 0; i < KU; ++i) {
            const int u = tid + i * kBT, r = u / (DK / KPER), c0 = (u % (DK / KPER)) * KPER;
            f.k[i] = gdn_u32x4{0u, 0u, 0u, 0u};
            if (u < KUNITS && r < n)
                f.k[i] = *reinterpret_cast<const gdn_u32x4*>(kp + ((size_t)(t0 + r) * H + h) * DK + c0);
        }
        f.t = reinterpret_cast<const float4*>(a.T + ch * kC * kC)[tid];
#pragma unroll
        for (int i = 0; i < VE; ++i) {
            const int e = tid + i * kBT, r = e / SL, j = e % SL;
            f.v[i] = r < n ? ld<Tin>(a.v, ((size_t)(t0 + r) * H + h) * dv + j0 + j) : 0.f;
        }
        f.g = tid < kC ? a.G[ch * kC + tid] : 0.f;
        f.gl = a.G[ch * kC + n - 1];
        f.b = tid < n ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
    };
    auto stash = [&](const Pref& f, int n) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KU; ++i) {
            const int u = tid + i * kBT, r = u / (DK / KPER), c0 = (u % (DK / KPER)) * KPER;
            if (u < KUNITS) {
                if constexpr (sizeof(Tin) == 2) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        Ks[r][c0 + 2 * q] = __uint_as_float(f.k[i][q] << 16);
                        Ks[r][c0 + 2 * q + 1] = __uint_as_float(f.k[i][q] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) Ks[r][c0 + q] = __uint_as_float(f.k[i][q]);
                }
            }
        }
        const int tr = tid / (kC / 4), tc = (tid % (kC / 4)) * 4;
        T[tr][tc] = f.t.x; T[tr][tc + 1] = f.t.y; T[tr][tc + 2] = f.t.z; T[tr][tc + 3] = f.t.w;
#pragma unroll
        for (int i = 0; i < VE; ++i) {
            const int e = tid + i * kBT;
            R[e / SL][e % SL] = f.v[i];
        }
        if (tid < kC) {
            gam[tid] = expf(f.g);
            w[tid] = tid < n ? expf(f.gl - f.g) : 0.f;
            Bt[tid] = f.b;
        }
    };
    Pref f;
    if (lo < hi) fetch(lo, min(kC, hi - lo), (size_t)cbase * H + h, f);
    for (int t0 = lo, c = cbase; t0 < hi; t0 += kC, ++c) {
        const int n = min(kC, hi - t0);
        const size_t ch = (size_t)c * H + h;
        __syncthreads();
        for (int u = tid; u < DK * SL / 4; u += kBT) {   // the state entering this chunk
            const int d = u / (SL / 4), j = (u % (SL / 4)) * 4;
            *reinterpret_cast<float4*>(a.Sc + ch * DK * dv + (size_t)d * dv + j0 + j) =
                make_float4(S[d][j], S[d][j + 1], S[d][j + 2], S[d][j + 3]);
        }
        stash(f, n);
        if (t0 + kC < hi) fetch(t0 + kC, min(kC, hi - t0 - kC), (size_t)(c + 1) * H + h, f);
        __syncthreads();
        if (wave < 4 * CT) {   // R = beta o (V - gamma o K S)
            const int rt = wave % 4, ct = wave / 4;
            const floatx4 ks = mma_f32_tile(&Ks[rt * 16][0], DK + 1, 1, &S[0][ct * 16], PR, 1, DK, zero);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rt * 16 + 4 * lg + i, j = ct * 16 + lc;
                R[r][j] = Bt[r] * (R[r][j] - gam[r] * ks[i]);
            }
        }
        __syncthreads();
        if (wave < 4 * CT) {   // W = w o (T R); T is lower triangular
            const int rt = wave % 4, ct = wave / 4;
            const floatx4 u = mma_f32_tile(&T[rt * 16][0], kC + 1, 1, &R[0][ct * 16], PR, 1, kC, zero);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rt * 16 + 4 * lg + i;
                W[r][ct * 16 + lc] = w[r] * u[i];
            }
        }
        __syncthreads();
        floatx4 sn = zero;   // S' = gamma_C S + K^T W (rows of K past n are zero)
        const int dt = wave % (DK / 16), ct = wave / (DK / 16);
        if (wave < (DK / 16) * CT) {
            const float gC = gam[n - 1];
            sn = mma_f32_tile(&Ks[0][dt * 16], 1, DK + 1, &W[0][ct * 16], PR, 1, kC, zero);
#pragma unroll
            for (int i = 0; i < 4; ++i) sn[i] += gC * S[dt * 16 + 4 * lg + i][ct * 16 + lc];
        }
        __syncthreads();
        if (wave < (DK / 16) * CT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) S[dt * 16 + 4 * lg + i][ct * 16 + lc] = sn[i];
        }
    }
}

// ------------------------------------------------------------------ scan: reverse sweep
// Every product of a chunk step runs on the fp32 matrix core, one 16x16 output tile per wave at a
// time (16 waves), with its operands read from LDS as strided views. SL dv columns per
// workgroup (scan_cols); K and Q rows stay in the input type in LDS.
constexpr int kScanT = 1024;
template <int DK, int SL, typename Tin, typename Tdy>
__global__ void __launch_bounds__(kScanT) bwd_scan_kernel(BwdArgs a) {
    constexpr int CT = SL / 16;                    // column tiles of a [64][SL] slice
    constexpr int PR = SL + 1;                     // padded row of a [64][SL] tile
    constexpr int KR = DK + (sizeof(Tin) == 2 ? 2 : 1);
    __shared__ Tin Ks[kC][KR], Qs[kC][KR];
    // state entering the chunk and the gradient after it; rows padded by one so the transposed
    // operand reads (16 rows, 4 columns per step) spread over the banks
    __shared__ float S[DK][PR], dS[DK][PR];
    __shared__ float T[kC][kC + 1], P[kC][kC + 1];
    // [64][SL] tiles: dY, KS, QS, U, KdS = K dS', dU, dR; late in the step QS and KS are reused
    // for gamma o dY and (beta gamma) o dR, and dR holds R = beta o (V - gamma o KS) until dR
    // itself is formed
    __shared__ float dY[kC][PR], KS[kC][PR], QS[kC][PR];
    __shared__ float U[kC][PR], KdS[kC][PR], dU[kC][PR], dR[kC][PR];
    __shared__ float gam[kC], w[kC], Bt[kC], dRV[kC];
    __shared__ float red[kScanT / kWave];

    const int slices = a.dv / SL;
    const int slice = blockIdx.x % slices;
    const int h = (blockIdx.x / slices) % a.H;
    const int sq = blockIdx.x / (slices * a.H);
    const int j0 = slice * SL, tid = threadIdx.x, H = a.H, dv = a.dv;
    const int wave = tid / kWave, lane = tid % kWave, lc = lane & 15, lg = lane >> 4;
    constexpr int NW = kScanT / kWave;
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    int lo, hi, cbase;
    seq_info(a, sq, lo, hi, cbase);
    const int nch = (hi - lo + kC - 1) / kC;
    const size_t st_off = ((size_t)sq * H + h) * DK * dv;
    for (int e = tid; e < DK * SL; e += kScanT) {
        const int d = e / SL, j = e % SL;
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
        load_rows_raw<DK, KR, Tin, kScanT>(a.k, t0, n, H, h, Ks);
        load_rows_raw<DK, KR, Tin, kScanT>(a.q, t0, n, H, h, Qs);
        for (int e = tid; e < kC * SL; e += kScanT) {
            const int r = e / SL, j = e % SL;
            dY[r][j] = r < n ? ld<Tdy>(a.dy, ((size_t)(t0 + r) * H + h) * dv + j0 + j) : 0.f;
        }
        for (int u = tid; u < DK * SL / 4; u += kScanT) {   // 16 bytes per load
            const int d = u / (SL / 4), j = (u % (SL / 4)) * 4;
            const float4 v = *reinterpret_cast<const float4*>(a.Sc + ch * DK * dv + (size_t)d * dv + j0 + j);
            S[d][j] = v.x; S[d][j + 1] = v.y; S[d][j + 2] = v.z; S[d][j + 3] = v.w;
        }
        load_tile64<kScanT>(a.T + ch * kC * kC, T);
        load_tile64<kScanT>(a.P + ch * kC * kC, P);
        if (tid < kC) {
            const float* Gc = a.G + ch * kC;
            gam[tid] = expf(Gc[tid]);
            w[tid] = tid < n ? expf(Gc[n - 1] - Gc[tid]) : 0.f;
            Bt[tid] = tid < n ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
        }
        __syncthreads();
        // ---- step 1: KS = K S, QS = Q S, KdS = K dS' (3 x 4 x CT tiles); <S, dS'>
        for (int tile = wave; tile < 12 * CT; tile += NW) {
            const int kind = tile / (4 * CT), rt = tile % 4, ct = (tile / 4) % CT;
            const Tin* A = kind == 1 ? &Qs[rt * 16][0] : &Ks[rt * 16][0];
            const float* B = kind == 2 ? &dS[0][ct * 16] : &S[0][ct * 16];
            const floatx4 acc = mma_f32_tile(A, KR, 1, B, PR, 1, DK, zero);
            float(*dst)[PR] = kind == 0 ? KS : (kind == 1 ? QS : KdS);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[rt * 16 + 4 * lg + i][ct * 16 + lc] = acc[i];
        }
        {
            float sdot = 0.f;
            for (int e = tid; e < DK * SL; e += kScanT) sdot += S[e / SL][e % SL] * dS[e / SL][e % SL];
            sdot = group_sum<kWave>(sdot);
            if (lane == 0) red[wave] = sdot;
        }
        __syncthreads();
        if (tid == 0) {
            float acc = 0.f;
            for (int i = 0; i < NW; ++i) acc += red[i];
            pvec[3 * kC] = acc;
        }
        for (int e = tid; e < kC * SL; e += kScanT) {   // R = beta o (V - gamma o KS), in dR
            const int r = e / SL, j = e % SL;
            const float vv = r < n ? ld<Tin>(a.v, ((size_t)(t0 + r) * H + h) * dv + j0 + j) : 0.f;
            dR[r][j] = Bt[r] * (vv - gam[r] * KS[r][j]);
        }
        __syncthreads();
        // ---- step 2: U = T R;  dU = w o KdS + P^T dY (2 x 4 x CT tiles)
        for (int tile = wave; tile < 8 * CT; tile += NW) {
            const int rt = tile % 4, ct = (tile / 4) % CT;
            if (tile < 4 * CT) {
                const floatx4 acc = mma_f32_tile(&T[rt * 16][0], kC + 1, 1, &dR[0][ct * 16], PR, 1,
                                                 kC, zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) U[rt * 16 + 4 * lg + i][ct * 16 + lc] = acc[i];
            } else {
                const floatx4 acc = mma_f32_tile(&P[0][rt * 16], 1, kC + 1, &dY[0][ct * 16], PR, 1,
                                                 kC, zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rt * 16 + 4 * lg + i, j = ct * 16 + lc;
                    dU[r][j] = w[r] * KdS[r][j] + acc[i];
                }
            }
        }
        __syncthreads();
        // ---- step 3: dR = T^T dU (4 x CT tiles); dq share (gamma o dY) S^T and dP = dY U^T
        if (wave < 4 * CT) {
            const int rt = wave % 4, ct = wave / 4;
            const floatx4 acc = mma_f32_tile(&T[0][rt * 16], 1, kC + 1, &dU[0][ct * 16], PR, 1, kC,
                                             zero);
#pragma unroll
            for (int i = 0; i < 4; ++i) dR[rt * 16 + 4 * lg + i][ct * 16 + lc] = acc[i];
        }
        for (int tile = (wave + NW - 4 * CT) % NW; tile < 4 * (DK / 16) + 16; tile += NW) {
            if (tile < 4 * (DK / 16)) {   // dq share tile (rt, dt)
                const int rt = tile / (DK / 16), dt = tile % (DK / 16);
                const floatx4 acc = mma_f32_tile(&dY[rt * 16][0], PR, 1, &S[dt * 16][0], 1, PR, SL,
                                                 zero);
                floatx4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = gam[rt * 16 + 4 * lg + i] * acc[i];
                reinterpret_cast<floatx4*>(pdq)[tile * kWave + lane] = o;
            } else {                      // dP tile (rt, it), lower with the diagonal
                const int t2 = tile - 4 * (DK / 16), rt = t2 >> 2, it = t2 & 3;
                const floatx4 acc = mma_f32_tile(&dY[rt * 16][0], PR, 1, &U[it * 16][0], 1, PR, SL,
                                                 zero);
                floatx4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rt * 16 + 4 * lg + i, c = it * 16 + lc;
                    o[i] = (c <= r && r < n) ? acc[i] : 0.f;
                }
                reinterpret_cast<floatx4*>(pdP)[t2 * kWave + lane] = o;
            }
        }
        __syncthreads();
        // ---- step 4: dv = beta o dR and, per token, sum_j dR V (the SL lanes of a row are an
        // aligned lane group); then the other per-token sums, the dk share and dA
        for (int e = tid; e < kC * SL; e += kScanT) {
            const int r = e / SL, j = e % SL;
            const size_t off = ((size_t)(t0 + min(r, n - 1)) * H + h) * dv + j0 + j;
            const float vv = r < n ? ld<Tin>(a.v, off) : 0.f;
            const float x = dR[r][j];
            if (r < n) a.dv_[off] = Bt[r] * x;
            const float rv = group_sum<SL>(x * vv);
            if (j == 0) dRV[r] = rv;
        }
        __syncthreads();
        if (tid < kC) {
            const int r = tid;
            float dwr = 0.f, dg1 = 0.f, dg2 = 0.f;
#pragma unroll 8
            for (int j = 0; j < SL; ++j) {
                dwr += KdS[r][j] * U[r][j];
                dg1 += dY[r][j] * QS[r][j];
                dg2 += dR[r][j] * KS[r][j];
            }
            pvec[r] = dRV[r] - gam[r] * dg2;   // sum_j dR (V - gamma KS)
            pvec[kC + r] = dg1 - Bt[r] * dg2;
            pvec[2 * kC + r] = dwr;
        }
        for (int tile = wave; tile < 4 * (DK / 16) + 16; tile += NW) {
            if (tile < 4 * (DK / 16)) {   // dk share: w o (U dS'^T) - (beta gamma) o (dR S^T)
                const int rt = tile / (DK / 16), dt = tile % (DK / 16);
                const floatx4 a1 = mma_f32_tile(&U[rt * 16][0], PR, 1, &dS[dt * 16][0], 1, PR, SL, zero);
                const floatx4 a2 = mma_f32_tile(&dR[rt * 16][0], PR, 1, &S[dt * 16][0], 1, PR, SL, zero);
                floatx4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rt * 16 + 4 * lg + i;
                    o[i] = w[r] * a1[i] - Bt[r] * gam[r] * a2[i];
                }
                reinterpret_cast<floatx4*>(pdk)[tile * kWave + lane] = o;
            } else {                      // dA = -(dR U^T), strictly lower
                const int t2 = tile - 4 * (DK / 16), rt = t2 >> 2, it = t2 & 3;
                const floatx4 acc = mma_f32_tile(&dR[rt * 16][0], PR, 1, &U[it * 16][0], 1, PR, SL, zero);
                floatx4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rt * 16 + 4 * lg + i, c = it * 16 + lc;
                    o[i] = (c < r && r < n) ? -acc[i] : 0.f;
                }
                reinterpret_cast<floatx4*>(pdA)[t2 * kWave + lane] = o;
            }
        }
        __syncthreads();
        // ---- step 5: dS = gamma_C dS' + Q^T (gamma o dY) - K^T ((beta gamma) o dR)
        for (int e = tid; e < kC * SL; e += kScanT) {   // scaled copies into QS and KS
            const int r = e / SL, j = e % SL;
            QS[r][j] = gam[r] * dY[r][j];
            KS[r][j] = Bt[r] * gam[r] * dR[r][j];
        }
        __syncthreads();
        constexpr int NT5 = (DK / 16) * CT;        // state tiles
        static_assert(NT5 <= 2 * NW, "dS tiles per wave");
        floatx4 dsn[2] = {zero, zero};
        const float gC = gam[n - 1];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tile = wave + u * NW, dt = tile % (DK / 16), ct = tile / (DK / 16);
            if (tile < NT5) {
                const floatx4 a1 = mma_f32_tile(&Qs[0][dt * 16], 1, KR, &QS[0][ct * 16], PR, 1, kC, zero);
                const floatx4 a2 = mma_f32_tile(&Ks[0][dt * 16], 1, KR, &KS[0][ct * 16], PR, 1, kC, zero);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dsn[u][i] = gC * dS[dt * 16 + 4 * lg + i][ct * 16 + lc] + a1[i] - a2[i];
            }
        }
        __syncthreads();   // every read of dS' is done
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tile = wave + u * NW, dt = tile % (DK / 16), ct = tile / (DK / 16);
            if (tile < NT5) {
#pragma unroll
                for (int i = 0; i < 4; ++i) dS[dt * 16 + 4 * lg + i][ct * 16 + lc] = dsn[u][i];
            }
        }
    }
    __syncthreads();
    if (a.dS0) {
        for (int e = tid; e < DK * SL; e += kScanT) {
            const int d = e / SL, j = e % SL;
            a.dS0[st_off + (size_t)d * dv + j0 + j] = dS[d][j];
        }
    }
}

// ------------------------------------------------------------------ finish per chunk-head
template <int DK, typename Tin>
__global__ void __launch_bounds__(kFinT, 4) bwd_finish_kernel(BwdArgs a) {
    // K and Q stay in their input type; dD = dA o A + dP o P and dA o Ak are needed only as row
    // and column sums, which are formed per 16x16 tile by shuffles. With bf16 inputs that is
    // 70 KB, so two workgroups share a CU (4 waves per SIMD, which caps the registers at 128).
    constexpr int KR = DK + (sizeof(Tin) == 2 ? 2 : 1);
    __shared__ Tin Ks[kC][KR], Qs[kC][KR];
    __shared__ float dKK[kC][kC + 1], dQK[kC][kC + 1];   // coefficients of k_r.k_i, q_r.k_i
    __shared__ float rsD[kC][4], rsA[kC][4];             // row sums of dD, dA o Ak per column tile
    __shared__ float csD[4][kC];                         // column sums of dD per row tile
    __shared__ float G[kC], Bt[kC], dG[kC], dgam[kC], dw[kC], dbs[kC];
    __shared__ float dgC;
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int t0, n;
    if (!chunk_info(a, c, t0, n)) return;
    const int H = a.H, slices = a.slices;
    const size_t ch = (size_t)c * H + h;
    load_rows_raw<DK, KR, Tin, kFinT>(a.k, t0, n, H, h, Ks);
    load_rows_raw<DK, KR, Tin, kFinT>(a.q, t0, n, H, h, Qs);
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
    }
    if (tid == 0) {
        float s0 = 0.f;
        for (int s = 0; s < slices; ++s)
            s0 += a.part[(ch * slices + s) * part_floats(DK) + 2 * kC * DK + 2 * kC * kC + 3 * kC];
        dgC = s0;
    }
    __syncthreads();
    // dA, dP summed over slices. With A = beta o Ak (Ak = e^{D} o KK^T) and P = e^{D} o QK^T:
    // dKK = beta o dA o e^{D}, dQK = dP o e^{D}, dbeta += rowsum(dA o Ak),
    // dD = beta o dA o Ak + dP o P. The shares are in tile layout: one 16-byte piece per lane.
    // Every lane of a wave runs the same iterations (kFinT is a multiple of the wave), so the
    // tile's row and column sums are shuffle reductions over its lanes.
    static_assert(kFinT % kWave == 0 && (16 * kWave) % kFinT == 0, "uniform tile loop");
    for (int idx = tid; idx < 16 * kWave; idx += kFinT) {
        const int t2 = idx / kWave, l = idx % kWave, rt = t2 >> 2, it = t2 & 3;
        floatx4 da = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < slices; ++s) {
            const floatx4* pp = reinterpret_cast<const floatx4*>(
                a.part + (ch * slices + s) * part_floats(DK) + 2 * kC * DK);
            da += pp[idx];
            dp += pp[kC * kC / 4 + idx];
        }
        float dd[4], dak[4], col = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = rt * 16 + 4 * (l >> 4) + u, i = it * 16 + (l & 15);
            const size_t e = (size_t)r * kC + i;
            const float ak = a.Ak[ch * kC * kC + e], pv = a.P[ch * kC * kC + e];
            const float dec = (i <= r && r < n) ? expf(G[r] - G[i]) : 0.f;
            dKK[r][i] = i < r ? Bt[r] * da[u] * dec : 0.f;
            dQK[r][i] = dp[u] * dec;
            dd[u] = Bt[r] * da[u] * ak + dp[u] * pv;
            dak[u] = da[u] * ak;
            col += dd[u];
        }
        // row sums: over the 16 lanes of a row group (lane bits 0-3); column sums: over the
        // 4 row groups (lane bits 4-5)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                dd[u] += __shfl_xor(dd[u], o, kWave);
                dak[u] += __shfl_xor(dak[u], o, kWave);
            }
        col += __shfl_xor(col, 16, kWave);
        col += __shfl_xor(col, 32, kWave);
        if ((l & 15) == 0)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                rsD[rt * 16 + 4 * (l >> 4) + u][it] = dd[u];
                rsA[rt * 16 + 4 * (l >> 4) + u][it] = dak[u];
            }
        if (l < 16) csD[rt][it * 16 + l] = col;
    }
    __syncthreads();
    if (tid < kC) {
        const int r = tid;
        const float rs = (rsD[r][0] + rsD[r][1]) + (rsD[r][2] + rsD[r][3]);
        const float cs = (csD[0][r] + csD[1][r]) + (csD[2][r] + csD[3][r]);
        const float db = (rsA[r][0] + rsA[r][1]) + (rsA[r][2] + rsA[r][3]);
        dbs[r] += db;
        dG[r] = rs - cs + dgam[r] * expf(G[r]) - dw[r] * (r < n ? expf(G[n - 1] - G[r]) : 0.f);
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
    // dq = sum of shares + dQK K;  dk = sum of shares + (dKK + dKK^T) K + dQK^T Q, one 16x16
    // output tile per wave on the matrix core (entries past n are zero on both sides)
    const int wave = tid / kWave, lane = tid % kWave, lc = lane & 15, lg = lane >> 4;
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int tile = wave; tile < (kC / 16) * (DK / 16); tile += kFinT / kWave) {
        const int rt = tile / (DK / 16), dt = tile % (DK / 16);
        floatx4 q0 = zero, k0 = zero;   // the slices' shares of this tile (tile layout)
        for (int s = 0; s < slices; ++s) {
            const floatx4* pp = reinterpret_cast<const floatx4*>(a.part + (ch * slices + s) * part_floats(DK));
            q0 += pp[tile * kWave + lane];
            k0 += pp[kC * DK / 4 + tile * kWave + lane];
        }
        const floatx4 q1 = mma_f32_tile(&dQK[rt * 16][0], kC + 1, 1, &Ks[0][dt * 16], KR, 1, kC, q0);
        floatx4 k1 = mma_f32_tile(&dKK[rt * 16][0], kC + 1, 1, &Ks[0][dt * 16], KR, 1, kC, k0);
        k1 = mma_f32_tile(&dKK[0][rt * 16], 1, kC + 1, &Ks[0][dt * 16], KR, 1, kC, k1);
        k1 = mma_f32_tile(&dQK[0][rt * 16], 1, kC + 1, &Qs[0][dt * 16], KR, 1, kC, k1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rt * 16 + 4 * lg + i, d = dt * 16 + lc;
            if (r >= n) continue;
            const size_t off = ((size_t)(t0 + r) * H + h) * DK + d;
            a.dq[off] = q1[i];
            a.dk_[off] = k1[i];
        }
    }
}

// dst = src, or zero without one (n float4 units; states are multiples of 4 floats)
__global__ void __launch_bounds__(256) copy_or_zero_kernel(float4* dst, const float4* src, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

size_t chunk_bwd_workspace(int ntok, int num_seqs, int H, int dk, int dv) {
    // room for either path: the bf16 one is taken by bf16 q, k, v, dy at dk = dv = 128
    const size_t f32 = bwd_layout(ntok, num_seqs, H, dk, dv).total;
    if (dk != 128 || dv != 128) return f32;
    return std::max(f32, chunk_bwd_bf16_workspace(ntok, num_seqs, H));
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
    a.Ak = reinterpret_cast<float*>(ws + L.Ak);
    a.P = reinterpret_cast<float*>(ws + L.P);
    a.T = reinterpret_cast<float*>(ws + L.T);
    a.Sc = reinterpret_cast<float*>(ws + L.Sc);
    a.part = reinterpret_cast<float*>(ws + L.part);
    const int nchunks = c.cu ? L.max_chunks : c.num_seqs * ((c.ntok / c.num_seqs + kC - 1) / kC);
    const int seq_blocks = c.num_seqs * c.H;
    if (nchunks == 0 || seq_blocks == 0) {
        // no tokens: dS0 = dS_T (a kernel, not a memset or copy node, so the call can be
        // captured in a graph like every other)
        const size_t n = (size_t)c.num_seqs * c.H * c.dk * c.dv;
        if (c.dS0 && n > 0) {
            const int blocks = (int)((n / 4 + 255) / 256);
            hipLaunchKernelGGL(copy_or_zero_kernel, dim3(blocks), dim3(256), 0, s,
                               reinterpret_cast<float4*>(c.dS0),
                               reinterpret_cast<const float4*>(c.dST), n / 4);
        }
        return hipGetLastError();
    }
    if (use_bwd_bf16(c)) return launch_chunk_bwd_bf16(c, s);
#define GDN_BWD(DK, TI, TD)                                                                     \
    do {                                                                                        \
        constexpr int SL = scan_cols<TI>();                                                     \
        a.slices = c.dv / SL;                                                                   \
        hipLaunchKernelGGL((bwd_ap_kernel<DK, TI>), dim3(nchunks, c.H), dim3(kFinT), 0, s, a);    \
        hipLaunchKernelGGL((bwd_states_kernel<DK, TI>), dim3(c.num_seqs * c.H * (c.dv / kStSL)), \
                           dim3(kBT), 0, s, a);                                                 \
        hipLaunchKernelGGL((bwd_scan_kernel<DK, SL, TI, TD>), dim3(c.num_seqs * c.H * a.slices), \
                           dim3(kScanT), 0, s, a);                                              \
        hipLaunchKernelGGL((bwd_finish_kernel<DK, TI>), dim3(nchunks, c.H), dim3(kFinT), 0, s, a); \
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
