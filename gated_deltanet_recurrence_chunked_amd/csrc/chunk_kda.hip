// Chunkwise delta rule with a per-channel (diagonal) decay on gfx950: the KDA-style variant
// of the Gated DeltaNet recurrence (fp32; the scan's products on the matrix core).
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
// Two kernels: a per-(chunk, head) prep forms T, P and the running log-decays Gc into the
// workspace (every exponential it takes is of a non-positive difference, so no factor can
// overflow); a scan per (sequence, head, slice of dv) forms Kg, Qg, Kc and e^{Gc[C]} from K, Q
// and Gc as it reads its matrix-core operands.
#include "gdn_device.h"
#include "gdn_inverse.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;
constexpr int kPT = 512;          // prep threads (one workgroup per CU fits its LDS)
constexpr int kST = 1024;         // scan threads: 16 waves hide the LDS latency of the small products
// dv columns per scan workgroup: 32 with bf16 inputs (K, Q sit in LDS as bf16, exactly), 16
// with fp32 inputs (their rows leave no LDS room for wider slices)
template <typename Tin> constexpr int kda_cols() { return sizeof(Tin) == 2 ? 32 : 16; }

struct KdaLayout {
    size_t T, P, Gw, total;
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
    L.Gw = take(ch * kC * (size_t)dk * sizeof(float));
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
    float *T, *P, *Gw;             // Gw: the chunk's running log-decays [64][dk] per chunk-head
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

// packed chunk index c -> its token range; false if c is past the last chunk (one pass over
// the sequences, so the cost per workgroup is linear in their number)
__device__ bool kda_chunk(const KdaArgs& a, int c, int& t0, int& n) {
    int base = 0;
    const int L = a.cu ? 0 : a.ntok / a.num_seqs;
    for (int s = 0; s < a.num_seqs; ++s) {
        const int lo = a.cu ? a.cu[s] : s * L;
        const int hi = a.cu ? a.cu[s + 1] : lo + L;
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
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// exact for a value widened from bf16 (its low 16 bits are zero)
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) {
    return (uint16_t)(__float_as_uint(x) >> 16);
}

// K and Q stay in their input type in LDS and share one region with A, which is written only
// after every product has read them (the products' results wait in registers across a
// barrier). With bf16 inputs that is 66 KB, so two workgroups share a CU (4 waves per SIMD,
// which caps the registers at 128).
template <int DK, typename Tin>
__global__ void __launch_bounds__(kPT, 4) kda_prep_kernel(KdaArgs a) {
    constexpr int KR = DK + (sizeof(Tin) == 2 ? 2 : 1);
    constexpr int kKQBytes = 2 * kC * KR * (int)sizeof(Tin);
    constexpr int kABytes = kC * (kC + 1) * (int)sizeof(float);
    __shared__ __attribute__((aligned(16))) unsigned char kqa[kKQBytes > kABytes ? kKQBytes : kABytes];
    __shared__ float Gc[kC][DK + 1];
    __shared__ float Bt[kC];
    Tin (*Ks)[KR] = reinterpret_cast<Tin (*)[KR]>(kqa);
    Tin (*Qs)[KR] = reinterpret_cast<Tin (*)[KR]>(kqa + kC * KR * sizeof(Tin));
    float (*A)[kC + 1] = reinterpret_cast<float (*)[kC + 1]>(kqa);
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, H = a.H;
    int t0, n;
    if (!kda_chunk(a, c, t0, n)) return;
    for (int u = tid; u < kC * DK / 4; u += kPT) {   // 4 channels per thread and step
        const int r = u / (DK / 4), d = (u % (DK / 4)) * 4;
        const bool ok = r < n;
        const size_t off = ((size_t)(t0 + min(r, n - 1)) * H + h) * DK + d;
        float kv[4], qv[4];
        Vec4<Tin>::load(static_cast<const Tin*>(a.k) + off, kv);
        Vec4<Tin>::load(static_cast<const Tin*>(a.q) + off, qv);
        const float4 gv = *reinterpret_cast<const float4*>(a.g + off);
        const float gs[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Ks[r][d + i] = from_f32<Tin>(ok ? kv[i] : 0.f);
            Qs[r][d + i] = from_f32<Tin>(ok ? qv[i] : 0.f);
            Gc[r][d + i] = ok ? gs[i] : 0.f;
        }
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
    // A (strictly lower) and P (lower with the diagonal). For a 16x16 tile below the diagonal
    // (row block rt > column block it), with m = 16 rt the first row of the row block,
    // e^{Gc_r - Gc_i} = e^{Gc_r - Gc_m} e^{Gc_m - Gc_i} with both exponents <= 0 (Gc falls along
    // the rows), so the tile is a plain product of decayed operands: one wave per tile on the
    // fp32 matrix core, the two exponentials formed as the operands are read (no overflow, and
    // no bound on g needed). The four diagonal tiles' 136 pairs each are formed element by
    // element; the tiles above are zero. P goes out at once; A waits in registers.
    const int wave = tid / kWave, lane = tid % kWave, lc = lane & 15, lg = lane >> 4;
    for (int e = tid; e < kC * kC; e += kPT) {
        const int r = e / kC, i = e % kC;
        if ((i >> 4) > (r >> 4)) a.P[ch * kC * kC + e] = 0.f;
    }
    floatx4 ak = {0.f, 0.f, 0.f, 0.f};
    if (wave < 6) {
        const int rt = wave < 1 ? 1 : (wave < 3 ? 2 : 3);
        const int it = wave - (rt * (rt - 1)) / 2;          // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
        const int m = 16 * rt, r = 16 * rt + lc, i = 16 * it + lc;
        floatx4 aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k0 = 0; k0 < DK; k0 += 4) {
            const int d = k0 + lg;
            const float gm = Gc[m][d];
            const float ea = fexp(Gc[r][d] - gm), eb = fexp(gm - Gc[i][d]);
            const float b = load1(&Ks[i][d]) * eb;
            ak = __builtin_amdgcn_mfma_f32_16x16x4f32(load1(&Ks[r][d]) * ea, b, ak, 0, 0, 0);
            aq = __builtin_amdgcn_mfma_f32_16x16x4f32(load1(&Qs[r][d]) * ea, b, aq, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {   // accumulator element u: row 4 lg + u, column lc
            const int rr = 16 * rt + 4 * lg + u, ii = 16 * it + lc;
            a.P[ch * kC * kC + rr * kC + ii] = aq[u];
        }
    }
    constexpr int kPairIt = (4 * 136 + kPT - 1) / kPT;   // diagonal pairs per thread, at most
    float kkv[kPairIt];
#pragma unroll
    for (int j = 0; j < kPairIt; ++j) {   // the diagonal tiles, pair by pair
        const int p = tid + j * kPT;
        kkv[j] = 0.f;
        if (p >= 4 * 136) continue;
        const int b = p / 136, q = p % 136;
        int rr = (int)((sqrtf(8.f * q + 1.f) - 1.f) * 0.5f);
        while (rr * (rr + 1) / 2 > q) --rr;                 // guard the float root
        while ((rr + 1) * (rr + 2) / 2 <= q) ++rr;
        const int r = 16 * b + rr, i = 16 * b + q - rr * (rr + 1) / 2;
        float kk = 0.f, qk = 0.f;
        if (r < n) {
#pragma unroll 4
            for (int d = 0; d < DK; ++d) {
                const float dec = fexp(Gc[r][d] - Gc[i][d]);
                const float kd = load1(&Ks[i][d]) * dec;
                kk += load1(&Ks[r][d]) * kd;
                qk += load1(&Qs[r][d]) * kd;
            }
        }
        kkv[j] = kk;
        a.P[ch * kC * kC + r * kC + i] = qk;
    }
    // the diagonal tiles' upper halves of P
    for (int e = tid; e < 4 * 256; e += kPT) {
        const int b = e / 256, r = 16 * b + (e % 256) / 16, i = 16 * b + e % 16;
        if (i > r) a.P[ch * kC * kC + r * kC + i] = 0.f;
    }
    __syncthreads();   // every read of K and Q is done: A takes their place
    for (int e = tid; e < kC * kC; e += kPT) {
        const int r = e / kC, i = e % kC;
        if ((i >> 4) > (r >> 4) || ((i >> 4) == (r >> 4) && i > r)) A[r][i] = 0.f;
    }
    if (wave < 6) {
        const int rt = wave < 1 ? 1 : (wave < 3 ? 2 : 3);
        const int it = wave - (rt * (rt - 1)) / 2;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int rr = 16 * rt + 4 * lg + u, ii = 16 * it + lc;
            A[rr][ii] = Bt[rr] * ak[u];        // rows past n: K, Q rows are zero there
        }
    }
#pragma unroll
    for (int j = 0; j < kPairIt; ++j) {
        const int p = tid + j * kPT;
        if (p >= 4 * 136) continue;
        const int b = p / 136, q = p % 136;
        int rr = (int)((sqrtf(8.f * q + 1.f) - 1.f) * 0.5f);
        while (rr * (rr + 1) / 2 > q) --rr;
        while ((rr + 1) * (rr + 2) / 2 <= q) ++rr;
        const int r = 16 * b + rr, i = 16 * b + q - rr * (rr + 1) / 2;
        A[r][i] = i < r ? Bt[r] * kkv[j] : 0.f;
    }
    // the running log-decays for the scan (rows past n repeat row n-1: their g is zero)
    for (int u = tid; u < kC * DK / 4; u += kPT) {
        const int r = u / (DK / 4), d = (u % (DK / 4)) * 4;
        reinterpret_cast<float4*>(a.Gw + ch * kC * DK)[u] =
            make_float4(Gc[r][d], Gc[r][d + 1], Gc[r][d + 2], Gc[r][d + 3]);
    }
    __syncthreads();
    // T = (I + A)^{-1} by one wave (16x16 diagonal blocks by DPP substitution, then fp32 MFMA
    // levels), in place in LDS, then written out by the whole workgroup
    if (tid < kWave) unit_lower_inverse64<kC + 1, true>(&A[0][0]);
    __syncthreads();
    for (int e = tid; e < kC * kC; e += kPT) a.T[ch * kC * kC + e] = A[e / kC][e % kC];
}

// ------------------------------------------------------------------ scan per (seq, head, slice)
// Each chunk step's products run on the fp32 matrix core (v_mfma_f32_16x16x4f32), one 16x16
// output tile per wave. The decayed operands are formed as they are read: Kg = K o e^{Gc},
// Qg = Q o e^{Gc}, Kc = K o e^{Gc[last] - Gc} (one exponential per operand element; every
// exponent is <= 0). The next chunk's K, Q, Gc, T, P, V and beta are fetched into registers
// while this chunk computes.
template <int DK, int SL, typename Tin, typename Tout>
__global__ void __launch_bounds__(kST) kda_scan_kernel(KdaArgs a) {
    constexpr int CT = SL / 16, PR = SL + 1;
    constexpr int KR = DK + (sizeof(Tin) == 2 ? 2 : 1);   // K, Q row stride (4-byte aligned)
    __shared__ Tin Ks[kC][KR], Qs[kC][KR];
    __shared__ float Gs[kC][DK + 1];
    __shared__ float T[kC][kC + 1], P[kC][kC + 1];
    __shared__ float S[DK][PR];
    __shared__ float R[kC][PR], U[kC][PR];
    __shared__ float Bt[kC];
    const int slices = a.dv / SL;
    const int slice = blockIdx.x % slices;
    const int h = (blockIdx.x / slices) % a.H;
    const int sq = blockIdx.x / (slices * a.H);
    const int j0 = slice * SL, tid = threadIdx.x, H = a.H, dv = a.dv;
    const int wave = tid / kWave, lane = tid % kWave, lc = lane & 15, lg = lane >> 4;
    constexpr int NW = kST / kWave;
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    constexpr int NY = 4 * CT, NS = (DK / 16) * CT;         // output and state tiles
    static_assert(NY <= NW && NY + NS <= 2 * NW, "tiles per wave");
    Tout* y = static_cast<Tout*>(a.y);
    int lo, hi, cbase;
    kda_seq(a, sq, lo, hi, cbase);
    const size_t st_off = ((size_t)sq * H + h) * DK * dv;
    for (int e = tid; e < DK * SL; e += kST) {
        const int d = e / SL, j = e % SL;
        S[d][j] = a.S0 ? a.S0[st_off + (size_t)d * dv + j0 + j] : 0.f;
    }

    constexpr int PER = 16 / sizeof(Tin), KUNITS = kC * DK / PER;
    constexpr int KU = (KUNITS + kST - 1) / kST, GU = kC * DK / 4 / kST, VE = kC * SL / kST;
    static_assert(GU >= 1 && kC * kC / 4 == kST && VE >= 1, "prefetch shape");
    struct Pref {
        gdn_u32x4 k[KU], q[KU];
        float4 g[GU], t, p;
        float v[VE], b;
    };
    auto fetch = [&](int t0, int n, size_t ch, Pref& f) __attribute__((always_inline)) {
        const Tin* kp = static_cast<const Tin*>(a.k);
        const Tin* qp = static_cast<const Tin*>(a.q);
#pragma unroll
        for (int i = 0; i < KU; ++i) {
            const int u = tid + i * kST, r = u / (DK / PER), c0 = (u % (DK / PER)) * PER;
            f.k[i] = gdn_u32x4{0u, 0u, 0u, 0u};
            f.q[i] = gdn_u32x4{0u, 0u, 0u, 0u};
            if (u < KUNITS && r < n) {
                const size_t off = ((size_t)(t0 + r) * H + h) * DK + c0;
                f.k[i] = *reinterpret_cast<const gdn_u32x4*>(kp + off);
                f.q[i] = *reinterpret_cast<const gdn_u32x4*>(qp + off);
            }
        }
#pragma unroll
        for (int i = 0; i < GU; ++i) f.g[i] = reinterpret_cast<const float4*>(a.Gw + ch * kC * DK)[tid + i * kST];
        f.t = reinterpret_cast<const float4*>(a.T + ch * kC * kC)[tid];
        f.p = reinterpret_cast<const float4*>(a.P + ch * kC * kC)[tid];
#pragma unroll
        for (int i = 0; i < VE; ++i) {
            const int e = tid + i * kST, r = e / SL, j = e % SL;
            f.v[i] = r < n ? ldx<Tin>(a.v, ((size_t)(t0 + r) * H + h) * dv + j0 + j) : 0.f;
        }
        f.b = tid < n ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
    };
    auto put4 = [](float* d, float4 x) __attribute__((always_inline)) {
        d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
    };
    auto stash = [&](const Pref& f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KU; ++i) {
            const int u = tid + i * kST, r = u / (DK / PER), c0 = (u % (DK / PER)) * PER;
            if (u < KUNITS) {
                uint32_t* dk_ = reinterpret_cast<uint32_t*>(&Ks[r][c0]);
                uint32_t* dq_ = reinterpret_cast<uint32_t*>(&Qs[r][c0]);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    dk_[w] = f.k[i][w];
                    dq_[w] = f.q[i][w];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < GU; ++i) {
            const int u = tid + i * kST;
            put4(&Gs[u / (DK / 4)][(u % (DK / 4)) * 4], f.g[i]);
        }
        put4(&T[tid / (kC / 4)][(tid % (kC / 4)) * 4], f.t);
        put4(&P[tid / (kC / 4)][(tid % (kC / 4)) * 4], f.p);
#pragma unroll
        for (int i = 0; i < VE; ++i) {
            const int e = tid + i * kST;
            R[e / SL][e % SL] = f.v[i];
        }
        if (tid < kC) Bt[tid] = f.b;
    };

    Pref f;
    if (lo < hi) fetch(lo, min(kC, hi - lo), (size_t)cbase * H + h, f);
    for (int t0 = lo, c = cbase; t0 < hi; t0 += kC, ++c) {
        const int n = min(kC, hi - t0), last = n - 1;
        __syncthreads();
        stash(f);
        if (t0 + kC < hi) fetch(t0 + kC, min(kC, hi - t0 - kC), (size_t)(c + 1) * H + h, f);
        __syncthreads();
        if (wave < NY) {   // R = beta o (V - Kg S)
            const int rt = wave % 4, ct = wave / 4, r = rt * 16 + lc;
            floatx4 ks = zero;
#pragma unroll 4
            for (int k0 = 0; k0 < DK; k0 += 4) {
                const int d = k0 + lg;
                ks = __builtin_amdgcn_mfma_f32_16x16x4f32(load1(&Ks[r][d]) * fexp(Gs[r][d]),
                                                          S[d][ct * 16 + lc], ks, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = rt * 16 + 4 * lg + i, j = ct * 16 + lc;
                R[rr][j] = Bt[rr] * (R[rr][j] - ks[i]);
            }
        }
        __syncthreads();
        if (wave < NY) {   // U = T R (T lower triangular)
            const int rt = wave % 4, ct = wave / 4;
            const floatx4 u = mma_f32_tile(&T[rt * 16][0], kC + 1, 1, &R[0][ct * 16], PR, 1, kC, zero);
#pragma unroll
            for (int i = 0; i < 4; ++i) U[rt * 16 + 4 * lg + i][ct * 16 + lc] = u[i];
        }
        __syncthreads();
        // Y = Qg S + P U (rows past n are not stored) and S' = e^{Gc[last]} o S + Kc^T U, the
        // latter held in registers until every read of S is done
        floatx4 sn[2] = {zero, zero};
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            const int tile = wave + uu * NW;
            if (tile < NY) {
                const int rt = tile % 4, ct = tile / 4, r = rt * 16 + lc;
                floatx4 acc = zero;
#pragma unroll 4
                for (int k0 = 0; k0 < DK; k0 += 4) {
                    const int d = k0 + lg;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(load1(&Qs[r][d]) * fexp(Gs[r][d]),
                                                               S[d][ct * 16 + lc], acc, 0, 0, 0);
                }
                acc = mma_f32_tile(&P[rt * 16][0], kC + 1, 1, &U[0][ct * 16], PR, 1, kC, acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = rt * 16 + 4 * lg + i;
                    if (rr < n) store1(y + ((size_t)(t0 + rr) * H + h) * dv + j0 + ct * 16 + lc, acc[i]);
                }
            } else if (tile < NY + NS) {
                const int t2 = tile - NY, dt = t2 % (DK / 16), ct = t2 / (DK / 16);
                const int d = dt * 16 + lc;                  // this lane's key channel (A row)
                const float gl = Gs[last][d];
                floatx4 acc = zero;
#pragma unroll 4
                for (int k0 = 0; k0 < kC; k0 += 4) {
                    const int i = k0 + lg;                   // token (contraction index)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(load1(&Ks[i][d]) * fexp(gl - Gs[i][d]),
                                                               U[i][ct * 16 + lc], acc, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int dd = dt * 16 + 4 * lg + i;
                    sn[uu][i] = acc[i] + fexp(Gs[last][dd]) * S[dd][ct * 16 + lc];
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            const int tile = wave + uu * NW;
            if (tile >= NY && tile < NY + NS) {
                const int t2 = tile - NY, dt = t2 % (DK / 16), ct = t2 / (DK / 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[dt * 16 + 4 * lg + i][ct * 16 + lc] = sn[uu][i];
            }
        }
    }
    __syncthreads();
    if (a.ST) {
        for (int e = tid; e < DK * SL; e += kST) {
            const int d = e / SL, j = e % SL;
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
    a.Gw = reinterpret_cast<float*>(ws + L.Gw);
    const int nchunks = c.cu ? L.max_chunks : c.num_seqs * ((c.ntok / c.num_seqs + kC - 1) / kC);
    if (c.num_seqs * c.H == 0) return hipSuccess;
#define GDN_KDA(DK, TI, TO)                                                                      \
    do {                                                                                         \
        constexpr int SL = kda_cols<TI>();                                                       \
        if (nchunks > 0)                                                                         \
            hipLaunchKernelGGL((kda_prep_kernel<DK, TI>), dim3(nchunks, c.H), dim3(kPT), 0, s, a); \
        hipLaunchKernelGGL((kda_scan_kernel<DK, SL, TI, TO>), dim3(c.num_seqs * c.H * (c.dv / SL)), \
                           dim3(kST), 0, s, a);                                                 \
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
