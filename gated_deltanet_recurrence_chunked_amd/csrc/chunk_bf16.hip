// Chunkwise gated delta rule on gfx950 matrix cores (bf16 operands, fp32 accumulation,
// fp32 state). Reading notes of "On the Design of Qwen3.8-Next Architecture", section
// 2.1.1, eqs. (1)-(5); chunk length C = 64.
//
// Inside one chunk of one (sequence, head), with G_r the running sum of g = log(alpha),
// gamma_r = e^{G_r}, unrolling eq. (5) gives (rows = tokens):
//   A[r,i] = beta_r e^{G_r-G_i} (k_r . k_i) for i < r,   T = (I + A)^{-1}   (unit lower)
//   P[r,i] = e^{G_r-G_i} (q_r . k_i) for i <= r
//   R      = diag(beta) (V - diag(gamma) K S)             U = T R
//   Y      = diag(gamma) Q S + P U
//   S_next = gamma_C S + K^T diag(gamma_C / gamma) U
// Operands that are not exact bf16 inputs (S, R, T, U, P) enter the MFMAs as hi + lo bf16
// pairs (about 16 significant bits), so each such product costs two or three MFMAs.
// T and P depend on the chunk's q, k, g, beta only, so they are produced for every chunk at
// once by chunk_prep_kernel (massively parallel: KK^T and QK^T on MFMA, the 64x64 unit
// lower-triangular inverse by fp32 forward substitution). chunk_scan_kernel then walks the
// chunks of each (sequence, head) in order. The columns of S, V, U and Y are independent, so
// a scan workgroup owns a 32-column slice of dv: 4 workgroups per head at dv = 128, mapped to
// the same XCD so the shared q, k, T, P tiles are fetched from HBM once and hit that XCD's L2.
//
// MFMA v_mfma_f32_32x32x16_bf16 operand layout (lane l of 64): A element j is A[l%32][(l/32)*8+j],
// B element j is B[(l/32)*8+j][l%32], accumulator element i is C[8(i/4)+4(l/32)+i%4][l%32].
// Every LDS tile is stored with the contraction index contiguous (A as [row][k], B as
// [col][k]) so each operand fragment is one 16-byte LDS read; rows are padded by 16 bytes
// so the 32 rows read by one fragment load fall in distinct banks.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kC = 64;                // chunk length
constexpr int kThreads = 256;         // 4 waves
constexpr int kDK = 128;              // key dim of the matrix-core path
constexpr int kSl = 32;               // dv columns per scan workgroup
constexpr int kStrD = kDK + 8;        // LDS row stride (elements) of [*, 128] bf16 tiles
constexpr int kStrC = kC + 8;         // LDS row stride (elements) of [*, 64] bf16 tiles
constexpr int kStrA = kC + 4;         // LDS row stride of the fp32 A matrix
constexpr int kMaxSorted = 1024;      // longest-first ordering up to this many sequences

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 frag(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// accumulator element i of lane l -> tile row
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Stores the 32x32 accumulator tile, converted to bf16, transposed: dst[col][row0 + row].
__device__ __forceinline__ void store_acc_t(uint16_t* dst, int stride, int row0, const f32x16& c,
                                            int lane) {
    uint16_t* base = dst + (lane & 31) * stride + row0 + 4 * (lane >> 5);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        u32x2 v;
        v.x = pack_bf2(c[4 * q + 0], c[4 * q + 1]);
        v.y = pack_bf2(c[4 * q + 2], c[4 * q + 3]);
        *reinterpret_cast<u32x2*>(base + 8 * q) = v;
    }
}

// Same, as a two-term bf16 split: hi = bf16(x), lo = bf16(x - hi), so hi + lo carries about
// 16 significant bits; products against it take two MFMAs.
__device__ __forceinline__ void store_acc_t2(uint16_t* hi, uint16_t* lo, int stride, int row0,
                                             const f32x16& c, int lane) {
    const int off = (lane & 31) * stride + row0 + 4 * (lane >> 5);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        u32x2 vh, vl;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float x0 = c[4 * q + 2 * e], x1 = c[4 * q + 2 * e + 1];
            const uint32_t hp = pack_bf2(x0, x1);   // one v_cvt_pk_bf16_f32
            vh[e] = hp;
            vl[e] = pack_bf2(x0 - __uint_as_float(hp << 16), x1 - __uint_as_float(hp & 0xffff0000u));
        }
        *reinterpret_cast<u32x2*>(hi + off + 8 * q) = vh;
        *reinterpret_cast<u32x2*>(lo + off + 8 * q) = vl;
    }
}

struct Layout {
    size_t cs, ord, T, Tlo, P, Plo, total;
    int max_chunks;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Layout ws_layout(int ntok, int num_seqs, int H) {
    Layout L;
    L.max_chunks = (ntok + kC - 1) / kC + num_seqs;
    size_t o = 0;
    L.cs = o;  o = align256(o + sizeof(int32_t) * (num_seqs + 1));
    L.ord = o; o = align256(o + sizeof(int32_t) * num_seqs);
    const size_t tile = (size_t)kC * kC * sizeof(uint16_t);
    L.T = o;   o = align256(o + tile * L.max_chunks * H);
    L.Tlo = o; o = align256(o + tile * L.max_chunks * H);
    L.P = o;   o = align256(o + tile * L.max_chunks * H);
    L.Plo = o; o = align256(o + tile * L.max_chunks * H);
    L.total = o;
    return L;
}

struct DevArgs {
    const uint16_t *q, *k, *v;
    const float *g, *beta, *S0;
    float* ST;
    void* y;
    const int32_t* cu;          // NULL: equal lengths
    int32_t* chunk_start;       // [num_seqs+1] (varlen)
    int32_t* order;             // [num_seqs] longest first (varlen)
    uint16_t *Tw, *Tlw, *Pw, *Plw;  // [max_chunks][H][64][64]; T = Tw + Tlw, P = Pw + Plw (hi + lo)
    int num_seqs, ntok, H, dv, L;  // L: equal length (when cu == NULL)
    int y_bf16;
};

// ------------------------------------------------------------------ chunk table (varlen)
__global__ void __launch_bounds__(kThreads) chunk_table_kernel(DevArgs a) {
    __shared__ int scan[kThreads];
    const int tid = threadIdx.x;
    int running = 0;
    if (tid == 0) a.chunk_start[0] = 0;
    for (int base = 0; base < a.num_seqs; base += kThreads) {
        const int s = base + tid;
        const int c = s < a.num_seqs ? (a.cu[s + 1] - a.cu[s] + kC - 1) / kC : 0;
        scan[tid] = c;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {
            const int v = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += v;
            __syncthreads();
        }
        if (s < a.num_seqs) a.chunk_start[s + 1] = running + scan[tid];
        running += scan[kThreads - 1];
        __syncthreads();
    }
    // longest sequences first, so their scans start first (stable for equal lengths)
    for (int i = tid; i < a.num_seqs; i += kThreads) {
        if (a.num_seqs > kMaxSorted) {
            a.order[i] = i;
            continue;
        }
        const int Li = a.cu[i + 1] - a.cu[i];
        int rank = 0;
        for (int j = 0; j < a.num_seqs; ++j) {
            const int Lj = a.cu[j + 1] - a.cu[j];
            rank += (Lj > Li) || (Lj == Li && j < i);
        }
        a.order[rank] = i;
    }
}

// Rows [0, 64) of one chunk of a [ntok, H, 128] bf16 tensor: 256 threads x 4 x 16 bytes,
// fetched into registers (all loads in flight together; rows >= n read row n-1 and are
// zeroed when written to LDS, so no load sits behind a branch).
// The chunk's base address is wave-uniform (scalar registers); a lane adds a 32-bit offset.
__device__ __forceinline__ void fetch_rows128(u32x4 (&R)[4], const uint16_t* src, int t0, int n,
                                              int H, int h) {
    const uint16_t* base = src + ((size_t)t0 * H + h) * kDK;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = threadIdx.x + kThreads * it;
        const int r = min(idx >> 4, n - 1), d0 = (idx & 15) * 8;
        R[it] = *reinterpret_cast<const u32x4*>(base + (r * H * kDK + d0));
    }
}
__device__ __forceinline__ void put_rows128(uint16_t* dst, const u32x4 (&R)[4], int n) {
    if (n == kC) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = threadIdx.x + kThreads * it;
            *reinterpret_cast<u32x4*>(dst + (idx >> 4) * kStrD + (idx & 15) * 8) = R[it];
        }
        return;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = threadIdx.x + kThreads * it;
        const int r = idx >> 4, d0 = (idx & 15) * 8;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(dst + r * kStrD + d0) = r < n ? R[it] : z;
    }
}

// Wave 0: the chunk's gates (lane = token; rows >= n read row n-1, zeroed below).
__device__ __forceinline__ void fetch_gates(const DevArgs& a, int t0, int n, int h, float& gv,
                                            float& bv) {
    const int r = min((int)(threadIdx.x & (kWave - 1)), n - 1);
    const size_t base = (size_t)t0 * a.H + h;
    gv = a.g[base + r * a.H];
    bv = a.beta[base + r * a.H];
}

// Wave 0: running sum of g over the chunk (rows >= n contribute 0), written with beta.
__device__ __forceinline__ void chunk_gates(float gv, float bv, int n, float* sG, float* sB,
                                            float* sGam, float* sGd) {
    const int lane = threadIdx.x;
    if (lane >= n) {
        gv = 0.f;
        bv = 0.f;
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float o = __shfl_up(gv, off, kWave);
        if (lane >= off) gv += o;
    }
    const float gC = __shfl(gv, kC - 1, kWave);
    sG[lane] = gv;
    sB[lane] = bv;
    if (sGam) sGam[lane] = fexp(gv);
    if (sGd) sGd[lane] = fexp(gC - gv);
}

// chunk index -> (sequence, first token, length)
__device__ __forceinline__ bool chunk_of(const DevArgs& a, int chunk, int& seq, int& t0, int& n) {
    if (!a.cu) {
        const int cps = (a.L + kC - 1) / kC;
        if (cps == 0) return false;
        seq = chunk / cps;
        if (seq >= a.num_seqs) return false;
        const int c = chunk - seq * cps;
        t0 = seq * a.L + c * kC;
        n = min(kC, a.L - c * kC);
        return true;
    }
    if (chunk >= a.chunk_start[a.num_seqs]) return false;
    int lo = 0, hi = a.num_seqs;   // chunk_start[lo] <= chunk < chunk_start[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.chunk_start[mid] <= chunk) lo = mid; else hi = mid;
    }
    seq = lo;
    const int c = chunk - a.chunk_start[seq];
    t0 = a.cu[seq] + c * kC;
    n = min(kC, a.cu[seq + 1] - t0);
    return true;
}

// ------------------------------------------------------------------ per-chunk T and P
// One wave per (chunk, head). The MFMA operands of K K^T and Q K^T are read from global
// memory straight into registers in fragment layout (a lane's 8 consecutive d_k of one row
// are one 16-byte load), so only the fp32 A matrix lives in LDS and eight chunk-heads share
// a CU: while one wave waits on its loads or on the forward substitution (a lane per column
// of T), the other wave on its SIMD issues.
constexpr int kPrepThreads = kWave;

__global__ void __launch_bounds__(kPrepThreads, 2) chunk_prep_kernel(DevArgs a) {
    __shared__ __attribute__((aligned(16))) float sA[kC * kStrA];
    __shared__ float sG[kC], sB[kC];

    const int chunk = blockIdx.x, h = blockIdx.y;
    int seq, t0, n;
    if (!chunk_of(a, chunk, seq, t0, n)) return;
    const int lane = threadIdx.x;

    // fragment rows (lane % 32) and (32 + lane % 32); rows >= n are zero
    const int r0 = lane & 31, r1 = 32 + (lane & 31);
    const uint16_t* k0p = a.k + ((size_t)(t0 + min(r0, n - 1)) * a.H + h) * kDK + (lane >> 5) * 8;
    const uint16_t* k1p = a.k + ((size_t)(t0 + min(r1, n - 1)) * a.H + h) * kDK + (lane >> 5) * 8;
    const uint16_t* q0p = a.q + ((size_t)(t0 + min(r0, n - 1)) * a.H + h) * kDK + (lane >> 5) * 8;
    const uint16_t* q1p = a.q + ((size_t)(t0 + min(r1, n - 1)) * a.H + h) * kDK + (lane >> 5) * 8;
    u32x4 fk0[8], fk1[8], fq0[8], fq1[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        fk0[kk] = *reinterpret_cast<const u32x4*>(k0p + kk * 16);
        fk1[kk] = *reinterpret_cast<const u32x4*>(k1p + kk * 16);
        fq0[kk] = *reinterpret_cast<const u32x4*>(q0p + kk * 16);
        fq1[kk] = *reinterpret_cast<const u32x4*>(q1p + kk * 16);
    }
    float gv, bv;
    fetch_gates(a, t0, n, h, gv, bv);
    chunk_gates(gv, bv, n, sG, sB, nullptr, nullptr);
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool v0 = r0 < n, v1 = r1 < n;

    // lower tiles of K K^T and Q K^T: (rows 0-31, cols 0-31), (32-63, 0-31), (32-63, 32-63)
    f32x16 ckk[3], cqk[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        ckk[t] = f32x16{};
        cqk[t] = f32x16{};
    }
#pragma unroll
    for (int kk = 0; kk < kDK / 16; ++kk) {
        const bf16x8 k0 = __builtin_bit_cast(bf16x8, v0 ? fk0[kk] : z);
        const bf16x8 k1 = __builtin_bit_cast(bf16x8, v1 ? fk1[kk] : z);
        const bf16x8 q0 = __builtin_bit_cast(bf16x8, v0 ? fq0[kk] : z);
        const bf16x8 q1 = __builtin_bit_cast(bf16x8, v1 ? fq1[kk] : z);
        ckk[0] = mfma(k0, k0, ckk[0]);
        ckk[1] = mfma(k1, k0, ckk[1]);
        ckk[2] = mfma(k1, k1, ckk[2]);
        cqk[0] = mfma(q0, k0, cqk[0]);
        cqk[1] = mfma(q1, k0, cqk[1]);
        cqk[2] = mfma(q1, k1, cqk[2]);
    }
    __syncthreads();   // gates visible

    const size_t tile = ((size_t)chunk * a.H + h) * kC * kC;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int R0 = t == 0 ? 0 : 32, C0 = t == 2 ? 32 : 0;
        const int c = C0 + (lane & 31);
        const float Gc = sG[c];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = R0 + acc_row(i, lane);
            const float dec = c <= r ? fexp(sG[r] - Gc) : 0.f;
            sA[r * kStrA + c] = c < r ? sB[r] * dec * ckk[t][i] : 0.f;
            cqk[t][i] *= dec;   // P, written out after T
        }
    }
    __syncthreads();
    // T = (I + A)^{-1} in 32x32 blocks: T = [[T0, 0], [T10, T1]] with T0 = (I + A00)^{-1},
    // T1 = (I + A11)^{-1}, T10 = -T1 A10 T0.
    // (1) the two diagonal inverses by forward substitution, one half-wave each, a lane per
    //     column (4 partial sums per row);
    const int half = lane >> 5, c = lane & 31, off = 32 * half;
    float t[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        const float* Ar = sA + (off + r) * kStrA + off;
        float acc[4] = {r == c ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < r; ++i) acc[i & 3] -= Ar[i] * t[i];
        t[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    __syncthreads();   // all reads of A00 and A11 done: T0 and T1 take their place
#pragma unroll
    for (int r = 0; r < 32; ++r) sA[(off + r) * kStrA + off + c] = t[r];
    __syncthreads();
    // (2) X = A10 T0 and T10 = -T1 X on the fp32 matrix cores (v_mfma_f32_32x32x2_f32: lane l
    //     supplies A[l%32][l/32] and B[l/32][l%32] of each k-pair); X goes through the unused
    //     upper-right block of the tile.
    f32x16 X = {};
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
        const int k = 2 * s2 + half;
        X = __builtin_amdgcn_mfma_f32_32x32x2f32(sA[(32 + c) * kStrA + k], sA[k * kStrA + c], X, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[acc_row(i, lane) * kStrA + 32 + c] = X[i];
    __syncthreads();
    f32x16 T10 = {};
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
        const int k = 2 * s2 + half;
        T10 = __builtin_amdgcn_mfma_f32_32x32x2f32(sA[(32 + c) * kStrA + 32 + k], sA[k * kStrA + 32 + c],
                                                  T10, 0, 0, 0);
    }
    // (3) T and P as hi + lo bf16 tiles, assembled in LDS (the A matrix is dead now) and
    //     written as whole 128-byte rows. T's upper-right block is never read; it is zero.
    __syncthreads();
    uint16_t* sH = reinterpret_cast<uint16_t*>(sA);   // [64][64] hi
    uint16_t* sL = sH + kC * kC;                      // [64][64] lo
    auto put = [&](int r, int cc, float v) {
        const uint16_t hb = f2bf(v);
        sH[r * kC + cc] = hb;
        sL[r * kC + cc] = f2bf(v - bf2f(hb));
    };
    auto flush = [&](uint16_t* dh, uint16_t* dl) {
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kC * kC / 8 / kWave; ++it) {
            const int e = (lane + kWave * it) * 8;
            *reinterpret_cast<u32x4*>(dh + tile + e) = *reinterpret_cast<const u32x4*>(sH + e);
            *reinterpret_cast<u32x4*>(dl + tile + e) = *reinterpret_cast<const u32x4*>(sL + e);
        }
        __syncthreads();
    };
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        put(off + r, off + c, t[r]);
        put(r, 32 + c, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) put(32 + acc_row(i, lane), c, -T10[i]);
    flush(a.Tw, a.Tlw);
#pragma unroll
    for (int tt = 0; tt < 3; ++tt) {
        const int R0 = tt == 0 ? 0 : 32, C0 = tt == 2 ? 32 : 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) put(R0 + acc_row(i, lane), C0 + c, cqk[tt][i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) put(acc_row(i, lane), 32 + c, 0.f);
    flush(a.Pw, a.Plw);
}

// ------------------------------------------------------------------ sequential chunk scan
constexpr int kStrV = kSl + 8;

// Next chunk's inputs, held in registers while the current chunk computes (all loads are
// unconditional so the compiler keeps them in VGPRs and waits for them only where used).
#define GDN_FETCH_STAGE(T0, N, TILE)                                                           \
    do {                                                                                       \
        fetch_rows128(stq, a.q, (T0), (N), a.H, h);                                            \
        fetch_rows128(stk, a.k, (T0), (N), a.H, h);                                            \
        _Pragma("unroll") for (int it = 0; it < 2; ++it) {                                     \
            const int off = tid * 8 + kThreads * 8 * it;   /* = row * 64 + col */              \
            stt[it] = *reinterpret_cast<const u32x4*>(a.Tw + (TILE) + off);                    \
            sttl[it] = *reinterpret_cast<const u32x4*>(a.Tlw + (TILE) + off);                  \
            stp[it] = *reinterpret_cast<const u32x4*>(a.Pw + (TILE) + off);                    \
            stpl[it] = *reinterpret_cast<const u32x4*>(a.Plw + (TILE) + off);                  \
        }                                                                                      \
        const int vr = min(tid >> 2, (N) - 1);                                                 \
        stv = *reinterpret_cast<const u32x4*>(a.v + ((size_t)(T0) * a.H + h) * a.dv + j0 +    \
                                              (vr * a.H * a.dv + (tid & 3) * 8));              \
        fetch_gates(a, (T0), (N), h, stg, stb);                                                \
    } while (0)

template <typename Ty>
__global__ void __launch_bounds__(kThreads) chunk_scan_kernel(DevArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sQ[kC * kStrD];
    __shared__ __attribute__((aligned(16))) uint16_t sK[kC * kStrD];
    __shared__ __attribute__((aligned(16))) uint16_t sT[kC * kStrC];
    __shared__ __attribute__((aligned(16))) uint16_t sTl[kC * kStrC];
    __shared__ __attribute__((aligned(16))) uint16_t sP[kC * kStrC];
    __shared__ __attribute__((aligned(16))) uint16_t sPl[kC * kStrC];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kC * kStrV];
    __shared__ __attribute__((aligned(16))) uint16_t sSt[kSl * kStrD];    // S^T hi
    __shared__ __attribute__((aligned(16))) uint16_t sStl[kSl * kStrD];   // S^T lo
    __shared__ __attribute__((aligned(16))) uint16_t sRt[kSl * kStrC];
    __shared__ __attribute__((aligned(16))) uint16_t sRtl[kSl * kStrC];
    __shared__ __attribute__((aligned(16))) uint16_t sUt[kSl * kStrC];
    __shared__ __attribute__((aligned(16))) uint16_t sUtl[kSl * kStrC];
    __shared__ __attribute__((aligned(16))) uint16_t sUht[kSl * kStrC];   // (diag(gamma_C/gamma) U)^T
    __shared__ __attribute__((aligned(16))) uint16_t sUhtl[kSl * kStrC];
    constexpr int kStrY = sizeof(Ty) == 2 ? kSl + 8 : kSl + 4;          // 16-byte aligned rows
    __shared__ __attribute__((aligned(16))) Ty sY[kC * kStrY];            // the chunk's y slice
    __shared__ float sG[kC], sB[kC], sGam[kC], sGd[kC];

    // block -> (pair, slice): the slices of one pair are 8 blocks apart, so the same XCD
    const int nsl = a.dv / kSl;
    const int b = blockIdx.x;
    const int group = b / (8 * nsl), within = b % (8 * nsl);
    const int slice = within >> 3;
    const int pair = group * 8 + (within & 7);
    if (pair >= a.num_seqs * a.H) return;
    const int rank = pair / a.H, h = pair % a.H;
    const int seq = a.order ? a.order[rank] : rank;
    int lo, hi, cbase;
    if (a.cu) {
        lo = a.cu[seq];
        hi = a.cu[seq + 1];
        cbase = a.chunk_start[seq];
    } else {
        lo = seq * a.L;
        hi = lo + a.L;
        cbase = seq * ((a.L + kC - 1) / kC);
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j0 = slice * kSl;
    const int col = lane & 31;
    const int kofs = (lane >> 5) * 8;
    const size_t sbase = ((size_t)seq * a.H + h) * kDK * a.dv;

    // state rows [32 wave, 32 wave + 32) of this slice, accumulator layout
    f32x16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = 32 * wave + acc_row(i, lane);
        S[i] = a.S0 ? a.S0[sbase + (size_t)row * a.dv + j0 + col] : 0.f;
    }
    store_acc_t2(sSt, sStl, kStrD, 32 * wave, S, lane);

    const int nchunks = (hi - lo + kC - 1) / kC;
    u32x4 stq[4], stk[4], stt[2], sttl[2], stp[2], stpl[2], stv;
    float stg, stb;
    if (nchunks > 0) GDN_FETCH_STAGE(lo, min(kC, hi - lo), ((size_t)cbase * a.H + h) * kC * kC);
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = lo + c * kC;
        const int n = min(kC, hi - t0);
        // ---- commit the staged chunk to LDS
        put_rows128(sQ, stq, n);
        put_rows128(sK, stk, n);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = tid + kThreads * it;
            const int o = (idx >> 3) * kStrC + (idx & 7) * 8;
            *reinterpret_cast<u32x4*>(sT + o) = stt[it];
            *reinterpret_cast<u32x4*>(sTl + o) = sttl[it];
            *reinterpret_cast<u32x4*>(sP + o) = stp[it];
            *reinterpret_cast<u32x4*>(sPl + o) = stpl[it];
        }
        {
            const int r = tid >> 2;
            const u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(sV + r * kStrV + (tid & 3) * 8) = (n == kC || r < n) ? stv : z;
        }
        if (wave == 0) chunk_gates(stg, stb, n, sG, sB, sGam, sGd);
        __syncthreads();
        // ---- prefetch the next chunk while this one computes (the last chunk re-reads itself)
        {
            const int cn = min(c + 1, nchunks - 1);
            const int t1 = lo + cn * kC;
            GDN_FETCH_STAGE(t1, min(kC, hi - t1), ((size_t)(cbase + cn) * a.H + h) * kC * kC);
        }

        // ---- step 1: [Q; K] S (waves 0, 1: Q rows; waves 2, 3: K rows), S = S_hi + S_lo
        f32x16 acc = {};
        {
            const uint16_t* Arow = (wave < 2 ? sQ : sK) + (32 * (wave & 1) + col) * kStrD + kofs;
            const uint16_t* Bh = sSt + col * kStrD + kofs;
            const uint16_t* Bl = sStl + col * kStrD + kofs;
#pragma unroll
            for (int kk = 0; kk < kDK / 16; ++kk) {
                const bf16x8 af = frag(Arow + kk * 16);
                acc = mfma(af, frag(Bh + kk * 16), acc);
                acc = mfma(af, frag(Bl + kk * 16), acc);
            }
        }
        if (wave >= 2) {
            // R = beta (V - gamma K S)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 32 * (wave - 2) + acc_row(i, lane);
                acc[i] = sB[r] * (bf2f(sV[r * kStrV + col]) - sGam[r] * acc[i]);
            }
            store_acc_t2(sRt, sRtl, kStrC, 32 * (wave - 2), acc, lane);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] *= sGam[32 * wave + acc_row(i, lane)];
        }
        __syncthreads();

        // ---- step 2: U = T R (T is unit lower triangular: rows 0-31 need k < 32 only),
        //      T = T_hi + T_lo, R = R_hi + R_lo (the lo x lo term is below fp32 rounding)
        if (wave >= 2) {
            const int r0 = 32 * (wave - 2);
            f32x16 u = {};
            const uint16_t* Ah = sT + (r0 + col) * kStrC + kofs;
            const uint16_t* Al = sTl + (r0 + col) * kStrC + kofs;
            const uint16_t* Bh = sRt + col * kStrC + kofs;
            const uint16_t* Bl = sRtl + col * kStrC + kofs;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 2 * (wave - 1)) {
                    const bf16x8 ah = frag(Ah + kk * 16), bh = frag(Bh + kk * 16);
                    u = mfma(ah, bh, u);
                    u = mfma(ah, frag(Bl + kk * 16), u);
                    u = mfma(frag(Al + kk * 16), bh, u);
                }
            }
            store_acc_t2(sUt, sUtl, kStrC, r0, u, lane);
#pragma unroll
            for (int i = 0; i < 16; ++i) u[i] *= sGd[r0 + acc_row(i, lane)];
            store_acc_t2(sUht, sUhtl, kStrC, r0, u, lane);
        }
        __syncthreads();

        // ---- step 3a: Y = gamma Q S + P U  (waves 0, 1), P = P_hi + P_lo, U = U_hi + U_lo
        if (wave < 2) {
            const uint16_t* Ah = sP + (32 * wave + col) * kStrC + kofs;
            const uint16_t* Al = sPl + (32 * wave + col) * kStrC + kofs;
            const uint16_t* Bh = sUt + col * kStrC + kofs;
            const uint16_t* Bl = sUtl + col * kStrC + kofs;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 2 * (wave + 1)) {
                    const bf16x8 ah = frag(Ah + kk * 16), bh = frag(Bh + kk * 16);
                    acc = mfma(ah, bh, acc);
                    acc = mfma(ah, frag(Bl + kk * 16), acc);
                    acc = mfma(frag(Al + kk * 16), bh, acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) store1(sY + (32 * wave + acc_row(i, lane)) * kStrY + col, acc[i]);
        }
        // ---- step 3b: S = gamma_C S + K^T Uh  (rows 32 wave.. of S; K^T fragments read
        //      column-wise from the row-major K tile)
        {
            const float gC = sGam[kC - 1];
#pragma unroll
            for (int i = 0; i < 16; ++i) S[i] *= gC;
            const int d = 32 * wave + col;
            const uint16_t* Bh = sUht + col * kStrC + kofs;
            const uint16_t* Bl = sUhtl + col * kStrC + kofs;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int ko = kk * 16 + kofs;
                bf16x8 af;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    af[j] = __builtin_bit_cast(__bf16, sK[(ko + j) * kStrD + d]);
                S = mfma(af, frag(Bh + kk * 16), S);
                S = mfma(af, frag(Bl + kk * 16), S);
            }
            store_acc_t2(sSt, sStl, kStrD, 32 * wave, S, lane);
        }
        __syncthreads();
        // ---- the chunk's y slice: 16-byte stores of whole rows
        {
            constexpr int kPer = 8 / sizeof(Ty) * 2;          // elements per 16 bytes
            constexpr int kRowPieces = kSl / kPer;
#pragma unroll
            for (int it = 0; it < kC * kRowPieces / kThreads; ++it) {
                const int idx = tid + kThreads * it;
                const int r = idx / kRowPieces, c0 = (idx % kRowPieces) * kPer;
                if (r < n)
                    *reinterpret_cast<u32x4*>(static_cast<Ty*>(a.y) + ((size_t)(t0 + r) * a.H + h) * a.dv +
                                              j0 + c0) = *reinterpret_cast<const u32x4*>(sY + r * kStrY + c0);
            }
        }
    }
    if (a.ST) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 32 * wave + acc_row(i, lane);
            a.ST[sbase + (size_t)row * a.dv + j0 + col] = S[i];
        }
    }
}
#undef GDN_FETCH_STAGE

}  // namespace

size_t chunk_bf16_workspace(int ntok, int num_seqs, int H) {
    return ws_layout(ntok, num_seqs, H).total;
}

hipError_t launch_chunk_bf16(const ChunkArgs& c, hipStream_t s) {
    const Layout L = ws_layout(c.ntok, c.num_seqs, c.H);
    char* ws = static_cast<char*>(c.workspace);
    DevArgs a;
    a.q = static_cast<const uint16_t*>(c.q);
    a.k = static_cast<const uint16_t*>(c.k);
    a.v = static_cast<const uint16_t*>(c.v);
    a.g = c.g; a.beta = c.beta; a.S0 = c.S0; a.ST = c.ST; a.y = c.y;
    a.cu = c.cu;
    a.chunk_start = c.cu ? reinterpret_cast<int32_t*>(ws + L.cs) : nullptr;
    a.order = c.cu ? reinterpret_cast<int32_t*>(ws + L.ord) : nullptr;
    a.Tw = reinterpret_cast<uint16_t*>(ws + L.T);
    a.Tlw = reinterpret_cast<uint16_t*>(ws + L.Tlo);
    a.Pw = reinterpret_cast<uint16_t*>(ws + L.P);
    a.Plw = reinterpret_cast<uint16_t*>(ws + L.Plo);
    a.num_seqs = c.num_seqs; a.ntok = c.ntok; a.H = c.H; a.dv = c.dv;
    a.L = c.cu ? 0 : c.ntok / c.num_seqs;
    a.y_bf16 = c.y_bf16;
    if (c.cu) hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kThreads), 0, s, a);
    const int nchunks = c.cu ? L.max_chunks : c.num_seqs * ((a.L + kC - 1) / kC);
    if (nchunks > 0)
        hipLaunchKernelGGL(chunk_prep_kernel, dim3(nchunks, c.H), dim3(kPrepThreads), 0, s, a);
    const int nsl = c.dv / kSl;
    const int pairs = c.num_seqs * c.H;
    const int blocks = (pairs + 7) / 8 * 8 * nsl;
    if (c.y_bf16)
        hipLaunchKernelGGL(chunk_scan_kernel<uint16_t>, dim3(blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(chunk_scan_kernel<float>, dim3(blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gdn
