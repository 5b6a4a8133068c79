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
// The state-side operands S, R and U enter the MFMAs as hi + lo bf16 pairs (about 16
// significant bits: two MFMAs per product); the chunk-local T and P are single bf16.
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
    size_t cs, ord, T, P, Gt, total;
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
    L.P = o;   o = align256(o + tile * L.max_chunks * H);
    L.Gt = o;  o = align256(o + sizeof(float) * 3 * kC * (size_t)L.max_chunks * H);
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
    uint16_t *Tw, *Pw;          // [max_chunks][H][64][64] bf16
    float* Gw;                  // [max_chunks][H][3][64]: beta, gamma = e^G, gamma_C / gamma
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
    {
        // the chunk's beta, gamma_r = e^{G_r} and gamma_C / gamma_r for the scan
        float* gw = a.Gw + ((size_t)chunk * a.H + h) * 3 * kC;
        float Gr = lane < n ? gv : 0.f;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float o = __shfl_up(Gr, off, kWave);
            if (lane >= off) Gr += o;
        }
        const float GC = __shfl(Gr, kC - 1, kWave);
        gw[lane] = lane < n ? bv : 0.f;
        gw[kC + lane] = fexp(Gr);
        gw[2 * kC + lane] = fexp(GC - Gr);
    }
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
    // (3) T and P as bf16 tiles, assembled in LDS (the A matrix is dead now) and written as
    //     whole 128-byte rows. T's upper-right block is never read; it is zero.
    __syncthreads();
    uint16_t* sH = reinterpret_cast<uint16_t*>(sA);   // [64][64]
    auto put = [&](int r, int cc, float v) { sH[r * kC + cc] = f2bf(v); };
    auto flush = [&](uint16_t* dh) {
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kC * kC / 8 / kWave; ++it) {
            const int e = (lane + kWave * it) * 8;
            *reinterpret_cast<u32x4*>(dh + tile + e) = *reinterpret_cast<const u32x4*>(sH + e);
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
    flush(a.Tw);
#pragma unroll
    for (int tt = 0; tt < 3; ++tt) {
        const int R0 = tt == 0 ? 0 : 32, C0 = tt == 2 ? 32 : 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) put(R0 + acc_row(i, lane), C0 + c, cqk[tt][i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) put(acc_row(i, lane), 32 + c, 0.f);
    flush(a.Pw);
}

// ------------------------------------------------------------------ sequential chunk scan
// One 8-wave workgroup per (sequence, head, 32-column dv slice); two waves per SIMD, so the
// latency of one wave's LDS reads and MFMAs hides behind the other's work. Products are
// tiled in 16x16 blocks (v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][(l/16)*8+j] and
// B[(l/16)*8+j][l%16]; accumulator element i is C[(l/16)*4+i][l%16]) and every wave owns
// 16 rows of each product:
//   step 1  waves 0-3: rows 16w.. of Q S (kept for Y);  waves 4-7: rows of K S -> R
//   step 2  waves 4-7: rows of U = T R (and diag(gamma_C/gamma) U)
//   step 3  waves 0-3: rows of Y = gamma Q S + P U;  all waves: d_k rows 16w.. of the state
// The fp32 state lives in registers (2 tiles per wave); bf16 hi + lo copies of S, R, U go
// through LDS as the next product's B operand.
constexpr int kScanThreads = 512;
constexpr int kStrV = kSl + 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16 accumulator tile -> transposed bf16 hi + lo: dst[col0 + col][row0 + row]
__device__ __forceinline__ void store16_t2(uint16_t* hi, uint16_t* lo, int stride, int row0, int col0,
                                           const f32x4& c, int lane) {
    const int off = (col0 + (lane & 15)) * stride + row0 + 4 * (lane >> 4);
    u32x2 vh, vl;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float x0 = c[2 * e], x1 = c[2 * e + 1];
        const uint32_t hp = pack_bf2(x0, x1);
        vh[e] = hp;
        vl[e] = pack_bf2(x0 - __uint_as_float(hp << 16), x1 - __uint_as_float(hp & 0xffff0000u));
    }
    *reinterpret_cast<u32x2*>(hi + off) = vh;
    *reinterpret_cast<u32x2*>(lo + off) = vl;
}

template <typename Ty>
__global__ void __launch_bounds__(kScanThreads) chunk_scan_kernel(DevArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sQ[kC * kStrD];
    __shared__ __attribute__((aligned(16))) uint16_t sK[kC * kStrD];
    __shared__ __attribute__((aligned(16))) uint16_t sKt[kDK * kStrC];    // K^T: [d_k][token]
    __shared__ __attribute__((aligned(16))) uint16_t sT[kC * kStrC];
    __shared__ __attribute__((aligned(16))) uint16_t sP[kC * kStrC];
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
    __shared__ __attribute__((aligned(16))) float sGates[3 * kC];       // beta, gamma, gamma_C/gamma
    const float* sB = sGates;
    const float* sGam = sGates + kC;
    const float* sGd = sGates + 2 * kC;

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
    const int c16 = lane & 15;              // tile column
    const int r4 = 4 * (lane >> 4);         // first of the lane's 4 accumulator rows
    const int kq = (lane >> 4) * 8;         // the lane's k offset inside a 32-wide k step
    const int rb = wave & 3;                // 16-row block of steps 1-3a
    const size_t sbase = ((size_t)seq * a.H + h) * kDK * a.dv;

    // state rows [16 wave, 16 wave + 16) x 32 columns: two 16x16 accumulator tiles
    f32x4 S[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * wave + r4 + i;
            S[ct][i] = a.S0 ? a.S0[sbase + (size_t)row * a.dv + j0 + 16 * ct + c16] : 0.f;
        }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) store16_t2(sSt, sStl, kStrD, 16 * wave, 16 * ct, S[ct], lane);

    // next chunk's inputs, staged in registers while the current chunk computes
    const int nchunks = (hi - lo + kC - 1) / kC;
    // K pieces are taken token-fastest across lanes (token idx % 64, d_k group idx / 64), so
    // the transposed copy K^T is written as contiguous 128-byte runs of one d_k row.
    u32x4 stq[2], stk[2], stt, stp, stv, stgt;
    auto fetch = [&](int t0, int n, size_t tile) {
        const uint16_t* qb = a.q + ((size_t)t0 * a.H + h) * kDK;
        const uint16_t* kb = a.k + ((size_t)t0 * a.H + h) * kDK;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = tid + kScanThreads * it;
            const int r = min(idx >> 4, n - 1), d0 = (idx & 15) * 8;
            stq[it] = *reinterpret_cast<const u32x4*>(qb + (r * a.H * kDK + d0));
            const int rk = min(idx & 63, n - 1), dk0 = (idx >> 6) * 8;
            stk[it] = *reinterpret_cast<const u32x4*>(kb + (rk * a.H * kDK + dk0));
        }
        const int off = tid * 8;   // row * 64 + col of the 64x64 tiles
        stt = *reinterpret_cast<const u32x4*>(a.Tw + tile + off);
        stp = *reinterpret_cast<const u32x4*>(a.Pw + tile + off);
        const int vr = min((tid & 255) >> 2, n - 1);
        stv = *reinterpret_cast<const u32x4*>(a.v + ((size_t)t0 * a.H + h) * a.dv + j0 +
                                              (vr * a.H * a.dv + (tid & 3) * 8));
        stgt = *reinterpret_cast<const u32x4*>(a.Gw + tile / (kC * kC) * 3 * kC + 4 * (tid % 48));
    };
    if (nchunks > 0) fetch(lo, min(kC, hi - lo), ((size_t)cbase * a.H + h) * kC * kC);

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = lo + c * kC;
        const int n = min(kC, hi - t0);
        // ---- commit the staged chunk to LDS
        {
            const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int idx = tid + kScanThreads * it;
                const int r = idx >> 4, o = r * kStrD + (idx & 15) * 8;
                *reinterpret_cast<u32x4*>(sQ + o) = (n == kC || r < n) ? stq[it] : z;
                const int rk = idx & 63, dk0 = (idx >> 6) * 8;
                const u32x4 kv = (n == kC || rk < n) ? stk[it] : z;
                *reinterpret_cast<u32x4*>(sK + rk * kStrD + dk0) = kv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sKt[(dk0 + 2 * e) * kStrC + rk] = uint16_t(kv[e] & 0xffffu);
                    sKt[(dk0 + 2 * e + 1) * kStrC + rk] = uint16_t(kv[e] >> 16);
                }
            }
            if (tid < 48) *reinterpret_cast<u32x4*>(sGates + 4 * tid) = stgt;
            const int o = (tid >> 3) * kStrC + (tid & 7) * 8;
            *reinterpret_cast<u32x4*>(sT + o) = stt;
            *reinterpret_cast<u32x4*>(sP + o) = stp;
            if (tid < 256) {
                const int r = tid >> 2;
                *reinterpret_cast<u32x4*>(sV + r * kStrV + (tid & 3) * 8) = (n == kC || r < n) ? stv : z;
            }
        }
        __syncthreads();
        // ---- prefetch the next chunk (the last chunk re-reads itself)
        {
            const int cn = min(c + 1, nchunks - 1);
            const int t1 = lo + cn * kC;
            fetch(t1, min(kC, hi - t1), ((size_t)(cbase + cn) * a.H + h) * kC * kC);
        }

        // ---- step 1: rows 16 rb.. of Q S (waves 0-3) or K S (waves 4-7), S = S_hi + S_lo
        f32x4 acc[2] = {f32x4{}, f32x4{}};
        {
            const uint16_t* Arow = (wave < 4 ? sQ : sK) + (16 * rb + c16) * kStrD + kq;
#pragma unroll
            for (int kk = 0; kk < kDK / 32; ++kk) {
                const bf16x8 af = frag(Arow + kk * 32);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const uint16_t* Bp = (16 * ct + c16) * kStrD + kq + kk * 32 + sSt;
                    acc[ct] = mfma16(af, frag(Bp), acc[ct]);
                    acc[ct] = mfma16(af, frag(Bp - sSt + sStl), acc[ct]);
                }
            }
        }
        if (wave >= 4) {
            // R = beta (V - gamma K S)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rb + r4 + i;
                    acc[ct][i] = sB[r] * (bf2f(sV[r * kStrV + 16 * ct + c16]) - sGam[r] * acc[ct][i]);
                }
                store16_t2(sRt, sRtl, kStrC, 16 * rb, 16 * ct, acc[ct], lane);
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[ct][i] *= sGam[16 * rb + r4 + i];
        }
        __syncthreads();

        // ---- step 2 (waves 4-7): U rows 16 rb.. = T R, R = R_hi + R_lo;
        //      T is unit lower triangular, so rows < 32 need only k < 32
        if (wave >= 4) {
            const int nk = rb < 2 ? 1 : 2;
            f32x4 u[2] = {f32x4{}, f32x4{}};
            const uint16_t* Ah = sT + (16 * rb + c16) * kStrC + kq;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk < nk) {
                    const bf16x8 ah = frag(Ah + kk * 32);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        const int bo = (16 * ct + c16) * kStrC + kq + kk * 32;
                        u[ct] = mfma16(ah, frag(sRt + bo), u[ct]);
                        u[ct] = mfma16(ah, frag(sRtl + bo), u[ct]);
                    }
                }
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                store16_t2(sUt, sUtl, kStrC, 16 * rb, 16 * ct, u[ct], lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) u[ct][i] *= sGd[16 * rb + r4 + i];
                store16_t2(sUht, sUhtl, kStrC, 16 * rb, 16 * ct, u[ct], lane);
            }
        }
        __syncthreads();

        // ---- step 3a (waves 0-3): Y rows 16 rb.. = gamma Q S + P U, U = U_hi + U_lo
        if (wave < 4) {
            const int nk = rb < 2 ? 1 : 2;
            const uint16_t* Ah = sP + (16 * rb + c16) * kStrC + kq;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk < nk) {
                    const bf16x8 ah = frag(Ah + kk * 32);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        const int bo = (16 * ct + c16) * kStrC + kq + kk * 32;
                        acc[ct] = mfma16(ah, frag(sUt + bo), acc[ct]);
                        acc[ct] = mfma16(ah, frag(sUtl + bo), acc[ct]);
                    }
                }
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) store1(sY + (16 * rb + r4 + i) * kStrY + 16 * ct + c16, acc[ct][i]);
        }
        // ---- step 3b (all waves): state rows 16 w.. = gamma_C S + K^T Uh
        {
            const float gC = sGam[kC - 1];
            const uint16_t* Arow = sKt + (16 * wave + c16) * kStrC + kq;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 af = frag(Arow + kk * 32);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    if (kk == 0) S[ct] *= gC;
                    const int bo = (16 * ct + c16) * kStrC + kq + kk * 32;
                    S[ct] = mfma16(af, frag(sUht + bo), S[ct]);
                    S[ct] = mfma16(af, frag(sUhtl + bo), S[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) store16_t2(sSt, sStl, kStrD, 16 * wave, 16 * ct, S[ct], lane);
        }
        __syncthreads();
        // ---- the chunk's y slice: 16-byte stores of whole rows
        {
            constexpr int kPer = 16 / sizeof(Ty);             // elements per 16 bytes
            constexpr int kRowPieces = kSl / kPer;
            const int idx = tid;
            if (idx < kC * kRowPieces) {
                const int r = idx / kRowPieces, c0 = (idx % kRowPieces) * kPer;
                if (r < n)
                    *reinterpret_cast<u32x4*>(static_cast<Ty*>(a.y) + ((size_t)(t0 + r) * a.H + h) * a.dv +
                                              j0 + c0) = *reinterpret_cast<const u32x4*>(sY + r * kStrY + c0);
            }
        }
    }
    if (a.ST) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * wave + r4 + i;
                a.ST[sbase + (size_t)row * a.dv + j0 + 16 * ct + c16] = S[ct][i];
            }
    }
}

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
    a.Pw = reinterpret_cast<uint16_t*>(ws + L.P);
    a.Gw = reinterpret_cast<float*>(ws + L.Gt);
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
        hipLaunchKernelGGL(chunk_scan_kernel<uint16_t>, dim3(blocks), dim3(kScanThreads), 0, s, a);
    else
        hipLaunchKernelGGL(chunk_scan_kernel<float>, dim3(blocks), dim3(kScanThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gdn
