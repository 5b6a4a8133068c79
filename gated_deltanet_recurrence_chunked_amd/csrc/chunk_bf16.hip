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
// The residual R and the update U (and diag(gamma_C/gamma) U) enter the MFMAs as hi + lo bf16
// pairs (about 16 significant bits: two MFMAs per product); the fp32 state S is rounded to a
// single bf16 operand, like q, k and the chunk-local T and P.
// T and P depend on the chunk's q, k, g, beta only, so they are produced for every chunk at
// once by chunk_prep_kernel (massively parallel: KK^T and QK^T on MFMA, the 64x64 unit
// lower-triangular inverse by fp32 forward substitution and 32x32 fp32 MFMA blocks).
// chunk_scan_kernel then walks the chunks of each (sequence, head) in order. The columns of
// S, V, U and Y are independent, so a scan workgroup owns a 32-column slice of d_v: 4
// workgroups per head at d_v = 128, mapped to the same XCD so the shared q, k, T, P tiles are
// fetched from HBM once and hit that XCD's L2.
//
// MFMA v_mfma_f32_32x32x16_bf16 operand layout (lane l of 64): A element j is A[l%32][(l/32)*8+j],
// B element j is B[(l/32)*8+j][l%32], accumulator element i is C[8(i/4)+4(l/32)+i%4][l%32].
#include "gdn_device.h"
#include "gdn_inverse.h"
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

// Wave 0: the chunk's gates (lane = token; rows >= n read row n-1, zeroed below).
__device__ __forceinline__ void fetch_gates(const DevArgs& a, int t0, int n, int h, float& gv,
                                            float& bv) {
    const int r = min((int)(threadIdx.x & (kWave - 1)), n - 1);
    const size_t base = (size_t)t0 * a.H + h;
    gv = a.g[base + r * a.H];
    bv = a.beta[base + r * a.H];
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
// a CU. T = (I + A)^{-1} (A strictly lower triangular) is built in three levels:
//   (1) the four 16x16 diagonal blocks by forward substitution in registers: lane (b, c)
//       owns column c of block b, and the entry A[r][i] it needs is broadcast from lane
//       (b, i) of its 16-lane row by DPP (row_newbcast), so no LDS traffic;
//   (2) 16 -> 32: T_10 = -T_11 (A_10 T_00) for the blocks (1,0) and (3,2), on the fp32
//       matrix cores (v_mfma_f32_16x16x4_f32);
//   (3) 32 -> 64: the same with 32x32 blocks (v_mfma_f32_32x32x2_f32).
// T and P leave through LDS as fp32 rows converted to bf16 with 16-byte global stores.
constexpr int kPrepThreads = kWave;

typedef float f32x4p __attribute__((ext_vector_type(4)));

// [64][64] fp32 tile in LDS (row stride kStrA) -> bf16 rows in global memory
__device__ __forceinline__ void store_tile_bf16(const float* src, uint16_t* dst, int lane) {
#pragma unroll
    for (int it = 0; it < kC * kC / 8 / kWave; ++it) {
        const int e = (lane + kWave * it) * 8, r = e / kC, c0 = e % kC;
        const f32x4p x0 = *reinterpret_cast<const f32x4p*>(src + r * kStrA + c0);
        const f32x4p x1 = *reinterpret_cast<const f32x4p*>(src + r * kStrA + c0 + 4);
        u32x4 o;
        o.x = pack_bf2(x0[0], x0[1]);
        o.y = pack_bf2(x0[2], x0[3]);
        o.z = pack_bf2(x1[0], x1[1]);
        o.w = pack_bf2(x1[2], x1[3]);
        *reinterpret_cast<u32x4*>(dst + e) = o;
    }
}

// T, P and the gate rows of one (chunk, head), by one wave. (gv, bv) are g and beta of row
// min(lane, n-1). sA, sG, sB are the wave's own LDS; the barriers inside are workgroup-wide,
// so in a workgroup of several waves every wave calls this together (one head each).
__device__ __forceinline__ void prep_chunk_head(const DevArgs& a, int chunk, int h, int t0, int n,
                                                float gv, float bv, float* sA, float* sG,
                                                float* sB) {
    const int lane = threadIdx.x & (kWave - 1);

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
    {
        // running sum G of g over the chunk (rows >= n add nothing), and the chunk's beta,
        // gamma_r = e^{G_r} and gamma_C / gamma_r for the scan
        float Gr = lane < n ? gv : 0.f;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float o = __shfl_up(Gr, off, kWave);
            if (lane >= off) Gr += o;
        }
        const float GC = __shfl(Gr, kC - 1, kWave);
        const float br = lane < n ? bv : 0.f;
        float* gw = a.Gw + ((size_t)chunk * a.H + h) * 3 * kC;
        gw[lane] = br;
        gw[kC + lane] = fexp(Gr);
        gw[2 * kC + lane] = fexp(GC - Gr);
        sG[lane] = Gr;
        sB[lane] = br;
    }
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

    // A[r][c] = beta_r e^{G_r - G_c} (k_r . k_c) for c < r, else 0 (fp32, to LDS);
    // P[r][c] = e^{G_r - G_c} (q_r . k_c) for c <= r (kept in registers).
    // Accumulator element i of lane l is row R0 + 8(i/4) + 4(l/32) + i%4 of column C0 + l%32,
    // so a lane's rows come in 4 runs of 4: the gates of each run are one 16-byte read.
    {
        f32x4p Grow[2][4], Brow[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 32 * rb + 8 * q + 4 * (lane >> 5);
                Grow[rb][q] = *reinterpret_cast<const f32x4p*>(sG + r);
                Brow[rb][q] = *reinterpret_cast<const f32x4p*>(sB + r);
            }
        const float Gcol[2] = {sG[lane & 31], sG[32 + (lane & 31)]};
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int rb = t == 0 ? 0 : 1, cb = t == 2 ? 1 : 0;
            const int c = 32 * cb + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int q = i >> 2, e = i & 3;
                const int r = 32 * rb + 8 * q + 4 * (lane >> 5) + e;
                const float dec = c <= r ? fexp(Grow[rb][q][e] - Gcol[cb]) : 0.f;
                sA[r * kStrA + c] = c < r ? Brow[rb][q][e] * dec * ckk[t][i] : 0.f;
                cqk[t][i] *= dec;
            }
        }
        // the upper-right block of A is zero
#pragma unroll
        for (int i = 0; i < 16; ++i) sA[acc_row(i, lane) * kStrA + 32 + (lane & 31)] = 0.f;
    }
    __syncthreads();

    // T = (I + A)^{-1} in three levels (16x16 blocks by DPP substitution, then fp32 MFMA)
    unit_lower_inverse64<kStrA, false>(sA);
    const int c = lane & 31;
    const size_t tile = ((size_t)chunk * a.H + h) * kC * kC;
    store_tile_bf16(sA, a.Tw + tile, lane);
    __syncthreads();   // T read out: P takes its place
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int R0 = t == 0 ? 0 : 32, C0 = t == 2 ? 32 : 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) sA[(R0 + acc_row(i, lane)) * kStrA + C0 + c] = cqk[t][i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[acc_row(i, lane) * kStrA + 32 + c] = 0.f;
    __syncthreads();
    store_tile_bf16(sA, a.Pw + tile, lane);
}

__global__ void __launch_bounds__(kPrepThreads, 2) chunk_prep_kernel(DevArgs a) {
    __shared__ __attribute__((aligned(16))) float sA[kC * kStrA];
    __shared__ __attribute__((aligned(16))) float sG[kC], sB[kC];
    const int chunk = blockIdx.x, h = blockIdx.y;
    int seq, t0, n;
    if (!chunk_of(a, chunk, seq, t0, n)) return;
    float gv, bv;
    fetch_gates(a, t0, n, h, gv, bv);
    prep_chunk_head(a, chunk, h, t0, n, gv, bv, sA, sG, sB);
}

// ------------------------------------------------------------------ fused front end
// eqs. (6)-(10) of the notes for one chunk of HPW heads, then each head's T and P (one wave
// per head), in one workgroup: conv (width 4, zero input before the sequence start) -> SiLU
// -> L2Norm for q and k, conv -> SiLU for v, the gates beta = sigmoid(b), g = -e^A
// softplus(a + dt_bias). q, k, v leave in bf16 (the scan reads them) with plain stores, so the
// T/P stage that follows the barrier reads q and k back from L2, not HBM.
// Stream layout: a thread owns 8 adjacent channels (one 16-byte bf16 store) of a strip of
// D/8 consecutive rows; the D/8 threads of one (row, head) are adjacent lanes, so the L2Norm
// is an in-register shuffle reduction. The 3 rows before a strip are its conv window.
// A thread's rows of one stream come in P pieces of RP consecutive rows, each with the 3 rows
// before it as its conv window: issue() puts a piece's loads in flight, run() computes and
// stores it. Two pieces are in flight at a time (the next one loads while this one runs).
template <int HPW, int D, typename Tin>
struct FrontPiece {
    static constexpr int G = HPW * D / 8;              // channel groups of the head group
    static constexpr int RS = kC * G / (HPW * kWave);  // rows per thread per stream (D / 8)
    static constexpr int P = sizeof(Tin) == 2 ? 2 : 4; // pieces per stream
    static constexpr int RP = RS / P;                  // rows per piece
    typename Vec8<Tin>::Raw raw[RP + 3];               // rows r0-3 .. r0+RP-1

    __device__ __forceinline__ static int first_row(int part) {
        return (threadIdx.x / G) * RS + part * RP;
    }

    __device__ __forceinline__ void issue(const FrontArgs& f, int role, int part, int t0, int n,
                                          int seq_lo, int h0, int H) {
        const int r0 = first_row(part), c = h0 * D + (threadIdx.x % G) * 8;
        const Tin* x = static_cast<const Tin*>(f.x[role]);
        // addresses clamped into the chunk's sequence: rows before its start are zeroed in
        // run(), rows past n are not stored
#pragma unroll
        for (int j = 0; j < RP + 3; ++j) {
            const int t = min(max(t0 + r0 - 3 + j, seq_lo), t0 + n - 1);
            raw[j] = Vec8<Tin>::template load_raw<true>(x + (size_t)t * H * D + c);
        }
    }

    __device__ __forceinline__ void run(const FrontArgs& f, int role, int part, int t0, int n,
                                        int seq_lo, int h0, int H) const {
        const int r0 = first_row(part), c = h0 * D + (threadIdx.x % G) * 8;
        uint16_t* out = f.out[role];
        float w[8][4];
        {
            const float4* wp = reinterpret_cast<const float4*>(f.w[role] + (size_t)c * 4);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 t = wp[i];
                w[i][0] = t.x; w[i][1] = t.y; w[i][2] = t.z; w[i][3] = t.w;
            }
        }
        float win[3][8];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            Vec8<Tin>::unpack(raw[j], win[j]);
            if (t0 + r0 - 3 + j < seq_lo)
#pragma unroll
                for (int i = 0; i < 8; ++i) win[j][i] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < RP; ++j) {
            float xi[8], act[8], ss = 0.f;
            Vec8<Tin>::unpack(raw[j + 3], xi);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                act[i] = siluf_(conv4(w[i][0], w[i][1], w[i][2], w[i][3], win[0][i], win[1][i],
                                      win[2][i], xi[i]));
                ss = __builtin_fmaf(act[i], act[i], ss);
            }
            if (role < 2) {
                ss = group_sum<D / 8>(ss);
                const float inv = frsq(ss + f.l2_eps);
#pragma unroll
                for (int i = 0; i < 8; ++i) act[i] *= inv;
            }
            if (r0 + j < n) Vec8<uint16_t>::store(out + (size_t)(t0 + r0 + j) * H * D + c, act);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                win[0][i] = win[1][i];
                win[1][i] = win[2][i];
                win[2][i] = xi[i];
            }
        }
    }
};

template <int HPW, int DV, typename Tin>
__global__ void __launch_bounds__(HPW * kWave, 2) chunk_front_kernel(DevArgs a, FrontArgs f) {
    __shared__ __attribute__((aligned(16))) float sA[HPW][kC * kStrA];
    __shared__ __attribute__((aligned(16))) float sG[HPW][kC], sB[HPW][kC];
    const int chunk = blockIdx.x, h0 = blockIdx.y * HPW;
    int seq, t0, n;
    if (!chunk_of(a, chunk, seq, t0, n)) return;
    const int seq_lo = a.cu ? a.cu[seq] : seq * a.L, H = a.H;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, h = h0 + wave;
    const size_t e = (size_t)(t0 + min(lane, n - 1)) * H + h;
    const float ar = f.a_raw[e], br = f.b_raw[e];
    {
        // pieces in order q0..q(P-1), k0..k(P-1), v0..; buffers x0/x1 alternate (P is even)
        using PK = FrontPiece<HPW, kDK, Tin>;
        using PV = FrontPiece<HPW, DV, Tin>;
        constexpr int NQK = 2 * PK::P;
        PK x0, x1;
        PV y0, y1;
        x0.issue(f, 0, 0, t0, n, seq_lo, h0, H);
#pragma unroll
        for (int i = 0; i < NQK; i += 2) {
            x1.issue(f, (i + 1) / PK::P, (i + 1) % PK::P, t0, n, seq_lo, h0, H);
            x0.run(f, i / PK::P, i % PK::P, t0, n, seq_lo, h0, H);
            if (i + 2 < NQK) x0.issue(f, (i + 2) / PK::P, (i + 2) % PK::P, t0, n, seq_lo, h0, H);
            else y0.issue(f, 2, 0, t0, n, seq_lo, h0, H);
            x1.run(f, (i + 1) / PK::P, (i + 1) % PK::P, t0, n, seq_lo, h0, H);
        }
#pragma unroll
        for (int i = 0; i < PV::P; i += 2) {
            y1.issue(f, 2, i + 1, t0, n, seq_lo, h0, H);
            y0.run(f, 2, i, t0, n, seq_lo, h0, H);
            if (i + 2 < PV::P) y0.issue(f, 2, i + 2, t0, n, seq_lo, h0, H);
            y1.run(f, 2, i + 1, t0, n, seq_lo, h0, H);
        }
    }
    // gates: wave = head of the group, lane = row (rows >= n repeat row n-1, as the prep expects)
    const float gv = gate_g(f.A_log[h], ar, f.dt_bias[h]);
    const float bv = gate_beta(br);
    if (f.g_out && lane < n) {
        f.g_out[e] = gv;
        f.beta_out[e] = bv;
    }
    __syncthreads();   // the chunk's q, k rows of every head are written (and in L2)
    prep_chunk_head(a, chunk, h, t0, n, gv, bv, sA[wave], sG[wave], sB[wave]);
}

// ------------------------------------------------------------------ sequential chunk scan
// One 4-wave workgroup per (sequence, head, 32-column slice of d_v), one wave per SIMD:
//   waves 0-1 ("chain" waves) carry the recurrence of one 16-column slice each,
//     K S -> R -> U = T R -> W = diag(gamma_C/gamma) U -> S = gamma_C S + K^T W;
//   wave 2 (the "output" wave), one chunk behind the chain, forms Y^T = gamma-scaled
//     S^T Q^T + U^T P^T for both slices (they share the Q and P fragments) and stores y;
//   wave 3 (the loader) streams, with direct global->LDS loads, the chain's tiles (K, T, the
//     V slice and the gate rows) one chunk ahead into a two-slot ring and the output wave's
//     tiles (Q, P, the gate rows) into two slots of their own.
// The chain waves hand each chunk's bf16 state operand and fp32 U to the output wave through
// a double-buffered LDS exchange, so the MFMAs and VALU work off the chain run on other SIMDs
// and only the loader issues global loads.
//
// A chain wave keeps everything that depends on the state in registers: products are
// v_mfma_f32_16x16x32_bf16 tiles (lane l = (c, g), c = l%16, g = l/16, supplies A[c][8g+j]
// and B[8g+j][c]; accumulator element i is C[4g+i][c]). An accumulator therefore holds, per
// lane, 4 rows of one column, while an operand needs 8 consecutive contraction indices of one
// row or column. Instead of moving data between lanes, the rows of a tile are relabelled:
// tile 2s+a of a 64-row (tokens) or 128-row (d_k) dimension has row r standing for index
// 32s + 8(r/4) + 4a + r%4. With that labelling, accumulator tiles 2s and 2s+1 of one lane
// hold exactly indices 32s+8g .. 32s+8g+7 of their column, i.e. the operand fragment of
// contraction step s: the state S, the residual R and the update U go from accumulator to
// bf16 operand in registers (and are the same fragments whether they enter a product as A or
// as B). The relabelling only changes which LDS row an operand lane reads (the tiles stay
// row-major); the K^T operand of the state update comes from the row-major K tile through
// the transposing LDS read ds_read_b64_tr_b16. Y^T has d_v rows, so an output lane stores 4
// adjacent y values of one token.
//
// R, U and W enter their products as bf16 hi + lo pairs (two MFMAs per product). LDS tiles are
// row-major with 16-byte units XOR-swizzled by a function of the row, so the 16 rows read by
// one fragment load and the 4x4 rows/units read by one transposing load spread over the banks.
constexpr int kScanThreads = 256;
constexpr int kRing = 2;
constexpr int kOffK = 0;                      // ring slot layout, in bf16 elements
constexpr int kOffT = kOffK + kC * kDK;
constexpr int kOffV = kOffT + kC * kC;
constexpr int kOffG = kOffV + kC * kSl;       // 3 x 64 floats (+ 256 bytes of padding)
constexpr int kSlot = kOffG + 512;

constexpr int kQOffQ = 0;                     // output slot layout, in bf16 elements
constexpr int kQOffP = kQOffQ + kC * kDK;
constexpr int kQOffG = kQOffP + kC * kC;      // 3 x 64 floats (+ 256 bytes of padding)
constexpr int kQPSlot = kQOffG + 512;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte unit swizzle of LDS row `row`: distinct for the 8 rows {0..7} and for {0-3, 8-11}
// (+ any multiple of 4), and spreads the 4 consecutive rows of a transposing read.
__device__ __forceinline__ int swz(int row) {
    return (((row & 1) << 2) | ((row >> 1) & 3)) ^ (((row >> 3) & 1) << 1);
}

// tile row r of tile t (2s + a) of a relabelled dimension -> index 32s + 8(r/4) + 4a + r%4
__device__ __forceinline__ int relabel(int t, int r) {
    return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3);
}

__device__ __forceinline__ s16x4 lds_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<uint16_t*>(p)));
}

// two fp32 accumulator quads -> bf16 hi and lo operand fragments (8 values each)
__device__ __forceinline__ void split8(const f32x4& x0, const f32x4& x1, bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float a0 = e < 2 ? x0[2 * e] : x1[2 * e - 4];
        const float a1 = e < 2 ? x0[2 * e + 1] : x1[2 * e - 3];
        const uint32_t hp = pack_bf2(a0, a1);
        h[e] = hp;
        l[e] = pack_bf2(a0 - __uint_as_float(hp << 16), a1 - __uint_as_float(hp & 0xffff0000u));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// two fp32 accumulator quads -> one bf16 operand fragment (8 values)
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x4& x0, const f32x4& x1) {
    const u32x4 h = {pack_bf2(x0[0], x0[1]), pack_bf2(x0[2], x0[3]), pack_bf2(x1[0], x1[1]),
                     pack_bf2(x1[2], x1[3])};
    return __builtin_bit_cast(bf16x8, h);
}

__device__ __forceinline__ void dma16(const void* src, uint16_t* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_dst), 16, 0, 0);
}

// Workgroup barrier that orders LDS accesses only (global loads and stores stay in flight).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The output waves' side of that barrier. Their direct loads into the ring are tracked by the
// vector-memory counter, which they wait on explicitly (for the chunk they owe) before it, so
// the chunk just issued stays in flight across it (a fence would wait for it too); their own
// LDS reads are complete at the barrier (lgkmcnt), and the memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void dma_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// keeps the instruction scheduler from moving anything across this point (reads issued before
// it stay ahead of the MFMAs after it)
#define GDN_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Interleaving request for the scheduling region it closes: nm times {one MFMA, up to nv VALU
// instructions, up to nd LDS reads}.
#define GDN_IGLP(nm, nv, nd)                                  \
    _Pragma("unroll") for (int i_ = 0; i_ < (nm); ++i_) {     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    \
        __builtin_amdgcn_sched_group_barrier(0x002, (nv), 0); \
        __builtin_amdgcn_sched_group_barrier(0x100, (nd), 0); \
    }

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding)
#define GDN_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00)

template <typename Ty>
__global__ void __launch_bounds__(kScanThreads) chunk_scan_kernel(DevArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ring[kRing * kSlot];      // the chain's tiles
    __shared__ __attribute__((aligned(16))) uint16_t qpbuf[2 * kQPSlot];     // the output wave's tiles
    // chain -> output exchange: [chunk parity][slice][8 x 64 lanes x 16 bytes]; rows 0-3 hold
    // the bf16 state fragments of contraction steps 0-3, rows 4-7 the fp32 U tiles
    __shared__ __attribute__((aligned(16))) u32x4 xbuf[2][2][8 * 64];

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
    const int nchunks = (hi - lo + kC - 1) / kC;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform branches
    const int j0 = slice * kSl;
    const int c16 = lane & 15, g = lane >> 4;

    if (wave == 3) {
        // ================= loader wave
        // Step c refills ring slot (c + 1) % 2 with chunk c + 1's K, T, V slice and gate rows
        // for the chain (the slot held chunk c - 1, which the chain finished before this step's
        // barrier) and output slot c % 2 with chunk c's Q, P and gate rows for the output wave
        // (which used that slot for chunk c - 2 during the previous step), then waits for both
        // before the barrier. For a full chunk the per-lane global offsets do not depend on the
        // chunk, so they are formed once; a chunk adds wave-uniform bases.
        int offk[16], offv[4];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 4 * i + (lane >> 4), u = (lane & 15) ^ swz(row);
            offk[i] = (row * a.H + h) * kDK + u * 8;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) offv[i] = ((16 * i + (lane >> 2)) * a.H + h) * a.dv + j0 + (lane & 3) * 8;
        // [64][128] tile rows of a chunk of x (q or k), 16-byte units swizzled per row
        auto rows128 = [&](const uint16_t* x, int t0, int n, uint16_t* dst) __attribute__((always_inline)) {
            const uint16_t* xb = x + (size_t)t0 * a.H * kDK;
            if (n == kC) {
#pragma unroll
                for (int i = 0; i < 16; ++i) dma16(xb + offk[i], dst + i * 512);
            } else {   // the ragged last chunk: rows >= n repeat row n - 1
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 4 * i + (lane >> 4), u = (lane & 15) ^ swz(row);
                    dma16(xb + (min(row, n - 1) * a.H + h) * kDK + u * 8, dst + i * 512);
                }
            }
        };
        auto tile64 = [&](const uint16_t* src, uint16_t* dst) __attribute__((always_inline)) {   // [64][64]
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = 8 * i + (lane >> 3), u = (lane & 7) ^ swz(row);
                dma16(src + row * kC + u * 8, dst + i * 512);
            }
        };
        auto chain_tiles = [&](int ck) __attribute__((always_inline)) {
            const int t0 = lo + ck * kC, n = min(kC, hi - t0);
            const size_t ch = (size_t)(cbase + ck) * a.H + h;   // chunk-head index
            uint16_t* slot = ring + (ck & 1) * kSlot;
            rows128(a.k, t0, n, slot + kOffK);
            const uint16_t* vb = a.v + (size_t)t0 * a.H * a.dv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * i + (lane >> 2);
                const int o = n == kC ? offv[i] : (min(row, n - 1) * a.H + h) * a.dv + j0 + (lane & 3) * 8;
                dma16(vb + o, slot + kOffV + i * 512);
            }
            tile64(a.Tw + ch * kC * kC, slot + kOffT);
            dma16(a.Gw + ch * 3 * kC + (lane % 48) * 4, slot + kOffG);
        };
        auto output_tiles = [&](int ck) __attribute__((always_inline)) {
            const int t0 = lo + ck * kC, n = min(kC, hi - t0);
            const size_t ch = (size_t)(cbase + ck) * a.H + h;
            uint16_t* slot = qpbuf + (ck & 1) * kQPSlot;
            rows128(a.q, t0, n, slot + kQOffQ);
            tile64(a.Pw + ch * kC * kC, slot + kQOffP);
            dma16(a.Gw + ch * 3 * kC + (lane % 48) * 4, slot + kQOffG);
        };
        if (nchunks > 0) chain_tiles(0);
        GDN_WAIT_VMCNT(0);
        dma_barrier();
        for (int c = 0; c <= nchunks; ++c) {
            if (c + 1 < nchunks) chain_tiles(c + 1);
            if (c < nchunks) output_tiles(c);
            GDN_WAIT_VMCNT(0);
            dma_barrier();
        }
        return;
    }
    if (wave == 2) {
        // ================= output wave: Y^T of both 16-column slices, one chunk behind the chain
        // Y^T = gamma (S^T Q^T) + U^T P^T: S^T and U^T are the chain's operand fragments (lane
        // (c, g): d_v row c, contraction indices 32s + 8g ..), Q and P the B operands with
        // natural token columns; a lane holds 4 adjacent d_v of token 16 rt + c16 of y.
        int oqf[2], opf[2];
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            oqf[sp] = kQOffQ + c16 * kDK + (((4 * sp + g) ^ swz(c16)) << 3);
            opf[sp] = kQOffP + c16 * kC + (((4 * sp + g) ^ swz(c16)) << 3);
        }
        const size_t ytok = (size_t)a.H * a.dv;   // elements between consecutive tokens of y
        Ty* const ylane = static_cast<Ty*>(a.y) + (size_t)h * a.dv + j0 + 4 * g + (size_t)c16 * ytok;
        auto output = [&](int cy) __attribute__((always_inline)) {
            const uint16_t* slot = qpbuf + (cy & 1) * kQPSlot;
            const float* sGq = reinterpret_cast<const float*>(slot + kQOffG);
            bf16x8 qf[4][4], pf[4][2];
            float gq[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                // rows 16 apart share the swizzle, units 8 apart are 64 elements apart
#pragma unroll
                for (int s = 0; s < 4; ++s) qf[rt][s] = frag(slot + oqf[s & 1] + rt * 16 * kDK + (s >> 1) * 64);
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (s <= (rt >> 1)) pf[rt][s] = frag(slot + opf[s] + rt * 16 * kC);
                gq[rt] = sGq[kC + 16 * rt + c16];
            }
            f32x4 YT[2][4];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const u32x4* xb = xbuf[cy & 1][sl];
                bf16x8 Sb[4];
                f32x4 U[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) Sb[s] = __builtin_bit_cast(bf16x8, xb[s * 64 + lane]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) U[rt] = __builtin_bit_cast(f32x4, xb[(4 + rt) * 64 + lane]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) YT[sl][rt] = f32x4{};
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) YT[sl][rt] = mfma16(Sb[s], qf[rt][s], YT[sl][rt]);
                bf16x8 Uh[2], Ul[2];
                split8(U[0], U[1], Uh[0], Ul[0]);
                split8(U[2], U[3], Uh[1], Ul[1]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) YT[sl][rt] *= gq[rt];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) YT[sl][rt] = mfma16(Uh[0], pf[rt][0], YT[sl][rt]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) YT[sl][rt] = mfma16(Ul[0], pf[rt][0], YT[sl][rt]);
#pragma unroll
                for (int rt = 2; rt < 4; ++rt) YT[sl][rt] = mfma16(Uh[1], pf[rt][1], YT[sl][rt]);
#pragma unroll
                for (int rt = 2; rt < 4; ++rt) YT[sl][rt] = mfma16(Ul[1], pf[rt][1], YT[sl][rt]);
            }
            // y is written once and never read here: streaming (nontemporal) stores keep its
            // lines from displacing the q, k, T and P lines the head's other slices still read
            // from the shared L2
            const int ty = lo + cy * kC, ny = min(kC, hi - ty);
            Ty* const yc = ylane + (size_t)ty * ytok;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if (16 * rt + c16 < ny) {
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl) {
                        Ty* yp = yc + (size_t)(16 * rt) * ytok + 16 * sl;
                        if constexpr (sizeof(Ty) == 2) {
                            u32x2 o;
                            o.x = pack_bf2(YT[sl][rt][0], YT[sl][rt][1]);
                            o.y = pack_bf2(YT[sl][rt][2], YT[sl][rt][3]);
                            __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(yp));
                        } else {
                            __builtin_nontemporal_store(YT[sl][rt], reinterpret_cast<f32x4*>(yp));
                        }
                    }
                }
            }
        };
        // step c (after its barrier) forms chunk c - 1's y from the exchange buffer the chain
        // filled and the output slot the loader filled during step c - 1
        lds_barrier();   // chunk 0 in the ring
        for (int c = 0; c <= nchunks; ++c) {
            if (c >= 1) output(c - 1);
            lds_barrier();
        }
        return;
    }

    // ================= chain waves: d_v columns j0w .. j0w + 15
    const int j0w = j0 + 16 * wave;
    const size_t sbase = ((size_t)seq * a.H + h) * kDK * a.dv;

    // state: tile t holds d_k rows relabel(t, 4g + i) of column j0w + c16
    f32x4 S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) S[t] = f32x4{};
    if (a.S0) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[t][i] = a.S0[sbase + (size_t)relabel(t, 4 * g + i) * a.dv + j0w + c16];
    }
    bf16x8 Sb[4];   // S as bf16 operand fragments, one per contraction step
#pragma unroll
    for (int s = 0; s < 4; ++s) Sb[s] = to_bf16x8(S[2 * s], S[2 * s + 1]);

    // Per-lane LDS offsets (elements, from the ring slot) of the fragment reads. The swizzle
    // sees only the low 4 bits of a row, so rows 16 or 32 apart and units 8 apart are constant
    // offsets from one of these bases and become immediates of the LDS reads.
    int okf[2][2], otf[2][2], okt[2][2];
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2) {
        const int r = relabel(a2, c16);
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            okf[a2][sp] = kOffK + r * kDK + (((4 * sp + g) ^ swz(r)) << 3);
            otf[a2][sp] = kOffT + r * kC + (((4 * sp + g) ^ swz(r)) << 3);
        }
    }
    const int jj = (lane & 15) >> 2, r4 = lane & 3;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int tok = 8 * g + jj + 4 * hf;
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) okt[hf][tp] = kOffK + tok * kDK + (((4 * tp + r4) ^ swz(tok)) << 3);
    }
    const int ov = kOffV + (8 * g + jj) * kSl + 16 * wave + 4 * r4;

    lds_barrier();   // chunk 0 in the ring
    for (int c = 0; c <= nchunks; ++c) {
        if (c == nchunks) {   // the output waves finish the last chunk
            lds_barrier();
            break;
        }
        const uint16_t* slot = ring + (c % kRing) * kSlot;
        const float* sG = reinterpret_cast<const float*>(slot + kOffG);   // beta | gamma | gamma_C/gamma
        u32x4* xb = xbuf[c & 1][wave];
        auto kfrag = [&](int rt, int s) {   // A of K S: K[relabel(rt, c16)][32s + 8g ..]
            return frag(slot + okf[rt & 1][s & 1] + (rt >> 1) * 32 * kDK + (s >> 1) * 64);
        };
        auto tfrag = [&](int rt, int s) {   // A of T R: T[relabel(rt, c16)][32s + 8g ..]
            return frag(slot + otf[rt & 1][s] + (rt >> 1) * 32 * kC);
        };
        auto ktr = [&](int t, int s, int hf) {   // K^T[relabel(t, c16)][32s + 8g + 4hf ..]
            return lds_tr16(slot + okt[hf][(t >> 1) & 1] + s * 32 * kDK + (t >> 2) * 64 + 4 * (t & 1));
        };
        auto grow = [&](int which, int rt) {   // gate row `which` at the lane's 4 relabelled tokens
            return *reinterpret_cast<const f32x4*>(sG + which * kC + 8 * g + 32 * (rt >> 1) + 4 * (rt & 1));
        };

        // The chain K S -> R -> U = T R -> W -> S update; the fp32 -> bf16 splits and gate
        // scalings between its links are VALU work. Each block is one scheduling region whose
        // MFMAs are interleaved with VALU work that does not feed them and with the LDS reads
        // of later regions.
        bf16x8 kf[4][4];
        f32x4 KS[4];
        auto mma_k = [&](int s) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) KS[rt] = mfma16(kf[s][rt], Sb[s], KS[rt]);
        };
        auto load_k = [&](int s) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) kf[s][rt] = kfrag(rt, s);
        };
        load_k(0);
        load_k(1);
        const float gC = sG[kC + kC - 1];
        GDN_SCHED_FENCE();
        // ---- K S step 0 | the state operand to the output waves | gamma_C S (tiles 0-3) |
        //      K fragments of steps 2-3
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) KS[rt] = f32x4{};
        mma_k(0);
#pragma unroll
        for (int s = 0; s < 4; ++s) xb[s * 64 + lane] = __builtin_bit_cast(u32x4, Sb[s]);
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t] *= gC;
        load_k(2);
        load_k(3);
        GDN_IGLP(4, 4, 2);
        GDN_SCHED_FENCE();
        // ---- K S step 1 | gamma_C S (tiles 4-7) | gate rows and V at the lane's tokens
        f32x4 bet[4], gam[4];
        s16x4 vv[4];
        mma_k(1);
#pragma unroll
        for (int t = 4; t < 8; ++t) S[t] *= gC;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            bet[rt] = grow(0, rt);
            gam[rt] = grow(1, rt);
            vv[rt] = lds_tr16(slot + ov + (32 * (rt >> 1) + 4 * (rt & 1)) * kSl);
        }
        GDN_IGLP(4, 4, 3);
        GDN_SCHED_FENCE();
        // ---- K S steps 2-3 | T fragments, gamma_C / gamma
        bf16x8 tf[4][2];
        f32x4 gd[4];
        mma_k(2);
        mma_k(3);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
                if (s <= (rt >> 1)) tf[rt][s] = tfrag(rt, s);
            gd[rt] = grow(2, rt);
        }
        GDN_IGLP(8, 1, 2);
        GDN_SCHED_FENCE();
        // ---- R = beta (V - gamma KS) and its split | K^T fragments of tiles 0-1
        s16x4 kt[8][2][2];   // K^T fragments [d_k tile][step][half]
        auto load_kt = [&](int t) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) kt[t][s][hf] = ktr(t, s, hf);
        };
        f32x4 R[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                R[rt][i] = bet[rt][i] * (bf2f(uint16_t(vv[rt][i])) - gam[rt][i] * KS[rt][i]);
        bf16x8 Rh[2], Rl[2];
        split8(R[0], R[1], Rh[0], Rl[0]);
        split8(R[2], R[3], Rh[1], Rl[1]);
        load_kt(0);
        load_kt(1);
        GDN_SCHED_FENCE();
        // ---- U = T R (T unit lower triangular: token rows < 32 need step 0 only) |
        //      K^T fragments of tiles 2-3
        f32x4 U[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) U[rt] = f32x4{};
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) U[rt] = mfma16(tf[rt][0], Rh[0], U[rt]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) U[rt] = mfma16(tf[rt][0], Rl[0], U[rt]);
#pragma unroll
        for (int rt = 2; rt < 4; ++rt) U[rt] = mfma16(tf[rt][1], Rh[1], U[rt]);
#pragma unroll
        for (int rt = 2; rt < 4; ++rt) U[rt] = mfma16(tf[rt][1], Rl[1], U[rt]);
        load_kt(2);
        load_kt(3);
        GDN_IGLP(12, 1, 1);
        GDN_SCHED_FENCE();
        // ---- U to the output waves | W = diag(gamma_C / gamma) U and its split |
        //      K^T fragments of tiles 4-5
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) xb[(4 + rt) * 64 + lane] = __builtin_bit_cast(u32x4, U[rt]);
        bf16x8 Wh[2], Wl[2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) U[rt] *= gd[rt];
        split8(U[0], U[1], Wh[0], Wl[0]);
        split8(U[2], U[3], Wh[1], Wl[1]);
        load_kt(4);
        load_kt(5);
        GDN_SCHED_FENCE();
        // ---- S = gamma_C S + K^T W, each finished pair of tiles split for the next chunk |
        //      K^T fragments of tiles 6-7
        auto upd = [&](int t) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x2 p0 = __builtin_bit_cast(u32x2, kt[t][s][0]);
                const u32x2 p1 = __builtin_bit_cast(u32x2, kt[t][s][1]);
                const u32x4 pk = {p0.x, p0.y, p1.x, p1.y};
                const bf16x8 ktf = __builtin_bit_cast(bf16x8, pk);
                S[t] = mfma16(ktf, Wh[s], S[t]);
                S[t] = mfma16(ktf, Wl[s], S[t]);
            }
            if (t & 1) Sb[t >> 1] = to_bf16x8(S[t - 1], S[t]);
        };
#pragma unroll
        for (int t = 0; t < 4; ++t) upd(t);
        load_kt(6);
        load_kt(7);
        GDN_IGLP(16, 2, 1);
        GDN_SCHED_FENCE();
#pragma unroll
        for (int t = 4; t < 8; ++t) upd(t);
        GDN_IGLP(16, 1, 0);
        GDN_SCHED_FENCE();
        lds_barrier();   // past this barrier the ring slot is refilled and xb is read
    }
    if (a.ST) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.ST[sbase + (size_t)relabel(t, 4 * g + i) * a.dv + j0w + c16] = S[t][i];
    }
}

}  // namespace

size_t chunk_bf16_workspace(int ntok, int num_seqs, int H) {
    return ws_layout(ntok, num_seqs, H).total;
}

template <int HPW, typename Tin>
static void launch_front(const DevArgs& a, const FrontArgs& f, int nchunks, int dv, hipStream_t s) {
    const dim3 grid(nchunks, a.H / HPW);
    if (dv == 128)
        hipLaunchKernelGGL((chunk_front_kernel<HPW, 128, Tin>), grid, dim3(HPW * kWave), 0, s, a, f);
    else
        hipLaunchKernelGGL((chunk_front_kernel<HPW, 64, Tin>), grid, dim3(HPW * kWave), 0, s, a, f);
}

template <typename Tin>
static void launch_front_h(const DevArgs& a, const FrontArgs& f, int nchunks, int dv, hipStream_t s) {
    if (a.H % 4 == 0) launch_front<4, Tin>(a, f, nchunks, dv, s);
    else if (a.H % 2 == 0) launch_front<2, Tin>(a, f, nchunks, dv, s);
    else launch_front<1, Tin>(a, f, nchunks, dv, s);
}

hipError_t launch_chunk_bf16(const ChunkArgs& c, hipStream_t s, const FrontArgs* front) {
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
    if (nchunks > 0 && front && front->in_bf16)
        launch_front_h<uint16_t>(a, *front, nchunks, c.dv, s);
    else if (nchunks > 0 && front)
        launch_front_h<float>(a, *front, nchunks, c.dv, s);
    else if (nchunks > 0)
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
