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
// lower-triangular inverse by fp32 forward substitution and 32x32 fp32 MFMA blocks; the
// sliced forward scans form P themselves). A scan kernel then walks the chunks of each
// (sequence, head) in order: chunk_scan_fwd_kernel (tiles two chunks ahead) or
// chunk_scan_kernel for the forward prefill, chunk_scan_kernel for the backward's
// states-only sweep, chunk_scan_wide_kernel for the per-channel-decay prefill and for the
// prefill with the output gate in its epilogue (256 or more equal-length pairs). The columns of
// S, V, U and Y are independent, so a scan workgroup owns a 32-column slice of d_v: 4
// workgroups per head at d_v = 128, mapped to the same XCD so the shared q, k, T, P tiles are
// fetched from HBM once and hit that XCD's L2.
//
// MFMA v_mfma_f32_32x32x16_bf16 operand layout (lane l of 64): A element j is A[l%32][(l/32)*8+j],
// B element j is B[(l/32)*8+j][l%32], accumulator element i is C[8(i/4)+4(l/32)+i%4][l%32].
#include "gdn_device.h"
#include "gdn_inverse.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

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
    L.Gt = o;  o = align256(o + sizeof(float) * kGateRows * kC * (size_t)L.max_chunks * H);
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
                                // (per-channel decay: beta [64] | e^{Gc_C} [128])
    uint16_t* Xw;               // per-channel decay only: [max_chunks][H][3][64][128] bf16
                                // Kg = K o e^{Gc}, Kc = K o e^{Gc_C - Gc}, Qg = Q o e^{Gc}
    const float* gk;            // per-channel decay only: log-decays [ntok][H][128]
    float* Sst;                 // states-only scan: fp32 state entering each chunk,
                                // [max_chunks][H][d_v][d_k] (S^T, d_k contiguous)
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

// T, P (kP) and the gate rows of one (chunk, head), by one wave. (gv, bv) are g and beta of
// row min(lane, n-1). sA, sG, sB are the wave's own LDS; the barriers inside are
// workgroup-wide, so in a workgroup of several waves every wave calls this together (one head
// each). Without kP, Q is not read and P not formed (the sliced scan forms P itself).
template <bool kP>
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
        if constexpr (kP) {
            fq0[kk] = *reinterpret_cast<const u32x4*>(q0p + kk * 16);
            fq1[kk] = *reinterpret_cast<const u32x4*>(q1p + kk * 16);
        }
    }
    {
        // running sum G of g over the chunk (rows >= n add nothing), and the chunk's beta,
        // gamma_r = e^{G_r}, gamma_C / gamma_r and G_r for the scan
        float Gr = lane < n ? gv : 0.f;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float o = __shfl_up(Gr, off, kWave);
            if (lane >= off) Gr += o;
        }
        const float GC = __shfl(Gr, kC - 1, kWave);
        const float br = lane < n ? bv : 0.f;
        float* gw = a.Gw + ((size_t)chunk * a.H + h) * kGateRows * kC;
        gw[lane] = br;
        gw[kC + lane] = fexp(Gr);
        gw[2 * kC + lane] = fexp(GC - Gr);
        gw[3 * kC + lane] = Gr;
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
        ckk[0] = mfma(k0, k0, ckk[0]);
        ckk[1] = mfma(k1, k0, ckk[1]);
        ckk[2] = mfma(k1, k1, ckk[2]);
        if constexpr (kP) {
            const bf16x8 q0 = __builtin_bit_cast(bf16x8, v0 ? fq0[kk] : z);
            const bf16x8 q1 = __builtin_bit_cast(bf16x8, v1 ? fq1[kk] : z);
            cqk[0] = mfma(q0, k0, cqk[0]);
            cqk[1] = mfma(q1, k0, cqk[1]);
            cqk[2] = mfma(q1, k1, cqk[2]);
        }
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
                if constexpr (kP) cqk[t][i] *= dec;
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
    if constexpr (!kP) return;
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

template <bool kP>
__global__ void __launch_bounds__(kPrepThreads, 2) chunk_prep_kernel(DevArgs a) {
    __shared__ __attribute__((aligned(16))) float sA[kC * kStrA];
    __shared__ __attribute__((aligned(16))) float sG[kC], sB[kC];
    const int chunk = blockIdx.x, h = blockIdx.y;
    int seq, t0, n;
    if (!chunk_of(a, chunk, seq, t0, n)) return;
    float gv, bv;
    fetch_gates(a, t0, n, h, gv, bv);
    prep_chunk_head<kP>(a, chunk, h, t0, n, gv, bv, sA, sG, sB);
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
constexpr int kOffG = kOffV + kC * kSl;       // kGateRows x 64 floats
constexpr int kSlot = kOffG + 512;

constexpr int kQOffQ = 0;                     // output slot layout, in bf16 elements
constexpr int kQOffP = kQOffQ + kC * kDK;
constexpr int kQOffG = kQOffP + kC * kC;      // kGateRows x 64 floats
constexpr int kQPSlot = kQOffG + 512;
// kPS (P formed in the scan): three slots of the Q tile and the gate rows, then two P tiles
constexpr int kQGSlot = kC * kDK + 512;
constexpr int kPSOffP = 3 * kQGSlot;
constexpr int kPSBuf = kPSOffP + 2 * kC * kC;


// kStates: the backward's forward sweep. The chain stores the fp32 state entering every chunk
// (Sst) and nothing else: no Q, P loads, no output wave work, no y.
// kPS: P = (Q K^T) o e^{G_r - G_i} (i <= r) is formed here, from the Q tile and the K tile
// already in LDS, instead of being read from the prep's tiles: the prep then reads no Q and
// writes no P. An eighth wave (wave 7, which shares the loader's SIMD; waves 4-6 only keep the
// barrier count) forms chunk c's P during step c into a P slot the output wave reads in step
// c + 1; Q now arrives one step earlier and stays two more, so it takes three slots.
template <typename Ty, bool kStates = false, bool kPS = false>
__global__ void __launch_bounds__(kPS ? 2 * kScanThreads : kScanThreads) chunk_scan_kernel(DevArgs a) {
    // the states-only sweep has the LDS for a third ring slot: its tiles arrive two chunks ahead
    constexpr int kR = kStates ? 3 : kRing;
    __shared__ __attribute__((aligned(16))) uint16_t ring[kR * kSlot];      // the chain's tiles
    __shared__ __attribute__((aligned(16))) uint16_t qpbuf[kPS ? kPSBuf : 2 * kQPSlot];   // the output wave's
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

    if constexpr (kPS) {
        if (wave == 7) {
            // ================= P wave (on the loader's SIMD): step c forms chunk c's P from the
            // Q and K tiles the loader brought in during step c - 1, into P slot c % 2, as the
            // swizzled row-major bf16 tile the prep would have written. Tile (rt, it) is formed transposed, A = K rows, B = Q rows, so
            // lane (c16, g) holds P[16 rt + c16][16 it + 4g .. + 3]: one 8-byte LDS store.
            auto form_p = [&](int ck) __attribute__((always_inline)) {
                const int n = min(kC, hi - (lo + ck * kC));
                const uint16_t* qs = qpbuf + (ck % 3) * kQGSlot;
                const uint16_t* ks = ring + (ck & 1) * kSlot + kOffK;
                const float* Gs = reinterpret_cast<const float*>(qs + kC * kDK) + 3 * kC;   // G
                uint16_t* ps = qpbuf + kPSOffP + (ck & 1) * kC * kC;
                const int swc = swz(c16);
                bf16x8 kf[4][4], qf[4][4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int o = (16 * t + c16) * kDK + (((4 * (s & 1) + g) ^ swc) << 3) + (s >> 1) * 64;
                        kf[t][s] = frag(ks + o);
                        qf[t][s] = frag(qs + o);
                    }
                constexpr int kRt[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
                constexpr int kIt[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
                f32x4 acc[10];
#pragma unroll
                for (int t = 0; t < 10; ++t) acc[t] = f32x4{};
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int t = 0; t < 10; ++t) acc[t] = mfma16(kf[kIt[t]][s], qf[kRt[t]][s], acc[t]);
                float gr[4];
                f32x4 gc[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    gr[t] = Gs[16 * t + c16];
                    gc[t] = *reinterpret_cast<const f32x4*>(Gs + 16 * t + 4 * g);
                }
                auto put = [&](int rt, int it, u32x2 v) __attribute__((always_inline)) {
                    *reinterpret_cast<u32x2*>(ps + (16 * rt + c16) * kC + (((2 * it + (g >> 1)) ^ swc) << 3) +
                                              4 * (g & 1)) = v;
                };
#pragma unroll
                for (int t = 0; t < 10; ++t) {
                    const int rt = kRt[t], it = kIt[t], r = 16 * rt + c16;
                    float pv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int col = 16 * it + 4 * g + e;
                        pv[e] = (col <= r && col < n) ? acc[t][e] * fexp(gr[rt] - gc[it][e]) : 0.f;
                    }
                    put(rt, it, u32x2{pack_bf2(pv[0], pv[1]), pack_bf2(pv[2], pv[3])});
                }
                // tiles above the diagonal that the output wave's fragments still cover
                put(0, 1, u32x2{0u, 0u});
                put(2, 3, u32x2{0u, 0u});
            };
            lds_barrier();   // chunk 0's tiles in
            for (int c = 0; c <= nchunks; ++c) {
                if (c < nchunks) form_p(c);
                lds_barrier();
            }
            return;
        }
        if (wave >= 4) {   // waves 4-6 only keep the barrier count (they exist so that wave 7
            lds_barrier();  // shares the loader's SIMD)
            for (int c = 0; c <= nchunks; ++c) lds_barrier();
            return;
        }
    }
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
            uint16_t* slot = ring + (ck % kR) * kSlot;
            rows128(a.k, t0, n, slot + kOffK);
            const uint16_t* vb = a.v + (size_t)t0 * a.H * a.dv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * i + (lane >> 2);
                const int o = n == kC ? offv[i] : (min(row, n - 1) * a.H + h) * a.dv + j0 + (lane & 3) * 8;
                dma16(vb + o, slot + kOffV + i * 512);
            }
            tile64(a.Tw + ch * kC * kC, slot + kOffT);
            dma16(a.Gw + ch * kGateRows * kC + lane * 4, slot + kOffG);
        };
        auto output_tiles = [&](int ck) __attribute__((always_inline)) {
            const int t0 = lo + ck * kC, n = min(kC, hi - t0);
            const size_t ch = (size_t)(cbase + ck) * a.H + h;
            uint16_t* slot = qpbuf + (ck & 1) * kQPSlot;
            rows128(a.q, t0, n, slot + kQOffQ);
            tile64(a.Pw + ch * kC * kC, slot + kQOffP);
            dma16(a.Gw + ch * kGateRows * kC + lane * 4, slot + kQOffG);
        };
        // kPS: Q and the gate rows of chunk ck into Q slot ck % 3
        auto q_tiles = [&](int ck) __attribute__((always_inline)) {
            const int t0 = lo + ck * kC, n = min(kC, hi - t0);
            const size_t ch = (size_t)(cbase + ck) * a.H + h;
            uint16_t* slot = qpbuf + (ck % 3) * kQGSlot;
            rows128(a.q, t0, n, slot);
            dma16(a.Gw + ch * kGateRows * kC + lane * 4, slot + kC * kDK);
        };
        if constexpr (kStates) {
            // chunks c + 2 are loaded in step c (29 loads per lane: K 16, V 4, T 8, gate rows 1);
            // the wait before the barrier is for chunk c + 1, issued a step earlier
            if (nchunks > 0) chain_tiles(0);
            if (nchunks > 1) {
                chain_tiles(1);
                GDN_WAIT_VMCNT(29);
            } else {
                GDN_WAIT_VMCNT(0);
            }
            dma_barrier();
            for (int c = 0; c <= nchunks; ++c) {
                if (c + 2 < nchunks) {
                    chain_tiles(c + 2);
                    GDN_WAIT_VMCNT(29);
                } else {
                    GDN_WAIT_VMCNT(0);
                }
                dma_barrier();
            }
            return;
        }
        if (nchunks > 0) {
            chain_tiles(0);
            if constexpr (kPS) q_tiles(0);
        }
        GDN_WAIT_VMCNT(0);
        dma_barrier();
        for (int c = 0; c <= nchunks; ++c) {
            if constexpr (kPS) {
                if (c + 1 < nchunks) {
                    chain_tiles(c + 1);
                    q_tiles(c + 1);
                }
            } else {
                if (c + 1 < nchunks) chain_tiles(c + 1);
                if (!kStates && c < nchunks) output_tiles(c);
            }
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
        int oqf[2], opf[2];   // from the Q tile's and the P tile's start
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            oqf[sp] = c16 * kDK + (((4 * sp + g) ^ swz(c16)) << 3);
            opf[sp] = c16 * kC + (((4 * sp + g) ^ swz(c16)) << 3);
        }
        const size_t ytok = (size_t)a.H * a.dv;   // elements between consecutive tokens of y
        Ty* const ylane = static_cast<Ty*>(a.y) + (size_t)h * a.dv + j0 + 4 * g + (size_t)c16 * ytok;
        auto output = [&](int cy) __attribute__((always_inline)) {
            const uint16_t* slot = kPS ? qpbuf + (cy % 3) * kQGSlot : qpbuf + (cy & 1) * kQPSlot + kQOffQ;
            const uint16_t* pslot = kPS ? qpbuf + kPSOffP + (cy & 1) * kC * kC : slot - kQOffQ + kQOffP;
            const float* sGq = reinterpret_cast<const float*>(kPS ? slot + kC * kDK : slot - kQOffQ + kQOffG);
            // The two slices' accumulators (8) take turns in every product group, so no product
            // waits for the result of the one just issued; each accumulator still adds its
            // terms in the order S^T Q^T (s = 0..3), the gamma scaling, U^T P^T.
            bf16x8 qf[4][4], pf[4][2], Sb[2][4];
            f32x4 YT[2][4], U[2][4];
            float gq[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) Sb[sl][s] = __builtin_bit_cast(bf16x8, xbuf[cy & 1][sl][s * 64 + lane]);
                // rows 16 apart share the swizzle, units 8 apart are 64 elements apart
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) qf[rt][s] = frag(slot + oqf[s & 1] + rt * 16 * kDK + (s >> 1) * 64);
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) YT[sl][rt] = f32x4{};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Sb[sl][s], qf[rt][s], YT[sl][rt]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) U[sl][rt] = __builtin_bit_cast(f32x4, xbuf[cy & 1][sl][(4 + rt) * 64 + lane]);
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (s <= (rt >> 1)) pf[rt][s] = frag(pslot + opf[s] + rt * 16 * kC);
                gq[rt] = sGq[kC + 16 * rt + c16];
            }
            bf16x8 Uh[2][2], Ul[2][2];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                split8(U[sl][0], U[sl][1], Uh[sl][0], Ul[sl][0]);
                split8(U[sl][2], U[sl][3], Uh[sl][1], Ul[sl][1]);
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) YT[sl][rt] *= gq[rt];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Uh[sl][0], pf[rt][0], YT[sl][rt]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Ul[sl][0], pf[rt][0], YT[sl][rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Uh[sl][1], pf[rt][1], YT[sl][rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Ul[sl][1], pf[rt][1], YT[sl][rt]);
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
            if (!kStates && c >= 1) output(c - 1);
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
        const uint16_t* slot = ring + (c % kR) * kSlot;
        const float* sG = reinterpret_cast<const float*>(slot + kOffG);   // beta | gamma | gamma_C/gamma
        u32x4* xb = xbuf[c & 1][wave];
        if constexpr (kStates) {   // S[2s], S[2s+1] hold d_k rows 32s + 8g .. + 7 of column j0w + c16
            float* st = a.Sst + ((size_t)(cbase + c) * a.H + h) * kDK * kDK +
                        (size_t)(j0w + c16) * kDK + 8 * g;
#pragma unroll
            for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(st + 32 * (t >> 1) + 4 * (t & 1)) = S[t];
        }
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
        if constexpr (!kStates) {
#pragma unroll
            for (int s = 0; s < 4; ++s) xb[s * 64 + lane] = __builtin_bit_cast(u32x4, Sb[s]);
        }
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
        if constexpr (!kStates) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) xb[(4 + rt) * 64 + lane] = __builtin_bit_cast(u32x4, U[rt]);
        }
        bf16x8 Wh[2], Wl[2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) U[rt] *= gd[rt];
        split8(U[0], U[1], Wh[0], Wl[0]);
        split8(U[2], U[3], Wh[1], Wl[1]);
        load_kt(4);
        load_kt(5);
        GDN_SCHED_FENCE();
        // ---- S = gamma_C S + K^T W over tiles t0 .. t0 + 3, then their split for the next
        //      chunk | K^T fragments of tiles 6-7. Each tile adds its four products in the same
        //      order as before, but the four tiles take turns, so no product waits for the
        //      result of the one issued just before it (a dependent product stalls its wave for
        //      the whole matrix-core latency).
        auto upd4 = [&](int t0) {
            bf16x8 ktf[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const u32x2 p0 = __builtin_bit_cast(u32x2, kt[t0 + t][s][0]);
                    const u32x2 p1 = __builtin_bit_cast(u32x2, kt[t0 + t][s][1]);
                    const u32x4 pk = {p0.x, p0.y, p1.x, p1.y};
                    ktf[t][s] = __builtin_bit_cast(bf16x8, pk);
                }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int t = 0; t < 4; ++t) S[t0 + t] = mfma16(ktf[t][s], Wh[s], S[t0 + t]);
#pragma unroll
                for (int t = 0; t < 4; ++t) S[t0 + t] = mfma16(ktf[t][s], Wl[s], S[t0 + t]);
            }
            Sb[t0 >> 1] = to_bf16x8(S[t0], S[t0 + 1]);
            Sb[(t0 >> 1) + 1] = to_bf16x8(S[t0 + 2], S[t0 + 3]);
        };
        upd4(0);
        load_kt(6);
        load_kt(7);
        GDN_IGLP(16, 2, 1);
        GDN_SCHED_FENCE();
        upd4(4);
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

// ------------------------------------------------------------------ forward scan, tiles two ahead
// The forward form of the sliced scan above (P formed in the scan), with every tile a step needs
// arriving two chunks ahead instead of one: a chunk's loads from HBM take about as long as a step,
// so with one chunk of lead the step waited on them. The LDS holds three chunks of K, the V slice
// and the gate rows (ring), three Q tiles and two P tiles; T leaves the LDS: each chain wave loads
// its six T fragments straight from the workspace into registers, one chunk ahead (two buffers
// of them spill). The output
// wave forms chunk c's S^T Q^T in step c (from the state operand the chain left before step c's
// barrier), so a Q tile is read in the step of its chunk only, and finishes it in step c + 1
// (gamma, U^T P^T, store). Per accumulator the products are the sliced scan's, in its order.
constexpr int kFSlot = kC * kDK + kC * kSl + 512;   // K | V slice | gate rows (bf16 elements)
constexpr int kFOffV = kC * kDK;
constexpr int kFOffG = kFOffV + kC * kSl;
constexpr size_t kFwdMaxTBytes = size_t(128) << 20;   // T tiles of one call, see the launcher

template <typename Ty>
__global__ void __launch_bounds__(2 * kScanThreads) chunk_scan_fwd_kernel(DevArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ring[3 * kFSlot];
    __shared__ __attribute__((aligned(16))) uint16_t qbuf[3 * kC * kDK];
    __shared__ __attribute__((aligned(16))) uint16_t pbuf[2 * kC * kC];
    // [chunk parity][slice][8 x 64 lanes x 16 bytes]: rows 0-3 the bf16 state operand entering
    // the chunk (written by the chain before the step's barrier), rows 4-7 the chunk's fp32 U
    __shared__ __attribute__((aligned(16))) u32x4 xbuf[2][2][8 * 64];

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
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j0 = slice * kSl;
    const int c16 = lane & 15, g = lane >> 4;

    if (wave == 7) {
        // ================= P wave: step c forms chunk c's P into P slot c % 2 (as chunk_scan_kernel)
        auto form_p = [&](int ck) __attribute__((always_inline)) {
            const int n = min(kC, hi - (lo + ck * kC));
            const uint16_t* qs = qbuf + (ck % 3) * kC * kDK;
            const uint16_t* ks = ring + (ck % 3) * kFSlot;
            const float* Gs = reinterpret_cast<const float*>(ks + kFOffG) + 3 * kC;   // G
            uint16_t* ps = pbuf + (ck & 1) * kC * kC;
            const int swc = swz(c16);
            bf16x8 kf[4][4], qf[4][4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int o = (16 * t + c16) * kDK + (((4 * (s & 1) + g) ^ swc) << 3) + (s >> 1) * 64;
                    kf[t][s] = frag(ks + o);
                    qf[t][s] = frag(qs + o);
                }
            constexpr int kRt[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
            constexpr int kIt[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
            f32x4 acc[10];
#pragma unroll
            for (int t = 0; t < 10; ++t) acc[t] = f32x4{};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int t = 0; t < 10; ++t) acc[t] = mfma16(kf[kIt[t]][s], qf[kRt[t]][s], acc[t]);
            float gr[4];
            f32x4 gc[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                gr[t] = Gs[16 * t + c16];
                gc[t] = *reinterpret_cast<const f32x4*>(Gs + 16 * t + 4 * g);
            }
            auto put = [&](int rt, int it, u32x2 v) __attribute__((always_inline)) {
                *reinterpret_cast<u32x2*>(ps + (16 * rt + c16) * kC + (((2 * it + (g >> 1)) ^ swc) << 3) +
                                          4 * (g & 1)) = v;
            };
#pragma unroll
            for (int t = 0; t < 10; ++t) {
                const int rt = kRt[t], it = kIt[t], r = 16 * rt + c16;
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int col = 16 * it + 4 * g + e;
                    pv[e] = (col <= r && col < n) ? acc[t][e] * fexp(gr[rt] - gc[it][e]) : 0.f;
                }
                put(rt, it, u32x2{pack_bf2(pv[0], pv[1]), pack_bf2(pv[2], pv[3])});
            }
            put(0, 1, u32x2{0u, 0u});
            put(2, 3, u32x2{0u, 0u});
        };
        lds_barrier();   // chunk 0's tiles in
        for (int c = 0; c <= nchunks; ++c) {
            if (c < nchunks) form_p(c);
            lds_barrier();
        }
        return;
    }
    if (wave >= 4) {   // waves 4-6 only keep the barrier count (so that wave 7 shares wave 3's SIMD)
        lds_barrier();
        for (int c = 0; c <= nchunks; ++c) lds_barrier();
        return;
    }
    if (wave == 3) {
        // ================= loader: step c fills ring slot and Q slot (c + 2) % 3 with chunk c + 2
        // (they held chunk c - 1, finished before this step's barrier), then waits for chunk
        // c + 1's loads (issued a step earlier) before the barrier.
        int offk[16], offv[4];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 4 * i + (lane >> 4), u = (lane & 15) ^ swz(row);
            offk[i] = (row * a.H + h) * kDK + u * 8;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) offv[i] = ((16 * i + (lane >> 2)) * a.H + h) * a.dv + j0 + (lane & 3) * 8;
        auto rows128 = [&](const uint16_t* x, int t0, int n, uint16_t* dst) __attribute__((always_inline)) {
            const uint16_t* xb = x + (size_t)t0 * a.H * kDK;
            if (n == kC) {
#pragma unroll
                for (int i = 0; i < 16; ++i) dma16(xb + offk[i], dst + i * 512);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 4 * i + (lane >> 4), u = (lane & 15) ^ swz(row);
                    dma16(xb + (min(row, n - 1) * a.H + h) * kDK + u * 8, dst + i * 512);
                }
            }
        };
        // 37 loads per lane per chunk: K 16, V 4, gate rows 1, Q 16
        auto chunk_tiles = [&](int ck) __attribute__((always_inline)) {
            const int t0 = lo + ck * kC, n = min(kC, hi - t0);
            const size_t ch = (size_t)(cbase + ck) * a.H + h;
            uint16_t* slot = ring + (ck % 3) * kFSlot;
            rows128(a.k, t0, n, slot);
            const uint16_t* vb = a.v + (size_t)t0 * a.H * a.dv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * i + (lane >> 2);
                const int o = n == kC ? offv[i] : (min(row, n - 1) * a.H + h) * a.dv + j0 + (lane & 3) * 8;
                dma16(vb + o, slot + kFOffV + i * 512);
            }
            dma16(a.Gw + ch * kGateRows * kC + lane * 4, slot + kFOffG);
            rows128(a.q, t0, n, qbuf + (ck % 3) * kC * kDK);
        };
        if (nchunks > 0) chunk_tiles(0);
        if (nchunks > 1) {
            chunk_tiles(1);
            GDN_WAIT_VMCNT(37);
        } else {
            GDN_WAIT_VMCNT(0);
        }
        dma_barrier();
        for (int c = 0; c <= nchunks; ++c) {
            if (c + 2 < nchunks) {
                chunk_tiles(c + 2);
                GDN_WAIT_VMCNT(37);
            } else {
                GDN_WAIT_VMCNT(0);
            }
            dma_barrier();
        }
        return;
    }
    if (wave == 2) {
        // ================= output wave: step c starts chunk c (gamma-free S^T Q^T of both
        // slices) and finishes chunk c - 1 (gamma, U^T P^T, y)
        int oqf[2], opf[2];
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            oqf[sp] = c16 * kDK + (((4 * sp + g) ^ swz(c16)) << 3);
            opf[sp] = c16 * kC + (((4 * sp + g) ^ swz(c16)) << 3);
        }
        const size_t ytok = (size_t)a.H * a.dv;
        Ty* const ylane = static_cast<Ty*>(a.y) + (size_t)h * a.dv + j0 + 4 * g + (size_t)c16 * ytok;
        f32x4 YT[2][4];   // the chunk started in the previous step
        float gq[4];      // its gamma at the lane's 4 tokens
        auto finish = [&](int cy) __attribute__((always_inline)) {
            const uint16_t* pslot = pbuf + (cy & 1) * kC * kC;
            bf16x8 pf[4][2];
            f32x4 U[2][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) U[sl][rt] = __builtin_bit_cast(f32x4, xbuf[cy & 1][sl][(4 + rt) * 64 + lane]);
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (s <= (rt >> 1)) pf[rt][s] = frag(pslot + opf[s] + rt * 16 * kC);
            }
            bf16x8 Uh[2][2], Ul[2][2];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                split8(U[sl][0], U[sl][1], Uh[sl][0], Ul[sl][0]);
                split8(U[sl][2], U[sl][3], Uh[sl][1], Ul[sl][1]);
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) YT[sl][rt] *= gq[rt];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Uh[sl][0], pf[rt][0], YT[sl][rt]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Ul[sl][0], pf[rt][0], YT[sl][rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Uh[sl][1], pf[rt][1], YT[sl][rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Ul[sl][1], pf[rt][1], YT[sl][rt]);
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
        auto start = [&](int cs) __attribute__((always_inline)) {
            const uint16_t* qs = qbuf + (cs % 3) * kC * kDK;
            const float* sGq = reinterpret_cast<const float*>(ring + (cs % 3) * kFSlot + kFOffG);
            bf16x8 qf[4][4], Sb[2][4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) Sb[sl][s] = __builtin_bit_cast(bf16x8, xbuf[cs & 1][sl][s * 64 + lane]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) qf[rt][s] = frag(qs + oqf[s & 1] + rt * 16 * kDK + (s >> 1) * 64);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) gq[rt] = sGq[kC + 16 * rt + c16];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) YT[sl][rt] = f32x4{};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl) YT[sl][rt] = mfma16(Sb[sl][s], qf[rt][s], YT[sl][rt]);
        };
        lds_barrier();   // chunk 0's tiles and state operand in
        for (int c = 0; c <= nchunks; ++c) {
            if (c >= 1) finish(c - 1);
            GDN_SCHED_FENCE();
            if (c < nchunks) start(c);
            lds_barrier();
        }
        return;
    }

    // ================= chain waves: d_v columns j0w .. j0w + 15 (as chunk_scan_kernel's chain)
    const int j0w = j0 + 16 * wave;
    const size_t sbase = ((size_t)seq * a.H + h) * kDK * a.dv;
    f32x4 S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) S[t] = f32x4{};
    if (a.S0) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[t][i] = a.S0[sbase + (size_t)relabel(t, 4 * g + i) * a.dv + j0w + c16];
    }
    bf16x8 Sb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        Sb[s] = to_bf16x8(S[2 * s], S[2 * s + 1]);
        xbuf[0][wave][s * 64 + lane] = __builtin_bit_cast(u32x4, Sb[s]);
    }
    int okf[2][2], okt[2][2], otg[2][2];
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2) {
        const int r = relabel(a2, c16);
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            okf[a2][sp] = r * kDK + (((4 * sp + g) ^ swz(r)) << 3);
            otg[a2][sp] = r * kC + 8 * (4 * sp + g);   // T row r, unit 4 sp + g, in the workspace
        }
    }
    const int jj = (lane & 15) >> 2, r4 = lane & 3;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int tok = 8 * g + jj + 4 * hf;
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) okt[hf][tp] = tok * kDK + (((4 * tp + r4) ^ swz(tok)) << 3);
    }
    const int ov = kFOffV + (8 * g + jj) * kSl + 16 * wave + 4 * r4;
    // T fragments [row tile][step] of chunk ck (clamped to the last chunk) from the workspace
    auto load_t = [&](int ck, bf16x8 (&tf)[4][2]) __attribute__((always_inline)) {
        const size_t ch = (size_t)(cbase + min(ck, nchunks - 1)) * a.H + h;
        const uint16_t* tb = a.Tw + ch * kC * kC;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                if (s <= (rt >> 1)) tf[rt][s] = frag(tb + otg[rt & 1][s] + (rt >> 1) * 32 * kC);
    };

    auto step = [&](int c, bf16x8 (&tf)[4][2]) __attribute__((always_inline)) {
        const uint16_t* slot = ring + (c % 3) * kFSlot;
        const float* sG = reinterpret_cast<const float*>(slot + kFOffG);   // beta | gamma | gamma_C/gamma
        auto kfrag = [&](int rt, int s) {
            return frag(slot + okf[rt & 1][s & 1] + (rt >> 1) * 32 * kDK + (s >> 1) * 64);
        };
        auto ktr = [&](int t, int s, int hf) {
            return lds_tr16(slot + okt[hf][(t >> 1) & 1] + s * 32 * kDK + (t >> 2) * 64 + 4 * (t & 1));
        };
        auto grow = [&](int which, int rt) {
            return *reinterpret_cast<const f32x4*>(sG + which * kC + 8 * g + 32 * (rt >> 1) + 4 * (rt & 1));
        };
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
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) KS[rt] = f32x4{};
        mma_k(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t] *= gC;
        load_k(2);
        load_k(3);
        GDN_IGLP(4, 4, 2);
        GDN_SCHED_FENCE();
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
        f32x4 gd[4];
        mma_k(2);
        mma_k(3);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) gd[rt] = grow(2, rt);
        GDN_IGLP(8, 1, 1);
        GDN_SCHED_FENCE();
        s16x4 kt[8][2][2];
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
        // T of chunk c + 1 into the registers just used (in flight for a step; the prep wrote
        // it just before this kernel, and the launcher takes this kernel when the call's T
        // tiles fit well inside the Infinity Cache)
        load_t(c + 1, tf);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) xbuf[c & 1][wave][(4 + rt) * 64 + lane] = __builtin_bit_cast(u32x4, U[rt]);
        bf16x8 Wh[2], Wl[2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) U[rt] *= gd[rt];
        split8(U[0], U[1], Wh[0], Wl[0]);
        split8(U[2], U[3], Wh[1], Wl[1]);
        load_kt(4);
        load_kt(5);
        GDN_SCHED_FENCE();
        auto upd4 = [&](int t0) {
            bf16x8 ktf[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const u32x2 p0 = __builtin_bit_cast(u32x2, kt[t0 + t][s][0]);
                    const u32x2 p1 = __builtin_bit_cast(u32x2, kt[t0 + t][s][1]);
                    const u32x4 pk = {p0.x, p0.y, p1.x, p1.y};
                    ktf[t][s] = __builtin_bit_cast(bf16x8, pk);
                }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int t = 0; t < 4; ++t) S[t0 + t] = mfma16(ktf[t][s], Wh[s], S[t0 + t]);
#pragma unroll
                for (int t = 0; t < 4; ++t) S[t0 + t] = mfma16(ktf[t][s], Wl[s], S[t0 + t]);
            }
            Sb[t0 >> 1] = to_bf16x8(S[t0], S[t0 + 1]);
            Sb[(t0 >> 1) + 1] = to_bf16x8(S[t0 + 2], S[t0 + 3]);
        };
        upd4(0);
        load_kt(6);
        load_kt(7);
        GDN_IGLP(16, 2, 1);
        GDN_SCHED_FENCE();
        upd4(4);
        GDN_IGLP(16, 1, 0);
        GDN_SCHED_FENCE();
        // the next chunk's state operand, for the output wave (it starts that chunk next step)
#pragma unroll
        for (int s = 0; s < 4; ++s) xbuf[(c + 1) & 1][wave][s * 64 + lane] = __builtin_bit_cast(u32x4, Sb[s]);
        lds_barrier();   // past this barrier the ring slot is refilled and the exchange read
    };

    bf16x8 tf[4][2];
    if (nchunks > 0) load_t(0, tf);
    lds_barrier();   // chunks 0 (and 1) in the ring, the state operand in the exchange buffer
    for (int c = 0; c < nchunks; ++c) step(c, tf);
    GDN_WAIT_VMCNT(0);   // the last step's T loads (of no chunk still to come) land before exit
    lds_barrier();   // the output wave finishes the last chunk
    if (a.ST) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.ST[sbase + (size_t)relabel(t, 4 * g + i) * a.dv + j0w + c16] = S[t][i];
    }
}

// ------------------------------------------------------------------ per-channel decay: prep
// The per-channel-decay variant (the delta rule with Diag(alpha_t) over the key channels, as
// in the Kimi Delta Attention entry the reading notes compare GDN with): row c of the state
// decays by alpha_t[c] = e^{g_t[c]}. Inside a chunk, with Gc[r][c] the running sum of g over
// the chunk's tokens,
//   A[r,i] = beta_r sum_c k_r[c] k_i[c] e^{Gc[r][c]-Gc[i][c]} (i < r),  T = (I + A)^{-1}
//   P[r,i] = sum_c q_r[c] k_i[c] e^{Gc[r][c]-Gc[i][c]}          (i <= r)
//   U = T (beta o (V - Kg S)),  Y = Qg S + P U,  S' = e^{Gc[C]} o S + Kc^T U
// with Kg = K o e^{Gc}, Qg = Q o e^{Gc}, Kc = K o e^{Gc[C] - Gc} (exponents <= 0).
// This path takes the lower bound of that family's log-decay, g >= -5, to put A and P on the
// bf16 matrix cores: for a 16-token row block a with first row m, e^{Gc_r - Gc_i} =
// e^{Gc_r - Gc_m} e^{Gc_m - Gc_i}. The first factor lies in [e^-80, 1] (16 tokens of at most
// 5 each); the second is <= 1 for i in earlier blocks and in [1, e^80] inside block a, so
// every scaled operand stays far inside the bf16 / fp32 range and each 16x16 block of A and
// P is one product of scaled K, Q rows over the 128 channels (v_mfma_f32_16x16x32_bf16).
// One 256-thread workgroup per (chunk, head) writes Kg, Kc, Qg, T and P in bf16, and
// beta | e^{Gc[C]} for the scan.
constexpr int kKdaPrepThreads = 256;
constexpr int kGsStr = kDK + 4;   // row stride (floats) of the running log-decays in LDS

__global__ void __launch_bounds__(kKdaPrepThreads) kda_prep_bf16_kernel(DevArgs a) {
    __shared__ __attribute__((aligned(16))) float Gs[kC * kGsStr];
    __shared__ __attribute__((aligned(16))) float sA[kC * kStrA];
    __shared__ __attribute__((aligned(16))) uint16_t sP[kC * kC];
    __shared__ float sB[kC];
    const int chunk = blockIdx.x, h = blockIdx.y;
    int seq, t0, n;
    if (!chunk_of(a, chunk, seq, t0, n)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const size_t ch = (size_t)chunk * a.H + h;
    const size_t rowH = (size_t)a.H * kDK;   // elements between consecutive tokens of q, k, g

    // Every global load of the rows is issued up front and unconditionally (row n - 1 stands in
    // past the end and is zeroed after): a load under a branch is waited for where it joins.
    auto row8 = [&](const uint16_t* x, int r, int c0) {   // raw, row clamped
        return *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + min(r, n - 1)) * rowH + (size_t)h * kDK + c0);
    };
    constexpr int kUnits = kC * kDK / 8 / kKdaPrepThreads;   // 16-byte units per thread
    constexpr int kGUnits = kC * kDK / 4 / kKdaPrepThreads;  // log-decay float4s per thread
    u32x4 kws[kUnits], qws[kUnits];
    f32x4p gvs[kGUnits];
#pragma unroll
    for (int j = 0; j < kGUnits; ++j) {
        const int u = tid + j * kKdaPrepThreads, r = u / (kDK / 4), c4 = (u % (kDK / 4)) * 4;
        gvs[j] = *reinterpret_cast<const f32x4p*>(a.gk + (size_t)(t0 + min(r, n - 1)) * rowH + (size_t)h * kDK + c4);
    }
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
        const int u = tid + j * kKdaPrepThreads, r = u / (kDK / 8), c0 = (u % (kDK / 8)) * 8;
        kws[j] = row8(a.k, r, c0);
        qws[j] = row8(a.q, r, c0);
    }
    const float braw = a.beta[(size_t)(t0 + min(tid & (kC - 1), n - 1)) * a.H + h];
    // log-decays of the chunk's rows (rows >= n decay by nothing) and beta
#pragma unroll
    for (int j = 0; j < kGUnits; ++j) {
        const int u = tid + j * kKdaPrepThreads, r = u / (kDK / 4), c4 = (u % (kDK / 4)) * 4;
        const f32x4p z4 = {0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4p*>(&Gs[r * kGsStr + c4]) = r < n ? gvs[j] : z4;
    }
    if (tid < kC) sB[tid] = tid < n ? braw : 0.f;
    for (int e = tid; e < kC * kStrA; e += kKdaPrepThreads) sA[e] = 0.f;
    __syncthreads();
    {   // running sums down the tokens: thread (half, channel) sums its 32 rows in registers,
        // then the second half adds the first half's total
        const int c = tid & (kDK - 1), r0 = (tid >> 7) * (kC / 2);
        float v[kC / 2];
#pragma unroll
        for (int r = 0; r < kC / 2; ++r) v[r] = Gs[(r0 + r) * kGsStr + c];
#pragma unroll
        for (int r = 1; r < kC / 2; ++r) v[r] += v[r - 1];
#pragma unroll
        for (int r = 0; r < kC / 2; ++r) Gs[(r0 + r) * kGsStr + c] = v[r];
        __syncthreads();
        if (r0) {
            const float base = Gs[(kC / 2 - 1) * kGsStr + c];
#pragma unroll
            for (int r = 0; r < kC / 2; ++r) Gs[(r0 + r) * kGsStr + c] = v[r] + base;
        }
    }
    __syncthreads();

    // Kg, Kc, Qg rows (8 channels, one 16-byte store each; rows >= n are zero)
    auto bfv = [](const u32x4& w, int j) {
        const uint32_t x = w[j >> 1];
        return __uint_as_float((j & 1) ? (x & 0xffff0000u) : (x << 16));
    };
    uint16_t* xw = a.Xw + ch * 3 * kC * kDK;
    const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int jj = 0; jj < kUnits; ++jj) {
        const int u = tid + jj * kKdaPrepThreads;
        const int r = u / (kDK / 8), c0 = (u % (kDK / 8)) * 8;
        const u32x4 kw = r < n ? kws[jj] : z4, qw = r < n ? qws[jj] : z4;
        float kg[8], kc[8], qg[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float G = Gs[r * kGsStr + c0 + j], GC = Gs[(kC - 1) * kGsStr + c0 + j];
            const float e = fexp(G), ec = fexp(GC - G);
            kg[j] = bfv(kw, j) * e;
            qg[j] = bfv(qw, j) * e;
            kc[j] = bfv(kw, j) * ec;
        }
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = pack_bf2(kg[2 * j], kg[2 * j + 1]);
        *reinterpret_cast<u32x4*>(xw + r * kDK + c0) = o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = pack_bf2(kc[2 * j], kc[2 * j + 1]);
        *reinterpret_cast<u32x4*>(xw + kC * kDK + r * kDK + c0) = o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = pack_bf2(qg[2 * j], qg[2 * j + 1]);
        *reinterpret_cast<u32x4*>(xw + 2 * kC * kDK + r * kDK + c0) = o;
    }
    float* gw = a.Gw + ch * kGateRows * kC;   // beta | e^{Gc[C]}
    if (tid < kC) gw[tid] = sB[tid];
    else if (tid < kC + kDK) gw[tid] = fexp(Gs[(kC - 1) * kGsStr + tid - kC]);

    // the ten lower 16x16 blocks (row block ra >= column block rb) of A and P; wave w takes
    // blocks w, w + 4, w + 8 of the list (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
    for (int bi = wave; bi < 10; bi += kKdaPrepThreads / kWave) {
        const int ra = bi < 1 ? 0 : (bi < 3 ? 1 : (bi < 6 ? 2 : 3));
        const int rb = bi - ra * (ra + 1) / 2;
        const int m = 16 * ra, rl = 16 * ra + c16, rr = 16 * rb + c16;
        f32x4 cA = {0.f, 0.f, 0.f, 0.f}, cP = {0.f, 0.f, 0.f, 0.f};
        u32x4 kls[kDK / 32], qls[kDK / 32], krs[kDK / 32];
#pragma unroll
        for (int s2 = 0; s2 < kDK / 32; ++s2) {
            const int c0 = 32 * s2 + 8 * g;
            kls[s2] = row8(a.k, rl, c0);
            qls[s2] = row8(a.q, rl, c0);
            krs[s2] = row8(a.k, rr, c0);
        }
#pragma unroll
        for (int s2 = 0; s2 < kDK / 32; ++s2) {
            const int c0 = 32 * s2 + 8 * g;
            const u32x4 kl = rl < n ? kls[s2] : z4, ql = rl < n ? qls[s2] : z4, kr = rr < n ? krs[s2] : z4;
            float lk[8], lq[8], rk[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float gm = Gs[m * kGsStr + c0 + j];
                const float el = fexp(Gs[rl * kGsStr + c0 + j] - gm);
                const float er = fexp(gm - Gs[rr * kGsStr + c0 + j]);
                lk[j] = bfv(kl, j) * el;
                lq[j] = bfv(ql, j) * el;
                rk[j] = bfv(kr, j) * er;
            }
            u32x4 wl, wq, wr;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wl[j] = pack_bf2(lk[2 * j], lk[2 * j + 1]);
                wq[j] = pack_bf2(lq[2 * j], lq[2 * j + 1]);
                wr[j] = pack_bf2(rk[2 * j], rk[2 * j + 1]);
            }
            const bf16x8 fr = __builtin_bit_cast(bf16x8, wr);
            cA = mfma16(__builtin_bit_cast(bf16x8, wl), fr, cA);
            cP = mfma16(__builtin_bit_cast(bf16x8, wq), fr, cP);
        }
        // accumulator element i: row 16 ra + 4g + i, column 16 rb + c16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ra + 4 * g + i, c = 16 * rb + c16;
            sA[r * kStrA + c] = c < r ? sB[r] * cA[i] : 0.f;
            sP[r * kC + c] = c <= r ? uint16_t(pack_bf2(cP[i], 0.f) & 0xffffu) : uint16_t(0);
        }
    }
    // the blocks above the diagonal of P are zero
    for (int e = tid; e < kC * kC; e += kKdaPrepThreads) {
        const int r = e / kC, c = e % kC;
        if ((c >> 4) > (r >> 4)) sP[e] = 0;
    }
    __syncthreads();
    if (wave == 0) unit_lower_inverse64<kStrA, true>(sA);
    __syncthreads();
    const size_t tile = ch * kC * kC;
    for (int u = tid; u < kC * kC / 8; u += kKdaPrepThreads) {   // T and P, 8 elements per store
        const int r = u / (kC / 8), c0 = (u % (kC / 8)) * 8;
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = pack_bf2(sA[r * kStrA + c0 + 2 * j], sA[r * kStrA + c0 + 2 * j + 1]);
        *reinterpret_cast<u32x4*>(a.Tw + tile + r * kC + c0) = o;
        *reinterpret_cast<u32x4*>(a.Pw + tile + r * kC + c0) = *reinterpret_cast<const u32x4*>(&sP[r * kC + c0]);
    }
}

// ------------------------------------------------------------------ full-row scan
// One workgroup per (sequence, head) holding all 128 d_v columns: 8 waves, wave w runs the
// chain above for columns 16w .. 16w + 15 and also forms their output, Y = gamma Q S + P U
// (as the output wave above does, from the same operands in the same order). Every wave loads
// an eighth of the next chunk's tiles (K, V, Q, T, P and the gate rows) straight into LDS at
// the start of a step. With all the columns of a token's y in one workgroup, the gated
// zero-centred RMSNorm of eq. (11) (o = sigmoid(z) (1 + w) y / rms(y) over the d_v columns)
// runs in the scan's epilogue: the waves exchange their per-token sums of y^2 in LDS and
// chunk c's o is formed at the start of step c + 1, after the barrier both need anyway, so y
// need not leave the chip. Two waves share a SIMD and hide each other's latency: a CU does
// about 3.5 times the chunk-columns per unit time of the sliced scan, but holds one (sequence,
// head), so the launcher takes this kernel when the pairs fill the chip.
constexpr int kWideWaves = 8;
constexpr int kWOffK = 0;                    // [64][128] bf16, 16-byte units swizzled per row
constexpr int kWOffV = kWOffK + kC * kDK;    // [64][128], the same
constexpr int kWOffQ = kWOffV + kC * kDK;    // [64][128], the same
constexpr int kWOffT = kWOffQ + kC * kDK;    // [64][64], the same
constexpr int kWOffP = kWOffT + kC * kC;     // [64][64], the same
constexpr int kWOffG = kWOffP + kC * kC;     // beta | gamma | gamma_C / gamma | G
constexpr int kWSlot = kWOffG + 512;

struct GateDev {
    const void* z;          // [ntok, H, 128]
    const float* w;         // [128] zero-centred RMSNorm weight
    void* o;                // [ntok, H, 128]
    float eps;
};

// kKda: the per-channel-decay variant (see kda_prep_bf16_kernel). The ring slots then hold Kg
// (for K S), Kc (for the update, in V's place) and Qg, the gate rows are beta | e^{Gc[C]},
// V comes from global memory into registers (the end-of-step wait covers it), the state decays
// per row, and there are no scalar gamma factors.
// kWv: waves per workgroup (16 columns each). 8 gives the full row (the only form that can
// apply the gate); 4 or 2 split a (sequence, head) over 2 or 4 workgroups that each load the
// chunk's whole tiles (the same bytes from HBM, shared in L2: a pair's workgroups are 8 apart
// in the grid, so on one XCD), for calls with too few pairs to fill the chip.
template <typename Ty, bool kGate, typename Tz, typename To, bool kKda, int kWv>
__global__ void __launch_bounds__(kWv * kWave) chunk_scan_wide_kernel(DevArgs a, GateDev gd_) {
    static_assert(kWv == 8 || kWv == 4 || kWv == 2, "waves per workgroup");
    static_assert(!kGate || kWv == 8, "the gate needs every column of a row");
    constexpr int kNsl = kWideWaves / kWv;   // workgroups per (sequence, head)
    // The two slots are separate arrays and each half of the 2-unrolled chunk loop names its
    // slots statically: the compiler then sees that the direct loads into one slot cannot alias
    // the reads of the other, and inserts no wait for the loads in flight before those reads
    // (with one array and a computed slot it waits for all of them at the first LDS read).
    __shared__ __attribute__((aligned(16))) uint16_t ring0[kWSlot];
    __shared__ __attribute__((aligned(16))) uint16_t ring1[kWSlot];
    __shared__ float ssq[kGate ? 2 : 1][kWideWaves][kC];   // per-wave sums of y^2 per token

    // block -> (pair, slice): the slices of one pair are 8 blocks apart
    const int b = blockIdx.x;
    const int group = b / (8 * kNsl), within = b % (8 * kNsl);
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
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15, g = lane >> 4;
    const int j0w = slice * kWv * 16 + 16 * wave;
    constexpr int DV = 128;

    // ---- this wave's share of a chunk's tiles, loaded straight into `slot`
    auto load_chunk = [&](int ck, uint16_t* slot) __attribute__((always_inline)) {
        const int t0 = lo + ck * kC, n = min(kC, hi - t0);
        const size_t ch = (size_t)(cbase + ck) * a.H + h;
        // [64][128] rows of K, V and Q (Kg, Kc and Qg): 16 one-kilobyte pieces each, 16 / kWv
        // per wave
#pragma unroll
        for (int j = 0; j < 16 / kWv; ++j) {
            const int i = (16 / kWv) * wave + j;
            const int row = 4 * i + (lane >> 4), u = (lane & 15) ^ swz(row);
            if constexpr (kKda) {
                const uint16_t* xs = a.Xw + ch * 3 * kC * kDK + row * kDK + u * 8;
                dma16(xs, slot + kWOffK + i * 512);
                dma16(xs + kC * kDK, slot + kWOffV + i * 512);
                dma16(xs + 2 * kC * kDK, slot + kWOffQ + i * 512);
            } else {
                const size_t src = ((size_t)(t0 + min(row, n - 1)) * a.H + h) * kDK + u * 8;
                dma16(a.k + src, slot + kWOffK + i * 512);
                dma16(a.v + src, slot + kWOffV + i * 512);
                dma16(a.q + src, slot + kWOffQ + i * 512);
            }
        }
        // [64][64] T and P: 8 pieces each, 8 / kWv per wave
#pragma unroll
        for (int j = 0; j < 8 / kWv; ++j) {
            const int i = (8 / kWv) * wave + j;
            const int row = 8 * i + (lane >> 3), u = (lane & 7) ^ swz(row);
            dma16(a.Tw + ch * kC * kC + row * kC + u * 8, slot + kWOffT + i * 512);
            dma16(a.Pw + ch * kC * kC + row * kC + u * 8, slot + kWOffP + i * 512);
        }
        if (wave == 0) dma16(a.Gw + ch * kGateRows * kC + lane * 4, slot + kWOffG);
    };

    const size_t sbase = ((size_t)seq * a.H + h) * kDK * DV;
    f32x4 S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) S[t] = f32x4{};
    if (a.S0) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[t][i] = a.S0[sbase + (size_t)relabel(t, 4 * g + i) * DV + j0w + c16];
    }
    bf16x8 Sb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) Sb[s] = to_bf16x8(S[2 * s], S[2 * s + 1]);

    // per-lane LDS offsets (elements, from a slot) of the fragment reads (as chunk_scan_kernel)
    int okf[2][2], otf[2][2], okt[2][2], ovf[2], oqf[2], opf[2];
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2) {
        const int r = relabel(a2, c16);
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            okf[a2][sp] = kWOffK + r * kDK + (((4 * sp + g) ^ swz(r)) << 3);
            otf[a2][sp] = kWOffT + r * kC + (((4 * sp + g) ^ swz(r)) << 3);
        }
    }
    const int jj = (lane & 15) >> 2, r4 = lane & 3;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int tok = 8 * g + jj + 4 * hf;
        constexpr int kOffKT = kKda ? kWOffV : kWOffK;   // K^T of the update (Kc^T)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) okt[hf][tp] = kOffKT + tok * kDK + (((4 * tp + r4) ^ swz(tok)) << 3);
        // V^T at the lane's relabelled tokens: 4 consecutive tokens of column j0w + c16
        ovf[hf] = kWOffV + tok * kDK + (((2 * wave + (r4 >> 1)) ^ swz(tok)) << 3) + 4 * (r4 & 1);
    }
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
        oqf[sp] = kWOffQ + c16 * kDK + (((4 * sp + g) ^ swz(c16)) << 3);
        opf[sp] = kWOffP + c16 * kC + (((4 * sp + g) ^ swz(c16)) << 3);
    }

    // output: a lane holds y at token 16 rt + c16, columns j0w + 4g .. j0w + 4g + 3
    const size_t ytok = (size_t)a.H * DV;
    const size_t ylane = (size_t)h * DV + j0w + 4 * g + (size_t)c16 * ytok;
    float gain[4];
    if constexpr (kGate) {
#pragma unroll
        for (int i = 0; i < 4; ++i) gain[i] = 1.0f + gd_.w[j0w + 4 * g + i];
    }
    f32x4 YT[4];      // chunk c - 1's y, held across the barrier until it is stored
    float zv[4][4];   // z at the same positions
    auto epilogue = [&](int cy) __attribute__((always_inline)) {
        const int ty = lo + cy * kC, ny = min(kC, hi - ty);
        const float* part = &ssq[kGate ? (cy & 1) : 0][0][0];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int tk = 16 * rt + c16;
            float tot = 0.f;
#pragma unroll
            for (int w = 0; w < kWideWaves; ++w) tot += part[w * kC + tk];
            const float inv = frsq(tot * (1.0f / DV) + gd_.eps);
            float ov[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = sigmoidf_(zv[rt][i]) * (gain[i] * (YT[rt][i] * inv));
            if (tk < ny) {
                const size_t off = ylane + (size_t)(ty + 16 * rt) * ytok;
                if constexpr (sizeof(To) == 2) {
                    u32x2 o2;
                    o2.x = pack_bf2(ov[0], ov[1]);
                    o2.y = pack_bf2(ov[2], ov[3]);
                    __builtin_nontemporal_store(o2, reinterpret_cast<u32x2*>(static_cast<To*>(gd_.o) + off));
                } else {
                    __builtin_nontemporal_store(f32x4{ov[0], ov[1], ov[2], ov[3]},
                                                reinterpret_cast<f32x4*>(static_cast<To*>(gd_.o) + off));
                }
            }
        }
    };
    auto store_y = [&](int cy) __attribute__((always_inline)) {
        const int ty = lo + cy * kC, ny = min(kC, hi - ty);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (16 * rt + c16 < ny) {
                Ty* yp = static_cast<Ty*>(a.y) + ylane + (size_t)(ty + 16 * rt) * ytok;
                if constexpr (sizeof(Ty) == 2) {
                    u32x2 o2;
                    o2.x = pack_bf2(YT[rt][0], YT[rt][1]);
                    o2.y = pack_bf2(YT[rt][2], YT[rt][3]);
                    __builtin_nontemporal_store(o2, reinterpret_cast<u32x2*>(yp));
                } else {
                    __builtin_nontemporal_store(YT[rt], reinterpret_cast<f32x4*>(yp));
                }
            }
        }
    };
    auto load_z = [&](int cz) __attribute__((always_inline)) {
        const int tz = lo + cz * kC, nz = min(kC, hi - tz);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const Tz* zp = static_cast<const Tz*>(gd_.z) + (size_t)h * DV + j0w + 4 * g +
                           (size_t)(tz + min(16 * rt + c16, nz - 1)) * ytok;
            if constexpr (sizeof(Tz) == 2) {
                const u32x2 zz = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(zp));
                zv[rt][0] = __uint_as_float(zz.x << 16);
                zv[rt][1] = __uint_as_float(zz.x & 0xffff0000u);
                zv[rt][2] = __uint_as_float(zz.y << 16);
                zv[rt][3] = __uint_as_float(zz.y & 0xffff0000u);
            } else {
                const f32x4 zz = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(zp));
#pragma unroll
                for (int i = 0; i < 4; ++i) zv[rt][i] = zz[i];
            }
        }
    };

    // per-channel decay: V at the lane's relabelled tokens, column j0w + c16, from global
    // memory one chunk ahead (ragged rows repeat the last row; their beta is zero)
    uint16_t vcur[16], vnext[16];
    auto fetch_v = [&](int ck) __attribute__((always_inline)) {
        const int t0 = lo + ck * kC, n = min(kC, hi - t0);
        const uint16_t* vb = a.v + (size_t)h * DV + j0w + c16;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vnext[4 * rt + i] = vb[(size_t)(t0 + min(relabel(rt, 4 * g + i), n - 1)) * a.H * DV];
    };
    if (nchunks > 0) load_chunk(0, ring0);
    if constexpr (kKda) {
        if (nchunks > 0) fetch_v(0);
    }
    GDN_WAIT_VMCNT(0);
    lds_barrier();
    // Chunk c's results leave at the start of step c + 1, before that step's loads: the wait
    // for the loads at the end of a step (the vector-memory counter counts stores too, in issue
    // order) then never waits for stores issued in the same step.
    auto step = [&](int c, const uint16_t* slot, uint16_t* next) __attribute__((always_inline)) {
        if (c >= 1) {
            if constexpr (kGate) {
                epilogue(c - 1);
                if (a.y) store_y(c - 1);
            } else {
                store_y(c - 1);
            }
        }
        if (c + 1 < nchunks) load_chunk(c + 1, next);
        if constexpr (kKda) {
#pragma unroll
            for (int i = 0; i < 16; ++i) vcur[i] = vnext[i];
            if (c + 1 < nchunks) fetch_v(c + 1);
        }
        if constexpr (kGate) load_z(c);
        const float* sG = reinterpret_cast<const float*>(slot + kWOffG);   // beta | gamma | gamma_C/gamma
        auto kfrag = [&](int rt, int s) {
            return frag(slot + okf[rt & 1][s & 1] + (rt >> 1) * 32 * kDK + (s >> 1) * 64);
        };
        auto tfrag = [&](int rt, int s) { return frag(slot + otf[rt & 1][s] + (rt >> 1) * 32 * kC); };
        auto ktr = [&](int t, int s, int hf) {
            return lds_tr16(slot + okt[hf][(t >> 1) & 1] + s * 32 * kDK + (t >> 2) * 64 + 4 * (t & 1));
        };
        auto grow = [&](int which, int rt) {
            return *reinterpret_cast<const f32x4*>(sG + which * kC + 8 * g + 32 * (rt >> 1) + 4 * (rt & 1));
        };
        const float gC = kKda ? 1.f : sG[kC + kC - 1];

        // ---- K S and Q S (both against the state at the chunk start)
        f32x4 KS[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) KS[rt] = f32x4{};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 kf[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) kf[rt] = kfrag(rt, s);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) KS[rt] = mfma16(kf[rt], Sb[s], KS[rt]);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            YT[rt] = f32x4{};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                YT[rt] = mfma16(Sb[s], frag(slot + oqf[s & 1] + rt * 16 * kDK + (s >> 1) * 64), YT[rt]);
        }
        GDN_SCHED_FENCE();
        // ---- R = beta (V - gamma KS), split into bf16 hi + lo
        f32x4 R[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 bet = grow(0, rt);
            if constexpr (kKda) {   // R = beta (V - Kg S)
#pragma unroll
                for (int i = 0; i < 4; ++i) R[rt][i] = bet[i] * (bf2f(vcur[4 * rt + i]) - KS[rt][i]);
            } else {
                const f32x4 gam = grow(1, rt);
                const s16x4 vv = lds_tr16(slot + ovf[rt & 1] + (rt >> 1) * 32 * kDK);
#pragma unroll
                for (int i = 0; i < 4; ++i) R[rt][i] = bet[i] * (bf2f(uint16_t(vv[i])) - gam[i] * KS[rt][i]);
            }
        }
        bf16x8 Rh[2], Rl[2];
        split8(R[0], R[1], Rh[0], Rl[0]);
        split8(R[2], R[3], Rh[1], Rl[1]);
        GDN_SCHED_FENCE();
        // ---- U = T R (T unit lower triangular: token rows < 32 need step 0 only)
        f32x4 U[4];
        {
            bf16x8 tf[4][2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    if (s2 <= (rt >> 1)) tf[rt][s2] = tfrag(rt, s2);
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
        }
        GDN_SCHED_FENCE();
        // ---- Y^T = gamma (S^T Q^T) + U^T P^T, the order of the output wave above
        {
            bf16x8 Uh[2], Ul[2];
            split8(U[0], U[1], Uh[0], Ul[0]);
            split8(U[2], U[3], Uh[1], Ul[1]);
            if constexpr (!kKda) {   // gamma (S^T Q^T); Qg carries the decay already
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) YT[rt] *= sG[kC + 16 * rt + c16];
            }
            bf16x8 pf[4][2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    if (s2 <= (rt >> 1)) pf[rt][s2] = frag(slot + opf[s2] + rt * 16 * kC);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) YT[rt] = mfma16(Uh[0], pf[rt][0], YT[rt]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) YT[rt] = mfma16(Ul[0], pf[rt][0], YT[rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt) YT[rt] = mfma16(Uh[1], pf[rt][1], YT[rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt) YT[rt] = mfma16(Ul[1], pf[rt][1], YT[rt]);
        }
        GDN_SCHED_FENCE();
        // ---- W = diag(gamma_C / gamma) U, split; S = gamma_C S + K^T W
        bf16x8 Wh[2], Wl[2];
        if constexpr (!kKda) {   // Kc carries the per-channel decay to the chunk end
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) U[rt] *= grow(2, rt);
        }
        split8(U[0], U[1], Wh[0], Wl[0]);
        split8(U[2], U[3], Wh[1], Wl[1]);
        // four tiles at a time, taking turns (no product waits for the one just before it);
        // each tile adds its products in the order s2 = 0 hi, lo, s2 = 1 hi, lo
        auto upd4 = [&](int t0) __attribute__((always_inline)) {
            bf16x8 ktf[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if constexpr (kKda)   // e^{Gc[C]} at the tile's d_k rows relabel(t, 4g + i)
                    S[t0 + t] *= *reinterpret_cast<const f32x4*>(sG + kC + 32 * ((t0 + t) >> 1) + 8 * g +
                                                                 4 * (t & 1));
                else
                    S[t0 + t] *= gC;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const u32x2 p0 = __builtin_bit_cast(u32x2, ktr(t0 + t, s2, 0));
                    const u32x2 p1 = __builtin_bit_cast(u32x2, ktr(t0 + t, s2, 1));
                    const u32x4 pk = {p0.x, p0.y, p1.x, p1.y};
                    ktf[t][s2] = __builtin_bit_cast(bf16x8, pk);
                }
            }
            if constexpr (kGate) {
                // tile by tile: with the epilogue's registers live this order measured 2%
                // faster (the same additions per tile, so the same results)
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        S[t0 + t] = mfma16(ktf[t][s2], Wh[s2], S[t0 + t]);
                        S[t0 + t] = mfma16(ktf[t][s2], Wl[s2], S[t0 + t]);
                    }
            } else {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) S[t0 + t] = mfma16(ktf[t][s2], Wh[s2], S[t0 + t]);
#pragma unroll
                    for (int t = 0; t < 4; ++t) S[t0 + t] = mfma16(ktf[t][s2], Wl[s2], S[t0 + t]);
                }
            }
            Sb[t0 >> 1] = to_bf16x8(S[t0], S[t0 + 1]);
            Sb[(t0 >> 1) + 1] = to_bf16x8(S[t0 + 2], S[t0 + 3]);
        };
        upd4(0);
        upd4(4);
        GDN_SCHED_FENCE();
        if constexpr (kGate) {
            // this wave's sums of y^2 over its 16 columns, per token, for the epilogue
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                float ss = YT[rt][0] * YT[rt][0] + YT[rt][1] * YT[rt][1] + YT[rt][2] * YT[rt][2] +
                           YT[rt][3] * YT[rt][3];
                ss = sum_across<16>(ss);
                if (g == 0) ssq[c & 1][wave][16 * rt + c16] = ss;
            }
        }
        GDN_WAIT_VMCNT(0);
        lds_barrier();   // the next slot is in, and this slot and the sums may be reused
    };
    for (int c = 0; c < nchunks; c += 2) {
        step(c, ring0, ring1);
        if (c + 1 < nchunks) step(c + 1, ring1, ring0);
    }
    if (nchunks > 0) {
        if constexpr (kGate) {
            epilogue(nchunks - 1);
            if (a.y) store_y(nchunks - 1);
        } else {
            store_y(nchunks - 1);
        }
    }
    if (a.ST) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.ST[sbase + (size_t)relabel(t, 4 * g + i) * DV + j0w + c16] = S[t][i];
    }
}

}  // namespace

size_t chunk_bf16_workspace(int ntok, int num_seqs, int H) {
    return ws_layout(ntok, num_seqs, H).total;
}

// The full-row scan needs a (sequence, head) per CU to pay: below that the sliced scan's four
// workgroups per pair spread one pair's columns over four CUs, which is faster when CUs are
// left over. Without the output gate the sliced scan (which forms P itself, so its prep writes
// no P) is as fast or faster at every pair count measured: 256 pairs (B=8 H=32 T=4096) 0.62 vs
// 0.62 ms per prefill, 1,024 pairs (B=16 H=64 T=4096) 2.15 vs 2.33 ms, 64 packed sequences of
// log-uniform lengths at H=16 2.69 vs 3.31 ms. With the gate in its epilogue the full-row scan
// saves the output-gate kernel's pass over y: 0.99 vs 1.08 ms (256 uniform pairs, gate
// included), 3.88 vs 4.01 ms (1,024), while the packed sequences above still favour the sliced
// scan and the separate gate (5.08 vs 5.34 ms).
constexpr int kWideMinPairs = 256;
static bool use_wide_scan(int pairs, int dv, bool gated, bool packed) {
    return gated && !packed && dv == 128 && pairs >= kWideMinPairs;
}

template <typename Ty, bool kGate, typename Tz, typename To, bool kKda = false, int kWv = 8>
static void launch_wide(const DevArgs& a, const GateDev& gd, int pairs, hipStream_t s) {
    const int nsl = kWideWaves / kWv;
    hipLaunchKernelGGL((chunk_scan_wide_kernel<Ty, kGate, Tz, To, kKda, kWv>),
                       dim3((pairs + 7) / 8 * 8 * nsl), dim3(kWv * kWave), 0, s, a, gd);
}

static DevArgs dev_args(const ChunkArgs& c, const Layout& L) {
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
    a.Xw = nullptr;
    a.gk = nullptr;
    a.Sst = nullptr;
    a.num_seqs = c.num_seqs; a.ntok = c.ntok; a.H = c.H; a.dv = c.dv;
    a.L = c.cu ? 0 : c.ntok / c.num_seqs;
    a.y_bf16 = c.y_bf16;
    return a;
}

hipError_t launch_chunk_bf16(const ChunkArgs& c, hipStream_t s, const GateArgs* gate) {
    const Layout L = ws_layout(c.ntok, c.num_seqs, c.H);
    DevArgs a = dev_args(c, L);
    if (c.cu) hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kThreads), 0, s, a);
    const int nchunks = c.cu ? L.max_chunks : c.num_seqs * ((a.L + kC - 1) / kC);
    const int pairs = c.num_seqs * c.H;
    const bool wide = use_wide_scan(pairs, c.dv, gate != nullptr, c.cu != nullptr);
    // the sliced scan forms P itself (kPS): its prep writes T and the gate rows only
    if (nchunks > 0) {
        if (wide)
            hipLaunchKernelGGL(chunk_prep_kernel<true>, dim3(nchunks, c.H), dim3(kPrepThreads), 0, s, a);
        else
            hipLaunchKernelGGL(chunk_prep_kernel<false>, dim3(nchunks, c.H), dim3(kPrepThreads), 0, s, a);
    }
    if (wide) {   // only with the gate: it runs in the scan's epilogue
        GateDev gd{};
        gd.z = gate->z; gd.w = gate->w; gd.o = gate->o; gd.eps = gate->eps;
        a.y = gate->y_export;   // nullable: y is not stored unless exported
        const int key = (gate->z_bf16 << 1) | gate->o_bf16;
        switch (key) {
            case 0: launch_wide<uint16_t, true, float, float>(a, gd, pairs, s); break;
            case 1: launch_wide<uint16_t, true, float, uint16_t>(a, gd, pairs, s); break;
            case 2: launch_wide<uint16_t, true, uint16_t, float>(a, gd, pairs, s); break;
            default: launch_wide<uint16_t, true, uint16_t, uint16_t>(a, gd, pairs, s); break;
        }
        return hipGetLastError();
    }
    const int nsl = c.dv / kSl;
    const int blocks = (pairs + 7) / 8 * 8 * nsl;
    // Tiles two chunks ahead pay while the chain's one-chunk-ahead T reads hit the Infinity
    // Cache (256 MB): B=4 H=16 T=4096 (34 MB of T) 104 vs 108 us per scan; B=1 H=32 T=65536
    // (268 MB of T) 1626 vs 1584 us. Larger calls keep the one-chunk-ahead scan.
    const bool two_ahead = (size_t)nchunks * c.H * kC * kC * sizeof(uint16_t) <= kFwdMaxTBytes;
    if (two_ahead) {
        if (c.y_bf16)
            hipLaunchKernelGGL((chunk_scan_fwd_kernel<uint16_t>), dim3(blocks), dim3(2 * kScanThreads), 0, s, a);
        else
            hipLaunchKernelGGL((chunk_scan_fwd_kernel<float>), dim3(blocks), dim3(2 * kScanThreads), 0, s, a);
    } else if (c.y_bf16) {
        hipLaunchKernelGGL((chunk_scan_kernel<uint16_t, false, true>), dim3(blocks), dim3(2 * kScanThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL((chunk_scan_kernel<float, false, true>), dim3(blocks), dim3(2 * kScanThreads), 0, s, a);
    }
    if (gate) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_output_gate(c.y, c.y_bf16, gate->z, gate->z_bf16, gate->w, c.ntok, c.H, c.dv,
                                  gate->eps, gate->o, gate->o_bf16, s);
    }
    return hipGetLastError();
}

ChunkTiles chunk_bf16_tiles(void* workspace, int ntok, int num_seqs, int H) {
    const Layout L = ws_layout(ntok, num_seqs, H);
    char* ws = static_cast<char*>(workspace);
    ChunkTiles t;
    t.chunk_start = reinterpret_cast<int32_t*>(ws + L.cs);
    t.order = reinterpret_cast<int32_t*>(ws + L.ord);
    t.T = reinterpret_cast<uint16_t*>(ws + L.T);
    t.P = reinterpret_cast<uint16_t*>(ws + L.P);
    t.Gw = reinterpret_cast<float*>(ws + L.Gt);
    t.max_chunks = L.max_chunks;
    return t;
}

hipError_t launch_chunk_bf16_states(const ChunkArgs& c, float* Sst, hipStream_t s) {
    const Layout L = ws_layout(c.ntok, c.num_seqs, c.H);
    DevArgs a = dev_args(c, L);
    a.Sst = Sst;
    a.y = nullptr;
    a.ST = nullptr;
    if (c.cu) hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kThreads), 0, s, a);
    const int nchunks = c.cu ? L.max_chunks : c.num_seqs * ((a.L + kC - 1) / kC);
    if (nchunks > 0)
        hipLaunchKernelGGL(chunk_prep_kernel<true>, dim3(nchunks, c.H), dim3(kPrepThreads), 0, s, a);
    const int pairs = c.num_seqs * c.H;
    const int blocks = (pairs + 7) / 8 * 8 * (c.dv / kSl);
    hipLaunchKernelGGL((chunk_scan_kernel<uint16_t, true>), dim3(blocks), dim3(kScanThreads), 0, s, a);
    return hipGetLastError();
}

// the per-channel-decay path with log-decays >= -5 (bf16 q, k, v; dk = dv = 128): the
// chunked prefill's tiles plus the Kg, Kc, Qg operand tiles
size_t kda_bf16_workspace(int ntok, int num_seqs, int H) {
    const Layout L = ws_layout(ntok, num_seqs, H);
    return L.total + align256((size_t)L.max_chunks * H * 3 * kC * kDK * sizeof(uint16_t));
}

hipError_t launch_kda_bf16(const ChunkArgs& c, const float* gk, hipStream_t s) {
    const Layout L = ws_layout(c.ntok, c.num_seqs, c.H);
    DevArgs a = dev_args(c, L);
    a.Xw = reinterpret_cast<uint16_t*>(static_cast<char*>(c.workspace) + L.total);
    a.gk = gk;
    if (c.cu) hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kThreads), 0, s, a);
    const int nchunks = c.cu ? L.max_chunks : c.num_seqs * ((a.L + kC - 1) / kC);
    if (nchunks > 0)
        hipLaunchKernelGGL(kda_prep_bf16_kernel, dim3(nchunks, c.H), dim3(kKdaPrepThreads), 0, s, a);
    const int pairs = c.num_seqs * c.H;
    const GateDev gd{};
    // enough workgroups to cover the chip: the full row when the pairs alone do, else a pair
    // split over 2 or 4 workgroups
    auto go = [&](auto ty) {
        using Ty = decltype(ty);
        if (pairs >= kWideMinPairs) launch_wide<Ty, false, uint16_t, uint16_t, true, 8>(a, gd, pairs, s);
        else if (2 * pairs >= kWideMinPairs) launch_wide<Ty, false, uint16_t, uint16_t, true, 4>(a, gd, pairs, s);
        else launch_wide<Ty, false, uint16_t, uint16_t, true, 2>(a, gd, pairs, s);
    };
    if (c.y_bf16) go(uint16_t{});
    else go(float{});
    return hipGetLastError();
}

}  // namespace gdn
