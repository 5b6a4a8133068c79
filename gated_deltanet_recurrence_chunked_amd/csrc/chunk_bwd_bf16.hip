// Backward of the chunkwise gated delta rule on the bf16 matrix cores (bf16 q, k, v and dy,
// d_k = d_v = 128, fp32 gradients). Reading notes of "On the Design of Qwen3.8-Next
// Architecture", section 2.1.1, eqs. (1)-(5); chunk length C = 64.
//
// Per chunk (G the running sum of g inside the chunk, gamma = e^G, w_r = e^{G_C - G_r}, T and P
// as in the forward):
//   KS = K S,  R = beta o (V - gamma o KS),  U = T R,  Y = gamma o (Q S) + P U,
//   S' = gamma_C S + K^T (w o U)
// and with dS' the gradient of the state leaving the chunk, its adjoints are
//   dW = K dS',  dU = w o dW + P^T dY,  dR = T^T dU,  dV = beta o dR,
//   dS = gamma_C dS' + Q^T (gamma o dY) - K^T ((beta gamma) o dR)
//   dA = -(dR U^T) (strictly lower),  dP = dY U^T (lower),
//   dQ = gamma o (dY S^T) + (dP o E) K,
//   dK = w o (U dS'^T) - (beta gamma) o (dR S^T) + (dKK + dKK^T) K + (dP o E)^T Q
// with E[r,i] = e^{G_r - G_i} and dKK = beta o dA o E, plus the per-token terms of dbeta and dg.
//
// Three sweeps instead of per-slice shares of the terms that sum over d_v:
//   1. the forward scan in its states-only form (chunk_bf16.hip) stores the fp32 state S
//      entering every chunk;
//   2. bwd_chain_kernel walks the chunks of each (sequence, head, 32-column slice) backwards
//      carrying dS in registers (the forward scan's structure with the adjoint products) and
//      stores the fp32 dS' of every chunk, and dS0;
//   3. bwd_chunk_kernel, one workgroup per (chunk, head), recomputes the chunk's U and dR from
//      S and dS' and forms every gradient of the chunk with all d_v columns at hand.
// Rounding (chosen with a bf16 emulation of these sweeps against the fp64 gradients): the
// products whose operands are fp32 take them as hi + lo bf16 pairs (R, dU, E = -(beta gamma) o
// dR and gamma o dY in the chain; in the per-chunk kernel S, dS', U, the coefficient matrices
// dP o E and dKK + dKK^T, and dR in dR U^T), except dR in dR S^T, single bf16. The chain takes
// dS single in K dS, as the forward takes S. Short sequences decide it: a one-token sequence's
// dg and dbeta are single sums that cancel, and single-bf16 S or dS' there costs up to 8% of
// them.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {

namespace {

constexpr int kC = 64;     // chunk length
constexpr int kD = 128;    // d_k = d_v
constexpr int kSl = 32;    // d_v columns per chain workgroup

struct BArgs {
    const uint16_t *q, *k, *v, *dy;
    const float *g, *beta, *dST;
    const int32_t* cu;                      // NULL: equal lengths L
    const int32_t *chunk_start, *order;     // varlen: first chunk per sequence, longest first
    const uint16_t *T, *P;                  // [chunk-head][64][64] bf16
    const float* Gw;                        // [chunk-head][3][64]: beta, gamma, gamma_C / gamma
    const float* Sst;                       // [chunk-head][d_v][d_k] fp32: S entering the chunk
    float* dSp;                             // [chunk-head][d_k][d_v] fp32: dS leaving the chunk
    float *dq, *dk, *dv, *dg, *dbeta, *dS0;
    int num_seqs, ntok, H, L;
};

__device__ __forceinline__ void seq_range(const BArgs& a, int seq, int& lo, int& hi, int& cbase) {
    if (a.cu) {
        lo = a.cu[seq];
        hi = a.cu[seq + 1];
        cbase = a.chunk_start[seq];
    } else {
        lo = seq * a.L;
        hi = lo + a.L;
        cbase = seq * ((a.L + kC - 1) / kC);
    }
}

// two transposing reads (rows r .. r+3 and r+4 .. r+7 of a column) -> one operand fragment
__device__ __forceinline__ bf16x8 tr_pair(const uint16_t* p0, const uint16_t* p1) {
    const u32x2 a = __builtin_bit_cast(u32x2, lds_tr16(p0));
    const u32x2 b = __builtin_bit_cast(u32x2, lds_tr16(p1));
    const u32x4 v = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------------------ reverse chain
// One 4-wave workgroup per (sequence, head, 32-column slice of d_v), the slices of a pair 8
// blocks apart (same XCD), sequences longest first:
//   waves 0-1 (chain) carry dS for 16 columns each, chunk by chunk from the last:
//     dW = K dS -> dU = w o dW + X -> dR = T^T dU -> E = -(beta gamma) o dR ->
//     dS = gamma_C dS + Z + K^T E,
//     with X = P^T dY and Z = Q^T (gamma o dY), which do not depend on dS;
//   wave 2 (helper) forms X and Z of the chunk the chain takes next, for both 16-column slices,
//     in the chain waves' accumulator layout, and hands them over through LDS;
//   wave 3 (loader) streams the chain's tiles (K, T, gate rows) into a two-slot ring one step
//     ahead and the helper's (Q, P, the dY slice, gate rows) one step ahead of the helper.
// The state sits in registers as in the forward scan: tile t of d_k holds rows relabel(t, .),
// so two accumulator tiles are one operand fragment of the next product. T^T and P^T (A
// operands with relabelled rows) and Q^T, K^T come from the row-major tiles through the
// transposing LDS read. Every chain step first stores the fp32 dS it starts from: the gradient
// of the state leaving that chunk, which the per-chunk kernel reads.
constexpr int kChainThreads = 256;
constexpr int kOffK = 0;                     // chain ring slot, in bf16 elements
constexpr int kOffT = kOffK + kC * kD;
constexpr int kOffG = kOffT + kC * kC;       // kGateRows x 64 floats
constexpr int kSlot = kOffG + 512;
constexpr int kHOffQ = 0;                    // helper slot
constexpr int kHOffP = kHOffQ + kC * kD;
constexpr int kHOffY = kHOffP + kC * kC;     // dY slice [64][32], rows unswizzled
constexpr int kHOffG = kHOffY + kC * kSl;
constexpr int kHSlot = kHOffG + 512;
constexpr int kXZ = 12 * kWave;              // per chain wave: X tiles 0-3, Z tiles 4-11

__global__ void __launch_bounds__(kChainThreads) bwd_chain_kernel(BArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ring[2 * kSlot];
    __shared__ __attribute__((aligned(16))) uint16_t hbuf[2 * kHSlot];
    __shared__ __attribute__((aligned(16))) u32x4 xz[2][2][kXZ];

    constexpr int nsl = kD / kSl;
    const int b = blockIdx.x;
    const int group = b / (8 * nsl), within = b % (8 * nsl);
    const int slice = within >> 3;
    const int pair = group * 8 + (within & 7);
    if (pair >= a.num_seqs * a.H) return;
    const int rank = pair / a.H, h = pair % a.H;
    const int seq = a.order ? a.order[rank] : rank;
    int lo, hi, cbase;
    seq_range(a, seq, lo, hi, cbase);
    const int nch = (hi - lo + kC - 1) / kC;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j0 = slice * kSl;
    const int c16 = lane & 15, g = lane >> 4;
    const int jj = (lane & 15) >> 2, r4 = lane & 3;
    // step m = 0 .. nch-1 takes chunk nch-1-m; steps -2 and -1 fill the pipeline

    if (wave == 3) {
        // ================= loader
        // step m: ring slot (m+1)&1 <- the chain's tiles of step m+1 (the chain used that slot
        // in step m-1); helper slot m&1 <- the helper's tiles of step m+2 (the helper used it
        // in step m-1 for step m)
        int offk[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 4 * i + (lane >> 4), u = (lane & 15) ^ swz(row);
            offk[i] = (row * a.H + h) * kD + u * 8;
        }
        auto rows128 = [&](const uint16_t* x, int t0, int n, uint16_t* dst) __attribute__((always_inline)) {
            const uint16_t* xb = x + (size_t)t0 * a.H * kD;
            if (n == kC) {
#pragma unroll
                for (int i = 0; i < 16; ++i) dma16(xb + offk[i], dst + i * 512);
            } else {   // the ragged chunk: rows >= n repeat row n - 1
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 4 * i + (lane >> 4), u = (lane & 15) ^ swz(row);
                    dma16(xb + (min(row, n - 1) * a.H + h) * kD + u * 8, dst + i * 512);
                }
            }
        };
        auto tile64 = [&](const uint16_t* src, uint16_t* dst) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = 8 * i + (lane >> 3), u = (lane & 7) ^ swz(row);
                dma16(src + row * kC + u * 8, dst + i * 512);
            }
        };
        auto chain_tiles = [&](int m) __attribute__((always_inline)) {
            const int c = nch - 1 - m, t0 = lo + c * kC, n = min(kC, hi - t0);
            const size_t ch = (size_t)(cbase + c) * a.H + h;
            uint16_t* slot = ring + (m & 1) * kSlot;
            rows128(a.k, t0, n, slot + kOffK);
            tile64(a.T + ch * kC * kC, slot + kOffT);
            dma16(a.Gw + ch * kGateRows * kC + lane * 4, slot + kOffG);
        };
        auto helper_tiles = [&](int m) __attribute__((always_inline)) {
            const int c = nch - 1 - m, t0 = lo + c * kC, n = min(kC, hi - t0);
            const size_t ch = (size_t)(cbase + c) * a.H + h;
            uint16_t* slot = hbuf + (m & 1) * kHSlot;
            rows128(a.q, t0, n, slot + kHOffQ);
            tile64(a.P + ch * kC * kC, slot + kHOffP);
            const uint16_t* yb = a.dy + (size_t)t0 * a.H * kD;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * i + (lane >> 2);
                dma16(yb + (min(row, n - 1) * a.H + h) * kD + j0 + (lane & 3) * 8, slot + kHOffY + i * 512);
            }
            dma16(a.Gw + ch * kGateRows * kC + lane * 4, slot + kHOffG);
        };
        for (int m = -2; m < nch; ++m) {
            if (m == -2) {
                if (nch > 0) helper_tiles(0);
            } else {
                if (m + 1 < nch) chain_tiles(m + 1);
                if (m + 2 < nch) helper_tiles(m + 2);
            }
            GDN_WAIT_VMCNT(0);
            dma_barrier();
        }
        return;
    }

    if (wave == 2) {
        // ================= helper: X = P^T dY (token tiles rt) and Z = Q^T (gamma o dY) (d_k
        // tiles t) of step mm's chunk, both slices, rows relabelled as the chain's accumulators
        int oq[2][2], op[2][2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int tok = 8 * g + jj + 4 * hf;
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                oq[hf][tp] = kHOffQ + tok * kD + (((4 * tp + r4) ^ swz(tok)) << 3);
                op[hf][tp] = kHOffP + tok * kC + (((4 * tp + r4) ^ swz(tok)) << 3);
            }
        }
        auto helper = [&](int mm) __attribute__((always_inline)) {
            const int c = nch - 1 - mm, t0 = lo + c * kC, n = min(kC, hi - t0);
            const uint16_t* slot = hbuf + (mm & 1) * kHSlot;
            const float* sG = reinterpret_cast<const float*>(slot + kHOffG);
            // Q^T[relabel(t, c16)][32s + 8g ..] and P^T[relabel(rt, c16)][32s + 8g ..] (P^T is
            // upper triangular: token tiles 2-3 need step 1 only)
            bf16x8 qt[8][2], pt[4][2];
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int o = s * 32 * kD + (t >> 2) * 64 + 4 * (t & 1);
                    qt[t][s] = tr_pair(slot + oq[0][(t >> 1) & 1] + o, slot + oq[1][(t >> 1) & 1] + o);
                }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (s >= (rt >> 1)) {
                        const int o = s * 32 * kC + 4 * (rt & 1);
                        pt[rt][s] = tr_pair(slot + op[0][rt >> 1] + o, slot + op[1][rt >> 1] + o);
                    }
            u32x4* const dst = &xz[mm & 1][0][0];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                // dY[32s + 8g + e][16 sl + c16] (zero past n) and its gamma-scaled hi + lo split
                bf16x8 yb[2], gh[2], gl[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint16_t* p = slot + kHOffY + (32 * s + 8 * g + jj) * kSl + 16 * sl + 4 * r4;
                    u32x4 raw = __builtin_bit_cast(u32x4, tr_pair(p, p + 4 * kSl));
                    const int tb = 32 * s + 8 * g;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t keep = (tb + 2 * e < n ? 0x0000ffffu : 0u) |
                                              (tb + 2 * e + 1 < n ? 0xffff0000u : 0u);
                        raw[e] &= keep;
                    }
                    yb[s] = __builtin_bit_cast(bf16x8, raw);
                    const f32x4 g0 = *reinterpret_cast<const f32x4*>(sG + kC + tb);
                    const f32x4 g1 = *reinterpret_cast<const f32x4*>(sG + kC + tb + 4);
                    f32x4 x0, x1;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        x0[2 * e] = __uint_as_float(raw[e] << 16) * g0[2 * e];
                        x0[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u) * g0[2 * e + 1];
                        x1[2 * e] = __uint_as_float(raw[2 + e] << 16) * g1[2 * e];
                        x1[2 * e + 1] = __uint_as_float(raw[2 + e] & 0xffff0000u) * g1[2 * e + 1];
                    }
                    split8(x0, x1, gh[s], gl[s]);
                }
                // products on one accumulator are kept apart by products on the others; each
                // accumulator adds its terms in the order step 0 (hi, lo), step 1 (hi, lo)
                f32x4 X[4], Z[8];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) X[rt] = f32x4{};
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) X[rt] = mfma16(pt[rt][0], yb[0], X[rt]);
#pragma unroll
                for (int rt = 3; rt >= 0; --rt) X[rt] = mfma16(pt[rt][1], yb[1], X[rt]);
#pragma unroll
                for (int t = 0; t < 8; ++t) Z[t] = f32x4{};
#pragma unroll
                for (int s = 0; s < 2; ++s) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) Z[t] = mfma16(qt[t][s], gh[s], Z[t]);
#pragma unroll
                    for (int t = 0; t < 8; ++t) Z[t] = mfma16(qt[t][s], gl[s], Z[t]);
                }
                u32x4* xo = dst + sl * kXZ;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) xo[rt * kWave + lane] = __builtin_bit_cast(u32x4, X[rt]);
#pragma unroll
                for (int t = 0; t < 8; ++t) xo[(4 + t) * kWave + lane] = __builtin_bit_cast(u32x4, Z[t]);
            }
        };
        for (int m = -2; m < nch; ++m) {
            if (m >= -1 && m + 1 < nch) helper(m + 1);
            lds_barrier();
        }
        return;
    }

    // ================= chain waves: d_v columns j0w .. j0w + 15
    const int j0w = j0 + 16 * wave;
    const size_t sbase = ((size_t)seq * a.H + h) * kD * kD;
    f32x4 D[8];   // dS: tile t holds d_k rows relabel(t, 4g + i) of column j0w + c16
#pragma unroll
    for (int t = 0; t < 8; ++t) D[t] = f32x4{};
    if (a.dST) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) D[t][i] = a.dST[sbase + (size_t)relabel(t, 4 * g + i) * kD + j0w + c16];
    }
    bf16x8 Db[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) Db[s] = to_bf16x8(D[2 * s], D[2 * s + 1]);

    int okf[2][2], okt[2][2], ott[2][2];
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2) {
        const int r = relabel(a2, c16);
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) okf[a2][sp] = kOffK + r * kD + (((4 * sp + g) ^ swz(r)) << 3);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int tok = 8 * g + jj + 4 * hf;
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            okt[hf][tp] = kOffK + tok * kD + (((4 * tp + r4) ^ swz(tok)) << 3);
            ott[hf][tp] = kOffT + tok * kC + (((4 * tp + r4) ^ swz(tok)) << 3);
        }
    }
    float* const dsp_lane = a.dSp + j0w + c16;

    for (int m = -2; m < nch; ++m) {
        if (m < 0) {
            lds_barrier();
            continue;
        }
        const int c = nch - 1 - m;
        const size_t ch = (size_t)(cbase + c) * a.H + h;
        const uint16_t* slot = ring + (m & 1) * kSlot;
        const float* sG = reinterpret_cast<const float*>(slot + kOffG);   // beta | gamma | w
        const u32x4* xzb = xz[m & 1][wave];
        {   // the gradient of the state leaving this chunk
            float* dp = dsp_lane + ch * kD * kD;
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) dp[(size_t)relabel(t, 4 * g + i) * kD] = D[t][i];
        }
        auto kfrag = [&](int rt, int s) {   // K[relabel(rt, c16)][32s + 8g ..]
            return frag(slot + okf[rt & 1][s & 1] + (rt >> 1) * 32 * kD + (s >> 1) * 64);
        };
        auto ktr = [&](int t, int s) {      // K^T[relabel(t, c16)][32s + 8g ..]
            const int o = s * 32 * kD + (t >> 2) * 64 + 4 * (t & 1);
            return tr_pair(slot + okt[0][(t >> 1) & 1] + o, slot + okt[1][(t >> 1) & 1] + o);
        };
        auto ttr = [&](int rt, int s) {     // T^T[relabel(rt, c16)][32s + 8g ..]
            const int o = s * 32 * kC + 4 * (rt & 1);
            return tr_pair(slot + ott[0][rt >> 1] + o, slot + ott[1][rt >> 1] + o);
        };
        auto grow = [&](int which, int rt) {   // gate row at the lane's 4 relabelled tokens
            return *reinterpret_cast<const f32x4*>(sG + which * kC + 8 * g + 32 * (rt >> 1) + 4 * (rt & 1));
        };

        // ---- dW = K dS
        bf16x8 kf[4][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) kf[s][rt] = kfrag(rt, s);
        f32x4 dW[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dW[rt] = f32x4{};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) dW[rt] = mfma16(kf[s][rt], Db[s], dW[rt]);
        // ---- dU = w o dW + X and its split; T^T fragments (T^T upper triangular)
        bf16x8 tt[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                if (s >= (rt >> 1)) tt[rt][s] = ttr(rt, s);
        f32x4 dU[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 X = __builtin_bit_cast(f32x4, xzb[rt * kWave + lane]);
            dU[rt] = grow(2, rt) * dW[rt] + X;
        }
        bf16x8 dUh[2], dUl[2];
        split8(dU[0], dU[1], dUh[0], dUl[0]);
        split8(dU[2], dU[3], dUh[1], dUl[1]);
        // ---- dR = T^T dU
        // tiles 0-1 take steps 0 and 1, tiles 2-3 step 1; per tile: step 0 hi, lo, step 1 hi, lo,
        // with the tiles taking turns
        f32x4 dR[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dR[rt] = f32x4{};
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) dR[rt] = mfma16(tt[rt][0], dUh[0], dR[rt]);
#pragma unroll
        for (int rt = 2; rt < 4; ++rt) dR[rt] = mfma16(tt[rt][1], dUh[1], dR[rt]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) dR[rt] = mfma16(tt[rt][0], dUl[0], dR[rt]);
#pragma unroll
        for (int rt = 2; rt < 4; ++rt) dR[rt] = mfma16(tt[rt][1], dUl[1], dR[rt]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) dR[rt] = mfma16(tt[rt][1], dUh[1], dR[rt]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) dR[rt] = mfma16(tt[rt][1], dUl[1], dR[rt]);
        // ---- E = -(beta gamma) o dR and its split; K^T fragments
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dR[rt] *= -(grow(0, rt) * grow(1, rt));
        bf16x8 Eh[2], El[2];
        split8(dR[0], dR[1], Eh[0], El[0]);
        split8(dR[2], dR[3], Eh[1], El[1]);
        // ---- dS = gamma_C dS + Z + K^T E
        const float gC = sG[kC + kC - 1];
        // four tiles at a time, taking turns; per tile: step 0 hi, lo, step 1 hi, lo
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += 4) {
            bf16x8 kt[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 Z = __builtin_bit_cast(f32x4, xzb[(4 + t0 + t) * kWave + lane]);
                D[t0 + t] = gC * D[t0 + t] + Z;
#pragma unroll
                for (int s = 0; s < 2; ++s) kt[t][s] = ktr(t0 + t, s);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int t = 0; t < 4; ++t) D[t0 + t] = mfma16(kt[t][s], Eh[s], D[t0 + t]);
#pragma unroll
                for (int t = 0; t < 4; ++t) D[t0 + t] = mfma16(kt[t][s], El[s], D[t0 + t]);
            }
            Db[t0 >> 1] = to_bf16x8(D[t0], D[t0 + 1]);
            Db[(t0 >> 1) + 1] = to_bf16x8(D[t0 + 2], D[t0 + 3]);
        }
        lds_barrier();   // past this barrier the ring slot is refilled and xz rewritten
    }
    if (a.dS0) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dS0[sbase + (size_t)relabel(t, 4 * g + i) * kD + j0w + c16] = D[t][i];
    }
}


// ------------------------------------------------------------------ per-chunk gradients
// One 8-wave workgroup per (chunk, head) with every d_v column, so the terms that sum over d_v
// are formed whole (no shares to write and add up). LDS holds the chunk's K, Q, dY rows as bf16
// tiles (rows swizzled in 16-byte units as in the scans) plus one 64 KB region reused by the
// phases; S and dS' reach the products from registers, as hi + lo fragments of the fp32 values
// each lane loads in the order its fragments need:
//   1. wave w owns d_v columns 16w .. 16w+15 and all 64 tokens (rows relabelled, so each
//      accumulator is the next product's operand): KS = K S, R, U = T R, dW = K dS',
//      X = P^T dY, dU, dR = T^T dU; dv leaves; U and dR go to the region as bf16 hi + lo rows;
//      the region held V, T and P until then;
//   2. the products over d_v: dA = -(dR U^T), dP = dY U^T with K K^T and Q K^T for the gate
//      terms (wave w: lower 16x16 tiles w and w + 8), and dY S^T, dR S^T, U dS'^T for the
//      d_k columns 16w .. 16w+15;
//   3. the coefficient matrices dP o E, (dA o E) beta + its transpose and (dP o E)^T as hi +
//      lo tiles in the region, their products with K and Q, and dq, dk out; then dbeta and dg
//      from the per-token sums every phase left in LDS.
constexpr int kGradThreads = 512;
constexpr int kGradWaves = kGradThreads / kWave;

// element (r, c) of a row-major bf16 tile of 128 / 64 columns, 16-byte units swizzled by row
__device__ __forceinline__ int e128(int r, int c) { return r * kD + ((((c >> 3) ^ swz(r))) << 3) + (c & 7); }
__device__ __forceinline__ int e64(int r, int c) { return r * kC + ((((c >> 3) ^ swz(r))) << 3) + (c & 7); }

// chunk index -> (sequence, first token, length); false past the last chunk
__device__ __forceinline__ bool chunk_range(const BArgs& a, int chunk, int& t0, int& n) {
    if (!a.cu) {
        const int cps = (a.L + kC - 1) / kC;
        if (cps == 0) return false;
        const int seq = chunk / cps;
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
    t0 = a.cu[lo] + (chunk - a.chunk_start[lo]) * kC;
    n = min(kC, a.cu[lo + 1] - t0);
    return true;
}

__device__ __forceinline__ float sum16(float x) { return group_sum<16>(x); }   // a 16-lane row

__global__ void __launch_bounds__(kGradThreads) bwd_chunk_kernel(BArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t Kl[kC * kD], Ql[kC * kD], Yl[kC * kD];
    // phase 1: V [64][128] | T [64][64] | P [64][64]
    // phase 2: U hi | U lo | dR hi | dR lo, [64][128] each
    // phase 3: dQK hi | lo, M hi | lo, dQK^T hi | lo, [64][64] each
    __shared__ __attribute__((aligned(16))) uint16_t reg[4 * kC * kD];
    __shared__ float red_w[4][kGradWaves][kC];   // per wave: dbeta (dR part), dgam (Q, K parts), dw
    __shared__ float red_t[3][4][kC];            // per tile: row and column sums of dD, dbeta (A part)
    __shared__ float red_gc[kGradWaves];
    __shared__ float sG[kC], sGam[kC], sW[kC], sB[kC];

    const int chunk = blockIdx.x, h = blockIdx.y;
    int t0, n;
    if (!chunk_range(a, chunk, t0, n)) return;
    const int H = a.H;
    const size_t ch = (size_t)chunk * H + h;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, g = lane >> 4;
    const int jj = (lane & 15) >> 2, r4 = lane & 3;
    uint16_t* const Vl = reg;
    uint16_t* const Tl = reg + kC * kD;
    uint16_t* const Pl = Tl + kC * kC;
    const float* const Sg = a.Sst + ch * kD * kD;   // S^T [d_v][d_k]
    const float* const dSg = a.dSp + ch * kD * kD;  // dS' [d_k][d_v]

    // ---------------- phase 0: tiles into LDS (rows >= n zero), gates. S and dS' are read in
    // the fragment order their products consume them and stay in registers:
    //   sr  S^T[j][32 s + 8 g .. + 7] (j = 16 wave + c16): B of K S,
    //   dwv dS'[32 s + 8 g + e][j]: B of K dS',
    //   dsv dS'[d][32 s + 8 g .. + 7] (d = 16 wave + c16): B of U dS'^T, and dS' of <S, dS'>.
    const int j = 16 * wave + c16;
    f32x4 dsv[4][2], sr[4][2];
    float dwv[4][8];
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
        u32x4 rk[2], rq[2], ry[2], rv[2], rt_, rp;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = tid + i * kGradThreads, row = u >> 4, un = u & 15;
            const size_t off = ((size_t)(t0 + min(row, n - 1)) * H + h) * kD + un * 8;
            const bool ok = row < n;
            rk[i] = ok ? *reinterpret_cast<const u32x4*>(a.k + off) : z;
            rq[i] = ok ? *reinterpret_cast<const u32x4*>(a.q + off) : z;
            ry[i] = ok ? *reinterpret_cast<const u32x4*>(a.dy + off) : z;
            rv[i] = ok ? *reinterpret_cast<const u32x4*>(a.v + off) : z;
        }
        rt_ = reinterpret_cast<const u32x4*>(a.T + ch * kC * kC)[tid];
        rp = reinterpret_cast<const u32x4*>(a.P + ch * kC * kC)[tid];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4* src = reinterpret_cast<const f32x4*>(dSg + (size_t)j * kD + 32 * i + 8 * g);
            dsv[i][0] = src[0];
            dsv[i][1] = src[1];
            const f32x4* ss = reinterpret_cast<const f32x4*>(Sg + (size_t)j * kD + 32 * i + 8 * g);
            sr[i][0] = ss[0];
            sr[i][1] = ss[1];
#pragma unroll
            for (int e = 0; e < 8; ++e) dwv[i][e] = dSg[(size_t)(32 * i + 8 * g + e) * kD + j];
        }
        if (wave == 0) {
            // both gate loads in flight together, unconditionally (row n - 1 past the end)
            const size_t gr = (size_t)(t0 + min(lane, n - 1)) * H + h;
            const float graw = a.g[gr], braw = a.beta[gr];
            const float gv = lane < n ? graw : 0.f;
            float Gr = gv;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float o = __shfl_up(Gr, off, kWave);
                if (lane >= off) Gr += o;
            }
            const float GC = __shfl(Gr, kC - 1, kWave);
            sG[lane] = Gr;
            sGam[lane] = fexp(Gr);
            sW[lane] = lane < n ? fexp(GC - Gr) : 0.f;
            sB[lane] = lane < n ? braw : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = tid + i * kGradThreads, row = u >> 4, un = u & 15;
            const int o = row * kD + ((un ^ swz(row)) << 3);
            *reinterpret_cast<u32x4*>(Kl + o) = rk[i];
            *reinterpret_cast<u32x4*>(Ql + o) = rq[i];
            *reinterpret_cast<u32x4*>(Yl + o) = ry[i];
            *reinterpret_cast<u32x4*>(Vl + o) = rv[i];
        }
        {
            const int row = tid >> 3, un = tid & 7, o = row * kC + ((un ^ swz(row)) << 3);
            *reinterpret_cast<u32x4*>(Tl + o) = rt_;
            *reinterpret_cast<u32x4*>(Pl + o) = rp;
        }
    }
    __syncthreads();

    // ---------------- phase 1: columns j = 16 wave + c16, tokens relabelled
    auto tokq = [&](int rt) { return 8 * g + 32 * (rt >> 1) + 4 * (rt & 1); };   // the lane's 4 tokens
    auto row4 = [&](const float* v, int rt) { return *reinterpret_cast<const f32x4*>(v + tokq(rt)); };
    auto trcol = [&](const uint16_t* base, int k0, int col0) {
        // X[k0 + 0..7][col0 + c16] of a row-major [*][128] tile (k0 = 32 s + 8 g)
        return tr_pair(base + e128(k0 + jj, col0 + 4 * r4), base + e128(k0 + 4 + jj, col0 + 4 * r4));
    };
    auto trrel = [&](const uint16_t* base, int k0, int rt) {
        // X^T[relabel(rt, c16)][k0 + 0..7] of a row-major [64][64] tile
        const int col = 32 * (rt >> 1) + 8 * r4 + 4 * (rt & 1);
        return tr_pair(base + e64(k0 + jj, col), base + e64(k0 + 4 + jj, col));
    };
    f32x4 U[4], dR[4];
    {
        bf16x8 Sh[4], Slo[4], dWh[4], dWl[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            split8(sr[s][0], sr[s][1], Sh[s], Slo[s]);
            const f32x4 x0 = {dwv[s][0], dwv[s][1], dwv[s][2], dwv[s][3]};
            const f32x4 x1 = {dwv[s][4], dwv[s][5], dwv[s][6], dwv[s][7]};
            split8(x0, x1, dWh[s], dWl[s]);
        }
        f32x4 KS[4], dW[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            KS[rt] = f32x4{};
            dW[rt] = f32x4{};
        }
        // Products on one accumulator are kept apart by products on the others (a product that
        // needs the result of the one just issued waits out the matrix core's latency); every
        // accumulator adds its terms in the order of the formula (hi, then lo, per step).
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 kf[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) kf[rt] = frag(Kl + e128(relabel(rt, c16), 32 * s + 8 * g));
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                KS[rt] = mfma16(kf[rt], Sh[s], KS[rt]);
                dW[rt] = mfma16(kf[rt], dWh[s], dW[rt]);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                KS[rt] = mfma16(kf[rt], Slo[s], KS[rt]);
                dW[rt] = mfma16(kf[rt], dWl[s], dW[rt]);
            }
        }
        // R = beta o (V - gamma o KS); V at the accumulator positions (4 tokens of column j)
        f32x4 R[4], VG[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const u32x2 vv = __builtin_bit_cast(u32x2, lds_tr16(Vl + e128(tokq(rt) + jj, 16 * wave + 4 * r4)));
            const f32x4 vf = {__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xffff0000u),
                              __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xffff0000u)};
            VG[rt] = vf - row4(sGam, rt) * KS[rt];
            R[rt] = row4(sB, rt) * VG[rt];
        }
        bf16x8 Rh[2], Rl[2];
        split8(R[0], R[1], Rh[0], Rl[0]);
        split8(R[2], R[3], Rh[1], Rl[1]);
        // U = T R (T lower triangular: token tiles 0-1 need step 0 only)
        {
            bf16x8 tf[4][2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                U[rt] = f32x4{};
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (s <= (rt >> 1)) tf[rt][s] = frag(Tl + e64(relabel(rt, c16), 32 * s + 8 * g));
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) U[rt] = mfma16(tf[rt][0], Rh[0], U[rt]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) U[rt] = mfma16(tf[rt][0], Rl[0], U[rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt) U[rt] = mfma16(tf[rt][1], Rh[1], U[rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt) U[rt] = mfma16(tf[rt][1], Rl[1], U[rt]);
        }
        // dU = w o dW + P^T dY (P^T upper triangular)
        bf16x8 yb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) yb[s] = trcol(Yl, 32 * s + 8 * g, 16 * wave);
        f32x4 dU[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dU[rt] = row4(sW, rt) * dW[rt];
        // token tiles 0-1 take steps 0 and 1, tiles 2-3 step 1 only (P^T upper triangular)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) dU[rt] = mfma16(trrel(Pl, 8 * g, rt), yb[0], dU[rt]);
#pragma unroll
        for (int rt = 3; rt >= 0; --rt) dU[rt] = mfma16(trrel(Pl, 32 + 8 * g, rt), yb[1], dU[rt]);
        bf16x8 dUh[2], dUl[2];
        split8(dU[0], dU[1], dUh[0], dUl[0]);
        split8(dU[2], dU[3], dUh[1], dUl[1]);
        // dR = T^T dU (upper triangular)
        {
            // tiles 0-1: steps 0 and 1, tiles 2-3: step 1 (T^T upper triangular); per tile the
            // order is step 0 hi, lo, step 1 hi, lo
            bf16x8 tt[4][2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                dR[rt] = f32x4{};
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (s >= (rt >> 1)) tt[rt][s] = trrel(Tl, 32 * s + 8 * g, rt);
            }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) dR[rt] = mfma16(tt[rt][0], dUh[0], dR[rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt) dR[rt] = mfma16(tt[rt][1], dUh[1], dR[rt]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) dR[rt] = mfma16(tt[rt][0], dUl[0], dR[rt]);
#pragma unroll
            for (int rt = 2; rt < 4; ++rt) dR[rt] = mfma16(tt[rt][1], dUl[1], dR[rt]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) dR[rt] = mfma16(tt[rt][1], dUh[1], dR[rt]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) dR[rt] = mfma16(tt[rt][1], dUl[1], dR[rt]);
        }
        // dv = beta o dR; per-token sum of dR o (V - gamma KS) over this wave's columns
        float* dvp = a.dv + ((size_t)t0 * H + h) * kD + j;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 bt = row4(sB, rt);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = tokq(rt) + i;
                if (tok < n) dvp[(size_t)tok * H * kD] = bt[i] * dR[rt][i];
                const float sdb = sum16(dR[rt][i] * VG[rt][i]);
                if (c16 == 0) red_w[0][wave][tok] = sdb;
            }
        }
    }
    // S[d][32 s + 8 g + e] (d = 16 wave + c16) for phase 2: B of dY S^T and dR S^T, and S of
    // <S, dS'>; loaded now so they arrive during phase 2a
    float scol[4][8];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) scol[s][e] = Sg[(size_t)(32 * s + 8 * g + e) * kD + j];
    __syncthreads();   // V, T, P no longer read: the region takes U and dR
    {
        uint16_t* const Uh = reg;
        uint16_t* const Ul = reg + kC * kD;
        uint16_t* const Rh = reg + 2 * kC * kD;
        uint16_t* const Rl = reg + 3 * kC * kD;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = e128(tokq(rt) + i, j);
                const uint16_t uh = f2bf(U[rt][i]);
                Uh[o] = uh;
                Ul[o] = f2bf(U[rt][i] - bf2f(uh));
                const uint16_t rh = f2bf(dR[rt][i]);
                Rh[o] = rh;
                Rl[o] = f2bf(dR[rt][i] - bf2f(rh));
            }
    }
    __syncthreads();

    // ---------------- phase 2a: lower 16x16 tiles of dA, dP (and K K^T, Q K^T), natural order
    const uint16_t* const Uh = reg;
    const uint16_t* const Ul = reg + kC * kD;
    const uint16_t* const Rh = reg + 2 * kC * kD;
    const uint16_t* const Rlo = reg + 3 * kC * kD;
    constexpr int kTiles = 10;
    f32x4 dKKt[2], dQKt[2];
    int trt[2], tit[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tile = wave + q * kGradWaves;
        int rt = 0;
        while ((rt + 1) * (rt + 2) / 2 <= tile) ++rt;   // tile -> (rt, it), it <= rt
        trt[q] = rt;
        tit[q] = tile - rt * (rt + 1) / 2;
        dKKt[q] = f32x4{};
        dQKt[q] = f32x4{};
        if (tile >= kTiles) continue;
        const int it = tit[q];
        f32x4 dA = {}, dP = {}, KK = {}, QK = {};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int ar = e128(16 * rt + c16, 32 * s + 8 * g), br = e128(16 * it + c16, 32 * s + 8 * g);
            const bf16x8 uh = frag(Uh + br), ul = frag(Ul + br), kb = frag(Kl + br);
            const bf16x8 ya = frag(Yl + ar);
            dA = mfma16(frag(Rh + ar), uh, dA);
            dP = mfma16(ya, uh, dP);
            KK = mfma16(frag(Kl + ar), kb, KK);
            QK = mfma16(frag(Ql + ar), kb, QK);
            dA = mfma16(frag(Rlo + ar), uh, dA);
            dP = mfma16(ya, ul, dP);
        }
        float rs_d[4], rs_a[4], cs = 0.f;
        const int col = 16 * it + c16;
        const float Gc = sG[col];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * g + i;
            const float dec = (col <= r && r < n) ? fexp(sG[r] - Gc) : 0.f;
            const float ea = col < r ? dec : 0.f;
            const float b = sB[r];
            const float da = -dA[i];
            dKKt[q][i] = b * da * ea;
            dQKt[q][i] = dP[i] * dec;
            const float dd = b * da * ea * KK[i] + dP[i] * dec * QK[i];
            rs_d[i] = sum16(dd);
            rs_a[i] = sum16(da * ea * KK[i]);
            cs += dd;
        }
        cs = sum_across<16>(cs);
        if (c16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                red_t[0][it][16 * rt + 4 * g + i] = rs_d[i];
                red_t[2][it][16 * rt + 4 * g + i] = rs_a[i];
            }
        if (g == 0) red_t[1][rt][col] = cs;
    }

    // ---------------- phase 2b: d_k columns d = 16 wave + c16 of dY S^T, dR S^T, U dS'^T
    const int d = j;
    f32x4 dQa[4], dKa[4];
    {
        f32x4 Q1[4], K2[4], K1[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            Q1[rt] = f32x4{};
            K2[rt] = f32x4{};
            K1[rt] = f32x4{};
        }
        float gc = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int k0 = 32 * s + 8 * g;
            const f32x4 s0 = {scol[s][0], scol[s][1], scol[s][2], scol[s][3]};   // S[d][k0 ..]
            const f32x4 s1 = {scol[s][4], scol[s][5], scol[s][6], scol[s][7]};
            const f32x4 x0 = dsv[s][0], x1 = dsv[s][1];                           // dS'[d][k0 ..]
            bf16x8 sbh, sbl, dh, dl;
            split8(s0, s1, sbh, sbl);
            split8(x0, x1, dh, dl);
#pragma unroll
            for (int e = 0; e < 4; ++e) gc += s0[e] * x0[e] + s1[e] * x1[e];
            // per accumulator: Q1 and K2 hi then lo; K1 uh dh, ul dh, uh dl
            bf16x8 uh[4], ya[4], ra[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int ar = e128(16 * rt + c16, k0);
                uh[rt] = frag(Uh + ar);
                ya[rt] = frag(Yl + ar);
                ra[rt] = frag(Rh + ar);
                Q1[rt] = mfma16(ya[rt], sbh, Q1[rt]);
                K2[rt] = mfma16(ra[rt], sbh, K2[rt]);
                K1[rt] = mfma16(uh[rt], dh, K1[rt]);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                Q1[rt] = mfma16(ya[rt], sbl, Q1[rt]);
                K2[rt] = mfma16(ra[rt], sbl, K2[rt]);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) K1[rt] = mfma16(frag(Ul + e128(16 * rt + c16, k0)), dh, K1[rt]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) K1[rt] = mfma16(uh[rt], dl, K1[rt]);
        }
        gc = group_sum<kWave>(gc);
        if (lane == 0) red_gc[wave] = gc;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 gm = *reinterpret_cast<const f32x4*>(sGam + 16 * rt + 4 * g);
            const f32x4 wr = *reinterpret_cast<const f32x4*>(sW + 16 * rt + 4 * g);
            const f32x4 br = *reinterpret_cast<const f32x4*>(sB + 16 * rt + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * g + i, o = e128(r, d);
                const float qv = bf2f(Ql[o]), kv = bf2f(Kl[o]);
                const float s1 = sum16(qv * Q1[rt][i]);
                const float s2 = sum16(kv * K2[rt][i]);
                const float s3 = sum16(kv * K1[rt][i]);
                if (c16 == 0) {
                    red_w[1][wave][r] = s1;
                    red_w[2][wave][r] = s2;
                    red_w[3][wave][r] = s3;
                }
                dQa[rt][i] = gm[i] * Q1[rt][i];
                dKa[rt][i] = wr[i] * K1[rt][i] - br[i] * gm[i] * K2[rt][i];
            }
        }
    }
    __syncthreads();   // U and dR no longer read: the region takes the coefficient matrices

    // ---------------- phase 3: dQK, M = dKK + dKK^T, dQK^T as hi + lo [64][64] tiles
    uint16_t* const QKh = reg;
    uint16_t* const QKl = reg + kC * kC;
    uint16_t* const Mh = reg + 2 * kC * kC;
    uint16_t* const Ml = reg + 3 * kC * kC;
    uint16_t* const QTh = reg + 4 * kC * kC;
    uint16_t* const QTl = reg + 5 * kC * kC;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (wave + q * kGradWaves >= kTiles) continue;
        const int rt = trt[q], it = tit[q], col = 16 * it + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * g + i;
            const uint16_t qh = f2bf(dQKt[q][i]), ql = f2bf(dQKt[q][i] - bf2f(qh));
            const uint16_t mh = f2bf(dKKt[q][i]), ml = f2bf(dKKt[q][i] - bf2f(mh));
            int o = e64(r, col);
            QKh[o] = qh; QKl[o] = ql;
            if (rt != it || col <= r) {   // the upper part of a diagonal tile is M's transpose
                Mh[o] = mh; Ml[o] = ml;
            }
            o = e64(col, r);   // transposed position
            QTh[o] = qh; QTl[o] = ql;
            if (rt != it) {
                Mh[o] = mh; Ml[o] = ml;
                QKh[o] = 0; QKl[o] = 0;
                const int o2 = e64(r, col);
                QTh[o2] = 0; QTl[o2] = 0;
            } else if (col < r) {
                Mh[o] = mh; Ml[o] = ml;
            }
        }
    }
    __syncthreads();
    // per accumulator and step: dQK hi, lo; M hi, lo, then dQK^T hi, lo (as the formula reads);
    // the four token tiles take turns
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int k0 = 32 * s + 8 * g;
        const bf16x8 kb = trcol(Kl, k0, 16 * wave);
        const bf16x8 qb = trcol(Ql, k0, 16 * wave);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int ar = e64(16 * rt + c16, k0);
            if (s <= (rt >> 1)) dQa[rt] = mfma16(frag(QKh + ar), kb, dQa[rt]);   // dQK lower triangular
            dKa[rt] = mfma16(frag(Mh + ar), kb, dKa[rt]);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int ar = e64(16 * rt + c16, k0);
            if (s <= (rt >> 1)) dQa[rt] = mfma16(frag(QKl + ar), kb, dQa[rt]);
            dKa[rt] = mfma16(frag(Ml + ar), kb, dKa[rt]);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            if (s >= (rt >> 1)) dKa[rt] = mfma16(frag(QTh + e64(16 * rt + c16, k0)), qb, dKa[rt]);   // dQK^T upper
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            if (s >= (rt >> 1)) dKa[rt] = mfma16(frag(QTl + e64(16 * rt + c16, k0)), qb, dKa[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * g + i;
            if (r < n) {
                const size_t o = ((size_t)(t0 + r) * H + h) * kD + d;
                a.dq[o] = dQa[rt][i];
                a.dk[o] = dKa[rt][i];
            }
        }
    }
    // dbeta and dg of the chunk's tokens (wave 0, lane = token)
    if (wave == 0) {
        const int r = lane, rb = r >> 4;
        float db = 0.f, dg1 = 0.f, dg2 = 0.f, dw = 0.f, rs = 0.f, cs = 0.f, gc = 0.f;
#pragma unroll
        for (int w = 0; w < kGradWaves; ++w) {
            db += red_w[0][w][r];
            dg1 += red_w[1][w][r];
            dg2 += red_w[2][w][r];
            dw += red_w[3][w][r];
            gc += red_gc[w];
        }
        for (int it = 0; it <= rb; ++it) {
            rs += red_t[0][it][r];
            db += red_t[2][it][r];
        }
        for (int rt = rb; rt < 4; ++rt) cs += red_t[1][rt][r];
        const bool ok = r < n;
        const float gam = sGam[r], wr = sW[r];
        const float dgam = dg1 - sB[r] * dg2;
        float dG = ok ? rs - cs + dgam * gam - dw * wr : 0.f;
        float tot = ok ? dw * wr : 0.f;
        tot = group_sum<kWave>(tot);
        if (r == n - 1) dG += gc * sGam[n - 1] + tot;
        // dg = reverse running sum of dG over the chunk
        float acc = dG;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const float v = __shfl_down(acc, o, kWave);
            if (lane + o < kWave) acc += v;
        }
        if (ok) {
            const size_t row = (size_t)(t0 + r) * H + h;
            a.dg[row] = acc;
            a.dbeta[row] = db;
        }
    }
}

}  // namespace

bool use_bwd_bf16(const ChunkBwdArgs& c) {
    return c.in_bf16 && c.dy_bf16 && c.dk == kD && c.dv == kD;
}

// the forward tiles of the bf16 prefill, then S^T and dS' (fp32) per chunk-head
static size_t bwd_bf16_offsets(int ntok, int num_seqs, int H, size_t& off_S, size_t& off_dS) {
    const size_t ch = (size_t)((ntok + kC - 1) / kC + num_seqs) * H;
    off_S = (chunk_bf16_workspace(ntok, num_seqs, H) + 255) & ~(size_t)255;
    off_dS = off_S + ((ch * kD * kD * sizeof(float) + 255) & ~(size_t)255);
    return off_dS + ch * kD * kD * sizeof(float);
}

size_t chunk_bwd_bf16_workspace(int ntok, int num_seqs, int H) {
    size_t a, b;
    return bwd_bf16_offsets(ntok, num_seqs, H, a, b);
}

hipError_t launch_chunk_bwd_bf16(const ChunkBwdArgs& c, hipStream_t s) {
    size_t off_S, off_dS;
    bwd_bf16_offsets(c.ntok, c.num_seqs, c.H, off_S, off_dS);
    char* ws = static_cast<char*>(c.workspace);
    float* Sst = reinterpret_cast<float*>(ws + off_S);
    // 1. forward sweep: chunk table, T and P, the state entering every chunk
    ChunkArgs f{};
    f.q = c.q; f.k = c.k; f.v = c.v; f.in_bf16 = 1; f.y_bf16 = 1;
    f.g = c.g; f.beta = c.beta; f.S0 = c.S0; f.ST = nullptr; f.cu = c.cu;
    f.num_seqs = c.num_seqs; f.ntok = c.ntok; f.H = c.H; f.dk = c.dk; f.dv = c.dv;
    f.y = nullptr; f.workspace = c.workspace; f.workspace_bytes = off_S;
    hipError_t e = launch_chunk_bf16_states(f, Sst, s);
    if (e != hipSuccess) return e;
    const ChunkTiles t = chunk_bf16_tiles(c.workspace, c.ntok, c.num_seqs, c.H);
    BArgs a;
    a.q = static_cast<const uint16_t*>(c.q);
    a.k = static_cast<const uint16_t*>(c.k);
    a.v = static_cast<const uint16_t*>(c.v);
    a.dy = static_cast<const uint16_t*>(c.dy);
    a.g = c.g; a.beta = c.beta; a.dST = c.dST; a.cu = c.cu;
    a.chunk_start = c.cu ? t.chunk_start : nullptr;
    a.order = c.cu ? t.order : nullptr;
    a.T = t.T; a.P = t.P; a.Gw = t.Gw;
    a.Sst = Sst;
    a.dSp = reinterpret_cast<float*>(ws + off_dS);
    a.dq = c.dq; a.dk = c.dk_; a.dv = c.dv_; a.dg = c.dg; a.dbeta = c.dbeta; a.dS0 = c.dS0;
    a.num_seqs = c.num_seqs; a.ntok = c.ntok; a.H = c.H;
    a.L = c.cu ? 0 : c.ntok / c.num_seqs;
    // 2. reverse chain per (sequence, head, 32-column slice)
    const int pairs = c.num_seqs * c.H;
    const int blocks = (pairs + 7) / 8 * 8 * (kD / kSl);
    hipLaunchKernelGGL(bwd_chain_kernel, dim3(blocks), dim3(kChainThreads), 0, s, a);
    // 3. every gradient per (chunk, head)
    const int nchunks = c.cu ? t.max_chunks : c.num_seqs * ((a.L + kC - 1) / kC);
    if (nchunks > 0)
        hipLaunchKernelGGL(bwd_chunk_kernel, dim3(nchunks, c.H), dim3(kGradThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gdn
