// Pre- and post-processing of the Gated DeltaNet layer on gfx950: memory-bound streaming
// kernels (reading notes of "On the Design of Qwen3.8-Next Architecture", section 2.1.1).
//
//   preprocess  : eqs. (6)-(8) ShortConv (width 4, depthwise, causal) -> SiLU -> L2Norm on
//                 q and k, ShortConv -> SiLU on v; eqs. (9)-(10) the per-head gates.
//   output gate : eq. (11) without W_o, sigmoid(z) * zero-centred RMSNorm(y).
//
// Layout: token-major [ntok, H, d], so one token's H*d channels are contiguous. A thread
// owns 8 consecutive channels (one 16-byte bf16 or 32-byte fp32 access), a workgroup of
// 256 threads owns a 2048-channel tile, and the d/8 lanes of one head are adjacent lanes
// of one wave, so the L2Norm / RMSNorm reductions are in-register shuffles.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kPreThreads = 256;
constexpr int kPreTile = kPreThreads * 8;   // channels per workgroup
constexpr int kPreTokens = 64;              // tokens per workgroup (3-token conv halo)
constexpr int kConvK = 4;
constexpr int kPreGroup = 1;                // tokens per step (loaded one step ahead)

struct PreKernelArgs {
    PreprocessArgs a;
    int tiles[3];        // channel tiles per stream
    int gate_blocks;     // 1 if gates are computed
};

// Index of the sequence holding token t: largest s with cu[s] <= t (skips empty sequences).
__device__ __forceinline__ int seq_of(const int32_t* cu, int num_seqs, int t) {
    int lo = 0, hi = num_seqs;   // invariant: cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

template <typename Tin, typename Tout>
__device__ void conv_stream(const PreprocessArgs& a, int role, int tile, int t0) {
    const int d = a.d[role];
    const int C = a.H * d;
    const int c = tile * kPreTile + threadIdx.x * 8;
    if (c >= C) return;   // whole heads drop out together (C and the tile are multiples of d)
    const Tin* x = static_cast<const Tin*>(a.x[role]);
    Tout* out = static_cast<Tout*>(a.out[role]);
    const bool norm = role < 2;

    float w[8][kConvK];
    {
        const float4* wp = reinterpret_cast<const float4*>(a.w[role] + (size_t)c * kConvK);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 t = wp[i];
            w[i][0] = t.x; w[i][1] = t.y; w[i][2] = t.z; w[i][3] = t.w;
        }
    }
    const int t1 = min(a.ntok, t0 + kPreTokens);

    // sequence bookkeeping (uniform over the workgroup)
    int s, seq_lo, seq_hi;
    if (a.cu) {
        s = seq_of(a.cu, a.num_seqs, t0);
        seq_lo = a.cu[s];
        seq_hi = a.cu[s + 1];
    } else {
        const int L = a.ntok / a.num_seqs;
        s = t0 / L;
        seq_lo = s * L;
        seq_hi = seq_lo + L;
    }

    // Carried conv history (optional): [num_seqs, 3, hC] rows of this stream's channels,
    // row 2 the input just before the sequence start. Absent, the history is zero.
    const Tin* hin = static_cast<const Tin*>(a.hin);
    Tin* hout = static_cast<Tin*>(a.hout);
    const int hoff = role == 0 ? 0 : (role == 1 ? a.H * a.d[0] : 2 * a.H * a.d[0]);
    auto hist_row = [&](int seq, int r) __attribute__((always_inline)) {
        return (size_t)(seq * 3 + r) * a.hC + hoff + c;
    };
    // history of sequence `seq` into the window (the conv restarts at its first token)
    auto restart = [&](int seq, float (&wn)[3][8]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            if (hin) {
                Vec8<Tin>::load(hin + hist_row(seq, r), wn[r]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) wn[r][i] = 0.f;
            }
        }
    };

    // history window: win[0] = x[t-3] ... win[2] = x[t-1]; before the sequence start it
    // comes from the carried history
    float win[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int src = t0 - 3 + j;
        if (src >= seq_lo) {
            Vec8<Tin>::load(x + (size_t)src * C + c, win[j]);
        } else if (hin) {
            Vec8<Tin>::load(hin + hist_row(s, 3 - (seq_lo - src)), win[j]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) win[j][i] = 0.f;
        }
    }

    // kPreGroup tokens per step, software-pipelined: the next step's rows are loaded while
    // this step's conv / SiLU / L2Norm runs (the window recurrence runs on registers). These
    // rows are read once (the next workgroup's 3-token history aside), so they stream past
    // the caches and leave them to q, k, v, which the prefill reads next.
    typename Vec8<Tin>::Raw nxt[kPreGroup];
    auto issue = [&](int tb) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kPreGroup; ++j)
            nxt[j] = Vec8<Tin>::template load_raw<true>(x + (size_t)min(tb + j, t1 - 1) * C + c);
    };
    issue(t0);
    for (int tb = t0; tb < t1; tb += kPreGroup) {
        float grp[kPreGroup][8];
#pragma unroll
        for (int j = 0; j < kPreGroup; ++j) Vec8<Tin>::unpack(nxt[j], grp[j]);
        if (tb + kPreGroup < t1) issue(tb + kPreGroup);   // the next group loads under this one's math
#pragma unroll
        for (int j = 0; j < kPreGroup; ++j) {
            const int t = tb + j;
            if (t >= t1) break;
            if (t >= seq_hi) {   // crossed into the next non-empty sequence: history restarts
                if (a.cu) {
                    while (a.cu[s + 1] <= t) ++s;
                    seq_hi = a.cu[s + 1];
                } else {
                    ++s;
                    seq_hi += a.ntok / a.num_seqs;
                }
                restart(s, win);
            }
            // the last three inputs of a sequence become its carried history
            if (hout && t >= seq_hi - 3) Vec8<Tin>::store(hout + hist_row(s, 3 - (seq_hi - t)), grp[j]);
            float act[8];
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float sv = siluf_(conv4(w[i][0], w[i][1], w[i][2], w[i][3], win[0][i],
                                              win[1][i], win[2][i], grp[j][i]));
                act[i] = sv;
                ss = __builtin_fmaf(sv, sv, ss);
            }
            if (norm) {
                ss = (d == 128) ? group_sum<16>(ss) : group_sum<8>(ss);
                const float inv = frsq(ss + a.l2_eps);
#pragma unroll
                for (int i = 0; i < 8; ++i) act[i] *= inv;
            }
            Vec8<Tout>::store(out + (size_t)t * C + c, act);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                win[0][i] = win[1][i];
                win[1][i] = win[2][i];
                win[2][i] = grp[j][i];
            }
        }
    }
}

__device__ void gates_block(const PreprocessArgs& a, int t0) {
    const int n = min(kPreTokens, a.ntok - t0) * a.H;
    for (int i = threadIdx.x; i < n; i += kPreThreads) {
        const size_t e = (size_t)t0 * a.H + i;
        const int h = i % a.H;
        a.g[e] = gate_g(a.A_log[h], a.a_raw[e], a.dt_bias[h]);
        a.beta[e] = gate_beta(a.b_raw[e]);
    }
}

// Carried history of sequences shorter than 3 tokens (empty ones included): their older rows
// are the input history shifted by the sequence length (zero without one). The rows of the
// sequence's own tokens are written by the conv. Copies 16-byte units of raw input.
__global__ void __launch_bounds__(kPreThreads) conv_carry_kernel(PreprocessArgs a, int elem_bytes) {
    const int s = blockIdx.x;
    const int L = a.cu ? a.cu[s + 1] - a.cu[s] : a.ntok / a.num_seqs;
    if (L >= 3) return;
    const int units = a.hC * elem_bytes / 16;   // 16-byte units per history row
    const uint4* hin = static_cast<const uint4*>(a.hin);
    uint4* hout = static_cast<uint4*>(a.hout);
    for (int r = 0; r < 3 - L; ++r)
        for (int u = threadIdx.x; u < units; u += kPreThreads)
            hout[(size_t)(s * 3 + r) * units + u] =
                hin ? hin[(size_t)(s * 3 + r + L) * units + u] : make_uint4(0u, 0u, 0u, 0u);
}

template <typename Tin, typename Tout>
__global__ void __launch_bounds__(kPreThreads) preprocess_kernel(PreKernelArgs p) {
    const int t0 = blockIdx.x * kPreTokens;
    int y = blockIdx.y;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        if (y < p.tiles[r]) {
            conv_stream<Tin, Tout>(p.a, r, y, t0);
            return;
        }
        y -= p.tiles[r];
    }
    if (y < p.gate_blocks) gates_block(p.a, t0);
}

hipError_t launch_preprocess(const PreprocessArgs& a, hipStream_t s) {
    PreKernelArgs p;
    p.a = a;
    int ny = 0;
    for (int r = 0; r < 3; ++r) {
        p.tiles[r] = a.x[r] ? (a.H * a.d[r] + kPreTile - 1) / kPreTile : 0;
        ny += p.tiles[r];
    }
    p.gate_blocks = a.a_raw ? 1 : 0;
    ny += p.gate_blocks;
    // the conv taps mark the conv part as asked for: x may be NULL when ntok == 0
    const bool carry = a.hout && a.w[0];
    if (carry)
        hipLaunchKernelGGL(conv_carry_kernel, dim3(a.num_seqs), dim3(kPreThreads), 0, s, a,
                           a.in_bf16 ? 2 : 4);
    if (ny == 0 || a.ntok == 0) return carry ? hipGetLastError() : hipSuccess;
    dim3 grid((a.ntok + kPreTokens - 1) / kPreTokens, ny);
    if (a.in_bf16 && a.out_bf16)
        hipLaunchKernelGGL((preprocess_kernel<uint16_t, uint16_t>), grid, dim3(kPreThreads), 0, s, p);
    else if (a.in_bf16)
        hipLaunchKernelGGL((preprocess_kernel<uint16_t, float>), grid, dim3(kPreThreads), 0, s, p);
    else if (a.out_bf16)
        hipLaunchKernelGGL((preprocess_kernel<float, uint16_t>), grid, dim3(kPreThreads), 0, s, p);
    else
        hipLaunchKernelGGL((preprocess_kernel<float, float>), grid, dim3(kPreThreads), 0, s, p);
    return hipGetLastError();
}

// --------------------------------------------------------------------------- output gate
constexpr int kGateThreads = 256;

template <typename Ty, typename Tz, typename To, int DV>
__global__ void __launch_bounds__(kGateThreads)
output_gate_kernel(const Ty* __restrict__ y, const Tz* __restrict__ z, const float* __restrict__ w,
                   long rows, float eps, To* __restrict__ o) {
    constexpr int LPR = DV / 8;                    // lanes per (token, head) row
    constexpr int RPB = kGateThreads / LPR;        // rows per workgroup pass
    const int lane_c = (threadIdx.x % LPR) * 8;
    float gain[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) gain[i] = 1.0f + w[lane_c + i];
    // two row groups per step, so four 16-byte loads per thread are in flight together; z and
    // o are touched once and stream past the caches, y (just written by the prefill) does not
    const long tiles = (rows + 2 * RPB - 1) / (2 * RPB);   // 2 RPB rows per workgroup tile
    for (long bt = blockIdx.x; bt < tiles; bt += gridDim.x) {
        const long r0 = bt * 2 * RPB + threadIdx.x / LPR, r1 = r0 + RPB;
        if (r0 >= rows) break;
        const size_t off0 = (size_t)r0 * DV + lane_c;
        const size_t off1 = (size_t)(r1 < rows ? r1 : r0) * DV + lane_c;
        float yv[2][8], zv[2][8];
        Vec8<Ty>::load(y + off0, yv[0]);
        Vec8<Tz>::template load<true>(z + off0, zv[0]);
        Vec8<Ty>::load(y + off1, yv[1]);
        Vec8<Tz>::template load<true>(z + off1, zv[1]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += yv[u][i] * yv[u][i];
            ss = group_sum<LPR>(ss);
            const float inv = frsq(ss * (1.0f / DV) + eps);
            float ov[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) ov[i] = sigmoidf_(zv[u][i]) * (gain[i] * (yv[u][i] * inv));
            // unconditional: past the last row, row group 1 recomputes row r0 and stores the same
            // values again (a conditional store lets the compiler sink z's second load under it,
            // after row group 0's math, which costs a second memory round trip per step)
            Vec8<To>::template store<true>(o + (u ? off1 : off0), ov);
        }
    }
}

template <int DV>
static void launch_gate_dv(const void* y, int yb, const void* z, int zb, const float* w, long rows,
                           float eps, void* o, int ob, hipStream_t s) {
    constexpr int RPB = kGateThreads / (DV / 8);
    // one tile per workgroup: capping the grid (each workgroup then walks several tiles) was
    // slower on large calls, 5.1M rows 712 us at 16,384 workgroups and 692 at 65,536 against
    // 664 uncapped, and the same on 262,144 rows (8,192 tiles)
    const long blocks = (rows + 2 * RPB - 1) / (2 * RPB);
    const int grid = (int)(blocks < 0x7fffffffL ? blocks : 0x7fffffffL);
#define GDN_GATE(TY, TZ, TO)                                                                 \
    hipLaunchKernelGGL((output_gate_kernel<TY, TZ, TO, DV>), dim3(grid), dim3(kGateThreads), 0, s, \
                       static_cast<const TY*>(y), static_cast<const TZ*>(z), w, rows, eps,   \
                       static_cast<TO*>(o))
    const int key = (yb << 2) | (zb << 1) | ob;
    switch (key) {
        case 0: GDN_GATE(float, float, float); break;
        case 1: GDN_GATE(float, float, uint16_t); break;
        case 2: GDN_GATE(float, uint16_t, float); break;
        case 3: GDN_GATE(float, uint16_t, uint16_t); break;
        case 4: GDN_GATE(uint16_t, float, float); break;
        case 5: GDN_GATE(uint16_t, float, uint16_t); break;
        case 6: GDN_GATE(uint16_t, uint16_t, float); break;
        default: GDN_GATE(uint16_t, uint16_t, uint16_t); break;
    }
#undef GDN_GATE
}

hipError_t launch_output_gate(const void* y, int y_bf16, const void* z, int z_bf16, const float* w,
                              int ntok, int H, int dv, float eps, void* o, int o_bf16,
                              hipStream_t s) {
    const long rows = (long)ntok * H;
    if (rows == 0) return hipSuccess;
    if (dv == 128)
        launch_gate_dv<128>(y, y_bf16, z, z_bf16, w, rows, eps, o, o_bf16, s);
    else
        launch_gate_dv<64>(y, y_bf16, z, z_bf16, w, rows, eps, o, o_bf16, s);
    return hipGetLastError();
}

}  // namespace gdn
