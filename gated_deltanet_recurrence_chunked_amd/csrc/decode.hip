// Single-token recurrent step of the gated delta rule on gfx950 (reading notes of
// "On the Design of Qwen3.8-Next Architecture", section 2.1.1, eqs. (1)-(4)):
//   S~ = alpha S;  e = v - S~^T k;  S = S~ + beta k e^T;  y = S^T q
// rewritten for one pass over S:  with sk = S^T k and sq = S^T q of the OLD state,
//   e = v - alpha sk,   y = alpha sq + beta (k.q) e,   S_new = alpha S + beta k e^T.
//
// HBM-bound (about 0.9 flop per byte): each (sequence, head) state (dk*dv fp32) is read
// once and written once, in place. One 256-thread workgroup owns one state; a thread owns
// 4 adjacent columns (one 16-byte access) of dk/RG rows, so every wave reads whole
// contiguous rows. The state stays in registers between the two reductions and the write.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kDecThreads = 256;

template <int DK, int DV, typename Tin, typename Tout>
__global__ void __launch_bounds__(kDecThreads)
decode_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
              const float* __restrict__ g, const float* __restrict__ beta, float* state,
              Tout* __restrict__ y) {
    constexpr int TPR = DV / 4;              // threads per state row
    constexpr int RG = kDecThreads / TPR;    // row groups
    constexpr int RPT = DK / RG;             // rows per thread
    constexpr int RGW = kWave / TPR;         // row groups per wave
    constexpr int NW = kDecThreads / kWave;
    static_assert(RPT >= 1 && DK % RG == 0, "shape");

    __shared__ float ks[DK], qs[DK];
    __shared__ float red[NW][2][DV];

    const int head = blockIdx.x;             // flattened (sequence, head)
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int c = (tid % TPR) * 4;
    const int rg = tid / TPR;

    // the token's loads first and unconditional (a load under a branch is waited for at the
    // join, and the counter completes loads in issue order), then the state's
    const int ek = min(tid, 2 * DK - 1);
    const Tin kq_in = ((ek < DK ? k : q) + (size_t)head * DK)[ek < DK ? ek : ek - DK];   // raw
    float vv[4];
    Vec4<Tin>::load(v + (size_t)head * DV + c, vv);
    __builtin_amdgcn_sched_barrier(0);
    float* S = state + (size_t)head * DK * DV;
    float s[RPT][4];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const floatx4 t = __builtin_nontemporal_load(
            reinterpret_cast<const floatx4*>(S + (size_t)(rg + RG * i) * DV + c));
        s[i][0] = t.x; s[i][1] = t.y; s[i][2] = t.z; s[i][3] = t.w;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (tid < DK) ks[tid] = load1(&kq_in);
    else if (tid < 2 * DK) qs[tid - DK] = load1(&kq_in);
    const float a = expf(g[head]);
    const float b = beta[head];
    __syncthreads();

    // k.q (every wave computes it; no extra barrier)
    float kq = 0.f;
#pragma unroll
    for (int i = lane; i < DK; i += kWave) kq += ks[i] * qs[i];
    kq = group_sum<kWave>(kq);

    float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kr = ks[rg + RG * i], qr = qs[rg + RG * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pk[j] += s[i][j] * kr;
            pq[j] += s[i][j] * qr;
        }
    }
    // reduce over the row groups of this wave (lanes TPR apart), then across waves in LDS
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        pk[j] = sum_across<TPR>(pk[j]);
        pq[j] = sum_across<TPR>(pq[j]);
    }
    if (lane < TPR) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            red[wave][0][c + j] = pk[j];
            red[wave][1][c + j] = pq[j];
        }
    }
    __syncthreads();
    float e[4], yo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            sk += red[w][0][c + j];
            sq += red[w][1][c + j];
        }
        e[j] = vv[j] - a * sk;
        yo[j] = a * sq + b * kq * e[j];
    }
    (void)RGW;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float bk = b * ks[rg + RG * i];
        floatx4 t;
        t.x = a * s[i][0] + bk * e[0];
        t.y = a * s[i][1] + bk * e[1];
        t.z = a * s[i][2] + bk * e[2];
        t.w = a * s[i][3] + bk * e[3];
        __builtin_nontemporal_store(t, reinterpret_cast<floatx4*>(S + (size_t)(rg + RG * i) * DV + c));
    }
    if (rg == 0) Vec4<Tout>::store(y + (size_t)head * DV + c, yo);
}

// ----------------------------------------------------------------------------------------
// Persistent form of the single-token step for d_k = d_v = 128, the shape of the serving
// workloads: one 1024-thread workgroup per CU, each walking heads blockIdx.x, + gridDim.x, ...
// with the next head's state and token loads issued before the current head's reductions and
// stores, so a CU's state reads keep streaming while the previous head is reduced and written
// back (8,192 heads: 186 us per step against 190 for one workgroup per head). A thread owns 4
// columns of 4 consecutive rows (one address, the rows at immediate offsets). Same arithmetic
// as decode_kernel per element; the partial sums over the state rows are grouped differently
// (per thread, then per wave, then over the 16 waves in order), so results can differ from it
// in the last bits. Two 512-thread workgroups per CU measured 196 us, and a third head in
// flight (registers spilled) 193 us.
constexpr int kPipeThreads = 1024;
constexpr int kPipePerCU = 1;
constexpr int kPipeWavesPerSimd = kPipeThreads / 256 * kPipePerCU;

// workgroup barrier ordering LDS accesses only: the next head's global loads stay in flight
__device__ __forceinline__ void pipe_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename Tin, typename Tout>
__global__ void __launch_bounds__(kPipeThreads) __attribute__((amdgpu_waves_per_eu(kPipeWavesPerSimd, kPipeWavesPerSimd)))
decode_pipe_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
                   const float* __restrict__ g, const float* __restrict__ beta, float* state,
                   Tout* __restrict__ y, int heads) {
    constexpr int DK = 128, DV = 128;
    constexpr int TPR = DV / 4;               // threads per state row (4 columns each)
    constexpr int RG = kPipeThreads / TPR;    // row groups
    constexpr int RPT = DK / RG;              // rows per thread
    constexpr int NW = kPipeThreads / kWave;
    __shared__ float ks[2][DK], qs[2][DK];
    __shared__ float red[2][NW][2][DV];   // per-wave partial S^T k, S^T q
    __shared__ float fin[2][2][DV];       // their sums over the waves

    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int c = (tid % TPR) * 4;
    const int rg = tid / TPR;
    const int ek = min(tid, 2 * DK - 1);   // threads 0..255: one element of k (then q)

    struct Head {
        float s[RPT][4];
        float vv[4];
        Tin kq;
        float g, b;
    };
    // all of a head's loads, issued together and unconditionally
    auto load = [&](int head, Head& H) __attribute__((always_inline)) {
        H.kq = ((ek < DK ? k : q) + (size_t)head * DK)[ek < DK ? ek : ek - DK];
        Vec4<Tin>::load(v + (size_t)head * DV + c, H.vv);
        H.g = g[head];
        H.b = beta[head];
        const float* S = state + (size_t)head * DK * DV;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const floatx4 t = __builtin_nontemporal_load(
                reinterpret_cast<const floatx4*>(S + (size_t)(RPT * rg + i) * DV + c));
            H.s[i][0] = t.x; H.s[i][1] = t.y; H.s[i][2] = t.z; H.s[i][3] = t.w;
        }
    };
    // the step for one head whose loads were issued earlier; p selects the LDS buffers
    auto process = [&](int head, int p, const Head& H) __attribute__((always_inline)) {
        if (tid < DK) ks[p][tid] = load1(&H.kq);
        else if (tid < 2 * DK) qs[p][tid - DK] = load1(&H.kq);
        const float a = expf(H.g);
        const float b = H.b;
        pipe_barrier();
        float kq = 0.f;
#pragma unroll
        for (int i = lane; i < DK; i += kWave) kq += ks[p][i] * qs[p][i];
        kq = group_sum<kWave>(kq);
        float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float kr = ks[p][RPT * rg + i], qr = qs[p][RPT * rg + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pk[j] += H.s[i][j] * kr;
                pq[j] += H.s[i][j] * qr;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pk[j] = sum_across<TPR>(pk[j]);
            pq[j] = sum_across<TPR>(pq[j]);
        }
        if (lane < TPR) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                red[p][wave][0][c + j] = pk[j];
                red[p][wave][1][c + j] = pq[j];
            }
        }
        pipe_barrier();
        if (tid < 2 * DV) {   // one (column, S^T k | S^T q) sum per thread, waves in order
            const int col = tid % DV, which = tid / DV;
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) t += red[p][w][which][col];
            fin[p][which][col] = t;
        }
        pipe_barrier();
        float e[4], yo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float sk = fin[p][0][c + j], sq = fin[p][1][c + j];
            e[j] = H.vv[j] - a * sk;
            yo[j] = a * sq + b * kq * e[j];
        }
        float* S = state + (size_t)head * DK * DV;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float bk = b * ks[p][RPT * rg + i];
            floatx4 t;
            t.x = a * H.s[i][0] + bk * e[0];
            t.y = a * H.s[i][1] + bk * e[1];
            t.z = a * H.s[i][2] + bk * e[2];
            t.w = a * H.s[i][3] + bk * e[3];
            __builtin_nontemporal_store(t, reinterpret_cast<floatx4*>(S + (size_t)(RPT * rg + i) * DV + c));
        }
        if (rg == 0) Vec4<Tout>::store(y + (size_t)head * DV + c, yo);
    };

    const int G = gridDim.x;
    const int h0 = blockIdx.x;
    if (h0 >= heads) return;
    const int n = (heads - h0 + G - 1) / G;
    Head A, B;
    load(h0, A);
    int j = 0;
    for (; j + 2 < n; j += 2) {
        load(h0 + (j + 1) * G, B);
        process(h0 + j * G, 0, A);
        load(h0 + (j + 2) * G, A);
        process(h0 + (j + 1) * G, 1, B);
    }
    if (j + 1 < n) {
        load(h0 + (j + 1) * G, B);
        process(h0 + j * G, 0, A);
        process(h0 + (j + 1) * G, 1, B);
    } else {
        process(h0 + j * G, 0, A);
    }
}

// ----------------------------------------------------------------------------------------
// The whole decode step of the token mixer in one kernel: eqs. (6)-(10) on this step's
// projected inputs with the carried conv history (depthwise width-4 conv -> SiLU -> L2Norm
// for q and k, conv -> SiLU for v, the per-head gates), then the single-token update above,
// then eq. (11) without W_o (o = sigmoid(z) (1 + w) y / rms(y) over the dv channels).
// The state pass is the same as decode_kernel's; the extra bytes (history, x, z, o) are about
// 3% of the state's, and the front end runs while the state loads are in flight. q and k stay
// fp32 (never rounded to bf16 between steps); their L2 norms are folded into the products.
template <int DK, int DV, typename Tin, typename Tout>
__global__ void __launch_bounds__(kDecThreads) decode_fused_kernel(DecodeFusedArgs f) {
    constexpr int TPR = DV / 4;
    constexpr int RG = kDecThreads / TPR;
    constexpr int RPT = DK / RG;
    constexpr int NW = kDecThreads / kWave;
    static_assert(RPT >= 1 && DK % RG == 0, "shape");

    __shared__ float ks[DK], qs[DK], vs[DV];
    __shared__ float red[NW][2][DV];

    const int head = blockIdx.x, H = f.H;
    const int n = head / H, h = head % H;
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int c = (tid % TPR) * 4;
    const int rg = tid / TPR;

    // The token's loads (inputs, conv history and taps, z) are issued first and unconditionally
    // (channel indices clamped; a load under a branch is waited for at the join), then the
    // state's: the conv and the L2 norms run while the state is still arriving.
    constexpr int NCH = 2 * DK + DV;                                  // q | k | v channels
    constexpr int CPT = (NCH + kDecThreads - 1) / kDecThreads;        // channels per thread
    Tin* hist = static_cast<Tin*>(f.conv_state) + (size_t)n * 3 * f.hC;
    Tin xin[CPT], hv[CPT][3];
    float4 wv[CPT];
    int hcs[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int ch = min(tid + u * kDecThreads, NCH - 1);
        const int role = ch < DK ? 0 : (ch < 2 * DK ? 1 : 2);
        const int cl = ch - (role == 0 ? 0 : (role == 1 ? DK : 2 * DK));
        const int d = role < 2 ? DK : DV;
        const int cs = h * d + cl;                                   // channel in its stream
        const int hc = (role == 0 ? 0 : (role == 1 ? H * DK : 2 * H * DK)) + cs;
        hcs[u] = hc;
        // stream pointers selected from the (scalar) arguments, not indexed per lane
        const Tin* xs = static_cast<const Tin*>(role == 0 ? f.x[0] : (role == 1 ? f.x[1] : f.x[2]));
        const float* ws = role == 0 ? f.w[0] : (role == 1 ? f.w[1] : f.w[2]);
        xin[u] = xs[(size_t)n * H * d + cs];
        hv[u][0] = hist[hc];
        hv[u][1] = hist[f.hC + hc];
        hv[u][2] = hist[2 * f.hC + hc];
        wv[u] = reinterpret_cast<const float4*>(ws)[cs];
    }
    float zv[4];
    Vec4<Tin>::load(static_cast<const Tin*>(f.z) + (size_t)head * DV + c, zv);
    __builtin_amdgcn_sched_barrier(0);
    float* S = f.state + (size_t)head * DK * DV;
    float s[RPT][4];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const floatx4 t = __builtin_nontemporal_load(
            reinterpret_cast<const floatx4*>(S + (size_t)(rg + RG * i) * DV + c));
        s[i][0] = t.x; s[i][1] = t.y; s[i][2] = t.z; s[i][3] = t.w;
    }
    __builtin_amdgcn_sched_barrier(0);

    // conv over [history rows 0..2, x]; the history shifts by one token in place (each
    // channel's four values are touched by this thread only)
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int ch = tid + u * kDecThreads;
        if (ch < NCH) {
            const int role = ch < DK ? 0 : (ch < 2 * DK ? 1 : 2);
            const int cl = ch - (role == 0 ? 0 : (role == 1 ? DK : 2 * DK));
            const float4 w = wv[u];
            const float cu = conv4(w.x, w.y, w.z, w.w, load1(&hv[u][0]), load1(&hv[u][1]),
                                   load1(&hv[u][2]), load1(&xin[u]));
            hist[hcs[u]] = hv[u][1];
            hist[f.hC + hcs[u]] = hv[u][2];
            hist[2 * f.hC + hcs[u]] = xin[u];
            const float act = siluf_(cu);
            if (role == 0) qs[cl] = act;
            else if (role == 1) ks[cl] = act;
            else vs[cl] = act;
        }
    }
    const float a = expf(gate_g(f.A_log[h], f.a_raw[head], f.dt_bias[h]));
    const float b = gate_beta(f.b_raw[head]);
    __syncthreads();

    // L2 norms of q and k and the raw k.q (every wave, no extra barrier)
    float nq = 0.f, nk = 0.f, kq = 0.f;
#pragma unroll
    for (int i = lane; i < DK; i += kWave) {
        nq += qs[i] * qs[i];
        nk += ks[i] * ks[i];
        kq += ks[i] * qs[i];
    }
    nq = group_sum<kWave>(nq);
    nk = group_sum<kWave>(nk);
    kq = group_sum<kWave>(kq);
    const float iq = frsq(nq + f.l2_eps), ik = frsq(nk + f.l2_eps);
    kq *= iq * ik;

    float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kr = ks[rg + RG * i], qr = qs[rg + RG * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pk[j] += s[i][j] * kr;
            pq[j] += s[i][j] * qr;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        pk[j] = sum_across<TPR>(pk[j]);
        pq[j] = sum_across<TPR>(pq[j]);
    }
    if (lane < TPR) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            red[wave][0][c + j] = pk[j];
            red[wave][1][c + j] = pq[j];
        }
    }
    __syncthreads();
    float e[4], yo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            sk += red[w][0][c + j];
            sq += red[w][1][c + j];
        }
        e[j] = vs[c + j] - a * (sk * ik);
        yo[j] = a * (sq * iq) + b * kq * e[j];
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float bk = b * ik * ks[rg + RG * i];
        floatx4 t;
        t.x = a * s[i][0] + bk * e[0];
        t.y = a * s[i][1] + bk * e[1];
        t.z = a * s[i][2] + bk * e[2];
        t.w = a * s[i][3] + bk * e[3];
        __builtin_nontemporal_store(t, reinterpret_cast<floatx4*>(S + (size_t)(rg + RG * i) * DV + c));
    }
    if (rg == 0) {   // the TPR lanes of row group 0 (an aligned group of wave 0) hold all of y
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) ss += yo[j] * yo[j];
        ss = group_sum<TPR>(ss);
        const float inv = frsq(ss * (1.0f / DV) + f.rms_eps);
        float ov[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = sigmoidf_(zv[j]) * ((1.0f + f.norm_w[c + j]) * (yo[j] * inv));
        Vec4<Tout>::store(static_cast<Tout*>(f.o) + (size_t)head * DV + c, ov);
        if (f.y) Vec4<Tout>::store(static_cast<Tout*>(f.y) + (size_t)head * DV + c, yo);
    }
}

// ----------------------------------------------------------------------------------------
// Persistent form of decode_fused_kernel for d_k = d_v = 128, as decode_pipe_kernel is of
// decode_kernel: one 1024-thread workgroup per CU walks heads blockIdx.x, + gridDim.x, ...
// with the next head's inputs, history, taps, z, gate scalars and state loaded (unconditionally,
// channel indices clamped) before the current head's conv, reductions and stores. A head's
// conv history channels are its own, so the next head's history reads and this head's
// in-place history writes touch different elements. Per element the arithmetic is
// decode_fused_kernel's; the sums over state rows are grouped as in decode_pipe_kernel.
// N=256 H=32: 184-187 us per step against 197-202 for one workgroup per head.
template <typename Tin, typename Tout>
__global__ void __launch_bounds__(kPipeThreads) __attribute__((amdgpu_waves_per_eu(kPipeWavesPerSimd, kPipeWavesPerSimd)))
decode_fused_pipe_kernel(DecodeFusedArgs f) {
    constexpr int DK = 128, DV = 128;
    constexpr int TPR = DV / 4;
    constexpr int RG = kPipeThreads / TPR;
    constexpr int RPT = DK / RG;
    constexpr int NW = kPipeThreads / kWave;
    constexpr int NCH = 2 * DK + DV;   // q | k | v channels, one per thread
    static_assert(NCH <= kPipeThreads, "one channel per thread");
    __shared__ float ks[2][DK], qs[2][DK], vs[2][DV];
    __shared__ float red[2][NW][2][DV];
    __shared__ float fin[2][2][DV];

    const int H = f.H, heads = f.N * f.H;
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int c = (tid % TPR) * 4;
    const int rg = tid / TPR;
    const int ch = min(tid, NCH - 1);
    const int role = ch < DK ? 0 : (ch < 2 * DK ? 1 : 2);
    const int cl = ch - (role == 0 ? 0 : (role == 1 ? DK : 2 * DK));
    const int dr = role < 2 ? DK : DV;
    const Tin* xs = static_cast<const Tin*>(role == 0 ? f.x[0] : (role == 1 ? f.x[1] : f.x[2]));
    const float* ws = role == 0 ? f.w[0] : (role == 1 ? f.w[1] : f.w[2]);
    const int hoff = role == 0 ? 0 : (role == 1 ? H * DK : 2 * H * DK);

    struct Head {
        float s[RPT][4];
        float zv[4];
        float4 wv;
        Tin xin, hv[3];
        float ar, br, Al, db;
    };
    auto load = [&](int head, Head& X) __attribute__((always_inline)) {
        const int n = head / H, h = head % H;
        const int cs = h * dr + cl, hc = hoff + cs;
        const Tin* hist = static_cast<const Tin*>(f.conv_state) + (size_t)n * 3 * f.hC;
        X.xin = xs[(size_t)n * H * dr + cs];
        X.hv[0] = hist[hc];
        X.hv[1] = hist[f.hC + hc];
        X.hv[2] = hist[2 * f.hC + hc];
        X.wv = reinterpret_cast<const float4*>(ws)[cs];
        Vec4<Tin>::load(static_cast<const Tin*>(f.z) + (size_t)head * DV + c, X.zv);
        X.ar = f.a_raw[head];
        X.br = f.b_raw[head];
        X.Al = f.A_log[h];
        X.db = f.dt_bias[h];
        const float* S = f.state + (size_t)head * DK * DV;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const floatx4 t = __builtin_nontemporal_load(
                reinterpret_cast<const floatx4*>(S + (size_t)(RPT * rg + i) * DV + c));
            X.s[i][0] = t.x; X.s[i][1] = t.y; X.s[i][2] = t.z; X.s[i][3] = t.w;
        }
    };
    auto process = [&](int head, int p, const Head& X) __attribute__((always_inline)) {
        const int n = head / H, h = head % H;
        if (tid < NCH) {   // conv over [history rows 0..2, x]; the history shifts in place
            Tin* hist = static_cast<Tin*>(f.conv_state) + (size_t)n * 3 * f.hC;
            const int hc = hoff + h * dr + cl;
            const float cu = conv4(X.wv.x, X.wv.y, X.wv.z, X.wv.w, load1(&X.hv[0]), load1(&X.hv[1]),
                                   load1(&X.hv[2]), load1(&X.xin));
            hist[hc] = X.hv[1];
            hist[f.hC + hc] = X.hv[2];
            hist[2 * f.hC + hc] = X.xin;
            const float act = siluf_(cu);
            if (role == 0) qs[p][cl] = act;
            else if (role == 1) ks[p][cl] = act;
            else vs[p][cl] = act;
        }
        const float a = expf(gate_g(X.Al, X.ar, X.db));
        const float b = gate_beta(X.br);
        pipe_barrier();
        float nq = 0.f, nk = 0.f, kq = 0.f;
#pragma unroll
        for (int i = lane; i < DK; i += kWave) {
            nq += qs[p][i] * qs[p][i];
            nk += ks[p][i] * ks[p][i];
            kq += ks[p][i] * qs[p][i];
        }
        nq = group_sum<kWave>(nq);
        nk = group_sum<kWave>(nk);
        kq = group_sum<kWave>(kq);
        const float iq = frsq(nq + f.l2_eps), ik = frsq(nk + f.l2_eps);
        kq *= iq * ik;
        float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float kr = ks[p][RPT * rg + i], qr = qs[p][RPT * rg + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pk[j] += X.s[i][j] * kr;
                pq[j] += X.s[i][j] * qr;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pk[j] = sum_across<TPR>(pk[j]);
            pq[j] = sum_across<TPR>(pq[j]);
        }
        if (lane < TPR) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                red[p][wave][0][c + j] = pk[j];
                red[p][wave][1][c + j] = pq[j];
            }
        }
        pipe_barrier();
        if (tid < 2 * DV) {
            const int col = tid % DV, which = tid / DV;
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) t += red[p][w][which][col];
            fin[p][which][col] = t;
        }
        pipe_barrier();
        float e[4], yo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            e[j] = vs[p][c + j] - a * (fin[p][0][c + j] * ik);
            yo[j] = a * (fin[p][1][c + j] * iq) + b * kq * e[j];
        }
        float* S = f.state + (size_t)head * DK * DV;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float bk = b * ik * ks[p][RPT * rg + i];
            floatx4 t;
            t.x = a * X.s[i][0] + bk * e[0];
            t.y = a * X.s[i][1] + bk * e[1];
            t.z = a * X.s[i][2] + bk * e[2];
            t.w = a * X.s[i][3] + bk * e[3];
            __builtin_nontemporal_store(t, reinterpret_cast<floatx4*>(S + (size_t)(RPT * rg + i) * DV + c));
        }
        if (rg == 0) {   // the TPR lanes of row group 0 hold all of y
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) ss += yo[j] * yo[j];
            ss = group_sum<TPR>(ss);
            const float inv = frsq(ss * (1.0f / DV) + f.rms_eps);
            float ov[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) ov[j] = sigmoidf_(X.zv[j]) * ((1.0f + f.norm_w[c + j]) * (yo[j] * inv));
            Vec4<Tout>::store(static_cast<Tout*>(f.o) + (size_t)head * DV + c, ov);
            if (f.y) Vec4<Tout>::store(static_cast<Tout*>(f.y) + (size_t)head * DV + c, yo);
        }
    };

    const int G = gridDim.x;
    const int h0 = blockIdx.x;
    if (h0 >= heads) return;
    const int cnt = (heads - h0 + G - 1) / G;
    Head A, B;
    load(h0, A);
    int j = 0;
    for (; j + 2 < cnt; j += 2) {
        load(h0 + (j + 1) * G, B);
        process(h0 + j * G, 0, A);
        load(h0 + (j + 2) * G, A);
        process(h0 + (j + 1) * G, 1, B);
    }
    if (j + 1 < cnt) {
        load(h0 + (j + 1) * G, B);
        process(h0 + j * G, 0, A);
        process(h0 + (j + 1) * G, 1, B);
    } else {
        process(h0 + j * G, 0, A);
    }
}

// ----------------------------------------------------------------------------------------
// T consecutive tokens per sequence in one pass over the state: the chunkwise form of eq. (5)
// with the chunk being the T new tokens. With G_t = g_1 + ... + g_t (g = log alpha) and
// sk_t = S^T k_t, sq_t = S^T q_t of the state S the call starts from:
//   U_t = beta_t (v_t - e^{G_t} sk_t) - sum_{i<t} beta_t e^{G_t - G_i} (k_t.k_i) U_i
//   y_t = e^{G_t} sq_t + sum_{i<=t} e^{G_t - G_i} (q_t.k_i) U_i
//   S_t = e^{G_t} S + sum_{i<=t} e^{G_t - G_i} k_i U_i^T
// (U_t = beta_t e_t of eqs. (2)-(3); expanding eqs. (1)-(4) token by token gives these
// sums). All 2T column reductions run against the one state in registers, so the state is
// read once and written once however many tokens the step carries. Decays are exp of
// differences of the running sum (never above 1).
// One workgroup per state: 512 threads (two per CU) for T <= 4, 256 (one wave per SIMD) for
// T = 8, whose per-token arrays need the registers; a thread holds dk / (threads / (dv / 4))
// contiguous rows of 4 columns, as the single-token kernel's threads do. Measured at N = 256,
// H = 32 (us per step, 256 / 512 threads): T = 4 219 / 214, T = 8 386 / 501. Column sums: in
// registers over a thread's rows, across the wave's row groups by VALU lane exchanges, then
// once per (value, column) across the waves in LDS. kDecColSplit > 1 would give each
// workgroup 1/kDecColSplit of the columns (a column's sums and update need only that column);
// measured slower at split 2 (the per-workgroup token work is repeated and each workgroup
// moves half the bytes). The fused variant uses 512-thread workgroups at every T: its front
// end has 2 dk + dv channels to convolve, one per thread.
template <bool kFused, int kMaxDecT> constexpr int dm_threads() {
    return (kFused || kMaxDecT <= 4) ? 512 : 256;
}
template <bool kFused, int kMaxDecT> constexpr int dm_min_waves() {
    return kMaxDecT <= 4 ? 4 : 2;
}
constexpr int kDecColSplit = 1;

// With kFused the step starts from the projected streams instead of q, k, v, g, beta: one
// thread per channel runs the width-4 conv over the carried history and the T new inputs
// (SiLU; the history moves on by T inputs), the gates come from a_raw, b_raw, the L2 norms of
// q_t, k_t are applied in LDS, and the output gate runs after the state pass (the TPR lanes of
// the first row group hold all of y_t, parked in LDS meanwhile) instead of storing y.
struct MultiArgs {
    const void *q, *k, *v;                 // [N, T, H, d] (unfused)
    const float *g, *beta;                 // [N, T, H] (unfused)
    const void* x[3];                      // xq, xk, xv [N, T, H, d] (fused)
    const float* w[3];                     // conv taps [H*d, 4]
    const void* hin;                       // conv history in [N, 3, hC], x dtype
    void* hout;                            // conv history out (may equal hin)
    int hC;
    const float *a_raw, *b_raw, *A_log, *dt_bias;
    float l2_eps;
    const void* z;                         // [N, T, H, dv], x dtype
    const float* norm_w;
    float rms_eps;
    void* o;                               // [N, T, H, dv] (fused)
    float* state;
    void* y;                               // [N, T, H, dv]; nullable when fused
    float* steps;                          // nullable
    int T, H;
};

// kMaxDecT (2, 4 or 8) bounds T at compile time: the per-token register arrays are sized by
// it, so a short step does not pay the registers (and occupancy) of the longest one.
template <int DK, int DV, int kMaxDecT, typename Tin, typename Tout, bool kFused>
__global__ void __launch_bounds__((dm_threads<kFused, kMaxDecT>()), (dm_min_waves<kFused, kMaxDecT>()))
decode_multi_kernel(MultiArgs m) {
    const Tin* __restrict__ q = static_cast<const Tin*>(m.q);
    const Tin* __restrict__ k = static_cast<const Tin*>(m.k);
    const Tin* __restrict__ v = static_cast<const Tin*>(m.v);
    Tout* __restrict__ y = static_cast<Tout*>(m.y);
    float* state = m.state;
    float* __restrict__ steps = m.steps;
    const int T = m.T, H = m.H;
    constexpr int DVS = DV / kDecColSplit;       // columns of this workgroup
    constexpr int TPR = DVS / 4;                 // threads per state row
    constexpr int kDecMultiThreads = dm_threads<kFused, kMaxDecT>();
    constexpr int RG = kDecMultiThreads / TPR;   // row groups
    constexpr int RPT = DK / RG;                 // contiguous rows per thread
    constexpr int NW = kDecMultiThreads / kWave;
    constexpr int NV = 2 * kMaxDecT;             // column sums per token pair: S^T k_t, S^T q_t
    static_assert(RPT >= 1 && DK % RG == 0 && TPR <= kWave, "shape");

    __shared__ __attribute__((aligned(16))) float ks[kMaxDecT][DK];
    __shared__ __attribute__((aligned(16))) float qs[kMaxDecT][DK];
    __shared__ __attribute__((aligned(16))) float red[NW][NV][DVS];  // per-wave column partials
    __shared__ __attribute__((aligned(16))) float fin[NV][DVS];      // column sums
    // token-pair scalars: A[t][i] = beta_t e^{G_t-G_i} k_t.k_i (i < t),
    // P[t][i] = e^{G_t-G_i} q_t.k_i (i <= t), D[t][i] = e^{G_t-G_i} (i <= t)
    __shared__ float Am[kMaxDecT][kMaxDecT], Pm[kMaxDecT][kMaxDecT], Dm[kMaxDecT][kMaxDecT];
    __shared__ float Gs[kMaxDecT], Bs[kMaxDecT];   // G_t and beta_t
    __shared__ __attribute__((aligned(16))) float vs[kFused ? kMaxDecT : 1][kFused ? DV : 4];
    __shared__ __attribute__((aligned(16))) float zs[kFused ? kMaxDecT : 1][kFused ? DV : 4];
    __shared__ float gl[kMaxDecT];

    const int head = blockIdx.x / kDecColSplit;   // flattened (sequence, head)
    const int n = head / H, h = head % H;
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int cl = (tid % TPR) * 4;               // column within this workgroup's half
    const int c = (blockIdx.x % kDecColSplit) * DVS + cl;
    const int r0 = (tid / TPR) * RPT;             // first of this thread's rows
    auto tok = [&](int t) { return (size_t)(n * T + t) * H + h; };   // (token, head) row

    float* S = state + (size_t)head * DK * DV;
    float s[RPT][4];
    // The state's loads follow the tokens': the token-pair products need only q and k, so they
    // run while the state is still arriving (the vector-memory counter completes loads in
    // issue order, so loads issued before the state's can be waited for alone).
    auto load_state = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const floatx4 x = __builtin_nontemporal_load(
                reinterpret_cast<const floatx4*>(S + (size_t)(r0 + i) * DV + c));
            s[i][0] = x.x; s[i][1] = x.y; s[i][2] = x.z; s[i][3] = x.w;
        }
    };
    float vv[kMaxDecT][4];
    if constexpr (!kFused) {
        // every token load is issued before any is used, unconditionally (tokens past T read
        // token T - 1 and are dropped): a load under a branch is waited for at the join
        constexpr int KQ = (kMaxDecT * DK + kDecMultiThreads - 1) / kDecMultiThreads;
        float kr[KQ], qr[KQ], gv[kMaxDecT], bv[kMaxDecT];
#pragma unroll
        for (int u = 0; u < KQ; ++u) {
            const int i = tid + u * kDecMultiThreads, t = min(i / DK, T - 1), r = i % DK;
            kr[u] = load1(k + tok(t) * DK + r);
            qr[u] = load1(q + tok(t) * DK + r);
        }
#pragma unroll
        for (int t = 0; t < kMaxDecT; ++t) {
            const int tc = min(t, T - 1);
            Vec4<Tin>::load(v + tok(tc) * DV + c, vv[t]);
            gv[t] = m.g[tok(tc)];
            bv[t] = m.beta[tok(tc)];
        }
        __builtin_amdgcn_sched_barrier(0);
        load_state();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < KQ; ++u) {
            const int i = tid + u * kDecMultiThreads, t = i / DK, r = i % DK;
            if (t < T) {
                ks[t][r] = kr[u];
                qs[t][r] = qr[u];
            }
        }
        if (tid == 0) {
            float run = 0.f;
#pragma unroll
            for (int t = 0; t < kMaxDecT; ++t)
                if (t < T) {
                    run += gv[t];
                    Gs[t] = run;
                    Bs[t] = bv[t];
                }
        }
        __syncthreads();
    } else {
        // conv over [history rows 0..2, x_0 .. x_{T-1}], one channel (of q | k | v) per thread.
        // Every load of the step's inputs is issued first and unconditionally (indices clamped;
        // a load under a branch is waited for at the join), then the state's, then the conv
        // and the gates run while the state arrives.
        static_assert(2 * DK + DV <= kDecMultiThreads, "one channel per thread");
        constexpr int ZPT = (kMaxDecT * DV + kDecMultiThreads - 1) / kDecMultiThreads;
        const Tin* hin = static_cast<const Tin*>(m.hin) + (size_t)n * 3 * m.hC;
        Tin* hout = static_cast<Tin*>(m.hout) + (size_t)n * 3 * m.hC;
        const int ch = min(tid, 2 * DK + DV - 1);
        const int role = ch < DK ? 0 : (ch < 2 * DK ? 1 : 2);
        const int cl2 = ch - (role == 0 ? 0 : (role == 1 ? DK : 2 * DK));
        const int d = role < 2 ? DK : DV;
        const int cs = h * d + cl2;
        const int hc = (role == 0 ? 0 : (role == 1 ? H * DK : 2 * H * DK)) + cs;
        // stream pointers selected from the (scalar) arguments, not indexed per lane
        const Tin* xs = static_cast<const Tin*>(role == 0 ? m.x[0] : (role == 1 ? m.x[1] : m.x[2]));
        const float* ws = role == 0 ? m.w[0] : (role == 1 ? m.w[1] : m.w[2]);
        const float4 w = reinterpret_cast<const float4*>(ws)[cs];
        Tin buf[3 + kMaxDecT];   // history then the new inputs, raw
        buf[0] = hin[hc];
        buf[1] = hin[m.hC + hc];
        buf[2] = hin[2 * m.hC + hc];
#pragma unroll
        for (int t = 0; t < kMaxDecT; ++t) buf[3 + t] = xs[tok(min(t, T - 1)) * d + cl2];
        Tin zr[ZPT];
#pragma unroll
        for (int u = 0; u < ZPT; ++u) {
            const int e = min(tid + u * kDecMultiThreads, T * DV - 1);
            zr[u] = static_cast<const Tin*>(m.z)[tok(e / DV) * DV + e % DV];
        }
        const int tg = min(tid, T - 1);
        const float ar = m.a_raw[tok(tg)], br = m.b_raw[tok(tg)];
        __builtin_amdgcn_sched_barrier(0);
        load_state();
        __builtin_amdgcn_sched_barrier(0);
        if (tid < 2 * DK + DV) {
            float* dst = role == 0 ? &qs[0][0] : (role == 1 ? &ks[0][0] : &vs[0][0]);
            const int stride = role < 2 ? DK : DV;
#pragma unroll
            for (int t = 0; t < kMaxDecT; ++t)
                if (t < T)
                    dst[t * stride + cl2] = siluf_(conv4(w.x, w.y, w.z, w.w, load1(&buf[t]),
                                                         load1(&buf[t + 1]), load1(&buf[t + 2]),
                                                         load1(&buf[t + 3])));
            // the next history: the last 3 of the T + 3 inputs (read above, so in place is safe)
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                Tin nv = buf[j];
#pragma unroll
                for (int t = 1; t <= kMaxDecT; ++t)
                    if (t == T) nv = buf[j + t];
                hout[j * m.hC + hc] = nv;
            }
        }
        // gates: thread t forms token t's; z comes in now for the epilogue's output gate
        if (tid < T) {
            gl[tid] = gate_g(m.A_log[h], ar, m.dt_bias[h]);
            Bs[tid] = gate_beta(br);
        }
#pragma unroll
        for (int u = 0; u < ZPT; ++u) {
            const int e = tid + u * kDecMultiThreads;
            if (e < T * DV) zs[e / DV][e % DV] = load1(&zr[u]);
        }
        __syncthreads();
        if (tid == 0) {
            float run = 0.f;
            for (int t = 0; t < T; ++t) {
                run += gl[t];
                Gs[t] = run;
            }
        }
        // L2Norm of q_t and k_t in place, one token per wave
        for (int t = wave; t < T; t += NW) {
            float nq = 0.f, nk = 0.f;
            for (int r = lane; r < DK; r += kWave) {
                nq += qs[t][r] * qs[t][r];
                nk += ks[t][r] * ks[t][r];
            }
            nq = group_sum<kWave>(nq);
            nk = group_sum<kWave>(nk);
            const float iq = frsq(nq + m.l2_eps), ik = frsq(nk + m.l2_eps);
            for (int r = lane; r < DK; r += kWave) {
                qs[t][r] *= iq;
                ks[t][r] *= ik;
            }
        }
#pragma unroll
        for (int t = 0; t < kMaxDecT; ++t)
            if (t < T)
#pragma unroll
                for (int j = 0; j < 4; ++j) vv[t][j] = vs[t][c + j];
        __syncthreads();
    }

    // rows r0+i0 .. r0+i0+3 of a token vector (LDS; one 16-byte read when they fit)
    auto row4 = [&](const float* vec, int i0, float (&out)[4]) __attribute__((always_inline)) {
        if constexpr (RPT % 4 == 0) {
            const floatx4 x = *reinterpret_cast<const floatx4*>(vec + r0 + i0);
            out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = i0 + i < RPT ? vec[r0 + i0 + i] : 0.f;
        }
    };

    // token-pair scalars, one pair per wave in turn
    for (int p = wave; p < T * T; p += NW) {
        const int t = p / T, i = p % T;
        if (i > t) continue;   // wave-uniform
        float kk = 0.f, qk = 0.f;
        for (int r = lane; r < DK; r += kWave) {
            kk += ks[t][r] * ks[i][r];
            qk += qs[t][r] * ks[i][r];
        }
        kk = group_sum<kWave>(kk);
        qk = group_sum<kWave>(qk);
        if (lane == 0) {
            const float d = expf(Gs[t] - Gs[i]);
            Dm[t][i] = d;
            Pm[t][i] = d * qk;
            Am[t][i] = i < t ? Bs[t] * d * kk : 0.f;
        }
    }

    // column partials of S^T k_t and S^T q_t over this thread's rows, then over the wave's
    // row groups (lanes TPR apart); lanes of the first row group write the wave's partial
#pragma unroll
    for (int t = 0; t < kMaxDecT; ++t) {
        if (t < T) {
            float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i0 = 0; i0 < RPT; i0 += 4) {   // 4 rows of k_t and q_t at a time
                float kr[4], qr[4];
                row4(ks[t], i0, kr);
                row4(qs[t], i0, qr);
#pragma unroll
                for (int i = 0; i < 4 && i0 + i < RPT; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pk[j] += s[i0 + i][j] * kr[i];
                        pq[j] += s[i0 + i][j] * qr[i];
                    }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pk[j] = sum_across<TPR>(pk[j]);
                pq[j] = sum_across<TPR>(pq[j]);
            }
            if (lane < TPR) {
                *reinterpret_cast<floatx4*>(&red[wave][2 * t][cl]) = floatx4{pk[0], pk[1], pk[2], pk[3]};
                *reinterpret_cast<floatx4*>(&red[wave][2 * t + 1][cl]) = floatx4{pq[0], pq[1], pq[2], pq[3]};
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < 2 * T * DVS; e += kDecMultiThreads) {   // across the waves, once
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += (&red[w][0][0])[e];
        (&fin[0][0])[e] = acc;
    }
    __syncthreads();

    // U_t and y_t for this thread's 4 columns (every row group forms them; the first stores y)
    float U[kMaxDecT][4];
#pragma unroll
    for (int t = 0; t < kMaxDecT; ++t) {
        if (t < T) {
            const float gt = expf(Gs[t]), bt = Bs[t];
            const floatx4 sk = *reinterpret_cast<const floatx4*>(&fin[2 * t][cl]);
            const floatx4 sq = *reinterpret_cast<const floatx4*>(&fin[2 * t + 1][cl]);
            float yo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float u = bt * (vv[t][j] - gt * sk[j]);
#pragma unroll
                for (int i = 0; i < kMaxDecT; ++i)
                    if (i < t) u -= Am[t][i] * U[i][j];
                U[t][j] = u;
                float yv = gt * sq[j];
#pragma unroll
                for (int i = 0; i < kMaxDecT; ++i)
                    if (i <= t) yv += Pm[t][i] * U[i][j];
                yo[j] = yv;
            }
            if constexpr (!kFused) {
                if (r0 == 0) Vec4<Tout>::store(y + tok(t) * DV + c, yo);
            } else if (r0 == 0) {   // parked in this thread's own slots of vs (v_t is in vv now)
                *reinterpret_cast<floatx4*>(&vs[t][c]) = floatx4{yo[0], yo[1], yo[2], yo[3]};
            }
        }
    }

    // S_t = e^{G_t} S + sum_{i<=t} e^{G_t-G_i} k_i U_i^T: every step's state when asked for,
    // the last one in place
    // Four rows at a time, so only a 4 x 4 block of the new state is live beside the old one.
    auto state_at = [&](int t, float* dst) __attribute__((always_inline)) {
        const float gt = expf(Gs[t]);
#pragma unroll
        for (int rb = 0; rb < RPT; rb += 4) {
            float o[4][4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) o[r][j] = rb + r < RPT ? gt * s[rb + r][j] : 0.f;
#pragma unroll
            for (int i = 0; i < kMaxDecT; ++i) {
                if (i <= t) {
                    const float d = Dm[t][i];
                    float kr[4];
                    row4(ks[i], rb, kr);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float dk = d * kr[r];
#pragma unroll
                        for (int j = 0; j < 4; ++j) o[r][j] += dk * U[i][j];
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4 && rb + r < RPT; ++r)
                __builtin_nontemporal_store(floatx4{o[r][0], o[r][1], o[r][2], o[r][3]},
                                            reinterpret_cast<floatx4*>(dst + (size_t)(r0 + rb + r) * DV + c));
        }
    };
    if (steps)
        for (int t = 0; t < T; ++t) state_at(t, steps + ((size_t)(n * T + t) * H + h) * DK * DV);
    state_at(T - 1, S);
    if constexpr (kFused) {
        // the output gate, after the state pass (its registers are free by now): the TPR lanes of
        // the first row group (an aligned group of wave 0) hold all DV columns of every y_t
        if (r0 == 0) {
            for (int t = 0; t < T; ++t) {
                const floatx4 yv = *reinterpret_cast<const floatx4*>(&vs[t][c]);
                const float yo[4] = {yv[0], yv[1], yv[2], yv[3]};
                float ss = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) ss += yo[j] * yo[j];
                ss = group_sum<TPR>(ss);
                const float inv = frsq(ss * (1.0f / DV) + m.rms_eps);
                float ov[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ov[j] = sigmoidf_(zs[t][c + j]) * ((1.0f + m.norm_w[c + j]) * (yo[j] * inv));
                Vec4<Tout>::store(static_cast<Tout*>(m.o) + tok(t) * DV + c, ov);
                if (y) Vec4<Tout>::store(y + tok(t) * DV + c, yo);
            }
        }
    }
}

template <int DK, int DV, int MT, bool kFused>
static void launch_dec_multi_t(const MultiArgs& m, int in_bf16, int out_bf16, int heads,
                               hipStream_t s) {
#define GDN_DECM(TI, TO)                                                                        \
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, MT, TI, TO, kFused>),                         \
                       dim3(heads * kDecColSplit), dim3(dm_threads<kFused, MT>()), 0, s, m)
    if (in_bf16 && out_bf16) GDN_DECM(uint16_t, uint16_t);
    else if (in_bf16) GDN_DECM(uint16_t, float);
    else if (out_bf16) GDN_DECM(float, uint16_t);
    else GDN_DECM(float, float);
#undef GDN_DECM
}

template <int DK, int DV, bool kFused>
static void launch_dec_multi(const MultiArgs& m, int in_bf16, int out_bf16, int heads,
                             hipStream_t s) {
    static_assert(kMaxDecodeTokens == 8, "token buckets");
    if (m.T <= 2) launch_dec_multi_t<DK, DV, 2, kFused>(m, in_bf16, out_bf16, heads, s);
    else if (m.T <= 4) launch_dec_multi_t<DK, DV, 4, kFused>(m, in_bf16, out_bf16, heads, s);
    else launch_dec_multi_t<DK, DV, 8, kFused>(m, in_bf16, out_bf16, heads, s);
}

template <bool kFused>
static void launch_dec_multi_shape(const MultiArgs& m, int in_bf16, int out_bf16, int heads,
                                   int dk, int dv, hipStream_t s) {
    if (dk == 128 && dv == 128) launch_dec_multi<128, 128, kFused>(m, in_bf16, out_bf16, heads, s);
    else if (dk == 128 && dv == 64) launch_dec_multi<128, 64, kFused>(m, in_bf16, out_bf16, heads, s);
    else if (dk == 64 && dv == 128) launch_dec_multi<64, 128, kFused>(m, in_bf16, out_bf16, heads, s);
    else launch_dec_multi<64, 64, kFused>(m, in_bf16, out_bf16, heads, s);
}

// compute units of the current device (cached per device)
static int device_cus() {
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

template <int DK, int DV>
static void launch_dec(const void* q, const void* k, const void* v, int in_bf16, const float* g,
                       const float* beta, float* state, int heads, void* y, int y_bf16,
                       hipStream_t s) {
    if constexpr (DK == 128 && DV == 128) {
        const int grid = std::min(heads, kPipePerCU * device_cus());
#define GDN_DECP(TI, TO)                                                                          \
    hipLaunchKernelGGL((decode_pipe_kernel<TI, TO>), dim3(grid), dim3(kPipeThreads), 0, s,        \
                       static_cast<const TI*>(q), static_cast<const TI*>(k),                      \
                       static_cast<const TI*>(v), g, beta, state, static_cast<TO*>(y), heads)
        if (in_bf16 && y_bf16) GDN_DECP(uint16_t, uint16_t);
        else if (in_bf16) GDN_DECP(uint16_t, float);
        else if (y_bf16) GDN_DECP(float, uint16_t);
        else GDN_DECP(float, float);
#undef GDN_DECP
        return;
    }
#define GDN_DEC(TI, TO)                                                                        \
    hipLaunchKernelGGL((decode_kernel<DK, DV, TI, TO>), dim3(heads), dim3(kDecThreads), 0, s,  \
                       static_cast<const TI*>(q), static_cast<const TI*>(k),                   \
                       static_cast<const TI*>(v), g, beta, state, static_cast<TO*>(y))
    if (in_bf16 && y_bf16) GDN_DEC(uint16_t, uint16_t);
    else if (in_bf16) GDN_DEC(uint16_t, float);
    else if (y_bf16) GDN_DEC(float, uint16_t);
    else GDN_DEC(float, float);
#undef GDN_DEC
}

hipError_t launch_decode(const void* q, const void* k, const void* v, int in_bf16, const float* g,
                         const float* beta, float* state, int N, int H, int dk, int dv, void* y,
                         int y_bf16, hipStream_t s) {
    const int heads = N * H;
    if (heads == 0) return hipSuccess;
    if (dk == 128 && dv == 128) launch_dec<128, 128>(q, k, v, in_bf16, g, beta, state, heads, y, y_bf16, s);
    else if (dk == 128 && dv == 64) launch_dec<128, 64>(q, k, v, in_bf16, g, beta, state, heads, y, y_bf16, s);
    else if (dk == 64 && dv == 128) launch_dec<64, 128>(q, k, v, in_bf16, g, beta, state, heads, y, y_bf16, s);
    else launch_dec<64, 64>(q, k, v, in_bf16, g, beta, state, heads, y, y_bf16, s);
    return hipGetLastError();
}

template <int DK, int DV>
static void launch_dec_fused(const DecodeFusedArgs& f, hipStream_t s) {
    if constexpr (DK == 128 && DV == 128) {
        const dim3 pgrid(std::min(f.N * f.H, kPipePerCU * device_cus())), pblock(kPipeThreads);
        if (f.in_bf16 && f.out_bf16)
            hipLaunchKernelGGL((decode_fused_pipe_kernel<uint16_t, uint16_t>), pgrid, pblock, 0, s, f);
        else if (f.in_bf16)
            hipLaunchKernelGGL((decode_fused_pipe_kernel<uint16_t, float>), pgrid, pblock, 0, s, f);
        else if (f.out_bf16)
            hipLaunchKernelGGL((decode_fused_pipe_kernel<float, uint16_t>), pgrid, pblock, 0, s, f);
        else
            hipLaunchKernelGGL((decode_fused_pipe_kernel<float, float>), pgrid, pblock, 0, s, f);
        return;
    }
    const dim3 grid(f.N * f.H), block(kDecThreads);
    if (f.in_bf16 && f.out_bf16)
        hipLaunchKernelGGL((decode_fused_kernel<DK, DV, uint16_t, uint16_t>), grid, block, 0, s, f);
    else if (f.in_bf16)
        hipLaunchKernelGGL((decode_fused_kernel<DK, DV, uint16_t, float>), grid, block, 0, s, f);
    else if (f.out_bf16)
        hipLaunchKernelGGL((decode_fused_kernel<DK, DV, float, uint16_t>), grid, block, 0, s, f);
    else
        hipLaunchKernelGGL((decode_fused_kernel<DK, DV, float, float>), grid, block, 0, s, f);
}

hipError_t launch_decode_fused(const DecodeFusedArgs& f, int dk, int dv, hipStream_t s) {
    if (f.N * f.H == 0) return hipSuccess;
    if (dk == 128 && dv == 128) launch_dec_fused<128, 128>(f, s);
    else if (dk == 128 && dv == 64) launch_dec_fused<128, 64>(f, s);
    else if (dk == 64 && dv == 128) launch_dec_fused<64, 128>(f, s);
    else launch_dec_fused<64, 64>(f, s);
    return hipGetLastError();
}

hipError_t launch_decode_multi(const void* q, const void* k, const void* v, int in_bf16,
                               const float* g, const float* beta, float* state, int N, int T,
                               int H, int dk, int dv, void* y, int y_bf16, float* steps,
                               hipStream_t s) {
    const int heads = N * H;
    if (heads == 0) return hipSuccess;
    MultiArgs m = {};
    m.q = q; m.k = k; m.v = v; m.g = g; m.beta = beta;
    m.state = state; m.y = y; m.steps = steps; m.T = T; m.H = H;
    launch_dec_multi_shape<false>(m, in_bf16, y_bf16, heads, dk, dv, s);
    return hipGetLastError();
}

hipError_t launch_decode_fused_multi(const DecodeFusedArgs& f, const void* hin, int T,
                                     float* steps, int dk, int dv, hipStream_t s) {
    const int heads = f.N * f.H;
    if (heads == 0) return hipSuccess;
    MultiArgs m = {};
    for (int r = 0; r < 3; ++r) {
        m.x[r] = f.x[r];
        m.w[r] = f.w[r];
    }
    m.hin = hin; m.hout = f.conv_state; m.hC = f.hC;
    m.a_raw = f.a_raw; m.b_raw = f.b_raw; m.A_log = f.A_log; m.dt_bias = f.dt_bias;
    m.l2_eps = f.l2_eps;
    m.z = f.z; m.norm_w = f.norm_w; m.rms_eps = f.rms_eps; m.o = f.o;
    m.state = f.state; m.y = f.y; m.steps = steps; m.T = T; m.H = f.H;
    launch_dec_multi_shape<true>(m, f.in_bf16, f.out_bf16, heads, dk, dv, s);
    return hipGetLastError();
}

}  // namespace gdn
