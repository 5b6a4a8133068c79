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

    float* S = state + (size_t)head * DK * DV;
    float s[RPT][4];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const floatx4 t = __builtin_nontemporal_load(
            reinterpret_cast<const floatx4*>(S + (size_t)(rg + RG * i) * DV + c));
        s[i][0] = t.x; s[i][1] = t.y; s[i][2] = t.z; s[i][3] = t.w;
    }
    if (tid < DK) ks[tid] = load1(k + (size_t)head * DK + tid);
    else if (tid < 2 * DK) qs[tid - DK] = load1(q + (size_t)head * DK + tid - DK);
    float vv[4];
    Vec4<Tin>::load(v + (size_t)head * DV + c, vv);
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
    for (int o = TPR; o < kWave; o <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pk[j] += __shfl_xor(pk[j], o, kWave);
            pq[j] += __shfl_xor(pq[j], o, kWave);
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

template <int DK, int DV>
static void launch_dec(const void* q, const void* k, const void* v, int in_bf16, const float* g,
                       const float* beta, float* state, int heads, void* y, int y_bf16,
                       hipStream_t s) {
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

}  // namespace gdn
