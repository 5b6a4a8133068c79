// The unit lower-triangular inverse T = (I + A)^{-1} of a 64x64 chunk matrix on gfx950, shared by
// the chunked kernels. A (strictly lower) is fp32 in LDS, row stride ST floats; it is replaced
// by T in place (upper triangle zero on entry and on exit). One wave computes it, in three
// levels:
//   (1) the four 16x16 diagonal blocks by forward substitution in registers: lane (b, c) owns
//       column c of block b, and the entry A[r][i] it needs is broadcast from lane (b, i) of
//       its 16-lane row by DPP (row_newbcast), so no LDS traffic;
//   (2) 16 -> 32: T_10 = -T_11 (A_10 T_00) for the blocks (1,0) and (3,2), on the fp32
//       matrix cores (v_mfma_f32_16x16x4_f32);
//   (3) 32 -> 64: the same with 32x32 blocks (v_mfma_f32_32x32x2_f32).
// kWaveOnly: the calling wave is alone in this work (its workgroup's other waves wait at a
// later barrier), so the steps are ordered by waiting for its own LDS operations (a wave's
// LDS operations complete in order); otherwise every wave of the workgroup calls it together
// (one matrix each) and the steps are workgroup barriers.
#pragma once
#include "gdn_device.h"

namespace gdn {

typedef float inv_f32x4 __attribute__((ext_vector_type(4)));
typedef float inv_f32x16 __attribute__((ext_vector_type(16)));

template <int I> __device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + I, 0xF, 0xF, false));
}
// lane i of the caller's 16-lane row (i a compile-time constant after unrolling)
__device__ __forceinline__ float row_bcast(int i, float v) {
    switch (i) {
        case 0: return row_bcast<0>(v);   case 1: return row_bcast<1>(v);
        case 2: return row_bcast<2>(v);   case 3: return row_bcast<3>(v);
        case 4: return row_bcast<4>(v);   case 5: return row_bcast<5>(v);
        case 6: return row_bcast<6>(v);   case 7: return row_bcast<7>(v);
        case 8: return row_bcast<8>(v);   case 9: return row_bcast<9>(v);
        case 10: return row_bcast<10>(v); case 11: return row_bcast<11>(v);
        case 12: return row_bcast<12>(v); case 13: return row_bcast<13>(v);
        case 14: return row_bcast<14>(v); default: return row_bcast<15>(v);
    }
}

// accumulator element i of lane l of a 32x32 fp32 MFMA tile -> tile row
__device__ __forceinline__ int inv_acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

template <int ST, bool kWaveOnly>
__device__ __forceinline__ void unit_lower_inverse64(float* sA) {
    auto sync = []() __attribute__((always_inline)) {
        if constexpr (kWaveOnly) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            __builtin_amdgcn_wave_barrier();
        } else {
            __syncthreads();
        }
    };
    const int lane = threadIdx.x & 63;
    typedef inv_f32x4 f32x4p;
    typedef inv_f32x16 f32x16;
    // (1) the 16x16 diagonal blocks: lane (b, c) owns column c of block b
    {
        const int b = lane >> 4, c = lane & 15, d0 = 16 * b;
        float Acol[16], t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) Acol[r] = sA[(d0 + r) * ST + d0 + c];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc[4] = {r == c ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < r; ++i) acc[i & 3] -= row_bcast(i, Acol[r]) * t[i];
            t[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
        sync();   // every lane has read its column of A
#pragma unroll
        for (int r = 0; r < 16; ++r) sA[(d0 + r) * ST + d0 + c] = t[r];
    }
    sync();
    // (2) 16 -> 32: for the blocks (1,0) and (3,2), Y = A_10 T_00 then T_10 = -T_11 Y, on
    //     v_mfma_f32_16x16x4_f32 (lane (c, g) supplies A[c][4k + g] and B[4k + g][c]; the
    //     accumulator holds C[4g + i][c]). Y goes through the block itself (A_10 is dead).
    {
        const int c = lane & 15, g = lane >> 4;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int o0 = 32 * p, o1 = 32 * p + 16;   // block rows / columns of T_00 and T_11
            f32x4p Y = {};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                Y = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(o1 + c) * ST + o0 + 4 * kk + g],
                                                         sA[(o0 + 4 * kk + g) * ST + o0 + c], Y, 0, 0, 0);
            sync();   // all reads of A_10 done
#pragma unroll
            for (int i = 0; i < 4; ++i) sA[(o1 + 4 * g + i) * ST + o0 + c] = Y[i];
            sync();
            f32x4p T10 = {};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                T10 = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(o1 + c) * ST + o1 + 4 * kk + g],
                                                           sA[(o1 + 4 * kk + g) * ST + o0 + c], T10, 0, 0, 0);
            sync();   // all reads of Y done
#pragma unroll
            for (int i = 0; i < 4; ++i) sA[(o1 + 4 * g + i) * ST + o0 + c] = -T10[i];
        }
    }
    sync();
    // (3) 32 -> 64: X = A10 T0 and T10 = -T1 X on v_mfma_f32_32x32x2_f32 (lane l supplies
    //     A[l%32][l/32] and B[l/32][l%32] of each k-pair); X goes through the unused
    //     upper-right block of the tile.
    const int half = lane >> 5, c = lane & 31;
    f32x16 X = {};
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
        const int k = 2 * s2 + half;
        X = __builtin_amdgcn_mfma_f32_32x32x2f32(sA[(32 + c) * ST + k], sA[k * ST + c], X, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[inv_acc_row(i, lane) * ST + 32 + c] = X[i];
    sync();
    f32x16 T10 = {};
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
        const int k = 2 * s2 + half;
        T10 = __builtin_amdgcn_mfma_f32_32x32x2f32(sA[(32 + c) * ST + 32 + k], sA[k * ST + 32 + c],
                                                  T10, 0, 0, 0);
    }
    sync();   // all reads of A10 and X done
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        sA[(32 + inv_acc_row(i, lane)) * ST + c] = -T10[i];
        sA[inv_acc_row(i, lane) * ST + 32 + c] = 0.f;   // T's upper-right block
    }
    sync();
}

}  // namespace gdn
