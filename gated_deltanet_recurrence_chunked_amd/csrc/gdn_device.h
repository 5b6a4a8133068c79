// Device helpers shared by the gfx950 kernels of libgdn: bf16 <-> fp32, typed vector
// loads and stores, wave64 reductions, and the math functions of the gates.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;

typedef float floatx4 __attribute__((ext_vector_type(4)));

// --------------------------------------------------------------------------- bf16
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// two floats -> packed bf16 pair (lo in bits 0-15), one v_cvt_pk_bf16_f32
typedef __bf16 gdn_bf16x2 __attribute__((ext_vector_type(2)));
typedef float gdn_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    const gdn_f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, gdn_bf16x2));
}

// --------------------------------------------------------------------------- typed 8-wide IO
// Element type tags: float (fp32) or uint16_t (bf16 bits). The *_stream forms use
// nontemporal accesses, for data a kernel touches exactly once: such lines then do not
// displace the lines that the next kernel of the pipeline reads back (the outputs just
// written stay cached for their consumer).
typedef uint32_t gdn_u32x4 __attribute__((ext_vector_type(4)));

template <bool kStream> __device__ __forceinline__ gdn_u32x4 ld16(const void* p) {
    const gdn_u32x4* q = reinterpret_cast<const gdn_u32x4*>(p);
    if constexpr (kStream) return __builtin_nontemporal_load(q);
    else return *q;
}
template <bool kStream> __device__ __forceinline__ void st16(void* p, const gdn_u32x4& v) {
    gdn_u32x4* q = reinterpret_cast<gdn_u32x4*>(p);
    if constexpr (kStream) __builtin_nontemporal_store(v, q);
    else *q = v;
}

template <typename T> struct Vec8;

template <> struct Vec8<float> {
    struct Raw {
        gdn_u32x4 a, b;
    };
    template <bool kStream = false>
    static __device__ __forceinline__ Raw load_raw(const float* p) {
        return Raw{ld16<kStream>(p), ld16<kStream>(p + 4)};
    }
    static __device__ __forceinline__ void unpack(const Raw& r, float (&x)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = __uint_as_float(r.a[i]);
            x[4 + i] = __uint_as_float(r.b[i]);
        }
    }
    template <bool kStream = false>
    static __device__ __forceinline__ void load(const float* p, float (&x)[8]) {
        const gdn_u32x4 a = ld16<kStream>(p), b = ld16<kStream>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = __uint_as_float(a[i]);
            x[4 + i] = __uint_as_float(b[i]);
        }
    }
    template <bool kStream = false>
    static __device__ __forceinline__ void store(float* p, const float (&x)[8]) {
        const gdn_u32x4 a = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                             __float_as_uint(x[3])};
        const gdn_u32x4 b = {__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]),
                             __float_as_uint(x[7])};
        st16<kStream>(p, a);
        st16<kStream>(p + 4, b);
    }
};

template <> struct Vec8<uint16_t> {
    struct Raw {
        gdn_u32x4 a;
    };
    template <bool kStream = false>
    static __device__ __forceinline__ Raw load_raw(const uint16_t* p) {
        return Raw{ld16<kStream>(p)};
    }
    static __device__ __forceinline__ void unpack(const Raw& r, float (&x)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(r.a[i] << 16);
            x[2 * i + 1] = __uint_as_float(r.a[i] & 0xffff0000u);
        }
    }
    template <bool kStream = false>
    static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[8]) {
        const gdn_u32x4 a = ld16<kStream>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(a[i] << 16);
            x[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
        }
    }
    template <bool kStream = false>
    static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[8]) {
        const gdn_u32x4 a = {pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]),
                             pack_bf2(x[6], x[7])};
        st16<kStream>(p, a);
    }
};

// 4-wide
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ void load(const float* p, float (&x)[4]) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&x)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    }
};
template <> struct Vec4<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[4]) {
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        x[0] = __uint_as_float(a.x << 16);
        x[1] = __uint_as_float(a.x & 0xffff0000u);
        x[2] = __uint_as_float(a.y << 16);
        x[3] = __uint_as_float(a.y & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[4]) {
        uint2 a;
        a.x = pack_bf2(x[0], x[1]);
        a.y = pack_bf2(x[2], x[3]);
        *reinterpret_cast<uint2*>(p) = a;
    }
};

template <typename T> __device__ __forceinline__ float load1(const T* p);
template <> __device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) { return bf2f(*p); }

template <typename T> __device__ __forceinline__ void store1(T* p, float x);
template <> __device__ __forceinline__ void store1<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void store1<uint16_t>(uint16_t* p, float x) { *p = f2bf(x); }

// --------------------------------------------------------------------------- fp32 matrix core
// acc (a 16x16 tile) += A (16 x K) B (K x 16) on v_mfma_f32_16x16x4f32, whose products and sums
// are full fp32. Element (r, k) of A is A[r * ar + k * ak] and element (k, c) of B is
// B[k * bk + c * bc], so transposed views are strides; operands are fp32, or bf16 (uint16_t) that
// widen exactly. K is a multiple of 4. One wave computes
// the tile: lane l supplies A(l%16, k0 + l/16) and B(k0 + l/16, l%16) per step and holds
// C(4 (l/16) + i, l%16) in acc[i].
template <typename TA, typename TB>
__device__ __forceinline__ floatx4 mma_f32_tile(const TA* A, int ar, int ak, const TB* B, int bk,
                                                int bc, int K, floatx4 acc) {
    const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
    const TA* pa = A + c * ar + g * ak;
    const TB* pb = B + g * bk + c * bc;
#pragma unroll 4
    for (int k0 = 0; k0 < K; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(load1(pa + k0 * ak), load1(pb + k0 * bk), acc, 0,
                                                   0, 0);
    return acc;
}

// --------------------------------------------------------------------------- reductions
// Lane exchanges that stay in the VALU (a shuffle through ds_bpermute is an LDS round trip):
// v_permlane32_swap / v_permlane16_swap (gfx950) exchange the two 32-lane halves / the rows
// of each 32-lane half, so r[0] + r[1] of a value swapped with itself is x + x[lane ^ 32] /
// x + x[lane ^ 16] in every lane; DPP row rotations reach the lanes of a 16-lane row.
template <int o>
__device__ __forceinline__ float xor_sum(float x) {
    static_assert(o == 16 || o == 32, "lane distance");
    const uint32_t u = __float_as_uint(x);
    if constexpr (o == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}
template <int n>
__device__ __forceinline__ float row_ror(float x) {   // lane l <- lane 16 (l / 16) + (l + n) % 16
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + n, 0xF, 0xF, false));
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64), every lane of a group
// getting the group's sum. The pairing is a butterfly over lane distances width/2 .. 1 (within
// a 16-lane row, rotating by 8, 4, 2, 1 pairs the same values as distances 8, 4, 2, 1), so the
// rounding is the same whichever lane exchange carries a step.
template <int width>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(width >= 1 && width <= 64 && (width & (width - 1)) == 0, "width");
    if constexpr (width == 64) x = xor_sum<32>(x);
    if constexpr (width >= 32) x = xor_sum<16>(x);
    if constexpr (width >= 16) {
        x += row_ror<8>(x);
        x += row_ror<4>(x);
        x += row_ror<2>(x);
        x += row_ror<1>(x);
    } else {
#pragma unroll
        for (int o = width / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
    }
    return x;
}
// x summed over the lanes lane ^ d for d = from, 2 from, .., 32 (from a power of two): the
// lanes that share lane % from
template <int from>
__device__ __forceinline__ float sum_across(float x) {
    static_assert(from >= 1 && from <= 32 && (from & (from - 1)) == 0, "lane distance");
#pragma unroll
    for (int o = from; o < 16; o <<= 1) x += __shfl_xor(x, o, kWave);
    if constexpr (from <= 16) x = xor_sum<16>(x);
    x = xor_sum<32>(x);
    return x;
}

// --------------------------------------------------------------------------- fast math
// Single hardware instructions (v_exp_f32, v_rcp_f32, v_rsq_f32), each within about one ulp
// in the range these kernels use; the accurate library forms cost ~10-25 instructions each
// and made the streaming kernels VALU-bound.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float frsq(float x) { return __builtin_amdgcn_rsqf(x); }

// --------------------------------------------------------------------------- gate math
__device__ __forceinline__ float sigmoidf_(float x) { return frcp(1.0f + fexp(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x * frcp(1.0f + fexp(-x)); }

// The width-4 causal conv of one channel, oldest tap first (w[3] multiplies the current input),
// with its fused multiply-adds spelled out, so every kernel that evaluates it (the preprocess,
// the fused prefill front end, the fused decode) rounds identically.
__device__ __forceinline__ float conv4(float w0, float w1, float w2, float w3, float x0, float x1,
                                       float x2, float x3) {
    return __builtin_fmaf(w3, x3, __builtin_fmaf(w2, x2, __builtin_fmaf(w1, x1, w0 * x0)));
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}): no overflow, no cancellation
__device__ __forceinline__ float softplusf_(float x) {
    return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

// The per-head gates of eqs. (9)-(10): g = log(alpha) = -e^{A} softplus(a + dt_bias),
// beta = sigmoid(b).
__device__ __forceinline__ float gate_g(float A_log, float a_raw, float dt_bias) {
    return -expf(A_log) * softplusf_(a_raw + dt_bias);
}
__device__ __forceinline__ float gate_beta(float b_raw) { return sigmoidf_(b_raw); }

}  // namespace gdn
