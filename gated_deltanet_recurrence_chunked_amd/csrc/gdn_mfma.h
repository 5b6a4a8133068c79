// Matrix-core and LDS building blocks of the bf16 chunked kernels on gfx950: operand
// fragments of v_mfma_f32_16x16x32_bf16 / 32x32x16_bf16, the transposing LDS read, the
// 16-byte unit swizzle of LDS tiles, the row relabelling that lets an accumulator serve as
// the next product's operand, hi + lo bf16 splits, direct global -> LDS loads and the
// barriers and scheduling hints the pipelined scans use.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_device.h"

namespace gdn {

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

}  // namespace gdn
