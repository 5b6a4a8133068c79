// Measurement aids: the two ceilings the library's roofline figures are read against, measured
// on the device itself rather than taken from the data sheet.
//   stream_kernel  16-byte nontemporal loads and stores over a buffer, the access pattern of
//                  the streaming kernels (decode state, preprocess, output gate). With src ==
//                  dst it is the in-place read-modify-write stream of the decode state.
//   mfma_kernel    back-to-back v_mfma_f32_32x32x16_bf16 on four independent accumulators per
//                  wave, the instruction of the prefill's dense tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_launch.h"

namespace gdn {
namespace {

typedef float f32x4m __attribute__((ext_vector_type(4)));
typedef float f32x16m __attribute__((ext_vector_type(16)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8m;

constexpr int kStreamThreads = 256;
constexpr int kMfmaThreads = 256;

// src and dst are either the same buffer or disjoint (checked by the caller), so no
// __restrict__: the in-place form reads each 16 bytes before it writes them. One 16-byte unit
// per thread and as many workgroups as that takes: of the shapes measured on the device (1, 2,
// 4, 8 and 16 units per thread, grid-stride loops of 1024 to 8192 workgroups, plain and
// nontemporal accesses) this one streams fastest.
__global__ void __launch_bounds__(kStreamThreads) stream_kernel(const f32x4m* src, f32x4m* dst,
                                                                size_t n16) {
    const size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ void __launch_bounds__(kMfmaThreads) mfma_kernel(float* sink, int iters) {
    const int lane = threadIdx.x & 63;
    // operands that the compiler cannot fold: small values from the lane and block index
    bf16x8m a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)((float)((lane + j) & 7) * 0.125f);
        b[j] = (__bf16)((float)((blockIdx.x + j) & 3) * 0.25f);
    }
    f32x16m c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
    if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_mb_stream(const void* src, void* dst, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    const size_t grid = (n16 + kStreamThreads - 1) / kStreamThreads;
    if (grid > 0x7fffffffu) return hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)grid), dim3(kStreamThreads), 0, s,
                       static_cast<const f32x4m*>(src), static_cast<f32x4m*>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_mb_mfma(float* sink, int workgroups, int iters, hipStream_t s) {
    if (workgroups == 0) return hipSuccess;
    hipLaunchKernelGGL(mfma_kernel, dim3(workgroups), dim3(kMfmaThreads), 0, s, sink, iters);
    return hipGetLastError();
}

}  // namespace gdn
