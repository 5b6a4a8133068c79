// Host-only stand-ins for the kernel launchers and workspace-size helpers of libgdn, so the
// C ABI's host validation (gdn_api.hip) can be built with AddressSanitizer and
// UndefinedBehaviorSanitizer and driven on a machine without a GPU. Every launcher records that
// it was reached and returns success; nothing touches device memory.
#include <hip/hip_runtime.h>

#include "gdn_launch.h"

int g_launches = 0;

extern "C" const char* hipGetErrorString(hipError_t) { return "stubbed HIP error"; }

namespace gdn {

static hipError_t reached() {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_preprocess(const PreprocessArgs&, hipStream_t) { return reached(); }
hipError_t launch_output_gate(const void*, int, const void*, int, const float*, int, int, int,
                              float, void*, int, hipStream_t) { return reached(); }
hipError_t launch_decode(const void*, const void*, const void*, int, const float*, const float*,
                         float*, int, int, int, int, void*, int, hipStream_t) { return reached(); }
hipError_t launch_decode_fused(const DecodeFusedArgs&, int, int, hipStream_t) { return reached(); }
hipError_t launch_decode_fused_multi(const DecodeFusedArgs&, const void*, int, float*, int, int,
                                     hipStream_t) { return reached(); }
hipError_t launch_decode_multi(const void*, const void*, const void*, int, const float*,
                               const float*, float*, int, int, int, int, int, void*, int, float*,
                               hipStream_t) { return reached(); }
hipError_t launch_chunk_fp32(const ChunkArgs&, hipStream_t) { return reached(); }
hipError_t launch_chunk_bf16(const ChunkArgs&, hipStream_t, const GateArgs*) { return reached(); }
hipError_t launch_chunk_bwd(const ChunkBwdArgs&, hipStream_t) { return reached(); }
hipError_t launch_kda_bf16(const ChunkArgs&, const float*, hipStream_t) { return reached(); }
hipError_t launch_chunk_kda(const ChunkKdaArgs&, hipStream_t) { return reached(); }
hipError_t launch_mb_stream(const void*, void*, size_t, hipStream_t) { return reached(); }
hipError_t launch_mb_mfma(float*, int, int, hipStream_t) { return reached(); }
hipError_t noalloc_scratch(void** ptr) {
    *ptr = reinterpret_cast<void*>(uintptr_t(0x7f0000000000ull));
    return hipSuccess;
}
bool use_wide_scan(int pairs, int dv) { return dv == 128 && pairs >= 256; }

// sizes of the same order as the real layouts (any value works for the validation paths)
size_t chunk_bf16_workspace(int ntok, int num_seqs, int H) {
    return ((size_t)ntok / 64 + num_seqs + 1) * H * 17408 + 8 * ((size_t)num_seqs + 1);
}
size_t chunk_bwd_workspace(int ntok, int num_seqs, int H, int dk, int dv) {
    return ((size_t)ntok / 64 + num_seqs + 1) * H * ((size_t)dk * dv * 4 + 65536);
}
size_t kda_bf16_workspace(int ntok, int num_seqs, int H) {
    return ((size_t)ntok / 64 + num_seqs + 1) * H * 66560;
}
size_t chunk_kda_workspace(int ntok, int num_seqs, int H, int dk) {
    return ((size_t)ntok / 64 + num_seqs + 1) * H * ((size_t)dk * 512 + 16384);
}

}  // namespace gdn
