// Host-side launchers of the libgdn kernels (internal; the public ABI is include/gdn.h).
// Each launcher assumes its arguments were validated by the caller and returns the
// HIP error of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct PreprocessArgs {
    const void* x[3];     // xq, xk, xv (NULL: stream skipped)
    const float* w[3];    // conv taps [H*d, 4]
    void* out[3];         // q, k, v
    int d[3];             // dk, dk, dv
    int in_bf16, out_bf16;
    const float *a_raw, *b_raw, *A_log, *dt_bias;  // NULL a_raw: gates skipped
    float *g, *beta;
    const int32_t* cu;    // NULL: equal lengths
    int num_seqs, ntok, H;
    float l2_eps;
    // carried conv history [num_seqs, 3, hC] in the input dtype, channels q | k | v
    // (hC = H * (2 dk + dv)); NULL hin: zero history, NULL hout: not written
    const void* hin;
    void* hout;
    int hC;
};
hipError_t launch_preprocess(const PreprocessArgs& a, hipStream_t s);

hipError_t launch_output_gate(const void* y, int y_bf16, const void* z, int z_bf16,
                              const float* w, int ntok, int H, int dv, float eps, void* o,
                              int o_bf16, hipStream_t s);

hipError_t launch_decode(const void* q, const void* k, const void* v, int in_bf16,
                         const float* g, const float* beta, float* state, int N, int H,
                         int dk, int dv, void* y, int y_bf16, hipStream_t s);

// one decode step from the projected streams: conv with the carried history (updated in
// place), gates, the state update and the output gate in one kernel
struct DecodeFusedArgs {
    const void* x[3];          // xq, xk [N, H, dk], xv [N, H, dv]
    const float* w[3];         // conv taps [H*d, 4]
    void* conv_state;          // [N, 3, hC], x dtype, in/out
    int hC;                    // H * (2 dk + dv)
    const float *a_raw, *b_raw, *A_log, *dt_bias;
    float l2_eps;
    float* state;              // [N, H, dk, dv] fp32, in/out
    const void* z;             // [N, H, dv], x dtype
    const float* norm_w;       // [dv]
    float rms_eps;
    void* o;                   // [N, H, dv]
    void* y;                   // nullable, o dtype
    int N, H, in_bf16, out_bf16;
};
hipError_t launch_decode_fused(const DecodeFusedArgs& f, int dk, int dv, hipStream_t s);
// T <= kMaxDecodeTokens tokens per sequence through the fused step: the conv history is read
// from hin and written to f.conv_state (which may equal hin); steps (nullable) as decode_multi
hipError_t launch_decode_fused_multi(const DecodeFusedArgs& f, const void* hin, int T,
                                     float* steps, int dk, int dv, hipStream_t s);
// T <= kMaxDecodeTokens tokens per sequence; steps (nullable): the state after each token
constexpr int kMaxDecodeTokens = 8;
hipError_t launch_decode_multi(const void* q, const void* k, const void* v, int in_bf16,
                               const float* g, const float* beta, float* state, int N, int T,
                               int H, int dk, int dv, void* y, int y_bf16, float* steps,
                               hipStream_t s);

struct ChunkArgs {
    const void *q, *k, *v;
    int in_bf16, y_bf16;
    const float *g, *beta, *S0;
    float* ST;
    const int32_t* cu;    // NULL: equal lengths
    int num_seqs, ntok, H, dk, dv;
    void* y;
    void* workspace;
    size_t workspace_bytes;
};
// all-fp32 chunked path (vector ALU)
hipError_t launch_chunk_fp32(const ChunkArgs& a, hipStream_t s);

// The device address of this GPU's library-owned scratch array (GDN_NOALLOC_SCRATCH_BYTES,
// gdn_noalloc.hip), looked up on the first call per device; it never allocates.
hipError_t noalloc_scratch(void** ptr);

// measurement aids (microbench.hip)
hipError_t launch_mb_stream(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_mb_mfma(float* sink, int workgroups, int iters, hipStream_t s);

// bf16 matrix-core chunked path (dk = 128): per-chunk T/P kernel + sequential scan kernel
size_t chunk_bf16_workspace(int ntok, int num_seqs, int H);
// The gated output of eq. (11) applied to the prefill's y (the fused prefill): inside the scan
// when the full-row scan runs (256 or more (sequence, head) pairs of equal length, d_v = 128),
// else by the output-gate kernel after it (reading ChunkArgs::y).
struct GateArgs {
    const void* z;        // [ntok, H, dv]
    int z_bf16;
    const float* w;       // [dv]
    float eps;
    void* o;              // [ntok, H, dv]
    int o_bf16;
    void* y_export;       // nullable: y (bf16) is also stored here when the scan applies the gate
};
// per-channel-decay prefill with log-decays >= -5 on the bf16 matrix cores (dk = dv = 128);
// gk: log-decays [ntok, H, 128]; ChunkArgs::g unused
size_t kda_bf16_workspace(int ntok, int num_seqs, int H);
hipError_t launch_kda_bf16(const ChunkArgs& a, const float* gk, hipStream_t s);
hipError_t launch_chunk_bf16(const ChunkArgs& a, hipStream_t s, const GateArgs* gate = nullptr);

// Gate rows the bf16 path keeps per (chunk, head), 64 floats each: beta, gamma = e^G,
// gamma_C / gamma and G (the running sum of g over the chunk); the per-channel-decay path puts
// beta and e^{Gc[C]} (128 values) in the first three.
constexpr int kGateRows = 4;

// The bf16 path's per-chunk tiles inside its workspace (the layout launch_chunk_bf16 uses).
struct ChunkTiles {
    int32_t* chunk_start;   // [num_seqs + 1] first packed chunk of each sequence (varlen)
    int32_t* order;         // [num_seqs] sequences longest first (varlen)
    uint16_t *T, *P;        // [max_chunks][H][64][64] bf16
    float* Gw;              // [max_chunks][H][kGateRows][64]: beta, gamma = e^G, gamma_C / gamma, G
    int max_chunks;
};
ChunkTiles chunk_bf16_tiles(void* workspace, int ntok, int num_seqs, int H);
// The backward's forward sweep on the bf16 path (dk = dv = 128): the chunk table, T and P per
// chunk, and the state entering every chunk as fp32 S^T [max_chunks][H][dv][dk] in Sst; no y.
hipError_t launch_chunk_bf16_states(const ChunkArgs& a, float* Sst, hipStream_t s);

// backward of the chunked gated delta rule: bf16 q, k, v, dy with dk = dv = 128 on the bf16
// matrix cores (chunk_bwd_bf16.hip), everything else in fp32 (chunk_bwd.hip)
struct ChunkBwdArgs {
    const void *q, *k, *v, *dy;
    int in_bf16, dy_bf16;
    const float *g, *beta, *S0, *dST;
    const int32_t* cu;    // NULL: equal lengths
    int num_seqs, ntok, H, dk, dv;
    float *dq, *dk_, *dv_, *dg, *dbeta, *dS0;
    void* workspace;
};
size_t chunk_bwd_workspace(int ntok, int num_seqs, int H, int dk, int dv);
hipError_t launch_chunk_bwd(const ChunkBwdArgs& a, hipStream_t s);
bool use_bwd_bf16(const ChunkBwdArgs& a);
size_t chunk_bwd_bf16_workspace(int ntok, int num_seqs, int H);
hipError_t launch_chunk_bwd_bf16(const ChunkBwdArgs& a, hipStream_t s);

// per-channel-decay (KDA-style) chunked forward (fp32 vector ALU)
struct ChunkKdaArgs {
    const void *q, *k, *v;
    int in_bf16, y_bf16;
    const float *g, *beta, *S0;   // g: [ntok, H, dk]
    float* ST;
    const int32_t* cu;
    int num_seqs, ntok, H, dk, dv;
    void* y;
    void* workspace;
};
size_t chunk_kda_workspace(int ntok, int num_seqs, int H, int dk);
hipError_t launch_chunk_kda(const ChunkKdaArgs& a, hipStream_t s);

}  // namespace gdn
