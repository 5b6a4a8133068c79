// Drives every entry point of the C ABI through its host validation, on valid arguments (the
// stubbed launchers are reached) and on invalid ones (a status code and a message, nothing
// launched). Built with -fsanitize=address,undefined: a read past a host array, a signed
// overflow in an extent check or a misaligned access ends the run with a report.
// Device pointers are fake aligned addresses: validation never dereferences them.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "gdn.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(call, want)                                                                  \
    do {                                                                                    \
        const int got_ = (call);                                                            \
        const char* msg_ = gdn_last_error();                                                \
        if (got_ != (want) || (got_ != 0 && (msg_ == nullptr || strlen(msg_) == 0))) {      \
            fprintf(stderr, "line %d: %s -> %d (want %d): %s\n", __LINE__, #call, got_,    \
                    (want), msg_ ? msg_ : "(null)");                                        \
            ++failures;                                                                     \
        }                                                                                   \
    } while (0)

static void* P(uintptr_t i) { return reinterpret_cast<void*>(0x100000000ull + (i << 24)); }
static float* F(uintptr_t i) { return static_cast<float*>(P(i)); }
static void* MIS = reinterpret_cast<void*>(0x100000004ull);

int main() {
    const int BF = GDN_BF16, FP = GDN_F32;
    const int ntok = 300, H = 4, dk = 128, dv = 128, N = 3;
    std::vector<int32_t> cu = {0, 0, 1, 64, 65, 300};
    const int nseq = (int)cu.size() - 1;
    std::vector<int32_t> bad_cu = {0, 70, 60, 64, 65, 300};
    const size_t ws = gdn_chunk_prefill_workspace_size(ntok, nseq, H, dk, dv, BF);
    const int32_t* cud = reinterpret_cast<const int32_t*>(P(40));

    // preprocess: full, gates only, invalid
    EXPECT(gdn_preprocess(P(1), P(2), P(3), BF, F(4), F(5), F(6), 4, F(7), F(8), F(9), F(10), cud,
                          nseq, ntok, H, dk, dv, 1e-6f, P(11), P(12), P(13), BF, F(14), F(15),
                          nullptr), 0);
    EXPECT(gdn_preprocess(nullptr, nullptr, nullptr, FP, nullptr, nullptr, nullptr, 4, F(7), F(8),
                          F(9), F(10), nullptr, 1, ntok, H, dk, dv, 0.f, nullptr, nullptr, nullptr,
                          FP, F(14), F(15), nullptr), 0);
    EXPECT(gdn_preprocess(P(1), P(2), P(3), BF, F(4), F(5), F(6), 3, F(7), F(8), F(9), F(10), cud,
                          nseq, ntok, H, dk, dv, 1e-6f, P(11), P(12), P(13), BF, F(14), F(15),
                          nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_preprocess(MIS, P(2), P(3), BF, F(4), F(5), F(6), 4, F(7), F(8), F(9), F(10), cud,
                          nseq, ntok, H, dk, dv, 1e-6f, P(11), P(12), P(13), BF, F(14), F(15),
                          nullptr), GDN_ERR_ALIGN);
    EXPECT(gdn_preprocess(P(1), P(2), P(3), 9, F(4), F(5), F(6), 4, F(7), F(8), F(9), F(10), cud,
                          nseq, ntok, H, dk, dv, 1e-6f, P(11), P(12), P(13), BF, F(14), F(15),
                          nullptr), GDN_ERR_DTYPE);
    EXPECT(gdn_preprocess_stateful(P(1), P(2), P(3), BF, F(4), F(5), F(6), 4, F(7), F(8), F(9),
                                   F(10), cud, nseq, ntok, H, dk, dv, 1e-6f, P(11), P(12), P(13),
                                   BF, F(14), F(15), P(16), P(17), nullptr), 0);
    EXPECT(gdn_preprocess_stateful(P(1), P(2), P(3), BF, F(4), F(5), F(6), 4, F(7), F(8), F(9),
                                   F(10), cud, nseq, ntok, H, dk, dv, 1e-6f, P(11), P(12), P(13),
                                   BF, F(14), F(15), P(16), P(16), nullptr), GDN_ERR_SHAPE);

    // chunked prefill: packed, equal lengths, empty, invalid offsets, extents, workspace
    for (int dt : {BF, FP}) {
        const size_t w = gdn_chunk_prefill_workspace_size(ntok, nseq, H, dk, dv, dt);
        EXPECT(gdn_chunk_prefill(P(1), P(2), P(3), dt, F(4), F(5), F(6), F(7), cud, cu.data(),
                                 nseq, ntok, H, dk, dv, P(8), dt, w ? P(9) : nullptr, w, nullptr), 0);
        EXPECT(gdn_chunk_prefill(P(1), P(2), P(3), dt, F(4), F(5), F(6), F(7), cud, bad_cu.data(),
                                 nseq, ntok, H, dk, dv, P(8), dt, P(9), w, nullptr), GDN_ERR_SEQLENS);
    }
    EXPECT(gdn_chunk_prefill(P(1), P(2), P(3), BF, F(4), F(5), nullptr, nullptr, nullptr, nullptr,
                             4, 256, H, dk, dv, P(8), BF, P(9), ws, nullptr), 0);
    EXPECT(gdn_chunk_prefill(P(1), P(2), P(3), BF, F(4), F(5), nullptr, nullptr, nullptr, nullptr,
                             4, 250, H, dk, dv, P(8), BF, P(9), ws, nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_chunk_prefill(nullptr, nullptr, nullptr, BF, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr, 1, 0, H, dk, dv, nullptr, BF, P(9), ws, nullptr), 0);
    EXPECT(gdn_chunk_prefill(P(1), P(2), P(3), BF, F(4), F(5), nullptr, nullptr, nullptr, nullptr,
                             1, 1 << 30, 64, dk, dv, P(8), BF, P(9), (size_t)-1, nullptr),
           GDN_ERR_SHAPE);
    EXPECT(gdn_chunk_prefill(P(1), P(2), P(3), BF, F(4), F(5), nullptr, nullptr, nullptr, nullptr,
                             1, ntok, H, dk, dv, P(8), BF, P(9), 16, nullptr), GDN_ERR_WORKSPACE);
    EXPECT(gdn_chunk_prefill_noalloc(P(1), P(2), P(3), BF, F(4), F(5), F(6), F(7), cud, cu.data(),
                                     nseq, ntok, H, dk, dv, P(8), BF, nullptr), 0);
    EXPECT(gdn_chunk_prefill_noalloc(P(1), P(2), P(3), BF, F(4), F(5), nullptr, nullptr, nullptr,
                                     nullptr, 1, 1 << 20, 8, dk, dv, P(8), BF, nullptr),
           GDN_ERR_WORKSPACE);

    // backward and the per-channel-decay prefill
    const size_t wb = gdn_chunk_backward_workspace_size(ntok, nseq, H, dk, dv);
    EXPECT(gdn_chunk_backward(P(1), P(2), P(3), BF, F(4), F(5), F(6), P(7), BF, F(8), cud,
                              cu.data(), nseq, ntok, H, dk, dv, F(9), F(10), F(11), F(12), F(13),
                              F(14), P(15), wb, nullptr), 0);
    EXPECT(gdn_chunk_backward(P(1), P(2), P(3), BF, F(4), F(5), F(6), P(7), BF, F(8), cud,
                              cu.data(), nseq, ntok, H, dk, 96, F(9), F(10), F(11), F(12), F(13),
                              F(14), P(15), wb, nullptr), GDN_ERR_SHAPE);
    const size_t wk = gdn_kda_chunk_prefill_workspace_size(ntok, nseq, H, dk);
    EXPECT(gdn_kda_chunk_prefill(P(1), P(2), P(3), BF, F(4), F(5), F(6), F(7), cud, cu.data(),
                                 nseq, ntok, H, dk, dv, P(8), BF, P(9), wk, nullptr), 0);

    const size_t wkb = gdn_kda_chunk_prefill_bounded_workspace_size(ntok, nseq, H);
    EXPECT(gdn_kda_chunk_prefill_bounded(P(1), P(2), P(3), BF, F(4), F(5), F(6), F(7), cud,
                                         cu.data(), nseq, ntok, H, dk, dv, P(8), BF, P(9), wkb,
                                         nullptr), 0);
    EXPECT(gdn_kda_chunk_prefill_bounded(P(1), P(2), P(3), FP, F(4), F(5), F(6), F(7), cud,
                                         cu.data(), nseq, ntok, H, dk, dv, P(8), BF, P(9), wkb,
                                         nullptr), GDN_ERR_DTYPE);
    EXPECT(gdn_kda_chunk_prefill_bounded(P(1), P(2), P(3), BF, F(4), F(5), F(6), F(7), cud,
                                         cu.data(), nseq, ntok, H, 64, dv, P(8), BF, P(9), wkb,
                                         nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_kda_chunk_prefill_bounded(P(1), P(2), P(3), BF, static_cast<const float*>(MIS),
                                         F(5), F(6), F(7), cud, cu.data(), nseq, ntok, H, dk, dv,
                                         P(8), BF, P(9), wkb, nullptr), GDN_ERR_ALIGN);

    // decode
    EXPECT(gdn_decode_step(P(1), P(2), P(3), BF, F(4), F(5), F(6), N, H, dk, dv, P(7), BF,
                           nullptr), 0);
    EXPECT(gdn_decode_step(P(1), P(2), P(3), BF, F(4), F(5), F(6), N, H, 80, dv, P(7), BF,
                           nullptr), GDN_ERR_SHAPE);
    for (int T : {1, 4, GDN_DECODE_MAX_TOKENS})
        EXPECT(gdn_decode_multi(P(1), P(2), P(3), BF, F(4), F(5), F(6), N, T, H, dk, dv, P(7), BF,
                                F(8), nullptr), 0);
    EXPECT(gdn_decode_multi(P(1), P(2), P(3), BF, F(4), F(5), F(6), N, GDN_DECODE_MAX_TOKENS + 1,
                            H, dk, dv, P(7), BF, nullptr, nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_decode_multi(P(1), P(2), P(3), BF, F(4), F(5), F(6), N, 4, H, dk, dv, P(7), BF,
                            F(6), nullptr), GDN_ERR_SHAPE);

    // output gate and the fused entry points
    EXPECT(gdn_output_gate(P(1), BF, P(2), BF, F(3), ntok, H, dv, 1e-6f, P(4), BF, nullptr), 0);
    EXPECT(gdn_output_gate(P(1), BF, P(2), BF, F(3), ntok, H, dv, -1.f, P(4), BF, nullptr),
           GDN_ERR_SHAPE);
    const size_t wf = gdn_fused_prefill_workspace_size(ntok, nseq, H, dk, dv);
    EXPECT(gdn_fused_prefill(P(1), P(2), P(3), BF, F(4), F(5), F(6), 4, F(7), F(8), F(9), F(10),
                             1e-6f, P(11), BF, F(12), 1e-6f, F(13), F(14), cud, cu.data(), nseq,
                             ntok, H, dk, dv, P(15), BF, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr, P(16), wf, nullptr), 0);
    EXPECT(gdn_fused_prefill(P(1), P(2), P(3), BF, F(4), F(5), F(6), 4, F(7), F(8), F(9), F(10),
                             1e-6f, P(11), BF, F(12), 1e-6f, F(13), F(14), cud, cu.data(), nseq,
                             ntok, H, dk, dv, P(15), BF, nullptr, nullptr, nullptr, F(17), nullptr,
                             nullptr, P(16), wf, nullptr), GDN_ERR_NULL);
    EXPECT(gdn_fused_decode(P(1), P(2), P(3), BF, F(4), F(5), F(6), 4, P(7), F(8), F(9), F(10),
                            F(11), 1e-6f, F(12), P(13), F(14), 1e-6f, N, H, dk, dv, P(15), BF,
                            nullptr, nullptr), 0);
    EXPECT(gdn_fused_decode_multi(P(1), P(2), P(3), BF, F(4), F(5), F(6), 4, P(7), P(8), F(9),
                                  F(10), F(11), F(12), 1e-6f, F(13), P(14), F(15), 1e-6f, N, 4, H,
                                  dk, dv, P(16), BF, nullptr, F(17), nullptr), 0);

    // measurement aids
    EXPECT(gdn_mb_stream(P(1), P(2), 1 << 20, nullptr), 0);
    EXPECT(gdn_mb_stream(P(1), P(1), 1 << 20, nullptr), 0);
    EXPECT(gdn_mb_stream(P(1), static_cast<char*>(P(1)) + 16, 1 << 20, nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_mb_mfma_bf16(F(1), 64, 8, nullptr), 0);

    // workspace-size queries on sizes at and past the limits
    (void)gdn_chunk_prefill_workspace_size(0x7fffffff, 1, 1, 128, 128, BF);
    (void)gdn_chunk_backward_workspace_size(0x7fffffff, 1, 1, 128, 128);
    (void)gdn_fused_prefill_workspace_size(-1, 1, 1, 128, 128);
    printf("%d failures, %d launches reached, abi %d\n", failures, g_launches, gdn_abi_version());
    return failures ? 1 : 0;
}
