// Sanitizer driver for the host side of the C ABI (kda_api.hip): calls every
// entry point with the argument errors the CPU tests use, which are rejected
// on the host before any launch, plus the host-only size queries and status
// strings, under AddressSanitizer / UndefinedBehaviorSanitizer.  The kernel
// launchers are stubs here (validation never reaches them); a call that gets
// past validation needs the GPU runtime and, without a GPU, must come back as
// KDA_ERR_HIP.  Prints "abi sanitizer driver ok" and exits 0 when every call
// returned what it should.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"
#include "../../kimi_delta_attention_kda_amd/csrc/kda_launch.hpp"

namespace kda {
hipError_t launch_decode(const uint16_t *, const uint16_t *, const uint16_t *, const float *, const float *, float *,
                         const int32_t *, uint16_t *, int, int, int, int, float, int, int *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_extend(const uint16_t *, const uint16_t *, const uint16_t *, const float *, const float *, float *,
                         const int32_t *, uint16_t *, int, int, int, int, int, float, int, int *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_conv_decode(const uint16_t *, uint16_t *, const uint16_t *, const uint16_t *, const uint16_t *,
                              const uint16_t *, const float *, const float *, float *, const int32_t *, uint16_t *,
                              int, int, int, int, int, float, int, int *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t fwd_two_pass_eligible(long long, bool *) { return hipErrorNoDevice; }
size_t fwd_workspace_bytes(int dk, long long n_rows, int H) {
    return (size_t)(dk == 128 ? 13824 : 7424) * (size_t)(n_rows < 0 ? 0 : n_rows) * (size_t)(H < 0 ? 0 : H);
}
hipError_t launch_fwd_bf16(const FwdArgs &, int, int, void *, size_t, long long, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_fwd_f32(const FwdArgs &, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_chunk_o(const ChunkOArgs &, long long, hipStream_t) { return hipErrorInvalidValue; }
size_t bwd_workspace_bytes(int n_seq, int H, long long tokens) {
    return (size_t)4 * (4 * (size_t)tokens * H * (3 * 128 + 1) + 7 * (size_t)n_seq * H * 129);
}
hipError_t launch_bwd(const BwdArgs &, int, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace kda

static int fails = 0;
static void expect(long long got, long long want, const char *what) {
    if (got != want) {
        printf("FAIL %s: %lld, expected %lld\n", what, got, want);
        ++fails;
    }
}

int main() {
    void *A = reinterpret_cast<void *>(0x10000), *Bp = reinterpret_cast<void *>(0x20000);
    void *MIS = reinterpret_cast<void *>(0x20004);
    const float *Af = static_cast<const float *>(Bp);
    for (int s = 0; s >= -7; --s) {
        const char *str = kda_status_str(s);
        expect(str != nullptr && strlen(str) > 0, 1, "status string");
    }
    expect(strcmp(kda_status_str(0), "ok"), 0, "status ok");
    // chunk_fwd: chunk size, head dims, dtype, shapes, NULLs, alignment, empty
    auto chunk = [&](int chunk_, int dk, int dtype, int H, int n_seq, const void *cu, int B, const void *q,
                     void *o, void *ws, size_t wsb) {
        return kda_chunk_fwd(q, A, A, A, A, Af, Af, nullptr, static_cast<const int32_t *>(cu), chunk_, o, nullptr, B,
                             16, H, dk, 128, n_seq, 0.1f, (kda_dtype)dtype, ws, wsb, nullptr);
    };
    expect(chunk(32, 128, 1, 1, 1, nullptr, 1, A, A, nullptr, 0), KDA_ERR_UNSUPPORTED, "chunk size");
    expect(chunk(16, 96, 1, 1, 1, nullptr, 1, A, A, nullptr, 0), KDA_ERR_UNSUPPORTED, "dk");
    expect(chunk(16, 128, 0, 1, 1, nullptr, 1, A, A, nullptr, 0), KDA_ERR_UNSUPPORTED, "fp32 at dk 128");
    expect(chunk(16, 128, 1, 0, 1, nullptr, 1, A, A, nullptr, 0), KDA_ERR_SHAPE, "H = 0");
    expect(chunk(16, 128, 1, 1, 2, nullptr, 1, A, A, nullptr, 0), KDA_ERR_SHAPE, "n_seq != B");
    expect(chunk(16, 128, 1, 1, 2, A, 2, A, A, nullptr, 0), KDA_ERR_SHAPE, "packed B != 1");
    expect(chunk(16, 128, 1, 1, 1, nullptr, 1, nullptr, A, nullptr, 0), KDA_ERR_NULL, "q NULL");
    expect(chunk(16, 128, 1, 1, 1, nullptr, 1, A, MIS, nullptr, 0), KDA_ERR_ALIGN, "o misaligned");
    expect(chunk(16, 128, 1, 1, 1, nullptr, 1, A, A, MIS, 1 << 20), KDA_ERR_ALIGN, "workspace misaligned");
    expect(chunk(16, 128, 1, 1, 0, nullptr, 0, A, A, nullptr, 0), KDA_OK, "nothing to do");
    expect(chunk(16, 128, 1, 1, 1, nullptr, 1, A, A, nullptr, 0), KDA_ERR_HIP, "valid call without a GPU");
    expect((long long)kda_chunk_fwd_workspace_bytes(4, 4096, 16, 128, 128, 4, 0), 13824LL * 4 * 256 * 16,
           "workspace bytes dense");
    expect((long long)kda_chunk_fwd_workspace_bytes(1, 129830, 32, 128, 128, 32, 1),
           13824LL * 32 * ((129830 + 15) / 16 + 32), "workspace bytes packed");
    expect((long long)kda_chunk_fwd_workspace_bytes(1, 16, 1, 96, 128, 1, 0), 0, "workspace bytes bad dk");
    // the allocation-free variant
    expect(kda_chunk_fwd_noalloc(A, A, A, A, A, Af, Af, nullptr, nullptr, 32, A, nullptr, 1, 16, 1, 128, 128, 1,
                                 0.1f, KDA_BF16, nullptr), KDA_ERR_UNSUPPORTED, "noalloc chunk size");
    expect(kda_chunk_fwd_noalloc(nullptr, A, A, A, A, Af, Af, nullptr, nullptr, 16, A, nullptr, 1, 16, 1, 128, 128,
                                 1, 0.1f, KDA_BF16, nullptr), KDA_ERR_NULL, "noalloc q NULL");
    expect(kda_chunk_fwd_noalloc(A, A, A, A, A, Af, Af, nullptr, nullptr, 16, A, nullptr, 1, 16, 1, 128, 128, 1,
                                 0.1f, KDA_BF16, nullptr), KDA_ERR_HIP, "noalloc without a GPU");
    // states, pool
    expect(kda_chunk_fwd_states(A, A, A, A, A, Af, Af, nullptr, nullptr, 16, A, nullptr, nullptr, 1, 16, 1, 128,
                                128, 1, 0.1f, KDA_BF16, nullptr, 0, nullptr), KDA_ERR_NULL, "states h_chunks NULL");
    expect(kda_chunk_fwd_pool(A, A, A, A, A, Af, Af, static_cast<float *>(A), static_cast<const int32_t *>(Bp),
                              nullptr, 16, A, 1, 16, 1, 128, 128, 1, 0, 0.1f, KDA_BF16, nullptr, 0, nullptr),
           KDA_ERR_SHAPE, "pool P = 0");
    // decode family
    expect(kda_decode_step(A, A, A, Af, Af, static_cast<float *>(A), static_cast<const int32_t *>(A), A, 4, 2, 3,
                           128, 128, 8, 0.1f, 1, nullptr), KDA_ERR_SHAPE, "decode HV % H");
    expect(kda_decode_step(A, A, A, Af, Af, static_cast<float *>(A), static_cast<const int32_t *>(MIS), A, 4, 2, 4,
                           128, 128, 8, 0.1f, 1, nullptr), KDA_ERR_ALIGN, "decode idx misaligned");
    expect(kda_decode_extend(A, A, A, Af, Af, static_cast<float *>(A), static_cast<const int32_t *>(A), nullptr, 4, 3,
                             2, 4, 128, 128, 8, 0.1f, 1, nullptr), KDA_ERR_NULL, "extend o NULL");
    expect(kda_conv_decode_step(A, static_cast<uint16_t *>(A), A, nullptr, A, A, Af, Af, static_cast<float *>(A),
                                static_cast<const int32_t *>(A), A, 4, 2, 4, 128, 128, 5, 8, 0.1f, 1, nullptr),
           KDA_ERR_UNSUPPORTED, "conv width 5");
    // chunk-parallel output and backward
    expect(kda_chunk_o(A, A, A, A, A, Af, Af, static_cast<const float *>(A), nullptr, A, 2, 20, 1, 128, 128, 2, 3,
                       0.1f, KDA_BF16, nullptr), KDA_ERR_SHAPE, "chunk_o rows");
    expect((long long)kda_backward_workspace_bytes(2, 3, 64, 128, 100), 0, "backward workspace bad dk");
    expect(kda_device_check(nullptr), KDA_ERR_HIP, "device check without a GPU");
    if (fails) return 1;
    printf("abi sanitizer driver ok\n");
    return 0;
}
