// kda_launch.hpp -- host-side launchers of the KDA kernels (internal to the
// library; the public interface is include/kda.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Bits of the per-device error word that kernels set on invalid input found
// in device memory (sticky until kda_device_check reads and clears them).
#define KDA_DEVERR_SLOT 1   // a live pool slot index >= P (treated as a pad)

namespace kda {

// Report an out-of-range slot: a vector atomic OR into the error word.
__device__ __forceinline__ void slot_error(int *err) {
    __hip_atomic_fetch_or(err, KDA_DEVERR_SLOT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Pool-addressed launchers: slots are state_idx[n] in [0, P); a negative
// index is a pad row, an index >= P is treated as a pad and sets
// KDA_DEVERR_SLOT in *err.
hipError_t launch_decode(const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                         const float *A_log, const float *dt_bias, float *pool,
                         const int32_t *state_idx, uint16_t *o, int B, int H, int HV, int P,
                         float scale, int l2norm, int *err, hipStream_t stream);
hipError_t launch_extend(const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                         const float *A_log, const float *dt_bias, float *pool,
                         const int32_t *state_idx, uint16_t *o, int B, int T, int H, int HV, int P,
                         float scale, int l2norm, int *err, hipStream_t stream);

hipError_t launch_conv_decode(const uint16_t *x, uint16_t *conv_state, const uint16_t *cw,
                              const uint16_t *cb, const uint16_t *a, const uint16_t *b,
                              const float *A_log, const float *dt_bias, float *pool,
                              const int32_t *state_idx, uint16_t *o, int B, int H, int HV, int W, int P,
                              float scale, int l2norm, int *err, hipStream_t stream);

// Chunkwise prefill (kda_fwd.hip for bf16, kda_fwd_f32.hip for fp32).
struct FwdArgs {
    const void *q, *k, *v, *g_raw, *beta_raw;
    const float *A_log, *dt_bias, *h0;
    const int32_t *state_idx;   // NULL: h0 / h_T row = sequence; else row = state_idx[sequence] (< 0 or >= P: none)
    const int32_t *cu_seqlens;
    void *o;
    float *h_T;
    float *h_chunks;     // NULL, or [N_chunks][H][DV][DK]: the state entering every chunk
    int T, H, n_seq;     // T: per-sequence length for dense input, total tokens if cu_seqlens
    int P;               // pool slots (state_idx only)
    float scale;
    int *err;            // the device error word
};
// bf16: one pass, or (with a workspace of at least fwd_workspace_bytes for
// n_rows chunk rows, and chains fewer than the compute units) two passes.
// Whether the bf16 prefill takes its two-pass form for this many (sequence,
// head) chains on the current device (given a large enough workspace).
hipError_t fwd_two_pass_eligible(long long chains, bool *two);
size_t fwd_workspace_bytes(int dk, long long n_rows, int H);
hipError_t launch_fwd_bf16(const FwdArgs &a, int dk, int dv, void *ws, size_t ws_bytes, long long n_rows,
                           hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs &a, int dk, int dv, hipStream_t stream);

struct ChunkOArgs {
    const void *q, *k, *v, *g_raw, *beta_raw;
    const float *A_log, *dt_bias, *h_chunks;
    const int32_t *cu_seqlens;
    void *o;
    int T, H;           // T: per-sequence length for dense input, total tokens if cu_seqlens
    int n_seq;          // sequences (bounds the search of a chunk row in cu_seqlens)
    float scale;
};
hipError_t launch_chunk_o(const ChunkOArgs &a, long long n_chunks, hipStream_t stream);

struct BwdArgs {
    const void *q, *k, *v, *g_raw, *beta_raw, *do_;
    const float *A_log, *dt_bias, *h_chunks, *dh_T;
    const int32_t *cu_seqlens;
    void *dq, *dk, *dv, *dg_raw, *dbeta_raw;
    float *dA_log, *ddt_bias, *dh0;
    void *work;           // caller's workspace (bwd_workspace_bytes)
    int T, H, n_seq;      // T: per-sequence length for dense input, total tokens if cu_seqlens
    long long T_all;      // total tokens
    float scale;
};
// The chunkwise backward (kda_backward.hip): bf16, d = 128.  The workspace
// holds every chunk's reverse-chain operands, gradient row and parameter sums.
size_t bwd_workspace_bytes(int n_seq, int H, long long tokens);
hipError_t launch_bwd(const BwdArgs &a, int dtype, hipStream_t stream);

}  // namespace kda
