// kda_launch.hpp -- host-side launchers of the KDA kernels (internal to the
// library; the public interface is include/kda.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Chunk-forward team ring: slots per team, bytes per slot, producer
// workgroups per team, and the largest number of teams one launch uses.
#define KDA_RING 8
#define KDA_RING_SLOT_BYTES 24576
#define KDA_PRODUCER_WGS 4
#define KDA_MAX_TEAMS 256

namespace kda {

hipError_t launch_decode(const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                         const float *A_log, const float *dt_bias, float *pool,
                         const int32_t *state_idx, uint16_t *o, int B, int H, int HV,
                         float scale, int l2norm, hipStream_t stream);

struct ChunkArgs {
    const void *q, *k, *v, *g_raw, *beta_raw;
    const float *A_log, *dt_bias, *h0;
    const int32_t *cu_seqlens;
    void *o;
    float *h_T;
    int T, H, n_seq;     // T: per-sequence length for dense input, total tokens if cu_seqlens
    float scale;
    // workspace (device memory owned by the library)
    unsigned char *ring;   // KDA_MAX_TEAMS * KDA_RING * KDA_RING_SLOT_BYTES
    int *flags;            // ready[KDA_MAX_TEAMS*KDA_RING], used[...], err  (zeroed per launch)
    int *ready, *used, *err;
    int n_teams;           // set by the launcher
};

// Device bytes of the chunk-forward workspace.
inline size_t chunk_workspace_bytes() {
    return (size_t)KDA_MAX_TEAMS * KDA_RING * KDA_RING_SLOT_BYTES +
           sizeof(int) * (2 * (size_t)KDA_MAX_TEAMS * KDA_RING + 64);
}

// dtype: 0 = float32, 1 = bfloat16 activations.
hipError_t launch_chunk_fwd(const ChunkArgs &a, int dtype, int dk, int dv, hipStream_t stream);

}  // namespace kda
