// kda_launch.hpp -- host-side launchers of the KDA kernels (internal to the
// library; the public interface is include/kda.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Chunk-forward team ring: slots per team, bytes per slot, and the largest
// number of teams one launch uses.
#ifndef KDA_RING
#define KDA_RING 8
#endif
#define KDA_RING_SLOT_BYTES 24576   // largest slot; a launch uses its payload's copy size
#define KDA_MAX_TEAMS 256
// Per-team flag block (ints): ready[KDA_RING] at 0, used[KDA_RING] at 32, so
// each array has a cache line to itself and no line is shared between teams
// (teams run on different XCDs).
#define KDA_TEAM_FLAG_INTS 64

namespace kda {

// Producer workgroups per team of the chunkwise prefill (each builds every
// fourth chunk of the team's chains).
constexpr int KDA_PRODUCER_WGS = 4;

hipError_t launch_decode(const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                         const float *A_log, const float *dt_bias, float *pool,
                         const int32_t *state_idx, uint16_t *o, int B, int H, int HV,
                         float scale, int l2norm, hipStream_t stream);
hipError_t launch_extend(const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                         const float *A_log, const float *dt_bias, float *pool,
                         const int32_t *state_idx, uint16_t *o, int B, int T, int H, int HV,
                         float scale, int l2norm, hipStream_t stream);

hipError_t launch_conv_decode(const uint16_t *x, uint16_t *conv_state, const uint16_t *cw,
                              const uint16_t *cb, const uint16_t *a, const uint16_t *b,
                              const float *A_log, const float *dt_bias, float *pool,
                              const int32_t *state_idx, uint16_t *o, int B, int H, int HV, int W,
                              float scale, int l2norm, hipStream_t stream);

struct ChunkArgs {
    const void *q, *k, *v, *g_raw, *beta_raw;
    const float *A_log, *dt_bias, *h0;
    const int32_t *state_idx;   // NULL: h0 / h_T row = sequence; else row = state_idx[sequence] (< 0: none)
    const int32_t *cu_seqlens;
    void *o;
    float *h_T;
    float *h_chunks;     // NULL, or [N_chunks][H][DV][DK]: the state entering every chunk
    int T, H, n_seq;     // T: per-sequence length for dense input, total tokens if cu_seqlens
    float scale;
    // workspace (device memory owned by the library)
    unsigned char *ring;   // KDA_MAX_TEAMS * KDA_RING * KDA_RING_SLOT_BYTES
    int *flags;            // [KDA_MAX_TEAMS][KDA_TEAM_FLAG_INTS], then err (zeroed per launch)
    int *err;
    int n_teams;           // set by the launcher
    int teams_per_xcd;     // set by the launcher
    int pair_half;         // workgroups per XCD in the first dispatch round (0: no CU pairing)
};

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
    float *work;          // caller's workspace: the partial sums below
    float *part, *part_beta, *params;   // set by the launcher (inside work)
    int T, H, n_seq;      // T: per-sequence length for dense input, total tokens if cu_seqlens
    long long T_all;      // total tokens
    float scale;
};
size_t bwd_workspace_bytes(int n_seq, int H, long long tokens);
hipError_t launch_bwd(const BwdArgs &a, int dtype, hipStream_t stream);

// Bytes of the flag area (team blocks, then a 256-byte block for the error word).
inline size_t chunk_flag_bytes() { return sizeof(int) * ((size_t)KDA_MAX_TEAMS * KDA_TEAM_FLAG_INTS + 64); }
// Device bytes of the chunk-forward workspace.
inline size_t chunk_workspace_bytes() {
    return (size_t)KDA_MAX_TEAMS * KDA_RING * KDA_RING_SLOT_BYTES + chunk_flag_bytes();
}

// dtype: 0 = float32, 1 = bfloat16 activations.
hipError_t launch_chunk_fwd(const ChunkArgs &a, int dtype, int dk, int dv, hipStream_t stream);

}  // namespace kda
