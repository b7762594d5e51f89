// kda_backward.hip -- gradients of the KDA forward for gfx950: the entry
// point's launcher and the final reduction of the gate parameters' gradients.
//
// The backward is chunkwise ([LA-06] "06 · linear 路线（一）：kernel trick、RNN
// 等价与三种计算形式", chunkwise form: a reverse loop over chunks from the
// states stored at chunk boundaries; gate and beta of [SGL-PR] "SGLang PR
// #26586 (KDA packed decode)").  Its three passes live with the forward's
// kernels, whose operand layouts and helpers they share (kda_fwd.hip):
//   1. the reverse chain's state-independent operands of every chunk, all
//      chunks in parallel (the forward's prep);
//   2. the reverse chain: one sequential loop over the chunks of each
//      (sequence, head) that carries dS (the gradient with respect to the
//      state) in fp32 MFMA accumulators, leaving dS and dU for every chunk;
//   3. every chunk's gradients of q, k, v, g_raw and beta_raw in parallel, and
//      the chunk's sums of the gradients of dt_bias and A_log.
// Here those per-chunk sums are added: first over BWD_SPLIT slices of chunk
// rows, then over the slices, in a fixed order (deterministic, no atomics).
#include <stdint.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {
constexpr int NP = 128 + 1;   // d dt_bias (128 channels), d A_log

// Slice b of the rows of head h: the column sums of rows [b * per, (b + 1) * per).
__global__ __launch_bounds__(192) void params_slice_kernel(const float *__restrict__ part, float *__restrict__ red,
                                                           int n_rows, int H)
{
    const int b = blockIdx.x, head = blockIdx.y, col = threadIdx.x;
    if (col >= NP) return;
    const int per = (n_rows + BWD_SPLIT - 1) / BWD_SPLIT;
    const int r0 = b * per, r1 = min(n_rows, r0 + per);
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    int r = r0;
    for (; r + 4 <= r1; r += 4)
#pragma unroll
        for (int u = 0; u < 4; ++u) s[u] += part[((size_t)(r + u) * H + head) * NP + col];
    for (int u = 0; r < r1; ++r, ++u) s[u] += part[((size_t)r * H + head) * NP + col];
    red[((size_t)head * BWD_SPLIT + b) * NP + col] = (s[0] + s[1]) + (s[2] + s[3]);
}

__global__ __launch_bounds__(192) void params_final_kernel(const float *__restrict__ red, float *__restrict__ dA_log,
                                                           float *__restrict__ ddt_bias)
{
    const int head = blockIdx.x, col = threadIdx.x;
    if (col >= NP) return;
    float s = 0.f;
    for (int b = 0; b < BWD_SPLIT; ++b) s += red[((size_t)head * BWD_SPLIT + b) * NP + col];
    if (col < NP - 1) {
        if (ddt_bias) ddt_bias[(size_t)head * (NP - 1) + col] = s;
    } else if (dA_log) {
        dA_log[head] = s;
    }
}

// Chunk rows of n_seq sequences holding `tokens` tokens in all: at most one
// partial chunk per sequence.
long long bwd_rows_bound(int n_seq, long long tokens) { return (tokens + 15) / 16 + n_seq; }
}  // namespace

size_t bwd_workspace_bytes(int n_seq, int H, long long tokens)
{
    return bwd_ws_layout(bwd_rows_bound(n_seq, tokens), H).bytes;
}

hipError_t launch_bwd(const BwdArgs &a, int dtype, hipStream_t stream)
{
    if ((long long)a.n_seq * a.H == 0) return hipSuccess;
    if (dtype != 1) return hipErrorInvalidValue;
    const long long rows = bwd_rows_bound(a.n_seq, a.T_all);
    if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipError_t e = launch_bwd_chunkwise(a, rows, stream);
    if (e != hipSuccess) return e;
    const BwdWs l = bwd_ws_layout(rows, a.H);
    unsigned char *ws = static_cast<unsigned char *>(a.work);
    hipLaunchKernelGGL(params_slice_kernel, dim3(BWD_SPLIT, (unsigned)a.H), dim3(192), 0, stream,
                       reinterpret_cast<const float *>(ws + l.part), reinterpret_cast<float *>(ws + l.red), (int)rows,
                       a.H);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(params_final_kernel, dim3((unsigned)a.H), dim3(192), 0, stream,
                       reinterpret_cast<const float *>(ws + l.red), a.dA_log, a.ddt_bias);
    return hipGetLastError();
}

}  // namespace kda
