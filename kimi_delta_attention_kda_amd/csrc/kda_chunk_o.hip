// kda_chunk_o.hip -- the chunk-parallel output pass of the materialised form,
// for gfx950.
//
// [LA-06] "06 · linear 路线（一）：kernel trick、RNN 等价与三种计算形式" (chunkwise
// form) and [TL-KDA] "TileLang 实战：KDA 从零到一 -- Chunked 线性注意力" section 6
// store the state entering every chunk and then compute each chunk's outputs
// independently.  Given S0 (the state before the chunk, [dv][dk], stored by
// kda_chunk_fwd_states), per chunk of C = 16 tokens ([FKDA-LM] "FlashKDA 里的
// L 矩阵和 Mqk 矩阵是什么": L, Mqk and INV; gate and beta of [SGL-PR] "SGLang PR
// #26586 (KDA packed decode)"):
//   G_i = sum_{t<=i} g_t (per channel),  k~_i = k_i e^{G_i},  q~_i = scale q_i e^{G_i}
//   L_ij   = -beta_i sum_c k_ic k_jc e^{G_ic - G_jc}      (i > j)
//   Mqk_ij =  scale sum_c q_ic k_jc e^{G_ic - G_jc}       (i >= j)
//   U = (I - L)^{-1} beta (v - k~ S0^T),   O = q~ S0^T + Mqk U.
//
// MI355X mapping: one 256-thread workgroup per (chunk, head), no cross-
// workgroup synchronisation.  The two d_k x d_v products with the state
// (k~ S0^T, q~ S0^T) run on bf16 16x16x32 MFMA: each wave takes 32 of the 128
// output columns, and its B fragments are loaded straight from S0's rows
// (d_k is contiguous in them), issued first so the 64 KiB per workgroup
// stream in while the gate, L, Mqk and INV are built.  L and Mqk are formed
// from the per-pair exponents G_i - G_j <= 0 (no factored e^{+-G}, so nothing
// can overflow) and, with INV (forward substitution), U and O, stay in fp32.
#include <stdint.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {
constexpr int C = 16, DK = 128, DV = 128;
}

__global__ __launch_bounds__(256) void chunk_o_kernel(ChunkOArgs a)
{
    // channel-major (token index fastest), so that threads working on different
    // token pairs read different banks: gate (log2 units), then its cumulative
    // sum; scale q and k in fp32 (zero past the chunk's tokens)
    __shared__ float GT[DK][C], qT[DK][C], kT[DK][C];
    __shared__ float2 part[2][C * (C + 1) / 2];  // L and Mqk sums over the two channel halves
    __shared__ __attribute__((aligned(16))) uint16_t kt[C][DK], qt[C][DK];   // k~, q~ as bf16
    __shared__ float Lm[C][C], Mq[C][C], Inv[C][C];
    __shared__ float vs[C][DV], us[C][DV];       // v, then u; U
    __shared__ float bs[C];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, lq = lane >> 4;
    const size_t H = a.H;
    const int head = blockIdx.x % a.H;
    const size_t crow = blockIdx.x / a.H;        // h_chunks row
    // sequence and chunk of this row
    int seq, c;
    size_t bos;
    int len;
    if (a.cu_seqlens) {
        size_t acc = 0;
        seq = 0;
        for (;; ++seq) {
            const int l = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
            const size_t nchs = (size_t)((l + C - 1) / C);
            if (crow < acc + nchs) break;
            acc += nchs;
        }
        c = (int)(crow - acc);
        bos = (size_t)a.cu_seqlens[seq];
        len = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
    } else {
        const int nchk = (a.T + C - 1) / C;
        seq = (int)(crow / nchk);
        c = (int)(crow - (size_t)seq * nchk);
        bos = (size_t)seq * a.T;
        len = a.T;
    }
    const size_t tok0 = bos + (size_t)c * C;
    const int nt = min(C, len - c * C);

    // ---- S0 fragments first: wave w, column tile ct (n = 32w + 16ct + ln),
    // K-step s: channels 32s + 8lq .. + 7 of S0's row n
    const float *S0 = a.h_chunks + (crow * H + head) * (size_t)DV * DK;
    f32x4 sf[2][4][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float *p = S0 + (size_t)(32 * w + 16 * ct + ln) * DK + 32 * s + 8 * lq;
            sf[ct][s][0] = *reinterpret_cast<const f32x4 *>(p);
            sf[ct][s][1] = *reinterpret_cast<const f32x4 *>(p + 4);
        }

    // ---- inputs: thread t takes token t / 16, channels 8 (t % 16) .. + 7
    const float A = expf(a.A_log[head]);
    {
        const int t = tid >> 4, c8 = 8 * (tid & 15);
        const bool live = t < nt;
        const size_t i0 = ((tok0 + (live ? t : 0)) * H + head) * DK + c8;
        uint4 qw = make_uint4(0, 0, 0, 0), kw = qw, aw = qw, vw = qw;
        if (live) {
            qw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + i0);
            kw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + i0);
            aw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.g_raw) + i0);
            vw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + i0);
        }
        const uint32_t qa[4] = {qw.x, qw.y, qw.z, qw.w}, ka[4] = {kw.x, kw.y, kw.z, kw.w},
                       aa[4] = {aw.x, aw.y, aw.z, aw.w}, va[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sh = 16 * (e & 1);
            // g in log2 units: -A log2(1 + 2^{z log2 e}) (softplus = z above z = 20)
            const float y = (bf16_to_f32((uint16_t)(aa[e >> 1] >> sh)) + a.dt_bias[(size_t)head * DK + c8 + e]) * kLog2e;
            const float sp2 = y > 20.f * kLog2e ? y : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(y));
            GT[c8 + e][t] = live ? -A * sp2 : 0.f;
            qT[c8 + e][t] = a.scale * bf16_to_f32((uint16_t)(qa[e >> 1] >> sh));
            kT[c8 + e][t] = bf16_to_f32((uint16_t)(ka[e >> 1] >> sh));
            vs[t][c8 + e] = bf16_to_f32((uint16_t)(va[e >> 1] >> sh));
        }
        if (tid < C) {
            const float b = tid < nt ? bf16_to_f32(static_cast<const uint16_t *>(a.beta_raw)[(tok0 + tid) * H + head]) : 0.f;
            bs[tid] = tid < nt ? sigmoid_f(b) : 0.f;
        }
    }
    __syncthreads();
    // chunk-local cumulative gate, per channel
    if (tid < DK) {
        float run = 0.f;
#pragma unroll
        for (int t = 0; t < C; ++t) {
            run += GT[tid][t];
            GT[tid][t] = run;
        }
    }
    __syncthreads();
    // k~, q~ (bf16 MFMA operands); L and Mqk from per-pair exponents
    {
        const int t = tid >> 4, c8 = 8 * (tid & 15);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float eg = __builtin_amdgcn_exp2f(GT[c8 + e][t]);
            kt[t][c8 + e] = f32_to_bf16(kT[c8 + e][t] * eg);
            qt[t][c8 + e] = f32_to_bf16(qT[c8 + e][t] * eg);
        }
    }
    // L and Mqk: pair p = (i, j), i >= j, over channel half hf (tasks p + 136 hf)
    constexpr int NPAIR = C * (C + 1) / 2;
    for (int task = tid; task < 2 * NPAIR; task += 256) {
        const int hf = task >= NPAIR ? 1 : 0, p = task - hf * NPAIR;
        int i = 0;
        while ((i + 1) * (i + 2) / 2 <= p) ++i;
        const int j = p - i * (i + 1) / 2;
        float sl = 0.f, sm = 0.f;
#pragma unroll 8
        for (int cc = 64 * hf; cc < 64 * hf + 64; ++cc) {
            const float e = __builtin_amdgcn_exp2f(GT[cc][i] - GT[cc][j]);   // exponent <= 0
            const float kj = kT[cc][j] * e;
            sl += kT[cc][i] * kj;
            sm += qT[cc][i] * kj;
        }
        part[hf][p] = make_float2(sl, sm);
    }
    __syncthreads();
    if (tid < NPAIR) {
        int i = 0;
        while ((i + 1) * (i + 2) / 2 <= tid) ++i;
        const int j = tid - i * (i + 1) / 2;
        const float sl = part[0][tid].x + part[1][tid].x, sm = part[0][tid].y + part[1][tid].y;
        Lm[i][j] = i > j ? -bs[i] * sl : 0.f;
        Mq[i][j] = sm;
        if (i != j) {
            Lm[j][i] = 0.f;
            Mq[j][i] = 0.f;
        }
    }
    __syncthreads();
    // INV = (I - L)^{-1} by forward substitution, one column per thread
    if (tid < C) {
        const int j = tid;
        float x[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float s = i == j ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < C; ++m)
                if (m < i) s += Lm[i][m] * x[m];
            x[i] = i < j ? 0.f : s;
            Inv[i][j] = x[i];
        }
    }
    // W = k~ S0^T and Qs = q~ S0^T on MFMA (A fragments: row ln = token, channels 32s + 8lq ..)
    f32x4 W[2], Qs[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        W[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        Qs[ct] = W[ct];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(&kt[ln][32 * s + 8 * lq]);
        const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(&qt[ln][32 * s + 8 * lq]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                b[e] = static_cast<__bf16>(sf[ct][s][0][e]);
                b[4 + e] = static_cast<__bf16>(sf[ct][s][1][e]);
            }
            W[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, b, W[ct], 0, 0, 0);
            Qs[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, b, Qs[ct], 0, 0, 0);
        }
    }
    // u = beta (v - W): C layout, rows 4lq + r, column n
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int n = 32 * w + 16 * ct + ln;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lq + r;
            us[i][n] = bs[i] * (vs[i][n] - W[ct][r]);
        }
    }
    __syncthreads();
    // U = INV u (fp32), into vs
    f32x4 U[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int n = 32 * w + 16 * ct + ln;
        float ucol[C];
#pragma unroll
        for (int m = 0; m < C; ++m) ucol[m] = us[m][n];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lq + r;
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < C; ++m) s += Inv[i][m] * ucol[m];
            U[ct][r] = s;
        }
    }
    __syncthreads();   // all of u read before U overwrites the v buffer
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int n = 32 * w + 16 * ct + ln;
#pragma unroll
        for (int r = 0; r < 4; ++r) vs[4 * lq + r][n] = U[ct][r];
    }
    __syncthreads();
    // O = Qs + Mqk U, stored for the chunk's tokens
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int n = 32 * w + 16 * ct + ln;
        float Ucol[C];
#pragma unroll
        for (int m = 0; m < C; ++m) Ucol[m] = vs[m][n];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lq + r;
            float s = Qs[ct][r];
#pragma unroll
            for (int m = 0; m < C; ++m) s += Mq[i][m] * Ucol[m];
            if (i < nt) static_cast<uint16_t *>(a.o)[((tok0 + i) * H + head) * DV + n] = f32_to_bf16(s);
        }
    }
}

hipError_t launch_chunk_o(const ChunkOArgs &a, long long n_chunks, hipStream_t stream)
{
    if (n_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(chunk_o_kernel, dim3((unsigned)(n_chunks * a.H)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
