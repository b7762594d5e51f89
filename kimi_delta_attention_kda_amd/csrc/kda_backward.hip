// kda_backward.hip -- gradients of the KDA forward for gfx950.
//
// The forward, per (sequence, head) and token t ([TL-KDA] "TileLang 实战：KDA
// 从零到一 -- Chunked 线性注意力" section 1; gate and beta of [SGL-PR] "SGLang PR
// #26586 (KDA packed decode)", implementation notes item 1):
//   z = a_t + dt_bias, g = -A softplus(z) with A = exp(A_log), e = exp(g),
//   beta = sigmoid(b_t), qb = scale q_t,
//   S' = S Diag(e);  w = S' k;  u = beta (v - w);  S+ = S' + u k^T;  o = S+ qb.
// Its adjoint, with D the gradient of the loss with respect to S+:
//   D += do qb^T;            dqb = S+^T do
//   du = D k;                dk += D^T u;           dS' = D
//   dv = beta du;            dbeta = du . (v - w);  dw = -beta du
//   dS' += dw k^T;           dk += S'^T dw
//   dg = sum_rows(dS' o S'); D <- dS' Diag(e)       (gradient for S)
//   dz = -A sigmoid(z) dg;   dA_log += dg . g;      ddt_bias += dz;  db = dbeta beta (1 - beta)
// [LA-06] "06 · linear 路线（一）" (chunkwise form) runs the backward as a
// reverse loop over chunks from the states stored at chunk boundaries; this
// kernel does the same: chunks in reverse, each restarted from its stored
// entering state (kda_chunk_fwd_states), its 16 per-token states recomputed in
// fp32 and kept in the caller's workspace, then the adjoint token by token.
//
// MI355X mapping: one 512-thread workgroup per (sequence, head) chain, the
// state and its gradient in registers on the T=1 decode kernel's layout
// (half p, thread (g, j): rows 64p + g + 16r, r < 4, and columns 4j.., 64+4j..).
// Row sums (w, du) run over the 16 lanes of a row group with DPP; column sums
// (dq, dk, dg) and the beta sum over rows go through LDS.  No atomics: the
// result is deterministic.  The per-chain sums of dA_log and ddt_bias are
// reduced over sequences by a second small kernel.
#include <stdint.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int BCH = 16;      // tokens per chunk (the forward's chunk and snapshot spacing)
constexpr int BK = 128, BV = 128;

template <bool BF16>
__device__ __forceinline__ float ld(const void *p, size_t i) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
    else return static_cast<const float *>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ void st(void *p, size_t i, float x) {
    if constexpr (BF16) static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
    else static_cast<float *>(p)[i] = x;
}

}  // namespace

template <bool BF16>
__global__ __launch_bounds__(512) void bwd_kernel(BwdArgs a)
{
    constexpr int ROWS = BV / 32;
    __shared__ f32x4 Lq[BCH][BK / 4], Lk[BCH][BK / 4], Le[BCH][BK / 4], Lg[BCH][BK / 4], Ls[BCH][BK / 4];
    __shared__ float Lv[BCH][BV], Ldo[BCH][BV], Lu[BCH][BV], Lvw[BCH][BV];
    __shared__ float Lbeta[BCH];
    __shared__ float red[3][32][BK];     // column partials of dqb, dk, dg per row group
    __shared__ float rowred[32];         // beta-gradient partials per row group

    const int chain = blockIdx.x;
    const int seq = chain / a.H, head = chain - seq * a.H;
    size_t bos;
    int len;
    size_t cbase;   // h_chunks row of this sequence's first chunk
    if (a.cu_seqlens) {
        bos = (size_t)a.cu_seqlens[seq];
        len = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
        cbase = 0;
        for (int s2 = 0; s2 < seq; ++s2) cbase += (size_t)((a.cu_seqlens[s2 + 1] - a.cu_seqlens[s2] + BCH - 1) / BCH);
    } else {
        bos = (size_t)seq * a.T;
        len = a.T;
        cbase = (size_t)seq * ((a.T + BCH - 1) / BCH);
    }
    const int nch = (len + BCH - 1) / BCH;
    const int tid = threadIdx.x;
    const int half = tid >> 8, tl = tid & 255, g = tl >> 4, j = tl & 15;
    const int r0 = 64 * half;
    const int grp = 16 * half + g;                    // row group 0..31
    const size_t H = a.H;
    const float A = expf(a.A_log[head]);

    // gradient of the state after the last token
    f32x4 D[ROWS][2];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            if (a.dh_T) {
                const size_t at = (((size_t)seq * H + head) * BV + r0 + g + 16 * r) * BK + 4 * j + 64 * h2;
                D[r][h2] = *reinterpret_cast<const f32x4 *>(a.dh_T + at);
            } else {
                D[r][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    float acc_dt = 0.f, acc_A = 0.f;   // threads 256..383 own column tid - 256 of ddt_bias / dA_log
    float *scr = a.work + (size_t)chain * BCH * BV * BK;

    for (int c = nch - 1; c >= 0; --c) {
        const int t0 = c * BCH;
        const int nt = min(BCH, len - t0);
        // ---- stage the chunk's per-token values
        {
            const int tt = tid >> 5, c4 = 4 * (tid & 31);
            if (tt < nt) {
                const size_t tok = bos + t0 + tt;
                f32x4 qv, kv, ev, gv, sv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t i = (tok * H + head) * BK + c4 + e;
                    const float z = ld<BF16>(a.g_raw, i) + a.dt_bias[(size_t)head * BK + c4 + e];
                    const float sp = z > 20.f ? z : log1pf(expf(z));
                    qv[e] = a.scale * ld<BF16>(a.q, i);
                    kv[e] = ld<BF16>(a.k, i);
                    gv[e] = -A * sp;
                    ev[e] = expf(gv[e]);
                    sv[e] = sigmoid_f(z);
                }
                Lq[tt][tid & 31] = qv;
                Lk[tt][tid & 31] = kv;
                Le[tt][tid & 31] = ev;
                Lg[tt][tid & 31] = gv;
                Ls[tt][tid & 31] = sv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t iv = (tok * H + head) * BV + c4 + e;
                    Lv[tt][c4 + e] = ld<BF16>(a.v, iv);
                    Ldo[tt][c4 + e] = ld<BF16>(a.do_, iv);
                }
            }
            if (tid < nt) Lbeta[tid] = sigmoid_f(ld<BF16>(a.beta_raw, (bos + t0 + tid) * H + head));
        }
        __syncthreads();

        // ---- forward recompute from the stored entering state; keep every token's
        // entering state (this thread's elements) in the workspace
        f32x4 S[ROWS][2];
        {
            const float *hc = a.h_chunks + ((cbase + c) * H + head) * (size_t)BV * BK;
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    S[r][h2] = *reinterpret_cast<const f32x4 *>(hc + (size_t)(r0 + g + 16 * r) * BK + 4 * j + 64 * h2);
        }
        for (int tt = 0; tt < nt; ++tt) {
            float *sc = scr + (size_t)tt * BV * BK;
            f32x4 e4[2], k4[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                e4[h2] = Le[tt][j + 16 * h2];
                k4[h2] = Lk[tt][j + 16 * h2];
            }
            const float beta = Lbeta[tt];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const int row = r0 + g + 16 * r;
                float w = 0.f;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    *reinterpret_cast<f32x4 *>(sc + (size_t)row * BK + 4 * j + 64 * h2) = S[r][h2];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        S[r][h2][e] *= e4[h2][e];
                        w += S[r][h2][e] * k4[h2][e];
                    }
                }
                w = row16_sum(w);
                const float vw = Lv[tt][row] - w;
                const float u = beta * vw;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[r][h2][e] += u * k4[h2][e];
                if (j == 0) {
                    Lu[tt][row] = u;
                    Lvw[tt][row] = vw;
                }
            }
        }
        __syncthreads();

        // ---- adjoint, tokens in reverse
        for (int tt = nt - 1; tt >= 0; --tt) {
            const size_t tok = bos + t0 + tt;
            const float *sc = scr + (size_t)tt * BV * BK;
            f32x4 e4[2], k4[2], q4[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                e4[h2] = Le[tt][j + 16 * h2];
                k4[h2] = Lk[tt][j + 16 * h2];
                q4[h2] = Lq[tt][j + 16 * h2];
            }
            const float beta = Lbeta[tt];
            f32x4 pq[2] = {}, pk[2] = {}, pg[2] = {};
            float pb = 0.f;
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const int row = r0 + g + 16 * r;
                const float u = Lu[tt][row], vw = Lvw[tt][row], dO = Ldo[tt][row];
                f32x4 Sd[2], Sp[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sc + (size_t)row * BK + 4 * j + 64 * h2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Sd[h2][e] = s0[e] * e4[h2][e];           // S'
                        Sp[h2][e] = Sd[h2][e] + u * k4[h2][e];   // S+
                    }
                }
                float du = 0.f;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        D[r][h2][e] += dO * q4[h2][e];
                        pq[h2][e] += Sp[h2][e] * dO;
                        du += D[r][h2][e] * k4[h2][e];
                    }
                du = row16_sum(du);
                const float dw = -beta * du;
                if (j == 0) {
                    st<BF16>(a.dv, (tok * H + head) * BV + row, beta * du);
                    pb += du * vw;
                }
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float dSd = D[r][h2][e] + dw * k4[h2][e];
                        pk[h2][e] += D[r][h2][e] * u + Sd[h2][e] * dw;
                        pg[h2][e] += dSd * Sd[h2][e];
                        D[r][h2][e] = dSd * e4[h2][e];
                    }
            }
            // column partials of this row group -> LDS
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                *reinterpret_cast<f32x4 *>(&red[0][grp][4 * j + 64 * h2]) = pq[h2];
                *reinterpret_cast<f32x4 *>(&red[1][grp][4 * j + 64 * h2]) = pk[h2];
                *reinterpret_cast<f32x4 *>(&red[2][grp][4 * j + 64 * h2]) = pg[h2];
            }
            if (j == 0) rowred[grp] = pb;
            __syncthreads();
            if (tid < 3 * BK) {
                const int qty = tid >> 7, col = tid & (BK - 1);
                float sum = 0.f;
#pragma unroll 8
                for (int gg = 0; gg < 32; ++gg) sum += red[qty][gg][col];
                const size_t i = (tok * H + head) * BK + col;
                if (qty == 0) {
                    st<BF16>(a.dq, i, a.scale * sum);
                } else if (qty == 1) {
                    st<BF16>(a.dk, i, sum);
                } else {
                    const f32x4 gz = Lg[tt][col >> 2], sz = Ls[tt][col >> 2];
                    const float dz = -A * sz[col & 3] * sum;
                    st<BF16>(a.dg_raw, i, dz);
                    acc_dt += dz;
                    acc_A += sum * gz[col & 3];
                }
            } else if (tid == 3 * BK) {
                float sb = 0.f;
                for (int gg = 0; gg < 32; ++gg) sb += rowred[gg];
                const float beta_t = Lbeta[tt];
                st<BF16>(a.dbeta_raw, tok * H + head, sb * beta_t * (1.f - beta_t));
            }
            __syncthreads();
        }
    }

    // gradient of the initial state
    if (a.dh0) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const size_t at = (((size_t)seq * H + head) * BV + r0 + g + 16 * r) * BK + 4 * j + 64 * h2;
                *reinterpret_cast<f32x4 *>(a.dh0 + at) = D[r][h2];
            }
    }
    // this chain's sums for ddt_bias (per channel) and dA_log
    float *part = a.work_params + (size_t)chain * (BK + 1);
    if (tid >= 2 * BK && tid < 3 * BK) part[tid - 2 * BK] = acc_dt;
    // dA_log: sum the 128 column threads' terms (they are waves 4 and 5)
    __syncthreads();
    if (tid >= 2 * BK && tid < 3 * BK) red[0][0][tid - 2 * BK] = acc_A;
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
        for (int cc = 0; cc < BK; ++cc) s += red[0][0][cc];
        part[BK] = s;
    }
}

// dA_log[h] and ddt_bias[h, :] from the per-chain sums, summed over sequences.
__global__ __launch_bounds__(128) void bwd_params_kernel(const float *__restrict__ part, float *__restrict__ dA_log,
                                                          float *__restrict__ ddt_bias, int n_seq, int H)
{
    const int head = blockIdx.x, col = threadIdx.x;
    float sdt = 0.f, sA = 0.f;
    for (int s = 0; s < n_seq; ++s) {
        const float *p = part + ((size_t)s * H + head) * (BK + 1);
        sdt += p[col];
        if (col == 0) sA += p[BK];
    }
    if (ddt_bias) ddt_bias[(size_t)head * BK + col] = sdt;
    if (col == 0 && dA_log) dA_log[head] = sA;
}

size_t bwd_workspace_bytes(int n_seq, int H)
{
    const size_t chains = (size_t)n_seq * H;
    return chains * ((size_t)BCH * BV * BK + BK + 1) * sizeof(float);
}

hipError_t launch_bwd(const BwdArgs &args, int dtype, hipStream_t stream)
{
    BwdArgs a = args;
    const int n_chains = a.n_seq * a.H;
    if (n_chains == 0) return hipSuccess;
    a.work_params = a.work + (size_t)n_chains * BCH * BV * BK;
    if (dtype != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_kernel<true>, dim3((unsigned)n_chains), dim3(512), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_params_kernel, dim3((unsigned)a.H), dim3(BK), 0, stream, a.work_params, a.dA_log,
                       a.ddt_bias, a.n_seq, a.H);
    return hipGetLastError();
}

}  // namespace kda
