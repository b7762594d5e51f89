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
// fp32 and kept in registers (both token loops fully unrolled, 128 VGPRs of
// history per thread), then the adjoint token by token.
//
// MI355X mapping: four 512-thread workgroups per (sequence, head) chain, one
// per quarter of the state's 128 rows (rows are independent given the token's
// vectors), so the prefill workload's 64 chains fill 256 compute units.  A
// thread holds one row and 8 columns (4j.., 64+4j..) of the state and of its
// gradient in registers; the row sums (w, du) run over the 16 lanes of a row
// group with DPP.  The column sums (dq, dk, dg) and the beta sum over a
// quarter's rows go through LDS and are written per token and quarter; a
// second kernel adds the quarters, applies the chain rule through the gate
// and beta, and sums dA_log and ddt_bias over token blocks, and a third sums
// those blocks.  No atomics: the result is deterministic.
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

constexpr int NQ = 4;            // row quarters per chain (workgroups per chain)
constexpr int QR = BV / NQ;      // rows per workgroup
constexpr int TB = 16;           // tokens per block of the finishing kernel

template <bool BF16>
__global__ __launch_bounds__(512) void bwd_kernel(BwdArgs a)
{
    __shared__ f32x4 Lq[BCH][BK / 4], Lk[BCH][BK / 4], Le[BCH][BK / 4];
    __shared__ float Lv[BCH][QR], Ldo[BCH][QR], Lu[BCH][QR], Lvw[BCH][QR];
    __shared__ float Lbeta[BCH];
    __shared__ float Ldtb[BK];                  // dt_bias of the head
    // column partials of dqb, dk, dg and the beta terms per row, double-buffered
    // over tokens so one barrier per token suffices: token t's partials are
    // summed while token t-1's are written to the other buffer, and the barrier
    // of token t-1 orders the sums of t before the writes of t-2
    __shared__ float red[2][3][QR][BK];
    __shared__ float rowred[2][QR];

    const int chain = blockIdx.x / NQ, quarter = blockIdx.x - chain * NQ;
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
    const int g = tid >> 4, j = tid & 15;             // row g of the quarter, columns 4j.., 64+4j..
    const int row = quarter * QR + g;
    const size_t H = a.H;
    const float A = expf(a.A_log[head]);

    // gradient of the state after the last token (this thread's row and columns)
    f32x4 D[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        if (a.dh_T) {
            const size_t at = (((size_t)seq * H + head) * BV + row) * BK + 4 * j + 64 * h2;
            D[h2] = *reinterpret_cast<const f32x4 *>(a.dh_T + at);
        } else {
            D[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // A chunk's inputs as this thread loads them (token tid / 32, channels
    // 4 (tid % 32) .. + 3 of q, k and g_raw; this quarter's v and do of row
    // tid % 32; beta of token tid if tid < 16) and its entering state (this
    // thread's elements).  The next chunk's are loaded halfway through this
    // chunk's adjoint, when half the history registers are free, so no chunk
    // waits for memory.  Tokens past the sequence repeat its last token (in
    // bounds; never used).
    struct Raw {
        float q[4], k[4], g[4], v, dO, b;
        f32x4 S[2];
    } raw;
    const int st_t = tid >> 5, st_c4 = 4 * (tid & 31), st_r = tid & 31;
    auto load_raw = [&](int c) {
        const int nt = min(BCH, len - c * BCH);
        const size_t tok = bos + (size_t)c * BCH + min(st_t, nt - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t i = (tok * H + head) * BK + st_c4 + e;
            raw.q[e] = ld<BF16>(a.q, i);
            raw.k[e] = ld<BF16>(a.k, i);
            raw.g[e] = ld<BF16>(a.g_raw, i);
        }
        const size_t iv = (tok * H + head) * BV + quarter * QR + st_r;
        raw.v = ld<BF16>(a.v, iv);
        raw.dO = ld<BF16>(a.do_, iv);
        raw.b = tid < nt ? ld<BF16>(a.beta_raw, (bos + (size_t)c * BCH + tid) * H + head) : 0.f;
        const float *hc = a.h_chunks + (((cbase + c) * H + head) * BV + row) * (size_t)BK;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) raw.S[h2] = *reinterpret_cast<const f32x4 *>(hc + 4 * j + 64 * h2);
    };
    if (nch > 0) load_raw(nch - 1);
    if (tid < BK) Ldtb[tid] = a.dt_bias[(size_t)head * BK + tid];
    __syncthreads();

    for (int c = nch - 1; c >= 0; --c) {
        const int t0 = c * BCH;
        const int nt = min(BCH, len - t0);
        // ---- stage the chunk's per-token values
        {
            const int tt = st_t;
            if (tt < nt) {
                f32x4 qv, kv, ev;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qv[e] = a.scale * raw.q[e];
                    kv[e] = raw.k[e];
                    ev[e] = gate_decay(raw.g[e] + Ldtb[st_c4 + e], A);   // hardware exp2 / log2
                }
                Lq[tt][tid & 31] = qv;
                Lk[tt][tid & 31] = kv;
                Le[tt][tid & 31] = ev;
                Lv[tt][st_r] = raw.v;
                Ldo[tt][st_r] = raw.dO;
            }
            if (tid < nt) Lbeta[tid] = sigmoid_f(raw.b);
        }
        __syncthreads();

        // ---- forward recompute from the stored entering state; keep every token's
        // entering state (this thread's elements) in registers
        f32x4 S[2] = {raw.S[0], raw.S[1]};
        f32x4 hist[BCH][2];   // entering state of every token of the chunk (this thread's elements)
#pragma unroll
        for (int tt = 0; tt < BCH; ++tt) {
            if (tt < nt) {
            float w = 0.f;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const f32x4 e4 = Le[tt][j + 16 * h2], k4 = Lk[tt][j + 16 * h2];
                hist[tt][h2] = S[h2];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    S[h2][e] *= e4[e];
                    w += S[h2][e] * k4[e];
                }
            }
            w = row16_sum(w);
            const float vw = Lv[tt][g] - w;
            const float u = Lbeta[tt] * vw;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const f32x4 k4 = Lk[tt][j + 16 * h2];
#pragma unroll
                for (int e = 0; e < 4; ++e) S[h2][e] += u * k4[e];
            }
            if (j == 0) {
                Lu[tt][g] = u;
                Lvw[tt][g] = vw;
            }
            }
        }
        __syncthreads();

        // ---- adjoint, tokens in reverse (fully unrolled: the history stays in registers)
#pragma unroll
        for (int tt = BCH - 1; tt >= 0; --tt) {
            if (tt == BCH / 2 - 1 && c > 0) load_raw(c - 1);   // half the history is free now
            if (tt < nt) {
            const size_t tok = bos + t0 + tt;
            const int rb = tt & 1;
            const f32x4 scur[2] = {hist[tt][0], hist[tt][1]};
            const float beta = Lbeta[tt];
            const float u = Lu[tt][g], vw = Lvw[tt][g], dO = Ldo[tt][g];
            f32x4 e4[2], k4[2], Sd[2], Sp[2];
            float du = 0.f;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                e4[h2] = Le[tt][j + 16 * h2];
                k4[h2] = Lk[tt][j + 16 * h2];
                const f32x4 q4 = Lq[tt][j + 16 * h2];
                const f32x4 s0 = scur[h2];
                f32x4 pq;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Sd[h2][e] = s0[e] * e4[h2][e];              // S'
                    Sp[h2][e] = Sd[h2][e] + u * k4[h2][e];      // S+
                    D[h2][e] += dO * q4[e];
                    pq[e] = Sp[h2][e] * dO;
                    du += D[h2][e] * k4[h2][e];
                }
                *reinterpret_cast<f32x4 *>(&red[rb][0][g][4 * j + 64 * h2]) = pq;
            }
            du = row16_sum(du);
            const float dw = -beta * du;
            if (j == 0) {
                st<BF16>(a.dv, (tok * H + head) * BV + row, beta * du);
                rowred[rb][g] = du * vw;
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                f32x4 pk, pg;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float dSd = D[h2][e] + dw * k4[h2][e];
                    pk[e] = D[h2][e] * u + Sd[h2][e] * dw;
                    pg[e] = dSd * Sd[h2][e];
                    D[h2][e] = dSd * e4[h2][e];
                }
                *reinterpret_cast<f32x4 *>(&red[rb][1][g][4 * j + 64 * h2]) = pk;
                *reinterpret_cast<f32x4 *>(&red[rb][2][g][4 * j + 64 * h2]) = pg;
            }
            __syncthreads();
            // this quarter's column sums and beta term for the token
            if (tid < 3 * BK) {
                const int qty = tid >> 7, col = tid & (BK - 1);
                float sum = 0.f;
#pragma unroll 8
                for (int gg = 0; gg < QR; ++gg) sum += red[rb][qty][gg][col];
                a.part[((size_t)quarter * a.T_all + tok) * H * (3 * BK) + head * (3 * BK) + qty * BK + col] = sum;
            } else if (tid == 3 * BK) {
                float sb = 0.f;
                for (int gg = 0; gg < QR; ++gg) sb += rowred[rb][gg];
                a.part_beta[((size_t)quarter * a.T_all + tok) * H + head] = sb;
            }
            }
        }
        __syncthreads();   // the chunk's sums done before the next chunk's staging and writes
    }

    // gradient of the initial state
    if (a.dh0) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const size_t at = (((size_t)seq * H + head) * BV + row) * BK + 4 * j + 64 * h2;
            *reinterpret_cast<f32x4 *>(a.dh0 + at) = D[h2];
        }
    }
}

// Per token block and head: add the quarters' column sums and apply the chain
// rule through q's scale, the gate (dz = -A sigmoid(z) dg with
// z = g_raw + dt_bias) and beta (db = dbeta beta (1 - beta)); the block's sums
// of dz (ddt_bias) and dg . g (dA_log) go to params[block][head].
template <bool BF16>
__global__ __launch_bounds__(BK) void bwd_finish_kernel(BwdArgs a)
{
    __shared__ float sA[BK];
    const int blk = blockIdx.x, head = blockIdx.y, col = threadIdx.x;
    const size_t H = a.H;
    const float A = expf(a.A_log[head]);
    const float dtb = a.dt_bias[(size_t)head * BK + col];
    float acc_dt = 0.f, acc_A = 0.f;
    const size_t tend = min((size_t)a.T_all, (size_t)(blk + 1) * TB);
#pragma unroll 4
    for (size_t tok = (size_t)blk * TB; tok < tend; ++tok) {
        float sq = 0.f, sk = 0.f, sg = 0.f;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
            const float *p = a.part + ((size_t)qq * a.T_all + tok) * H * (3 * BK) + head * (3 * BK);
            sq += p[col];
            sk += p[BK + col];
            sg += p[2 * BK + col];
        }
        const size_t i = (tok * H + head) * BK + col;
        st<BF16>(a.dq, i, a.scale * sq);
        st<BF16>(a.dk, i, sk);
        const float z = ld<BF16>(a.g_raw, i) + dtb;
        const float sp = z > 20.f ? z : log1pf(expf(z));
        const float dz = -A * sigmoid_f(z) * sg;
        st<BF16>(a.dg_raw, i, dz);
        acc_dt += dz;
        acc_A += sg * (-A * sp);
        if (col == 0) {
            float sb = 0.f;
#pragma unroll
            for (int qq = 0; qq < NQ; ++qq) sb += a.part_beta[((size_t)qq * a.T_all + tok) * H + head];
            const float beta = sigmoid_f(ld<BF16>(a.beta_raw, tok * H + head));
            st<BF16>(a.dbeta_raw, tok * H + head, sb * beta * (1.f - beta));
        }
    }
    float *pp = a.params + ((size_t)blk * H + head) * (BK + 1);
    pp[col] = acc_dt;
    sA[col] = acc_A;
    __syncthreads();
    if (col == 0) {
        float s = 0.f;
        for (int cc = 0; cc < BK; ++cc) s += sA[cc];
        pp[BK] = s;
    }
}

// dA_log[h] and ddt_bias[h, :] from the per-block sums.
__global__ __launch_bounds__(BK) void bwd_params_kernel(const float *__restrict__ part, float *__restrict__ dA_log,
                                                         float *__restrict__ ddt_bias, int n_blk, int H)
{
    const int head = blockIdx.x, col = threadIdx.x;
    // eight independent partial sums keep eight loads in flight (fixed order: deterministic)
    float sdt[8] = {}, sA[8] = {};
    int s = 0;
    for (; s + 8 <= n_blk; s += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float *p = part + ((size_t)(s + u) * H + head) * (BK + 1);
            sdt[u] += p[col];
            if (col == 0) sA[u] += p[BK];
        }
    }
    for (int u = 0; s < n_blk; ++s, ++u) {
        const float *p = part + ((size_t)s * H + head) * (BK + 1);
        sdt[u] += p[col];
        if (col == 0) sA[u] += p[BK];
    }
    float tdt = 0.f, tA = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) { tdt += sdt[u]; tA += sA[u]; }
    if (ddt_bias) ddt_bias[(size_t)head * BK + col] = tdt;
    if (col == 0 && dA_log) dA_log[head] = tA;
}

size_t bwd_workspace_bytes(int n_seq, int H, long long tokens)
{
    (void)n_seq;
    const size_t nblk = (size_t)((tokens + TB - 1) / TB);
    return sizeof(float) * ((size_t)NQ * tokens * H * (3 * BK + 1)   // quarter column sums, beta terms
                            + nblk * H * (BK + 1));                    // block parameter sums
}

hipError_t launch_bwd(const BwdArgs &args, int dtype, hipStream_t stream)
{
    BwdArgs a = args;
    const int n_chains = a.n_seq * a.H;
    if (n_chains == 0) return hipSuccess;
    if (dtype != 1) return hipErrorInvalidValue;
    const size_t H = a.H;
    a.part = a.work;
    a.part_beta = a.part + (size_t)NQ * a.T_all * H * (3 * BK);
    a.params = a.part_beta + (size_t)NQ * a.T_all * H;
    const int nblk = (int)((a.T_all + TB - 1) / TB);
    if (a.T_all > 0) {
        hipLaunchKernelGGL(bwd_kernel<true>, dim3((unsigned)(n_chains * NQ)), dim3(512), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(bwd_finish_kernel<true>, dim3((unsigned)nblk, (unsigned)a.H), dim3(BK), 0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        // no tokens: dh0 = dh_T; parameter gradients zero
        hipLaunchKernelGGL(bwd_kernel<true>, dim3((unsigned)(n_chains * NQ)), dim3(512), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(bwd_params_kernel, dim3((unsigned)a.H), dim3(BK), 0, stream, a.params, a.dA_log,
                       a.ddt_bias, nblk, a.H);
    return hipGetLastError();
}

}  // namespace kda
