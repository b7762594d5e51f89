// kda_fwd_f32.hip -- chunkwise KDA prefill with fp32 activations (d_k = 64),
// for gfx950.
//
// Pages cited by title and section:
//   [TL-KDA]  "TileLang 实战：KDA 从零到一 -- Chunked 线性注意力": section 1
//             (recurrence, (d_v, d_k) state), 6.4 (sequential chunk loop in
//             the block), 6.4.2 (state update after the chunk's output).
//   [FKDA-LM] "FlashKDA 里的 L 矩阵和 Mqk 矩阵是什么": "30秒速览", "L 矩阵的构造",
//             "Mqk 矩阵的构造", "K2 内核如何消费".
//   [SGL-PR]  "SGLang PR #26586 (KDA packed decode)": gate and beta formulas.
//
// The fp32 build serves the small fp32 workload, whose tolerance (1e-4
// max-abs) asks for fp32 arithmetic throughout.  One 256-thread workgroup per
// (sequence, head) walks its chunks in order with everything in LDS:
//   * the next chunk's inputs loaded into registers while the current chunk
//     computes;
//   * gate and per-token decays per (token, channel), the cumulative gate per
//     channel (one thread per channel, 16 adds), the decayed operands per
//     (token, channel);
//   * L and Mqk exactly: for column j the factor e^{G_i - G_j} of rows i >= j
//     is the running product of the tokens' decays (all <= 1), so no factored
//     e^{+-G} can overflow; the channel sums are 16-lane DPP reductions;
//   * W = k~ S, Qs = q~ S, O = Qs + Mqk U and S <- Diag(e^{G_C}) S + k^r^T U on
//     the fp32 matrix core (v_mfma_f32_16x16x4f32), operands read from LDS;
//   * U from (I - L) U = beta (v - W) by forward substitution (one thread per
//     state column), which is the Neumann product INV u of the pages computed
//     row by row.
#include <stdint.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int CH = 16, DK = 64, NTHR = 256;

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void sync_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int DV>
struct F32Lay {
    float q[CH][DK], k[CH][DK], kt[CH][DK], qt[CH][DK], kr[CH][DK], dd[CH][DK];
    float v[CH][DV], u[CH][DV];
    float S[DK][DV];
    float Lm[CH][CH], Mq[CH][CH];
    float beta[CH], eg[DK], gc[DK];
};

}  // namespace

template <int DV, bool SNAP>
__global__ __launch_bounds__(NTHR) void fwd_f32_kernel(FwdArgs a)
{
    __shared__ __attribute__((aligned(16))) F32Lay<DV> sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 15, lq = lane >> 4;
    const int seq = blockIdx.x / a.H, head = blockIdx.x % a.H;
    size_t bos;
    int len;
    if (a.cu_seqlens) {
        bos = (size_t)a.cu_seqlens[seq];
        len = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
    } else {
        bos = (size_t)seq * a.T;
        len = a.T;
    }
    const int nch = (len + CH - 1) / CH;
    int hrow = a.state_idx ? a.state_idx[seq] : seq;
    if (a.state_idx && hrow >= a.P) {
        if (tid == 0) slot_error(a.err);
        hrow = -1;
    }
    const size_t H = a.H;
    const size_t hb = ((size_t)(hrow < 0 ? 0 : hrow) * H + head) * DV * DK;
    // state as S[c][v] (d_k x d_v); memory rows are [v][c]
    for (int i = tid; i < DK * DV; i += NTHR) {
        const int vv = i / DK, cc = i % DK;
        sm.S[cc][vv] = (a.h0 && hrow >= 0) ? a.h0[hb + i] : 0.f;
    }
    size_t cbase = 0;
    if (SNAP) {
        if (a.cu_seqlens) {
            for (int s2 = 0; s2 < seq; ++s2) cbase += (size_t)((a.cu_seqlens[s2 + 1] - a.cu_seqlens[s2] + CH - 1) / CH);
        } else {
            cbase = (size_t)seq * ((a.T + CH - 1) / CH);
        }
    }
    const float A_exp = expf(a.A_log[head]);
    const float *q = static_cast<const float *>(a.q), *k = static_cast<const float *>(a.k);
    const float *gr = static_cast<const float *>(a.g_raw), *v = static_cast<const float *>(a.v);
    const float *br = static_cast<const float *>(a.beta_raw);
    float *o = static_cast<float *>(a.o);
    // Thread tid takes elements tid + NTHR r of a chunk's 16 x DK (and 16 x DV)
    // tiles: always channel tid % DK, tokens tid / DK + 4 r.
    constexpr int NE = CH * DK / NTHR, NV = CH * DV / NTHR;
    static_assert(NTHR % DK == 0 && NTHR % DV == 0, "element ownership");
    const int ce = tid % DK;
    const float dtb = a.dt_bias[(size_t)head * DK + ce];
    float rq[NE], rk[NE], rg[NE], rv[NV], rb = 0.f;
    // chunk x's inputs into the registers (rows past the sequence's end are
    // not read; they are zeroed when the registers are stored)
    auto load = [&](int x) {
        const int rem = min(CH, len - x * CH);
        const size_t tok0 = bos + (size_t)x * CH;
#pragma unroll
        for (int r = 0; r < NE; ++r) {
            const int tt = (tid + NTHR * r) / DK;
            const size_t g = ((tok0 + min(tt, rem - 1)) * H + head) * DK + ce;
            rq[r] = q[g];
            rk[r] = k[g];
            rg[r] = gr[g];
        }
#pragma unroll
        for (int r = 0; r < NV; ++r) {
            const int i = tid + NTHR * r, tt = i / DV;
            rv[r] = v[((tok0 + min(tt, rem - 1)) * H + head) * DV + i % DV];
        }
        if (tid < CH) rb = br[(tok0 + min(tid, rem - 1)) * H + head];
    };
    if (nch > 0) load(0);
    sync_lds();

    for (int x = 0; x < nch; ++x) {
        const int rem = min(CH, len - x * CH);
        const size_t tok0 = bos + (size_t)x * CH;
        if (SNAP) {
            const size_t at = ((cbase + x) * H + head) * DV * DK;
            for (int i = tid; i < DK * DV; i += NTHR) a.h_chunks[at + i] = sm.S[i % DK][i / DK];
        }
        // ---- inputs (pad tokens: zero), the gate and the per-token decays
#pragma unroll
        for (int r = 0; r < NE; ++r) {
            const int tt = (tid + NTHR * r) / DK;
            const bool live = tt < rem;
            sm.q[tt][ce] = live ? rq[r] : 0.f;
            sm.k[tt][ce] = live ? rk[r] : 0.f;
            const float g = live ? -A_exp * softplus_f(rg[r] + dtb) : 0.f;
            sm.kt[tt][ce] = g;   // the gate, replaced below by its cumulative sum, then by k~
            sm.dd[tt][ce] = expf(g);
        }
#pragma unroll
        for (int r = 0; r < NV; ++r) {
            const int i = tid + NTHR * r, tt = i / DV;
            sm.v[tt][i % DV] = tt < rem ? rv[r] : 0.f;
        }
        if (tid < CH) sm.beta[tid] = tid < rem ? sigmoid_f(rb) : 0.f;
        if (x + 1 < nch) load(x + 1);   // in flight while this chunk computes
        sync_lds();
        // ---- cumulative gate per channel
        if (tid < DK) {
            float G = 0.f;
#pragma unroll
            for (int tt = 0; tt < CH; ++tt) {
                G += sm.kt[tt][tid];
                sm.kt[tt][tid] = G;
            }
            sm.eg[tid] = expf(G);
            sm.gc[tid] = G;
        }
        sync_lds();
        // ---- decayed operands per (token, channel)
        const float GC = sm.gc[ce];   // the chunk's total gate in this channel
#pragma unroll
        for (int r = 0; r < NE; ++r) {
            const int tt = (tid + NTHR * r) / DK;
            const float Gs = sm.kt[tt][ce];
            const float e = expf(Gs);
            sm.kt[tt][ce] = sm.k[tt][ce] * e;
            sm.qt[tt][ce] = sm.q[tt][ce] * e * a.scale;
            sm.kr[tt][ce] = sm.k[tt][ce] * expf(GC - Gs);
        }
        sync_lds();
        // ---- L and Mqk: thread (j, cg) sums channels cg, cg + 16, ...; rows i >= j
        {
            const int j = tid >> 4, cg = tid & 15;
            float aL[CH], aM[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) { aL[i] = 0.f; aM[i] = 0.f; }
            for (int cc = cg; cc < DK; cc += 16) {
                const float kj = sm.k[j][cc];
                float f = 1.f;
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    if (i >= j) {
                        if (i > j) f *= sm.dd[i][cc];
                        aL[i] += sm.k[i][cc] * kj * f;
                        aM[i] += sm.q[i][cc] * kj * f;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const float sl = row16_sum(aL[i]), sq = row16_sum(aM[i]);
                if (cg == 0) {
                    sm.Lm[i][j] = i > j ? -sm.beta[i] * sl : 0.f;
                    sm.Mq[i][j] = i >= j ? a.scale * sq : 0.f;
                }
            }
        }
        sync_lds();
        // ---- W = k~ S, Qs = q~ S (C layout, tile n per wave); u = beta (v - W) into sm.u
        constexpr int NT = DV / 16;
        f32x4 Qs[(NT + 3) / 4];
#pragma unroll
        for (int ti = 0; ti < (NT + 3) / 4; ++ti) {
            const int n = wv + 4 * ti;
            if (n < NT) {
                f32x4 W = {0.f, 0.f, 0.f, 0.f}, Q = W;
                for (int kk = 0; kk < DK / 4; ++kk) {
                    const float b = sm.S[4 * kk + lq][16 * n + ln];
                    W = mma_f32(sm.kt[ln][4 * kk + lq], b, W);
                    Q = mma_f32(sm.qt[ln][4 * kk + lq], b, Q);
                }
                Qs[ti] = Q;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tt = 4 * lq + i;
                    sm.u[tt][16 * n + ln] = sm.beta[tt] * (sm.v[tt][16 * n + ln] - W[i]);
                }
            }
        }
        sync_lds();
        // ---- U: (I - L) U = u, row by row (one thread per column)
        if (tid < DV) {
            float Uc[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                float s = sm.u[i][tid];
#pragma unroll
                for (int j = 0; j < i; ++j) s += sm.Lm[i][j] * Uc[j];
                Uc[i] = s;
            }
#pragma unroll
            for (int i = 0; i < CH; ++i) sm.u[i][tid] = Uc[i];
        }
        sync_lds();
        // ---- O = Qs + Mqk U; S <- Diag(e^{G_C}) S + k^r^T U
#pragma unroll
        for (int ti = 0; ti < (NT + 3) / 4; ++ti) {
            const int n = wv + 4 * ti;
            if (n < NT) {
                f32x4 O = Qs[ti];
#pragma unroll
                for (int kk = 0; kk < CH / 4; ++kk)
                    O = mma_f32(sm.Mq[ln][4 * kk + lq], sm.u[4 * kk + lq][16 * n + ln], O);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tt = 4 * lq + i;
                    if (tt < rem) o[((tok0 + tt) * H + head) * DV + 16 * n + ln] = O[i];
                }
            }
        }
        for (int tile = wv; tile < (DK / 16) * NT; tile += 4) {
            const int mt = tile / NT, n = tile % NT;
            f32x4 Sa;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int cc = 16 * mt + 4 * lq + i;
                Sa[i] = sm.eg[cc] * sm.S[cc][16 * n + ln];
            }
#pragma unroll
            for (int kk = 0; kk < CH / 4; ++kk)
                Sa = mma_f32(sm.kr[4 * kk + lq][16 * mt + ln], sm.u[4 * kk + lq][16 * n + ln], Sa);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.S[16 * mt + 4 * lq + i][16 * n + ln] = Sa[i];
        }
        sync_lds();
    }
    if (a.h_T && hrow >= 0)
        for (int i = tid; i < DK * DV; i += NTHR) a.h_T[hb + i] = sm.S[i % DK][i / DK];
}

hipError_t launch_fwd_f32(const FwdArgs &a, int dk, int dv, hipStream_t stream)
{
    if (dk != DK || (dv != 64 && dv != 128)) return hipErrorInvalidValue;
    const long long wgs = (long long)a.n_seq * a.H;
    if (wgs == 0) return hipSuccess;
    if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
#define KDA_F32(DVV, SN) \
    hipLaunchKernelGGL((fwd_f32_kernel<DVV, SN>), dim3((unsigned)wgs), dim3(NTHR), 0, stream, a)
    if (dv == 128) {
        if (a.h_chunks) KDA_F32(128, true); else KDA_F32(128, false);
    } else {
        if (a.h_chunks) KDA_F32(64, true); else KDA_F32(64, false);
    }
#undef KDA_F32
    return hipGetLastError();
}

}  // namespace kda
