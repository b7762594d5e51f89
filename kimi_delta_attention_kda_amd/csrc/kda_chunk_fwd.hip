// kda_chunk_fwd.hip -- chunkwise KDA prefill for gfx950 (CDNA4).
//
// Pages cited by title and section:
//   [TL-KDA]  "TileLang 实战：KDA 从零到一 -- Chunked 线性注意力": section 1
//             (recurrence, (d_v, d_k) state), section 6.4 (sequence axis kept
//             out of the grid: one block walks all chunks with a loop-carried
//             state), 6.4.1 (split d_v, never d_k), 6.4.2 (state update after
//             the chunk's output write-back), 6.4.3 (log-domain gate).
//   [FKDA-LM] "FlashKDA 里的 L 矩阵和 Mqk 矩阵是什么": paragraphs "30秒速览"
//             (U, out and state-advance formulas), "L 矩阵的构造" (strictly
//             lower, row-scaled by beta), "Mqk 矩阵的构造" (lower including the
//             diagonal), "为什么 CHUNK16" (L^16 = 0, inverse by Neumann
//             squaring with 6 16x16 products), "K2 内核如何消费" (the four
//             steps and the state advance reusing U).
//   [SGL-PR]  "SGLang PR #26586 (KDA packed decode)": gate and beta formulas.
//
// What one workgroup computes.  A workgroup owns one chain = (sequence, head,
// d_v slab of BDV = 64 columns).  It walks the sequence in chunks of C = 16
// tokens; the fp32 state slab S^T (d_k x BDV) lives in MFMA accumulator
// registers for the whole walk.  Per chunk, with G the chunk-local cumulative
// gate (G_i = sum_{j<=i} g_j, per channel):
//   prep   (threads 0..dk-1, one channel each, tokens in order):
//          e^{g_t}, prefix products e^{G_t}, suffix products e^{G_C - G_t};
//          k~ = k e^G, q~ = q e^G, k^r = k e^{G_C - G}; band operands for L/Mqk;
//   L, Mqk (waves 0 and 1): 16x16 MFMA contractions over d_k;
//          L_ij = -beta_i sum_c k_ic k_jc e^{G_ic - G_jc}  (i > j),
//          Mqk_ij = sum_c q_ic k_jc e^{G_ic - G_jc}        (i >= j);
//   INV    (wave 0): (I - L)^{-1} = (I + L)(I + L^2)(I + L^4)(I + L^8);
//   per wave, one 16-column tile of the slab:
//          W = k~ S^T, Qs = q~ S^T;  u = beta (v - W);  U = INV u;
//          O = scale (Qs + Mqk U);  S^T <- Diag(e^{G_C}) S^T + k^r^T U.
// Sign of L: the recurrence gives (I + A) U = u with A_ij = beta_i <k~_i, k_j e^{-G_j}>,
// so L := -A and U = (I - L)^{-1} u (the page prints the series both ways).
//
// Overflow-safe L / Mqk.  The factored form <k_i e^{G_i}, k_j e^{-G_j}> of the
// page leaves the fp32 range once a channel decays by more than ~88 nats
// inside a chunk, which the gate distribution reaches (per-token decays above
// 70 nats occur).  Instead the chunk is cut into four blocks of four tokens.
// Block J's columns are scaled relative to the cumulative gate at the block's
// last token e_J, and every row i >= 4J relative to the same point:
//   col_j = k_j 2^{g'_j - g'_{e_J}} (<= 1),  row_i = k_i 2^{g'_{e_J} - g'_i},
// where g' is the cumulative decay in log2 units with each token's decay
// clipped at 24 (e^{g} floored at 2^-24).  Then row_i col_j = k_i k_j 2^{g'_j - g'_i}
// is exact for every pair whose true decay gap is at most 24 and at most
// 2^-24 otherwise (a term below fp32 rounding of the O(1) entries).  Within a
// block the row factor is at most 2^72, so nothing overflows, and an operand
// that underflows only drops terms below 2^-54.  The four blocks have
// disjoint columns, so their four MFMA passes accumulate into one tile.
// The operands of the state contractions (k~, q~, k^r) and the state decay
// use the unclipped gates; all their factors are <= 1.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int CH = 16;       // chunk length (tokens)
constexpr int NW = 4;        // waves per workgroup
constexpr int NTHR = 64 * NW;
constexpr int NBAND = 4;     // token blocks of the banded L / Mqk

template <bool BF16> struct Elem;
template <> struct Elem<true> { using T = uint16_t; };
template <> struct Elem<false> { using T = float; };

template <bool BF16, int DK>
struct alignas(16) Smem {
    using E = typename Elem<BF16>::T;
    static constexpr int PK = DK + (BF16 ? 8 : 4);   // padded channel rows
    static constexpr int PT = CH + (BF16 ? 8 : 4);   // padded token rows
    alignas(16) E kd[CH][PK];                // k e^{G}             [token][channel]
    alignas(16) E qd[CH][PK];                // q e^{G}             [token][channel]
    alignas(16) E kr[DK][PT];                // k e^{G_C - G}       [channel][token]
    alignas(16) E br[NBAND][2][CH][PK];      // band rows (k, q)    [band][k|q][token][channel]
    alignas(16) E bc[CH][PK];                // band columns        [token][channel]
    alignas(16) float L[CH][CH + 1];
    alignas(16) float M[CH][CH + 1];
    alignas(16) float P[2][CH][CH + 1];
    alignas(16) float X[2][CH][CH + 1];
    alignas(16) float beta[CH];
    alignas(16) float eg[DK];                // e^{G_C}
};

template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::T to_elem(float x) {
    if constexpr (BF16) return f32_to_bf16(x);
    else return x;
}

template <bool BF16>
__device__ __forceinline__ float load_act(const void *p, size_t i) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
    else return static_cast<const float *>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_act(void *p, size_t i, float x) {
    if constexpr (BF16) static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
    else static_cast<float *>(p)[i] = x;
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-lane row / 4-group coordinates of the 16x16 MFMA layouts:
//   A (16 x K): lane (ln, lq) holds row ln, K slice lq;
//   B (K x 16): lane (ln, lq) holds column ln, K slice lq;
//   C (16 x 16): lane (ln, lq) holds rows 4lq .. 4lq+3 of column ln.

// D += A B for 16x16 fp32 matrices in LDS (row stride CH+1), 4 fp32 MFMAs.
__device__ __forceinline__ f32x4 mm16(const float (*A)[CH + 1], const float (*B)[CH + 1],
                                      f32x4 acc, int ln, int lq) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_f32(A[ln][4 * s + lq], B[4 * s + lq][ln], acc);
    return acc;
}
__device__ __forceinline__ f32x4 ld_c(const float (*D)[CH + 1], int ln, int lq) {
    f32x4 c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = D[4 * lq + i][ln];
    return c;
}
__device__ __forceinline__ void st_c(float (*D)[CH + 1], f32x4 c, int ln, int lq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) D[4 * lq + i][ln] = c[i];
}

// bf16 hi/lo split of 4 values into one 8-wide operand [hi0..hi3, lo0..lo3].
__device__ __forceinline__ bf16x8 split_hilo(f32x4 x) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 hi = static_cast<__bf16>(x[i]);
        r[i] = hi;
        r[4 + i] = static_cast<__bf16>(x[i] - static_cast<float>(hi));
    }
    return r;
}
// A operand that pairs with split_hilo B operands: row values a[0..3] used
// for both the hi and the lo K slots.  `lo` selects the rounding remainder.
__device__ __forceinline__ bf16x8 dup_row(const float *a, bool lo) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 hi = static_cast<__bf16>(a[i]);
        const __bf16 v = lo ? static_cast<__bf16>(a[i] - static_cast<float>(hi)) : hi;
        r[i] = v;
        r[4 + i] = v;
    }
    return r;
}

template <bool BF16, int DK, int DV>
__global__ __launch_bounds__(NTHR) void chunk_fwd_kernel(ChunkArgs args)
{
    constexpr int BDV = 16 * NW;
    static_assert(DV % BDV == 0, "slab width must divide d_v");
    constexpr int NSLAB = DV / BDV;
    constexpr int MT = DK / 16;          // 16-channel tiles of the state
    using S_t = Smem<BF16, DK>;
    using E = typename S_t::E;
    __shared__ S_t sm;

    const int H = args.H;
    const int chain = blockIdx.x / NSLAB;
    const int slab = blockIdx.x - chain * NSLAB;
    const int h = chain % H;
    const int seq = chain / H;
    size_t bos;
    int len;
    if (args.cu_seqlens) {
        bos = (size_t)args.cu_seqlens[seq];
        len = args.cu_seqlens[seq + 1] - args.cu_seqlens[seq];
    } else {
        bos = (size_t)seq * args.T;
        len = args.T;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, lq = lane >> 4;
    const int v0 = slab * BDV + 16 * w;   // first column of this wave's tile

    // State tile of this wave in the C layout: S[mt][i] = S^T[16 mt + 4 lq + i][v0 + ln].
    f32x4 S[MT];
    const size_t hbase = (((size_t)seq * H + h) * DV + v0 + ln) * DK;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        if (args.h0) S[mt] = *reinterpret_cast<const f32x4 *>(args.h0 + hbase + 16 * mt + 4 * lq);
        else S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const float A_exp = expf(args.A_log[h]);
    const float dt_c = tid < DK ? args.dt_bias[(size_t)h * DK + tid] : 0.f;
    const int nchunks = (len + CH - 1) / CH;

    for (int ck = 0; ck < nchunks; ++ck) {
        const size_t tok0 = bos + (size_t)ck * CH;
        const int rem = min(CH, len - ck * CH);
        __syncthreads();   // previous chunk's readers are done with sm

        // ------------------------------------------------------------ prep
        if (tid < DK) {
            const int c = tid;
            float kk[CH], qq[CH], al[CH];
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                if (t < rem) {
                    const size_t off = ((tok0 + t) * H + h) * DK + c;
                    kk[t] = load_act<BF16>(args.k, off);
                    qq[t] = load_act<BF16>(args.q, off);
                    const float x = load_act<BF16>(args.g_raw, off) + dt_c;
                    al[t] = exp2f(-A_exp * softplus_f(x) * kLog2e);   // e^{g_t}
                } else {
                    kk[t] = 0.f; qq[t] = 0.f; al[t] = 1.f;
                }
            }
            float P = 1.f;
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                P *= al[t];
                sm.kd[t][c] = to_elem<BF16>(kk[t] * P);
                sm.qd[t][c] = to_elem<BF16>(qq[t] * P);
            }
            sm.eg[c] = P;
            float Q = 1.f;
#pragma unroll
            for (int t = CH - 1; t >= 0; --t) {
                sm.kr[c][t] = to_elem<BF16>(kk[t] * Q);
                Q *= al[t];
            }
            float ac[CH];
#pragma unroll
            for (int t = 0; t < CH; ++t) ac[t] = fmaxf(al[t], 0x1p-24f);
#pragma unroll
            for (int J = 0; J < NBAND; ++J) {
                const int e = 4 * J + 3;
                float cf = 1.f;
#pragma unroll
                for (int t = e; t >= 4 * J; --t) {
                    sm.bc[t][c] = to_elem<BF16>(kk[t] * cf);
                    const float rb = __builtin_amdgcn_rcpf(cf);
                    sm.br[J][0][t][c] = to_elem<BF16>(kk[t] * rb);
                    sm.br[J][1][t][c] = to_elem<BF16>(qq[t] * rb);
                    cf *= ac[t];
                }
                float R = 1.f;
#pragma unroll
                for (int t = e + 1; t < CH; ++t) {
                    R *= ac[t];
                    sm.br[J][0][t][c] = to_elem<BF16>(kk[t] * R);
                    sm.br[J][1][t][c] = to_elem<BF16>(qq[t] * R);
                }
#pragma unroll
                for (int t = 0; t < 4 * J; ++t) {
                    sm.br[J][0][t][c] = to_elem<BF16>(0.f);
                    sm.br[J][1][t][c] = to_elem<BF16>(0.f);
                }
            }
        }
        if (tid >= 64 * (NW - 1) && tid < 64 * (NW - 1) + CH) {
            const int t = tid - 64 * (NW - 1);
            sm.beta[t] = t < rem ? sigmoid_f(load_act<BF16>(args.beta_raw, (tok0 + t) * H + h)) : 0.f;
        }
        __syncthreads();

        // ------------------------------------------ L + INV (wave 0), Mqk (wave 1)
        if (w < 2) {
            const int which = w;   // 0: key rows -> L, 1: query rows -> Mqk
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J < NBAND; ++J) {
                const bool colv = (ln >> 2) == J;
                if constexpr (BF16) {
#pragma unroll
                    for (int s = 0; s < DK / 32; ++s) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sm.br[J][which][ln][32 * s + 8 * lq]);
                        bf16x8 b = *reinterpret_cast<const bf16x8 *>(&sm.bc[ln][32 * s + 8 * lq]);
                        if (!colv) b = bf16x8{};
                        acc = mfma_bf16(a, b, acc);
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < DK / 4; ++s) {
                        const float a = sm.br[J][which][ln][4 * s + lq];
                        const float b = colv ? sm.bc[ln][4 * s + lq] : 0.f;
                        acc = mfma_f32(a, b, acc);
                    }
                }
            }
            if (which == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * lq + i;
                    sm.L[r][ln] = r > ln ? -sm.beta[r] * acc[i] : 0.f;
                }
                // Neumann squaring: X <- X (I + P^2) with P <- P^2, from X = I + L, P = L.
                f32x4 X;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * lq + i;
                    X[i] = (r == ln ? 1.f : 0.f) + (r > ln ? sm.L[r][ln] : 0.f);
                }
                st_c(sm.X[0], X, ln, lq);
                const float (*Pc)[CH + 1] = sm.L;
                int xb = 0;
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    const f32x4 Pn = mm16(Pc, Pc, f32x4{0.f, 0.f, 0.f, 0.f}, ln, lq);
                    st_c(sm.P[r & 1], Pn, ln, lq);
                    Pc = sm.P[r & 1];
                    X = mm16(sm.X[xb], Pc, X, ln, lq);
                    xb ^= 1;
                    st_c(sm.X[xb], X, ln, lq);
                }
                // INV is now in sm.X[1] (three steps: X[0] -> X[1] -> X[0] -> X[1]).
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * lq + i;
                    sm.M[r][ln] = r >= ln ? acc[i] : 0.f;
                }
            }
        }
        __syncthreads();

        // ------------------------------------------------ recurrence (every wave)
        const float (*INV)[CH + 1] = sm.X[1];
        f32x4 W = {0.f, 0.f, 0.f, 0.f}, Qs = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF16) {
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                bf16x8 b;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    b[i] = static_cast<__bf16>(S[2 * s][i]);
                    b[4 + i] = static_cast<__bf16>(S[2 * s + 1][i]);
                }
                bf16x8 ak, aq;
                const bf16x4 k0 = *reinterpret_cast<const bf16x4 *>(&sm.kd[ln][32 * s + 4 * lq]);
                const bf16x4 k1 = *reinterpret_cast<const bf16x4 *>(&sm.kd[ln][32 * s + 16 + 4 * lq]);
                const bf16x4 q0 = *reinterpret_cast<const bf16x4 *>(&sm.qd[ln][32 * s + 4 * lq]);
                const bf16x4 q1 = *reinterpret_cast<const bf16x4 *>(&sm.qd[ln][32 * s + 16 + 4 * lq]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ak[i] = k0[i]; ak[4 + i] = k1[i];
                    aq[i] = q0[i]; aq[4 + i] = q1[i];
                }
                W = mfma_bf16(ak, b, W);
                Qs = mfma_bf16(aq, b, Qs);
            }
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    W = mfma_f32(sm.kd[ln][16 * mt + 4 * lq + i], S[mt][i], W);
                    Qs = mfma_f32(sm.qd[ln][16 * mt + 4 * lq + i], S[mt][i], Qs);
                }
        }
        // u = beta (v - W)
        f32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lq + i;
            const float vv = r < rem ? load_act<BF16>(args.v, ((tok0 + r) * H + h) * DV + v0 + ln) : 0.f;
            u[i] = sm.beta[r] * (vv - W[i]);
        }
        f32x4 U = {0.f, 0.f, 0.f, 0.f}, O;
        float rowbuf[4];
        if constexpr (BF16) {
            const bf16x8 bu = split_hilo(u);
#pragma unroll
            for (int i = 0; i < 4; ++i) rowbuf[i] = INV[ln][4 * lq + i];
            U = mfma_bf16(dup_row(rowbuf, false), bu, U);
            U = mfma_bf16(dup_row(rowbuf, true), bu, U);
            const bf16x8 bU = split_hilo(U);
#pragma unroll
            for (int i = 0; i < 4; ++i) rowbuf[i] = sm.M[ln][4 * lq + i];
            O = mfma_bf16(dup_row(rowbuf, false), bU, Qs);
            O = mfma_bf16(dup_row(rowbuf, true), bU, O);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 e = *reinterpret_cast<const f32x4 *>(&sm.eg[16 * mt + 4 * lq]);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[mt][i] *= e[i];
                const bf16x4 kr4 = *reinterpret_cast<const bf16x4 *>(&sm.kr[16 * mt + ln][4 * lq]);
                bf16x8 a;
#pragma unroll
                for (int i = 0; i < 4; ++i) { a[i] = kr4[i]; a[4 + i] = kr4[i]; }
                S[mt] = mfma_bf16(a, bU, S[mt]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) U = mfma_f32(INV[ln][4 * lq + i], u[i], U);
            O = Qs;
#pragma unroll
            for (int i = 0; i < 4; ++i) O = mfma_f32(sm.M[ln][4 * lq + i], U[i], O);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 e = *reinterpret_cast<const f32x4 *>(&sm.eg[16 * mt + 4 * lq]);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[mt][i] *= e[i];
#pragma unroll
                for (int i = 0; i < 4; ++i) S[mt] = mfma_f32(sm.kr[16 * mt + ln][4 * lq + i], U[i], S[mt]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lq + i;
            if (r < rem) store_act<BF16>(args.o, ((tok0 + r) * H + h) * DV + v0 + ln, args.scale * O[i]);
        }
    }

    if (args.h_T) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            *reinterpret_cast<f32x4 *>(args.h_T + hbase + 16 * mt + 4 * lq) = S[mt];
    }
}

template <bool BF16, int DK, int DV>
static hipError_t launch_one(const ChunkArgs &a, hipStream_t stream)
{
    constexpr int NSLAB = DV / (16 * NW);
    const unsigned grid = (unsigned)a.n_seq * (unsigned)a.H * NSLAB;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_fwd_kernel<BF16, DK, DV>), dim3(grid), dim3(NTHR), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, int dtype, int dk, int dv, hipStream_t stream)
{
    if (dtype == 1) {
        if (dk == 128 && dv == 128) return launch_one<true, 128, 128>(a, stream);
        if (dk == 128 && dv == 64) return launch_one<true, 128, 64>(a, stream);
        if (dk == 64 && dv == 128) return launch_one<true, 64, 128>(a, stream);
        if (dk == 64 && dv == 64) return launch_one<true, 64, 64>(a, stream);
    } else {
        if (dk == 64 && dv == 128) return launch_one<false, 64, 128>(a, stream);
        if (dk == 64 && dv == 64) return launch_one<false, 64, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
