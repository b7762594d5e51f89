// kda_fwd.hip -- chunkwise KDA prefill for gfx950 (CDNA4), bf16 activations.
//
// Pages cited by title and section:
//   [TL-KDA]  "TileLang 实战：KDA 从零到一 -- Chunked 线性注意力": section 1
//             (recurrence, (d_v, d_k) state), 6.4 (the state is carried
//             through a sequential chunk loop inside the block: the sequence
//             axis stays out of the grid), 6.4.1 (split d_v, never d_k),
//             6.4.2 (the state advances after the chunk's output).
//   [FKDA-LM] "FlashKDA 里的 L 矩阵和 Mqk 矩阵是什么": "30秒速览" (U, output and
//             state advance), "L 矩阵的构造" (strictly lower, rows scaled by
//             beta), "Mqk 矩阵的构造" (lower including the diagonal), "为什么
//             CHUNK16" (L^16 = 0; inverse by Neumann squaring), "K2 内核如何消费".
//   [SGL-PR]  "SGLang PR #26586 (KDA packed decode)": gate and beta formulas.
//
// Per chunk of C = 16 tokens of one (sequence, head), with G the chunk-local
// cumulative gate (per channel), S the state as d_k x d_v (the transpose of
// the stored [d_v][d_k]) and beta = diag(beta_i):
//   k~ = k e^G,  q~ = q e^G,  k^r = k e^{G_C - G}
//   L_ij = -beta_i sum_c k_ic k_jc e^{G_ic - G_jc} (i > j),  Mqk_ij = sum_c q_ic k_jc e^{G_ic - G_jc} (i >= j)
//   INV = (I - L)^-1 = (I + L)(I + L^2)(I + L^4)(I + L^8)
// The pages' U = INV beta (v - k~ S) is used in its factored ("WY") form
//   w = INV beta k~,  u' = INV beta v,  U = u' - w S,
// so that only U = u' - w S sits on the state's critical path, then
//   O = scale (q~ S + Mqk U),  S <- Diag(e^{G_C}) S + k^r^T U   (after the output).
// Sign of L: the recurrence gives (I + A) U = u with A_ij = beta_i <k~_i, k_j e^{-G_j}>,
// so L := -A (the page prints the series both ways).
//
// Work split on MI355X.  One workgroup owns one (sequence, head, d_v column
// group) for the whole sequence: no other workgroup and no device memory
// besides the inputs and outputs is involved.  Its waves have two roles:
//   * NPW = d_k / 32 PREP waves build everything that does not depend on the
//     state, in three pipelined stages, each chunk's stages in successive
//     iterations of the chunk loop:
//       A (chunk it+3, all prep waves): gate, cumulative gate, decayed
//         operands, this wave's 32-channel partials of L, L^T and Mqk^T on the
//         matrix core, layout transposes of k~, k^r and v (below);
//       B1 (chunk it+2, wave 0): sums the partials, applies masks and beta,
//         INV by Neumann squaring, INV beta;
//       B2 (chunk it+1, the other prep waves): w and u' on the matrix core;
//   * NCW CONSUMER waves, each owning SPW slabs of 16 state columns in fp32
//     MFMA accumulators, run the recurrence for chunk it:
//       W' = w S, Qs^T = S^T q~^T, decay, U = u' - W', O^T = Qs^T + U^T Mqk^T,
//       S += k^r^T U.
//   The stages hand over through LDS; one workgroup barrier per chunk.
//   A chain whose columns are split over G groups repeats the prep in each
//   group (used when the chains are fewer than the compute units).
//
// Operand layouts.  For a 16 x 16 tile X the "C layout" is the MFMA
// accumulator layout: lane (lq, ln) = (lane / 16, lane % 16) holds
// X[4 lq + i][ln], i = 0..3.  A K = 16 product X Y on v_mfma_f32_16x16x16_bf16
// takes the C layout of X^T as its A operand and the C layout of Y as its B
// operand, so chained 16 x 16 products need no data movement.  A K = 32
// operand of v_mfma_f32_16x16x32_bf16 holds 8 K values per lane; the state
// tiles are ordered so that the 8 K values of lane quarter lq in K block s are
// the 8 consecutive channels 32 s + 8 lq .. +7 (state tile m, row 4 lq + i
// <-> channel chan(m, lq, i)), which is exactly one 16-byte load of a token's
// q or k row.  A C-layout copy of a row-loaded bf16 tile is one MFMA with a
// 0/1 selector (exact), used for k~, k^r (per 16 channels) and v (per 16
// columns).  The output is computed transposed (O^T), whose C layout gives
// every lane 4 consecutive columns of one token: one 8-byte store.
//
// Overflow-safe L / Mqk.  The factored form <k_i e^{G_i}, k_j e^{-G_j}> leaves
// the fp32 range once a channel decays by more than ~88 nats inside a chunk.
// A wave whose 32 channels all decay by at most 100 (log2 units) inside the
// chunk ("mild") uses rows k~ = k 2^G (<= 1) and columns k 2^-G (<= 2^100).
// Otherwise ("strong") two 8-token row blocks each take the clipped cumulative
// decay at the end of the previous block as reference, with each token's
// decay clipped at 2^-12: rows <= 1, columns <= 2^96, one MFMA pass per block.
// A pair whose true decay gap exceeds 12 (log2) is then computed as at most
// 2^-12 instead of its smaller true value; every other pair is exact.
// Precision: bf16 MFMA operands, fp32 accumulation; the state is fp32 and
// U = u' - w S rides the state update as a hi + lo bf16 pair.
#include <stdint.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int CH = 16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                     c, 0, 0, 0);
}
constexpr f32x4 Z4 = {0.f, 0.f, 0.f, 0.f};

__device__ __forceinline__ bf16x4 pack4(f32x4 x) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = static_cast<__bf16>(x[i]);
    return r;
}
__device__ __forceinline__ bf16x8 pack8(const float (&x)[8]) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(x[i]);
    return r;
}
__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
    return r;
}
// x = hi + lo, both bf16 (hi = RNE(x), lo = RNE(x - hi)): ~2^-16 relative
__device__ __forceinline__ bf16x8 hilo(f32x4 x) {
    bf16x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = static_cast<__bf16>(x[i]);
        l[i] = static_cast<__bf16>(x[i] - static_cast<float>(h[i]));
    }
    return cat4(h, l);
}
__device__ __forceinline__ f32x4 plus_eye(f32x4 X, int ln, int lq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) X[i] += (4 * lq + i == ln) ? 1.f : 0.f;
    return X;
}
// X Y in C layout from XT = C layout of X^T and Y in C layout (single bf16).
__device__ __forceinline__ f32x4 prod(f32x4 XT, f32x4 Y) { return mma16(pack4(XT), pack4(Y), Z4); }

// DPP inside a 16-lane row: inclusive scan over the row's 16 tokens, and the
// broadcast of lane n of the row.
__device__ __forceinline__ float scan16(float x) {
    x += dpp_f<0x111>(x);
    x += dpp_f<0x112>(x);
    x += dpp_f<0x114>(x);
    x += dpp_f<0x118>(x);
    return x;
}
template <int N>
__device__ __forceinline__ float row_bcast(float x) { return dpp_f<0x150 + N>(x); }

__device__ __forceinline__ void lds_barrier() {   // LDS-only barrier: global loads stay in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Channel of row 4 lq + i of state tile m (and of the matching rows of every
// C-layout channel tile): the 8 K values a lane feeds to a 16x16x32 MFMA in K
// block s are then the 8 consecutive channels 32 s + 8 lq .. +7.
__device__ __forceinline__ constexpr int chan(int m, int lq, int i) { return 32 * (m >> 1) + 8 * lq + 4 * (m & 1) + i; }

template <int DK, int DV, int NCW, int SPW>
struct Lay {
    static constexpr int NPW = DK / 32;           // prep waves (one 32-channel block each)
    static constexpr int NKB = DK / 32;           // K blocks of the state products
    static constexpr int NMT = DK / 16;           // state row tiles
    static constexpr int NCOL = NCW * SPW * 16;   // columns of the group
    static constexpr int G = DV / NCOL;           // column groups per chain
    static constexpr int NVT = NCOL / 16;         // 16-column tiles of the group
    static constexpr int NVB = (NCOL + 31) / 32;  // 32-column v blocks
    static constexpr int VPW = (NVB + NPW - 1) / NPW;   // v blocks per prep wave
    static constexpr int NW = NPW + NCW;
    static constexpr int NTHR = 64 * NW;
    // per chunk, read by the consumers (4 buffers: written 3 iterations ahead)
    static constexpr int QF = 0;                    // q~ B fragments   [NKB][64] x 16 B
    static constexpr int KR = QF + NKB * 1024;      // k^r C tiles      [NMT][64] x 8 B (bf16)
    static constexpr int EG = KR + NMT * 512;       // e^{G_C}          [DK] fp32
    static constexpr int MQ = EG + DK * 4;          // Mqk^T C tile     [64] x 8 B (bf16)
    static constexpr int QKE = MQ + 512;
    static constexpr int WF = 0;                    // w A fragments    [NKB][64] x 16 B   (2 buffers)
    static constexpr int UP = WF + NKB * 1024;      // u' C tiles       [NVT][64] x 16 B (fp32)
    static constexpr int WUM = UP + NVT * 1024;
    static constexpr int KT = 0;                    // k~ C tiles       [NMT][64] x 8 B    (3 buffers)
    static constexpr int VT = KT + NMT * 512;       // v C tiles        [NVT][64] x 8 B
    static constexpr int KV = VT + NVT * 512;
    static constexpr int PART = NPW * 3 * 1024;     // per prep wave: L, L^T, Mqk^T partials (2 buffers)
    static constexpr int O_QKE = 0;
    static constexpr int O_WUM = O_QKE + 4 * QKE;
    static constexpr int O_KV = O_WUM + 2 * WUM;
    static constexpr int O_PART = O_KV + 3 * KV;
    static constexpr int O_INVB = O_PART + 2 * PART;   // C layout of (INV beta)^T, bf16  (2 buffers)
    static constexpr int O_BETA = O_INVB + 2 * 512;    // beta [16]                         (2 buffers)
    static constexpr int O_SEQ = O_BETA + 2 * 64;      // the sequence this workgroup takes
    static constexpr int BYTES = O_SEQ + 16;
    static_assert(DK == 64 || DK == 128, "d_k");
    static_assert(NCOL * G == DV && NCOL % 16 == 0, "column groups");
    static_assert(BYTES <= 160 * 1024, "LDS");
};

// Packed sequences with at most this many entries are taken longest first.
constexpr int LPT_MAX = 128;

// Inputs of one chunk as a prep lane holds them: token t = lane % 16, the
// 8 channels 32 w + 8 (lane / 16) .. +7 of q, k, g_raw; v blocks; beta_raw.
template <int VPW>
struct In {
    uint4 k, q, a;
    uint4 v[VPW];
    uint16_t b;
};

struct Chain {
    size_t bos;
    int len, nch, seq, head, hrow;
};

}  // namespace

template <int DK, int DV, int NCW, int SPW, bool SNAP>
__global__ __launch_bounds__(64 * (DK / 32 + NCW)) void fwd_kernel(FwdArgs a)
{
    using L = Lay<DK, DV, NCW, SPW>;
    constexpr int NPW = L::NPW, NKB = L::NKB, NMT = L::NMT, NVT = L::NVT, NVB = L::NVB, VPW = L::VPW;
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lq = lane >> 4;
    const int group = blockIdx.x % L::G;
    const int slot = blockIdx.x / L::G;
    const int col0 = group * L::NCOL;

    // ---- which (sequence, head): heads inner; packed sequences longest first
    Chain c;
    c.head = slot % a.H;
    const int rank = slot / a.H;
    if (a.cu_seqlens && a.n_seq <= LPT_MAX) {
        int *sseq = reinterpret_cast<int *>(lds + L::O_SEQ);
        for (int s = tid; s < a.n_seq; s += L::NTHR) {
            const int ls = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
            int r = 0;
            for (int s2 = 0; s2 < a.n_seq; ++s2) {
                const int l2 = a.cu_seqlens[s2 + 1] - a.cu_seqlens[s2];
                r += (l2 > ls) || (l2 == ls && s2 < s);
            }
            if (r == rank) *sseq = s;
        }
        lds_barrier();
        c.seq = __builtin_amdgcn_readfirstlane(*sseq);
    } else {
        c.seq = rank;
    }
    if (a.cu_seqlens) {
        c.bos = (size_t)a.cu_seqlens[c.seq];
        c.len = a.cu_seqlens[c.seq + 1] - a.cu_seqlens[c.seq];
    } else {
        c.bos = (size_t)c.seq * a.T;
        c.len = a.T;
    }
    c.nch = (c.len + CH - 1) / CH;
    c.hrow = a.state_idx ? a.state_idx[c.seq] : c.seq;
    if (a.state_idx && c.hrow >= a.P) {   // out-of-range slot: start from zero, keep no state, report
        if (tid == 0) slot_error(a.err);
        c.hrow = -1;
    }
    const size_t H = a.H;
    const size_t hbase = (((size_t)(c.hrow < 0 ? 0 : c.hrow) * H + c.head) * DV + col0) * DK;

    if (c.nch == 0) {   // empty sequence: h_T = h0 (or zeros), nothing else
        if (a.h_T && c.hrow >= 0)
            for (int i = tid; i < L::NCOL * DK; i += L::NTHR)
                a.h_T[hbase + i] = a.h0 ? a.h0[hbase + i] : 0.f;
        return;
    }

    if (wv >= NPW) {
        // ======================================================= consumer
        const int cw = wv - NPW;
        f32x4 S[SPW][NMT];
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int n = cw * SPW + j;
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                if (a.h0 && c.hrow >= 0)
                    S[j][m] = *reinterpret_cast<const f32x4 *>(a.h0 + hbase + (size_t)(16 * n + ln) * DK + chan(m, lq, 0));
                else
                    S[j][m] = Z4;
            }
        }
        size_t cbase = 0;   // h_chunks row of the sequence's first chunk
        if (SNAP) {
            if (a.cu_seqlens) {
                for (int s2 = 0; s2 < c.seq; ++s2)
                    cbase += (size_t)((a.cu_seqlens[s2 + 1] - a.cu_seqlens[s2] + CH - 1) / CH);
            } else {
                cbase = (size_t)c.seq * ((a.T + CH - 1) / CH);
            }
        }
        const float scale = a.scale;
        for (int it = -3; it < c.nch; ++it) {
            if (it >= 0) {
                const int x = it;
                const unsigned char *qke = lds + L::O_QKE + (x & 3) * L::QKE;
                const unsigned char *wum = lds + L::O_WUM + (x & 1) * L::WUM;
                // the state entering the chunk, as bf16 K fragments (B of W' = w S, A of Qs^T = S^T q~^T)
                bf16x8 bS[SPW][NKB];
#pragma unroll
                for (int j = 0; j < SPW; ++j)
#pragma unroll
                    for (int s = 0; s < NKB; ++s) bS[j][s] = cat4(pack4(S[j][2 * s]), pack4(S[j][2 * s + 1]));
                if constexpr (SNAP) {
                    const size_t at = (((cbase + x) * H + c.head) * DV + col0) * DK;
#pragma unroll
                    for (int j = 0; j < SPW; ++j) {
                        const int n = cw * SPW + j;
#pragma unroll
                        for (int m = 0; m < NMT; ++m)
                            __builtin_nontemporal_store(S[j][m], reinterpret_cast<f32x4 *>(
                                a.h_chunks + at + (size_t)(16 * n + ln) * DK + chan(m, lq, 0)));
                    }
                }
                f32x4 W[SPW], Qs[SPW];
#pragma unroll
                for (int j = 0; j < SPW; ++j) { W[j] = Z4; Qs[j] = Z4; }
#pragma unroll
                for (int s = 0; s < NKB; ++s) {
                    const bf16x8 wf = *reinterpret_cast<const bf16x8 *>(wum + L::WF + (s * 64 + lane) * 16);
                    const bf16x8 qf = *reinterpret_cast<const bf16x8 *>(qke + L::QF + (s * 64 + lane) * 16);
#pragma unroll
                    for (int j = 0; j < SPW; ++j) {
                        W[j] = mma32(wf, bS[j][s], W[j]);
                        Qs[j] = mma32(bS[j][s], qf, Qs[j]);
                    }
                }
                // decay the fp32 state: S <- Diag(e^{G_C}) S
#pragma unroll
                for (int m = 0; m < NMT; ++m) {
                    const f32x4 eg = *reinterpret_cast<const f32x4 *>(qke + L::EG + chan(m, lq, 0) * 4);
#pragma unroll
                    for (int j = 0; j < SPW; ++j) S[j][m] *= eg;
                }
                const bf16x4 mq = *reinterpret_cast<const bf16x4 *>(qke + L::MQ + lane * 8);
                const bf16x8 bmq = cat4(mq, mq);
                const int rem = min(CH, c.len - x * CH);
                bf16x8 bU[SPW];
#pragma unroll
                for (int j = 0; j < SPW; ++j) {
                    const int n = cw * SPW + j;
                    const f32x4 up = *reinterpret_cast<const f32x4 *>(wum + L::UP + (n * 64 + lane) * 16);
                    bU[j] = hilo(up - W[j]);   // U = u' - w S as [hi | lo]
                    // O^T = Qs^T + U^T Mqk^T; lane: 4 consecutive columns of token ln
                    const f32x4 O = mma32(bU[j], bmq, Qs[j]);
                    if (ln < rem) {
                        uint2 v2;
                        v2.x = pack_bf16x2(scale * O[0], scale * O[1]);
                        v2.y = pack_bf16x2(scale * O[2], scale * O[3]);
                        const size_t at = ((c.bos + (size_t)x * CH + ln) * H + c.head) * DV + col0 + 16 * n + 4 * lq;
                        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.o) + at) = v2;
                    }
                }
                // S += k^r^T U (the k^r values repeated for the hi and lo halves of U)
#pragma unroll
                for (int m = 0; m < NMT; ++m) {
                    const bf16x4 kr = *reinterpret_cast<const bf16x4 *>(qke + L::KR + (m * 64 + lane) * 8);
                    const bf16x8 bkr = cat4(kr, kr);
#pragma unroll
                    for (int j = 0; j < SPW; ++j) S[j][m] = mma32(bkr, bU[j], S[j][m]);
                }
            }
            lds_barrier();
        }
        if (a.h_T && c.hrow >= 0) {
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                const int n = cw * SPW + j;
#pragma unroll
                for (int m = 0; m < NMT; ++m)
                    *reinterpret_cast<f32x4 *>(a.h_T + hbase + (size_t)(16 * n + ln) * DK + chan(m, lq, 0)) = S[j][m];
            }
        }
        return;
    }

    // =========================================================== prep
    const int w = wv;
    const int t = ln, r = lq;                 // token, 8-channel unit within the wave's 32 channels
    const float A_exp = expf(a.A_log[c.head]);
    float dtl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dtl[e] = a.dt_bias[(size_t)c.head * DK + 32 * w + 8 * r + e] * kLog2e;
    // 0/1 selectors: C-layout copies of row-loaded tiles (the channels of
    // state tile 2w + h; columns 16 (2 vb + h) .. + 15 of a v block)
    bf16x8 sel_c[2], sel_v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sel_c[h][e] = static_cast<__bf16>((lq == (ln >> 2) && e == 4 * h + (ln & 3)) ? 1.f : 0.f);
            sel_v[h][e] = static_cast<__bf16>((lq == 2 * h + (ln >> 3) && e == (ln & 7)) ? 1.f : 0.f);
        }

    auto load = [&](In<VPW> &in, int x) {
        const int rem = min(CH, c.len - x * CH);
        const size_t tok = c.bos + (size_t)x * CH + min(t, rem - 1);   // rows past the end repeat the last live row
        const size_t off = (tok * H + c.head) * DK + 32 * w + 8 * r;
        in.k = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + off);
        in.q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + off);
        in.a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.g_raw) + off);
#pragma unroll
        for (int i = 0; i < VPW; ++i) {
            const int vb = w + NPW * i;
            if (vb < NVB && 32 * vb + 8 * r < L::NCOL)
                in.v[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) +
                                                           (tok * H + c.head) * DV + col0 + 32 * vb + 8 * r);
            else
                in.v[i] = uint4{0u, 0u, 0u, 0u};
        }
        in.b = (w == 0) ? static_cast<const uint16_t *>(a.beta_raw)[tok * H + c.head] : (uint16_t)0;
    };

    // ---- stage A: chunk x from the inputs in `in`
    auto stage_a = [&](const In<VPW> &in, int x) {
        const int rem = min(CH, c.len - x * CH);
        const bool live = t < rem;
        const float nA = live ? -A_exp : 0.f;
        unsigned char *qke = lds + L::O_QKE + (x & 3) * L::QKE;
        unsigned char *kv = lds + L::O_KV + (x % 3) * L::KV;
        float kf[8], qf[8], gv[8], Gm[8], GC[8], e1[8], kd[8], qd[8], kr[8];
        const uint32_t kw[4] = {in.k.x, in.k.y, in.k.z, in.k.w};
        const uint32_t qw[4] = {in.q.x, in.q.y, in.q.z, in.q.w};
        const uint32_t aw[4] = {in.a.x, in.a.y, in.a.z, in.a.w};
        bool deep = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sh = (e & 1) ? 0 : 16;
            const uint32_t mk = (e & 1) ? 0xffff0000u : 0xffffffffu;
            kf[e] = live ? __builtin_bit_cast(float, (kw[e >> 1] << sh) & mk) : 0.f;
            qf[e] = live ? __builtin_bit_cast(float, (qw[e >> 1] << sh) & mk) : 0.f;
            const float af = __builtin_bit_cast(float, (aw[e >> 1] << sh) & mk);
            const float y = __builtin_fmaf(af, kLog2e, dtl[e]);        // (a + dt_bias) log2 e
            const float sp = y > 20.0f * kLog2e ? y : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(y));
            gv[e] = nA * sp;                                            // gate, log2 units; pads do not decay
            Gm[e] = scan16(gv[e]);
            GC[e] = row_bcast<15>(Gm[e]);
            deep |= GC[e] < -100.f;
            e1[e] = __builtin_amdgcn_exp2f(Gm[e]);
            kd[e] = kf[e] * e1[e];
            qd[e] = qf[e] * e1[e];
        }
        const bf16x8 bkd = pack8(kd), bqd = pack8(qd);
        f32x4 pL, pLT, pMT;
        if (__ballot(deep) == 0) {
            // mild: rows k~ (<= 1), columns k 2^-G (<= 2^100); k^r = k 2^-G 2^{G_C}
            float kh[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kh[e] = kf[e] * __builtin_amdgcn_exp2f(-Gm[e]);
                kr[e] = kh[e] * row_bcast<15>(e1[e]);
            }
            const bf16x8 bkh = pack8(kh);
            pL = mma32(bkd, bkh, Z4);
            pLT = mma32(bkh, bkd, Z4);
            pMT = mma32(bkh, bqd, Z4);
        } else {
            // strong: two 8-token row blocks, each token's decay clipped at 2^-12
            constexpr float CLIP = 12.f;
            float Gp[8], Bf1[8], R[8], Rq[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kr[e] = kf[e] * __builtin_amdgcn_exp2f(GC[e] - Gm[e]);
                Gp[e] = scan16(fmaxf(gv[e], -CLIP));
                Bf1[e] = row_bcast<7>(Gp[e]);
                const float f = __builtin_amdgcn_exp2f(Gp[e] - (t >= 8 ? Bf1[e] : 0.f));   // <= 1
                R[e] = kf[e] * f;
                Rq[e] = qf[e] * f;
            }
            const bf16x8 bR = pack8(R), bRq = pack8(Rq);
            pL = pLT = pMT = Z4;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                float Cc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    Cc[e] = t < 8 * (bb + 1) ? kf[e] * __builtin_amdgcn_exp2f((bb ? Bf1[e] : 0.f) - Gp[e]) : 0.f;
                const bf16x8 bC = pack8(Cc);
                const f32x4 Lb = mma32(bR, bC, Z4), LTb = mma32(bC, bR, Z4), MTb = mma32(bC, bRq, Z4);
                if ((4 * r) / 8 == bb) pL = Lb;          // C-layout rows 4r .. 4r+3 of L lie in block bb
                if (t / 8 == bb) { pLT = LTb; pMT = MTb; }   // row t of L (as column t of L^T), of Mqk
            }
        }
        const bf16x8 bkr = pack8(kr);
        // payload of the consumers: q~ fragments, e^{G_C}, k^r C tiles
        *reinterpret_cast<bf16x8 *>(qke + L::QF + (w * 64 + lane) * 16) = bqd;
        if (t == CH - 1) {
            float *eg = reinterpret_cast<float *>(qke + L::EG) + 32 * w + 8 * r;
            *reinterpret_cast<f32x4 *>(eg) = f32x4{e1[0], e1[1], e1[2], e1[3]};
            *reinterpret_cast<f32x4 *>(eg + 4) = f32x4{e1[4], e1[5], e1[6], e1[7]};
        }
        f32x4 *pp = reinterpret_cast<f32x4 *>(lds + L::O_PART + (x & 1) * L::PART) + (w * 3) * 64 + lane;
        pp[0] = pL;
        pp[64] = pLT;
        pp[128] = pMT;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = 2 * w + h;
            *reinterpret_cast<bf16x4 *>(kv + L::KT + (m * 64 + lane) * 8) = pack4(mma32(bkd, sel_c[h], Z4));
            *reinterpret_cast<bf16x4 *>(qke + L::KR + (m * 64 + lane) * 8) = pack4(mma32(bkr, sel_c[h], Z4));
        }
#pragma unroll
        for (int i = 0; i < VPW; ++i) {
            const int vb = w + NPW * i;
            if (vb < NVB) {
                const bf16x8 bv = __builtin_bit_cast(bf16x8, in.v[i]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int n = 2 * vb + h;
                    if (n < NVT)
                        *reinterpret_cast<bf16x4 *>(kv + L::VT + (n * 64 + lane) * 8) = pack4(mma32(bv, sel_v[h], Z4));
                }
            }
        }
        if (w == 0 && r == 0) {
            float *bs = reinterpret_cast<float *>(lds + L::O_BETA + (x & 1) * 64);
            bs[t] = live ? sigmoid_f(bf16_to_f32(in.b)) : 0.f;
        }
    };

    // ---- stage B1 (wave 0): L, L^T, Mqk^T from the partials; INV; (INV beta)^T
    auto stage_b1 = [&](int x) {
        const f32x4 *pp = reinterpret_cast<const f32x4 *>(lds + L::O_PART + (x & 1) * L::PART) + lane;
        f32x4 Lm = Z4, LT = Z4, MT = Z4;
#pragma unroll
        for (int ww = 0; ww < NPW; ++ww) {
            Lm += pp[ww * 192];
            LT += pp[ww * 192 + 64];
            MT += pp[ww * 192 + 128];
        }
        const float *bs = reinterpret_cast<const float *>(lds + L::O_BETA + (x & 1) * 64);
        const f32x4 brow = *reinterpret_cast<const f32x4 *>(bs + 4 * lq);
        const float bcol = bs[ln];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * lq + i;
            Lm[i] = row > ln ? -brow[i] * Lm[i] : 0.f;   // L[row][ln], strictly lower
            LT[i] = ln > row ? -bcol * LT[i] : 0.f;      // L[ln][row]
            MT[i] = ln >= row ? MT[i] : 0.f;             // Mqk[ln][row], lower including the diagonal
        }
        const f32x4 L2 = prod(LT, Lm), L2T = prod(Lm, LT);
        const f32x4 L4 = prod(L2T, L2), L4T = prod(L2, L2T);
        const f32x4 L8 = prod(L4T, L4);
        // P1^T = ((I + L)(I + L^2))^T,  P2 = (I + L^4)(I + L^8),  INV^T = P2^T P1^T
        const f32x4 P1T = prod(plus_eye(L2, ln, lq), plus_eye(LT, ln, lq));
        const f32x4 P2 = prod(plus_eye(L4T, ln, lq), plus_eye(L8, ln, lq));
        const f32x4 IT = prod(P2, P1T);
        *reinterpret_cast<bf16x4 *>(lds + L::O_INVB + (x & 1) * 512 + lane * 8) = pack4(IT * brow);
        *reinterpret_cast<bf16x4 *>(lds + L::O_QKE + (x & 3) * L::QKE + L::MQ + lane * 8) = pack4(MT);
    };

    // ---- stage B2 (prep waves 1 ..): w = INV beta k~ (as C tiles of w^T) and u' = INV beta v
    auto stage_b2 = [&](int x) {
        const bf16x4 ib = *reinterpret_cast<const bf16x4 *>(lds + L::O_INVB + (x & 1) * 512 + lane * 8);
        const unsigned char *kv = lds + L::O_KV + (x % 3) * L::KV;
        unsigned char *wum = lds + L::O_WUM + (x & 1) * L::WUM;
        for (int job = w - 1; job < NKB + NVT; job += NPW - 1) {
            if (job < NKB) {
                const bf16x4 k0 = *reinterpret_cast<const bf16x4 *>(kv + L::KT + ((2 * job) * 64 + lane) * 8);
                const bf16x4 k1 = *reinterpret_cast<const bf16x4 *>(kv + L::KT + ((2 * job + 1) * 64 + lane) * 8);
                *reinterpret_cast<bf16x8 *>(wum + L::WF + (job * 64 + lane) * 16) =
                    cat4(pack4(mma16(k0, ib, Z4)), pack4(mma16(k1, ib, Z4)));
            } else {
                const int n = job - NKB;
                const bf16x4 vt = *reinterpret_cast<const bf16x4 *>(kv + L::VT + (n * 64 + lane) * 8);
                *reinterpret_cast<f32x4 *>(wum + L::UP + (n * 64 + lane) * 16) = mma16(ib, vt, Z4);
            }
        }
    };

    In<VPW> in0, in1;
    load(in0, 0);
    // chunk x's inputs sit in in[x & 1], loaded one iteration before stage A uses them
    auto body = [&](int it, In<VPW> &use, In<VPW> &fill) {
        // the only loads in flight here are `use`'s, issued an iteration ago: wait
        // for them now, so that no later wait covers the loads issued next
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        asm volatile("" ::: "memory");
        if (it + 4 < c.nch) load(fill, it + 4);
        if (w == 0 && it + 2 >= 0 && it + 2 < c.nch) stage_b1(it + 2);
        if (it + 3 < c.nch) stage_a(use, it + 3);
        if (w > 0 && it + 1 >= 0 && it + 1 < c.nch) stage_b2(it + 1);
        lds_barrier();
    };
    for (int it = -3; it < c.nch; it += 2) {
        body(it, in0, in1);
        if (it + 1 < c.nch) body(it + 1, in1, in0);
    }
}

namespace {

template <int DK, int DV, int NCW, int SPW, bool SNAP>
hipError_t launch_t(const FwdArgs &a, hipStream_t stream)
{
    using L = Lay<DK, DV, NCW, SPW>;
    const long long wgs = (long long)a.n_seq * a.H * L::G;
    if (wgs == 0) return hipSuccess;
    if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_kernel<DK, DV, NCW, SPW, SNAP>), dim3((unsigned)wgs), dim3(L::NTHR), 0, stream, a);
    return hipGetLastError();
}

// Column groups per chain: the fewest that give at least one workgroup per
// compute unit (the prep is repeated in every group of a chain).
template <int DK, int DV, bool SNAP>
hipError_t launch_dims(const FwdArgs &a, int n_cu, hipStream_t stream)
{
    const long long chains = (long long)a.n_seq * a.H;
    int G = 1;
    while (G < DV / 16 && chains * G < n_cu) G *= 2;
    if constexpr (DV == 128) {
        switch (G) {
        case 1: return launch_t<DK, DV, 4, 2, SNAP>(a, stream);
        case 2: return launch_t<DK, DV, 4, 1, SNAP>(a, stream);
        case 4: return launch_t<DK, DV, 2, 1, SNAP>(a, stream);
        default: return launch_t<DK, DV, 1, 1, SNAP>(a, stream);
        }
    } else {
        switch (G) {
        case 1: return launch_t<DK, DV, 2, 2, SNAP>(a, stream);
        case 2: return launch_t<DK, DV, 2, 1, SNAP>(a, stream);
        default: return launch_t<DK, DV, 1, 1, SNAP>(a, stream);
        }
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, int dk, int dv, hipStream_t stream)
{
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
#define KDA_FWD(DKV, DVV)                                                                  \
    if (dk == DKV && dv == DVV)                                                            \
        return a.h_chunks ? launch_dims<DKV, DVV, true>(a, n_cu, stream)                   \
                          : launch_dims<DKV, DVV, false>(a, n_cu, stream);
    KDA_FWD(128, 128)
    KDA_FWD(128, 64)
    KDA_FWD(64, 128)
    KDA_FWD(64, 64)
#undef KDA_FWD
    return hipErrorInvalidValue;
}

}  // namespace kda
