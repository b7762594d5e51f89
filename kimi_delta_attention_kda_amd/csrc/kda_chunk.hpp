// kda_chunk.hpp -- the chunk machinery shared by the prefill (kda_fwd.hip)
// and the backward (kda_backward.hip) for gfx950 (CDNA4), bf16 activations:
// MFMA helpers, the prep stages, the recurrence step, chunk addressing and
// the direct global-to-LDS loads.
//
// Pages cited by title and section:
//   [TL-KDA]  "TileLang 实战：KDA 从零到一 -- Chunked 线性注意力": section 1
//             (recurrence, (d_v, d_k) state), 6.4 (the state is carried
//             through a sequential chunk loop inside the block: the sequence
//             axis stays out of the grid), 6.4.1 (split d_v, never d_k),
//             6.4.2 (the state advances after the chunk's output).
//   [LA-06]   "06 · linear 路线（一）：kernel trick、RNN 等价与三种计算形式":
//             chunkwise form (the state-independent per-chunk terms can be
//             formed for all chunks in parallel ahead of the recurrence).
//   [FKDA-LM] "FlashKDA 里的 L 矩阵和 Mqk 矩阵是什么": "30秒速览" (U, output and
//             state advance), "L 矩阵的构造" (strictly lower, rows scaled by
//             beta), "Mqk 矩阵的构造" (lower including the diagonal), "为什么
//             CHUNK16" (L^16 = 0; inverse by Neumann squaring), "K2 内核如何消费"
//             (a prep step and a recurrence step that consumes its operands).
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
// Everything that does not depend on the state (the "prep") is built by prep
// waves in three stages per chunk:
//   A  (NPW = d_k / 32 waves, one 32-channel block each): gate, cumulative gate,
//      decayed operands, this block's partials of L, L^T and Mqk^T on the
//      matrix core, layout copies of k~, k^r (and v);
//   B1 (one wave): sums the partials, masks, beta, INV by Neumann squaring, INV beta;
//   B2 (stage-A waves 1 ..): w on the matrix core (u' = INV beta v is formed
//      by the recurrence's waves from the v C tiles).
// The recurrence runs in consumer waves, each owning slabs of 16 state columns
// in fp32 MFMA accumulators:
//   W' = w S, Qs^T = S^T q~^T, decay, U = u' - W', O^T = Qs^T + U^T Mqk^T, S += k^r^T U.
//
// Operand layouts.  For a 16 x 16 tile X the "C layout" is the MFMA
// accumulator layout: lane (lq, ln) = (lane / 16, lane % 16) holds
// X[4 lq + i][ln], i = 0..3.  A K = 16 product X Y in the 16x16x16 bf16 layout
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
#pragma once

#include <stdint.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int CH = 16;

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// A K = 16 product (the v_mfma_f32_16x16x16_bf16 operand layout: lane (lq, ln)
// holds A[ln][4 lq .. +3] and B[4 lq .. +3][ln]) issued as v_mfma_f32_16x16x32_bf16
// with the upper four K values of every lane zero: the same sum, and on gfx950
// the same issue rate.  The 16x16x16 instruction itself gave wrong results in
// some instruction sequences here (a 16x16 product of selector copies came out
// wrong in its second channel tile while the same code built on the K = 32
// instruction was exact to fp32 rounding), so no kernel uses it.
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16x4 z = {};
    bf16x8 a8, b8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a8[i] = a[i];
        a8[4 + i] = z[i];
        b8[i] = b[i];
        b8[4 + i] = z[i];
    }
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c, 0, 0, 0);
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
// Both read 0 from a source lane outside the row (bound control set), so no
// register has to be cleared first.
template <int CTRL>
__device__ __forceinline__ float dpp_z(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                                                 true));
}
__device__ __forceinline__ float scan16(float x) {
    x += dpp_z<0x111>(x);
    x += dpp_z<0x112>(x);
    x += dpp_z<0x114>(x);
    x += dpp_z<0x118>(x);
    return x;
}
// The same scan over 8 independent values, step by step across all of them
// (each step's 8 operations are independent, so no DPP read waits on the
// write just before it).
__device__ __forceinline__ void scan16x8(float (&x)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += dpp_z<0x111>(x[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += dpp_z<0x112>(x[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += dpp_z<0x114>(x[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += dpp_z<0x118>(x[e]);
}
template <int N>
__device__ __forceinline__ float row_bcast(float x) { return dpp_z<0x150 + N>(x); }

__device__ __forceinline__ void lds_barrier() {   // LDS-only barrier: global loads stay in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void vm_wait_all() {   // all of this wave's global loads have landed
    __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0)
    asm volatile("" ::: "memory");
}

// Channel of row 4 lq + i of state tile m (and of the matching rows of every
// C-layout channel tile): the 8 K values a lane feeds to a 16x16x32 MFMA in K
// block s are then the 8 consecutive channels 32 s + 8 lq .. +7.
__device__ __forceinline__ constexpr int chan(int m, int lq, int i) { return 32 * (m >> 1) + 8 * lq + 4 * (m & 1) + i; }

// Consumer operands of one chunk (a workspace row of the two-pass form; the
// one-pass form keeps the same pieces in LDS): byte offsets.
template <int DK>
struct Pay {
    static constexpr int NKB = DK / 32, NMT = DK / 16;
    static constexpr int QF = 0;                    // q~ B fragments   [NKB][64] x 16 B
    static constexpr int WF = QF + NKB * 1024;      // w A fragments    [NKB][64] x 16 B
    static constexpr int KR = WF + NKB * 1024;      // k^r C tiles      [NMT][64] x 8 B (bf16)
    static constexpr int EG = KR + NMT * 512;       // e^{G_C}          [DK] fp32
    static constexpr int MQ = EG + DK * 4;          // Mqk^T C tile     [64] x 8 B (bf16)
    static constexpr int IB = MQ + 512;             // (INV beta)^T C tile [64] x 8 B (bf16)
    static constexpr int BYTES = IB + 512;
};

template <int DK, int DV, int NCW, int SPW>
struct Lay {
    using P = Pay<DK>;
    static constexpr int NPW = DK / 32;           // stage-A waves (one 32-channel block each)
    static constexpr int NKB = DK / 32;           // K blocks of the state products
    static constexpr int NMT = DK / 16;           // state row tiles
    static constexpr int NCOL = NCW * SPW * 16;   // columns of the group
    static constexpr int G = DV / NCOL;           // column groups per chain
    static constexpr int NVT = NCOL / 16;         // 16-column tiles of the group
    static constexpr int NVB = (NCOL + 31) / 32;  // 32-column v blocks
    static constexpr int VPW = (NVB + NPW - 1) / NPW;   // v blocks per stage-A wave
    static constexpr int NW = NPW + 1 + NCW;       // stage-A waves, the INV wave, consumers
    static constexpr int NTHR = 64 * NW;
    static constexpr int PAY = P::BYTES;          // consumer operands (4 buffers: written from 3 iterations ahead)
    static constexpr int KT = 0;                  // k~ C tiles [NMT][64] x 8 B  (4 buffers)
    static constexpr int VT = KT + NMT * 512;     // v C tiles  [NVT][64] x 8 B
    static constexpr int KV = VT + NVT * 512;
    static constexpr int PART = NPW * 3 * 1024;   // per stage-A wave: L, L^T, Mqk^T partials (2 buffers)
    static constexpr int O_PAY = 0;
    static constexpr int O_KV = O_PAY + 4 * PAY;
    static constexpr int O_PART = O_KV + 4 * KV;
    static constexpr int O_BETA = O_PART + 2 * PART;   // beta [16] (2 buffers)
    static constexpr int O_SEQ = O_BETA + 2 * 64;      // the sequence this workgroup takes
    static constexpr int BYTES = O_SEQ + 16;
    static_assert(DK == 64 || DK == 128, "d_k");
    static_assert(NCOL * G == DV && NCOL % 16 == 0, "column groups");
    static_assert(BYTES <= 160 * 1024, "LDS");
};

// Packed sequences with at most this many entries are taken longest first.
constexpr int LPT_MAX = 128;

// Inputs of one chunk as a stage-A lane holds them: token t = lane % 16, the
// 8 channels 32 w + 8 (lane / 16) .. +7 of q, k, g_raw; v blocks; beta_raw.
template <int VPW>
struct In {
    uint4 k, q, a;
    uint4 v[VPW > 0 ? VPW : 1];
    uint16_t b;
};

// ------------------------------------------------------------------ prep
// One stage-A wave: its 32-channel block, its constants, its loads and stage A.
template <int DK, int VPW>
struct Prep {
    static constexpr int NPW = DK / 32;
    int w, t, r, lane, ln, lq;
    float A_exp, dtl[8];
    bf16x8 sel_c[2], sel_v[2];

    // the channel block and lane (all that load needs)
    __device__ __forceinline__ void place(int wave, int lane_) {
        w = wave;
        lane = lane_;
        ln = lane & 15;
        lq = lane >> 4;
        t = ln;
        r = lq;
    }
    __device__ __forceinline__ void init(const FwdArgs &a, int head, int wave, int lane_) {
        place(wave, lane_);
        A_exp = expf(a.A_log[head]);
#pragma unroll
        for (int e = 0; e < 8; ++e) dtl[e] = a.dt_bias[(size_t)head * DK + 32 * w + 8 * r + e] * kLog2e;
        // 0/1 selectors: C-layout copies of row-loaded tiles (the channels of
        // state tile 2w + h; columns 16 (2 vb + h) .. + 15 of a v block)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sel_c[h][e] = static_cast<__bf16>((lq == (ln >> 2) && e == 4 * h + (ln & 3)) ? 1.f : 0.f);
                sel_v[h][e] = static_cast<__bf16>((lq == 2 * h + (ln >> 3) && e == (ln & 7)) ? 1.f : 0.f);
            }
    }

    // Loads of chunk x of the sequence starting at token bos with len tokens
    // (x < ceil(len / 16)); v blocks vb = w, w + NPW, ... (< nvb) of the
    // columns col0 .. col0 + ncol of a row of dv columns.
    __device__ __forceinline__ void load(In<VPW> &in, const FwdArgs &a, size_t bos, int len, int x, int head,
                                         int dv, int col0, int ncol, int nvb) const {
        const size_t H = a.H;
        const int rem = min(CH, len - x * CH);
        const size_t tok = bos + (size_t)x * CH + min(t, rem - 1);   // rows past the end repeat the last live row
        const size_t off = (tok * H + head) * DK + 32 * w + 8 * r;
        in.k = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + off);
        in.q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + off);
        in.a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.g_raw) + off);
#pragma unroll
        for (int i = 0; i < VPW; ++i) {
            const int vb = w + NPW * i;
            if (vb < nvb && 32 * vb + 8 * r < ncol)
                in.v[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) +
                                                           (tok * H + head) * dv + col0 + 32 * vb + 8 * r);
            else
                in.v[i] = uint4{0u, 0u, 0u, 0u};
        }
        in.b = (w == 0) ? static_cast<const uint16_t *>(a.beta_raw)[tok * H + head] : (uint16_t)0;
    }

    // Stage A of a chunk with `rem` live tokens, the arithmetic: q~ and k~ (bf16
    // K fragments of this block's 32 channels), k^r, e^G of each token and
    // channel (e1; the chunk's e^{G_C} in the lanes of token 15), this block's
    // partials of L, L^T and Mqk^T (before masks and beta).
    struct Out {
        bf16x8 bqd, bkd, bkr;
        float e1[8];
        f32x4 pL, pLT, pMT;
    };
    __device__ __forceinline__ void stage_a_core(const In<VPW> &in, int rem, Out &o) const {
        const bool live = t < rem;
        const float nA = live ? -A_exp : 0.f;
        float kf[8], qfv[8], gv[8], Gm[8], kd[8], qd[8], krv[8];
        // pad tokens: k and q read as zero (their rows repeat the last live row)
        const uint32_t lm = live ? 0xffffffffu : 0u;
        const uint32_t kw[4] = {in.k.x & lm, in.k.y & lm, in.k.z & lm, in.k.w & lm};
        const uint32_t qw[4] = {in.q.x & lm, in.q.y & lm, in.q.z & lm, in.q.w & lm};
        const uint32_t aw[4] = {in.a.x, in.a.y, in.a.z, in.a.w};
        // the gate is never positive, so G falls along the chunk and its lowest value
        // over all lanes is the lowest chunk total G_C
        float gmin = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sh = (e & 1) ? 0 : 16;
            const uint32_t mk = (e & 1) ? 0xffff0000u : 0xffffffffu;
            kf[e] = __builtin_bit_cast(float, (kw[e >> 1] << sh) & mk);
            qfv[e] = __builtin_bit_cast(float, (qw[e >> 1] << sh) & mk);
            const float af = __builtin_bit_cast(float, (aw[e >> 1] << sh) & mk);
            const float y = __builtin_fmaf(af, kLog2e, dtl[e]);        // (a + dt_bias) log2 e
            const float sp = y > 20.0f * kLog2e ? y : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(y));
            gv[e] = nA * sp;                                            // gate, log2 units; pads do not decay
            Gm[e] = gv[e];
        }
        scan16x8(Gm);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gmin = fminf(gmin, Gm[e]);
            o.e1[e] = __builtin_amdgcn_exp2f(Gm[e]);
            kd[e] = kf[e] * o.e1[e];
            qd[e] = qfv[e] * o.e1[e];
        }
        o.bkd = pack8(kd);
        o.bqd = pack8(qd);
        if (__ballot(gmin < -100.f) == 0) {
            // mild: rows k~ (<= 1), columns k 2^-G (<= 2^100); k^r = k 2^-G 2^{G_C}
            float kh[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kh[e] = kf[e] * __builtin_amdgcn_exp2f(-Gm[e]);
                krv[e] = kh[e] * row_bcast<15>(o.e1[e]);
            }
            const bf16x8 bkh = pack8(kh);
            o.pL = mma32(o.bkd, bkh, Z4);
            o.pLT = mma32(bkh, o.bkd, Z4);
            o.pMT = mma32(bkh, o.bqd, Z4);
        } else {
            // strong: two 8-token row blocks, each token's decay clipped at 2^-12
            constexpr float CLIP = 12.f;
            float Gp[8], Bf1[8], R[8], Rq[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                krv[e] = kf[e] * __builtin_amdgcn_exp2f(row_bcast<15>(Gm[e]) - Gm[e]);
                Gp[e] = scan16(fmaxf(gv[e], -CLIP));
                Bf1[e] = row_bcast<7>(Gp[e]);
                const float f = __builtin_amdgcn_exp2f(Gp[e] - (t >= 8 ? Bf1[e] : 0.f));   // <= 1
                R[e] = kf[e] * f;
                Rq[e] = qfv[e] * f;
            }
            const bf16x8 bR = pack8(R), bRq = pack8(Rq);
            o.pL = o.pLT = o.pMT = Z4;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                float Cc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    Cc[e] = t < 8 * (bb + 1) ? kf[e] * __builtin_amdgcn_exp2f((bb ? Bf1[e] : 0.f) - Gp[e]) : 0.f;
                const bf16x8 bC = pack8(Cc);
                const f32x4 Lb = mma32(bR, bC, Z4), LTb = mma32(bC, bR, Z4), MTb = mma32(bC, bRq, Z4);
                if ((4 * r) / 8 == bb) o.pL = Lb;          // C-layout rows 4r .. 4r+3 of L lie in block bb
                if (t / 8 == bb) { o.pLT = LTb; o.pMT = MTb; }   // row t of L (as column t of L^T), of Mqk
            }
        }
        o.bkr = pack8(krv);
    }
    // e^{G_C} of this block's channels from the lanes of token 15
    __device__ __forceinline__ void store_eg(const Out &o, float *eg) const {
        if (t == CH - 1) {
            float *egw = eg + 32 * w + 8 * r;
            *reinterpret_cast<f32x4 *>(egw) = f32x4{o.e1[0], o.e1[1], o.e1[2], o.e1[3]};
            *reinterpret_cast<f32x4 *>(egw + 4) = f32x4{o.e1[4], o.e1[5], o.e1[6], o.e1[7]};
        }
    }
    // C tiles 2w + h of a row-loaded channel block (one selector MFMA each)
    __device__ __forceinline__ bf16x4 ctile(bf16x8 x, int h) const { return pack4(mma32(x, sel_c[h], Z4)); }

    // Stage A of a chunk with `rem` live tokens.  Writes q~ fragments (qf),
    // e^{G_C} (eg), k^r C tiles (kr), k~ C tiles (kt), v C tiles (vt, nvt
    // tiles of nvb blocks; none if vt is NULL), this wave's L / L^T / Mqk^T
    // partials (part) and, from wave 0, beta (beta).
    __device__ __forceinline__ void stage_a(const In<VPW> &in, int rem, unsigned char *qf, float *eg,
                                            unsigned char *kr, unsigned char *kt, unsigned char *vt, int nvb, int nvt,
                                            f32x4 *part, float *beta) const {
        Out o;
        stage_a_core(in, rem, o);
        *reinterpret_cast<bf16x8 *>(qf + (w * 64 + lane) * 16) = o.bqd;
        store_eg(o, eg);
        f32x4 *pp = part + (w * 3) * 64 + lane;
        pp[0] = o.pL;
        pp[64] = o.pLT;
        pp[128] = o.pMT;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = 2 * w + h;
            *reinterpret_cast<bf16x4 *>(kt + (m * 64 + lane) * 8) = ctile(o.bkd, h);
            *reinterpret_cast<bf16x4 *>(kr + (m * 64 + lane) * 8) = ctile(o.bkr, h);
        }
        if (vt) {
#pragma unroll
            for (int i = 0; i < VPW; ++i) {
                const int vb = w + NPW * i;
                if (vb < nvb) {
                    const bf16x8 bv = __builtin_bit_cast(bf16x8, in.v[i]);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int n = 2 * vb + h;
                        if (n < nvt)
                            *reinterpret_cast<bf16x4 *>(vt + (n * 64 + lane) * 8) = pack4(mma32(bv, sel_v[h], Z4));
                    }
                }
            }
        }
        if (w == 0 && r == 0) beta[t] = t < rem ? sigmoid_f(bf16_to_f32(in.b)) : 0.f;
    }
};

// Stage B1 from the summed partials of L, L^T, Mqk^T and beta (brow: tokens
// 4 lq .. +3 of this lane, bcol: token ln): masks, beta, INV by Neumann
// squaring.  Returns the C layouts of (INV beta)^T and Mqk^T, in bf16.
__device__ __forceinline__ void b1_core(f32x4 Lm, f32x4 LT, f32x4 MT, f32x4 brow, float bcol, int lane, bf16x4 &ib,
                                        bf16x4 &mq) {
    const int ln = lane & 15, lq = lane >> 4;
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
    ib = pack4(IT * brow);
    mq = pack4(MT);
}

// Stage B1 (one wave): L, L^T, Mqk^T from the NPW partials; INV; writes the
// C layout of (INV beta)^T (bf16) to ib and of Mqk^T (bf16) to mq.
template <int NPW>
__device__ __forceinline__ void stage_b1(const f32x4 *part, const float *beta, unsigned char *ib, unsigned char *mq,
                                         int lane) {
    const int ln = lane & 15, lq = lane >> 4;
    const f32x4 *pp = part + lane;
    f32x4 Lm = Z4, LT = Z4, MT = Z4;
#pragma unroll
    for (int ww = 0; ww < NPW; ++ww) {
        Lm += pp[ww * 192];
        LT += pp[ww * 192 + 64];
        MT += pp[ww * 192 + 128];
    }
    bf16x4 ibv, mqv;
    b1_core(Lm, LT, MT, *reinterpret_cast<const f32x4 *>(beta + 4 * lq), beta[ln], lane, ibv, mqv);
    *reinterpret_cast<bf16x4 *>(ib + lane * 8) = ibv;
    *reinterpret_cast<bf16x4 *>(mq + lane * 8) = mqv;
}

// w = INV beta k~ for K block s: the A fragment of W' = w S (from the C tiles
// 2s, 2s+1 of k~ and the C layout of (INV beta)^T).
__device__ __forceinline__ bf16x8 w_frag2(bf16x4 k0, bf16x4 k1, bf16x4 ib) {
    return cat4(pack4(mma16(k0, ib, Z4)), pack4(mma16(k1, ib, Z4)));
}
__device__ __forceinline__ bf16x8 w_frag(const unsigned char *kt, bf16x4 ib, int s, int lane) {
    return w_frag2(*reinterpret_cast<const bf16x4 *>(kt + ((2 * s) * 64 + lane) * 8),
                   *reinterpret_cast<const bf16x4 *>(kt + ((2 * s + 1) * 64 + lane) * 8), ib);
}

// One chunk of the recurrence for SPW slabs of 16 columns: S holds the state
// entering the chunk and leaves with the state after it; O gets O^T / scale.
template <int NKB, int NMT, int SPW>
__device__ __forceinline__ void rec_step(f32x4 (&S)[SPW][NMT], const bf16x8 (&qf)[NKB], const bf16x8 (&wf)[NKB],
                                         const bf16x4 (&kr)[NMT], const f32x4 (&eg)[NMT], bf16x4 mq,
                                         const f32x4 (&up)[SPW], f32x4 (&O)[SPW]) {
    // the state entering the chunk, as bf16 K fragments (B of W' = w S, A of Qs^T = S^T q~^T)
    bf16x8 bS[SPW][NKB];
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
        for (int s = 0; s < NKB; ++s) bS[j][s] = cat4(pack4(S[j][2 * s]), pack4(S[j][2 * s + 1]));
    f32x4 W[SPW], Qs[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) { W[j] = Z4; Qs[j] = Z4; }
#pragma unroll
    for (int s = 0; s < NKB; ++s)
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            W[j] = mma32(wf[s], bS[j][s], W[j]);
            Qs[j] = mma32(bS[j][s], qf[s], Qs[j]);
        }
    // decay the fp32 state: S <- Diag(e^{G_C}) S
#pragma unroll
    for (int m = 0; m < NMT; ++m)
#pragma unroll
        for (int j = 0; j < SPW; ++j) S[j][m] *= eg[m];
    const bf16x8 bmq = cat4(mq, mq);
    bf16x8 bU[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        bU[j] = hilo(up[j] - W[j]);            // U = u' - w S as [hi | lo]
        O[j] = mma32(bU[j], bmq, Qs[j]);       // O^T = Qs^T + U^T Mqk^T
    }
    // S += k^r^T U (the k^r values repeated for the hi and lo halves of U)
#pragma unroll
    for (int m = 0; m < NMT; ++m) {
        const bf16x8 bkr = cat4(kr[m], kr[m]);
#pragma unroll
        for (int j = 0; j < SPW; ++j) S[j][m] = mma32(bkr, bU[j], S[j][m]);
    }
}

// O^T in C layout: lane (lq, ln) holds columns 4 lq .. +3 of token ln.
__device__ __forceinline__ void store_o(void *o, size_t row, size_t H, int head, int dv, int col, f32x4 O,
                                        float scale) {
    uint2 v2;
    v2.x = pack_bf16x2(scale * O[0], scale * O[1]);
    v2.y = pack_bf16x2(scale * O[2], scale * O[3]);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(o) + (row * H + head) * dv + col) = v2;
}

struct Chain {
    size_t bos;
    int len, nch, seq, head, hrow;
};
// Sequence `seq`, head `head`: token range, chunk count and state row (a
// pool slot >= P is reported and treated as none).
__device__ __forceinline__ Chain chain_of(const FwdArgs &a, int seq, int head, bool report) {
    Chain c;
    c.seq = seq;
    c.head = head;
    if (a.cu_seqlens) {
        c.bos = (size_t)a.cu_seqlens[seq];
        c.len = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
    } else {
        c.bos = (size_t)seq * a.T;
        c.len = a.T;
    }
    c.nch = (c.len + CH - 1) / CH;
    c.hrow = a.state_idx ? a.state_idx[seq] : seq;
    if (a.state_idx && c.hrow >= a.P) {
        if (report) slot_error(a.err);
        c.hrow = -1;
    }
    return c;
}
// Chunks of the sequences before `seq` (the row of its first chunk in the
// chunk-indexed arrays).
__device__ __forceinline__ size_t chunk_base(const FwdArgs &a, int seq) {
    if (!a.cu_seqlens) return (size_t)seq * ((a.T + CH - 1) / CH);
    size_t b = 0;
    for (int s2 = 0; s2 < seq; ++s2) b += (size_t)((a.cu_seqlens[s2 + 1] - a.cu_seqlens[s2] + CH - 1) / CH);
    return b;
}

// Chunk row `row` of the concatenated chunk rows (sequence 0's chunks, then
// sequence 1's, ...): its sequence, chunk, first token and length; seq =
// n_seq past the last row.
struct RowPos {
    size_t bos;
    int seq, x, len;
};
__device__ __forceinline__ RowPos row_pos(const FwdArgs &a, long long row) {
    RowPos p;
    p.x = 0;
    p.bos = 0;
    p.len = 0;
    if (!a.cu_seqlens) {
        const int nch = (a.T + CH - 1) / CH;
        p.seq = nch > 0 ? (int)(row / nch) : a.n_seq;
        if (p.seq < a.n_seq) {
            p.x = (int)(row - (long long)p.seq * nch);
            p.bos = (size_t)p.seq * a.T;
            p.len = a.T;
        } else {
            p.seq = a.n_seq;
        }
        return p;
    }
    for (p.seq = 0; p.seq < a.n_seq; ++p.seq) {
        const int len = a.cu_seqlens[p.seq + 1] - a.cu_seqlens[p.seq];
        const int nch = (len + CH - 1) / CH;
        if (row < nch) {
            p.x = (int)row;
            p.bos = (size_t)a.cu_seqlens[p.seq];
            p.len = len;
            return p;
        }
        row -= nch;
    }
    return p;
}

}  // namespace

// Prep waves per workgroup of the per-chunk kernels (one wave per (chunk row, head)).
constexpr int PREP_WAVES = 4;

// Direct global-to-LDS loads for the chunk loops of the recurrences: a
// chunk's operands reach a ring of RING LDS slots, RING - 1 chunks ahead.
// The loads are issued from inline assembly (the compiler would otherwise
// wait for all of them before every LDS read); each is counted in the
// wave's vmcnt, which drains in issue order.
namespace {
constexpr int RING = 5;

// Direct global-to-LDS loads of 16 bytes per lane: load i of a group reads
// base + voff + 1024 i (the last one voff_last + 1024 i) into LDS bytes
// lds + 1024 i + 16 lane .. (the instruction offset moves both addresses; m0,
// the LDS address register, is set for the group and then restored).
template <int N>
__device__ __forceinline__ void dma_group(const void *base, unsigned voff, unsigned voff_last, unsigned lds) {
    static_assert(N >= 1 && N <= 4, "one 4 KiB group");
    // wave-uniform operands, made explicit for the scalar-register constraints
    lds = __builtin_amdgcn_readfirstlane(lds);
    const uint64_t b64 = reinterpret_cast<uint64_t>(base);
    base = reinterpret_cast<const void *>(
        ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)(b64 >> 32)) << 32) |
        (unsigned)__builtin_amdgcn_readfirstlane((unsigned)b64));
    unsigned keep;
    if constexpr (N == 4)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, %3\n\t"
                     "global_load_lds_dwordx4 %1, %3 offset:1024\n\t"
                     "global_load_lds_dwordx4 %1, %3 offset:2048\n\t"
                     "global_load_lds_dwordx4 %2, %3 offset:3072\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(keep) : "v"(voff), "v"(voff_last), "s"(base), "s"(lds) : "memory");
    else if constexpr (N == 3)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, %3\n\t"
                     "global_load_lds_dwordx4 %1, %3 offset:1024\n\t"
                     "global_load_lds_dwordx4 %2, %3 offset:2048\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(keep) : "v"(voff), "v"(voff_last), "s"(base), "s"(lds) : "memory");
    else if constexpr (N == 2)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, %3\n\t"
                     "global_load_lds_dwordx4 %2, %3 offset:1024\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(keep) : "v"(voff), "v"(voff_last), "s"(base), "s"(lds) : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, %2\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(keep) : "v"(voff_last), "s"(base), "s"(lds) : "memory");
}
// NB bytes (a multiple of 16) from base into LDS at lds, in 1 KiB loads; the
// lanes of the last load that would pass the end re-read its last 16 bytes
// (landing in LDS padding past NB).
template <int NB>
__device__ __forceinline__ void dma_bytes(const unsigned char *base, unsigned lds, int lane) {
    constexpr int NL = (NB + 1023) / 1024;
#pragma unroll
    for (int g = 0; g < (NL + 3) / 4; ++g) {
        const int first = 4 * g;
        const unsigned voff = 4096u * g + 16u * lane;
        if (first + 4 < NL) {
            dma_group<4>(base, voff, voff, lds + 4096u * g);
        } else {
            // the group holding the last load: its clamped offset, relative to the load's instruction offset
            const unsigned last = (unsigned)min((NL - 1) * 1024 + 16 * lane, NB - 16) - 1024u * (NL - 1 - first);
            switch (NL - first) {
            case 4: dma_group<4>(base, voff, last, lds + 4096u * g); break;
            case 3: dma_group<3>(base, voff, last, lds + 4096u * g); break;
            case 2: dma_group<2>(base, voff, last, lds + 4096u * g); break;
            default: dma_group<1>(base, voff, last, lds + 4096u * g); break;
            }
        }
    }
}
// Wait until at most n of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait_le() {
    static_assert(N >= 0 && N <= 63, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}
template <int ND, int K = RING - 1>
__device__ __forceinline__ void vm_wait_chunks(int k) {   // at most k chunks of ND loads outstanding
    if constexpr (K == 0) {
        vm_wait_le<0>();
    } else {
        if (k >= K) vm_wait_le<K * ND>();
        else vm_wait_chunks<ND, K - 1>(k);
    }
}
}  // namespace

}  // namespace kda
