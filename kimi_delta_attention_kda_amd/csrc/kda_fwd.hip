// kda_fwd.hip -- chunkwise KDA prefill for gfx950 (CDNA4), bf16 activations.
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
//   B2 (stage-A waves 1 ..): w (and u') on the matrix core.
// The recurrence runs in consumer waves, each owning slabs of 16 state columns
// in fp32 MFMA accumulators:
//   W' = w S, Qs^T = S^T q~^T, decay, U = u' - W', O^T = Qs^T + U^T Mqk^T, S += k^r^T U.
//
// Two ways to run it (the launcher picks by the number of (sequence, head)
// chains against the compute units, and by the caller's workspace):
//   * ONE PASS (fwd_kernel): one workgroup per (sequence, head, column group)
//     holds prep and consumer waves; the three prep stages of successive
//     chunks run three iterations ahead of the consumers and hand over through
//     LDS, one barrier per chunk.  No memory besides the arguments.  A chain
//     split over G column groups repeats the prep in each group, so this is
//     the form for many chains.
//   * TWO PASSES (prep_kernel, then rec_kernel), for chains fewer than the
//     compute units: every chunk's prep runs once, all chunks in parallel, and
//     its consumer operands (q~, w, k^r, e^{G_C}, Mqk^T, INV beta; 13.5 KiB
//     per chunk and head at d_k = 128) go to the caller's workspace; then one
//     single-wave workgroup per (sequence, head, 16 columns) walks the chunks,
//     prefetching the next chunk's operands straight into registers, forming
//     u' = INV beta v from its own columns of v and running the recurrence.
//     No workgroup waits on another in either pass.
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
    static constexpr int UP = NVT * 1024;         // u' C tiles [NVT][64] x 16 B fp32 (2 buffers)
    static constexpr int KT = 0;                  // k~ C tiles [NMT][64] x 8 B  (3 buffers)
    static constexpr int VT = KT + NMT * 512;     // v C tiles  [NVT][64] x 8 B
    static constexpr int KV = VT + NVT * 512;
    static constexpr int PART = NPW * 3 * 1024;   // per stage-A wave: L, L^T, Mqk^T partials (2 buffers)
    static constexpr int O_PAY = 0;
    static constexpr int O_UP = O_PAY + 4 * PAY;
    static constexpr int O_KV = O_UP + 2 * UP;
    static constexpr int O_PART = O_KV + 3 * KV;
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

    __device__ __forceinline__ void init(const FwdArgs &a, int head, int wave, int lane_) {
        w = wave;
        lane = lane_;
        ln = lane & 15;
        lq = lane >> 4;
        t = ln;
        r = lq;
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
        float kf[8], qfv[8], gv[8], Gm[8], GC[8], kd[8], qd[8], krv[8];
        const uint32_t kw[4] = {in.k.x, in.k.y, in.k.z, in.k.w};
        const uint32_t qw[4] = {in.q.x, in.q.y, in.q.z, in.q.w};
        const uint32_t aw[4] = {in.a.x, in.a.y, in.a.z, in.a.w};
        bool deep = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sh = (e & 1) ? 0 : 16;
            const uint32_t mk = (e & 1) ? 0xffff0000u : 0xffffffffu;
            kf[e] = live ? __builtin_bit_cast(float, (kw[e >> 1] << sh) & mk) : 0.f;
            qfv[e] = live ? __builtin_bit_cast(float, (qw[e >> 1] << sh) & mk) : 0.f;
            const float af = __builtin_bit_cast(float, (aw[e >> 1] << sh) & mk);
            const float y = __builtin_fmaf(af, kLog2e, dtl[e]);        // (a + dt_bias) log2 e
            const float sp = y > 20.0f * kLog2e ? y : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(y));
            gv[e] = nA * sp;                                            // gate, log2 units; pads do not decay
            Gm[e] = scan16(gv[e]);
            GC[e] = row_bcast<15>(Gm[e]);
            deep |= GC[e] < -100.f;
            o.e1[e] = __builtin_amdgcn_exp2f(Gm[e]);
            kd[e] = kf[e] * o.e1[e];
            qd[e] = qfv[e] * o.e1[e];
        }
        o.bkd = pack8(kd);
        o.bqd = pack8(qd);
        if (__ballot(deep) == 0) {
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
                krv[e] = kf[e] * __builtin_amdgcn_exp2f(GC[e] - Gm[e]);
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

// =========================================================== one pass
template <int DK, int DV, int NCW, int SPW, bool SNAP>
__global__ __launch_bounds__(64 * (DK / 32 + 1 + NCW)) void fwd_kernel(FwdArgs a)
{
    using L = Lay<DK, DV, NCW, SPW>;
    using P = Pay<DK>;
    constexpr int NPW = L::NPW, NKB = L::NKB, NMT = L::NMT, NVT = L::NVT, NVB = L::NVB, VPW = L::VPW;
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lq = lane >> 4;
    const int group = blockIdx.x % L::G;
    const int slot = blockIdx.x / L::G;
    const int col0 = group * L::NCOL;

    // ---- which (sequence, head): heads inner; packed sequences longest first
    const int rank = slot / a.H;
    int seq = rank;
    if (a.cu_seqlens && a.n_seq <= LPT_MAX) {
        int *sseq = reinterpret_cast<int *>(lds + L::O_SEQ);
        for (int s = tid; s < a.n_seq; s += L::NTHR) {
            const int ls = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
            int rk = 0;
            for (int s2 = 0; s2 < a.n_seq; ++s2) {
                const int l2 = a.cu_seqlens[s2 + 1] - a.cu_seqlens[s2];
                rk += (l2 > ls) || (l2 == ls && s2 < s);
            }
            if (rk == rank) *sseq = s;
        }
        lds_barrier();
        seq = __builtin_amdgcn_readfirstlane(*sseq);
    }
    const Chain c = chain_of(a, seq, slot % a.H, tid == 0);
    const size_t H = a.H;
    const size_t hbase = (((size_t)(c.hrow < 0 ? 0 : c.hrow) * H + c.head) * DV + col0) * DK;

    if (c.nch == 0) {   // empty sequence: h_T = h0 (or zeros), nothing else
        if (a.h_T && c.hrow >= 0)
            for (int i = tid; i < L::NCOL * DK; i += L::NTHR)
                a.h_T[hbase + i] = a.h0 ? a.h0[hbase + i] : 0.f;
        return;
    }

    if (wv > NPW) {
        // ======================================================= consumer
        const int cw = wv - NPW - 1;
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
        const size_t cbase = SNAP ? chunk_base(a, c.seq) : 0;
        for (int it = -3; it < c.nch; ++it) {
            if (it >= 0) {
                const int x = it;
                const unsigned char *pay = lds + L::O_PAY + (x & 3) * L::PAY;
                const unsigned char *ups = lds + L::O_UP + (x & 1) * L::UP;
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
                bf16x8 qf[NKB], wf[NKB];
                bf16x4 kr[NMT];
                f32x4 eg[NMT], up[SPW], O[SPW];
#pragma unroll
                for (int s = 0; s < NKB; ++s) {
                    wf[s] = *reinterpret_cast<const bf16x8 *>(pay + P::WF + (s * 64 + lane) * 16);
                    qf[s] = *reinterpret_cast<const bf16x8 *>(pay + P::QF + (s * 64 + lane) * 16);
                }
#pragma unroll
                for (int m = 0; m < NMT; ++m) {
                    eg[m] = *reinterpret_cast<const f32x4 *>(pay + P::EG + chan(m, lq, 0) * 4);
                    kr[m] = *reinterpret_cast<const bf16x4 *>(pay + P::KR + (m * 64 + lane) * 8);
                }
                const bf16x4 mq = *reinterpret_cast<const bf16x4 *>(pay + P::MQ + lane * 8);
#pragma unroll
                for (int j = 0; j < SPW; ++j)
                    up[j] = *reinterpret_cast<const f32x4 *>(ups + ((cw * SPW + j) * 64 + lane) * 16);
                rec_step<NKB, NMT, SPW>(S, qf, wf, kr, eg, mq, up, O);
                const int rem = min(CH, c.len - x * CH);
                if (ln < rem) {
#pragma unroll
                    for (int j = 0; j < SPW; ++j)
                        store_o(a.o, c.bos + (size_t)x * CH + ln, H, c.head, DV, col0 + 16 * (cw * SPW + j) + 4 * lq,
                                O[j], a.scale);
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
    auto part = [&](int x) { return reinterpret_cast<f32x4 *>(lds + L::O_PART + (x & 1) * L::PART); };
    auto beta = [&](int x) { return reinterpret_cast<float *>(lds + L::O_BETA + (x & 1) * 64); };
    auto pay = [&](int x) { return lds + L::O_PAY + (x & 3) * L::PAY; };
    auto kv = [&](int x) { return lds + L::O_KV + (x % 3) * L::KV; };
    if (wv == NPW) {
        // the INV wave: stage B1 of chunk it + 2 in iteration it
        for (int it = -3; it < c.nch; ++it) {
            const int x = it + 2;
            if (x >= 0 && x < c.nch) stage_b1<NPW>(part(x), beta(x), pay(x) + P::IB, pay(x) + P::MQ, lane);
            lds_barrier();
        }
        return;
    }
    Prep<DK, VPW> pr;
    pr.init(a, c.head, wv, lane);
    In<VPW> in0, in1;
    pr.load(in0, a, c.bos, c.len, 0, c.head, DV, col0, L::NCOL, NVB);
    // chunk x's inputs sit in in[x & 1], loaded one iteration before stage A uses them
    auto body = [&](int it, In<VPW> &use, In<VPW> &fill) {
        // the only loads in flight here are `use`'s, issued an iteration ago: wait
        // for them now, so that no later wait covers the loads issued next
        vm_wait_all();
        if (it + 4 < c.nch) pr.load(fill, a, c.bos, c.len, it + 4, c.head, DV, col0, L::NCOL, NVB);
        const int xa = it + 3;
        if (xa < c.nch) {
            unsigned char *p = pay(xa);
            pr.stage_a(use, min(CH, c.len - xa * CH), p + P::QF, reinterpret_cast<float *>(p + P::EG), p + P::KR,
                       kv(xa) + L::KT, kv(xa) + L::VT, NVB, NVT, part(xa), beta(xa));
        }
        const int xb = it + 1;
        if (wv > 0 && xb >= 0 && xb < c.nch) {
            // stage B2: w fragments into the chunk's operands, u' tiles
            const bf16x4 ib = *reinterpret_cast<const bf16x4 *>(pay(xb) + P::IB + lane * 8);
            const unsigned char *kvb = kv(xb);
            unsigned char *ups = lds + L::O_UP + (xb & 1) * L::UP;
            for (int job = wv - 1; job < NKB + NVT; job += NPW - 1) {
                if (job < NKB) {
                    *reinterpret_cast<bf16x8 *>(pay(xb) + P::WF + (job * 64 + lane) * 16) =
                        w_frag(kvb + L::KT, ib, job, lane);
                } else {
                    const int n = job - NKB;
                    const bf16x4 vt = *reinterpret_cast<const bf16x4 *>(kvb + L::VT + (n * 64 + lane) * 8);
                    *reinterpret_cast<f32x4 *>(ups + (n * 64 + lane) * 16) = mma16(ib, vt, Z4);
                }
            }
        }
        lds_barrier();
    };
    for (int it = -3; it < c.nch; it += 2) {
        body(it, in0, in1);
        if (it + 1 < c.nch) body(it + 1, in1, in0);
    }
}

// =========================================================== two passes
// Pass 1: one wave per (chunk row, head), independent of every other wave:
// stage A over the d_k / 32 channel blocks in turn (the partials of L, L^T,
// Mqk^T summed in registers), then B1 and B2, writing the chunk's consumer
// operands to its workspace row (chunk row) * H + head.  Chunk rows run over
// sequence 0's chunks, then sequence 1's, ...
constexpr int PREP_WAVES = 4;
#ifndef KDA_PREP_OCC
#define KDA_PREP_OCC
#endif

template <int DK>
__global__ __launch_bounds__(64 * PREP_WAVES) KDA_PREP_OCC void prep_kernel(FwdArgs a, unsigned char *ws, long long n_rows)
{
    constexpr int NPW = DK / 32, NMT = DK / 16, NKB = DK / 32;
    using P = Pay<DK>;
    __shared__ float l_beta[PREP_WAVES][CH];
    const int lane = threadIdx.x & 63, ln = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long item = (long long)blockIdx.x * PREP_WAVES + wv;
    const long long row = item / a.H;
    const int head = (int)(item - row * a.H);
    if (row >= n_rows) return;
    const RowPos p = row_pos(a, row);   // the host's row count is an upper bound for packed input
    if (p.seq >= a.n_seq) return;
    unsigned char *pw = ws + (size_t)(row * a.H + head) * P::BYTES;
    const int rem = min(CH, p.len - p.x * CH);
    f32x4 Lm = Z4, LT = Z4, MT = Z4;
    bf16x4 kt[NMT];
    float beta = 0.f;
#pragma unroll
    for (int w = 0; w < NPW; ++w) {
        Prep<DK, 0> pr;
        pr.init(a, head, w, lane);
        In<0> in;
        pr.load(in, a, p.bos, p.len, p.x, head, 0, 0, 0, 0);
        typename Prep<DK, 0>::Out o;
        pr.stage_a_core(in, rem, o);
        *reinterpret_cast<bf16x8 *>(pw + P::QF + (w * 64 + lane) * 16) = o.bqd;
        pr.store_eg(o, reinterpret_cast<float *>(pw + P::EG));
        Lm += o.pL;
        LT += o.pLT;
        MT += o.pMT;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            kt[2 * w + h] = pr.ctile(o.bkd, h);
            *reinterpret_cast<bf16x4 *>(pw + P::KR + ((2 * w + h) * 64 + lane) * 8) = pr.ctile(o.bkr, h);
        }
        if (w == 0) beta = ln < rem ? sigmoid_f(bf16_to_f32(in.b)) : 0.f;
    }
    // beta of tokens 4 lq .. +3 and of token ln, through this wave's LDS row
    if (lq == 0) l_beta[wv][ln] = beta;
    __builtin_amdgcn_wave_barrier();
    const f32x4 brow = *reinterpret_cast<const f32x4 *>(&l_beta[wv][4 * lq]);
    const float bcol = l_beta[wv][ln];
    bf16x4 ib, mq;
    b1_core(Lm, LT, MT, brow, bcol, lane, ib, mq);
    *reinterpret_cast<bf16x4 *>(pw + P::MQ + lane * 8) = mq;
    *reinterpret_cast<bf16x4 *>(pw + P::IB + lane * 8) = ib;
#pragma unroll
    for (int s2 = 0; s2 < NKB; ++s2)
        *reinterpret_cast<bf16x8 *>(pw + P::WF + (s2 * 64 + lane) * 16) = w_frag2(kt[2 * s2], kt[2 * s2 + 1], ib);
}

// Pass 2: one wave per (sequence, head, SPW slabs of 16 columns).  Workgroup
// b takes chain 8 (b / 8 / NSG) + b % 8 and slab group (b / 8) % NSG, so that
// the slab groups of a chain share blockIdx % 8 (the XCD, whose L2 then serves
// the chain's operands to all of them; placement only affects speed).
//
// A chunk's operands (its workspace row, padded to whole KiB, and the wave's
// 16 x 16 SPW bf16 tile of v) reach LDS by direct global-to-LDS loads, RING
// chunks ahead, so the recurrence never waits on memory latency.  The loads
// are issued from inline assembly: the compiler would otherwise wait for all
// of them before every LDS read.  Each is counted in this wave's vmcnt, which
// drains in issue order, so waiting until at most n loads remain outstanding,
// n = the loads issued after chunk x's, guarantees chunk x has landed.
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

template <int DK, int DV, int SPW, bool SNAP>
__global__ __launch_bounds__(64) void rec_kernel(FwdArgs a, const unsigned char *ws)
{
    constexpr int NKB = DK / 32, NMT = DK / 16, NSG = DV / (16 * SPW);
    using P = Pay<DK>;
    constexpr int NPAY = (P::BYTES + 1023) / 1024;   // 1 KiB loads of a workspace row
    constexpr int ND = NPAY + 1;                     // and one for the v tile
    constexpr int SLOT = ND * 1024, VT = NPAY * 1024;
    static_assert((RING - 1) * ND <= 63, "loads in flight exceed the vmcnt field");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[RING * SLOT];
    const int lane = threadIdx.x, ln = lane & 15, lq = lane >> 4;
    const int b8 = blockIdx.x / 8;
    const int chain = 8 * (b8 / NSG) + blockIdx.x % 8;
    const int sg = b8 % NSG;
    if (chain >= a.n_seq * a.H) return;
    const Chain c = chain_of(a, chain / a.H, chain % a.H, lane == 0 && sg == 0);
    const size_t H = a.H;
    const int col0 = sg * SPW * 16;
    const size_t hbase = (((size_t)(c.hrow < 0 ? 0 : c.hrow) * H + c.head) * DV + col0) * DK;
    f32x4 S[SPW][NMT];
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
        for (int m = 0; m < NMT; ++m)
            S[j][m] = (a.h0 && c.hrow >= 0)
                          ? *reinterpret_cast<const f32x4 *>(a.h0 + hbase + (size_t)(16 * j + ln) * DK + chan(m, lq, 0))
                          : Z4;
    const size_t cbase = chunk_base(a, c.seq);
    // identity as a K = 16 B operand: the product of a row-loaded 16 x 16 tile with it is its C layout
    bf16x4 eye;
#pragma unroll
    for (int e = 0; e < 4; ++e) eye[e] = static_cast<__bf16>(4 * lq + e == ln ? 1.f : 0.f);
    const unsigned ring_lds =
        __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) unsigned char *)ring);
    // v tile in LDS: token t at t * 32 SPW bytes, 8 columns per lane; for SPW = 1
    // lanes 32 .. 63 repeat lanes 0 .. 31 into the unused upper half.
    const int vt_tok = (lane & 63) / (2 * SPW) % 16, vt_col = 8 * ((lane & 63) % (2 * SPW));
    auto issue = [&](int x) {   // chunk x's loads into ring slot x % RING
        const unsigned slot = ring_lds + (unsigned)((x % RING) * SLOT);
        dma_bytes<P::BYTES>(ws + ((cbase + x) * H + c.head) * P::BYTES, slot, lane);
        const int rem = min(CH, c.len - x * CH);
        const uint16_t *v0 = static_cast<const uint16_t *>(a.v) + ((c.bos + (size_t)x * CH) * H + c.head) * DV + col0;
        dma_group<1>(v0, 0u, (unsigned)(((size_t)min(vt_tok, rem - 1) * H * DV + vt_col) * 2), slot + VT);
    };
    auto step = [&](int x) {
        const unsigned char *row = ring + (x % RING) * SLOT;
        if constexpr (SNAP) {
            const size_t at = (((cbase + x) * H + c.head) * DV + col0) * DK;
#pragma unroll
            for (int j = 0; j < SPW; ++j)
#pragma unroll
                for (int m = 0; m < NMT; ++m)
                    __builtin_nontemporal_store(S[j][m], reinterpret_cast<f32x4 *>(
                        a.h_chunks + at + (size_t)(16 * j + ln) * DK + chan(m, lq, 0)));
        }
        // operands from the ring slot, in the order the chunk consumes them:
        // v as lane (lq, ln) = token ln, columns 4 lq .. +3 of each 16-column slab
        bf16x4 vv[SPW];
#pragma unroll
        for (int j = 0; j < SPW; ++j)
            vv[j] = *reinterpret_cast<const bf16x4 *>(row + VT + ln * 32 * SPW + (16 * j + 4 * lq) * 2);
        const bf16x4 ib = *reinterpret_cast<const bf16x4 *>(row + P::IB + lane * 8);
        bf16x8 qf[NKB], wf[NKB];
        bf16x4 kr[NMT];
        f32x4 eg[NMT];
#pragma unroll
        for (int s = 0; s < NKB; ++s) wf[s] = *reinterpret_cast<const bf16x8 *>(row + P::WF + (s * 64 + lane) * 16);
#pragma unroll
        for (int s = 0; s < NKB; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(row + P::QF + (s * 64 + lane) * 16);
#pragma unroll
        for (int m = 0; m < NMT; ++m) eg[m] = *reinterpret_cast<const f32x4 *>(row + P::EG + chan(m, lq, 0) * 4);
        const bf16x4 mq = *reinterpret_cast<const bf16x4 *>(row + P::MQ + lane * 8);
#pragma unroll
        for (int m = 0; m < NMT; ++m) kr[m] = *reinterpret_cast<const bf16x4 *>(row + P::KR + (m * 64 + lane) * 8);
        f32x4 up[SPW], O[SPW];
#pragma unroll
        for (int j = 0; j < SPW; ++j)   // u' = INV beta v (v in C layout by an identity product)
            up[j] = mma16(ib, pack4(mma16(vv[j], eye, Z4)), Z4);
        rec_step<NKB, NMT, SPW>(S, qf, wf, kr, eg, mq, up, O);
        const int rem = min(CH, c.len - x * CH);
        if (ln < rem) {
#pragma unroll
            for (int j = 0; j < SPW; ++j)
                store_o(a.o, c.bos + (size_t)x * CH + ln, H, c.head, DV, col0 + 16 * j + 4 * lq, O[j], a.scale);
        }
    };
    for (int x = 0; x < min(RING - 1, c.nch); ++x) issue(x);
    for (int x = 0; x < c.nch; ++x) {
        // slot (x + RING - 1) % RING held chunk x - 1, whose LDS reads are done
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        if (x + RING - 1 < c.nch) issue(x + RING - 1);
        vm_wait_chunks<ND>(min(RING - 1, c.nch - 1 - x));   // chunks x + 1 .. x + RING - 1 may still fly
        step(x);
    }
    if (a.h_T && c.hrow >= 0) {
#pragma unroll
        for (int j = 0; j < SPW; ++j)
#pragma unroll
            for (int m = 0; m < NMT; ++m)
                *reinterpret_cast<f32x4 *>(a.h_T + hbase + (size_t)(16 * j + ln) * DK + chan(m, lq, 0)) = S[j][m];
    }
}

// =========================================================== backward
// The chunkwise backward ([LA-06] "06 · linear 路线（一）", chunkwise form: a
// reverse loop over chunks).  Per chunk, with dS' the gradient of the loss
// with respect to the state after the chunk and dO_s = scale dO, the forward
// S' = D S + k^r^T U, U = u' - w S, O = scale (q~ S + Mqk U) gives
//   dU = k^r dS' + Mqk^T dO_s,   dS = D dS' + q~^T dO_s - w^T dU,
// the mirror of the forward recurrence: one sequential MFMA chain per chunk
// that needs only state-independent operands (k^r, q~, w, e^{G_C}, Mqk) and
// dO.  bwd_prep_kernel forms those operands as the forward's prep does (the
// same stage A / B1 / B2 code), in the layouts the reverse chain consumes;
// bwd_rec_kernel walks the chunks in reverse and stores dS' for every chunk,
// from which the gradients of every input are formed chunk-parallel.

// Operands of one chunk for the reverse chain (a workspace row): byte offsets.
template <int DK>
struct BPay {
    static constexpr int NKB = DK / 32, NMT = DK / 16;
    static constexpr int KRA = 0;                   // k^r A fragments over channels [NKB][64] x 16 B
    static constexpr int QC = KRA + NKB * 1024;     // scale q~ C tiles (tokens x tile channels) [NMT][64] x 8 B
    static constexpr int WC = QC + NMT * 512;       // -w C tiles [NMT][64] x 8 B
    static constexpr int EG = WC + NMT * 512;       // e^{G_C} [DK] fp32
    static constexpr int MS = EG + DK * 4;          // scale Mqk C tile [64] x 8 B
    static constexpr int REC = MS + 512;            // (the reverse chain reads up to here)
    static constexpr int AT = REC;                  // A (strictly lower, no beta) C tile [64] x 16 B fp32
    static constexpr int BYTES = AT + 1024;
};

// One wave per (chunk row, head), as prep_kernel.
template <int DK>
__global__ __launch_bounds__(64 * PREP_WAVES) void bwd_prep_kernel(FwdArgs a, unsigned char *ws, long long n_rows)
{
    constexpr int NPW = DK / 32, NMT = DK / 16;
    using P = BPay<DK>;
    __shared__ float l_beta[PREP_WAVES][CH];
    const int lane = threadIdx.x & 63, ln = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long item = (long long)blockIdx.x * PREP_WAVES + wv;
    const long long row = item / a.H;
    const int head = (int)(item - row * a.H);
    if (row >= n_rows) return;
    const RowPos p = row_pos(a, row);
    if (p.seq >= a.n_seq) return;
    unsigned char *pw = ws + (size_t)(row * a.H + head) * P::BYTES;
    const int rem = min(CH, p.len - p.x * CH);
    f32x4 Lm = Z4, LT = Z4, MT = Z4;
    bf16x4 kt[NMT];
    float beta = 0.f;
#pragma unroll
    for (int w = 0; w < NPW; ++w) {
        Prep<DK, 0> pr;
        pr.init(a, head, w, lane);
        In<0> in;
        pr.load(in, a, p.bos, p.len, p.x, head, 0, 0, 0, 0);
        typename Prep<DK, 0>::Out o;
        pr.stage_a_core(in, rem, o);
        *reinterpret_cast<bf16x8 *>(pw + P::KRA + (w * 64 + lane) * 16) = o.bkr;
        pr.store_eg(o, reinterpret_cast<float *>(pw + P::EG));
        Lm += o.pL;
        LT += o.pLT;
        MT += o.pMT;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            kt[2 * w + h] = pr.ctile(o.bkd, h);
            *reinterpret_cast<bf16x4 *>(pw + P::QC + ((2 * w + h) * 64 + lane) * 8) =
                pack4(mma32(o.bqd, pr.sel_c[h], Z4) * a.scale);
        }
        if (w == 0) beta = ln < rem ? sigmoid_f(bf16_to_f32(in.b)) : 0.f;
    }
    if (lq == 0) l_beta[wv][ln] = beta;
    __builtin_amdgcn_wave_barrier();
    const f32x4 brow = *reinterpret_cast<const f32x4 *>(&l_beta[wv][4 * lq]);
    const float bcol = l_beta[wv][ln];
    {
        f32x4 At;
#pragma unroll
        for (int i = 0; i < 4; ++i) At[i] = 4 * lq + i > ln ? Lm[i] : 0.f;
        *reinterpret_cast<f32x4 *>(pw + P::AT + lane * 16) = At;
    }
    bf16x4 ib, mq;
    b1_core(Lm, LT, MT, brow, bcol, lane, ib, mq);
    // C(Mqk) from C(Mqk^T) by a product with the identity (exact), scaled
    bf16x4 eye;
#pragma unroll
    for (int e = 0; e < 4; ++e) eye[e] = static_cast<__bf16>(4 * lq + e == ln ? 1.f : 0.f);
    *reinterpret_cast<bf16x4 *>(pw + P::MS + lane * 8) = pack4(mma16(mq, eye, Z4) * a.scale);
    // C(-w_m) = C(-(INV beta) k~_m): the product of C((INV beta)^T), negated, with C(k~_m)
    bf16x4 nib;
#pragma unroll
    for (int e = 0; e < 4; ++e) nib[e] = -ib[e];
#pragma unroll
    for (int m = 0; m < NMT; ++m)
        *reinterpret_cast<bf16x4 *>(pw + P::WC + (m * 64 + lane) * 8) = pack4(mma16(nib, kt[m], Z4));
}

// Gradient rows the reverse chain leaves for the chunk-parallel pass, one per
// (chunk row, head): dS' as bf16 fragments (slab sg, channel block cb, lane
// (lq, ln): column 16 sg + ln, channels 32 cb + 8 lq .. +7) and dU in C layout
// (fp32; tokens x the slab's columns).  Byte offsets.
struct GRow {
    static constexpr int DM = 0;
    static constexpr int DU = 8 * 4 * 1024;
    static constexpr int BYTES = DU + 8 * 1024;
};

// The reverse chain: one single-wave workgroup per (chain, 16 state columns),
// chunks from last to first; dS' (fp32, in the forward state's registers and
// layout) starts from dh_T; for every chunk it leaves dS' and dU in a gradient
// row, and the gradient before the first chunk goes to dh0.  Operands reach a
// ring of LDS slots by direct global-to-LDS loads, RING - 1 chunks ahead,
// counted as in rec_kernel.
template <int DK, int DV>
__global__ __launch_bounds__(64) void bwd_rec_kernel(FwdArgs a, const unsigned char *ws, const float *dh_T,
                                                      const void *dO, unsigned char *grows, float *dh0)
{
    constexpr int NKB = DK / 32, NMT = DK / 16, NSG = DV / 16;
    static_assert(DK == 128 && DV == 128, "gradient rows are laid out for d = 128");
    using P = BPay<DK>;
    constexpr int NPAY = (P::REC + 1023) / 1024;
    constexpr int ND = NPAY + 1;                     // and one for the dO tile
    constexpr int SLOT = ND * 1024, DT = NPAY * 1024;
    static_assert((RING - 1) * ND <= 63, "loads in flight exceed the vmcnt field");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[RING * SLOT];
    const int lane = threadIdx.x, ln = lane & 15, lq = lane >> 4;
    const int b8 = blockIdx.x / 8;
    const int chain = 8 * (b8 / NSG) + blockIdx.x % 8;
    const int sg = b8 % NSG;
    if (chain >= a.n_seq * a.H) return;
    const Chain c = chain_of(a, chain / a.H, chain % a.H, false);
    const size_t H = a.H;
    const int col0 = sg * 16;
    const size_t hbase = (((size_t)c.seq * H + c.head) * DV + col0) * DK;
    f32x4 dS[NMT];
#pragma unroll
    for (int m = 0; m < NMT; ++m)
        dS[m] = dh_T ? *reinterpret_cast<const f32x4 *>(dh_T + hbase + (size_t)ln * DK + chan(m, lq, 0)) : Z4;
    const size_t cbase = chunk_base(a, c.seq);
    bf16x4 eye;
#pragma unroll
    for (int e = 0; e < 4; ++e) eye[e] = static_cast<__bf16>(4 * lq + e == ln ? 1.f : 0.f);
    const unsigned ring_lds =
        __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) unsigned char *)ring);
    const int vt_tok = (lane / 2) % 16, vt_col = 8 * (lane % 2);
    // the kk-th chunk walked is chunk nch - 1 - kk
    auto issue = [&](int kk) {
        const int x = c.nch - 1 - kk;
        const unsigned slot = ring_lds + (unsigned)((kk % RING) * SLOT);
        dma_bytes<P::REC>(ws + ((cbase + x) * H + c.head) * P::BYTES, slot, lane);
        const int rem = min(CH, c.len - x * CH);
        const uint16_t *d0 = static_cast<const uint16_t *>(dO) + ((c.bos + (size_t)x * CH) * H + c.head) * DV + col0;
        // dO rows past the sequence's end are zero gradients: the load re-reads
        // the last live row (in bounds) and the step zeroes it
        dma_group<1>(d0, 0u, (unsigned)(((size_t)min(vt_tok, rem - 1) * H * DV + vt_col) * 2), slot + DT);
    };
    auto step = [&](int kk) {
        const int x = c.nch - 1 - kk;
        const unsigned char *row = ring + (kk % RING) * SLOT;
        unsigned char *g = grows + ((cbase + x) * H + c.head) * (size_t)GRow::BYTES;
        // dS' of this chunk (the gradient with respect to the state after it)
#pragma unroll
        for (int cb = 0; cb < NKB; ++cb)
            __builtin_nontemporal_store(cat4(pack4(dS[2 * cb]), pack4(dS[2 * cb + 1])),
                                        reinterpret_cast<bf16x8 *>(g + GRow::DM + (sg * NKB + cb) * 1024 + lane * 16));
        const int rem = min(CH, c.len - x * CH);
        bf16x4 dOr = *reinterpret_cast<const bf16x4 *>(row + DT + ln * 32 + 8 * lq);
        if (ln >= rem) dOr = bf16x4{};
        const bf16x4 ms = *reinterpret_cast<const bf16x4 *>(row + P::MS + lane * 8);
        bf16x8 kra[NKB];
        bf16x4 wc[NMT], qc[NMT];
        f32x4 eg[NMT];
#pragma unroll
        for (int s2 = 0; s2 < NKB; ++s2) kra[s2] = *reinterpret_cast<const bf16x8 *>(row + P::KRA + (s2 * 64 + lane) * 16);
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            eg[m] = *reinterpret_cast<const f32x4 *>(row + P::EG + chan(m, lq, 0) * 4);
            wc[m] = *reinterpret_cast<const bf16x4 *>(row + P::WC + (m * 64 + lane) * 8);
            qc[m] = *reinterpret_cast<const bf16x4 *>(row + P::QC + (m * 64 + lane) * 8);
        }
        // dU = k^r dS' + Mqk^T dO_s  (C layout: tokens x the slab's columns)
        f32x4 dU = Z4, dU2 = Z4;
#pragma unroll
        for (int s2 = 0; s2 < NKB / 2; ++s2) {
            dU = mma32(kra[s2], cat4(pack4(dS[2 * s2]), pack4(dS[2 * s2 + 1])), dU);
            dU2 = mma32(kra[s2 + NKB / 2], cat4(pack4(dS[2 * s2 + NKB]), pack4(dS[2 * s2 + NKB + 1])), dU2);
        }
        const bf16x4 bdO = pack4(mma16(dOr, eye, Z4));              // C layout of dO (exact)
        dU = mma16(ms, bdO, dU + dU2);
        __builtin_nontemporal_store(dU, reinterpret_cast<f32x4 *>(g + GRow::DU + sg * 1024 + lane * 16));
        const bf16x8 bdU = hilo(dU);
        // dS = D dS' - w^T dU + q~^T dO_s
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            dS[m] *= eg[m];
            dS[m] = mma32(cat4(wc[m], wc[m]), bdU, dS[m]);
            dS[m] = mma16(qc[m], bdO, dS[m]);
        }
    };
    for (int kk = 0; kk < min(RING - 1, c.nch); ++kk) issue(kk);
    for (int kk = 0; kk < c.nch; ++kk) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the reused slot's reads are done
        if (kk + RING - 1 < c.nch) issue(kk + RING - 1);
        vm_wait_chunks<ND>(min(RING - 1, c.nch - 1 - kk));
        step(kk);
    }
    if (dh0) {
#pragma unroll
        for (int m = 0; m < NMT; ++m)
            *reinterpret_cast<f32x4 *>(dh0 + hbase + (size_t)ln * DK + chan(m, lq, 0)) = dS[m];
    }
}

// fp32 16x16 products on the matrix core (v_mfma_f32_16x16x4_f32, four K
// steps): X Y in C layout from XT = C layout of X^T and Y in C layout.
__device__ __forceinline__ f32x4 fprod(f32x4 XT, f32x4 Y) {
    f32x4 acc = Z4;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(XT[r], Y[r], acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ float rscan16(float x) {   // inclusive suffix sum over a 16-lane row
    x += dpp_f<0x101>(x);
    x += dpp_f<0x102>(x);
    x += dpp_f<0x104>(x);
    x += dpp_f<0x108>(x);
    return x;
}
__device__ __forceinline__ bf16x4 half4(bf16x8 x, int h) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = x[4 * h + i];
    return r;
}
__device__ __forceinline__ f32x4 unpack4(bf16x4 x) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = static_cast<float>(x[i]);
    return r;
}

// Element e of 8 packed bf16 words, as a float.
__device__ __forceinline__ float bf16_word(uint4 v, int e) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    return bf16_to_f32((uint16_t)(w[e >> 1] >> (16 * (e & 1))));
}
// The gate in log2 units, -A log2(1 + 2^{z log2 e}) (softplus taken as z above
// z = 20), zero on a token past the chunk's end.
__device__ __forceinline__ float gate2(float z, float A, bool live) {
    const float y = z * kLog2e;
    const float sp2 = y > 20.f * kLog2e ? y : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(y));
    return live ? -A * sp2 : 0.f;
}

// x = hi + lo with hi = RNE(x), lo = RNE(x - hi), both bf16 (~2^-16 relative).
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        __bf16 h, l;
        split_bf16(x[e], h, l);
        hi[e] = h;
        lo[e] = l;
    }
}

struct BwdOut {
    void *dq, *dk, *dv, *dg, *db;
    float *part;    // [chunk row][H][DK + 1]: the chunk's sums of d dt_bias (DK channels) and d A_log
};

// The chunk-parallel gradients: one 256-thread workgroup per (chunk row,
// head), from the state entering the chunk (S, the forward's stored state),
// the chunk's reverse-chain operands (A), its gradient row (dS', dU) and dO.
// With S as d_k x d_v, y = beta (v - k~ S), U = T y (T = (I + beta A)^{-1}),
// O = scale (q~ S + Mqk U) and S' = D S + k^r^T U:
//   dy = T^T dU,  dv = beta dy,  dbeta = sum_v dy (v - k~ S) + sum_j dB_ij A_ij,
//   dB = -dy U^T (strictly lower; B = beta A),  dMqk = dO_s U^T (lower),
//   dq~ = dO_s S^T,  dk~ = -(beta dy) S^T,  dk^r = U dS'^T,  dD = sum_v S o dS',
// then the pair terms of A and Mqk, the gate chain (G -> g -> g_raw, A_log,
// dt_bias) and the chunk's parameter sums.  The pair terms, with P = beta dB
// and Q = dMqk,
//   R^P_i = sum_{j<i} P_ij k_j E_ij,  R^M_i = sum_{j<=i} Q_ij k_j E_ij,
//   C_j = sum_{i>j} P_ij k_i E_ij + sum_{i>=j} Q_ij q_i E_ij,   E_ijc = e^{G_ic - G_jc},
// are 16 x 16 MFMA products in the factored form (rows e^{G - r}, columns
// e^{r - G}) around a reference r per channel: one for the chunk where its
// decay spans at most 2^200, else one per block of 8 tokens (the pair
// section below states the bounds).
//
// Wave w owns channels 32 w .. +31: lane (lq, ln) holds token ln and channels
// 32 w + 8 lq .. +7 for all elementwise work, which is also the row fragment
// of a 16x16x32 product over those channels and the C layout of the
// transposed products (d_k x tokens), so no result changes lanes.
template <int DK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_chunk_kernel(FwdArgs a, const float *Sst, const unsigned char *pays,
                                                         const unsigned char *grows, const void *dO, BwdOut out)
{
    static_assert(DK == 128 && DV == 128, "d = 128");
    constexpr int NVT = DV / 16;
    using P = BPay<DK>;
    __shared__ float LA[CH][CH + 1], PP[CH][CH + 1], QQ[CH][CH + 1];
    __shared__ float bs[CH], dbp[4][CH], red[4];
    __shared__ __attribute__((aligned(16))) float RF[4][2][32];   // per wave: block references of its channels
    // one region, two lives (a barrier between): the per-wave partials of W,
    // then U^T, (beta dy)^T and the per-wave 16 x 16 partials
    __shared__ __attribute__((aligned(16))) unsigned char big[4 * NVT * 64 * 16];
    auto Wp = reinterpret_cast<f32x4 (*)[NVT][64]>(big);
    auto UT = reinterpret_cast<bf16x4 (*)[64]>(big);
    auto BD = reinterpret_cast<bf16x4 (*)[64]>(big + NVT * 64 * 8);
    auto SmP = reinterpret_cast<f32x4 (*)[2][64]>(big + 2 * NVT * 64 * 8);
    static_assert(2 * NVT * 64 * 8 + 4 * 2 * 64 * 16 <= sizeof(big), "LDS");

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, lq = lane >> 4;
    const long long row = blockIdx.x / a.H;
    const int head = (int)(blockIdx.x - row * a.H);
    const size_t H = a.H;
    float *pp = out.part + ((size_t)row * H + head) * (DK + 1);
    const RowPos p = row_pos(a, row);
    if (p.seq >= a.n_seq) {   // a row past the sequences' chunks: zero parameter sums
        if (tid <= DK) pp[tid] = 0.f;
        return;
    }
    const int nt = min(CH, p.len - p.x * CH);
    const size_t tok0 = p.bos + (size_t)p.x * CH;
    const int t = ln, c0 = 32 * w + 8 * lq;
    const bool live = t < nt;
    const size_t trow = tok0 + min(t, nt - 1);     // rows past the end re-read the last live row (masked)
    const size_t ti = (trow * H + head) * DK + c0;
    const uint4 kw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + ti);
    const uint4 qw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + ti);
    const uint4 aw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.g_raw) + ti);
    const uint16_t braw = tid < CH ? static_cast<const uint16_t *>(a.beta_raw)[(tok0 + min(tid, nt - 1)) * H + head]
                                   : (uint16_t)0;
    const unsigned char *py = pays + ((size_t)row * H + head) * (size_t)P::BYTES;
    const f32x4 At = *reinterpret_cast<const f32x4 *>(py + P::AT + lane * 16);   // C(A)
    // dO and v rows: token ln, columns 16 vt + 4 lq .. +3 (zero past the chunk's end)
    const size_t to = (trow * H + head) * DV + 4 * lq;
    auto row4 = [&](const void *base, int vt) {
        const bf16x4 x = *reinterpret_cast<const bf16x4 *>(static_cast<const uint16_t *>(base) + to + 16 * vt);
        return live ? x : bf16x4{};
    };
    const unsigned char *gr = grows + ((size_t)row * H + head) * (size_t)GRow::BYTES;
    // every HBM read of the workgroup is issued here, ahead of the gate: S
    // (column 16 vt + ln, channels c0 .. +7), this wave's two column tiles of
    // v, dO and dU
    const float *S0 = Sst + ((size_t)row * H + head) * (size_t)DV * DK;
    f32x4 sf[NVT][2];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
        const float *ps = S0 + (size_t)(16 * vt + ln) * DK + c0;
        sf[vt][0] = *reinterpret_cast<const f32x4 *>(ps);
        sf[vt][1] = *reinterpret_cast<const f32x4 *>(ps + 4);
    }
    bf16x4 vr[2], dOv[2];
    f32x4 dUt[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int vt = 2 * w + u;
        vr[u] = row4(a.v, vt);
        dOv[u] = row4(dO, vt);
        dUt[u] = *reinterpret_cast<const f32x4 *>(gr + GRow::DU + vt * 1024 + lane * 16);
    }

    // ---- gate (log2 units) and its chunk-local cumulative sum G; k and q stay
    // packed (bf16 words, zero past the chunk's end) and are unpacked where used
    const float A = expf(a.A_log[head]);
    const uint4 kl = live ? kw : uint4{0u, 0u, 0u, 0u}, ql = live ? qw : uint4{0u, 0u, 0u, 0u};
    auto kf = [&](int e) { return bf16_word(kl, e); };
    auto qf = [&](int e) { return bf16_word(ql, e); };
    float z[8], G2[8];
    bool deep = false;
    {
        const uint32_t aa[4] = {aw.x, aw.y, aw.z, aw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sh = 16 * (e & 1);
            z[e] = bf16_to_f32((uint16_t)(aa[e >> 1] >> sh)) + a.dt_bias[(size_t)head * DK + c0 + e];
            G2[e] = scan16(gate2(z[e], A, live));
            deep |= row_bcast<0>(G2[e]) - row_bcast<15>(G2[e]) > 200.f;
        }
        deep = __ballot(deep) != 0;   // wave-uniform: a single reference would leave the fp32 range
    }
    if (tid < CH) bs[tid] = tid < nt ? sigmoid_f(bf16_to_f32(braw)) : 0.f;
    if (w == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) LA[4 * lq + r][ln] = At[r];
    }
    __syncthreads();
    // S kept as bf16
    bf16x8 sb[NVT];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) sb[vt] = cat4(pack4(sf[vt][0]), pack4(sf[vt][1]));

    // ---- T = (I + beta A)^{-1} = (I + L)(I + L^2)(I + L^4)(I + L^8), L = -beta A,
    // on the fp32 matrix core in C layout (every wave on its own)
    f32x4 eyef, brow;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        eyef[r] = 4 * lq + r == ln ? 1.f : 0.f;
        brow[r] = bs[4 * lq + r];
    }
    const float bcol = bs[ln];
    f32x4 IT, CT;
    {
        const f32x4 L = -(brow * At);
        const f32x4 LT = fprod(L, eyef);          // C(L^T)
        const f32x4 L2 = fprod(LT, L), L2T = fprod(L, LT);
        const f32x4 L4 = fprod(L2T, L2), L4T = fprod(L2, L2T);
        const f32x4 L8 = fprod(L4T, L4);
        const f32x4 P1T = fprod(plus_eye(L2, ln, lq), plus_eye(LT, ln, lq));
        const f32x4 P2 = fprod(plus_eye(L4T, ln, lq), plus_eye(L8, ln, lq));
        IT = fprod(P2, P1T);      // C(T^T)
        CT = fprod(IT, eyef);     // C(T)
    }
    bf16x4 eye16;
#pragma unroll
    for (int e = 0; e < 4; ++e) eye16[e] = static_cast<__bf16>(eyef[e]);

    // ---- W = k~ S over this wave's channels (partial)
    {
        float kt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kt[e] = kf(e) * __builtin_amdgcn_exp2f(G2[e]);
        const bf16x8 ktb = pack8(kt);
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) Wp[w][vt][lane] = mma32(ktb, sb[vt], Z4);
    }
    __syncthreads();

    // dS' fragments (same lanes and channels as S), wanted from phase 5 on
    bf16x8 dm[NVT];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
        dm[vt] = *reinterpret_cast<const bf16x8 *>(gr + GRow::DM + (vt * 4 + w) * 1024 + lane * 16);
    // ---- per column tile of this wave: r = v - W, y = beta r, U^T, dy, dy^T;
    // dv; partials of dbeta, dMqk = dO_s U^T and dy U^T
    {
        f32x4 dMq = Z4, dBp = Z4, dbl = Z4, W[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int vt = 2 * w + u;
            W[u] = ((Wp[0][vt][lane] + Wp[1][vt][lane]) + Wp[2][vt][lane]) + Wp[3][vt][lane];
        }
        __syncthreads();   // the region's next life
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int vt = 2 * w + u;
            const f32x4 r = mma16(vr[u], eye16, Z4) - W[u];
            const f32x4 y = brow * r;
            const f32x4 CUT = fprod(y, IT);             // C(U^T) = C(y^T T^T)
            const f32x4 Cdy = fprod(CT, dUt[u]);        // C(T^T dU)
            const f32x4 CdyT = fprod(dUt[u], CT);       // C(dU^T T)
            dbl += Cdy * r;
            const f32x4 dOsT = unpack4(dOv[u]) * a.scale;    // C(dO_s^T)
            dMq = dMq + fprod(dOsT, CUT);
            dBp = dBp + fprod(CdyT, CUT);
            const f32x4 bdyT = CdyT * bcol;              // C((beta dy)^T): token ln, columns 16 vt + 4 lq ..
            if (live) {
                uint2 pk;
                pk.x = pack_bf16x2(bdyT[0], bdyT[1]);
                pk.y = pack_bf16x2(bdyT[2], bdyT[3]);
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out.dv) + to + 16 * vt) = pk;
            }
            UT[vt][lane] = pack4(CUT);
            BD[vt][lane] = pack4(bdyT);
        }
        SmP[w][0][lane] = dMq;
        SmP[w][1][lane] = dBp;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float s = row16_sum(dbl[r]);
            if (ln == 0) dbp[w][4 * lq + r] = s;
        }
    }
    __syncthreads();
    // ---- Q = dMqk (lower), P = beta dB (strictly lower), dbeta, dbeta_raw
    {
        const int i = tid >> 4, j = tid & 15;
        const int src = 16 * (i >> 2) + j, comp = i & 3;
        float q = 0.f, db = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            q += SmP[ww][0][src][comp];
            db += SmP[ww][1][src][comp];
        }
        db = -db;                                  // dB = -dy U^T
        QQ[i][j] = i >= j ? q : 0.f;
        PP[i][j] = i > j ? bs[i] * db : 0.f;
        const float s = row16_sum(i > j ? db * LA[i][j] : 0.f);
        if (j == 0 && i < nt) {
            const float dbeta = ((dbp[0][i] + dbp[1][i]) + (dbp[2][i] + dbp[3][i])) + s;
            const float be = bs[i];
            static_cast<uint16_t *>(out.db)[(tok0 + i) * H + head] = f32_to_bf16(dbeta * be * (1.f - be));
        }
    }
    __syncthreads();

    // ---- dq~^T, dk~^T, dk^r^T (channels x tokens) over d_v on the matrix core:
    // S and dS' tiles transposed by products with the identity (exact); and
    // S^T dS' per 16-channel tile, whose diagonal is dD = sum_v S o dS'
    f32x4 aq[2] = {Z4, Z4}, ak[2] = {Z4, Z4}, ar[2] = {Z4, Z4}, dd[2] = {Z4, Z4};
#pragma unroll
    for (int u2 = 0; u2 < NVT / 2; ++u2) {
        const int v0 = 2 * u2, v1 = 2 * u2 + 1;
        const bf16x8 bo = cat4(row4(dO, v0), row4(dO, v1));
        const bf16x8 bb = cat4(BD[v0][lane], BD[v1][lane]);
        const bf16x8 bu = cat4(UT[v0][lane], UT[v1][lane]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8 as = cat4(pack4(mma16(half4(sb[v0], h), eye16, Z4)), pack4(mma16(half4(sb[v1], h), eye16, Z4)));
            const bf16x8 ad = cat4(pack4(mma16(half4(dm[v0], h), eye16, Z4)), pack4(mma16(half4(dm[v1], h), eye16, Z4)));
            aq[h] = mma32(as, bo, aq[h]);
            ak[h] = mma32(as, bb, ak[h]);
            ar[h] = mma32(ad, bu, ar[h]);
            dd[h] = mma32(as, ad, dd[h]);
        }
    }
    // dD of channel c0 + 4 h + i: the diagonal entry, held by lane (lq, 4 lq + i)
    float dD[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) dD[4 * h + i] = __shfl(dd[h][i], 20 * lq + i);

    // ---- dq, dk and dG (natural-log units) from the state path, with the
    // chunk decay's share of dG at the last token; the pair terms add to them
    float dq[8], dk[8], dG[8];
    const float qii = QQ[t][t];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float GC2 = row_bcast<15>(G2[e]);
        const float eg = __builtin_amdgcn_exp2f(G2[e]), er = __builtin_amdgcn_exp2f(GC2 - G2[e]);
        const float dqt = a.scale * aq[e >> 2][e & 3];
        const float dkt = -ak[e >> 2][e & 3];
        const float dkr = ar[e >> 2][e & 3];
        const float kv = kf(e), qv = qf(e), krv = kv * er;
        dq[e] = __builtin_fmaf(dqt, eg, qii * kv);        // with Q's diagonal term
        dk[e] = __builtin_fmaf(dkt, eg, __builtin_fmaf(dkr, er, qii * qv));
        dG[e] = (dqt * qv + dkt * kv) * eg - dkr * krv;
        const float gc = row16_sum(dkr * krv) + dD[e] * __builtin_amdgcn_exp2f(GC2);
        if (t == CH - 1) dG[e] += gc;
    }

    // ---- pair terms: RP, RM, CC as above and pG, their share of dG,
    // k (R^P - C^P) + q R^M - k C^M.  E_ij = 2^{l_i - r} 2^{r - l_j} is split
    // at a reference r into a row and a column factor, so the sums are 16 x 16
    // products over tokens (transposed: they land in this lane's token and
    // channels).  Where no channel of the wave decays by more than 2^-200 in
    // the chunk, l = G and r is the midpoint of G over the chunk: every factor
    // within 2^100, exact.  Otherwise l is the cumulative decay with each
    // token's decay clipped at 2^-27 and the tokens form two blocks of 8,
    // block b with r_b the midpoint of l over the block: rows of block b and
    // columns up to its end take r_b, every factor within 2^95 (a column of an
    // earlier block has a factor <= 1).  A pair whose true decay gap exceeds
    // 2^-27 is then taken as at most 2^-27 instead of its smaller true value.
    // Factors, P and Q enter the products as hi + lo bf16 pairs (to ~2^-16).
    // Every pair adds +X to one token's dG and -X to another's, which cancel
    // in the cumulative sum over the chunk, so pG takes both sides from the
    // same factors.  Q's diagonal (whose dG terms cancel exactly) stays out of
    // the products and is added to dq and dk exactly.
    {
        const int bt = deep ? t / 8 : 0;   // this token's block
        // block references of this lane's channels (every lane of the row
        // computes and stores the same values), through LDS so that the block
        // loop need not be unrolled
        float gl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gl[e] = deep ? scan16(fmaxf(gate2(z[e], A, live), -27.f)) : G2[e];
            const float l0 = row_bcast<0>(gl[e]), l15 = row_bcast<15>(gl[e]);
            RF[w][0][8 * lq + e] = deep ? 0.5f * (l0 + row_bcast<7>(gl[e])) : 0.5f * (l0 + l15);
            RF[w][1][8 * lq + e] = 0.5f * (row_bcast<8>(gl[e]) + l15);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
        // C(P), C(P^T), C(Q), C(Q^T) (Q without its diagonal) as hi + lo bf16
        bf16x4 cPh, cPl, cPTh, cPTl, cQh, cQl, cQTh, cQTl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool dg = 4 * lq + r == ln;
            __bf16 h, l;
            split_bf16(PP[4 * lq + r][ln], h, l);
            cPh[r] = h;
            cPl[r] = l;
            split_bf16(PP[ln][4 * lq + r], h, l);
            cPTh[r] = h;
            cPTl[r] = l;
            split_bf16(dg ? 0.f : QQ[4 * lq + r][ln], h, l);
            cQh[r] = h;
            cQl[r] = l;
            split_bf16(dg ? 0.f : QQ[ln][4 * lq + r], h, l);
            cQTh[r] = h;
            cQTl[r] = l;
        }
        const bf16x8 bPT = cat4(cPTh, cPTh), bQT = cat4(cQTh, cQTh), bP = cat4(cPh, cPh), bQ = cat4(cQh, cQh);
        // selector: C tile h of a row fragment (rows: tokens; columns: channels
        // c0 + 4 h + i as 4 lq + i of the transposed products)
        bf16x8 sel[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sel[h][e] = static_cast<__bf16>((lq == (ln >> 2) && e == 4 * h + (ln & 3)) ? 1.f : 0.f);
        const int nb = deep ? 2 : 1;
#pragma unroll 1
        for (int bb = 0; bb < nb; ++bb) {
            const bool col = !deep || t < 8 * (bb + 1);   // a column of block bb's products
            const f32x4 ra = *reinterpret_cast<const f32x4 *>(&RF[w][bb][8 * lq]);
            const f32x4 rb = *reinterpret_cast<const f32x4 *>(&RF[w][bb][8 * lq + 4]);
            const float ref[8] = {ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]};
            // row factor f (used where this token is in block bb, whose
            // reference is then its own) and column factor cs
            const bool own = bt == bb;
            float rw[8], qw8[8], cl[8], cs[8], f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                f[e] = __builtin_amdgcn_exp2f(gl[e] - ref[e]);
                rw[e] = own ? kf(e) * f[e] : 0.f;
                qw8[e] = own ? qf(e) * f[e] : 0.f;
                cs[e] = col ? __builtin_amdgcn_exp2f(ref[e] - gl[e]) : 0.f;
                cl[e] = kf(e) * cs[e];
            }
            bf16x8 rwh, rwl, qwh, qwl, clh, cll;
            split8(rw, rwh, rwl);
            split8(qw8, qwh, qwl);
            split8(cl, clh, cll);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // C tiles of the factors, hi and lo (exact selector copies); each
                // product is hi hi + lo hi + hi lo: one K = 32 and one K = 16 MFMA
                const bf16x4 ccH = pack4(mma32(clh, sel[h], Z4)), ccL = pack4(mma32(cll, sel[h], Z4));
                const bf16x4 crH = pack4(mma32(rwh, sel[h], Z4)), crL = pack4(mma32(rwl, sel[h], Z4));
                const bf16x4 cqH = pack4(mma32(qwh, sel[h], Z4)), cqL = pack4(mma32(qwl, sel[h], Z4));
                const bf16x8 cc2 = cat4(ccH, ccL), cr2 = cat4(crH, crL), cq2 = cat4(cqH, cqL);
                const f32x4 pk = mma16(ccH, cPTl, mma32(cc2, bPT, Z4));          // (P cl)^T
                const f32x4 qk = mma16(ccH, cQTl, mma32(cc2, bQT, Z4));          // (Q cl)^T
                const f32x4 ck = mma16(cqH, cQl, mma32(cq2, bQ, mma16(crH, cPl, mma32(cr2, bP, Z4))));   // (P^T rw + Q^T qw)^T
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = 4 * h + i;
                    // R^P, R^M: this token's own block only; C: every block
                    dq[e] = own ? __builtin_fmaf(f[e], qk[i], dq[e]) : dq[e];
                    dk[e] = __builtin_fmaf(cs[e], ck[i], own ? __builtin_fmaf(f[e], pk[i], dk[e]) : dk[e]);
                    dG[e] += rw[e] * pk[i] + qw8[e] * qk[i] - cl[e] * ck[i];   // rw, qw are 0 off block bb
                }
            }
        }
    }

    // ---- reverse cumulative sum dG -> dg, then g_raw, dt_bias, A_log
    float dgr[8], sA = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float dg = rscan16(dG[e]);
        const float dz = live ? -A * sigmoid_f(z[e]) * dg : 0.f;
        dgr[e] = dz;
        sA = __builtin_fmaf(dg, gate2(z[e], A, live) * 0.6931471805599453f, sA);   // g in natural-log units (0 on pads)
        const float sdt = row16_sum(dz);
        if (t == 0) pp[c0 + e] = sdt;
    }
    if (live) {
        uint4 vq, vk, vg;
        vq.x = pack_bf16x2(dq[0], dq[1]); vq.y = pack_bf16x2(dq[2], dq[3]);
        vq.z = pack_bf16x2(dq[4], dq[5]); vq.w = pack_bf16x2(dq[6], dq[7]);
        vk.x = pack_bf16x2(dk[0], dk[1]); vk.y = pack_bf16x2(dk[2], dk[3]);
        vk.z = pack_bf16x2(dk[4], dk[5]); vk.w = pack_bf16x2(dk[6], dk[7]);
        vg.x = pack_bf16x2(dgr[0], dgr[1]); vg.y = pack_bf16x2(dgr[2], dgr[3]);
        vg.z = pack_bf16x2(dgr[4], dgr[5]); vg.w = pack_bf16x2(dgr[6], dgr[7]);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out.dq) + ti) = vq;
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out.dk) + ti) = vk;
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out.dg) + ti) = vg;
    }
    sA = row16_sum(sA);
    sA += __shfl_xor(sA, 16);
    sA += __shfl_xor(sA, 32);
    if (lane == 0) red[w] = sA;
    __syncthreads();
    if (tid == 0) pp[DK] = (red[0] + red[1]) + (red[2] + red[3]);
}

#ifndef KDA_REC_SPW
#define KDA_REC_SPW 1
#endif

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

// One pass: column groups per chain, the fewest that give at least one
// workgroup per compute unit (the prep is repeated in every group of a chain).
template <int DK, int DV, bool SNAP>
hipError_t launch_one_pass(const FwdArgs &a, int n_cu, hipStream_t stream)
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

template <int DK, int DV, bool SNAP>
hipError_t launch_two_pass(const FwdArgs &a, unsigned char *ws, long long n_rows, hipStream_t stream)
{
    const long long wgs1 = (n_rows * a.H + PREP_WAVES - 1) / PREP_WAVES;
    if (wgs1 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (wgs1 > 0) {
        hipLaunchKernelGGL((prep_kernel<DK>), dim3((unsigned)wgs1), dim3(64 * PREP_WAVES), 0, stream, a, ws, n_rows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int SPW = KDA_REC_SPW, NSG = DV / (16 * SPW);
    const long long chains = (long long)a.n_seq * a.H;
    const long long wgs2 = 8 * NSG * ((chains + 7) / 8);
    if (wgs2 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rec_kernel<DK, DV, SPW, SNAP>), dim3((unsigned)wgs2), dim3(64), 0, stream, a,
                       (const unsigned char *)ws);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const FwdArgs &a, int n_cu, void *ws, size_t ws_bytes, long long n_rows, hipStream_t stream)
{
    const long long chains = (long long)a.n_seq * a.H;
    const bool two = ws && chains < n_cu && ws_bytes >= fwd_workspace_bytes(DK, n_rows, a.H);
    if (two)
        return a.h_chunks ? launch_two_pass<DK, DV, true>(a, static_cast<unsigned char *>(ws), n_rows, stream)
                          : launch_two_pass<DK, DV, false>(a, static_cast<unsigned char *>(ws), n_rows, stream);
    return a.h_chunks ? launch_one_pass<DK, DV, true>(a, n_cu, stream) : launch_one_pass<DK, DV, false>(a, n_cu, stream);
}

}  // namespace

size_t fwd_workspace_bytes(int dk, long long n_rows, int H)
{
    const size_t per = dk == 128 ? (size_t)Pay<128>::BYTES : (size_t)Pay<64>::BYTES;
    return per * (size_t)(n_rows < 0 ? 0 : n_rows) * (size_t)(H < 0 ? 0 : H);
}

hipError_t fwd_two_pass_eligible(long long chains, bool *two)
{
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    *two = chains < n_cu;
    return hipSuccess;
}

hipError_t launch_fwd_bf16(const FwdArgs &a, int dk, int dv, void *ws, size_t ws_bytes, long long n_rows,
                           hipStream_t stream)
{
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
#define KDA_FWD(DKV, DVV) \
    if (dk == DKV && dv == DVV) return launch_dims<DKV, DVV>(a, n_cu, ws, ws_bytes, n_rows, stream);
    KDA_FWD(128, 128)
    KDA_FWD(128, 64)
    KDA_FWD(64, 128)
    KDA_FWD(64, 64)
#undef KDA_FWD
    return hipErrorInvalidValue;
}


BwdWs bwd_ws_layout(long long n_rows, int H)
{
    BwdWs l;
    const size_t items = (size_t)n_rows * (size_t)H;
    l.pay = 0;
    l.grow = l.pay + ((items * BPay<128>::BYTES + 255) & ~(size_t)255);
    l.part = l.grow + items * (size_t)GRow::BYTES;
    l.red = l.part + items * (128 + 1) * sizeof(float);
    l.bytes = l.red + (size_t)H * BWD_SPLIT * (128 + 1) * sizeof(float);
    return l;
}

hipError_t launch_bwd_chunkwise(const BwdArgs &b, long long n_rows, hipStream_t stream)
{
    FwdArgs a{};
    a.q = b.q; a.k = b.k; a.v = b.v; a.g_raw = b.g_raw; a.beta_raw = b.beta_raw;
    a.A_log = b.A_log; a.dt_bias = b.dt_bias; a.cu_seqlens = b.cu_seqlens;
    a.T = b.T; a.H = b.H; a.n_seq = b.n_seq; a.scale = b.scale;
    const BwdWs l = bwd_ws_layout(n_rows, b.H);
    unsigned char *ws = static_cast<unsigned char *>(b.work);
    const long long items = n_rows * b.H;
    if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (items > 0) {
        hipLaunchKernelGGL((bwd_prep_kernel<128>), dim3((unsigned)((items + PREP_WAVES - 1) / PREP_WAVES)),
                           dim3(64 * PREP_WAVES), 0, stream, a, ws + l.pay, n_rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long long chains = (long long)b.n_seq * b.H;
    const long long wgs = 8 * 8 * ((chains + 7) / 8);
    if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (wgs > 0) {
        hipLaunchKernelGGL((bwd_rec_kernel<128, 128>), dim3((unsigned)wgs), dim3(64), 0, stream, a, ws + l.pay,
                           b.dh_T, b.do_, ws + l.grow, b.dh0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (items > 0) {
        BwdOut o;
        o.dq = b.dq; o.dk = b.dk; o.dv = b.dv; o.dg = b.dg_raw; o.db = b.dbeta_raw;
        o.part = reinterpret_cast<float *>(ws + l.part);
        hipLaunchKernelGGL((bwd_chunk_kernel<128, 128>), dim3((unsigned)items), dim3(256), 0, stream, a, b.h_chunks,
                           ws + l.pay, ws + l.grow, b.do_, o);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace kda
