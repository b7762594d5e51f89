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
// The per-chunk algebra, the prep stages, the operand layouts and the
// overflow-safe L / Mqk are those of kda_chunk.hpp.
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
//     wave per (sequence, head, 16 columns) walks the chunks, its operands
//     arriving RING - 1 chunks ahead in an LDS ring (issued by a loader wave
//     that serves one or two such waves), forming u' = INV beta v from its own
//     columns of v and running the recurrence.
//     No workgroup waits on another in either pass.
#include <stdint.h>

#include "kda_chunk.hpp"

namespace kda {


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
        // wave priority 1 here and in the stage-A waves, the B1 wave keeps 0: B1
        // has slack in every iteration, and the wave that shares a SIMD with a
        // stage-A wave and B1 sets the pace
        __builtin_amdgcn_s_setprio(1);
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
                const unsigned char *kvx = lds + L::O_KV + (x & 3) * L::KV;
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
                const bf16x4 ibx = *reinterpret_cast<const bf16x4 *>(pay + P::IB + lane * 8);
#pragma unroll
                for (int j = 0; j < SPW; ++j)   // u' = INV beta v from the chunk's v C tiles
                    up[j] = mma16(ibx, *reinterpret_cast<const bf16x4 *>(kvx + L::VT + ((cw * SPW + j) * 64 + lane) * 8), Z4);
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
    auto kv = [&](int x) { return lds + L::O_KV + (x & 3) * L::KV; };
    if (wv == NPW) {
        // the INV wave: stage B1 of chunk it + 2 in iteration it
        for (int it = -3; it < c.nch; ++it) {
            const int x = it + 2;
            if (x >= 0 && x < c.nch) stage_b1<NPW>(part(x), beta(x), pay(x) + P::IB, pay(x) + P::MQ, lane);
            lds_barrier();
        }
        return;
    }
    __builtin_amdgcn_s_setprio(1);   // as the consumers (the B1 wave keeps 0)
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
            // stage B2: w fragments into the chunk's operands
            const bf16x4 ib = *reinterpret_cast<const bf16x4 *>(pay(xb) + P::IB + lane * 8);
            const unsigned char *kvb = kv(xb);
            for (int job = wv - 1; job < NKB; job += NPW - 1) {
                *reinterpret_cast<bf16x8 *>(pay(xb) + P::WF + (job * 64 + lane) * 16) =
                    w_frag(kvb + L::KT, ib, job, lane);
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
    // every block's inputs are requested before the first is used: the two
    // halves of each 256-byte row of q, k and g_raw arrive together
    In<0> in[NPW];
#pragma unroll
    for (int w = 0; w < NPW; ++w) {
        Prep<DK, 0> pr;
        pr.place(w, lane);
        pr.load(in[w], a, p.bos, p.len, p.x, head, 0, 0, 0, 0);
    }
#pragma unroll
    for (int w = 0; w < NPW; ++w) {
        Prep<DK, 0> pr;
        pr.init(a, head, w, lane);
        typename Prep<DK, 0>::Out o;
        pr.stage_a_core(in[w], rem, o);
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
        if (w == 0) beta = ln < rem ? sigmoid_f(bf16_to_f32(in[0].b)) : 0.f;
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

// Pass 2: one workgroup per (sequence, head, NSW slabs of 16 columns), one
// wave per slab.  Workgroup b takes chain 8 (b / 8 / NSG) + b % 8 and slab
// group (b / 8) % NSG, so that the slab groups of a chain share blockIdx % 8
// (the XCD, whose L2 then serves the chain's operands to all of them;
// placement only affects speed).
//
// A chunk's operands (its workspace row, padded to whole KiB, and the
// group's 16 x 16 NSW bf16 tile of v) reach a ring of RING LDS slots by
// direct global-to-LDS loads, RING - 1 chunks ahead, so the recurrence never
// waits on memory latency; the slabs of a group share them, which halves the
// load instructions per slab with NSW = 2 (they, not the arithmetic, set the
// pace where two workgroups share a compute unit).  The loads are issued
// from inline assembly (the compiler would otherwise wait for all of them
// before every LDS read).  Each is counted in its wave's vmcnt, which drains
// in issue order, so waiting until at most n operations remain outstanding,
// n = those issued after chunk x's loads, guarantees chunk x has landed.
//  - With a loader wave (wave NSW), the loads' issue cycles leave the slab
//    waves' critical path.  One barrier per chunk: at barrier x chunk x has
//    landed and every slab wave has read every operand of chunk x - 1, whose
//    slot the loader then refills.
//  - The snapshot form with one slab per group (8 KiB of snapshot stores per
//    chunk) runs one wave that issues its loads and stores and waits on its
//    own count, which measured faster than a loader there.
template <int DK, int DV, int NSW, bool SNAP>
__global__ __launch_bounds__(64 * (NSW + 1)) void rec_kernel(FwdArgs a, const unsigned char *ws)
{
    constexpr bool LOADER = !SNAP || NSW > 1;   // a separate loader wave (wave NSW)
    constexpr int NKB = DK / 32, NMT = DK / 16, NSG = DV / (16 * NSW);
    using P = Pay<DK>;
    constexpr int NPAY = (P::BYTES + 1023) / 1024;   // 1 KiB loads of a workspace row
    constexpr int ND = NPAY + 1;                     // and one for the v tile
    constexpr int SLOT = ND * 1024, VT = NPAY * 1024;
    static_assert((RING - 1) * ND <= 63, "loads in flight exceed the vmcnt field");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[RING * SLOT];
    const int lane = threadIdx.x & 63, ln = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool loader = LOADER && wv == NSW;
    const int b8 = blockIdx.x / 8;
    const int chain = 8 * (b8 / NSG) + blockIdx.x % 8;
    const int sg = b8 % NSG;
    if (chain >= a.n_seq * a.H) return;
    const Chain c = chain_of(a, chain / a.H, chain % a.H, threadIdx.x == 0 && sg == 0);
    const size_t H = a.H;
    const int cols = sg * NSW * 16;                  // the group's first column
    const int col0 = cols + 16 * (loader ? 0 : wv);  // this wave's slab
    const size_t hbase = (((size_t)(c.hrow < 0 ? 0 : c.hrow) * H + c.head) * DV + col0) * DK;
    f32x4 S[1][NMT];   // the state of this wave's slab, from h0 below
    const size_t cbase = chunk_base(a, c.seq);
    // identity as a K = 16 B operand: the product of a row-loaded 16 x 16 tile with it is its C layout
    bf16x4 eye;
#pragma unroll
    for (int e = 0; e < 4; ++e) eye[e] = static_cast<__bf16>(4 * lq + e == ln ? 1.f : 0.f);
    const unsigned ring_lds =
        __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) unsigned char *)ring);
    // v tile of the group in LDS: token t at t * 32 NSW bytes, 8 columns per
    // lane; for NSW = 1 lanes 32 .. 63 repeat lanes 0 .. 31 into the unused upper half.
    const int vt_tok = lane / (2 * NSW) % 16, vt_col = 8 * (lane % (2 * NSW));
    auto issue = [&](int x) {   // chunk x's loads into ring slot x % RING
        const unsigned slot = ring_lds + (unsigned)((x % RING) * SLOT);
        dma_bytes<P::BYTES>(ws + ((cbase + x) * H + c.head) * P::BYTES, slot, lane);
        const int rem = min(CH, c.len - x * CH);
        const uint16_t *v0 = static_cast<const uint16_t *>(a.v) + ((c.bos + (size_t)x * CH) * H + c.head) * DV + cols;
        dma_group<1>(v0, 0u, (unsigned)(((size_t)min(vt_tok, rem - 1) * H * DV + vt_col) * 2), slot + VT);
    };
    auto step = [&](int x) {
        const unsigned char *row = ring + (x % RING) * SLOT;
        if constexpr (SNAP) {
            const size_t at = (((cbase + x) * H + c.head) * DV + col0) * DK;
#pragma unroll
            for (int m = 0; m < NMT; ++m)
                __builtin_nontemporal_store(S[0][m], reinterpret_cast<f32x4 *>(
                    a.h_chunks + at + (size_t)ln * DK + chan(m, lq, 0)));
        }
        // operands from the ring slot, in the order the chunk consumes them:
        // v as lane (lq, ln) = token ln, columns 4 lq .. +3 of this wave's slab
        const bf16x4 vv = *reinterpret_cast<const bf16x4 *>(row + VT + ln * 32 * NSW + (col0 - cols + 4 * lq) * 2);
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
        f32x4 up[1], O[1];
        up[0] = mma16(ib, pack4(mma16(vv, eye, Z4)), Z4);   // u' = INV beta v (v in C layout by an identity product)
        rec_step<NKB, NMT, 1>(S, qf, wf, kr, eg, mq, up, O);
        const int rem = min(CH, c.len - x * CH);
        if (ln < rem) store_o(a.o, c.bos + (size_t)x * CH + ln, H, c.head, DV, col0 + 4 * lq, O[0], a.scale);
    };
    const int nch = c.nch;
    if (loader) {
        for (int x = 0; x < min(RING - 1, nch); ++x) issue(x);
        for (int x = 0; x < nch; ++x) {
            vm_wait_chunks<ND>(min(RING - 2, nch - 1 - x));   // chunk x has landed
            lds_barrier();
            if (x + RING - 1 < nch) issue(x + RING - 1);       // into the slot of chunk x - 1
        }
        return;
    }
#pragma unroll
    for (int m = 0; m < NMT; ++m)
        S[0][m] = (a.h0 && c.hrow >= 0) ? *reinterpret_cast<const f32x4 *>(a.h0 + hbase + (size_t)ln * DK + chan(m, lq, 0))
                                        : Z4;
    if constexpr (LOADER) {
        for (int x = 0; x < nch; ++x) {
            lds_barrier();   // chunk x has landed; every read of chunk x - 1 is done
            step(x);
        }
    } else {
        // one wave: its own loads, counted together with its stores
        for (int x = 0; x < min(RING - 1, nch); ++x) issue(x);
        for (int x = 0; x < nch; ++x) {
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the slot to refill has been read
            if (x + RING - 1 < nch) issue(x + RING - 1);
            vm_wait_chunks<ND>(min(RING - 1, nch - 1 - x));   // chunks x + 1 .. x + RING - 1 may still fly
            step(x);
        }
    }
    if (a.h_T && c.hrow >= 0) {
#pragma unroll
        for (int m = 0; m < NMT; ++m)
            *reinterpret_cast<f32x4 *>(a.h_T + hbase + (size_t)ln * DK + chan(m, lq, 0)) = S[0][m];
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

template <int DK, int DV, int NSW, bool SNAP>
hipError_t launch_rec(const FwdArgs &a, unsigned char *ws, long long chains, hipStream_t stream)
{
    constexpr int NSG = DV / (16 * NSW);
    const long long wgs = 8 * NSG * ((chains + 7) / 8);
    if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rec_kernel<DK, DV, NSW, SNAP>), dim3((unsigned)wgs), dim3(SNAP && NSW == 1 ? 64 : 64 * (NSW + 1)), 0,
                       stream, a, (const unsigned char *)ws);
    return hipGetLastError();
}

// The recurrence takes two slabs per workgroup (one payload load for both)
// where that still gives every compute unit a workgroup.
template <int DK, int DV, bool SNAP>
hipError_t launch_two_pass(const FwdArgs &a, unsigned char *ws, long long n_rows, int n_cu, hipStream_t stream)
{
    const long long wgs1 = (n_rows * a.H + PREP_WAVES - 1) / PREP_WAVES;
    if (wgs1 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (wgs1 > 0) {
        hipLaunchKernelGGL((prep_kernel<DK>), dim3((unsigned)wgs1), dim3(64 * PREP_WAVES), 0, stream, a, ws, n_rows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long long chains = (long long)a.n_seq * a.H;
    if (chains * (DV / 32) >= n_cu) return launch_rec<DK, DV, 2, SNAP>(a, ws, chains, stream);
    return launch_rec<DK, DV, 1, SNAP>(a, ws, chains, stream);
}

template <int DK, int DV>
hipError_t launch_dims(const FwdArgs &a, int n_cu, void *ws, size_t ws_bytes, long long n_rows, hipStream_t stream)
{
    const long long chains = (long long)a.n_seq * a.H;
    const bool two = ws && chains < n_cu && ws_bytes >= fwd_workspace_bytes(DK, n_rows, a.H);
    if (two)
        return a.h_chunks ? launch_two_pass<DK, DV, true>(a, static_cast<unsigned char *>(ws), n_rows, n_cu, stream)
                          : launch_two_pass<DK, DV, false>(a, static_cast<unsigned char *>(ws), n_rows, n_cu, stream);
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

}  // namespace kda
