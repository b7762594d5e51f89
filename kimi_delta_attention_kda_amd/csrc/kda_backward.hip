// kda_backward.hip -- gradients of the KDA forward for gfx950 (CDNA4), bf16
// activations, d_k = d_v = 128.
//
// The backward is chunkwise ([LA-06] "06 · linear 路线（一）：kernel trick、RNN
// 等价与三种计算形式", chunkwise form: a reverse loop over chunks from the
// states stored at chunk boundaries; gate and beta of [SGL-PR] "SGLang PR
// #26586 (KDA packed decode)").  Three passes and a reduction, all on the
// caller's stream, sharing the prefill's operand layouts and helpers
// (kda_chunk.hpp):
//   1. bwd_prep_kernel: the reverse chain's state-independent operands of
//      every chunk, all chunks in parallel (the forward's prep stages);
//   2. bwd_rec_kernel: one sequential loop over the chunks of each (sequence,
//      head) that carries dS (the gradient with respect to the state) in fp32
//      MFMA accumulators, leaving dS and dU for every chunk;
//   3. bwd_chunk_kernel: every chunk's gradients of q, k, v, g_raw and
//      beta_raw in parallel, and the chunk's sums of the gradients of dt_bias
//      and A_log;
//   4. params_slice_kernel, params_final_kernel: those per-chunk sums added,
//      first over BWD_SPLIT slices of chunk rows, then over the slices, in a
//      fixed order (deterministic, no atomics).
#include <stdint.h>

#include "kda_chunk.hpp"

namespace kda {

// Per chunk, with dS' the gradient of the loss with respect to the state
// after the chunk and dO_s = scale dO, the forward S' = D S + k^r^T U,
// U = u' - w S, O = scale (q~ S + Mqk U) gives
//   dU = k^r dS' + Mqk^T dO_s,   dS = D dS' + q~^T dO_s - w^T dU,
// the mirror of the forward recurrence: one sequential MFMA chain per chunk
// that needs only state-independent operands (k^r, q~, w, e^{G_C}, Mqk) and
// dO, formed by the forward's prep stages.

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
        if (w == 0) beta = ln < rem ? sigmoid_f(bf16_to_f32(in[0].b)) : 0.f;
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

// The reverse chain: one workgroup per (chain, NSW slabs of 16 state
// columns), chunks from last to first: wave j < NSW carries its slab's dS'
// (fp32, in the forward state's registers and layout) from dh_T, leaves dS'
// and dU in a gradient row for every chunk and the gradient before the first
// chunk in dh0; wave NSW only loads, once for the group.  Operands reach a
// ring of LDS slots by direct global-to-LDS loads, RING - 1 chunks ahead,
// issued, counted and handed over (one barrier per chunk) as in the
// prefill's rec_kernel.
template <int DK, int DV, int NSW>
__global__ __launch_bounds__(64 * (NSW + 1)) void bwd_rec_kernel(FwdArgs a, const unsigned char *ws, const float *dh_T,
                                                      const void *dO, unsigned char *grows, float *dh0)
{
    constexpr int NKB = DK / 32, NMT = DK / 16, NSG = DV / (16 * NSW);
    static_assert(DK == 128 && DV == 128, "gradient rows are laid out for d = 128");
    using P = BPay<DK>;
    constexpr int NPAY = (P::REC + 1023) / 1024;
    constexpr int ND = NPAY + 1;                     // and one for the dO tile
    constexpr int SLOT = ND * 1024, DT = NPAY * 1024;
    static_assert((RING - 1) * ND <= 63, "loads in flight exceed the vmcnt field");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[RING * SLOT];
    const int lane = threadIdx.x & 63, ln = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool loader = wv == NSW;
    const int b8 = blockIdx.x / 8;
    const int chain = 8 * (b8 / NSG) + blockIdx.x % 8;
    const int sg = b8 % NSG;
    if (chain >= a.n_seq * a.H) return;
    const Chain c = chain_of(a, chain / a.H, chain % a.H, false);
    const size_t H = a.H;
    const int cols = sg * NSW * 16;                  // the group's first column
    const int slab = sg * NSW + (loader ? 0 : wv);   // this wave's slab
    const int col0 = 16 * slab;
    const size_t hbase = (((size_t)c.seq * H + c.head) * DV + col0) * DK;
    f32x4 dS[NMT];   // the reverse chain's gradient (wave 0), from dh_T below
    const size_t cbase = chunk_base(a, c.seq);
    bf16x4 eye;
#pragma unroll
    for (int e = 0; e < 4; ++e) eye[e] = static_cast<__bf16>(4 * lq + e == ln ? 1.f : 0.f);
    const unsigned ring_lds =
        __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) unsigned char *)ring);
    // dO tile of the group in LDS: token t at t * 32 NSW bytes, 8 columns per lane
    const int vt_tok = lane / (2 * NSW) % 16, vt_col = 8 * (lane % (2 * NSW));
    // the kk-th chunk walked is chunk nch - 1 - kk
    auto issue = [&](int kk) {
        const int x = c.nch - 1 - kk;
        const unsigned slot = ring_lds + (unsigned)((kk % RING) * SLOT);
        dma_bytes<P::REC>(ws + ((cbase + x) * H + c.head) * P::BYTES, slot, lane);
        const int rem = min(CH, c.len - x * CH);
        const uint16_t *d0 = static_cast<const uint16_t *>(dO) + ((c.bos + (size_t)x * CH) * H + c.head) * DV + cols;
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
                                        reinterpret_cast<bf16x8 *>(g + GRow::DM + (slab * NKB + cb) * 1024 + lane * 16));
        const int rem = min(CH, c.len - x * CH);
        bf16x4 dOr = *reinterpret_cast<const bf16x4 *>(row + DT + ln * 32 * NSW + (col0 - cols + 4 * lq) * 2);
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
        __builtin_nontemporal_store(dU, reinterpret_cast<f32x4 *>(g + GRow::DU + slab * 1024 + lane * 16));
        const bf16x8 bdU = hilo(dU);
        // dS = D dS' - w^T dU + q~^T dO_s
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            dS[m] *= eg[m];
            dS[m] = mma32(cat4(wc[m], wc[m]), bdU, dS[m]);
            dS[m] = mma16(qc[m], bdO, dS[m]);
        }
    };
    const int nch = c.nch;
    if (loader) {
        for (int kk = 0; kk < min(RING - 1, nch); ++kk) issue(kk);
        for (int kk = 0; kk < nch; ++kk) {
            vm_wait_chunks<ND>(min(RING - 2, nch - 1 - kk));   // the kk-th chunk has landed
            lds_barrier();
            if (kk + RING - 1 < nch) issue(kk + RING - 1);       // into the slot of the previous one
        }
        return;
    }
#pragma unroll
    for (int m = 0; m < NMT; ++m)
        dS[m] = dh_T ? *reinterpret_cast<const f32x4 *>(dh_T + hbase + (size_t)ln * DK + chan(m, lq, 0)) : Z4;
    for (int kk = 0; kk < nch; ++kk) {
        lds_barrier();   // the kk-th chunk has landed; every read of the previous one is done
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

namespace {
// The workspace: per (chunk row, head) the reverse chain's operands (BPay),
// the gradient row (GRow) and the parameter sums ([n_rows][H][129]), then
// the BWD_SPLIT slice sums per head ([H][BWD_SPLIT][129]).
constexpr int BWD_SPLIT = 64;
struct BwdWs {
    size_t pay, grow, part, red, bytes;
};
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
    // two slabs per workgroup (one payload load for both) where that still
    // gives every compute unit a workgroup
    const long long chains = (long long)b.n_seq * b.H;
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const bool two = chains * 4 >= n_cu;
    const long long wgs = 8 * (two ? 4 : 8) * ((chains + 7) / 8);
    if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (wgs > 0) {
        if (two)
            hipLaunchKernelGGL((bwd_rec_kernel<128, 128, 2>), dim3((unsigned)wgs), dim3(192), 0, stream, a, ws + l.pay,
                               b.dh_T, b.do_, ws + l.grow, b.dh0);
        else
            hipLaunchKernelGGL((bwd_rec_kernel<128, 128, 1>), dim3((unsigned)wgs), dim3(128), 0, stream, a, ws + l.pay,
                               b.dh_T, b.do_, ws + l.grow, b.dh0);
        e = hipGetLastError();
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
