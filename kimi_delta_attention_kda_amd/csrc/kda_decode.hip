// kda_decode.hip -- fused T=1 KDA decode step for gfx950.
//
// Follows the packed decode of [SGL-PR] ("SGLang PR #26586 (KDA packed
// decode)", section "实现拆解" item 1 and the kernel snippet): q/k/v are
// sliced out of one packed row by offset, the gate
// g = -exp(A_log) * softplus(a + dt_bias) and beta = sigmoid(b) are computed
// in registers, q and k are optionally L2-normalised (eps 1e-6 inside the
// square root) and q is scaled, then per state row
//   S' = S Diag(e^g);  u = beta (v - S' k);  S = S' + u k^T;  o = S q.
// A negative slot index marks a pad row: its output is zeroed and its state
// is not touched.
//
// MI355X mapping.  The step is HBM-bound (64 KiB of fp32 state read and
// written per (row, value head) against ~1 KiB of activations), so the kernel
// is one streaming pass:
//   * one 512-thread workgroup per (row, value head).  State rows are
//     independent given k, q and the gate, so each 256-thread half takes 64
//     of the 128 rows: in half p, thread (g, j) with g = t / 16 and
//     j = t % 16 (t = tid % 256) owns rows 64p + g + 16r (r < 4) and columns
//     [4j, 4j+4) u [64+4j, 64+4j+4): every wave-wide float4 access covers
//     four contiguous 256-byte row halves.  Halving the rows per thread
//     (72 VGPRs instead of 107) lets 7 waves share a SIMD; keeping both
//     halves in one workgroup keeps the dispatch count at one per item
//     (a workgroup per half, or per quarter, measured slower);
//   * all 8 float4 state loads of a thread are issued before any arithmetic
//     (64 KiB in flight per workgroup);
//   * the two row reductions S'k and S'q run over the 16 lanes of one row
//     group; o uses S q = S' q + u (k . q) so the state is read once;
//   * the updated state goes back with non-temporal stores.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

// One token's activations for one (row, value head), as a thread of the
// 512-thread workgroup loads them: its 8 q, k and a channels (bf16 pairs at
// columns 4j and 64+4j), the v values of its state rows and b.
template <int V_>
struct TokenRaw {
    uint2 qb[2], kb[2], ab[2];
    uint16_t vraw[V_ / 32];
    uint16_t braw;
};

// x: the token's packed qkv row; arow: its a row; bp: its b entry.
template <int K_, int V_>
__device__ __forceinline__ void load_token(TokenRaw<V_> &t, const uint16_t *x, const uint16_t *arow,
                                           const uint16_t *bp, int H, int hq, int hv, int j, int g,
                                           int r0)
{
    const int cols[2] = {4 * j, 64 + 4 * j};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        t.qb[h] = *reinterpret_cast<const uint2 *>(x + (size_t)hq * K_ + cols[h]);
        t.kb[h] = *reinterpret_cast<const uint2 *>(x + (size_t)H * K_ + (size_t)hq * K_ + cols[h]);
        t.ab[h] = *reinterpret_cast<const uint2 *>(arow + cols[h]);
    }
    const uint16_t *vrow = x + 2 * (size_t)H * K_ + (size_t)hv * V_ + r0;
#pragma unroll
    for (int r = 0; r < V_ / 32; ++r) t.vraw[r] = vrow[g + 16 * r];
    t.braw = *bp;
}

// Per-token values of [SGL-PR]'s update for the thread's 8 channels (columns
// 4j.. and 64+4j..): decay e^g, q (L2-normalised if asked, times scale) and k
// (L2-normalised if asked), the 16-lane sums k.q, and beta.  Every 16-lane row
// group computes the same values.
struct TokenPrep {
    float qv[8], kv[8], eg[8];
    float kq, beta;
};

// The rest of the per-token values once p.qv and p.kv hold the raw q and k
// channels: the decay from the thread's a channels (bf16 pairs) and dt_bias,
// the optional L2 norm, the q scale, k.q and beta.
__device__ __forceinline__ void prep_core(TokenPrep &p, const uint2 (&ab)[2], uint16_t braw,
                                          const f32x4 (&dt)[2], float A, float scale, int l2norm)
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t aw[2] = {ab[h].x, ab[h].y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint16_t ae = (uint16_t)(aw[e >> 1] >> (16 * (e & 1)));
            p.eg[4 * h + e] = gate_decay(bf16_to_f32(ae) + dt[h][e], A);
        }
    }
    if (l2norm) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) { sq += p.qv[c] * p.qv[c]; sk += p.kv[c] * p.kv[c]; }
        sq = row16_sum(sq);
        sk = row16_sum(sk);
        const float iq = 1.0f / sqrtf(sq + 1e-6f), ik = 1.0f / sqrtf(sk + 1e-6f);
#pragma unroll
        for (int c = 0; c < 8; ++c) { p.qv[c] *= iq; p.kv[c] *= ik; }
    }
    float kq = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) { p.qv[c] *= scale; kq += p.kv[c] * p.qv[c]; }
    p.kq = row16_sum(kq);
    p.beta = sigmoid_f(bf16_to_f32(braw));
}

template <int V_>
__device__ __forceinline__ void token_prep(TokenPrep &p, const TokenRaw<V_> &t, const f32x4 (&dt)[2],
                                           float A, float scale, int l2norm)
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t qw[2] = {t.qb[h].x, t.qb[h].y}, kw[2] = {t.kb[h].x, t.kb[h].y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p.qv[4 * h + e] = bf16_to_f32((uint16_t)(qw[e >> 1] >> (16 * (e & 1))));
            p.kv[4 * h + e] = bf16_to_f32((uint16_t)(kw[e >> 1] >> (16 * (e & 1))));
        }
    }
    prep_core(p, t.ab, t.braw, dt, A, scale, l2norm);
}

// The state rows of one token on the thread's registers s (rows g + 16 r of
// its half): S' = S Diag(e^g), u = beta (v - S'k), S = S' + u k^T and
// o = S'q + u (k.q).  row_done(r, o_r) runs once row r is final, so a caller
// can store it at once.
template <int V_, typename RowFn>
__device__ __forceinline__ void token_rows(f32x4 (&s)[V_ / 32][2], const TokenPrep &p,
                                           const float (&v)[V_ / 32], RowFn &&row_done)
{
    constexpr int ROWS = V_ / 32;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        float pk = 0.f, pq = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sv = s[r][h][e] * p.eg[4 * h + e];
                s[r][h][e] = sv;
                pk += sv * p.kv[4 * h + e];
                pq += sv * p.qv[4 * h + e];
            }
        pk = row16_sum(pk);
        pq = row16_sum(pq);
        const float u = p.beta * (v[r] - pk);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[r][h][e] += u * p.kv[4 * h + e];
        row_done(r, pq + u * p.kq);
    }
}

template <int K_, int V_>
__global__ __launch_bounds__(512) void decode_kernel(
    const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ a,
    const uint16_t *__restrict__ b, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, float *__restrict__ pool,
    const int32_t *__restrict__ state_idx, uint16_t *__restrict__ o, int H, int HV, int P,
    float scale, int l2norm, int *__restrict__ err)
{
    static_assert(K_ == 128 && V_ == 128, "decode kernel is built for K = V = 128");
    constexpr int ROWS = V_ / 32;  // rows per thread
    const int n = blockIdx.x / HV;
    const int hv = blockIdx.x - n * HV;
    const int tid = threadIdx.x & 255;
    const int r0 = (threadIdx.x >> 8) * (V_ / 2);  // first state row of this half
    const int j = tid & 15;
    const int g = tid >> 4;

    // Activation loads go out before the state loads: vmcnt retires in issue
    // order, so the gate arithmetic then overlaps the state's latency instead
    // of waiting behind it.  v is loaded here too, so no load follows the
    // first state store (vmcnt counts stores as well).
    const int hq = hv / (HV / H);
    const size_t D = 2 * (size_t)H * K_ + (size_t)HV * V_;
    TokenRaw<V_> tk;
    load_token<K_, V_>(tk, qkv + (size_t)n * D, a + ((size_t)n * HV + hv) * K_, b + (size_t)n * HV + hv,
                       H, hq, hv, j, g, r0);
    f32x4 dt[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        dt[h] = *reinterpret_cast<const f32x4 *>(dt_bias + (size_t)hv * K_ + 4 * j + 64 * h);
    const float A_l = A_log[hv];

    uint16_t *orow = o + ((size_t)n * HV + hv) * V_;
    const int idx = state_idx[n];
    if (idx < 0 || idx >= P) {  // pad slot (or one past the pool: reported): zero output, no state access
        if (idx >= P && threadIdx.x == 0) slot_error(err);
        if (threadIdx.x < V_) orow[threadIdx.x] = 0;
        return;
    }

    __builtin_amdgcn_sched_barrier(0);  // keep the activation loads ahead of the state loads
    float *S = pool + ((size_t)idx * HV + hv) * (size_t)(V_ * K_) + (size_t)r0 * K_;
    // state rows g + 16 r of this half, two float4 per row
    f32x4 s[ROWS][2];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const float *row = S + (size_t)(g + 16 * r) * K_;
        s[r][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + 4 * j));
        s[r][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + 64 + 4 * j));
    }

    const float A = __builtin_amdgcn_exp2f(A_l * kLog2e);
    TokenPrep pr;
    token_prep<V_>(pr, tk, dt, A, scale, l2norm);
    float vf[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) vf[r] = bf16_to_f32(tk.vraw[r]);
    token_rows<V_>(s, pr, vf, [&](int r, float ov) {
        const int row = g + 16 * r;
        float *dst = S + (size_t)row * K_;
        __builtin_nontemporal_store(s[r][0], reinterpret_cast<f32x4 *>(dst + 4 * j));
        __builtin_nontemporal_store(s[r][1], reinterpret_cast<f32x4 *>(dst + 64 + 4 * j));
        if (j == 0) orow[r0 + row] = f32_to_bf16(ov);
    });
}

// T tokens per row applied in order to the row's slot (the fused recurrent
// form with a token loop that [SGL-PR] names for extend and speculative
// verification): the slot is read once, kept in registers for all T tokens
// and written once.  Tokens go in windows of TW = 16:
//   * the workgroup loads a window's q, k, a and v rows (1 KiB per token) into
//     LDS, one 16-byte load per thread per 8 tokens, issued ahead of the state
//     loads for the first window: one memory latency per window;
//   * 16-lane row group tt then computes token tt's per-channel values (gate,
//     normalised q and k, k.q, beta; the lane layout and summation order of
//     the T = 1 kernel, so the results are bitwise the same) into LDS, once
//     per token instead of once per row group;
//   * the token loop reads them back and does only the row work;
//   * the window's outputs are gathered in LDS and stored as 256-byte rows.
// Token t of row n: qkv[(n T + t) D ..], a[(n T + t) HV K ..],
// b[(n T + t) HV ..], o[((n T + t) HV + hv) V ..].
template <int K_, int V_>
__global__ __launch_bounds__(512) void extend_kernel(
    const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ a,
    const uint16_t *__restrict__ b, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, float *__restrict__ pool,
    const int32_t *__restrict__ state_idx, uint16_t *__restrict__ o, int T, int H, int HV, int P,
    float scale, int l2norm, int *__restrict__ err)
{
    static_assert(K_ == 128 && V_ == 128, "extend kernel is built for K = V = 128");
    constexpr int ROWS = V_ / 32;
    constexpr int TW = 16;                   // tokens per window (one per 16-lane row group of a half)
    constexpr int UNITS = (3 * K_ + V_) / 8; // 16-byte units per token: q, k, a, v
    constexpr int PER = TW * UNITS / 512;    // units each thread loads per window
    __shared__ uint4 stage[TW * UNITS];      // [token][q | k | a | v] bf16
    __shared__ uint16_t bstage[TW];
    __shared__ f32x4 prep[TW][3][K_ / 4];    // [token][q | k | e^g][channel] fp32
    __shared__ float2 prep_s[TW];            // [token](k.q, beta)
    __shared__ uint4 ostage[TW * V_ / 8];    // [token][V] bf16

    const int n = blockIdx.x / HV;
    const int hv = blockIdx.x - n * HV;
    const int tid = threadIdx.x & 255;
    const int r0 = (threadIdx.x >> 8) * (V_ / 2);
    const int j = tid & 15;
    const int g = tid >> 4;
    const int hq = hv / (HV / H);
    const size_t D = 2 * (size_t)H * K_ + (size_t)HV * V_;
    const size_t tok0 = (size_t)n * T;

    const int idx = state_idx[n];
    if (idx < 0 || idx >= P) {  // pad row (or one past the pool: reported): zero outputs, no state access
        if (idx >= P && threadIdx.x == 0) slot_error(err);
        for (int i = threadIdx.x; i < T * (V_ / 8); i += 512)
            *reinterpret_cast<uint4 *>(o + ((tok0 + i / (V_ / 8)) * HV + hv) * V_ + 8 * (i % (V_ / 8))) =
                make_uint4(0, 0, 0, 0);
        return;
    }

    // Window loads: lane unit lu = threadIdx % 64 of the token rows
    // threadIdx / 64 and threadIdx / 64 + 8 (512 is a multiple of 64, so each
    // lane always loads the same unit: q, k, a or v, 16 bytes).
    const int lu = threadIdx.x & 63;
    const int ltok = threadIdx.x >> 6;
    const uint16_t *lbase;
    size_t lstride;
    if (lu < 32) {
        lbase = qkv + (lu < 16 ? (size_t)hq * K_ + 8 * lu : (size_t)H * K_ + (size_t)hq * K_ + 8 * (lu - 16));
        lstride = D;
    } else if (lu < 48) {
        lbase = a + (size_t)hv * K_ + 8 * (lu - 32);
        lstride = (size_t)HV * K_;
    } else {
        lbase = qkv + 2 * (size_t)H * K_ + (size_t)hv * V_ + 8 * (lu - 48);
        lstride = D;
    }
    struct Win {
        uint4 v[PER];
        uint16_t b;
    };
    auto load_window = [&](int t0, int nt) {
        Win w;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int tt = ltok + 8 * e;
            w.v[e] = tt < nt ? *reinterpret_cast<const uint4 *>(lbase + (tok0 + t0 + tt) * lstride)
                             : make_uint4(0, 0, 0, 0);
        }
        w.b = threadIdx.x < nt ? b[(tok0 + t0 + threadIdx.x) * HV + hv] : (uint16_t)0;
        return w;
    };
    const uint2 *st2 = reinterpret_cast<const uint2 *>(stage);
    const uint16_t *st16 = reinterpret_cast<const uint16_t *>(stage);
    f32x4 dt[2];
    float A = 0.f;
    // raw window -> LDS, then row group g < nt (first half) preps token g
    auto publish_window = [&](const Win &w, int nt) {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            if (ltok + 8 * e < nt) stage[threadIdx.x + 512 * e] = w.v[e];
        if (threadIdx.x < nt) bstage[threadIdx.x] = w.b;
        __syncthreads();
        if (threadIdx.x < 256 && g < nt) {
            TokenRaw<V_> tk;
            const uint2 *u2 = st2 + g * (UNITS * 2);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                tk.qb[h] = u2[j + 16 * h];
                tk.kb[h] = u2[32 + j + 16 * h];
                tk.ab[h] = u2[64 + j + 16 * h];
            }
            tk.braw = bstage[g];
            TokenPrep pr;
            token_prep<V_>(pr, tk, dt, A, scale, l2norm);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                prep[g][0][j + 16 * h] = f32x4{pr.qv[4 * h], pr.qv[4 * h + 1], pr.qv[4 * h + 2], pr.qv[4 * h + 3]};
                prep[g][1][j + 16 * h] = f32x4{pr.kv[4 * h], pr.kv[4 * h + 1], pr.kv[4 * h + 2], pr.kv[4 * h + 3]};
                prep[g][2][j + 16 * h] = f32x4{pr.eg[4 * h], pr.eg[4 * h + 1], pr.eg[4 * h + 2], pr.eg[4 * h + 3]};
            }
            if (j == 0) prep_s[g] = make_float2(pr.kq, pr.beta);
        }
        __syncthreads();
    };

    const int nt0 = T < TW ? T : TW;
    const Win w0 = load_window(0, nt0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
        dt[h] = *reinterpret_cast<const f32x4 *>(dt_bias + (size_t)hv * K_ + 4 * j + 64 * h);
    A = __builtin_amdgcn_exp2f(A_log[hv] * kLog2e);

    __builtin_amdgcn_sched_barrier(0);  // the first window's loads ahead of the state loads
    float *S = pool + ((size_t)idx * HV + hv) * (size_t)(V_ * K_) + (size_t)r0 * K_;
    f32x4 s[ROWS][2];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const float *row = S + (size_t)(g + 16 * r) * K_;
        s[r][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + 4 * j));
        s[r][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + 64 + 4 * j));
    }
    publish_window(w0, nt0);

    uint16_t *os16 = reinterpret_cast<uint16_t *>(ostage);
    for (int t0 = 0; t0 < T; t0 += TW) {
        const int nt = T - t0 < TW ? T - t0 : TW;
        if (t0 > 0) {
            publish_window(load_window(t0, nt), nt);
        }
        for (int tt = 0; tt < nt; ++tt) {
            TokenPrep pr;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 q4 = prep[tt][0][j + 16 * h], k4 = prep[tt][1][j + 16 * h],
                            e4 = prep[tt][2][j + 16 * h];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pr.qv[4 * h + e] = q4[e];
                    pr.kv[4 * h + e] = k4[e];
                    pr.eg[4 * h + e] = e4[e];
                }
            }
            const float2 ks = prep_s[tt];
            pr.kq = ks.x;
            pr.beta = ks.y;
            float vf[ROWS];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) vf[r] = bf16_to_f32(st16[tt * (UNITS * 8) + 3 * K_ + r0 + g + 16 * r]);
            token_rows<V_>(s, pr, vf, [&](int r, float ov) {
                if (j == 0) os16[tt * V_ + r0 + g + 16 * r] = f32_to_bf16(ov);
            });
        }
        __syncthreads();  // window outputs gathered; stage and prep free for the next window
        for (int i = threadIdx.x; i < nt * (V_ / 8); i += 512)
            *reinterpret_cast<uint4 *>(o + ((tok0 + t0 + i / (V_ / 8)) * HV + hv) * V_ + 8 * (i % (V_ / 8))) =
                ostage[i];
        __syncthreads();  // ostage read before the next window writes it
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        float *dst = S + (size_t)(g + 16 * r) * K_;
        __builtin_nontemporal_store(s[r][0], reinterpret_cast<f32x4 *>(dst + 4 * j));
        __builtin_nontemporal_store(s[r][1], reinterpret_cast<f32x4 *>(dst + 64 + 4 * j));
    }
}

// The short causal convolution before decode, fused with the decode step.
// [SGL-PR] (backend integration) runs causal_conv1d_update with silu on the
// packed projections as a launch of its own before the packed decode, its
// conv-state slots addressed by the same cache indices as the recurrent
// state.  Per channel c of a live row:
//   window = (cs[0, c], ..., cs[W-2, c], x[c])     oldest first
//   y[c]   = silu(bias[c] + sum_w weight[c, w] window[w]);  cs <- window[1 ..]
// and y takes the place of the packed q/k/v row of the decode step.
//
// One 512-thread workgroup per (row, q/k head): it convolves the q and k
// channels of that head and the v channels of the HV/H value heads that read
// it, so every conv-state channel has exactly one workgroup, which reads it
// before writing it.  y stays in LDS in fp32; the decode step of each of
// those value heads then runs on the T=1 kernel's thread layout.  The first
// value head's activation and state loads are issued before the convolution
// is computed, so its latency hides behind them.
template <int K_, int V_, int W_>
__global__ __launch_bounds__(512) void conv_decode_kernel(
    const uint16_t *__restrict__ x, uint16_t *__restrict__ conv_state,
    const uint16_t *__restrict__ cw, const uint16_t *__restrict__ cb,
    const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float *__restrict__ pool,
    const int32_t *__restrict__ state_idx, uint16_t *__restrict__ o, int H, int HV, int P,
    float scale, int l2norm, int *__restrict__ err)
{
    static_assert(K_ == 128 && V_ == 128, "conv decode kernel is built for K = V = 128");
    static_assert(W_ >= 2 && W_ <= 4, "conv width 2..4");
    constexpr int ROWS = V_ / 32;
    extern __shared__ float ybuf[];  // [q: K | k: K | v: G V] conv outputs, fp32
    const int n = blockIdx.x / H;
    const int hq = blockIdx.x - n * H;
    const int G = HV / H;
    const int tid = threadIdx.x & 255;
    const int r0 = (threadIdx.x >> 8) * (V_ / 2);
    const int j = tid & 15;
    const int g = tid >> 4;
    const size_t D = 2 * (size_t)H * K_ + (size_t)HV * V_;
    const int nch = 2 * K_ + G * V_;

    const int idx = state_idx[n];
    if (idx < 0 || idx >= P) {  // pad row (or one past the pool: reported): zero outputs, no state access
        if (idx >= P && threadIdx.x == 0) slot_error(err);
        for (int i = threadIdx.x; i < G * V_; i += 512) o[((size_t)n * HV + (size_t)hq * G) * V_ + i] = 0;
        return;
    }

    // channel ch of this workgroup -> column of the packed row
    auto column = [&](int ch) -> size_t {
        return ch < K_       ? (size_t)hq * K_ + ch
               : ch < 2 * K_ ? (size_t)H * K_ + (size_t)hq * K_ + (ch - K_)
                             : 2 * (size_t)H * K_ + (size_t)hq * G * V_ + (ch - 2 * K_);
    };
    const uint16_t *xrow = x + (size_t)n * D;
    uint16_t *cs = conv_state + (size_t)idx * (W_ - 1) * D;
    struct ConvIn {
        uint16_t xv, st[W_ - 1], wt[W_], bias;
    };
    auto conv_load = [&](int ch) {
        ConvIn c;
        const size_t col = column(ch);
        c.xv = xrow[col];
#pragma unroll
        for (int w = 0; w < W_ - 1; ++w) c.st[w] = cs[(size_t)w * D + col];
#pragma unroll
        for (int w = 0; w < W_; ++w) c.wt[w] = cw[col * W_ + w];
        c.bias = cb ? cb[col] : (uint16_t)0;
        return c;
    };
    auto conv_finish = [&](int ch, const ConvIn &c) {
        const size_t col = column(ch);
        float z = bf16_to_f32(c.bias);
#pragma unroll
        for (int w = 0; w < W_ - 1; ++w) z += bf16_to_f32(c.wt[w]) * bf16_to_f32(c.st[w]);
        z += bf16_to_f32(c.wt[W_ - 1]) * bf16_to_f32(c.xv);
        ybuf[ch] = z / (1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
#pragma unroll
        for (int w = 0; w < W_ - 1; ++w) cs[(size_t)w * D + col] = w + 1 < W_ - 1 ? c.st[w + 1] : c.xv;
    };

    // per value head: its a, dt_bias, b, A_log and state rows
    uint2 ab[2];
    f32x4 dt[2];
    uint16_t braw;
    float A_l;
    f32x4 s[ROWS][2];
    float *S;
    auto head_load = [&](int gi) {
        const int hv = hq * G + gi;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            ab[h] = *reinterpret_cast<const uint2 *>(a + ((size_t)n * HV + hv) * K_ + 4 * j + 64 * h);
            dt[h] = *reinterpret_cast<const f32x4 *>(dt_bias + (size_t)hv * K_ + 4 * j + 64 * h);
        }
        braw = b[(size_t)n * HV + hv];
        A_l = A_log[hv];
        __builtin_amdgcn_sched_barrier(0);  // activations ahead of the state loads
        S = pool + ((size_t)idx * HV + hv) * (size_t)(V_ * K_) + (size_t)r0 * K_;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const float *row = S + (size_t)(g + 16 * r) * K_;
            s[r][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + 4 * j));
            s[r][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + 64 + 4 * j));
        }
    };

    ConvIn c0;
    const bool has0 = (int)threadIdx.x < nch;
    if (has0) c0 = conv_load(threadIdx.x);
    head_load(0);
    if (has0) conv_finish(threadIdx.x, c0);
    for (int ch = threadIdx.x + 512; ch < nch; ch += 512) conv_finish(ch, conv_load(ch));
    __syncthreads();  // y complete in LDS

    for (int gi = 0; gi < G; ++gi) {
        if (gi > 0) head_load(gi);
        const int hv = hq * G + gi;
        TokenPrep pr;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4 q4 = *reinterpret_cast<const f32x4 *>(ybuf + 4 * j + 64 * h);
            const f32x4 k4 = *reinterpret_cast<const f32x4 *>(ybuf + K_ + 4 * j + 64 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pr.qv[4 * h + e] = q4[e];
                pr.kv[4 * h + e] = k4[e];
            }
        }
        prep_core(pr, ab, braw, dt, __builtin_amdgcn_exp2f(A_l * kLog2e), scale, l2norm);
        float vf[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) vf[r] = ybuf[2 * K_ + gi * V_ + r0 + g + 16 * r];
        uint16_t *orow = o + ((size_t)n * HV + hv) * V_;
        token_rows<V_>(s, pr, vf, [&](int r, float ov) {
            const int row = g + 16 * r;
            float *dst = S + (size_t)row * K_;
            __builtin_nontemporal_store(s[r][0], reinterpret_cast<f32x4 *>(dst + 4 * j));
            __builtin_nontemporal_store(s[r][1], reinterpret_cast<f32x4 *>(dst + 64 + 4 * j));
            if (j == 0) orow[r0 + row] = f32_to_bf16(ov);
        });
    }
}

hipError_t launch_decode(const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                         const float *A_log, const float *dt_bias, float *pool,
                         const int32_t *state_idx, uint16_t *o, int B, int H, int HV, int P,
                         float scale, int l2norm, int *err, hipStream_t stream)
{
    hipLaunchKernelGGL((decode_kernel<128, 128>), dim3((unsigned)(B * HV)), dim3(512), 0, stream,
                       qkv, a, b, A_log, dt_bias, pool, state_idx, o, H, HV, P, scale, l2norm, err);
    return hipGetLastError();
}

hipError_t launch_extend(const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                         const float *A_log, const float *dt_bias, float *pool,
                         const int32_t *state_idx, uint16_t *o, int B, int T, int H, int HV, int P,
                         float scale, int l2norm, int *err, hipStream_t stream)
{
    hipLaunchKernelGGL((extend_kernel<128, 128>), dim3((unsigned)(B * HV)), dim3(512), 0, stream,
                       qkv, a, b, A_log, dt_bias, pool, state_idx, o, T, H, HV, P, scale, l2norm, err);
    return hipGetLastError();
}

hipError_t launch_conv_decode(const uint16_t *x, uint16_t *conv_state, const uint16_t *cw,
                              const uint16_t *cb, const uint16_t *a, const uint16_t *b,
                              const float *A_log, const float *dt_bias, float *pool,
                              const int32_t *state_idx, uint16_t *o, int B, int H, int HV, int W, int P,
                              float scale, int l2norm, int *err, hipStream_t stream)
{
    const size_t lds = sizeof(float) * (2 * 128 + (size_t)(HV / H) * 128);
    const dim3 grid((unsigned)(B * H)), block(512);
    switch (W) {
    case 2:
        hipLaunchKernelGGL((conv_decode_kernel<128, 128, 2>), grid, block, lds, stream, x, conv_state, cw, cb, a,
                           b, A_log, dt_bias, pool, state_idx, o, H, HV, P, scale, l2norm, err);
        break;
    case 3:
        hipLaunchKernelGGL((conv_decode_kernel<128, 128, 3>), grid, block, lds, stream, x, conv_state, cw, cb, a,
                           b, A_log, dt_bias, pool, state_idx, o, H, HV, P, scale, l2norm, err);
        break;
    case 4:
        hipLaunchKernelGGL((conv_decode_kernel<128, 128, 4>), grid, block, lds, stream, x, conv_state, cw, cb, a,
                           b, A_log, dt_bias, pool, state_idx, o, H, HV, P, scale, l2norm, err);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kda
