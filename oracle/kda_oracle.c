/*
 * kda_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain fp64 CPU oracle for Kimi Delta Attention (KDA).  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load this library; the
 * product path never does.  It shares no code, header or constant with the HIP
 * library.
 *
 * Sources (web pages; cited by title and section):
 *   [TL-KDA]  "TileLang 实战：KDA 从零到一 -- Chunked 线性注意力", section 1:
 *             the recurrence S_t = S_{t-1} D_t (I - beta_t k_t k_t^T)
 *             + beta_t v_t k_t^T, o_t = S_t q_t, with D_t = diag(e^{g_t}) and
 *             S stored as (d_v, d_k).
 *   [SGL-PR]  "SGLang PR #26586 (KDA packed decode)", section "实现拆解" item 1
 *             and the fused_recurrent_kda_packed_decode_kernel snippet: the
 *             gate g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b),
 *             the optional in-kernel L2 norm of q and k (eps 1e-6 inside the
 *             square root), q scaled after normalisation, the update order
 *             decay -> delta -> write -> read, the packed qkv offsets, the
 *             GQA head map and the pad slot (index < 0 -> zero output, no
 *             state write).
 *
 * The per-token update below is the recurrence of [TL-KDA] section 1 written
 * as the four steps of [SGL-PR]:
 *     S <- S * diag(e^g)            (decay along the key axis)
 *     u <- beta * (v - S k)         (delta)
 *     S <- S + u k^T                (write)
 *     o <- S (scale * q)            (read after the write: o_t = S_t q_t)
 * Expanding S D (I - beta k k^T) + beta v k^T gives exactly these steps.
 *
 * softplus is evaluated exactly as max(x,0) + log1p(exp(-|x|)) (no threshold).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus_exact(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* One (sequence, head) chain of the token recurrence.
 * Activations are packed token-major: x[(tok*H + h)*d + c].
 * S is (dv, dk) row-major, updated in place.
 * Hc: NULL, or where the state before token t = C*i goes (for every i with
 * C*i < len), at Hc + i * Hc_stride. */
static void oracle_chain(const double *q, const double *k, const double *v,
                         const double *a, const double *b, double A_exp,
                         const double *dt, double *S, double *o,
                         int64_t tok0, int64_t len, int H, int h, int dk, int dv,
                         double scale, double *eg, double *u,
                         double *Hc, int C, int64_t Hc_stride)
{
    for (int64_t t = 0; t < len; ++t) {
        if (Hc && t % C == 0)
            memcpy(Hc + (t / C) * Hc_stride, S, sizeof(double) * (size_t)dv * dk);
        const int64_t tok = tok0 + t;
        const double *qt = q + (tok * H + h) * (int64_t)dk;
        const double *kt = k + (tok * H + h) * (int64_t)dk;
        const double *vt = v + (tok * H + h) * (int64_t)dv;
        const double *at = a + (tok * H + h) * (int64_t)dk;
        const double beta = sigmoid(b[tok * H + h]);
        for (int c = 0; c < dk; ++c)
            eg[c] = exp(-A_exp * softplus_exact(at[c] + dt[c]));
        /* decay, then delta: u = beta (v - S' k) */
        for (int r = 0; r < dv; ++r) {
            double *Sr = S + (int64_t)r * dk;
            double w = 0.0;
            for (int c = 0; c < dk; ++c) {
                Sr[c] *= eg[c];
                w += Sr[c] * kt[c];
            }
            u[r] = beta * (vt[r] - w);
        }
        /* write, then read with the updated state */
        double *ot = o + (tok * H + h) * (int64_t)dv;
        for (int r = 0; r < dv; ++r) {
            double *Sr = S + (int64_t)r * dk;
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) {
                Sr[c] += u[r] * kt[c];
                acc += Sr[c] * qt[c];
            }
            ot[r] = scale * acc;
        }
    }
}

/*
 * Chunk-free forward over packed variable-length sequences.
 *   q,k,a : [T_total, H, dk]   v, o : [T_total, H, dv]   b : [T_total, H]
 *   A_log : [H]  dt_bias : [H, dk]
 *   h0    : [n_seq, H, dv, dk] or NULL (zero initial state)
 *   hT    : [n_seq, H, dv, dk] or NULL
 *   cu_seqlens : [n_seq + 1] token offsets (int64)
 *   chains: optional list of chain ids (seq * H + head) to compute; NULL = all.
 *           Outputs of chains not listed are left untouched.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
static int oracle_fwd(const double *q, const double *k, const double *v,
                      const double *a, const double *b, const double *A_log,
                      const double *dt_bias, const double *h0,
                      const int64_t *cu_seqlens, int n_seq, int H, int dk, int dv,
                      double scale, const int32_t *chains, int n_chains,
                      double *o, double *hT, double *h_chunks, int C, int n_threads)
{
    if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !cu_seqlens || !o)
        return -1;
    if (h_chunks && C <= 0) return -1;
    if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    const int total = chains ? n_chains : n_seq * H;
    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
#endif
    for (int i = 0; i < total; ++i) {
        const int id = chains ? chains[i] : i;
        const int s = id / H, h = id % H;
        if (s < 0 || s >= n_seq) { err |= 1; continue; }
        double *S = (double *)malloc(sizeof(double) * ((size_t)dv * dk + dk + dv));
        if (!S) { err |= 1; continue; }
        double *eg = S + (size_t)dv * dk, *u = eg + dk;
        const size_t off = ((size_t)s * H + h) * (size_t)dv * dk;
        if (h0) memcpy(S, h0 + off, sizeof(double) * (size_t)dv * dk);
        else memset(S, 0, sizeof(double) * (size_t)dv * dk);
        double *Hc = NULL;
        if (h_chunks) {
            int64_t cb = 0;   /* chunks of the sequences before s */
            for (int s2 = 0; s2 < s; ++s2) cb += (cu_seqlens[s2 + 1] - cu_seqlens[s2] + C - 1) / C;
            Hc = h_chunks + (cb * H + h) * (int64_t)dv * dk;
        }
        oracle_chain(q, k, v, a, b, exp(A_log[h]), dt_bias + (size_t)h * dk, S, o,
                     cu_seqlens[s], cu_seqlens[s + 1] - cu_seqlens[s], H, h, dk, dv,
                     scale, eg, u, Hc, C, (int64_t)H * dv * dk);
        if (hT) memcpy(hT + off, S, sizeof(double) * (size_t)dv * dk);
        free(S);
    }
    (void)n_threads;
    return err ? -1 : 0;
}

int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *a, const double *b, const double *A_log,
                   const double *dt_bias, const double *h0,
                   const int64_t *cu_seqlens, int n_seq, int H, int dk, int dv,
                   double scale, const int32_t *chains, int n_chains,
                   double *o, double *hT, int n_threads)
{
    return oracle_fwd(q, k, v, a, b, A_log, dt_bias, h0, cu_seqlens, n_seq, H, dk, dv, scale,
                      chains, n_chains, o, hT, NULL, 0, n_threads);
}

/*
 * kda_oracle_fwd with the state entering every chunk of C tokens recorded:
 * h_chunks [N_chunks, H, dv, dk], row (chunks of the sequences before s) + c
 * holds the state of (s, head) before token C*c of s (the materialised form:
 * states stored at chunk boundaries).  N_chunks = sum over s of
 * ceil(len_s / C).
 */
int kda_oracle_fwd_states(const double *q, const double *k, const double *v,
                          const double *a, const double *b, const double *A_log,
                          const double *dt_bias, const double *h0,
                          const int64_t *cu_seqlens, int n_seq, int H, int dk, int dv,
                          double scale, const int32_t *chains, int n_chains,
                          double *o, double *hT, double *h_chunks, int C, int n_threads)
{
    if (!h_chunks) return -1;
    return oracle_fwd(q, k, v, a, b, A_log, dt_bias, h0, cu_seqlens, n_seq, H, dk, dv, scale,
                      chains, n_chains, o, hT, h_chunks, C, n_threads);
}

/*
 * T tokens per row over a state pool, each token one step of [SGL-PR]'s
 * decode update, in token order (the fused recurrent form with a token loop
 * that the page gives for extend and speculative verification):
 *   qkv  : [B, T, 2*H*K + HV*V]  (q heads, then k heads, then v heads)
 *   a    : [B, T, HV*K]   b : [B, T, HV]   A_log : [HV]   dt_bias : [HV*K]
 *   pool : [P, HV, V, K] updated in place for the referenced slots
 *   state_idx : [B]; a negative entry is a pad: zero outputs, no state write.
 *   o    : [B, T, HV, V]
 * Value head hv reads q/k head hv / (HV / H).  T = 1 is the decode step.
 */
int kda_oracle_extend(const double *qkv, const double *a, const double *b,
                      const double *A_log, const double *dt_bias, double *pool,
                      const int64_t *state_idx, int B, int T, int H, int HV, int K, int V,
                      int64_t P, double scale, int l2norm, double *o, int n_threads)
{
    if (!qkv || !a || !b || !A_log || !dt_bias || !pool || !state_idx || !o) return -1;
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || HV % H != 0 || K <= 0 || V <= 0) return -1;
    const int64_t row = 2 * (int64_t)H * K + (int64_t)HV * V;
    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 4) reduction(| : err)
#endif
    for (int i = 0; i < B * HV; ++i) {
        const int n = i / HV, hv = i % HV, hq = hv / (HV / H);
        const int64_t idx = state_idx[n];
        if (idx < 0) {
            for (int t = 0; t < T; ++t) {
                double *on = o + (((int64_t)n * T + t) * HV + hv) * V;
                for (int r = 0; r < V; ++r) on[r] = 0.0;
            }
            continue;
        }
        if (idx >= P) { err |= 1; continue; }
        double *buf = (double *)malloc(sizeof(double) * (3 * (size_t)K + V));
        if (!buf) { err |= 1; continue; }
        double *qv = buf, *kv = buf + K, *eg = buf + 2 * K, *u = buf + 3 * K;
        double *S = pool + (idx * HV + hv) * (int64_t)V * K;
        const double A_exp = exp(A_log[hv]);
        for (int t = 0; t < T; ++t) {
            const int64_t tok = (int64_t)n * T + t;
            const double *x = qkv + tok * row;
            double *on = o + (tok * HV + hv) * V;
            for (int c = 0; c < K; ++c) {
                qv[c] = x[(int64_t)hq * K + c];
                kv[c] = x[(int64_t)H * K + (int64_t)hq * K + c];
            }
            if (l2norm) {
                double sq = 0.0, sk = 0.0;
                for (int c = 0; c < K; ++c) { sq += qv[c] * qv[c]; sk += kv[c] * kv[c]; }
                const double nq = sqrt(sq + 1e-6), nk = sqrt(sk + 1e-6);
                for (int c = 0; c < K; ++c) { qv[c] /= nq; kv[c] /= nk; }
            }
            for (int c = 0; c < K; ++c) qv[c] *= scale;
            for (int c = 0; c < K; ++c)
                eg[c] = exp(-A_exp * softplus_exact(a[tok * HV * K + (int64_t)hv * K + c] +
                                                    dt_bias[(int64_t)hv * K + c]));
            const double beta = sigmoid(b[tok * HV + hv]);
            const double *vv = x + 2 * (int64_t)H * K + (int64_t)hv * V;
            for (int r = 0; r < V; ++r) {
                double *Sr = S + (int64_t)r * K;
                double w = 0.0;
                for (int c = 0; c < K; ++c) { Sr[c] *= eg[c]; w += Sr[c] * kv[c]; }
                u[r] = beta * (vv[r] - w);
            }
            for (int r = 0; r < V; ++r) {
                double *Sr = S + (int64_t)r * K;
                double acc = 0.0;
                for (int c = 0; c < K; ++c) { Sr[c] += u[r] * kv[c]; acc += Sr[c] * qv[c]; }
                on[r] = acc;
            }
        }
        free(buf);
    }
    (void)n_threads;
    return err ? -1 : 0;
}

/*
 * One T=1 decode step over a state pool, as in [SGL-PR]:
 *   qkv  : [B, 2*H*K + HV*V]  (q heads, then k heads, then v heads)
 *   a    : [B, HV*K]   b : [B, HV]   A_log : [HV]   dt_bias : [HV*K]
 *   pool : [P, HV, V, K] updated in place for the referenced slots
 *   state_idx : [B]; a negative entry is a pad: zero output row, no state write.
 *   o    : [B, HV, V]
 * Value head hv reads q/k head hv / (HV / H).
 */
int kda_oracle_decode(const double *qkv, const double *a, const double *b,
                      const double *A_log, const double *dt_bias, double *pool,
                      const int64_t *state_idx, int B, int H, int HV, int K, int V,
                      int64_t P, double scale, int l2norm, double *o, int n_threads)
{
    return kda_oracle_extend(qkv, a, b, A_log, dt_bias, pool, state_idx, B, 1, H, HV, K, V, P,
                             scale, l2norm, o, n_threads);
}

/*
 * Short causal convolution before decode, one new input per row ([SGL-PR],
 * backend integration: causal_conv1d_update on the packed projections with
 * activation "silu" and per-row conv-state slots given by the same cache
 * indices as the recurrent state).  The page names the call without defining
 * it; this is the plain depthwise causal convolution of width W whose state
 * holds each channel's last W-1 inputs.  Per channel c of row n with slot
 * idx = state_idx[n] >= 0:
 *   window = (cs[idx, 0, c], ..., cs[idx, W-2, c], x[n, c])    oldest first
 *   y[n, c] = silu(bias[c] + sum_w weight[c, w] * window[w]),  silu(z) = z / (1 + e^-z)
 *   cs[idx, :, c] <- window[1 .. W-1]
 * A pad row (idx < 0) gives y = 0 and writes no state.
 *   x [B, D]   conv_state [P, W-1, D]   weight [D, W]   bias [D] or NULL   y [B, D]
 */
int kda_oracle_conv_update(const double *x, double *conv_state, const double *weight,
                           const double *bias, const int64_t *state_idx, int B, int D, int W,
                           int64_t P, double *y)
{
    if (!x || !weight || !state_idx || !y || (W > 1 && !conv_state)) return -1;
    if (B < 0 || D <= 0 || W < 1) return -1;
    double *win = (double *)malloc(sizeof(double) * (size_t)W);
    if (!win) return -1;
    int err = 0;
    for (int n = 0; n < B; ++n) {
        const int64_t idx = state_idx[n];
        double *yn = y + (int64_t)n * D;
        if (idx < 0) {
            for (int c = 0; c < D; ++c) yn[c] = 0.0;
            continue;
        }
        if (idx >= P) { err = 1; continue; }
        double *cs = conv_state ? conv_state + idx * (int64_t)(W - 1) * D : NULL;
        for (int c = 0; c < D; ++c) {
            for (int w = 0; w < W - 1; ++w) win[w] = cs[(int64_t)w * D + c];
            win[W - 1] = x[(int64_t)n * D + c];
            double z = bias ? bias[c] : 0.0;
            for (int w = 0; w < W; ++w) z += weight[(int64_t)c * W + w] * win[w];
            yn[c] = z / (1.0 + exp(-z));
            for (int w = 0; w < W - 1; ++w) cs[(int64_t)w * D + c] = win[w + 1];
        }
    }
    free(win);
    return err ? -1 : 0;
}
