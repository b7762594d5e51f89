/* Sanitizer driver for the fp64 oracle (test infrastructure): runs every
 * entry point of kda_oracle.c on small seeded inputs, including the edge
 * cases the tests use (zero-length and ragged sequences, pad rows, a chain
 * subset, a width-1 convolution, invalid arguments), so that an
 * AddressSanitizer / UndefinedBehaviorSanitizer build sees each code path.
 * Prints "oracle sanitizer driver ok" and exits 0 when every call returned
 * what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_fwd(const double *q, const double *k, const double *v, const double *a, const double *b,
                   const double *A_log, const double *dt_bias, const double *h0, const int64_t *cu_seqlens,
                   int n_seq, int H, int dk, int dv, double scale, const int32_t *chains, int n_chains,
                   double *o, double *hT, int n_threads);
int kda_oracle_fwd_states(const double *q, const double *k, const double *v, const double *a, const double *b,
                          const double *A_log, const double *dt_bias, const double *h0,
                          const int64_t *cu_seqlens, int n_seq, int H, int dk, int dv, double scale,
                          const int32_t *chains, int n_chains, double *o, double *hT, double *h_chunks, int C,
                          int n_threads);
int kda_oracle_extend(const double *qkv, const double *a, const double *b, const double *A_log,
                      const double *dt_bias, double *pool, const int64_t *state_idx, int B, int T, int H, int HV,
                      int K, int V, int64_t P, double scale, int l2norm, double *o, int n_threads);
int kda_oracle_decode(const double *qkv, const double *a, const double *b, const double *A_log,
                      const double *dt_bias, double *pool, const int64_t *state_idx, int B, int H, int HV, int K,
                      int V, int64_t P, double scale, int l2norm, double *o, int n_threads);
int kda_oracle_conv_update(const double *x, double *conv_state, const double *weight, const double *bias,
                           const int64_t *state_idx, int B, int D, int W, int64_t P, double *y);

static uint64_t rng = 88172645463325252ull;
static double rnd(void) {   /* xorshift64, uniform in [-1, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double *vec(size_t n) {
    double *x = (double *)malloc(n * sizeof(double));
    if (!x) exit(2);
    for (size_t i = 0; i < n; ++i) x[i] = rnd();
    return x;
}
static int fails = 0;
static void expect(int got, int want, const char *what) {
    if (got != want) {
        printf("FAIL %s: returned %d, expected %d\n", what, got, want);
        ++fails;
    }
}
static int finite_all(const double *x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void) {
    /* prefill: packed lengths 0, 1, 16, 17, 5 (tokens 39), H = 2, dk = 8, dv = 6 */
    const int H = 2, dk = 8, dv = 6, n_seq = 5;
    const int64_t cu[6] = {0, 0, 1, 17, 34, 39};
    const int T = 39;
    double *q = vec((size_t)T * H * dk), *k = vec((size_t)T * H * dk), *v = vec((size_t)T * H * dv);
    double *a = vec((size_t)T * H * dk), *b = vec((size_t)T * H), *A_log = vec(H), *dt = vec((size_t)H * dk);
    double *h0 = vec((size_t)n_seq * H * dv * dk);
    double *o = (double *)calloc((size_t)T * H * dv, sizeof(double));
    double *hT = (double *)calloc((size_t)n_seq * H * dv * dk, sizeof(double));
    const int n_chunks = 0 + 1 + 1 + 2 + 1;   /* ceil(len / 16) per sequence */
    double *hc = (double *)calloc((size_t)n_chunks * H * dv * dk, sizeof(double));
    expect(kda_oracle_fwd(q, k, v, a, b, A_log, dt, h0, cu, n_seq, H, dk, dv, 0.35, NULL, 0, o, hT, 2), 0, "fwd");
    expect(kda_oracle_fwd(q, k, v, a, b, A_log, dt, NULL, cu, n_seq, H, dk, dv, 0.35, NULL, 0, o, hT, 1), 0,
           "fwd without h0");
    const int32_t chains[3] = {1, 6, 9};
    expect(kda_oracle_fwd(q, k, v, a, b, A_log, dt, h0, cu, n_seq, H, dk, dv, 0.35, chains, 3, o, hT, 2), 0,
           "fwd chain subset");
    expect(kda_oracle_fwd_states(q, k, v, a, b, A_log, dt, h0, cu, n_seq, H, dk, dv, 0.35, NULL, 0, o, hT, hc, 16, 2),
           0, "fwd_states");
    expect(kda_oracle_fwd_states(q, k, v, a, b, A_log, dt, h0, cu, n_seq, H, dk, dv, 0.35, NULL, 0, o, hT, NULL, 16,
                                 1), -1, "fwd_states without h_chunks");
    if (!finite_all(o, (size_t)T * H * dv) || !finite_all(hT, (size_t)n_seq * H * dv * dk)) {
        printf("FAIL fwd: non-finite output\n");
        ++fails;
    }

    /* decode and extend: B = 5 rows (one pad), H = 1, HV = 2, K = 4, V = 3, pool of 7 */
    const int B = 5, Hd = 1, HV = 2, K = 4, V = 3, Te = 3;
    const int64_t P = 7, idx[5] = {3, -1, 0, 6, 2};
    const int D = 2 * Hd * K + HV * V;
    double *qkv = vec((size_t)B * Te * D), *ad = vec((size_t)B * Te * HV * K), *bd = vec((size_t)B * Te * HV);
    double *Ad = vec(HV), *dtd = vec((size_t)HV * K), *pool = vec((size_t)P * HV * V * K);
    double *od = (double *)calloc((size_t)B * Te * HV * V, sizeof(double));
    expect(kda_oracle_decode(qkv, ad, bd, Ad, dtd, pool, idx, B, Hd, HV, K, V, P, 0.5, 1, od, 2), 0, "decode");
    expect(kda_oracle_extend(qkv, ad, bd, Ad, dtd, pool, idx, B, Te, Hd, HV, K, V, P, 0.5, 0, od, 2), 0, "extend");

    /* convolution: widths 4 and 1 (no state), with and without bias */
    const int Dc = 10, W = 4;
    double *x = vec((size_t)B * Dc), *cs = vec((size_t)P * (W - 1) * Dc), *w = vec((size_t)Dc * W);
    double *bias = vec(Dc), *y = (double *)calloc((size_t)B * Dc, sizeof(double));
    expect(kda_oracle_conv_update(x, cs, w, bias, idx, B, Dc, W, P, y), 0, "conv W=4");
    expect(kda_oracle_conv_update(x, cs, w, NULL, idx, B, Dc, W, P, y), 0, "conv W=4 no bias");
    expect(kda_oracle_conv_update(x, NULL, w, bias, idx, B, Dc, 1, P, y), 0, "conv W=1");
    expect(kda_oracle_conv_update(NULL, cs, w, bias, idx, B, Dc, W, P, y), -1, "conv without x");

    free(q); free(k); free(v); free(a); free(b); free(A_log); free(dt); free(h0); free(o); free(hT); free(hc);
    free(qkv); free(ad); free(bd); free(Ad); free(dtd); free(pool); free(od);
    free(x); free(cs); free(w); free(bias); free(y);
    if (fails) return 1;
    printf("oracle sanitizer driver ok\n");
    return 0;
}
