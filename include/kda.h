/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library.
 *
 * Entry points, all hand-written HIP for CDNA4:
 *
 *   kda_chunk_fwd       chunkwise prefill over dense or packed variable-length
 *                       sequences, returning the outputs and the final states;
 *   kda_chunk_o         the materialised form's chunk-parallel output pass;
 *   kda_backward        gradients of the prefill with respect to every input,
 *                       from the states kda_chunk_fwd_states stores;
 *   kda_chunk_fwd_pool  the same prefill with the states in a decode state
 *                       pool (read and updated in place through slot indices);
 *   kda_chunk_fwd_states  the same prefill that also stores the state entering
 *                       every chunk (the materialised form; its chunk-parallel
 *                       output pass is kda_chunk_fwd over chunk-length
 *                       sequences started from those states);
 *   kda_decode_step     one fused T=1 decode step over a pool of states;
 *   kda_decode_extend   T tokens per row applied to the pool states in one
 *                       launch (short extends, speculative verification);
 *   kda_conv_decode_step  the short causal convolution before decode fused
 *                       with the decode step.
 *
 * The method ([TL-KDA] section 1): per (sequence, head), with the state S
 * stored as (d_v, d_k),
 *     S_t = S_{t-1} Diag(e^{g_t}) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t (scale * q_t),
 * with the gate and beta of [SGL-PR]:
 *     g_t = -exp(A_log[h]) * softplus(g_raw_t + dt_bias[h, :]),
 *     beta_t = sigmoid(beta_raw_t).
 *
 * Sources, cited by page title and section:
 *   [TL-KDA]  "TileLang 实战：KDA 从零到一 -- Chunked 线性注意力"
 *   [LA-06]   "06 · linear 路线（一）：kernel trick、RNN 等价与三种计算形式"
 *   [FKDA-LM] "FlashKDA 里的 L 矩阵和 Mqk 矩阵是什么"
 *   [SGL-PR]  "SGLang PR #26586 (KDA packed decode)"
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller, contiguous
 *     and row-major as documented per argument, aligned to 16 bytes.
 *   - Arguments are validated on the host before anything is launched; on a
 *     validation error the call returns a negative kda_status and launches
 *     nothing.  After a launch, a launch failure is reported as KDA_ERR_HIP.
 *   - The calls enqueue work on `stream` and return without synchronising;
 *     results are ready once the caller synchronises the stream.  A kernel
 *     fault surfaces at that synchronisation.
 *   - No entry point allocates memory.  kda_backward takes a caller-owned
 *     workspace (size from kda_backward_workspace_bytes); the prefill entry
 *     points take an optional one (size from kda_chunk_fwd_workspace_bytes).
 *     Calls on different streams may overlap as long as they do not share a
 *     workspace: no kernel keeps state between launches or shares memory with
 *     another launch.
 *   - Invalid input that lives in device memory (a pool slot index >= P) is
 *     handled by the kernels as documented per entry point and recorded in a
 *     sticky per-device error word, which kda_device_check() reads and clears.
 *   - Results are deterministic (no atomics in the arithmetic): the same
 *     inputs give bitwise-identical outputs.
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    KDA_ERR_UNSUPPORTED = -3, /* valid but not built (head dim, chunk size, dtype) */
    KDA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    KDA_ERR_HIP = -5,         /* the HIP runtime reported an error at launch */
    KDA_ERR_SLOT = -6,        /* a kernel met a pool slot index >= P (see kda_device_check) */
    KDA_ERR_SCRATCH = -7      /* kda_chunk_fwd_noalloc: more workspace needed than its scratch holds */
} kda_status;

typedef enum {
    KDA_F32 = 0,   /* float32 activations */
    KDA_BF16 = 1   /* bfloat16 activations (round to nearest even on output) */
} kda_dtype;

/*
 * kda_chunk_fwd -- chunkwise KDA prefill ([FKDA-LM] paragraphs "30秒速览",
 * "L 矩阵的构造", "Mqk 矩阵的构造", "为什么 CHUNK16", "K2 内核如何消费";
 * sequence loop inside the workgroup as in [TL-KDA] section 6.4).
 *
 * Per chunk of C = 16 tokens of one (sequence, head), G the chunk-local
 * cumulative gate and S the state as (dk, dv):
 *   L  (16x16, strictly lower) and Mqk (16x16, lower incl. diagonal) by MFMA,
 *   INV = (I - L)^{-1} by Neumann squaring,
 *   U = INV beta (v - (k e^G) S) = u' - w S with u' = INV beta v, w = INV beta (k e^G),
 *   O = scale ((q e^G) S + Mqk U),
 *   S <- Diag(e^{G_C}) S + (k e^{G_C - G})^T U   (after the output).
 * The state-independent part of every chunk ("prep": gate, decayed operands,
 * L, Mqk, INV, w) is built by prep waves and the recurrence by consumer
 * waves that hold the fp32 state columns in MFMA accumulators.  Two forms:
 *   - one pass (no workspace needed): one workgroup carries one (sequence,
 *     head, group of state columns) through the whole sequence, its prep waves
 *     three chunks ahead of its consumer waves, hand-over through LDS.  With
 *     fewer chains than compute units the columns are split over several
 *     workgroups, each repeating the prep;
 *   - two passes (when `workspace` holds at least
 *     kda_chunk_fwd_workspace_bytes() bytes and the (sequence, head) chains are
 *     fewer than the compute units): a fully parallel pass writes every
 *     chunk's consumer operands into the workspace, then one wave per
 *     (sequence, head, 16 state columns), in workgroups of one or two such
 *     waves and a loader wave, runs the recurrence from them.
 * Both give the same results up to rounding order.  No workgroup waits on
 * another.  Packed sequences are scheduled longest first (up to 128).
 *
 * Layout (T_all = B*T for dense input, = T for packed input):
 *   q, k, g_raw : [T_all, H, dk]   activation dtype, q and k expected
 *                                  L2-normalised by the caller
 *   v, o        : [T_all, H, dv]   activation dtype
 *   beta_raw    : [T_all, H]       activation dtype (pre-sigmoid)
 *   A_log       : [H]              float32
 *   dt_bias     : [H, dk]          float32
 *   h0          : [n_seq, H, dv, dk] float32 initial states, or NULL for zero
 *   h_T         : [n_seq, H, dv, dk] float32 final states, or NULL to skip
 *   cu_seqlens  : NULL for dense input (n_seq must equal B, every sequence
 *                 has T tokens), or [n_seq + 1] int32 token offsets read on
 *                 the device (then B must be 1 and cu_seqlens[n_seq] == T;
 *                 the offsets must be non-decreasing -- not checked on the
 *                 host, because they live in device memory).
 *   chunk       : must be 16.
 *   dk, dv      : 64 or 128 each.
 *   scale       : multiplies q (usually dk^-1/2).
 *   dtype       : KDA_BF16 (dk, dv in {64, 128}) or KDA_F32 (dk = 64).
 *   workspace   : NULL, or caller-owned device memory of workspace_bytes
 *                 bytes (contents on entry do not matter; overwritten); see
 *                 kda_chunk_fwd_workspace_bytes.  Only the bf16 form uses it.
 * A zero-length sequence leaves its outputs untouched and writes h_T = h0
 * (or zeros).  T == 0 is accepted and launches nothing except the h_T copy.
 * Returns KDA_OK or a negative kda_status.
 */
int kda_chunk_fwd(const void *q, const void *k, const void *v,
                  const void *g_raw, const void *beta_raw,
                  const float *A_log, const float *dt_bias,
                  const float *h0, const int32_t *cu_seqlens, int chunk,
                  void *o, float *h_T,
                  int B, int T, int H, int dk, int dv, int n_seq,
                  float scale, kda_dtype dtype,
                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd_workspace_bytes -- bytes of workspace that let the prefill
 * entry points use their two-pass form: 13,824 (dk = 128) or 7,424 (dk = 64)
 * per chunk row and head, for ceil(T/16) * B chunk rows of dense input
 * (packed = 0) or ceil(T/16) + n_seq rows of packed input (packed != 0,
 * an upper bound: the lengths live in device memory).  0 for invalid sizes.
 */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int n_seq, int packed);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, layouts and results as kda_chunk_fwd
 * (bitwise: it launches the same kernels), without a workspace argument.
 * Where kda_chunk_fwd would take its two-pass form, this entry point uses a
 * fixed device array of KDA_NOALLOC_SCRATCH_BYTES (64 MiB) as the workspace,
 * and nothing else: no allocation, no library routine that allocates.  Each
 * GPU the library runs on holds one such array until the process ends; the
 * first call on a device looks up its address.  All calls on one GPU share
 * that array, so calls that overlap on one GPU (two streams, two threads)
 * race and must be serialised by the caller.  The array needs no clearing:
 * every workspace byte a call reads was written earlier in the same call.
 * Returns KDA_ERR_SCRATCH, launching nothing, when the two-pass form would
 * need more than the array (kda_chunk_fwd_workspace_bytes() above
 * KDA_NOALLOC_SCRATCH_BYTES: at d_k = 128, 4,854 chunk rows x heads); else as
 * kda_chunk_fwd.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
int kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                          const void *g_raw, const void *beta_raw,
                          const float *A_log, const float *dt_bias,
                          const float *h0, const int32_t *cu_seqlens, int chunk,
                          void *o, float *h_T,
                          int B, int T, int H, int dk, int dv, int n_seq,
                          float scale, kda_dtype dtype, hipStream_t stream);

/*
 * kda_chunk_fwd_states -- kda_chunk_fwd that also writes the state entering
 * every chunk: the materialised form of [LA-06] (chunkwise form: the states at
 * chunk boundaries are stored, then the outputs are a chunk-parallel pass) and
 * of [TL-KDA] section 6 (a state snapshot per chunk).
 *
 *   h_chunks : [N_chunks, H, dv, dk] float32, written: row
 *              (chunks of the sequences before s) + c holds the state of
 *              (sequence s, head) before its chunk c (row 0 of a sequence = its
 *              h0, or zeros), in the layout of h_T.  N_chunks = sum over
 *              sequences of ceil(len / 16) (dense input: B * ceil(T / 16)).
 *              The caller sizes it (the lengths of packed input live in device
 *              memory and are not checked).
 * All other arguments, outputs and errors are those of kda_chunk_fwd; the
 * outputs are bitwise those of kda_chunk_fwd.  h_chunks is fp32 and exact, so
 * kda_chunk_fwd over the chunks as sequences of their own (cu_seqlens at every
 * chunk boundary, or for dense input with T % 16 == 0 the same buffers viewed
 * as B*T/16 sequences of 16 tokens) with h0 = h_chunks reproduces o bitwise,
 * every chunk an independent chain.
 */
int kda_chunk_fwd_states(const void *q, const void *k, const void *v,
                         const void *g_raw, const void *beta_raw,
                         const float *A_log, const float *dt_bias,
                         const float *h0, const int32_t *cu_seqlens, int chunk,
                         void *o, float *h_T, float *h_chunks,
                         int B, int T, int H, int dk, int dv, int n_seq,
                         float scale, kda_dtype dtype,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_o -- the chunk-parallel output pass of the materialised form
 * ([LA-06] chunkwise form; [TL-KDA] section 6): every chunk's outputs from the
 * state entering it, each chunk independently.  Per chunk of 16 tokens with
 * S0 = h_chunks[row] (G the chunk-local cumulative gate):
 *   U = (I - L)^{-1} beta (v - (k e^G) S0^T),  o = scale ((q e^G) S0^T + Mqk U),
 * L and Mqk as in kda_chunk_fwd (in fp32, their factors e^{G_i - G_j} as
 * running products of the tokens' decays).
 * Inputs as given to kda_chunk_fwd_states (q, k, v, g_raw, beta_raw, A_log,
 * dt_bias, cu_seqlens, B, T, H, n_seq, scale) and its h_chunks output;
 * n_chunks = its row count (sum of ceil(len / 16); B * ceil(T / 16) for
 * dense input, checked; with cu_seqlens the device-side lengths decide, and
 * rows past them are skipped).  Writes o [T_all, H, dv].  Built for bfloat16 with
 * dk = dv = 128 (else KDA_ERR_UNSUPPORTED; kda_chunk_fwd over chunk-length
 * sequences with h0 = h_chunks is the general route and reproduces
 * kda_chunk_fwd bitwise; this pass agrees with it to bf16 rounding).
 * Returns KDA_OK or a negative kda_status.
 */
int kda_chunk_o(const void *q, const void *k, const void *v,
                const void *g_raw, const void *beta_raw,
                const float *A_log, const float *dt_bias,
                const float *h_chunks, const int32_t *cu_seqlens, void *o,
                int B, int T, int H, int dk, int dv, int n_seq, int n_chunks,
                float scale, kda_dtype dtype, hipStream_t stream);

/*
 * kda_backward -- gradients of the forward of kda_chunk_fwd for a loss whose
 * gradients with respect to o and to the final states are do and dh_T: the
 * backward pass of [LA-06] (chunkwise form: a reverse loop over chunks from
 * the states stored at chunk boundaries).  Per chunk of 16 tokens, with S
 * the state entering it, dS' the gradient with respect to the state leaving
 * it (S as dk x dv), dO_s = scale do and the chunk's forward as in
 * kda_chunk_fwd, U = T beta (v - k~ S), O = scale (q~ S + Mqk U),
 * S' = D S + k^r^T U, where G is the cumulative gate, k~ = k e^G,
 * q~ = q e^G, k^r = k e^{G_C - G}, D = Diag(e^{G_C}), T = (I - L)^{-1} and
 * w = T beta k~:
 *   dU = k^r dS' + Mqk^T dO_s;  dS = D dS' + q~^T dO_s - w^T dU
 * (the sequential step, a reverse recurrence over chunks), then, for every
 * chunk in parallel, dv, dbeta, dq, dk and dG from S, dS', dU and the chunk's
 * pair terms; dg is the reverse cumulative sum of dG within the chunk, and
 * the chain rule through g = -exp(A_log) softplus(g_raw + dt_bias) and
 * beta = sigmoid(beta_raw) gives dg_raw, ddt_bias, dA_log and dbeta_raw;
 * dh0 is the gradient before the first chunk.
 *
 * Inputs: q, k, v, g_raw, beta_raw, A_log, dt_bias, cu_seqlens, scale,
 * B, T, H, n_seq and dtype exactly as given to kda_chunk_fwd_states;
 *   h_chunks  : its [N_chunks, H, dv, dk] float32 output for those inputs
 *               and h0;
 *   do_       : [T_all, H, dv] activation dtype;
 *   dh_T      : [n_seq, H, dv, dk] float32, or NULL for zero.
 * Outputs (written; NULL is allowed for dA_log, ddt_bias and dh0):
 *   dq, dk, dg_raw : [T_all, H, dk], dv : [T_all, H, dv], dbeta_raw : [T_all, H]
 *                    in the activation dtype;
 *   dA_log [H], ddt_bias [H, dk], dh0 [n_seq, H, dv, dk] float32.
 * workspace: device memory of at least kda_backward_workspace_bytes() bytes,
 * owned by the caller (55,812 bytes per (chunk of 16 tokens, head) for the
 * reverse chain's operands, the per-chunk gradient rows and parameter sums,
 * plus H * 64 * 129 floats); its contents on entry do not matter.
 * Built for dk = dv = 128 with bfloat16 activations (those of the d = 128
 * forward; other shapes and float32 return KDA_ERR_UNSUPPORTED).  The result
 * is deterministic (no atomics).  Returns KDA_OK or a negative kda_status.
 */
size_t kda_backward_workspace_bytes(int n_seq, int H, int dk, int dv, int64_t total_tokens);
int kda_backward(const void *q, const void *k, const void *v,
                 const void *g_raw, const void *beta_raw,
                 const float *A_log, const float *dt_bias,
                 const float *h_chunks, const int32_t *cu_seqlens,
                 const void *do_, const float *dh_T,
                 void *dq, void *dk, void *dv, void *dg_raw, void *dbeta_raw,
                 float *dA_log, float *ddt_bias, float *dh0,
                 void *workspace, size_t workspace_bytes,
                 int B, int T, int H, int dk_, int dv_, int n_seq,
                 float scale, kda_dtype dtype, hipStream_t stream);

/*
 * kda_chunk_fwd_pool -- the prefill of kda_chunk_fwd with the states kept in a
 * decode state pool instead of dense h0 / h_T arrays, so that a prefill (or an
 * extend of a running sequence) and the decode steps of kda_decode_step share
 * one state store ([SGL-PR]: the packed decode addresses its states through
 * the pool indices, a negative index marking a pad slot).
 *
 * Sequence s starts from state_pool[state_idx[s]] and its final state is
 * written back to that slot in place; state_idx[s] < 0 starts from the zero
 * state and keeps no final state.  Everything else (layouts, chunk, head
 * dims, dtype, cu_seqlens, scale) is as for kda_chunk_fwd.
 *
 *   state_pool : [P, H, dv, dk] float32 -- the layout of kda_decode_step's
 *                pool with HV = H, V = dv, K = dk; read and updated in place.
 *   state_idx  : [n_seq] int32 slot per sequence (device memory).  Live
 *                entries must be distinct and < P (duplicates race; not
 *                checked on the host because the indices live in device
 *                memory).  An entry >= P is treated like a negative one
 *                (zero start, no final state, no pool access) and recorded
 *                for kda_device_check.
 * Returns KDA_OK or a negative kda_status (KDA_ERR_SHAPE for P <= 0,
 * KDA_ERR_NULL for a missing pool or index array).
 */
int kda_chunk_fwd_pool(const void *q, const void *k, const void *v,
                       const void *g_raw, const void *beta_raw,
                       const float *A_log, const float *dt_bias,
                       float *state_pool, const int32_t *state_idx,
                       const int32_t *cu_seqlens, int chunk, void *o,
                       int B, int T, int H, int dk, int dv, int n_seq, int P,
                       float scale, kda_dtype dtype,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_decode_step -- fused T=1 KDA decode over a state pool ([SGL-PR],
 * section "实现拆解" item 1 and the packed decode kernel snippet).
 *
 * For every row n and value head hv (q/k head hq = hv / (HV / H)):
 *   idx = state_idx[n]; if idx < 0 (pad slot): o[n, hv, :] = 0, no state access.
 *   q, k taken from the packed row, optionally L2-normalised
 *   (x / sqrt(sum x^2 + 1e-6)), then q *= scale;
 *   g = -exp(A_log[hv]) * softplus(a[n, hv, :] + dt_bias[hv, :]), beta = sigmoid(b[n, hv]);
 *   S' = S Diag(e^g); u = beta (v - S' k); S = S' + u k^T; o = S q.
 * The state slot is read and written in place, in one pass over its bytes.
 *
 * Layout:
 *   qkv        : [B, 2*H*K + HV*V] bf16  (all q heads, then all k heads, then v heads)
 *   a          : [B, HV*K] bf16     b : [B, HV] bf16
 *   A_log      : [HV] float32       dt_bias : [HV*K] float32
 *   state_pool : [P, HV, V, K] float32, updated in place
 *   state_idx  : [B] int32 slot per row; < 0 marks a pad row.  Live entries
 *                must be distinct (duplicates race; not checked on the host
 *                because the indices live in device memory).  An entry >= P
 *                is handled as a pad row (zero output, no state access) and
 *                recorded for kda_device_check.
 *   o          : [B, HV, V] bf16
 *   K, V       : 128 each.  HV % H == 0.
 *   flags      : bit 0 set = L2-normalise q and k in the kernel.
 * Returns KDA_OK or a negative kda_status.
 */
int kda_decode_step(const void *qkv, const void *a, const void *b,
                    const float *A_log, const float *dt_bias,
                    float *state_pool, const int32_t *state_idx, void *o,
                    int B, int H, int HV, int K, int V, int P,
                    float scale, int flags, hipStream_t stream);

#define KDA_DECODE_L2NORM 1

/*
 * kda_decode_extend -- T tokens per row through the same update as
 * kda_decode_step, in token order, in one launch: the fused recurrent form
 * with a token loop that [SGL-PR] (section "实现拆解" and the review notes)
 * gives for extends and speculative (EAGLE) verification, which do not go
 * through the T=1 packed decode.  Each live slot is read once, carried
 * through the T tokens and written once, holding the state after token T-1.
 * With T = 1 the results are bitwise those of kda_decode_step.
 *
 * Layout (token t of row n is entry n*T + t of the token axis):
 *   qkv        : [B, T, 2*H*K + HV*V] bf16
 *   a          : [B, T, HV*K] bf16      b : [B, T, HV] bf16
 *   A_log      : [HV] float32           dt_bias : [HV*K] float32
 *   state_pool : [P, HV, V, K] float32, updated in place
 *   state_idx  : [B] int32 slot per row; < 0 marks a pad row (all T outputs
 *                zero, no state access).  Live entries must be distinct (not
 *                checked on the host: device memory); an entry >= P is
 *                handled as a pad row and recorded for kda_device_check.
 *   o          : [B, T, HV, V] bf16; o[n, t] is read from the state after
 *                token t.
 *   K, V       : 128 each.  HV % H == 0.  T >= 0 (T == 0 launches nothing).
 *   flags      : bit 0 set = L2-normalise q and k in the kernel.
 * Returns KDA_OK or a negative kda_status.
 */
int kda_decode_extend(const void *qkv, const void *a, const void *b,
                      const float *A_log, const float *dt_bias,
                      float *state_pool, const int32_t *state_idx, void *o,
                      int B, int T, int H, int HV, int K, int V, int P,
                      float scale, int flags, hipStream_t stream);

/*
 * kda_conv_decode_step -- the short causal convolution that produces the
 * packed q/k/v row, fused with one decode step ([SGL-PR], backend
 * integration: causal_conv1d_update with activation silu on mixed_qkv, its
 * conv-state slots addressed by the same cache indices as the recurrent
 * state, then the packed decode; there they are two launches).
 *
 * For every live row n (slot idx = state_idx[n]) and channel c of the packed
 * row (D = 2*H*K + HV*V channels):
 *   window = (conv_state[idx, 0, c], ..., conv_state[idx, W-2, c], mixed_qkv[n, c])
 *   y[c]   = silu(conv_bias[c] + sum_w conv_weight[c, w] * window[w]),
 *   conv_state[idx, :, c] <- window[1 .. W-1],
 * computed in fp32, and y (not rounded) is the qkv row of kda_decode_step's
 * update, which then updates state_pool[idx] and writes o[n].  A pad row
 * (idx < 0) gets zero outputs and touches neither state; so does a row with
 * idx >= P, which is also recorded for kda_device_check.
 *
 * Layout:
 *   mixed_qkv   : [B, D] bf16 (q heads, k heads, v heads, before the conv)
 *   conv_state  : [P, W-1, D] bf16, updated in place (oldest input first)
 *   conv_weight : [D, W] bf16       conv_bias : [D] bf16, or NULL for none
 *   a, b, A_log, dt_bias, state_pool, state_idx, o, scale, flags: as in
 *                 kda_decode_step (P slots for both states).
 *   K, V        : 128 each.  W: 2, 3 or 4.  HV % H == 0 and HV/H <= 126.
 * Returns KDA_OK or a negative kda_status.
 */
int kda_conv_decode_step(const void *mixed_qkv, void *conv_state,
                         const void *conv_weight, const void *conv_bias,
                         const void *a, const void *b,
                         const float *A_log, const float *dt_bias,
                         float *state_pool, const int32_t *state_idx, void *o,
                         int B, int H, int HV, int K, int V, int W, int P,
                         float scale, int flags, hipStream_t stream);

/*
 * kda_device_check -- synchronise `stream`, then read and clear the current
 * device's error word: KDA_ERR_SLOT if, since the last check, a kernel of
 * this library met a pool slot index >= P (kda_decode_step,
 * kda_decode_extend, kda_conv_decode_step, kda_chunk_fwd_pool; the row was
 * handled as a pad), else KDA_OK.  KDA_ERR_HIP if the synchronisation or the
 * copy fails.
 */
int kda_device_check(hipStream_t stream);

/* Human-readable name of a kda_status value (static string). */
const char *kda_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
