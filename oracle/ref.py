"""Plain numpy fp64 references for KDA -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  Nothing here is shared with the HIP library.

Sources (web pages, cited by title and section):
  [TL-KDA] "TileLang 实战：KDA 从零到一 -- Chunked 线性注意力"
           section 1 (recurrence and its (d_v, d_k) state layout),
           section 2.1 (level-1 chunk identity O_c = Q_c S_prev + tril(Q_c K_c^T) V_c),
           section 3.1 / 3.2 (reference A token loop, reference B cumsum + right shift),
           section 3.4 (consistency table, deliberate right-shift bug),
           section 6.4.2 (reference D: sequence loop over DV slabs, update after write-back).
  [LA-06]  "06 · linear 路线（一）：kernel trick、RNN 等价与三种计算形式"
           section 3.1 (parallel form ((Q K^T) ⊙ M) V), 3.2 (recurrent form),
           3.3 (chunkwise form, update after output).
  [FKDA-LM] "FlashKDA 里的 L 矩阵和 Mqk 矩阵是什么"
           paragraphs "30秒速览", "背景", "L 矩阵的构造", "Mqk 矩阵的构造",
           "为什么 CHUNK16" (Neumann squaring), "K2 内核如何消费 L 和 Mqk".
  [SGL-PR] "SGLang PR #26586 (KDA packed decode)", the decode kernel snippet.

Readings taken where the pages are garbled or silent (each restated in the
design notes):
  * [FKDA-LM] prints L with a positive sign but also the series
    I - L + L^2 - ... ; from the recurrence, (I + A) U = u with
    A_ij = beta_i <k~_i, k^_j> (i > j).  We set L := -A so that
    U = (I - L)^{-1} u = sum_{n<16} L^n u.
  * The element formula beta_i e^{G_i - G_j} (k_i . k_j) is the scalar-gate
    shorthand; per channel it is beta_i sum_c k_ic k_jc e^{G_ic - G_jc}.
  * L is strictly lower triangular; Mqk keeps the diagonal.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# gate pieces ([SGL-PR] decode snippet: g = -exp(A_log) * softplus(a + dt_bias),
# beta = sigmoid(b)); softplus evaluated exactly, with no threshold.
# ----------------------------------------------------------------------------
def softplus(x):
    x = np.asarray(x, F64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + e^{-x}), evaluated without overflow for either sign."""
    x = np.asarray(x, F64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate(a, A_log, dt_bias):
    """g[..., h, c] = -exp(A_log[h]) * softplus(a[..., h, c] + dt_bias[h, c])."""
    a = np.asarray(a, F64)
    return -np.exp(np.asarray(A_log, F64))[:, None] * softplus(a + np.asarray(dt_bias, F64))


def _seq_bounds(T_total, cu_seqlens):
    if cu_seqlens is None:
        return [(0, T_total)]
    cu = np.asarray(cu_seqlens, np.int64)
    return [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


# ----------------------------------------------------------------------------
# The oracle proper: token recurrence ([TL-KDA] section 1), update order of
# [SGL-PR]: decay, delta, write, read.
# Shapes (packed tokens): q,k,a [T,H,dk]; v [T,H,dv]; b [T,H];
# A_log [H]; dt_bias [H,dk]; h0 [N,H,dv,dk] or None; cu_seqlens [N+1] or None.
# Returns o [T,H,dv], hT [N,H,dv,dk].
# ----------------------------------------------------------------------------
def recurrent(q, k, v, a, b, A_log, dt_bias, h0=None, cu_seqlens=None, scale=None):
    q, k, v, b = (np.asarray(x, F64) for x in (q, k, v, b))
    T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    g = gate(a, A_log, dt_bias)                        # [T,H,dk]
    beta = sigmoid(b)                                  # [T,H]
    bounds = _seq_bounds(T, cu_seqlens)
    o = np.zeros((T, H, dv), F64)
    hT = np.zeros((len(bounds), H, dv, dk), F64)
    for s, (t0, t1) in enumerate(bounds):
        S = np.zeros((H, dv, dk), F64) if h0 is None else np.array(h0[s], F64)
        for t in range(t0, t1):
            S = S * np.exp(g[t])[:, None, :]                          # S D_t
            u = beta[t][:, None] * (v[t] - np.einsum("hvc,hc->hv", S, k[t]))
            S = S + u[:, :, None] * k[t][:, None, :]                  # + u k^T
            o[t] = scale * np.einsum("hvc,hc->hv", S, q[t])           # S_t q_t
        hT[s] = S
    return o, hT


def recurrent_matrix_form(q, k, v, a, b, A_log, dt_bias, h0=None, cu_seqlens=None, scale=None):
    """The recurrence exactly as printed in [TL-KDA] section 1, with explicit
    matrices: S_t = S_{t-1} D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t (scale q_t).  O(dk^3) per token: for tiny inputs only."""
    q, k, v, b = (np.asarray(x, F64) for x in (q, k, v, b))
    T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    g = gate(a, A_log, dt_bias)
    beta = sigmoid(b)
    I = np.eye(dk)
    bounds = _seq_bounds(T, cu_seqlens)
    o = np.zeros((T, H, dv), F64)
    hT = np.zeros((len(bounds), H, dv, dk), F64)
    for s, (t0, t1) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((dv, dk)) if h0 is None else np.array(h0[s, h], F64)
            for t in range(t0, t1):
                D = np.diag(np.exp(g[t, h]))
                kk = k[t, h][:, None]
                S = S @ D @ (I - beta[t, h] * (kk @ kk.T)) + beta[t, h] * (v[t, h][:, None] @ kk.T)
                o[t, h] = S @ (scale * q[t, h])
            hT[s, h] = S
    return o, hT


def decode_step(qkv, a, b, A_log, dt_bias, pool, state_idx, H, HV, K, V, scale=None, l2norm=True):
    """One T=1 step over a state pool ([SGL-PR] decode snippet).  Returns
    (o [B,HV,V], new_pool) without modifying the input pool."""
    qkv = np.asarray(qkv, F64)
    B = qkv.shape[0]
    if scale is None:
        scale = K ** -0.5
    pool = np.array(pool, F64, copy=True)
    o = np.zeros((B, HV, V), F64)
    a = np.asarray(a, F64).reshape(B, HV, K)
    b = np.asarray(b, F64).reshape(B, HV)
    dt = np.asarray(dt_bias, F64).reshape(HV, K)
    for n in range(B):
        idx = int(state_idx[n])
        if idx < 0:
            continue
        for hv in range(HV):
            hq = hv // (HV // H)
            qv = qkv[n, hq * K:(hq + 1) * K].copy()
            kv = qkv[n, H * K + hq * K:H * K + (hq + 1) * K].copy()
            vv = qkv[n, 2 * H * K + hv * V:2 * H * K + (hv + 1) * V]
            if l2norm:
                qv = qv / np.sqrt(np.sum(qv * qv) + 1e-6)
                kv = kv / np.sqrt(np.sum(kv * kv) + 1e-6)
            qv = qv * scale
            g = -np.exp(float(A_log[hv])) * softplus(a[n, hv] + dt[hv])
            beta = float(sigmoid(b[n, hv]))
            S = pool[idx, hv] * np.exp(g)[None, :]
            u = beta * (vv - S @ kv)
            S = S + u[:, None] * kv[None, :]
            o[n, hv] = S @ qv
            pool[idx, hv] = S
    return o, pool


# ----------------------------------------------------------------------------
# Chunkwise fp64 reference ([FKDA-LM]): per chunk of C tokens with entering
# state S0 (dv x dk):
#   G_i = sum_{j<=i} g_j (chunk-local, per channel)
#   L_ij  = -beta_i sum_c k_ic k_jc e^{G_ic - G_jc}   (i > j, strictly lower)
#   Mqk_ij = sum_c qs_ic k_jc e^{G_ic - G_jc}           (i >= j), qs = scale q
#   INV = (I - L)^{-1} by Neumann squaring (I+L)(I+L^2)(I+L^4)(I+L^8)...
#   u = beta * (v - (k * e^G) S0^T);  U = INV u
#   O = (qs * e^G) S0^T + Mqk U
#   S <- S0 * e^{G_C} + U^T (k * e^{G_C - G})
# Pairwise exponentials are evaluated directly (no factoring), so nothing
# overflows.  The state update comes after the chunk's output ([TL-KDA]
# section 6.4.2, [LA-06] section 3.3).
# ----------------------------------------------------------------------------
def neumann_inverse(L):
    """(I - L)^{-1} for strictly lower-triangular L of size n <= 2^m by
    repeated squaring: prod_{r<m} (I + L^{2^r}) ([FKDA-LM] 为什么 CHUNK16)."""
    n = L.shape[-1]
    I = np.eye(n)
    inv = I + L
    P = L
    span = 2
    while span < n:
        P = P @ P
        inv = inv @ (I + P)
        span *= 2
    return inv


def chunk_matrices(qc, kc, gc, betac, scale):
    """Per-chunk L, Mqk, INV for one head: qc,kc,gc [C,dk], betac [C]."""
    C = kc.shape[0]
    G = np.cumsum(gc, axis=0)                            # [C,dk]
    diff = G[:, None, :] - G[None, :, :]                 # [i,j,c] = G_ic - G_jc
    lower = np.tril(np.ones((C, C), bool))
    diff = np.where(lower[:, :, None], diff, -np.inf)    # i >= j only: e^{diff} <= 1
    E = np.exp(diff)
    KK = np.einsum("ic,jc,ijc->ij", kc, kc, E)
    QK = np.einsum("ic,jc,ijc->ij", scale * qc, kc, E)
    L = -betac[:, None] * np.tril(KK, -1)
    Mqk = np.tril(QK)
    return G, L, Mqk, neumann_inverse(L)


def chunkwise(q, k, v, a, b, A_log, dt_bias, h0=None, cu_seqlens=None, scale=None, C=16):
    q, k, v, b = (np.asarray(x, F64) for x in (q, k, v, b))
    T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    g = gate(a, A_log, dt_bias)
    beta = sigmoid(b)
    bounds = _seq_bounds(T, cu_seqlens)
    o = np.zeros((T, H, dv), F64)
    hT = np.zeros((len(bounds), H, dv, dk), F64)
    for s, (t0, t1) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((dv, dk)) if h0 is None else np.array(h0[s, h], F64)
            for c0 in range(t0, t1, C):
                c1 = min(c0 + C, t1)              # ragged tail: a shorter chunk
                qc, kc, vc = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h]
                G, L, Mqk, INV = chunk_matrices(qc, kc, g[c0:c1, h], beta[c0:c1, h], scale)
                kd = kc * np.exp(G)                       # k decayed
                qd = scale * qc * np.exp(G)               # q decayed
                kr = kc * np.exp(G[-1][None, :] - G)      # k restored to chunk end
                u = beta[c0:c1, h][:, None] * (vc - kd @ S.T)
                U = INV @ u
                o[c0:c1, h] = qd @ S.T + Mqk @ U
                S = S * np.exp(G[-1])[None, :] + U.T @ kr
            hT[s, h] = S
    return o, hT


# ----------------------------------------------------------------------------
# Level-1 references: the ungated accumulation S_t = S_{t-1} + k_t v_t^T with
# o_t = S_t^T q_t ([TL-KDA] section 2.1), in three structures whose agreement
# is the check of section 3.4.  Its chunk identity: with S_prev the sum of
# k v^T over every token before chunk c,
#     O_c = Q_c S_prev + tril(Q_c K_c^T) V_c.
# Inputs [B, N, H, D] (values [B, N, H, DV]); each head is handled alone.
# ----------------------------------------------------------------------------
def _each_head(fn, Q, K, V, *extra):
    """Apply fn(q [N, D], k [N, D], v [N, DV], *extra) -> [N, DV] to every
    (batch, head) and reassemble [B, N, H, DV]."""
    Q, K, V = (np.asarray(x, F64) for x in (Q, K, V))
    out = np.empty(Q.shape[:-1] + (V.shape[-1],))
    for bb, h in np.ndindex(Q.shape[0], Q.shape[2]):
        out[bb, :, h] = fn(Q[bb, :, h], K[bb, :, h], V[bb, :, h], *extra)
    return out


def _tokens(q, k, v):
    state = np.zeros((k.shape[1], v.shape[1]))
    res = np.empty((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        state += np.outer(k[t], v[t])
        res[t] = state.T @ q[t]
    return res


def level1_recurrent(Q, K, V):
    """Token by token: accumulate k_t v_t^T, then read with q_t."""
    return _each_head(_tokens, Q, K, V)


def _chunk_identity(q, k, v, C, inclusive):
    n = q.shape[0]
    starts = range(0, n, C)
    # every chunk's own contribution K_c^T V_c, then the state each chunk sees:
    # the sum over the chunks before it (inclusive=True also adds its own,
    # the off-by-one-chunk mistake: the chunk's keys are then counted twice)
    incr = [k[c0:c0 + C].T @ v[c0:c0 + C] for c0 in starts]
    seen, running = [], np.zeros((k.shape[1], v.shape[1]))
    for dS in incr:
        if inclusive:
            running = running + dS
            seen.append(running)
        else:
            seen.append(running)
            running = running + dS
    res = np.empty((n, v.shape[1]))
    for c0, S_prev in zip(starts, seen):
        qc, kc, vc = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C]
        res[c0:c0 + C] = qc @ S_prev + np.tril(qc @ kc.T) @ vc
    return res


def level1_chunked(Q, K, V, BC, right_shift=True):
    """The chunk identity with every chunk's entering state taken as the sum of
    the contributions of the chunks before it (all contributions formed
    first).  right_shift=False includes the chunk's own contribution too: the
    structural mistake whose error is O(1)."""
    return _each_head(_chunk_identity, Q, K, V, BC, not right_shift)


def _slab_walk(q, k, v, C, slab, read_first):
    n, dv = q.shape[0], v.shape[1]
    res = np.empty((n, dv))
    for j0 in range(0, dv, slab):                      # each slab of value columns alone
        cols = slice(j0, min(dv, j0 + slab))
        S = np.zeros((k.shape[1], cols.stop - cols.start))
        for c0 in range(0, n, C):                      # sequential walk over the chunks
            qc, kc, vc = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C, cols]
            if not read_first:                         # the mistake: advance before reading
                S = S + kc.T @ vc
            res[c0:c0 + C, cols] = qc @ S + np.tril(qc @ kc.T) @ vc
            if read_first:
                S = S + kc.T @ vc
    return res


def level1_dv_slab(Q, K, V, BC, block_dv, update_after_write=True):
    """The chunk identity walked chunk by chunk, each slab of block_dv value
    columns carrying its own slice of the state; the chunk's output is read
    before the state advances.  update_after_write=False advances first: the
    structural mistake whose error is O(1)."""
    return _each_head(_slab_walk, Q, K, V, BC, block_dv, update_after_write)


def parallel_form(Q, K, V, scale=1.0):
    """[LA-06] section 3.1: O = ((Q K^T) ⊙ M) V with the causal mask M
    (inclusive), materialising the N x N matrix.  Shapes [N, D]."""
    Q, K, V = (np.asarray(x, F64) for x in (Q, K, V))
    return np.tril((scale * Q) @ K.T) @ V
