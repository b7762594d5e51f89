"""fp64 gradients of the KDA forward -- TEST INFRASTRUCTURE ONLY.

Only tests and the benchmark may import this module; nothing here is shared
with the HIP library.

The forward is the token recurrence of [TL-KDA] "TileLang 实战：KDA 从零到一 --
Chunked 线性注意力", section 1, with the gate and beta of [SGL-PR] "SGLang PR
#26586 (KDA packed decode)" (implementation notes, item 1):
    g_t = -exp(A_log[h]) softplus(a_t + dt_bias[h]),  beta_t = sigmoid(b_t)
    S'  = S Diag(e^{g_t});  u = beta_t (v_t - S' k_t);  S = S' + u k_t^T
    o_t = S (scale q_t)
written here in plain PyTorch on the CPU in float64, and differentiated by
torch.autograd: the gradient of that definition, for a loss whose gradients
with respect to o and to the final states are given (do, dh_T).  The
backward pass that the pages name (a reverse loop over chunks, [LA-06]
"06 · linear 路线（一）" chunkwise form) computes exactly these derivatives.
"""
from __future__ import annotations

import numpy as np
import torch

F64 = torch.float64


def _t(x):
    return torch.as_tensor(np.asarray(x, np.float64), dtype=F64)


def forward_torch(q, k, v, a, b, A_log, dt_bias, h0, scale):
    """One (sequence) of packed tokens, all heads at once.
    q, k, a: [T, H, dk]; v: [T, H, dv]; b: [T, H]; A_log: [H];
    dt_bias: [H, dk]; h0: [H, dv, dk].  Returns (o [T, H, dv], h_T)."""
    T = q.shape[0]
    S = h0
    A = torch.exp(A_log)[:, None]                       # [H, 1]
    outs = []
    for t in range(T):
        g = -A * torch.nn.functional.softplus(a[t] + dt_bias)   # [H, dk]
        beta = torch.sigmoid(b[t])                      # [H]
        Sd = S * torch.exp(g)[:, None, :]               # decay along the key axis
        w = torch.einsum("hvk,hk->hv", Sd, k[t])
        u = beta[:, None] * (v[t] - w)
        S = Sd + u[:, :, None] * k[t][:, None, :]
        outs.append(torch.einsum("hvk,hk->hv", S, scale * q[t]))
    o = torch.stack(outs) if T else torch.zeros((0,) + v.shape[1:], dtype=F64)
    return o, S


def backward(q, k, v, a, b, A_log, dt_bias, do, h0=None, dh_T=None, cu_seqlens=None, scale=None):
    """Gradients of sum(o * do) + sum(h_T * dh_T) over packed sequences.

    q, k, a: [T, H, dk]; v, do: [T, H, dv]; b: [T, H]; A_log: [H];
    dt_bias: [H, dk]; h0, dh_T: [N, H, dv, dk] or None; cu_seqlens: [N+1] or
    None (one sequence).  Returns a dict of float64 arrays: dq, dk, dv, da
    (of the raw gate input), db (of the raw beta input), dA_log [H],
    ddt_bias [H, dk], dh0 [N, H, dv, dk]."""
    q, k, v, a, b, do = (_t(x) for x in (q, k, v, a, b, do))
    T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    cu = [0, T] if cu_seqlens is None else [int(x) for x in np.asarray(cu_seqlens)]
    N = len(cu) - 1
    h0 = torch.zeros((N, H, dv, dk), dtype=F64) if h0 is None else _t(h0).reshape(N, H, dv, dk)
    dh_T = None if dh_T is None else _t(dh_T).reshape(N, H, dv, dk)
    leaves = [x.clone().requires_grad_(True) for x in (q, k, v, a, b, _t(A_log), _t(dt_bias).reshape(H, dk), h0)]
    ql, kl, vl, al, bl, Al, dtl, h0l = leaves
    loss = torch.zeros((), dtype=F64)
    for s in range(N):
        t0, t1 = cu[s], cu[s + 1]
        o, hT = forward_torch(ql[t0:t1], kl[t0:t1], vl[t0:t1], al[t0:t1], bl[t0:t1], Al, dtl, h0l[s], scale)
        loss = loss + (o * do[t0:t1]).sum()
        if dh_T is not None:
            loss = loss + (hT * dh_T[s]).sum()
    grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    names = ("dq", "dk", "dv", "da", "db", "dA_log", "ddt_bias", "dh0")
    out = {}
    for n, g, x in zip(names, grads, leaves):
        out[n] = (torch.zeros_like(x) if g is None else g).detach().numpy()
    return out
