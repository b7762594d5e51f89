"""Seeded synthetic inputs for KDA prefill and decode.

This module only draws random numbers and quantises them; it holds none of the
attention arithmetic.  Both the HIP path (through its tests and benchmark) and
the fp64 oracle consume exactly the arrays produced here.

Recipe (numpy PCG64, float32 draws, then RNE rounding to the I/O dtype).
Small draws (variable lengths first, then A_log, dt_bias and slot indices)
come from `default_rng(seed)`.  Every large tensor is filled in blocks of 2^22
elements, block i from `default_rng(child_i)` where the children are spawned
from `SeedSequence(seed)` (one child per tensor, then one per block), so the
blocks can be drawn in parallel and the values do not depend on the thread
count.  The draws:
  * q, k ~ N(0,1), each head vector L2-normalised in float32 as
    x / sqrt(sum(x^2) + 1e-6) before rounding (the prefill consumes unit keys
    and queries; the decode path normalises in its kernel instead);
  * v ~ N(0,1); a ~ N(0,1) per (token, head, channel); b ~ N(0,1) per
    (token, head);
  * dt_bias ~ U(-1,1) per (head, channel); A_log ~ U(0, log 16) per head
    (U(0, log 4) for the long single-sequence workload);
  * an initial state, when present, ~ N(0, 0.02^2) in float32;
  * variable lengths ~ U{128..8192} (inclusive), drawn first.
bf16 values are stored as their uint16 bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

LOG16 = math.log(16.0)
LOG4 = math.log(4.0)


_BLOCK = 1 << 22


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def _blockwise(fn, n_elem, block=_BLOCK):
    """Run fn(i) for every block index; numpy releases the GIL in the work."""
    nblk = (n_elem + block - 1) // block
    if nblk <= 1:
        for i in range(nblk):
            fn(i)
        return
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fn, range(nblk)))


# ----------------------------------------------------------------------------
# bf16 helpers (bit level, round to nearest even)
# ----------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even."""
    src = np.ascontiguousarray(x, np.float32)
    out = np.empty(src.shape, np.uint16)
    fin, fout = src.reshape(-1).view(np.uint32), out.reshape(-1)

    def work(i):
        u = fin[i * _BLOCK:(i + 1) * _BLOCK]
        r = u >> np.uint32(16)
        r &= np.uint32(1)
        r += np.uint32(0x7FFF)
        r += u
        r >>= np.uint32(16)
        fout[i * _BLOCK:(i + 1) * _BLOCK] = r

    _blockwise(work, fin.size)
    return out


def bf16_to_f32(bits) -> np.ndarray:
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)




class _Streams:
    """Independent PCG64 streams for the large tensors of one workload."""

    def __init__(self, seed: int, n: int = 16):
        self._kids = np.random.SeedSequence(seed).spawn(n)
        self._next = 0

    def normal(self, shape, scale: float = 1.0) -> np.ndarray:
        ss = self._kids[self._next]
        self._next += 1
        out = np.empty(shape, np.float32)
        flat = out.reshape(-1)
        nblk = (flat.size + _BLOCK - 1) // _BLOCK
        blocks = ss.spawn(nblk)

        def fill(i):
            seg = flat[i * _BLOCK:(i + 1) * _BLOCK]
            np.random.default_rng(blocks[i]).standard_normal(out=seg, dtype=np.float32)
            if scale != 1.0:
                seg *= np.float32(scale)

        _blockwise(fill, flat.size)
        return out


def _l2norm_f32(x):
    """x / sqrt(sum(x^2) + 1e-6) over the last axis, in float32, in place."""
    x = np.ascontiguousarray(x, np.float32)
    rows = x.reshape(-1, x.shape[-1])
    per = max(1, _BLOCK // x.shape[-1])

    def work(i):
        seg = rows[i * per:(i + 1) * per]
        n = np.sqrt(np.einsum("ij,ij->i", seg, seg, dtype=np.float32)[:, None] + np.float32(1e-6))
        seg /= n

    _blockwise(work, rows.shape[0], per)
    return x


def _quant(x, dtype):
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _deq(x, dtype):
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


# ----------------------------------------------------------------------------
# Prefill
# ----------------------------------------------------------------------------
@dataclass
class Prefill:
    """Packed-token prefill inputs.  Activations are [B*T (or T_total), H, d]
    in the I/O dtype (float32 array, or uint16 bf16 bits)."""
    name: str
    dtype: str                      # "f32" or "bf16"
    B: int
    T: int                          # per-sequence length (dense) or total tokens (varlen)
    H: int
    dk: int
    dv: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray
    A_log: np.ndarray               # [H] float32
    dt_bias: np.ndarray             # [H, dk] float32
    h0: Optional[np.ndarray] = None  # [N, H, dv, dk] float32
    cu_seqlens: Optional[np.ndarray] = None  # [N+1] int32 (varlen) or None (dense)
    meta: dict = field(default_factory=dict)

    @property
    def n_seq(self) -> int:
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    @property
    def tokens(self) -> int:
        return self.q.shape[0]

    @property
    def scale(self) -> float:
        return self.dk ** -0.5

    def offsets(self) -> np.ndarray:
        if self.cu_seqlens is not None:
            return np.asarray(self.cu_seqlens, np.int64)
        return np.arange(self.B + 1, dtype=np.int64) * self.T

    def f64(self, heads=None) -> dict:
        """The exact stored values widened to float64 (oracle inputs), for all
        heads or a subset."""
        hs = slice(None) if heads is None else list(heads)
        deq = lambda x: _deq(x[:, hs], self.dtype).astype(np.float64)
        out = dict(q=deq(self.q), k=deq(self.k), v=deq(self.v), a=deq(self.a),
                   b=_deq(self.b[:, hs], self.dtype).astype(np.float64),
                   A_log=self.A_log[hs].astype(np.float64),
                   dt_bias=self.dt_bias[hs].astype(np.float64),
                   h0=None if self.h0 is None else self.h0[:, hs].astype(np.float64),
                   cu_seqlens=self.offsets(), scale=self.scale)
        return out


def cotangents(seed: int, tokens: int, H: int, dv: int, dk: int, n_seq: int, with_dhT: bool = True):
    """Gradients flowing into the forward's outputs for a backward test: do ~
    N(0, 1) per (token, head, column) as bf16 bits, and dh_T ~ N(0, 0.02^2)
    float32 (or None)."""
    st = _Streams(seed + 2000)
    do = bf16_bits(st.normal((tokens, H, dv)))
    dhT = st.normal((n_seq, H, dv, dk), 0.02) if with_dhT else None
    return do, dhT


def prefill(seed: int, B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16", *,
            lengths=None, n_var: int = 0, with_h0: bool = False, A_log_hi: float = LOG16,
            gate_stress: float = 0.0, name: str = "custom") -> Prefill:
    """Draw a prefill workload.

    Dense: B sequences of T tokens.  Varlen: pass `lengths` (list) or `n_var`
    (> 0: draw that many lengths ~ U{128..8192} first); B becomes 1 and T the
    total token count.  `gate_stress` > 0 sets that fraction of `a` entries to
    +30 (softplus ~ 30, i.e. per-token decays of 30*exp(A_log) nats)."""
    rng = np.random.default_rng(seed)
    cu = None
    if n_var > 0:
        lengths = rng.integers(128, 8192, endpoint=True, size=n_var)
    if lengths is not None:
        lengths = np.asarray(lengths, np.int64)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        n_tok, B_eff, T_eff = int(cu[-1]), 1, int(cu[-1])
    else:
        n_tok, B_eff, T_eff = B * T, B, T
    st = _Streams(seed)
    q = _l2norm_f32(st.normal((n_tok, H, dk)))
    k = _l2norm_f32(st.normal((n_tok, H, dk)))
    v = st.normal((n_tok, H, dv))
    a = st.normal((n_tok, H, dk))
    b = st.normal((n_tok, H))
    A_log = rng.uniform(0.0, A_log_hi, size=H).astype(np.float32)
    dt_bias = rng.uniform(-1.0, 1.0, size=(H, dk)).astype(np.float32)
    n_seq = B_eff if cu is None else len(cu) - 1
    h0 = st.normal((n_seq, H, dv, dk), 0.02) if with_h0 else None
    if gate_stress > 0:
        hit = rng.random(size=a.shape) < gate_stress
        a[hit] = np.float32(30.0)
    return Prefill(name=name, dtype=dtype, B=B_eff, T=T_eff, H=H, dk=dk, dv=dv,
                   q=_quant(q, dtype), k=_quant(k, dtype), v=_quant(v, dtype),
                   a=_quant(a, dtype), b=_quant(b, dtype), A_log=A_log, dt_bias=dt_bias,
                   h0=h0, cu_seqlens=cu, meta=dict(seed=seed))


# The four prefill workloads (seed = workload index).
PREFILL_WORKLOADS = {
    0: dict(name="tiny-f32 B1 H2 T256 d64", B=1, T=256, H=2, dk=64, dv=64, dtype="f32"),
    1: dict(name="prefill-bf16 B4 H16 T4096 d128", B=4, T=4096, H=16, dk=128, dv=128, dtype="bf16"),
    2: dict(name="varlen-bf16 32seq U[128,8192] H32 d128 h0", B=1, T=0, H=32, dk=128, dv=128,
            dtype="bf16", n_var=32, with_h0=True),
    3: dict(name="long-bf16 B1 H32 T131072 d128", B=1, T=131072, H=32, dk=128, dv=128,
            dtype="bf16", A_log_hi=LOG4),
}


def prefill_workload(i: int) -> Prefill:
    kw = dict(PREFILL_WORKLOADS[i])
    return prefill(i, **kw)


# ----------------------------------------------------------------------------
# Decode
# ----------------------------------------------------------------------------
@dataclass
class Decode:
    name: str
    B: int
    H: int
    HV: int
    K: int
    V: int
    P: int
    qkv: np.ndarray        # [B, 2*H*K + HV*V] bf16 bits
    a: np.ndarray          # [B, HV*K] bf16 bits
    b: np.ndarray          # [B, HV] bf16 bits
    A_log: np.ndarray      # [HV] f32
    dt_bias: np.ndarray    # [HV*K] f32
    pool: np.ndarray       # [P, HV, V, K] f32
    state_idx: np.ndarray  # [B] int32, -1 = pad
    meta: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return self.K ** -0.5

    def f64(self) -> dict:
        return dict(qkv=bf16_to_f32(self.qkv).astype(np.float64),
                    a=bf16_to_f32(self.a).astype(np.float64),
                    b=bf16_to_f32(self.b).astype(np.float64),
                    A_log=self.A_log.astype(np.float64), dt_bias=self.dt_bias.astype(np.float64))


def _unit_qk(qkv, H, K):
    """L2-normalise the q and k heads of packed rows (last axis), float32."""
    qk = _l2norm_f32(qkv[..., :2 * H * K].reshape(-1, K))
    qkv[..., :2 * H * K] = qk.reshape(qkv[..., :2 * H * K].shape)


def decode(seed: int, B: int, H: int, HV: int, K: int, V: int, P: int, n_pad: int, *,
           name: str = "custom", gate_stress: float = 0.0, unit_qk: bool = False) -> Decode:
    """Draw a decode workload: distinct slots (first B of a permutation of P),
    then `n_pad` random rows set to -1.  `unit_qk`: q and k heads drawn as unit
    vectors (for calls without the in-kernel norm)."""
    assert P >= B and HV % H == 0
    rng = np.random.default_rng(seed)
    st = _Streams(seed)
    D = 2 * H * K + HV * V
    qkv = st.normal((B, D))
    if unit_qk:
        _unit_qk(qkv, H, K)
    a = st.normal((B, HV * K))
    b = st.normal((B, HV))
    dt_bias = rng.uniform(-1.0, 1.0, size=HV * K).astype(np.float32)
    A_log = rng.uniform(0.0, LOG16, size=HV).astype(np.float32)
    pool = st.normal((P, HV, V, K), 0.02)
    idx = rng.permutation(P)[:B].astype(np.int32)
    if n_pad:
        idx[rng.choice(B, size=n_pad, replace=False)] = -1
    if gate_stress > 0:
        hit = rng.random(size=a.shape) < gate_stress
        a[hit] = np.float32(30.0)
    return Decode(name=name, B=B, H=H, HV=HV, K=K, V=V, P=P, qkv=bf16_bits(qkv), a=bf16_bits(a),
                  b=bf16_bits(b), A_log=A_log, dt_bias=dt_bias, pool=pool, state_idx=idx,
                  meta=dict(seed=seed))


def extend(seed: int, B: int, T: int, H: int, HV: int, K: int, V: int, P: int, n_pad: int, *,
           name: str = "custom", gate_stress: float = 0.0, unit_qk: bool = False) -> Decode:
    """Draw a T-token-per-row decode workload (extend / speculative verify):
    as `decode`, with qkv [B, T, D], a [B, T, HV*K] and b [B, T, HV]."""
    assert P >= B and HV % H == 0
    rng = np.random.default_rng(seed)
    st = _Streams(seed)
    D = 2 * H * K + HV * V
    qkv = st.normal((B, T, D))
    if unit_qk:
        _unit_qk(qkv, H, K)
    a = st.normal((B, T, HV * K))
    b = st.normal((B, T, HV))
    dt_bias = rng.uniform(-1.0, 1.0, size=HV * K).astype(np.float32)
    A_log = rng.uniform(0.0, LOG16, size=HV).astype(np.float32)
    pool = st.normal((P, HV, V, K), 0.02)
    idx = rng.permutation(P)[:B].astype(np.int32)
    if n_pad:
        idx[rng.choice(B, size=n_pad, replace=False)] = -1
    if gate_stress > 0:
        hit = rng.random(size=a.shape) < gate_stress
        a[hit] = np.float32(30.0)
    return Decode(name=name, B=B, H=H, HV=HV, K=K, V=V, P=P, qkv=bf16_bits(qkv), a=bf16_bits(a),
                  b=bf16_bits(b), A_log=A_log, dt_bias=dt_bias, pool=pool, state_idx=idx,
                  meta=dict(seed=seed, T=T))


@dataclass
class ConvDecode(Decode):
    """A decode workload whose qkv row is the input of the short convolution
    (mixed_qkv), with the convolution's state, weights and bias."""
    W: int = 4
    conv_state: np.ndarray = None   # [P, W-1, D] bf16 bits
    conv_weight: np.ndarray = None  # [D, W] bf16 bits
    conv_bias: np.ndarray = None    # [D] bf16 bits, or None

    def f64(self) -> dict:
        out = super().f64()
        out.update(conv_state=bf16_to_f32(self.conv_state).astype(np.float64),
                   conv_weight=bf16_to_f32(self.conv_weight).astype(np.float64),
                   conv_bias=None if self.conv_bias is None else bf16_to_f32(self.conv_bias).astype(np.float64))
        return out


def conv_decode(seed: int, B: int, H: int, HV: int, K: int, V: int, P: int, n_pad: int, W: int = 4, *,
                bias: bool = True, name: str = "custom") -> ConvDecode:
    """Draw a decode workload with the short convolution in front: as `decode`
    (mixed_qkv ~ N(0,1) in place of qkv), then the conv state ~ N(0,1) (earlier
    inputs of the same kind) and weights and bias ~ U(-1/sqrt(W), 1/sqrt(W))
    (the default initialisation of a depthwise convolution of width W)."""
    d = decode(seed, B=B, H=H, HV=HV, K=K, V=V, P=P, n_pad=n_pad, name=name)
    rng = np.random.default_rng(seed + 1000)
    D = 2 * H * K + HV * V
    st = _Streams(seed + 1000)
    cs = st.normal((P, W - 1, D))
    lim = 1.0 / np.sqrt(W)
    w = rng.uniform(-lim, lim, size=(D, W)).astype(np.float32)
    cb = rng.uniform(-lim, lim, size=D).astype(np.float32) if bias else None
    return ConvDecode(**{f: getattr(d, f) for f in ("name", "B", "H", "HV", "K", "V", "P", "qkv", "a", "b",
                                                     "A_log", "dt_bias", "pool", "state_idx", "meta")},
                      W=W, conv_state=bf16_bits(cs), conv_weight=bf16_bits(w),
                      conv_bias=None if cb is None else bf16_bits(cb))


DECODE_WORKLOAD = dict(name="decode-bf16 B256 H32 HV32 K128 V128 pool512 pad8",
                       B=256, H=32, HV=32, K=128, V=128, P=512, n_pad=8)


def decode_workload() -> Decode:
    return decode(4, **DECODE_WORKLOAD)
