"""fp64 CPU oracle for Kimi Delta Attention -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the benchmark's `cpu_baseline`
leg may import this package.  The product library never loads it and shares
no code with it.

`fwd`, `decode` and `extend` call the plain-C token recurrence in `kda_oracle.c`
and `conv_update` its short causal convolution
(OpenMP over independent (sequence, head) chains); `oracle.ref` holds the
numpy twins and the chunkwise / level-1 references used to pin it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile kda_oracle.c with gcc (fp64, OpenMP).  No fast-math: the
    oracle keeps IEEE semantics."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.kda_oracle_fwd.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_double, P,
                                       ctypes.c_int, P, P, ctypes.c_int]
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd_states.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_double, P,
                                              ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int]
        lib.kda_oracle_fwd_states.restype = ctypes.c_int
        lib.kda_oracle_decode.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, ctypes.c_double, ctypes.c_int, P,
                                          ctypes.c_int]
        lib.kda_oracle_decode.restype = ctypes.c_int
        lib.kda_oracle_extend.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, ctypes.c_double, ctypes.c_int, P,
                                          ctypes.c_int]
        lib.kda_oracle_extend.restype = ctypes.c_int
        lib.kda_oracle_conv_update.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int64, P]
        lib.kda_oracle_conv_update.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def fwd(q, k, v, a, b, A_log, dt_bias, h0=None, cu_seqlens=None, scale=None,
        chains=None, n_threads=None, out=None, chunk_states=None):
    """Token-recurrence forward over packed tokens.

    q,k,a: [T,H,dk]; v: [T,H,dv]; b: [T,H]; A_log: [H]; dt_bias: [H,dk];
    h0: [N,H,dv,dk] or None; cu_seqlens: [N+1] or None (one sequence).
    chains: optional iterable of chain ids (seq*H + head) to compute; other
    chains' outputs stay zero.  Returns (o [T,H,dv], hT [N,H,dv,dk]) in fp64.
    chunk_states=C also returns the state entering every chunk of C tokens,
    [sum_s ceil(len_s / C), H, dv, dk] (rows of the sequences in order).
    """
    q, k, v, a, b = (_f64(x) for x in (q, k, v, a, b))
    T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    cu = np.array([0, T], np.int64) if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, np.int64)
    n_seq = len(cu) - 1
    A_log, dt_bias = _f64(A_log), _f64(dt_bias).reshape(H, dk)
    h0 = None if h0 is None else _f64(h0).reshape(n_seq, H, dv, dk)
    o = np.zeros((T, H, dv)) if out is None else out
    hT = np.zeros((n_seq, H, dv, dk))
    ch = None if chains is None else np.ascontiguousarray(list(chains), np.int32)
    nthr = int(n_threads or default_threads())
    if chunk_states is None:
        rc = _load().kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
                                    _ptr(dt_bias), _ptr(h0), _ptr(cu), n_seq, H, dk, dv,
                                    float(scale), _ptr(ch), 0 if ch is None else len(ch),
                                    _ptr(o), _ptr(hT), nthr)
        if rc != 0:
            raise ValueError("kda_oracle_fwd rejected its arguments")
        return o, hT
    C = int(chunk_states)
    nc = int(((np.diff(cu) + C - 1) // C).sum())
    hc = np.zeros((nc, H, dv, dk))
    rc = _load().kda_oracle_fwd_states(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
                                       _ptr(dt_bias), _ptr(h0), _ptr(cu), n_seq, H, dk, dv,
                                       float(scale), _ptr(ch), 0 if ch is None else len(ch),
                                       _ptr(o), _ptr(hT), _ptr(hc), C, nthr)
    if rc != 0:
        raise ValueError("kda_oracle_fwd_states rejected its arguments")
    return o, hT, hc


def decode(qkv, a, b, A_log, dt_bias, pool, state_idx, H, HV, K, V, scale=None,
           l2norm=True, n_threads=None):
    """One T=1 decode step.  Returns (o [B,HV,V], new pool) in fp64; the input
    pool is not modified."""
    qkv = _f64(qkv)
    B = qkv.shape[0]
    if scale is None:
        scale = K ** -0.5
    pool = np.array(pool, np.float64, copy=True, order="C")
    idx = np.ascontiguousarray(state_idx, np.int64)
    o = np.zeros((B, HV, V))
    rc = _load().kda_oracle_decode(_ptr(qkv), _ptr(_f64(a)), _ptr(_f64(b)), _ptr(_f64(A_log)),
                                   _ptr(_f64(dt_bias)), _ptr(pool), _ptr(idx), B, H, HV, K, V,
                                   pool.shape[0], float(scale), int(bool(l2norm)), _ptr(o),
                                   int(n_threads or default_threads()))
    if rc != 0:
        raise ValueError("kda_oracle_decode rejected its arguments")
    return o, pool


def extend(qkv, a, b, A_log, dt_bias, pool, state_idx, H, HV, K, V, scale=None,
           l2norm=True, n_threads=None):
    """T decode steps per row in token order.  qkv: [B, T, 2HK + HV V];
    a: [B, T, HV K]; b: [B, T, HV].  Returns (o [B,T,HV,V], new pool) in fp64;
    the input pool is not modified."""
    qkv = _f64(qkv)
    B, T = qkv.shape[0], qkv.shape[1]
    if scale is None:
        scale = K ** -0.5
    pool = np.array(pool, np.float64, copy=True, order="C")
    idx = np.ascontiguousarray(state_idx, np.int64)
    o = np.zeros((B, T, HV, V))
    rc = _load().kda_oracle_extend(_ptr(qkv), _ptr(_f64(a)), _ptr(_f64(b)), _ptr(_f64(A_log)),
                                   _ptr(_f64(dt_bias)), _ptr(pool), _ptr(idx), B, T, H, HV, K, V,
                                   pool.shape[0], float(scale), int(bool(l2norm)), _ptr(o),
                                   int(n_threads or default_threads()))
    if rc != 0:
        raise ValueError("kda_oracle_extend rejected its arguments")
    return o, pool


def conv_update(x, conv_state, weight, bias, state_idx):
    """One causal-conv update per row (silu).  x: [B, D]; conv_state:
    [P, W-1, D]; weight: [D, W]; bias: [D] or None.  Returns (y [B, D], new
    conv_state) in fp64; the input state is not modified."""
    x = _f64(x)
    B, D = x.shape
    weight = _f64(weight).reshape(D, -1)
    W = weight.shape[1]
    idx = np.ascontiguousarray(state_idx, np.int64)
    if W > 1:
        cs = np.array(conv_state, np.float64, copy=True, order="C").reshape(-1, W - 1, D)
        P = cs.shape[0]
    else:   # width 1: no state
        cs, P = None, np.iinfo(np.int64).max
    y = np.zeros((B, D))
    rc = _load().kda_oracle_conv_update(_ptr(x), _ptr(cs), _ptr(weight),
                                        _ptr(None if bias is None else _f64(bias)), _ptr(idx),
                                        B, D, W, P, _ptr(y))
    if rc != 0:
        raise ValueError("kda_oracle_conv_update rejected its arguments")
    return y, cs


def conv_decode(mixed_qkv, conv_state, conv_weight, conv_bias, a, b, A_log, dt_bias, pool,
                state_idx, H, HV, K, V, scale=None, l2norm=True, n_threads=None):
    """The short convolution, then one decode step on its output (both slots
    addressed by state_idx).  Returns (o [B,HV,V], new pool, new conv_state)."""
    y, cs = conv_update(mixed_qkv, conv_state, conv_weight, conv_bias, state_idx)
    o, newpool = decode(y, a, b, A_log, dt_bias, pool, state_idx, H, HV, K, V, scale=scale,
                        l2norm=l2norm, n_threads=n_threads)
    return o, newpool, cs
