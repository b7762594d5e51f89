"""Python binding of libkda (MI355X / gfx950 Kimi Delta Attention).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/kda.h.  PyTorch provides device memory and
the current stream.  There is no CPU fallback: if the library is not built or
a tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")
_lib = None

KDA_F32, KDA_BF16 = 0, 1
KDA_DECODE_L2NORM = 1

EXPORTS = ("kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd_pool", "kda_chunk_fwd_states",
           "kda_device_check", "kda_decode_step",
           "kda_decode_extend", "kda_conv_decode_step", "kda_chunk_o", "kda_backward", "kda_backward_workspace_bytes",
           "kda_status_str")


class KDAError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH):
    """Load libkda.so (built by `__graft_entry__.build()` or
    `python kimi_delta_attention_kda_amd/build.py`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise KDAError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    Z = ctypes.c_size_t
    lib.kda_chunk_fwd.argtypes = [P, P, P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, F, I, P, Z, P]
    lib.kda_chunk_fwd.restype = I
    lib.kda_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, F, I, P]
    lib.kda_chunk_fwd_noalloc.restype = I
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.kda_chunk_fwd_workspace_bytes.restype = Z
    lib.kda_chunk_fwd_pool.argtypes = [P, P, P, P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, I, P, Z, P]
    lib.kda_chunk_fwd_pool.restype = I
    lib.kda_chunk_fwd_states.argtypes = [P, P, P, P, P, P, P, P, P, I, P, P, P, I, I, I, I, I, I, F, I, P, Z, P]
    lib.kda_chunk_fwd_states.restype = I
    lib.kda_decode_step.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P]
    lib.kda_decode_step.restype = I
    lib.kda_decode_extend.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.kda_decode_extend.restype = I
    lib.kda_conv_decode_step.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.kda_conv_decode_step.restype = I
    lib.kda_chunk_o.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.kda_chunk_o.restype = I
    lib.kda_backward_workspace_bytes.argtypes = [I, I, I, I, ctypes.c_int64]
    lib.kda_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_backward.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                 ctypes.c_size_t, I, I, I, I, I, I, F, I, P]
    lib.kda_backward.restype = I
    lib.kda_device_check.argtypes = [P]
    lib.kda_device_check.restype = I
    lib.kda_status_str.argtypes = [I]
    lib.kda_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise KDAError(f"libkda error {rc}: {load_library().kda_status_str(rc).decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(name, t, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise KDAError(f"{name} must be a GPU tensor (no CPU path exists)")
    if not t.is_contiguous():
        raise KDAError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise KDAError(f"{name} must be {dtype}, got {t.dtype}")


_CU_COUNT = {}


def chunk_fwd_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, n_seq: int, packed: bool) -> int:
    """Workspace bytes for the two-pass prefill (kda_chunk_fwd_workspace_bytes)."""
    return int(load_library().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, n_seq, int(bool(packed))))


def _workspace(workspace, act, B, T, H, dk, dv, n_seq, packed, device):
    """(pointer, bytes) of the prefill workspace.  "auto": allocate one (torch's
    caching allocator) when the two-pass form applies (bf16, fewer (sequence,
    head) chains than compute units); None: no workspace (one-pass form); a
    uint8 GPU tensor: used as given."""
    if workspace is None:
        return None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise KDAError('workspace must be "auto", None or a uint8 GPU tensor')
        if act != torch.bfloat16:
            return None, 0
        idx = device.index if device.index is not None else torch.cuda.current_device()
        if idx not in _CU_COUNT:
            _CU_COUNT[idx] = torch.cuda.get_device_properties(idx).multi_processor_count
        if n_seq * H >= _CU_COUNT[idx]:
            return None, 0
        nbytes = chunk_fwd_workspace_bytes(B, T, H, dk, dv, n_seq, packed)
        if nbytes == 0:
            return None, 0
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _dev("workspace", workspace, torch.uint8)
    return _ptr(workspace), workspace.numel()


def _state_shapes(o, h0, h_T, B, T, H, dk, dv, n_seq):
    if o.numel() != B * T * H * dv:
        raise KDAError("o must hold [B, T, H, dv] elements")
    for name, t in (("h0", h0), ("h_T", h_T)):
        if t is not None and t.numel() != n_seq * H * dv * dk:
            raise KDAError(f"{name} must hold [N, H, dv, dk] elements")


def _prefill_outputs(q, k, v, g_raw, beta_raw, A_log, dt_bias, h0, cu_seqlens, scale, output_final_state, o, h_T):
    """Shared argument checks of the prefill entry points: returns
    (B, T, H, dk, dv, n_seq, act, scale, o, h_T) with o / h_T allocated if None."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    act = q.dtype
    if act not in (torch.float32, torch.bfloat16):
        raise KDAError("activations must be float32 or bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw)):
        _dev(name, t, act)
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("h0", h0)):
        _dev(name, t, torch.float32)
    _dev("cu_seqlens", cu_seqlens, torch.int32)
    if k.shape != q.shape or g_raw.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or tuple(beta_raw.shape) != (B, T, H):
        raise KDAError("inconsistent activation shapes")
    n_seq = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if scale is None:
        scale = dk ** -0.5
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=act, device=q.device)
    _dev("o", o, act)
    if output_final_state and h_T is None:
        h_T = torch.empty((n_seq, H, dv, dk), dtype=torch.float32, device=q.device)
    _dev("h_T", h_T, torch.float32)
    _state_shapes(o, h0, h_T, B, T, H, dk, dv, n_seq)
    return B, T, H, dk, dv, n_seq, act, scale, o, h_T


def chunk_fwd(q, k, v, g_raw, beta_raw, A_log, dt_bias, h0=None, cu_seqlens=None,
              chunk: int = 16, scale=None, output_final_state: bool = True,
              o=None, h_T=None, stream=None, workspace="auto"):
    """Chunkwise KDA prefill.

    q, k, g_raw: [B, T, H, dk]; v: [B, T, H, dv]; beta_raw: [B, T, H] -- all
    float32 or all bfloat16 (q, k L2-normalised by the caller).
    A_log: [H] float32; dt_bias: [H, dk] float32.
    h0: [N, H, dv, dk] float32 or None.  cu_seqlens: [N+1] int32 (then B == 1).
    workspace: "auto", None (one-pass form) or a uint8 GPU tensor (see _workspace).
    Returns (o [B, T, H, dv], h_T [N, H, dv, dk] float32 or None)."""
    B, T, H, dk, dv, n_seq, act, scale, o, h_T = _prefill_outputs(
        q, k, v, g_raw, beta_raw, A_log, dt_bias, h0, cu_seqlens, scale, output_final_state, o, h_T)
    wsp, wsb = _workspace(workspace, act, B, T, H, dk, dv, n_seq, cu_seqlens is not None, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(load_library().kda_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw), _ptr(A_log), _ptr(dt_bias),
        _ptr(h0), _ptr(cu_seqlens), chunk, _ptr(o), _ptr(h_T), B, T, H, dk, dv, n_seq,
        float(scale), KDA_BF16 if act == torch.bfloat16 else KDA_F32, wsp, wsb, ctypes.c_void_p(stream)))
    return o, h_T


def chunk_fwd_noalloc(q, k, v, g_raw, beta_raw, A_log, dt_bias, h0=None, cu_seqlens=None,
                      chunk: int = 16, scale=None, o=None, h_T=None, stream=None):
    """kda_chunk_fwd_noalloc: chunk_fwd with its workspace taken from the
    library's fixed device array (NOALLOC_SCRATCH_BYTES per GPU) instead of an
    allocation.  o and h_T must be passed (this call allocates nothing); h_T may
    be None only if the final states are not wanted.  Calls that overlap on one
    GPU race.  Raises KDAError (KDA_ERR_SCRATCH) when the two-pass form would
    need more than the array."""
    if o is None:
        raise KDAError("chunk_fwd_noalloc allocates nothing: pass o (and h_T)")
    B, T, H, dk, dv, n_seq, act, scale, o, h_T = _prefill_outputs(
        q, k, v, g_raw, beta_raw, A_log, dt_bias, h0, cu_seqlens, scale, False, o, h_T)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(load_library().kda_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw), _ptr(A_log), _ptr(dt_bias),
        _ptr(h0), _ptr(cu_seqlens), chunk, _ptr(o), _ptr(h_T), B, T, H, dk, dv, n_seq,
        float(scale), KDA_BF16 if act == torch.bfloat16 else KDA_F32, ctypes.c_void_p(stream)))
    return o, h_T


def chunk_fwd_pool(q, k, v, g_raw, beta_raw, A_log, dt_bias, state_pool, state_idx,
                   cu_seqlens=None, chunk: int = 16, scale=None, o=None, stream=None, workspace="auto"):
    """Chunkwise KDA prefill with the states in a decode state pool.

    As chunk_fwd, but sequence s starts from state_pool[state_idx[s]] and its
    final state is written back there in place (state_idx[s] < 0: zero start,
    final state dropped).  state_pool: [P, H, dv, dk] float32 (the layout of
    decode_step's pool); state_idx: [N] int32 with distinct live entries.
    Returns o [B, T, H, dv]."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    act = q.dtype
    if act not in (torch.float32, torch.bfloat16):
        raise KDAError("activations must be float32 or bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw)):
        _dev(name, t, act)
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("state_pool", state_pool)):
        _dev(name, t, torch.float32)
    _dev("state_idx", state_idx, torch.int32)
    _dev("cu_seqlens", cu_seqlens, torch.int32)
    if k.shape != q.shape or g_raw.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or tuple(beta_raw.shape) != (B, T, H):
        raise KDAError("inconsistent activation shapes")
    n_seq = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, dv, dk):
        raise KDAError("state_pool must be [P, H, dv, dk]")
    if state_idx.numel() != n_seq:
        raise KDAError("state_idx must hold one slot per sequence")
    if scale is None:
        scale = dk ** -0.5
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=act, device=q.device)
    _dev("o", o, act)
    wsp, wsb = _workspace(workspace, act, B, T, H, dk, dv, n_seq, cu_seqlens is not None, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(load_library().kda_chunk_fwd_pool(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw), _ptr(A_log), _ptr(dt_bias),
        _ptr(state_pool), _ptr(state_idx), _ptr(cu_seqlens), chunk, _ptr(o), B, T, H, dk, dv, n_seq,
        state_pool.shape[0], float(scale), KDA_BF16 if act == torch.bfloat16 else KDA_F32,
        wsp, wsb, ctypes.c_void_p(stream)))
    return o


KDA_ERR_SLOT = -6
KDA_ERR_SCRATCH = -7
NOALLOC_SCRATCH_BYTES = 64 << 20   # KDA_NOALLOC_SCRATCH_BYTES


def device_check(stream=None) -> int:
    """Synchronise the stream, then read and clear the device error word:
    returns 0, or KDA_ERR_SLOT (-6) if a kernel met a pool slot index >= P
    since the last check (those rows were handled as pads)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = load_library().kda_device_check(ctypes.c_void_p(stream))
    if rc not in (0, KDA_ERR_SLOT):
        _check(rc)
    return rc


def decode_step(qkv, a, b, A_log, dt_bias, state_pool, state_idx, num_heads: int,
                num_v_heads: int, head_k_dim: int = 128, head_v_dim: int = 128, scale=None,
                l2norm: bool = True, o=None, stream=None):
    """One fused T=1 decode step; `state_pool` [P, HV, V, K] float32 is updated
    in place.  qkv: [B, 2*H*K + HV*V] bf16; a: [B, HV*K] bf16; b: [B, HV] bf16;
    A_log: [HV] f32; dt_bias: [HV*K] f32; state_idx: [B] int32 (< 0 = pad).
    Returns o [B, HV, V] bf16."""
    B = qkv.shape[0]
    H, HV, K, V = num_heads, num_v_heads, head_k_dim, head_v_dim
    for name, t in (("qkv", qkv), ("a", a), ("b", b)):
        _dev(name, t, torch.bfloat16)
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("state_pool", state_pool)):
        _dev(name, t, torch.float32)
    _dev("state_idx", state_idx, torch.int32)
    if qkv.shape[-1] != 2 * H * K + HV * V or a.numel() != B * HV * K or b.numel() != B * HV \
            or tuple(state_pool.shape[1:]) != (HV, V, K) or state_idx.numel() != B \
            or A_log.numel() != HV or dt_bias.numel() != HV * K:
        raise KDAError("inconsistent decode shapes")
    if scale is None:
        scale = K ** -0.5
    if o is None:
        o = torch.empty((B, HV, V), dtype=torch.bfloat16, device=qkv.device)
    _dev("o", o, torch.bfloat16)
    if o.numel() != B * HV * V:
        raise KDAError("o must hold [B, HV, V] elements")
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device).cuda_stream
    _check(load_library().kda_decode_step(
        _ptr(qkv), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(state_pool),
        _ptr(state_idx), _ptr(o), B, H, HV, K, V, state_pool.shape[0], float(scale),
        KDA_DECODE_L2NORM if l2norm else 0, ctypes.c_void_p(stream)))
    return o


def decode_extend(qkv, a, b, A_log, dt_bias, state_pool, state_idx, num_heads: int,
                  num_v_heads: int, head_k_dim: int = 128, head_v_dim: int = 128, scale=None,
                  l2norm: bool = True, o=None, stream=None):
    """T tokens per row through the decode update in one launch; `state_pool`
    [P, HV, V, K] float32 is updated in place and ends holding each live row's
    state after its last token.  qkv: [B, T, 2*H*K + HV*V] bf16; a: [B, T, HV*K]
    bf16; b: [B, T, HV] bf16; A_log: [HV] f32; dt_bias: [HV*K] f32; state_idx:
    [B] int32 (< 0 = pad).  Returns o [B, T, HV, V] bf16."""
    if qkv.dim() != 3:
        raise KDAError("qkv must be [B, T, 2*H*K + HV*V]")
    B, T = qkv.shape[0], qkv.shape[1]
    H, HV, K, V = num_heads, num_v_heads, head_k_dim, head_v_dim
    for name, t in (("qkv", qkv), ("a", a), ("b", b)):
        _dev(name, t, torch.bfloat16)
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("state_pool", state_pool)):
        _dev(name, t, torch.float32)
    _dev("state_idx", state_idx, torch.int32)
    if qkv.shape[-1] != 2 * H * K + HV * V or a.numel() != B * T * HV * K or b.numel() != B * T * HV \
            or tuple(state_pool.shape[1:]) != (HV, V, K) or state_idx.numel() != B \
            or A_log.numel() != HV or dt_bias.numel() != HV * K:
        raise KDAError("inconsistent decode-extend shapes")
    if scale is None:
        scale = K ** -0.5
    if o is None:
        o = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=qkv.device)
    _dev("o", o, torch.bfloat16)
    if o.numel() != B * T * HV * V:
        raise KDAError("o must hold [B, T, HV, V] elements")
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device).cuda_stream
    _check(load_library().kda_decode_extend(
        _ptr(qkv), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(state_pool),
        _ptr(state_idx), _ptr(o), B, T, H, HV, K, V, state_pool.shape[0], float(scale),
        KDA_DECODE_L2NORM if l2norm else 0, ctypes.c_void_p(stream)))
    return o


def conv_decode_step(mixed_qkv, conv_state, conv_weight, conv_bias, a, b, A_log, dt_bias,
                     state_pool, state_idx, num_heads: int, num_v_heads: int, head_k_dim: int = 128,
                     head_v_dim: int = 128, scale=None, l2norm: bool = True, o=None, stream=None):
    """The short causal convolution (silu) fused with one decode step; both
    `conv_state` [P, W-1, D] bf16 and `state_pool` [P, HV, V, K] float32 are
    updated in place for the live rows.  mixed_qkv: [B, D] bf16 before the
    conv; conv_weight: [D, W] bf16; conv_bias: [D] bf16 or None; the other
    arguments as in decode_step.  Returns o [B, HV, V] bf16."""
    B = mixed_qkv.shape[0]
    H, HV, K, V = num_heads, num_v_heads, head_k_dim, head_v_dim
    D = 2 * H * K + HV * V
    for name, t in (("mixed_qkv", mixed_qkv), ("conv_state", conv_state), ("conv_weight", conv_weight),
                    ("conv_bias", conv_bias), ("a", a), ("b", b)):
        _dev(name, t, torch.bfloat16)
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("state_pool", state_pool)):
        _dev(name, t, torch.float32)
    _dev("state_idx", state_idx, torch.int32)
    if conv_weight.dim() != 2 or conv_weight.shape[0] != D:
        raise KDAError("conv_weight must be [D, W]")
    W = conv_weight.shape[1]
    P = state_pool.shape[0]
    if mixed_qkv.shape[-1] != D or mixed_qkv.numel() != B * D or a.numel() != B * HV * K \
            or b.numel() != B * HV or tuple(state_pool.shape[1:]) != (HV, V, K) \
            or state_idx.numel() != B or A_log.numel() != HV or dt_bias.numel() != HV * K \
            or tuple(conv_state.shape) != (P, W - 1, D) \
            or (conv_bias is not None and conv_bias.numel() != D):
        raise KDAError("inconsistent conv-decode shapes")
    if scale is None:
        scale = K ** -0.5
    if o is None:
        o = torch.empty((B, HV, V), dtype=torch.bfloat16, device=mixed_qkv.device)
    _dev("o", o, torch.bfloat16)
    if o.numel() != B * HV * V:
        raise KDAError("o must hold [B, HV, V] elements")
    if stream is None:
        stream = torch.cuda.current_stream(mixed_qkv.device).cuda_stream
    _check(load_library().kda_conv_decode_step(
        _ptr(mixed_qkv), _ptr(conv_state), _ptr(conv_weight), _ptr(conv_bias), _ptr(a), _ptr(b),
        _ptr(A_log), _ptr(dt_bias), _ptr(state_pool), _ptr(state_idx), _ptr(o), B, H, HV, K, V, W, P,
        float(scale), KDA_DECODE_L2NORM if l2norm else 0, ctypes.c_void_p(stream)))
    return o


def n_chunks(T: int, B: int = 1, cu_seqlens=None, chunk: int = 16) -> int:
    """Rows of the materialised chunk states: sum over sequences of
    ceil(len / chunk) (reads cu_seqlens back to the host if given)."""
    if cu_seqlens is None:
        return B * ((T + chunk - 1) // chunk)
    lens = torch.diff(cu_seqlens.detach().to("cpu", torch.int64))
    return int(((lens + chunk - 1) // chunk).sum())


def chunk_fwd_states(q, k, v, g_raw, beta_raw, A_log, dt_bias, h0=None, cu_seqlens=None,
                     chunk: int = 16, scale=None, output_final_state: bool = True, o=None,
                     h_T=None, h_chunks=None, stream=None, workspace="auto"):
    """chunk_fwd that also returns the state entering every chunk.
    Returns (o, h_T, h_chunks [N_chunks, H, dv, dk] float32)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    act = q.dtype
    if act not in (torch.float32, torch.bfloat16):
        raise KDAError("activations must be float32 or bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw)):
        _dev(name, t, act)
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("h0", h0)):
        _dev(name, t, torch.float32)
    _dev("cu_seqlens", cu_seqlens, torch.int32)
    if k.shape != q.shape or g_raw.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or tuple(beta_raw.shape) != (B, T, H):
        raise KDAError("inconsistent activation shapes")
    n_seq = B if cu_seqlens is None else cu_seqlens.numel() - 1
    nc = n_chunks(T, B, cu_seqlens, chunk)
    if scale is None:
        scale = dk ** -0.5
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=act, device=q.device)
    _dev("o", o, act)
    if output_final_state and h_T is None:
        h_T = torch.empty((n_seq, H, dv, dk), dtype=torch.float32, device=q.device)
    _dev("h_T", h_T, torch.float32)
    if h_chunks is None:
        h_chunks = torch.empty((nc, H, dv, dk), dtype=torch.float32, device=q.device)
    _dev("h_chunks", h_chunks, torch.float32)
    if h_chunks.numel() != nc * H * dv * dk:
        raise KDAError("h_chunks must hold [N_chunks, H, dv, dk] elements")
    _state_shapes(o, h0, h_T, B, T, H, dk, dv, n_seq)
    wsp, wsb = _workspace(workspace, act, B, T, H, dk, dv, n_seq, cu_seqlens is not None, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(load_library().kda_chunk_fwd_states(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw), _ptr(A_log), _ptr(dt_bias),
        _ptr(h0), _ptr(cu_seqlens), chunk, _ptr(o), _ptr(h_T), _ptr(h_chunks), B, T, H, dk, dv, n_seq,
        float(scale), KDA_BF16 if act == torch.bfloat16 else KDA_F32, wsp, wsb, ctypes.c_void_p(stream)))
    return o, h_T, h_chunks


def chunk_o(q, k, v, g_raw, beta_raw, A_log, dt_bias, h_chunks, cu_seqlens=None, scale=None, o=None,
            stream=None):
    """The chunk-parallel output pass of the materialised form (kda_chunk_o):
    every chunk's outputs from its state in h_chunks, one workgroup per
    (chunk, head).  bfloat16, dk = dv = 128.  Returns o [B, T, H, dv]."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw)):
        _dev(name, t, torch.bfloat16)
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("h_chunks", h_chunks)):
        _dev(name, t, torch.float32)
    _dev("cu_seqlens", cu_seqlens, torch.int32)
    if k.shape != q.shape or g_raw.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or tuple(beta_raw.shape) != (B, T, H):
        raise KDAError("inconsistent activation shapes")
    n_seq = B if cu_seqlens is None else cu_seqlens.numel() - 1
    nc = n_chunks(T, B, cu_seqlens)
    if h_chunks.numel() != nc * H * dv * dk:
        raise KDAError("h_chunks must hold [N_chunks, H, dv, dk] elements")
    if scale is None:
        scale = dk ** -0.5
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    _dev("o", o, torch.bfloat16)
    if o.numel() != B * T * H * dv:
        raise KDAError("o must hold [B, T, H, dv] elements")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(load_library().kda_chunk_o(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw), _ptr(A_log), _ptr(dt_bias), _ptr(h_chunks),
        _ptr(cu_seqlens), _ptr(o), B, T, H, dk, dv, n_seq, nc, float(scale), KDA_BF16, ctypes.c_void_p(stream)))
    return o


def chunk_o_from_states(q, k, v, g_raw, beta_raw, A_log, dt_bias, h_chunks, cu_seqlens=None,
                        chunk: int = 16, scale=None, o=None, stream=None):
    """The chunk-parallel output pass of the materialised form through
    kda_chunk_fwd: every chunk as a sequence of its own, started from its
    state in h_chunks (so all chunks are independent chains; bitwise the
    outputs of kda_chunk_fwd).  Dense input with T % chunk == 0 is passed as
    B*T/chunk sequences of `chunk` tokens (same buffers); otherwise chunk
    boundaries are passed as cu_seqlens.  Returns o."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None and T % chunk == 0:
        nb = B * T // chunk
        shp = lambda x: x.view(nb, chunk, *x.shape[2:])
        o_ = None if o is None else shp(o)
        out, _ = chunk_fwd(shp(q), shp(k), shp(v), shp(g_raw), shp(beta_raw), A_log, dt_bias, h0=h_chunks,
                           chunk=chunk, scale=scale, output_final_state=False, o=o_, stream=stream)
        return out.view(B, T, H, dv)
    if cu_seqlens is None:
        bounds = [(s * T, (s + 1) * T) for s in range(B)]
    else:
        cu = cu_seqlens.detach().to("cpu", torch.int64).tolist()
        bounds = list(zip(cu[:-1], cu[1:]))
    edges = [0]
    for bos, eos in bounds:
        for st in range(bos, eos, chunk):
            edges.append(min(st + chunk, eos))
    ccu = torch.tensor(edges, dtype=torch.int32, device=q.device)
    flat = lambda x: x.reshape(1, B * T, *x.shape[2:])
    o_ = None if o is None else flat(o)
    out, _ = chunk_fwd(flat(q), flat(k), flat(v), flat(g_raw), flat(beta_raw), A_log, dt_bias, h0=h_chunks,
                       cu_seqlens=ccu, chunk=chunk, scale=scale, output_final_state=False, o=o_, stream=stream)
    return out.view(B, T, H, dv)


def backward(q, k, v, g_raw, beta_raw, A_log, dt_bias, h_chunks, do, dh_T=None, cu_seqlens=None,
             scale=None, workspace=None, stream=None):
    """Gradients of the chunkwise forward (see kda_backward in include/kda.h).
    q, k, v, g_raw, beta_raw, A_log, dt_bias, cu_seqlens, scale: as given to
    chunk_fwd_states; h_chunks: its third output; do: [B, T, H, dv] (the
    activation dtype); dh_T: [N, H, dv, dk] float32 or None.  Returns a dict:
    dq, dk, dv, dg_raw, dbeta_raw (activation dtype, shaped like their
    inputs), dA_log [H], ddt_bias [H, dk], dh0 [N, H, dv, dk] (float32)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    act = q.dtype
    if act not in (torch.float32, torch.bfloat16):
        raise KDAError("activations must be float32 or bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw), ("do", do)):
        _dev(name, t, act)
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("h_chunks", h_chunks), ("dh_T", dh_T)):
        _dev(name, t, torch.float32)
    _dev("cu_seqlens", cu_seqlens, torch.int32)
    if k.shape != q.shape or g_raw.shape != q.shape or v.shape[:3] != q.shape[:3] or do.shape != v.shape \
            or tuple(beta_raw.shape) != (B, T, H):
        raise KDAError("inconsistent activation shapes")
    n_seq = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if h_chunks.numel() != n_chunks(T, B, cu_seqlens) * H * dv * dk:
        raise KDAError("h_chunks must hold [N_chunks, H, dv, dk] elements")
    if dh_T is not None and dh_T.numel() != n_seq * H * dv * dk:
        raise KDAError("dh_T must hold [N, H, dv, dk] elements")
    if scale is None:
        scale = dk ** -0.5
    lib = load_library()
    need = lib.kda_backward_workspace_bytes(n_seq, H, dk, dv, B * T)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev("workspace", workspace)
    dev = q.device
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dg_raw=torch.empty_like(g_raw), dbeta_raw=torch.empty_like(beta_raw),
               dA_log=torch.empty((H,), dtype=torch.float32, device=dev),
               ddt_bias=torch.empty((H, dk), dtype=torch.float32, device=dev),
               dh0=torch.empty((n_seq, H, dv, dk), dtype=torch.float32, device=dev))
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _check(lib.kda_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw), _ptr(A_log), _ptr(dt_bias), _ptr(h_chunks),
        _ptr(cu_seqlens), _ptr(do), _ptr(dh_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
        _ptr(out["dg_raw"]), _ptr(out["dbeta_raw"]), _ptr(out["dA_log"]), _ptr(out["ddt_bias"]),
        _ptr(out["dh0"]), _ptr(workspace), workspace.numel() * workspace.element_size(), B, T, H, dk, dv,
        n_seq, float(scale), KDA_BF16 if act == torch.bfloat16 else KDA_F32, ctypes.c_void_p(stream)))
    return out


def backward_workspace_bytes(n_seq: int, H: int, total_tokens: int, dk: int = 128, dv: int = 128) -> int:
    """Bytes of device workspace kda_backward needs (0: unsupported shape)."""
    return int(load_library().kda_backward_workspace_bytes(n_seq, H, dk, dv, total_tokens))
