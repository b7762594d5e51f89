"""GPU test of kda_chunk_fwd_noalloc (through the C ABI): the allocation-free
prefill equals kda_chunk_fwd bit for bit on two calls in a row, the second
with a smaller input (the fixed scratch array keeps the first call's bytes),
in both launch forms (two passes through the scratch array; one pass with
no workspace), matches the oracle, and refuses, launching nothing, a call
whose two-pass workspace would not fit the array."""
import ctypes

import numpy as np
import pytest
import torch

import kimi_delta_attention_kda_amd as kda
import synth
from kda_testlib import assert_close, run_oracle, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def both(p):
    d = to_device(p)
    o_ref, h_ref = kda.chunk_fwd(**d, scale=p.scale)       # the existing entry point, workspace "auto"
    o = torch.full_like(o_ref, 7.0)
    hT = torch.full_like(h_ref, 7.0)
    kda.chunk_fwd_noalloc(**d, scale=p.scale, o=o, h_T=hT)
    assert kda.device_check() == 0
    return (o, hT), (o_ref, h_ref)


def test_noalloc_two_calls_then_smaller():
    for i, (lengths, H) in enumerate((([700, 45, 300, 1], 3), ([33, 5], 2))):
        p = synth.prefill(800 + i, B=1, T=0, H=H, dk=128, dv=128, dtype="bf16", lengths=lengths, with_h0=True)
        need = kda.chunk_fwd_workspace_bytes(1, p.tokens, H, 128, 128, p.n_seq, True)
        say("noalloc call", i, "lengths", lengths, "H", H, "workspace bytes", need)
        assert 0 < need <= kda.NOALLOC_SCRATCH_BYTES
        (o, hT), (o_ref, h_ref) = both(p)
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref), f"call {i}: differs from kda_chunk_fwd"
        ro, rh = run_oracle(p)
        assert_close(o.float().cpu().numpy().reshape(p.tokens, H, 128), ro, "bf16", f"call {i} o")
        assert_close(hT.cpu().numpy(), rh, "bf16", f"call {i} h_T")


def test_noalloc_many_chains_one_pass():
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    B, H = (n_cu + 7) // 8, 8
    p = synth.prefill(810, B=B, T=40, H=H, dk=64, dv=64, dtype="bf16")
    say("noalloc one-pass chains", B * H, "CUs", n_cu)
    (o, hT), (o_ref, h_ref) = both(p)
    assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)


def test_noalloc_refuses_beyond_scratch():
    T, H = 65536, 2
    need = kda.chunk_fwd_workspace_bytes(1, T, H, 128, 128, 1, False)
    assert need > kda.NOALLOC_SCRATCH_BYTES
    say("noalloc refusal", "T", T, "H", H, "needs", need)
    x = torch.zeros((1, T, H, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((1, T, H), dtype=torch.bfloat16, device="cuda")
    A_log = torch.zeros(H, dtype=torch.float32, device="cuda")
    dt = torch.zeros((H, 128), dtype=torch.float32, device="cuda")
    o = torch.full((1, T, H, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = kda.load_library().kda_chunk_fwd_noalloc(
        ptr(x), ptr(x), ptr(x), ptr(x), ptr(b), ptr(A_log), ptr(dt), None, None, 16, ptr(o), None,
        1, T, H, 128, 128, 1, ctypes.c_float(128 ** -0.5), 1, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == kda.KDA_ERR_SCRATCH
    assert bool((o == 3.0).all()), "a refused call must launch nothing"
