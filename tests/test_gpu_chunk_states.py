"""GPU parity of the materialised form (kda_chunk_fwd_states, then the
chunk-parallel output pass), through the C ABI:
- the stored state entering every chunk matches the fp64 oracle's states at
  chunk boundaries (dense, packed variable-length, fp32 and bf16, with and
  without h0, and the full prefill workload on sampled heads);
- the outputs and final states are bitwise those of kda_chunk_fwd;
- the chunk-parallel pass through kda_chunk_fwd (every chunk its own chain,
  started from its stored state) reproduces the outputs bitwise;
- the dedicated chunk-parallel kernel (kda_chunk_o, bf16 d = 128) matches the
  oracle's outputs within the bf16 tolerance."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_kda_amd as kda
import synth
from kda_testlib import assert_close, metrics, run_oracle, to_device

pytestmark = pytest.mark.gpu

CH = 16


def say(*a):
    print("[case]", *a, flush=True)


def oracle_states(p, heads=None):
    f = p.f64(heads)
    import oracle
    return oracle.fwd(f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], h0=f["h0"],
                      cu_seqlens=f["cu_seqlens"], scale=f["scale"], chunk_states=CH)


def check_states(p, heads=None, what=""):
    say(what, "tokens", p.tokens, "H", p.H, "dk", p.dk, "dv", p.dv, p.dtype)
    d = to_device(p)
    o1, hT1 = kda.chunk_fwd(**d, scale=p.scale)
    o2, hT2, hc = kda.chunk_fwd_states(**d, scale=p.scale)
    assert kda.device_check() == 0
    assert torch.equal(o1, o2) and torch.equal(hT1, hT2), what + ": outputs differ from kda_chunk_fwd"
    # chunk-parallel output pass from the stored states
    dd = {k_: v_ for k_, v_ in d.items() if k_ != "h0"}
    o3 = kda.chunk_o_from_states(**dd, h_chunks=hc, scale=p.scale)
    assert kda.device_check() == 0
    assert torch.equal(o1, o3), what + ": chunk-parallel pass differs"
    if p.dtype == "bf16" and p.dk == 128 and p.dv == 128:
        o4 = kda.chunk_o(**dd, h_chunks=hc, scale=p.scale)
        torch.cuda.synchronize()
        ro, _ = run_oracle(p, heads)
        hs_ = slice(None) if heads is None else list(heads)
        got4 = o4.float().cpu().numpy().reshape(p.tokens, p.H, p.dv)[:, hs_].astype(np.float64)
        m4 = assert_close(got4, ro, p.dtype, what + " kda_chunk_o")
        got1 = o1.float().cpu().numpy().reshape(p.tokens, p.H, p.dv)[:, hs_].astype(np.float64)
        say("  kda_chunk_o", m4, " vs fused", metrics(got4, got1))
    hs = slice(None) if heads is None else list(heads)
    got = hc[:, hs].cpu().numpy().astype(np.float64)
    _, _, want = oracle_states(p, heads)
    m = assert_close(got, want, p.dtype, what + " h_chunks")
    say("  h_chunks", m, "rows", got.shape[0])


SMALL = [
    dict(B=2, T=100, H=3, dk=128, dv=128, dtype="bf16", with_h0=True),
    dict(B=1, T=64, H=2, dk=128, dv=64, dtype="bf16"),
    dict(B=3, T=33, H=2, dk=64, dv=64, dtype="f32", with_h0=True),
    dict(B=1, T=0, H=2, dk=128, dv=128, dtype="bf16", lengths=[1, 16, 17, 0, 45, 130], with_h0=True),
    dict(B=2, T=48, H=2, dk=64, dv=128, dtype="bf16", gate_stress=0.05),
    # strong decays at d = 128: the chunk-parallel kernel's running decay products underflow
    dict(B=2, T=70, H=2, dk=128, dv=128, dtype="bf16", gate_stress=0.05, with_h0=True),
]


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_states_small(i):
    kw = dict(SMALL[i])
    lengths = kw.pop("lengths", None)
    p = synth.prefill(300 + i, lengths=lengths, **kw)
    check_states(p, what=f"states small{i}")


def test_states_workload1_full():
    """All heads: the stored states (1 GiB on the device, 2 GiB as fp64 on the
    host) and kda_chunk_o's outputs against the oracle."""
    check_states(synth.prefill_workload(1), heads=None, what="states prefill-bf16 B4 H16 T4096")


def test_chunk_o_extra_rows_skipped():
    """kda_chunk_o with packed sequences reads the lengths on the device: a
    row count above theirs (from a C caller) leaves the extra workgroups idle
    and the outputs unchanged."""
    import ctypes
    p = synth.prefill(320, B=1, T=0, H=2, dk=128, dv=128, dtype="bf16", lengths=[5, 33, 16, 0, 21])
    d = to_device(p)
    say("chunk_o extra rows", "tokens", p.tokens)
    _, _, hc = kda.chunk_fwd_states(**d, scale=p.scale)
    dd = {k_: v_ for k_, v_ in d.items() if k_ != "h0"}
    o_ref = kda.chunk_o(**dd, h_chunks=hc, scale=p.scale)
    torch.cuda.synchronize()
    o2 = torch.zeros_like(o_ref)
    B, T, H, dk = d["q"].shape
    nc = hc.shape[0]
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = kda.load_library().kda_chunk_o(
        ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["g_raw"]), ptr(d["beta_raw"]), ptr(d["A_log"]),
        ptr(d["dt_bias"]), ptr(hc), ptr(d["cu_seqlens"]), ptr(o2), B, T, H, dk, 128,
        d["cu_seqlens"].numel() - 1, nc + 7, ctypes.c_float(p.scale), 1,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(o2, o_ref)
