"""GPU parity of kda_chunk_fwd against the fp64 oracle (through the C ABI),
plus properties that must hold exactly: determinism, chunk-aligned
continuation and varlen = separate runs are bitwise; continuation at an
unaligned split and decode-vs-prefill agree within tolerance."""
import math

import numpy as np
import pytest
import torch

import kimi_delta_attention_kda_amd as kda
import synth
from kda_testlib import assert_close, full_parity, metrics, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def check(p, heads=None, seqs=None, what="", workspace="auto"):
    say(what or p.name, "shapes", p.tokens, p.H, p.dk, p.dv, p.dtype)
    o, hT = run_gpu(p, workspace=workspace)
    ro, rh = run_oracle(p, heads, seqs)
    if heads is not None:
        o, hT = o[:, heads], hT[:, heads]
    if seqs is not None:
        off = p.offsets()
        rows = np.concatenate([np.arange(off[s], off[s + 1]) for s in seqs])
        o, ro, hT, rh = o[rows], ro[rows], hT[seqs], rh[seqs]
    mo = assert_close(o, ro, p.dtype, what + " o")
    mh = assert_close(hT, rh, p.dtype, what + " h_T")
    say("  o", mo, " h_T", mh)
    return mo, mh


def test_workload0_tiny_fp32():
    check(synth.prefill_workload(0), what="tiny-f32")


SMALL = [
    dict(B=2, T=100, H=3, dk=128, dv=128, dtype="bf16", with_h0=True),
    dict(B=1, T=37, H=2, dk=64, dv=64, dtype="bf16"),
    dict(B=1, T=53, H=2, dk=128, dv=64, dtype="bf16", with_h0=True),
    dict(B=1, T=40, H=2, dk=64, dv=128, dtype="bf16"),
    dict(B=3, T=33, H=2, dk=64, dv=64, dtype="f32", with_h0=True),
    dict(B=1, T=0, H=2, dk=128, dv=128, dtype="bf16", lengths=[1, 16, 17, 0, 45, 130]),
    dict(B=1, T=200, H=4, dk=128, dv=128, dtype="bf16", gate_stress=0.05),
    dict(B=1, T=64, H=2, dk=64, dv=64, dtype="f32", gate_stress=0.1, A_log_hi=math.log(64)),
    dict(B=2, T=45, H=2, dk=64, dv=128, dtype="f32", with_h0=True),
    dict(B=1, T=1003, H=2, dk=64, dv=64, dtype="f32", with_h0=True),
]


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_small(i):
    kw = dict(SMALL[i])
    lengths = kw.pop("lengths", None)
    p = synth.prefill(100 + i, lengths=lengths, **kw)
    check(p, what=f"small{i}")


@pytest.mark.parametrize("dtype,dk,dv,H", [("bf16", 128, 128, 2), ("f32", 64, 64, 4)])
def test_many_short_sequences(dtype, dk, dv, H):
    """Packed sequences of 0..40 tokens, more (sequence, head) chains than the
    launch has teams: a team then runs several chains, most shorter than its
    producers' first chunks."""
    lengths = [int(x) for x in np.random.default_rng(7).integers(0, 41, size=24)]
    p = synth.prefill(400, B=1, T=0, H=H, dk=dk, dv=dv, dtype=dtype, lengths=lengths, with_h0=True)
    check(p, what=f"many-short {dtype} d{dk}x{dv} H{H}")


@pytest.mark.parametrize("form", ["one-pass", "two-pass"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64)])
def test_both_prefill_forms(form, dk, dv):
    """The one-pass kernel (no workspace) and the prep + recurrence pair (a
    workspace, fewer chains than compute units) each match the oracle, on a
    ragged packed batch that spans several 16-row prep blocks."""
    p = synth.prefill(500 + dk + dv, B=1, T=0, H=3, dk=dk, dv=dv, dtype="bf16",
                      lengths=[300, 1, 0, 47, 129], with_h0=True)
    if form == "one-pass":
        ws = None
    else:
        n = kda.chunk_fwd_workspace_bytes(1, p.tokens, p.H, dk, dv, p.n_seq, True)
        assert n > 0
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    check(p, what=f"{form} d{dk}x{dv}", workspace=ws)


def test_workload1_full():
    check(synth.prefill_workload(1), what="prefill-bf16 B4 H16 T4096")


def check_full(w, batch):
    """A whole workload, every output element and final state against the
    oracle (run in head batches), in the launch configuration the benchmark
    times (default workspace)."""
    p = synth.prefill_workload(w)
    say(p.name, "tokens", p.tokens, "H", p.H, "full parity, oracle batches of", batch, "heads")
    d = to_device(p)
    o, hT = kda.chunk_fwd(**d, scale=p.scale)
    assert kda.device_check() == 0
    eo, eh = full_parity(p, o, hT, batch)
    mo, mh = eo.check(p.dtype, p.name + " o"), eh.check(p.dtype, p.name + " h_T")
    say("  o", mo, " h_T", mh)


def test_workload2_full():
    check_full(2, batch=8)


def test_workload3_full():
    check_full(3, batch=16)


def test_deterministic_and_continuation():
    p = synth.prefill(7, B=1, T=160, H=2, dk=128, dv=128, dtype="bf16", with_h0=True)
    say("determinism + continuation", p.tokens)
    o1, h1 = run_gpu(p)
    o2, h2 = run_gpu(p)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
    for n, exact in ((64, True), (71, False)):
        a = synth.Prefill(**{**p.__dict__, "T": n, "q": p.q[:n], "k": p.k[:n], "v": p.v[:n],
                             "a": p.a[:n], "b": p.b[:n]})
        oa, ha = run_gpu(a)
        b = synth.Prefill(**{**p.__dict__, "T": p.T - n, "q": p.q[n:], "k": p.k[n:], "v": p.v[n:],
                             "a": p.a[n:], "b": p.b[n:], "h0": ha.astype(np.float32)})
        ob, hb = run_gpu(b)
        if exact:
            assert np.array_equal(np.concatenate([oa, ob]), o1) and np.array_equal(hb, h1)
        else:
            assert_close(np.concatenate([oa, ob]), o1, "bf16", "continuation o")
            assert_close(hb, h1, "bf16", "continuation h")


def test_varlen_equals_separate_runs():
    lengths = [19, 48, 3]
    p = synth.prefill(8, B=1, T=0, H=2, dk=64, dv=64, dtype="bf16", lengths=lengths, with_h0=True)
    say("varlen vs separate", lengths)
    o, hT = run_gpu(p)
    off = p.offsets()
    for s in range(len(lengths)):
        sl = slice(off[s], off[s + 1])
        ps = synth.Prefill(**{**p.__dict__, "B": 1, "T": lengths[s], "q": p.q[sl], "k": p.k[sl],
                              "v": p.v[sl], "a": p.a[sl], "b": p.b[sl], "h0": p.h0[s:s + 1],
                              "cu_seqlens": None})
        os_, hs = run_gpu(ps)
        assert np.array_equal(os_, o[sl]) and np.array_equal(hs[0], hT[s])


def test_zero_length_sequence_keeps_h0():
    p = synth.prefill(9, B=1, T=0, H=2, dk=128, dv=128, dtype="bf16", lengths=[0, 5], with_h0=True)
    say("zero-length sequence")
    o, hT = run_gpu(p)
    assert np.array_equal(hT[0], p.h0[0].astype(np.float64))


def test_prefill_graph_replay():
    """kda_chunk_fwd recorded in a HIP graph (its flag clear is a fill kernel,
    not a memset): every replay, with eager prefills in between, equals the
    eager result bitwise."""
    p = synth.prefill(78, B=2, T=300, H=4, dk=128, dv=128, dtype="bf16", with_h0=True)
    d = to_device(p)
    print("[case] prefill graph replay B2 T300 H4", flush=True)
    o_ref, h_ref = kda.chunk_fwd(**d, scale=p.scale)     # also sets up the library's workspace
    assert kda.device_check() == 0
    o, hT = torch.empty_like(o_ref), torch.empty_like(h_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.chunk_fwd(**d, scale=p.scale, o=o, h_T=hT)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kda.chunk_fwd(**d, scale=p.scale, o=o, h_T=hT)
    for _ in range(4):
        o.zero_()
        hT.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert kda.device_check() == 0
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
        o2, h2 = kda.chunk_fwd(**d, scale=p.scale)       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o2, o_ref) and torch.equal(h2, h_ref)
    del g
