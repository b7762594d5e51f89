"""GPU parity of kda_backward (through the C ABI) against the fp64 autograd
gradients of the oracle's recurrence: dense and packed sequences with ragged
lengths, a zero-length sequence, h0 and dh_T, gate stress, and one (sequence,
head) chain of the full prefill workload.  Also: deterministic, and the
gradients of a zero-length sequence's h0 are its dh_T.

Tolerance (bf16 I/O; bf16 MFMA operands, hi + lo bf16 pairs where errors
cancel or accumulate, fp32 accumulation): RMSE/RMS <= 5e-3 per gradient
tensor, and max-abs <= 2e-2 * max(1, max |reference|) -- a bf16 output of
magnitude m is rounded by up to m 2^-9 on its own, so the gradients, whose
scale is not fixed by the inputs' unit norms, get the forward's max-abs bound
relative to their largest entry."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_kda_amd as kda
import synth
from kda_testlib import metrics, to_device
from oracle import grad

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def close_grad(got, ref, what):
    m = metrics(got, ref)
    lim = 2e-2 * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
    msg = f"{what}: {m} max-abs limit {lim:.3g}"
    assert m["finite"], msg
    assert m["max_abs"] <= lim, msg
    assert m["rel_rmse"] <= 5e-3, msg
    return m


def run(p, seed, with_dhT=True):
    d = to_device(p)
    _, _, hc = kda.chunk_fwd_states(**d, scale=p.scale)
    assert kda.device_check() == 0
    do_bits, dhT = synth.cotangents(seed, p.tokens, p.H, p.dv, p.dk, len(p.offsets()) - 1, with_dhT)
    B, T = d["q"].shape[:2]
    do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).cuda().reshape(B, T, p.H, p.dv)
    dhT_d = None if dhT is None else torch.from_numpy(dhT).cuda()
    dd = {k_: v_ for k_, v_ in d.items() if k_ != "h0"}
    g = kda.backward(**dd, h_chunks=hc, do=do, dh_T=dhT_d, scale=p.scale)
    torch.cuda.synchronize()
    return g, do_bits, dhT


def check(p, seed, heads=None, seqs=None, what="", with_dhT=True, params=True):
    say(what, "tokens", p.tokens, "H", p.H, "seqs", len(p.offsets()) - 1)
    g, do_bits, dhT = run(p, seed, with_dhT)
    f = p.f64()
    off = p.offsets()
    hs = list(range(p.H)) if heads is None else list(heads)
    ss = list(range(len(off) - 1)) if seqs is None else list(seqs)
    # oracle over the chosen sequences and heads (sequences are independent)
    rows = np.concatenate([np.arange(off[s], off[s + 1]) for s in ss]) if ss else np.zeros(0, np.int64)
    cu = np.concatenate([[0], np.cumsum([off[s + 1] - off[s] for s in ss])])
    sel = lambda x: x[rows][:, hs]
    do = synth.bf16_to_f32(do_bits).astype(np.float64)
    ref = grad.backward(sel(f["q"]), sel(f["k"]), sel(f["v"]), sel(f["a"]), f["b"][rows][:, hs],
                        f["A_log"][hs], f["dt_bias"][hs], sel(do),
                        h0=None if f["h0"] is None else f["h0"][ss][:, hs],
                        dh_T=None if dhT is None else dhT[ss][:, hs].astype(np.float64), cu_seqlens=cu,
                        scale=p.scale)
    flat = lambda t, d_: t.float().cpu().numpy().reshape(p.tokens, p.H, d_)[rows][:, hs].astype(np.float64)
    out = {}
    out["dq"] = close_grad(flat(g["dq"], p.dk), ref["dq"], what + " dq")
    out["dk"] = close_grad(flat(g["dk"], p.dk), ref["dk"], what + " dk")
    out["dv"] = close_grad(flat(g["dv"], p.dv), ref["dv"], what + " dv")
    out["dg"] = close_grad(flat(g["dg_raw"], p.dk), ref["da"], what + " dg_raw")
    db = g["dbeta_raw"].float().cpu().numpy().reshape(p.tokens, p.H)[rows][:, hs].astype(np.float64)
    out["db"] = close_grad(db, ref["db"], what + " dbeta_raw")
    dh0 = g["dh0"].cpu().numpy()[ss][:, hs].astype(np.float64)
    out["dh0"] = close_grad(dh0, ref["dh0"], what + " dh0")
    if params:   # sums over all sequences: only when every sequence is in the reference
        out["dA"] = close_grad(g["dA_log"].cpu().numpy()[hs].astype(np.float64), ref["dA_log"], what + " dA_log")
        out["ddt"] = close_grad(g["ddt_bias"].cpu().numpy()[hs].astype(np.float64), ref["ddt_bias"],
                                what + " ddt_bias")
    for k_, m in out.items():
        say("  ", k_, m)
    return g


def test_backward_dense_ragged():
    p = synth.prefill(500, B=2, T=37, H=2, dk=128, dv=128, dtype="bf16", with_h0=True)
    check(p, 500, what="bwd dense B2 T37")


def test_backward_packed_with_empty_sequence():
    p = synth.prefill(501, B=1, T=0, H=2, dk=128, dv=128, dtype="bf16", lengths=[1, 16, 17, 0, 45],
                      with_h0=True)
    g = check(p, 501, what="bwd packed")
    # a zero-length sequence passes dh_T straight to dh0
    _, _, dhT = run(p, 501)
    assert np.array_equal(g["dh0"][3].cpu().numpy(), dhT[3])


def test_backward_gate_stress_no_dhT():
    p = synth.prefill(502, B=1, T=80, H=3, dk=128, dv=128, dtype="bf16", gate_stress=0.05)
    check(p, 502, what="bwd gate-stress", with_dhT=False)


def test_backward_many_chains_short():
    """64 (sequence, head) chains of 40 tokens: the reverse chain takes two slabs
    per workgroup here (the small cases above take one); three heads are checked."""
    p = synth.prefill(505, B=1, T=40, H=64, dk=128, dv=128, dtype="bf16", with_h0=True)
    check(p, 505, heads=[0, 37, 63], what="bwd B1 T40 H64", params=False)


def test_backward_deterministic():
    p = synth.prefill(503, B=2, T=50, H=2, dk=128, dv=128, dtype="bf16", with_h0=True)
    g1, _, _ = run(p, 503)
    g2, _, _ = run(p, 503)
    for k_ in g1:
        assert torch.equal(g1[k_], g2[k_]), k_


def test_backward_workload1_one_chain():
    p = synth.prefill_workload(1)
    check(p, 504, heads=[5], seqs=[2], what="bwd prefill-bf16 B4 H16 T4096 (seq 2, head 5)", params=False)
