"""GPU tests of the C-ABI boundary's contracts (through the binding):
- two prefills on two streams, each with its own caller-owned workspace, run
  concurrently and both match the oracle and their one-stream results bit for bit;
- a pool slot index >= P (a caller's bug that lives in device memory) is
  handled like a pad slot by every pool-addressed entry point: the results
  equal those of the same call with that index set to -1, bit for bit, every
  pool slot (and conv-state slot) included, and kda_device_check reports
  KDA_ERR_SLOT once, even when a valid launch ran in between."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_kda_amd as kda
import synth
from kda_testlib import assert_close, run_oracle, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def test_two_streams_separate_workspaces():
    probs = [synth.prefill(600, B=1, T=0, H=3, dk=128, dv=128, dtype="bf16", lengths=[700, 45, 300], with_h0=True),
             synth.prefill(601, B=2, T=513, H=2, dk=128, dv=64, dtype="bf16", with_h0=True)]
    say("two streams", [p.tokens for p in probs])
    ins = [to_device(p) for p in probs]
    ws = []
    for p in probs:
        packed = p.cu_seqlens is not None
        B, T = (1, p.tokens) if packed else (p.B, p.T)
        n = kda.chunk_fwd_workspace_bytes(B, T, p.H, p.dk, p.dv, p.n_seq, packed)
        assert n > 0
        ws.append(torch.empty(n, dtype=torch.uint8, device="cuda"))
    # each alone on the default stream
    ref = [kda.chunk_fwd(**d, scale=p.scale, workspace=w) for d, p, w in zip(ins, probs, ws)]
    assert kda.device_check() == 0
    # both at once, one per stream, each launched several times back to back
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    torch.cuda.synchronize()
    for _ in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                outs[i] = kda.chunk_fwd(**ins[i], scale=probs[i].scale, workspace=ws[i],
                                        stream=streams[i].cuda_stream)
    torch.cuda.synchronize()
    assert kda.device_check() == 0
    for i, p in enumerate(probs):
        o, hT = outs[i]
        assert torch.equal(o, ref[i][0]) and torch.equal(hT, ref[i][1]), f"stream {i} differs from its one-stream run"
        ro, rh = run_oracle(p)
        assert_close(o.float().cpu().numpy().reshape(p.tokens, p.H, p.dv), ro, "bf16", f"stream {i} o")
        assert_close(hT.cpu().numpy(), rh, "bf16", f"stream {i} h_T")


def _bad_and_pad(idx, P, row):
    """(index vector with row's slot set out of range, the same with a pad)."""
    bad, pad = idx.copy(), idx.copy()
    bad[row] = P + (row % 3) * 1000   # P itself and far past it
    pad[row] = -1
    return bad, pad


def _check_sticky(run_bad, run_pad):
    """run_bad(), then a valid run_pad(), then one check: the out-of-range
    slot is reported once and the word is clear afterwards."""
    assert kda.device_check() == 0
    a = run_bad()
    b = run_pad()
    assert kda.device_check() == kda.KDA_ERR_SLOT
    assert kda.device_check() == 0
    return a, b


@pytest.mark.parametrize("row", [0, 5])
def test_slot_out_of_range_decode(row):
    d = synth.decode(700 + row, B=8, H=2, HV=4, K=128, V=128, P=12, n_pad=1)
    live = np.flatnonzero(d.state_idx >= 0)
    r = int(live[row % len(live)])
    bad, pad = _bad_and_pad(d.state_idx, d.P, r)
    say("decode slot", bad[r], "P", d.P)

    def run(idx):
        pool = torch.from_numpy(d.pool).cuda()
        o = kda.decode_step(bf16_dev(d.qkv), bf16_dev(d.a), bf16_dev(d.b), torch.from_numpy(d.A_log).cuda(),
                            torch.from_numpy(d.dt_bias).cuda(), pool, torch.from_numpy(idx).cuda(), d.H, d.HV,
                            d.K, d.V, scale=d.scale)
        torch.cuda.synchronize()
        return o.cpu(), pool.cpu()

    (oa, pa), (ob, pb) = _check_sticky(lambda: run(bad), lambda: run(pad))
    assert torch.equal(oa, ob) and torch.equal(pa, pb)
    assert not oa[r].float().abs().sum()
    assert torch.equal(pa[d.state_idx[r]], torch.from_numpy(d.pool[d.state_idx[r]]))


def test_slot_out_of_range_extend():
    d = synth.extend(710, B=6, T=3, H=2, HV=4, K=128, V=128, P=9, n_pad=1)
    r = int(np.flatnonzero(d.state_idx >= 0)[1])
    bad, pad = _bad_and_pad(d.state_idx, d.P, r)
    say("extend slot", bad[r], "P", d.P)

    def run(idx):
        pool = torch.from_numpy(d.pool).cuda()
        o = kda.decode_extend(bf16_dev(d.qkv), bf16_dev(d.a), bf16_dev(d.b), torch.from_numpy(d.A_log).cuda(),
                              torch.from_numpy(d.dt_bias).cuda(), pool, torch.from_numpy(idx).cuda(), d.H, d.HV,
                              d.K, d.V, scale=d.scale)
        torch.cuda.synchronize()
        return o.cpu(), pool.cpu()

    (oa, pa), (ob, pb) = _check_sticky(lambda: run(bad), lambda: run(pad))
    assert torch.equal(oa, ob) and torch.equal(pa, pb)
    assert not oa[r].float().abs().sum()


def test_slot_out_of_range_conv_decode():
    d = synth.conv_decode(720, B=6, H=2, HV=4, K=128, V=128, P=9, n_pad=1, W=4)
    r = int(np.flatnonzero(d.state_idx >= 0)[2])
    bad, pad = _bad_and_pad(d.state_idx, d.P, r)
    say("conv decode slot", bad[r], "P", d.P)

    def run(idx):
        pool = torch.from_numpy(d.pool).cuda()
        cs = bf16_dev(d.conv_state)
        o = kda.conv_decode_step(bf16_dev(d.qkv), cs, bf16_dev(d.conv_weight),
                                 None if d.conv_bias is None else bf16_dev(d.conv_bias), bf16_dev(d.a),
                                 bf16_dev(d.b), torch.from_numpy(d.A_log).cuda(), torch.from_numpy(d.dt_bias).cuda(),
                                 pool, torch.from_numpy(idx).cuda(), d.H, d.HV, d.K, d.V, scale=d.scale)
        torch.cuda.synchronize()
        return o.cpu(), pool.cpu(), cs.cpu()

    (oa, pa, ca), (ob, pb, cb) = _check_sticky(lambda: run(bad), lambda: run(pad))
    assert torch.equal(oa, ob) and torch.equal(pa, pb) and torch.equal(ca.view(torch.int16), cb.view(torch.int16))
    assert not oa[r].float().abs().sum()


@pytest.mark.parametrize("workspace", [None, "auto"])
def test_slot_out_of_range_pool_prefill(workspace):
    """The pool prefill's contract for an index >= P is the one for a negative
    index: a zero start and no final state written (the outputs are still
    computed)."""
    p = synth.prefill(730, B=1, T=0, H=2, dk=128, dv=128, dtype="bf16", lengths=[40, 0, 77, 16])
    P = 7
    pool0 = np.random.default_rng(5).normal(0, 0.02, (P, p.H, p.dv, p.dk)).astype(np.float32)
    idx = np.array([3, 0, 5, 1], np.int32)
    bad, pad = _bad_and_pad(idx, P, 2)
    say("pool prefill slot", bad[2], "P", P, "workspace", workspace)
    d = to_device(p)
    d.pop("h0")

    def run(ix):
        pool = torch.from_numpy(pool0.copy()).cuda()
        o = kda.chunk_fwd_pool(**d, state_pool=pool, state_idx=torch.from_numpy(ix).cuda(), scale=p.scale,
                               workspace=workspace)
        torch.cuda.synchronize()
        return o.cpu(), pool.cpu()

    (oa, pa), (ob, pb) = _check_sticky(lambda: run(bad), lambda: run(pad))
    assert torch.equal(oa, ob) and torch.equal(pa, pb)
    assert torch.equal(pa[5], torch.from_numpy(pool0[5]))
