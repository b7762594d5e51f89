"""GPU parity of kda_decode_step against the fp64 oracle (through the C ABI):
the full B=256 workload, small shapes with grouped heads and pads, pad and
unreferenced slots left bitwise untouched, and decode stepped T times equal
to the prefill over the same T tokens."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_kda_amd as kda
import oracle
import synth
from kda_testlib import assert_close, run_gpu

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def run_decode(d: synth.Decode, pool_dev=None, l2norm=True):
    pool = torch.from_numpy(d.pool).cuda() if pool_dev is None else pool_dev
    o = kda.decode_step(bf16_dev(d.qkv), bf16_dev(d.a), bf16_dev(d.b),
                        torch.from_numpy(d.A_log).cuda(), torch.from_numpy(d.dt_bias).cuda(),
                        pool, torch.from_numpy(d.state_idx).cuda(), d.H, d.HV, d.K, d.V,
                        scale=d.scale, l2norm=l2norm)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), pool


def check_decode(d, l2norm=True, what=""):
    say(what, "B", d.B, "H", d.H, "HV", d.HV, "P", d.P)
    o, pool = run_decode(d, l2norm=l2norm)
    live = d.state_idx[d.state_idx >= 0]
    # oracle on the referenced slots only (remapped), fp64
    remap = np.full(d.P, -1, np.int64)
    remap[live] = np.arange(len(live))
    idx = np.where(d.state_idx >= 0, remap[np.maximum(d.state_idx, 0)], -1)
    f = d.f64()
    ro, rpool = oracle.decode(f["qkv"], f["a"], f["b"], f["A_log"], f["dt_bias"],
                              d.pool[live].astype(np.float64), idx, d.H, d.HV, d.K, d.V,
                              scale=d.scale, l2norm=l2norm)
    mo = assert_close(o, ro, "bf16", what + " o")
    got_pool = pool[torch.from_numpy(live).cuda().long()].cpu().numpy().astype(np.float64)
    ms = assert_close(got_pool, rpool, "bf16", what + " state")
    pads = d.state_idx < 0
    assert not o[pads].any()
    untouched = np.setdiff1d(np.arange(d.P), live)
    if len(untouched):
        assert np.array_equal(pool[torch.from_numpy(untouched).cuda().long()].cpu().numpy(),
                              d.pool[untouched])
    say("  o", mo, " state", ms)


def test_decode_workload_full():
    check_decode(synth.decode_workload(), what="decode B256 H32")


@pytest.mark.parametrize("B,H,HV,pads", [(1, 4, 4, 0), (4, 2, 8, 1), (32, 8, 16, 3), (128, 4, 4, 0)])
def test_decode_small(B, H, HV, pads):
    d = synth.decode(50 + B, B=B, H=H, HV=HV, K=128, V=128, P=B + 7, n_pad=pads)
    check_decode(d, what=f"decode B{B} H{H} HV{HV}")


def test_decode_without_l2norm_and_gate_stress():
    d = synth.decode(61, B=8, H=2, HV=4, K=128, V=128, P=12, n_pad=1, gate_stress=0.05)
    # without the in-kernel norm feed unit vectors so magnitudes stay O(1)
    d2 = synth.decode(62, B=8, H=2, HV=4, K=128, V=128, P=12, n_pad=1, unit_qk=True)
    check_decode(d, what="decode gate-stress")
    check_decode(d2, l2norm=False, what="decode no-l2norm")


def test_decode_steps_match_prefill():
    """T decode steps on one slot equal one prefill pass over the same T
    tokens (q, k pre-normalised, so the in-kernel norm is switched off)."""
    T, H, K = 24, 2, 128
    p = synth.prefill(70, B=1, T=T, H=H, dk=K, dv=K, dtype="bf16", with_h0=True)
    say("decode x T vs prefill", T)
    o_pre, h_pre = run_gpu(p)
    pool = torch.from_numpy(p.h0.copy()).cuda()                # [1, H, V, K] slot 0
    outs = []
    for t in range(T):
        qkv = np.concatenate([p.q[t].reshape(-1), p.k[t].reshape(-1), p.v[t].reshape(-1)])[None]
        d = synth.Decode(name="step", B=1, H=H, HV=H, K=K, V=K, P=1, qkv=qkv,
                         a=p.a[t].reshape(1, -1), b=p.b[t].reshape(1, -1), A_log=p.A_log,
                         dt_bias=p.dt_bias.reshape(-1), pool=p.h0, state_idx=np.zeros(1, np.int32))
        o, pool = run_decode(d, pool_dev=pool, l2norm=False)
        outs.append(o[0])
    assert_close(np.stack(outs), o_pre, "bf16", "decode-vs-prefill o")
    assert_close(pool.cpu().numpy(), h_pre, "bf16", "decode-vs-prefill state")


def test_decode_graph_replay():
    """kda_decode_step recorded in a HIP graph (a serving decode loop): each of
    several replays, with eager work and synchronisations between them, is
    bitwise the same step run eagerly on a copy of the pool."""
    d = synth.decode(63, B=32, H=4, HV=8, K=128, V=128, P=40, n_pad=2)
    say("decode graph replay B32 H4 HV8")
    ins = dict(qkv=bf16_dev(d.qkv), a=bf16_dev(d.a), b=bf16_dev(d.b), A_log=torch.from_numpy(d.A_log).cuda(),
               dt_bias=torch.from_numpy(d.dt_bias).cuda(), state_idx=torch.from_numpy(d.state_idx).cuda())
    pool_g = torch.from_numpy(d.pool).cuda()
    pool_e = pool_g.clone()
    o_g = torch.empty((d.B, d.HV, d.V), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kda.decode_step(**ins, state_pool=pool_g, num_heads=d.H, num_v_heads=d.HV, scale=d.scale, o=o_g)
    for rep in range(3):
        g.replay()
        o_e = kda.decode_step(**ins, state_pool=pool_e, num_heads=d.H, num_v_heads=d.HV, scale=d.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), rep
        assert torch.equal(pool_g, pool_e), rep
        float(torch.arange(1000, device="cuda", dtype=torch.float32).sum())   # eager work between replays
