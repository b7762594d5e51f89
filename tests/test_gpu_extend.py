"""GPU parity of kda_decode_extend (T tokens per row through the decode update
in one launch) against the fp64 oracle, through the C ABI.  It covers:
- small shapes with grouped heads and pads, gate stress and the un-normalised
  form;
- the full decode width (B = 256, HV = 32) at T = 4;
- T past one 16-token window (T = 37: three windows, the last partial);
- T = 1, which must be bitwise kda_decode_step;
- T tokens, which must be bitwise T successive kda_decode_step calls;
- pad rows and unreferenced slots left bitwise untouched."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_kda_amd as kda
import oracle
import synth
from kda_testlib import assert_close

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def dev_inputs(d):
    return dict(A_log=torch.from_numpy(d.A_log).cuda(), dt_bias=torch.from_numpy(d.dt_bias).cuda(),
                state_idx=torch.from_numpy(d.state_idx).cuda())


def run_extend(d, l2norm=True):
    pool = torch.from_numpy(d.pool).cuda()
    o = kda.decode_extend(bf16_dev(d.qkv), bf16_dev(d.a), bf16_dev(d.b), state_pool=pool,
                          num_heads=d.H, num_v_heads=d.HV, head_k_dim=d.K, head_v_dim=d.V,
                          scale=d.scale, l2norm=l2norm, **dev_inputs(d))
    torch.cuda.synchronize()
    return o, pool


def check_extend(d, l2norm=True, what=""):
    T = d.qkv.shape[1]
    say(what, "B", d.B, "T", T, "H", d.H, "HV", d.HV, "P", d.P)
    o_dev, pool = run_extend(d, l2norm=l2norm)
    o = o_dev.float().cpu().numpy().astype(np.float64)
    assert o.shape == (d.B, T, d.HV, d.V)
    live = d.state_idx[d.state_idx >= 0]
    # oracle on the referenced slots only (remapped), fp64
    remap = np.full(d.P, -1, np.int64)
    remap[live] = np.arange(len(live))
    idx = np.where(d.state_idx >= 0, remap[np.maximum(d.state_idx, 0)], -1)
    f = d.f64()
    ro, rpool = oracle.extend(f["qkv"], f["a"], f["b"], f["A_log"], f["dt_bias"],
                              d.pool[live].astype(np.float64), idx, d.H, d.HV, d.K, d.V,
                              scale=d.scale, l2norm=l2norm)
    mo = assert_close(o, ro, "bf16", what + " o")
    got_pool = pool[torch.from_numpy(live).cuda().long()].cpu().numpy().astype(np.float64)
    ms = assert_close(got_pool, rpool, "bf16", what + " state")
    assert not o[d.state_idx < 0].any()
    untouched = np.setdiff1d(np.arange(d.P), live)
    if len(untouched):
        assert np.array_equal(pool[torch.from_numpy(untouched).cuda().long()].cpu().numpy(),
                              d.pool[untouched])
    say("  o", mo, " state", ms)


@pytest.mark.parametrize("B,T,H,HV,pads", [(1, 2, 4, 4, 0), (6, 5, 2, 8, 1), (32, 4, 8, 16, 3),
                                           (16, 16, 4, 4, 2), (5, 37, 2, 4, 1)])
def test_extend_small(B, T, H, HV, pads):
    d = synth.extend(70 + B + T, B=B, T=T, H=H, HV=HV, K=128, V=128, P=B + 5, n_pad=pads)
    check_extend(d, what=f"extend B{B} T{T} H{H} HV{HV}")


def test_extend_gate_stress_and_no_l2norm():
    check_extend(synth.extend(81, B=8, T=6, H=2, HV=4, K=128, V=128, P=12, n_pad=1, gate_stress=0.05),
                 what="extend gate-stress")
    # without the in-kernel norm, unit q and k (un-normalised keys make
    # I - beta k k^T expand by ~|k|^2 per token)
    check_extend(synth.extend(82, B=8, T=6, H=2, HV=4, K=128, V=128, P=12, n_pad=1, unit_qk=True),
                 l2norm=False, what="extend no-l2norm")


def test_extend_full_width():
    w = dict(synth.DECODE_WORKLOAD)
    w.pop("name")
    d = synth.extend(83, T=4, name="extend-bf16 B256 T4 H32 HV32 K128 V128 pool512 pad8", **w)
    check_extend(d, what="extend B256 T4 H32")


def test_extend_T1_is_decode_step():
    d = synth.extend(84, B=24, T=1, H=4, HV=8, K=128, V=128, P=30, n_pad=2)
    say("extend T1 vs decode_step B24 H4 HV8")
    o1, p1 = run_extend(d)
    p2 = torch.from_numpy(d.pool).cuda()
    o2 = kda.decode_step(bf16_dev(d.qkv[:, 0]), bf16_dev(d.a[:, 0]), bf16_dev(d.b[:, 0]),
                         state_pool=p2, num_heads=d.H, num_v_heads=d.HV, scale=d.scale,
                         **dev_inputs(d))
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0].view(torch.int16), o2.view(torch.int16))
    assert torch.equal(p1, p2)


def test_extend_equals_successive_decode_steps():
    T = 6
    d = synth.extend(85, B=12, T=T, H=2, HV=8, K=128, V=128, P=16, n_pad=1)
    say("extend T6 vs 6 decode steps B12 H2 HV8")
    o1, p1 = run_extend(d)
    p2 = torch.from_numpy(d.pool).cuda()
    ins = dev_inputs(d)
    for t in range(T):
        ot = kda.decode_step(bf16_dev(d.qkv[:, t]), bf16_dev(d.a[:, t]), bf16_dev(d.b[:, t]),
                             state_pool=p2, num_heads=d.H, num_v_heads=d.HV, scale=d.scale, **ins)
        torch.cuda.synchronize()
        assert torch.equal(o1[:, t].view(torch.int16), ot.view(torch.int16)), t
    assert torch.equal(p1, p2)
