"""GPU parity of kda_conv_decode_step (short causal convolution with silu,
fused with one decode step) against the fp64 oracle's convolution followed by
its decode step, through the C ABI.  It covers:
- the full decode width (B = 256, H = HV = 32, W = 4) and small shapes with
  grouped heads (including three value heads per q/k head), widths 2-4 and
  pads;
- no bias, and the un-normalised form;
- the conv state of live slots, which must equal the shifted window exactly
  (it only moves bf16 inputs), and pad and unreferenced slots of both states,
  which must be left bitwise untouched."""
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


def check_conv_decode(d: synth.ConvDecode, l2norm=True, what=""):
    say(what, "B", d.B, "H", d.H, "HV", d.HV, "W", d.W, "P", d.P, "bias", d.conv_bias is not None)
    pool = torch.from_numpy(d.pool).cuda()
    cs = bf16_dev(d.conv_state)
    o = kda.conv_decode_step(bf16_dev(d.qkv), cs, bf16_dev(d.conv_weight),
                             None if d.conv_bias is None else bf16_dev(d.conv_bias), bf16_dev(d.a),
                             bf16_dev(d.b), torch.from_numpy(d.A_log).cuda(),
                             torch.from_numpy(d.dt_bias).cuda(), pool,
                             torch.from_numpy(d.state_idx).cuda(), d.H, d.HV, d.K, d.V, scale=d.scale,
                             l2norm=l2norm)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    got_cs = cs.view(torch.int16).cpu().numpy().view(np.uint16)

    live = d.state_idx[d.state_idx >= 0]
    remap = np.full(d.P, -1, np.int64)
    remap[live] = np.arange(len(live))
    idx = np.where(d.state_idx >= 0, remap[np.maximum(d.state_idx, 0)], -1)
    f = d.f64()
    ro, rpool, rcs = oracle.conv_decode(f["qkv"], f["conv_state"][live], f["conv_weight"], f["conv_bias"],
                                        f["a"], f["b"], f["A_log"], f["dt_bias"],
                                        d.pool[live].astype(np.float64), idx, d.H, d.HV, d.K, d.V,
                                        scale=d.scale, l2norm=l2norm)
    mo = assert_close(o, ro, "bf16", what + " o")
    got_pool = pool[torch.from_numpy(live).cuda().long()].cpu().numpy().astype(np.float64)
    ms = assert_close(got_pool, rpool, "bf16", what + " state")
    # the conv state only moves bf16 inputs: exact
    assert np.array_equal(synth.bf16_to_f32(got_cs[live]).astype(np.float64), rcs), what + " conv state"
    assert not o[d.state_idx < 0].any()
    untouched = np.setdiff1d(np.arange(d.P), live)
    if len(untouched):
        assert np.array_equal(pool[torch.from_numpy(untouched).cuda().long()].cpu().numpy(), d.pool[untouched])
        assert np.array_equal(got_cs[untouched], d.conv_state[untouched])
    say("  o", mo, " state", ms)


def test_conv_decode_workload_full():
    w = dict(synth.DECODE_WORKLOAD)
    w.pop("name")
    d = synth.conv_decode(4, W=4, name="conv-decode-bf16 B256 H32 HV32 K128 V128 W4 pool512 pad8", **w)
    check_conv_decode(d, what="conv-decode B256 H32 W4")


@pytest.mark.parametrize("B,H,HV,W,pads", [(1, 4, 4, 2, 0), (6, 2, 8, 3, 1), (32, 8, 16, 4, 3),
                                           (5, 1, 3, 4, 1)])
def test_conv_decode_small(B, H, HV, W, pads):
    d = synth.conv_decode(90 + B + W, B=B, H=H, HV=HV, K=128, V=128, P=B + 4, n_pad=pads, W=W)
    check_conv_decode(d, what=f"conv-decode B{B} H{H} HV{HV} W{W}")


def test_conv_decode_without_bias_and_norm():
    d = synth.conv_decode(97, B=8, H=2, HV=4, K=128, V=128, P=12, n_pad=1, W=4, bias=False)
    check_conv_decode(d, what="conv-decode no-bias")
    check_conv_decode(d, l2norm=False, what="conv-decode no-bias no-l2norm")
