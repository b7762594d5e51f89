"""GPU tests of kda_chunk_fwd_pool (through the C ABI): the pool-addressed
prefill equals the dense-state prefill bit for bit with the states gathered
from / scattered to the pool, matches the fp64 oracle, leaves unreferenced
slots untouched, treats a negative slot as a zero start with no final state,
and hands its states to kda_decode_step: a pool prefill over T tokens followed
by a decode step from the pool equals the prefill over T + 1 tokens."""
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


def pool_run(p, pool0, idx):
    d = to_device(p)
    d.pop("h0")
    pool = torch.from_numpy(pool0.copy()).cuda()
    o = kda.chunk_fwd_pool(**d, state_pool=pool, state_idx=torch.from_numpy(idx).cuda(), scale=p.scale)
    assert kda.device_check() == 0
    return (o.float().cpu().numpy().reshape(p.tokens, p.H, p.dv).astype(np.float64),
            pool.cpu().numpy())


@pytest.mark.parametrize("dk,dtype", [(128, "bf16"), (64, "f32")])
def test_pool_equals_dense_and_oracle(dk, dtype):
    lengths = [37, 0, 100, 16]
    p = synth.prefill(11, B=1, T=0, H=2, dk=dk, dv=dk, dtype=dtype, lengths=lengths, with_h0=False)
    P = 7
    idx = np.array([4, 1, -1, 6], np.int32)          # sequence 2: zero start, no final state
    pool0 = np.random.default_rng(12).normal(0.0, 0.02, (P, p.H, p.dv, p.dk)).astype(np.float32)
    say("pool prefill", dtype, "dk", dk, "lengths", lengths, "slots", idx.tolist())
    o_pool, pool1 = pool_run(p, pool0, idx)

    # dense-state run with the same states gathered from the pool
    h0 = np.stack([pool0[s] if s >= 0 else np.zeros_like(pool0[0]) for s in idx])
    pd = synth.Prefill(**{**p.__dict__, "h0": h0})
    d = to_device(pd)
    o_d, hT_d = kda.chunk_fwd(**d, scale=p.scale)
    assert kda.device_check() == 0
    o_d = o_d.float().cpu().numpy().reshape(p.tokens, p.H, p.dv).astype(np.float64)
    hT_d = hT_d.cpu().numpy()
    assert np.array_equal(o_pool, o_d)
    for s, slot in enumerate(idx):
        if slot >= 0:
            assert np.array_equal(pool1[slot], hT_d[s])
    untouched = sorted(set(range(P)) - set(int(x) for x in idx if x >= 0))
    assert np.array_equal(pool1[untouched], pool0[untouched])

    # the oracle on the same gathered states
    ro, rh = run_oracle(pd)
    assert_close(o_pool, ro, dtype, "pool o")
    live = [s for s in range(len(idx)) if idx[s] >= 0]
    assert_close(pool1[idx[live]].astype(np.float64), rh[live], dtype, "pool states")


def test_pool_prefill_then_decode_equals_longer_prefill():
    """Prefill T tokens into pool slots, decode token T from those slots: the
    decode output and the updated slots match a prefill over T + 1 tokens."""
    T, H, K, B = 40, 2, 128, 2
    p = synth.prefill(13, B=B, T=T + 1, H=H, dk=K, dv=K, dtype="bf16", with_h0=False)
    say("pool prefill then decode", "B", B, "T", T)
    full = to_device(p)
    o_full, h_full = kda.chunk_fwd(**{k: v for k, v in full.items() if k != "h0"}, scale=p.scale)
    assert kda.device_check() == 0
    o_full = o_full.float().cpu().numpy().astype(np.float64)      # [B, T+1, H, dv]
    h_full = h_full.cpu().numpy()

    P = 5
    idx = np.array([3, 0], np.int32)
    pool = torch.zeros((P, H, K, K), dtype=torch.float32, device="cuda")
    q, k, v, a, b = (x.reshape(B, T + 1, H, -1) for x in (p.q, p.k, p.v, p.a, p.b))
    head = synth.Prefill(**{**p.__dict__, "T": T, "q": q[:, :T].reshape(B * T, H, -1),
                            "k": k[:, :T].reshape(B * T, H, -1), "v": v[:, :T].reshape(B * T, H, -1),
                            "a": a[:, :T].reshape(B * T, H, -1), "b": b[:, :T].reshape(B * T, H)})
    d = to_device(head)
    d.pop("h0")
    idx_dev = torch.from_numpy(idx).cuda()
    kda.chunk_fwd_pool(**d, state_pool=pool, state_idx=idx_dev, scale=p.scale)
    assert kda.device_check() == 0
    qkv = np.concatenate([q[:, T].reshape(B, -1), k[:, T].reshape(B, -1), v[:, T].reshape(B, -1)], axis=1)
    o_dec = kda.decode_step(bf16_dev(qkv), bf16_dev(a[:, T].reshape(B, -1)), bf16_dev(b[:, T].reshape(B, -1)),
                            torch.from_numpy(p.A_log).cuda(), torch.from_numpy(p.dt_bias.reshape(-1)).cuda(),
                            pool, idx_dev, H, H, K, K, scale=p.scale, l2norm=False)
    torch.cuda.synchronize()
    assert_close(o_dec.float().cpu().numpy(), o_full[:, T], "bf16", "extend + decode o")
    assert_close(pool.cpu().numpy()[idx], h_full, "bf16", "extend + decode states")
