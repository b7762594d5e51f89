"""Seeded input generators: bf16 rounding checked against torch's own
float32 -> bfloat16 conversion (round to nearest even), shapes and the
documented variable-length draw.  CPU only."""
import numpy as np
import torch

import synth


def test_bf16_rne_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10.0 ** r.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, 1e-40], np.float32)])
    x = x.astype(np.float32)
    ours = synth.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = synth.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_prefill_shapes_and_units():
    p = synth.prefill(3, B=2, T=40, H=3, dk=16, dv=8, dtype="bf16")
    assert p.q.shape == (80, 3, 16) and p.v.shape == (80, 3, 8) and p.b.shape == (80, 3)
    q = synth.bf16_to_f32(p.q)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-2)
    assert p.A_log.min() >= 0 and p.A_log.max() <= np.log(16)
    f = p.f64()
    assert f["q"].dtype == np.float64 and np.array_equal(f["cu_seqlens"], [0, 40, 80])


def test_varlen_draw_seed2():
    """The 32 variable lengths are drawn first; seed 2 gives 129,830 tokens."""
    r = np.random.default_rng(2)
    lengths = r.integers(128, 8192, endpoint=True, size=32)
    assert lengths.sum() == 129830 and lengths.min() == 572 and lengths.max() == 8135


def test_decode_indices():
    d = synth.decode(5, B=20, H=2, HV=4, K=8, V=8, P=30, n_pad=3)
    live = d.state_idx[d.state_idx >= 0]
    assert (d.state_idx == -1).sum() == 3 and len(np.unique(live)) == len(live) and live.max() < 30
    assert d.qkv.shape == (20, 2 * 2 * 8 + 4 * 8) and d.pool.shape == (30, 4, 8, 8)
