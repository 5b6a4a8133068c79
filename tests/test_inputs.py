"""The seeded input generator: determinism, shapes, bf16 rounding (checked against torch's cast)."""
import numpy as np
import torch

from gated_deltanet_recurrence_chunked_amd import inputs as gi


def test_bf16_cast_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.0078125, 0.0, -0.0], np.float32)])
    ours = gi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = gi.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_seed_dependent():
    a = gi.checksums(gi.make_inputs(gi.PREFILL, 0, B=2, H=2, T=70))
    b = gi.checksums(gi.make_inputs(gi.PREFILL, 0, B=2, H=2, T=70))
    c = gi.checksums(gi.make_inputs(gi.PREFILL, 1, B=2, H=2, T=70))
    assert a == b
    assert a["xq"] != c["xq"]


def test_shapes_and_distributions():
    i0 = gi.make_inputs(gi.TINY_FP32)
    assert i0["q"].shape == (256, 2, 64) and i0["q"].dtype == np.float32
    assert np.allclose(np.linalg.norm(i0["q"].astype(np.float64), axis=-1), 1.0, atol=1e-6)
    assert np.all((np.exp(i0["A_log"]) >= 1) & (np.exp(i0["A_log"]) <= 16))
    i2 = gi.make_inputs(gi.LONG_CONTEXT, H=2, T=200)
    assert i2["k"].dtype == np.uint16 and i2["S0"].shape == (1, 2, 128, 128)
    i3 = gi.make_inputs(gi.DECODE, N=4, H=2, steps=3)
    assert i3["q"].shape == (3, 4, 2, 128) and i3["state"].shape == (4, 2, 128, 128)
    i4 = gi.make_inputs(gi.VARLEN, nseq=8, H=2, lmax=300)
    L = np.diff(i4["cu_seqlens"])
    assert len(L) == 8 and L.min() >= 128 and L.max() <= 300
    assert i4["xq"].shape[0] == i4["cu_seqlens"][-1]


def test_varlen_full_lengths():
    sh = gi.make_shape(gi.VARLEN)
    assert sh.num_seqs == 64
    assert 128 <= min(sh.lengths) and max(sh.lengths) <= 32768
