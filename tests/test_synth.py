"""Seeded input generators: determinism, bf16 rounding, the recipe's distributions."""
import numpy as np
import torch

from gated_delta_rule_59_amd import synth


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e3,
                        np.array([1.0, -0.0, 3.0e38, 1e-40, np.inf, -np.inf], np.float32),
                        # exact ties in both directions
                        np.array([1.00390625, 1.01171875, -1.00390625], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seeded_and_deterministic():
    a = synth.make_fwd(1, T=128, B=2, H=2)
    b = synth.make_fwd(1, T=128, B=2, H=2)
    for n in ("q", "k", "v", "alpha", "b", "w", "S0"):
        assert np.array_equal(a[n], b[n])
    c = synth.make_fwd(1, seed=5, T=128, B=2, H=2)
    assert not np.array_equal(a["q"], c["q"])


def test_recipe_distributions():
    x = synth.make_fwd(1, T=512, B=2, H=4)
    q = synth.bf16_bits_to_f32(x["q"]).reshape(x["q"].shape).astype(np.float64)
    k = synth.bf16_bits_to_f32(x["k"]).reshape(x["k"].shape).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=2e-2)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, atol=2e-2)
    a = synth.bf16_bits_to_f32(x["alpha"]).astype(np.float64)
    assert 0.0 < a.min() and a.max() <= 1.0
    assert abs(np.mean(np.log(a / (1 - np.clip(a, 0, 0.9999)))) - 4.0) < 0.2
    bb = synth.bf16_bits_to_f32(x["b"]).astype(np.float64)
    assert abs(bb.mean() - 0.5) < 0.01
    assert x["S0"].dtype == np.float32 and abs(x["S0"].std() - 0.02) < 1e-3


def test_varlen_variants():
    g = synth.make_varlen(lengths=[3, 70, 0, 129], H=2, dk=8, dv=4)
    assert list(g["cu_seqlens"]) == [0, 3, 73, 73, 202]
    kda = synth.make_varlen(lengths=[3, 70, 0, 129], H=2, dk=8, dv=4, variant="kda")
    bb = synth.bf16_bits_to_f32(kda["b"]).reshape(kda["b"].shape)
    ww = synth.bf16_bits_to_f32(kda["w"]).reshape(kda["w"].shape)
    assert np.all(bb == bb[..., :1]) and np.all(ww[..., :1] == bb[..., :1])
    gdn = synth.make_varlen(lengths=[3, 70, 0, 129], H=2, dk=8, dv=4, variant="gdn")
    aa = synth.bf16_bits_to_f32(gdn["alpha"]).reshape(gdn["alpha"].shape)
    assert np.all(aa == aa[..., :1])
    assert np.array_equal(g["q"], kda["q"]) and np.array_equal(g["q"], gdn["q"])
    full = synth.make_varlen(H=1, dk=8, dv=8)
    L = full["lengths"]
    assert len(L) == 32 and L.min() >= 128 and L.max() <= 8192


def test_decode_stream_steps_are_stable():
    s1 = synth.DecodeStream(N=4, H=2, dk=8, dv=8)
    s2 = synth.DecodeStream(N=4, H=2, dk=8, dv=8)
    assert np.array_equal(s1.S0, s2.S0)
    a3 = s1.step(3)
    s2.step(0)
    b3 = s2.step(3)
    for n in a3:
        assert np.array_equal(a3[n], b3[n])
