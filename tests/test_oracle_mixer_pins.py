"""Pins of the mixer prologue/epilogue oracle (oracle/mixer.py) to code
written separately from it: torch's CPU library routines (conv1d with one
group per channel and left padding, silu, normalize, sigmoid, rms_norm) in
float64, and closed forms.  CPU only.
"""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import mixer


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_conv(x, W):
    """x [B, T, H, d], W [H*d, K]: F.conv1d over time, one group per channel."""
    B, T, H, d = x.shape
    K = W.shape[1]
    xt = torch.from_numpy(x).reshape(B, T, H * d).permute(0, 2, 1)       # [B, C, T]
    y = F.conv1d(F.pad(xt, (K - 1, 0)), torch.from_numpy(W)[:, None, :], groups=H * d)
    return y.permute(0, 2, 1).reshape(B, T, H, d).numpy()


def test_conv_matches_conv1d():
    x = _rand(1, 2, 37, 3, 8)
    W = _rand(2, 3 * 8, 4)
    np.testing.assert_allclose(mixer.causal_conv(x, W), _torch_conv(x, W), rtol=1e-12, atol=1e-12)


def test_conv_one_hot_weights_shift():
    # W[c] = e_j: the output is the input delayed by K-1-j tokens, zeros first
    x = _rand(3, 1, 20, 2, 4)
    for j in range(4):
        W = np.zeros((8, 4))
        W[:, j] = 1.0
        y = mixer.causal_conv(x, W)
        lag = 3 - j
        np.testing.assert_array_equal(y[:, lag:], x[:, :20 - lag])
        assert not y[:, :lag].any()


def test_conv_restarts_at_packed_sequence_starts():
    lengths = [5, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    x = _rand(4, 1, cu[-1], 2, 4)
    W = _rand(5, 8, 4)
    y = mixer.causal_conv(x, W, cu_seqlens=cu)
    for n in range(3):
        seg = x[:, cu[n]:cu[n + 1]]
        np.testing.assert_allclose(y[:, cu[n]:cu[n + 1]], _torch_conv(seg, W), rtol=1e-12, atol=1e-12)


def test_prologue_matches_torch():
    B, T, H, dk, dv = 2, 30, 2, 8, 6
    xq, xk, xv = _rand(6, B, T, H, dk), _rand(7, B, T, H, dk), _rand(8, B, T, H, dv)
    ga, gb, gw = _rand(9, B, T, H, dk), _rand(10, B, T, H, dk), _rand(11, B, T, H, dv)
    Wq, Wk, Wv = _rand(12, H * dk, 4), _rand(13, H * dk, 4), _rand(14, H * dv, 4)
    q, k, v, a, b, w = mixer.prologue(xq, xk, xv, ga, gb, gw, Wq, Wk, Wv, l2_eps=0.0)
    tq = F.normalize(F.silu(torch.from_numpy(_torch_conv(xq, Wq))), dim=-1, eps=0.0).numpy()
    tk = F.normalize(F.silu(torch.from_numpy(_torch_conv(xk, Wk))), dim=-1, eps=0.0).numpy()
    tv = F.silu(torch.from_numpy(_torch_conv(xv, Wv))).numpy()
    np.testing.assert_allclose(q, tq, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(k, tk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-13)
    for got, x in ((a, ga), (b, gb), (w, gw)):
        np.testing.assert_allclose(got, torch.sigmoid(torch.from_numpy(x)).numpy(), rtol=1e-14)
    # unit norm per head-token
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-13)


def test_epilogue_matches_rms_norm_and_silu():
    o, g = _rand(15, 2, 9, 3, 16), _rand(16, 2, 9, 3, 16)
    gamma = _rand(17, 16)
    out = mixer.epilogue(o, g, gamma, rms_eps=1e-6)
    ref = F.rms_norm(torch.from_numpy(o), (16,), torch.from_numpy(gamma), eps=1e-6) * \
        F.silu(torch.from_numpy(g))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_closed_forms():
    # SiLU(0) = 0, sigmoid(0) = 1/2; RMSNorm of a constant row c is sign(c)
    # (eps -> 0); with gate pre-activation 0 the output is 0
    o = np.full((1, 1, 1, 8), -3.0)
    g = np.full((1, 1, 1, 8), 50.0)      # SiLU(50) = 50 to double precision
    np.testing.assert_allclose(mixer.epilogue(o, g, rms_eps=0.0), -50.0, rtol=1e-15)
    assert not mixer.epilogue(o, np.zeros_like(g)).any()
    _, _, _, a, _, _ = mixer.prologue(*[np.zeros((1, 2, 1, 4))] * 6, *[np.ones((4, 2))] * 3)
    np.testing.assert_array_equal(a, 0.5)


def test_bf16_bits_widen_exactly():
    from gated_delta_rule_59_amd import synth
    x = _rand(18, 1, 5, 1, 8).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    wide = synth.bf16_bits_to_f32(bits).reshape(x.shape)
    W = _rand(19, 8, 4)
    np.testing.assert_array_equal(mixer.causal_conv(bits, W), mixer.causal_conv(wide, W))
