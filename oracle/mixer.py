"""fp64 CPU oracle of the token mixer's elementwise prologue and epilogue --
TEST INFRASTRUCTURE (only tests, the smoke check and the bench's CPU-baseline
leg may import it; the product path never does).

The Gated DeltaNet-2 mixer (Japanese article, "architecture and benchmarks",
paragraph 1) feeds the recurrence through:
  - q and k: linear projection, short causal convolution, SiLU, L2
    normalisation per head-token;
  - v: linear projection, short causal convolution, SiLU;
  - the decay alpha, erase gate b and write gate w: linear branches through a
    sigmoid;
and reads it out through an RMSNorm times a SiLU output gate before the out
projection.  The projections (GEMMs) are outside this path; what follows is
the plainest reading of the rest, each step written out:

  causal depthwise convolution of width K, per channel c, within a sequence
  (tokens before its start count as zero):
      y_t[c] = sum_{j=0}^{K-1} W[c][j] * x_{t-K+1+j}[c]
  SiLU(y) = y * sigmoid(y),   sigmoid(y) = 1 / (1 + exp(-y))
  L2 normalisation over the dk channels of a (token, head):
      z = y / sqrt(sum_c y[c]^2 + eps_l2)
  RMSNorm over the dv channels of a (token, head), times the SiLU gate:
      out = o / sqrt(mean_c o[c]^2 + eps_rms) * gamma * SiLU(g)

Layouts: token tensors [B, T, H, d] (or packed [1, sum L, H, d] with
cu_seqlens); convolution weights [H*d, K] (channel h*d + c); gamma [dv]
(shared by the heads) or None (= 1).  Inputs in any float dtype or bf16 bits
are widened exactly to float64.
"""
from __future__ import annotations

import numpy as np


def _f64(x, dtype=None):
    x = np.asarray(x)
    if x.dtype == np.uint16:   # bf16 bit patterns
        x = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x.astype(np.float64)


def _sigmoid(y):
    return 1.0 / (1.0 + np.exp(-y))


def _silu(y):
    return y * _sigmoid(y)


def causal_conv(x, W, cu_seqlens=None):
    """x [B, T, H, d]; W [H*d, K]. Depthwise causal convolution per sequence."""
    x = _f64(x)
    W = _f64(W)
    B, T, H, d = x.shape
    K = W.shape[1]
    Wh = W.reshape(H, d, K)
    y = np.zeros_like(x)
    if cu_seqlens is None:
        bounds = [(bb, 0, T) for bb in range(B)]
    else:
        cu = np.asarray(cu_seqlens)
        bounds = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    for bb, s0, s1 in bounds:
        for t in range(s0, s1):
            acc = np.zeros((H, d))
            for j in range(K):
                src = t - K + 1 + j
                if src >= s0:
                    acc += Wh[:, :, j] * x[bb, src]
            y[bb, t] = acc
    return y


def prologue(xq, xk, xv, ga, gb, gw, Wq, Wk, Wv, cu_seqlens=None, l2_eps=1e-6):
    """Returns float64 q, k, v, alpha, b, w."""
    q = _silu(causal_conv(xq, Wq, cu_seqlens))
    k = _silu(causal_conv(xk, Wk, cu_seqlens))
    v = _silu(causal_conv(xv, Wv, cu_seqlens))
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + l2_eps)
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + l2_eps)
    return q, k, v, _sigmoid(_f64(ga)), _sigmoid(_f64(gb)), _sigmoid(_f64(gw))


def epilogue(o, g, gamma=None, rms_eps=1e-6):
    """RMSNorm of o over its last axis, times gamma and SiLU(g)."""
    o = _f64(o)
    g = _f64(g)
    r = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + rms_eps)
    if gamma is not None:
        r = r * _f64(gamma)
    return r * _silu(g)
