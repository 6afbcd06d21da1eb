"""GPU parity of the mixer prologue and epilogue (gdn2_prologue,
gdn2_epilogue) against the fp64 oracle (oracle/mixer.py), and of the chain
prologue -> gdn2_fwd -> epilogue against the oracles chained the same way.

Inputs: projected activations xq, xk, xv ~ N(0, 1); gate pre-activations
ga ~ N(4, 1) (the decay gates then sit near the workloads' sigmoid(N(4, 1))),
gb, gw, g ~ N(0, 1); convolution weights ~ N(0, 1/K); gamma ~ 1 + N(0, 0.1).
Bars: fp32 outputs max|err| <= 1e-4 max|ref| per tensor; bf16 outputs are
the rounding of an fp32 result, so |err| <= 2^-8 |ref| + 1e-5 max|ref|
elementwise.  The chain: 2e-2 rms, the forward's bar.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_59_amd as g
from gated_delta_rule_59_amd import synth
from gpu_util import say, to_dev
import oracle
from oracle import mixer

pytestmark = pytest.mark.gpu


def _inputs(seed, B, T, H, dk, dv, K, dtype):
    rng = np.random.Generator(np.random.PCG64(seed))
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    x = {"xq": f(B, T, H, dk), "xk": f(B, T, H, dk), "xv": f(B, T, H, dv),
         "ga": f(B, T, H, dk) + np.float32(4.0), "gb": f(B, T, H, dk), "gw": f(B, T, H, dv)}
    st = {n: synth.to_storage(a, dtype) for n, a in x.items()}
    W = {"conv_q": f(H * dk, K) / np.float32(np.sqrt(K)), "conv_k": f(H * dk, K) / np.float32(np.sqrt(K)),
         "conv_v": f(H * dv, K) / np.float32(np.sqrt(K))}
    return st, W


NAMES = ("xq", "xk", "xv", "ga", "gb", "gw")
OUTS = ("q", "k", "v", "alpha", "b", "w")


def _check_elementwise(got, ref, dtype, what):
    got = got.float().cpu().numpy().astype(np.float64)
    mx = float(np.max(np.abs(ref)))
    if dtype == "f32":
        err = float(np.max(np.abs(got - ref))) / max(mx, 1e-300)
        assert err <= 1e-4, f"{what}: max rel err {err:.2e}"
    else:
        excess = np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 1e-5 * mx)
        assert np.max(excess) <= 0, f"{what}: beyond bf16 rounding by {np.max(excess):.2e}"


def _run_prologue(st, W, dtype, cu=None):
    d = {n: to_dev(st[n], dtype) for n in NAMES}
    Wd = {n: torch.from_numpy(W[n]).cuda() for n in W}
    cud = None if cu is None else torch.from_numpy(cu).cuda()
    out = g.gdn2_prologue(*[d[n] for n in NAMES], Wd["conv_q"], Wd["conv_k"], Wd["conv_v"],
                          cu_seqlens=cud)
    torch.cuda.synchronize()
    return dict(zip(OUTS, out))


@pytest.mark.parametrize("B,T,H,dk,dv,K,dtype", [
    (2, 100, 2, 128, 128, 4, "bf16"), (1, 65, 3, 64, 128, 3, "bf16"), (1, 9, 2, 128, 64, 1, "bf16"),
    (2, 50, 2, 64, 64, 2, "f32"), (1, 130, 1, 128, 128, 4, "f32"),
])
def test_prologue(B, T, H, dk, dv, K, dtype):
    say(f"prologue B={B} T={T} H={H} dk={dk} dv={dv} K={K} {dtype}")
    st, W = _inputs(11, B, T, H, dk, dv, K, dtype)
    got = _run_prologue(st, W, dtype)
    ref = mixer.prologue(*[st[n] for n in NAMES], W["conv_q"], W["conv_k"], W["conv_v"])
    for n, r in zip(OUTS, ref):
        _check_elementwise(got[n], r, dtype, n)


def test_prologue_packed_restarts_convolution():
    lengths = [3, 0, 70, 1, 40]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    say(f"prologue packed lengths={lengths}")
    st, W = _inputs(12, 1, int(cu[-1]), 2, 128, 128, 4, "bf16")
    got = _run_prologue(st, W, "bf16", cu=cu)
    ref = mixer.prologue(*[st[n] for n in NAMES], W["conv_q"], W["conv_k"], W["conv_v"],
                         cu_seqlens=cu)
    for n, r in zip(OUTS, ref):
        _check_elementwise(got[n], r, "bf16", n)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prologue_packed_tiny_sequences(dtype):
    # runs of 8 (bf16) or 4 (fp32) tokens that hold several sequence starts,
    # empty sequences and sequences shorter than the convolution
    lengths = [1, 2, 0, 0, 5, 1, 9, 0, 17, 3, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    say(f"prologue packed tiny sequences lengths={lengths} {dtype}")
    st, W = _inputs(14, 1, int(cu[-1]), 3, 64, 128, 4, dtype)
    got = _run_prologue(st, W, dtype, cu=cu)
    ref = mixer.prologue(*[st[n] for n in NAMES], W["conv_q"], W["conv_k"], W["conv_v"],
                         cu_seqlens=cu)
    for n, r in zip(OUTS, ref):
        _check_elementwise(got[n], r, dtype, n)


def test_prologue_layer_1p3b_full():
    say("prologue full 1.3B-layer shape (B=8 T=4096 H=16 d=128), bf16")
    st, W = _inputs(13, 8, 4096, 16, 128, 128, 4, "bf16")
    got = _run_prologue(st, W, "bf16")
    ref = mixer.prologue(*[st[n][:, :300] for n in NAMES], W["conv_q"], W["conv_k"], W["conv_v"])
    for n, r in zip(OUTS, ref):   # the first 300 tokens of every sequence and head
        _check_elementwise(got[n][:, :300], r, "bf16", n)
    # and every token of one sequence and head
    sub = {n: np.ascontiguousarray(st[n][5:6, :, 9:10]) for n in NAMES}
    Wsub = {n: np.ascontiguousarray(W[n].reshape(16, -1, 4)[9]) for n in W}
    ref = mixer.prologue(*[sub[n] for n in NAMES], Wsub["conv_q"], Wsub["conv_k"], Wsub["conv_v"])
    for n, r in zip(OUTS, ref):
        _check_elementwise(got[n][5:6, :, 9:10], r, "bf16", n + " (sequence 5, head 9)")


@pytest.mark.parametrize("rows,H,dv,dtype,out,use_gamma", [
    (300, 2, 128, "bf16", "bf16", True), (300, 2, 128, "bf16", "f32", False),
    (77, 3, 64, "f32", "f32", True), (32768, 16, 128, "bf16", "bf16", True)])
def test_epilogue(rows, H, dv, dtype, out, use_gamma):
    say(f"epilogue rows={rows} H={H} dv={dv} {dtype} -> {out} gamma={use_gamma}")
    rng = np.random.Generator(np.random.PCG64(14))
    o = synth.to_storage(rng.standard_normal((rows, H, dv), dtype=np.float32), dtype)
    gt = synth.to_storage(rng.standard_normal((rows, H, dv), dtype=np.float32), dtype)
    gamma = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32) if use_gamma else None
    y = g.gdn2_epilogue(to_dev(o, dtype), to_dev(gt, dtype),
                        None if gamma is None else torch.from_numpy(gamma).cuda(),
                        out_dtype=torch.float32 if out == "f32" else None)
    torch.cuda.synchronize()
    ref = mixer.epilogue(o, gt, gamma)
    _check_elementwise(y, ref, out, "y")


def test_chain_prologue_forward_epilogue():
    # the mixer around the recurrence: prologue -> gdn2_fwd -> epilogue on the
    # GPU, against the oracles chained with the same bf16 rounding between steps
    B, T, H, d = 2, 300, 4, 128
    say(f"chain prologue -> fwd -> epilogue B={B} T={T} H={H} d={d} bf16")
    st, W = _inputs(15, B, T, H, d, d, 4, "bf16")
    rng = np.random.Generator(np.random.PCG64(16))
    gt = synth.to_storage(rng.standard_normal((B, T, H, d), dtype=np.float32), "bf16")
    gamma = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    pro = _run_prologue(st, W, "bf16")
    # o in fp32 between the forward and the epilogue (the gate in fp32 too)
    o, _ = g.gdn2_fwd(*[pro[n] for n in OUTS], out_dtype=torch.float32)
    y = g.gdn2_epilogue(o, to_dev(gt, "bf16").float(), torch.from_numpy(gamma).cuda())
    torch.cuda.synchronize()
    ref_pro = mixer.prologue(*[st[n] for n in NAMES], W["conv_q"], W["conv_k"], W["conv_v"])
    bits = [synth.to_storage(r.astype(np.float32), "bf16") for r in ref_pro]
    ref_o, _, _ = oracle.fwd(*bits)
    ref_y = mixer.epilogue(ref_o, gt, gamma)
    got = y.cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(got - ref_y)) / np.sqrt(np.mean(ref_y ** 2)))
    say(f"  chain max|err|/rms {err:.4f}")
    assert err <= 2e-2
