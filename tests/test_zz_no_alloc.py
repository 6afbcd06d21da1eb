"""gdn2_fwd_noalloc (the forward that allocates nothing, for callers that
cannot call hipMalloc) against gdn2_fwd_gates with a caller workspace, through
the C ABI: bit-identical outputs on consecutive calls that share the library's
per-GPU scratch (the second call smaller than the first), within the oracle
tolerance, and the size limit rejected before any launch.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_59_amd as g
from gated_delta_rule_59_amd import synth
from gpu_util import TOKENS, dev_inputs, oracle_fwd, say
from parity import assert_rms

pytestmark = pytest.mark.gpu


def _both(d, inp, gates=g.GATES_FULL):
    """(o, S_T) from gdn2_fwd_gates (torch workspace) and from gdn2_fwd_noalloc."""
    B, T, H, dk, dv = inp["B"], inp["T"], inp["H"], inp["dk"], inp["dv"]
    N = inp["num_seqs"]
    need = g.gdn2_fwd_workspace_size(B, T, H, dk, dv, N, g.GDN2_BF16)
    assert 0 < need <= g.GDN2_NOALLOC_SCRATCH_BYTES, "case must use the scratch"
    o1, S1 = g.gdn2_fwd_gates(*[d[n] for n in TOKENS], gates, S0=d["S0"],
                              cu_seqlens=d["cu_seqlens"], out_dtype=torch.float32)
    o2 = torch.full_like(o1, float("nan"))
    S2 = torch.full_like(S1, float("nan"))
    g.gdn2_fwd_noalloc(*[d[n] for n in TOKENS], gates, o2, S0=d["S0"], S_T=S2,
                       cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    return o1, S1, o2, S2


def _check(label, inp, d):
    say(f"no-alloc forward: {label}")
    o1, S1, o2, S2 = _both(d, inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2), f"{label}: outputs differ"
    ref_o, ref_S, _ = oracle_fwd(inp)
    assert_rms(o2, ref_o, f"{label} o")
    assert_rms(S2, ref_S, f"{label} S_T")


def test_noalloc_matches_workspace_forward():
    # two calls in a row on the segmented path, the second smaller, then a
    # packed batch: each call rewrites what it reads of the shared scratch
    inp = synth.make_fwd(2, B=1, T=8192, H=4, s0=True)
    _check("dense B=1 T=8192 H=4", inp, dev_inputs(inp))
    inp = synth.make_fwd(2, B=1, T=2048, H=2, s0=True)
    _check("dense B=1 T=2048 H=2 (smaller)", inp, dev_inputs(inp))
    inp = synth.make_varlen(4, lengths=[3000, 700, 0, 129], H=2)
    _check("packed lengths 3000, 700, 0, 129", inp, dev_inputs(inp))


def test_noalloc_rejects_oversized_plan():
    # a packed batch whose workspace would exceed the scratch: rejected with
    # GDN2_ERR_WORKSPACE before anything is launched
    say("no-alloc forward: oversized plan rejected")
    N, H, T = 100, 1, 200000
    need = g.gdn2_fwd_workspace_size(1, T, H, 128, 128, N, g.GDN2_BF16)
    assert need > g.GDN2_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    st = g.lib().gdn2_fwd_noalloc(*[g._ptr(dummy)] * 6, g.GATES_FULL, g.GDN2_BF16, None,
                                  g._ptr(o), g.GDN2_BF16, None, g._ptr(cu), N, 1, T, H, 128,
                                  128, g._stream(dummy.device))
    torch.cuda.synchronize()
    assert st == -3, st


def test_noalloc_token_serial_fp32_dk128():
    # fp32 inputs at dk = 128: the token-serial forward, segmented through the
    # scratch when its plan fits, unsegmented (no workspace) when it does not;
    # bit-identical to gdn2_fwd_gates either way
    from parity import assert_fp32
    for label, B, T, H in (("segmented B=1 T=2048 H=2", 1, 2048, 2),
                           ("segmented B=1 T=1500 H=1 (smaller)", 1, 1500, 1)):
        say(f"no-alloc forward, fp32 dk=128: {label}")
        need = g.gdn2_fwd_workspace_size(B, T, H, 128, 128, B, g.GDN2_F32)
        assert 0 < need <= g.GDN2_NOALLOC_SCRATCH_BYTES
        inp = synth.make_fwd(0, B=B, T=T, H=H, dk=128, dv=128, s0=True)
        d = dev_inputs(inp)
        o1, S1 = g.gdn2_fwd_gates(*[d[n] for n in TOKENS], g.GATES_FULL, S0=d["S0"])
        o2 = torch.full_like(o1, float("nan"))
        S2 = torch.full_like(S1, float("nan"))
        g.gdn2_fwd_noalloc(*[d[n] for n in TOKENS], g.GATES_FULL, o2, S0=d["S0"], S_T=S2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(S1, S2), f"{label}: outputs differ"
        ref_o, ref_S, _ = oracle_fwd(inp)
        assert_fp32(o2, ref_o, f"{label} o")
        assert_fp32(S2, ref_S, f"{label} S_T")


def test_noalloc_token_serial_oversized_plan_runs_unsegmented():
    # a segmented fp32 dk = 128 plan larger than the scratch: the call runs
    # the unsegmented token-serial forward instead of failing
    N, H = 8, 1
    lengths = [8192] * N
    say(f"no-alloc forward, fp32 dk=128, packed N={N} H={H}: plan beyond the scratch")
    inp = synth.make_varlen(4, lengths=lengths, H=H, dtype="f32")
    T = int(inp["T"])
    need = g.gdn2_fwd_workspace_size(1, T, H, 128, 128, N, g.GDN2_F32)
    assert need > g.GDN2_NOALLOC_SCRATCH_BYTES, need
    d = dev_inputs(inp)
    o = torch.full((1, T, H, 128), float("nan"), dtype=torch.float32, device="cuda")
    S = torch.full((N, H, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    g.gdn2_fwd_noalloc(*[d[n] for n in TOKENS], g.GATES_FULL, o, S0=d["S0"], S_T=S,
                       cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    from parity import assert_fp32
    ref_o, ref_S, _ = oracle_fwd(inp)
    assert_fp32(o, ref_o, "o")
    assert_fp32(S, ref_S, "S_T")
