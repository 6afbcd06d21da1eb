"""GPU parity of the reduced gate forms (gdn2_fwd_gates, gdn2_decode_gates).

Kimi Delta Attention form: b and w hold one value per (token, head); Gated
DeltaNet form: alpha too.  The drawn per-channel gates are cut to their first
channel; the oracle gets that value broadcast over every channel (the same
recurrence, with full-shape gates), the HIP path the [.., H] tensors.

Besides the oracle tolerance, each case checks the reduced form against
gdn2_fwd / gdn2_decode on the broadcast gates: the kernels widen a per-head
gate to the same per-channel values, so a form that read the wrong gate would
stand out.  The kernels that read the form at run time (fp32 inputs, decode)
give the same bits; the bf16 forward is compiled per form, and the compiler
may fuse multiplies differently once it sees equal channels, so there the
guard is max|diff| <= 2e-3 rms (ten times tighter than the oracle bar).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_59_amd as g
from gated_delta_rule_59_amd import synth
from gpu_util import TOKENS, dev_inputs, oracle_fwd, say, to_dev
import oracle
from parity import assert_fp32, assert_rms, assert_rms_bf16_out

pytestmark = pytest.mark.gpu

FORMS = {"kda": g.GATES_KDA, "gdn": g.GATES_GDN}


def _reduce(inp, form):
    """Cut b, w (and alpha for the GDN form) to their first channel: returns
    the per-head arrays [.., H] and puts their broadcast into inp."""
    names = ("b", "w") + (("alpha",) if form == g.GATES_GDN else ())
    ph = {}
    for n in names:
        x = inp[n]
        s = np.ascontiguousarray(x[..., 0])
        inp[n] = np.ascontiguousarray(np.broadcast_to(s[..., None], x.shape))
        ph[n] = s
    return ph


def _both(inp, ph, form, out_dtype=torch.float32):
    """(o, S_T) of the reduced form and of gdn2_fwd on the broadcast gates."""
    d = dev_inputs(inp)
    full = g.gdn2_fwd(*[d[n] for n in TOKENS], S0=d["S0"], cu_seqlens=d["cu_seqlens"],
                      out_dtype=out_dtype)
    for n, s in ph.items():
        d[n] = to_dev(s, inp["dtype"])
    red = g.gdn2_fwd_gates(*[d[n] for n in TOKENS], form, S0=d["S0"],
                           cu_seqlens=d["cu_seqlens"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return red, full


def _check(inp, red, full, fp32):
    ref_o, ref_S, _ = oracle_fwd(inp)
    (o, ST), (o_f, ST_f) = red, full
    if fp32:
        assert_fp32(o, ref_o, "o")
        assert_fp32(ST, ref_S, "S_T")
    else:
        assert_rms(o, ref_o, "o")
        assert_rms(ST, ref_S, "S_T")
    _same(o, o_f, fp32, "o")
    _same(ST, ST_f, fp32, "S_T")


def _same(red, full, exact, what):
    if exact:
        assert torch.equal(red, full), f"reduced gates differ from the broadcast full gates ({what})"
        return
    r, f = red.double(), full.double()
    rms = float(f.pow(2).mean().sqrt())
    # a bf16 result may also round to the neighbouring value: one bf16 spacing
    # (at most 2^-7 |x|) on top
    slack = f.abs() * 2.0 ** -7 if full.dtype == torch.bfloat16 else 0.0
    excess = float(((r - f).abs() - slack).max())
    assert excess <= 2e-3 * rms, \
        f"reduced gates vs broadcast full gates ({what}): {excess / rms:.2e} rms"


@pytest.mark.parametrize("form", ["kda", "gdn"])
@pytest.mark.parametrize("B,T,H,dk,dv,s0", [(2, 200, 2, 128, 128, True), (1, 130, 3, 64, 128, False),
                                            (1, 65, 2, 128, 64, True), (2, 257, 2, 64, 64, True),
                                            (3, 100, 1, 128, 128, True)])
def test_fwd_gates_bf16(form, B, T, H, dk, dv, s0):
    say(f"fwd gates={form} bf16 B={B} T={T} H={H} dk={dk} dv={dv} s0={s0}")
    inp = synth.make_fwd(1, B=B, T=T, H=H, dk=dk, dv=dv, s0=s0)
    ph = _reduce(inp, FORMS[form])
    red, full = _both(inp, ph, FORMS[form])
    _check(inp, red, full, fp32=False)


@pytest.mark.parametrize("form", ["kda", "gdn"])
def test_fwd_gates_bf16_output(form):
    say(f"fwd gates={form} bf16 output")
    inp = synth.make_fwd(1, B=1, T=150, H=2)
    ph = _reduce(inp, FORMS[form])
    (o, _), (o_f, _) = _both(inp, ph, FORMS[form], out_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    _same(o, o_f, False, "o, bf16")


@pytest.mark.parametrize("form", ["kda", "gdn"])
def test_fwd_gates_segmented(form):
    say(f"fwd gates={form} segmented: dense T=2048 H=2, packed [3000, 700, 0, 129]")
    inp = synth.make_fwd(2, B=1, T=2048, H=2)
    assert g.gdn2_fwd_workspace_size(1, 2048, 2, 128, 128, 1, g.GDN2_BF16) > 0
    ph = _reduce(inp, FORMS[form])
    red, full = _both(inp, ph, FORMS[form])
    _check(inp, red, full, fp32=False)
    inp = synth.make_varlen(4, lengths=[3000, 700, 0, 129], H=2)
    ph = _reduce(inp, FORMS[form])
    red, full = _both(inp, ph, FORMS[form])
    _check(inp, red, full, fp32=False)


@pytest.mark.parametrize("form", ["kda", "gdn"])
def test_fwd_gates_strong_decay(form):
    # alpha = 0.25 on tokens 20..59: beyond the fp16 range of the
    # midpoint-referenced tiles, so the sequence is redone token by token,
    # reading the per-head gates there too
    say(f"fwd gates={form} strong decay")
    inp = synth.make_fwd(1, B=1, T=300, H=2)
    a = synth.storage_to_f32(inp["alpha"], inp["dtype"]).reshape(inp["alpha"].shape).copy()
    a[:, 20:60] = 0.25
    inp["alpha"] = synth.to_storage(a, inp["dtype"])
    ph = _reduce(inp, FORMS[form])
    red, full = _both(inp, ph, FORMS[form])
    _check(inp, red, full, fp32=False)


@pytest.mark.parametrize("form", ["kda", "gdn"])
@pytest.mark.parametrize("dk,T", [(64, 200), (128, 97)])
def test_fwd_gates_fp32(form, dk, T):
    # dk = 64: the fp32 chunked kernel; dk = 128: the token-serial kernel
    say(f"fwd gates={form} fp32 dk={dk} T={T}")
    inp = synth.make_fwd(0, B=2, T=T, H=2, dk=dk, dv=dk, s0=True)
    ph = _reduce(inp, FORMS[form])
    red, full = _both(inp, ph, FORMS[form])
    _check(inp, red, full, fp32=True)


@pytest.mark.parametrize("form", ["kda", "gdn"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_decode_gates(form, dtype, d):
    say(f"decode gates={form} {dtype} d={d}: 24 steps against the oracle's forward")
    wl = 1 if dtype == "bf16" else 0
    inp = synth.make_fwd(wl, B=3, T=24, H=2, dk=d, dv=d, s0=True)
    ph = _reduce(inp, FORMS[form])
    d_in = dev_inputs(inp)
    S, S_f = d_in["S0"].clone(), d_in["S0"].clone()
    outs, outs_f = [], []
    for t in range(24):
        tok = {n: d_in[n][:, t].contiguous() for n in TOKENS}
        outs_f.append(g.gdn2_decode(*[tok[n] for n in TOKENS], S_f, out_dtype=torch.float32))
        for n, s in ph.items():
            tok[n] = to_dev(np.ascontiguousarray(s[:, t]), inp["dtype"])
        outs.append(g.gdn2_decode_gates(*[tok[n] for n in TOKENS], FORMS[form], S,
                                        out_dtype=torch.float32))
    torch.cuda.synchronize()
    o, o_f = torch.stack(outs, dim=1), torch.stack(outs_f, dim=1)
    ref_o, ref_S, _ = oracle_fwd(inp)
    if dtype == "bf16":
        assert_rms(o, ref_o, "o")
        assert_rms(S, ref_S, "S")
    else:
        assert_fp32(o, ref_o, "o")
        assert_fp32(S, ref_S, "S")
    assert torch.equal(o, o_f) and torch.equal(S, S_f)


@pytest.mark.parametrize("form", ["kda", "gdn"])
def test_fwd_gates_layer_1p3b(form):
    # full size (B=8, T=4096, H=16, d=128), in the launch configuration the
    # bench times: next to gdn2_fwd on the broadcast gates, which the
    # full-size parity tests hold against the oracle; a sampled head against
    # the oracle here
    say(f"fwd gates={form} 1.3B layer, full size")
    inp = synth.make_fwd(1)
    ph = _reduce(inp, FORMS[form])
    (o, ST), (o_f, ST_f) = _both(inp, ph, FORMS[form], out_dtype=torch.bfloat16)
    _same(o, o_f, False, "o, bf16")
    _same(ST, ST_f, False, "S_T")
    del o_f, ST_f
    sub = {n: np.ascontiguousarray(inp[n][5:6, :, 11:12]) for n in TOKENS}
    sub.update(S0=np.ascontiguousarray(inp["S0"][5:6, 11:12]), cu_seqlens=None)
    ref_o, ref_S, _ = oracle.fwd(*[sub[n] for n in TOKENS], S0=sub["S0"])
    assert_rms(ST[5:6, 11:12], ref_S, "S_T (sequence 5, head 11)")
    assert_rms_bf16_out(o[5:6, :, 11:12], ref_o, "o (sequence 5, head 11)")


@pytest.mark.parametrize("variant", ["kda", "gdn"])
def test_fwd_gates_workload4_varlen(variant):
    # the packed varlen workload (32 sequences), whose KDA and GDN variants
    # draw b = w = beta (and for GDN a scalar alpha) per (token, head): the
    # reduced form on those values next to the full-gate result, and
    # sequence 3 against the oracle
    say(f"fwd gates={variant} workload 4 varlen, full size")
    inp = synth.make_varlen(4, variant=variant)
    form = FORMS[variant]
    ph = _reduce(inp, form)
    (o, ST), (o_f, ST_f) = _both(inp, ph, form)
    _same(o, o_f, False, "o")
    _same(ST, ST_f, False, "S_T")
    cu = inp["cu_seqlens"]
    lo, hi = int(cu[3]), int(cu[4])
    sub = {n: np.ascontiguousarray(inp[n][:, lo:hi]) for n in TOKENS}
    ref_o, ref_S, _ = oracle.fwd(*[sub[n] for n in TOKENS])
    assert_rms(o[:, lo:hi], ref_o, "o (sequence 3)")
    assert_rms(ST[3:4], ref_S, "S_T (sequence 3)")


@pytest.mark.parametrize("form", ["kda", "gdn"])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_gates_fp32_varlen(form, d):
    # packed fp32 batches with empty and one-token sequences: the chunked
    # kernel (d = 64) and the token-serial kernel (d = 128) index the
    # per-head gates by packed token
    lengths = [5, 0, 130, 64, 1]
    say(f"fwd gates={form} fp32 varlen d={d} lengths={lengths}")
    inp = synth.make_varlen(4, lengths=lengths, H=2, dk=d, dv=d, dtype="f32")
    ph = _reduce(inp, FORMS[form])
    red, full = _both(inp, ph, FORMS[form])
    _check(inp, red, full, fp32=True)


@pytest.mark.parametrize("form", ["kda", "gdn"])
def test_fwd_gates_segmented_d64(form):
    say(f"fwd gates={form} segmented bf16 dk = dv = 64, T=2048 H=2")
    inp = synth.make_fwd(2, B=1, T=2048, H=2, dk=64, dv=64)
    assert g.gdn2_fwd_workspace_size(1, 2048, 2, 64, 64, 1, g.GDN2_BF16) > 0
    ph = _reduce(inp, FORMS[form])
    red, full = _both(inp, ph, FORMS[form])
    _check(inp, red, full, fp32=False)
