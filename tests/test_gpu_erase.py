"""GPU parity of the erase-on-rows reading of the erase gate
(GDN2_ERASE_ROWS: S_t = (I - (b k) k^T) Diag(alpha) S + k (w v)^T) against
the oracle under the same reading (oracle.fwd(..., erase="rows")).

The forward under this reading is the token-serial fp32 kernel (gdn2_fwd_ex);
decode is the single-pass kernel with the other update (gdn2_decode_ex).
Bars as for the default reading: fp32 inputs 1e-4 of max|x|, bf16 inputs
2e-2 of rms.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_59_amd as g
from gated_delta_rule_59_amd import synth
from gpu_util import TOKENS, bf16_rne, dev_inputs, say
import oracle
from parity import assert_fp32, assert_rms

pytestmark = pytest.mark.gpu


def _fwd_rows(d, out_dtype=None, gates=None, ph=None):
    args = [d[n] for n in TOKENS]
    if ph is not None:
        args = [ph.get(n, d[n]) for n in TOKENS]
    o, ST = g.gdn2_fwd_gates(*args, g.GATES_FULL if gates is None else gates, S0=d["S0"],
                             cu_seqlens=d["cu_seqlens"], out_dtype=out_dtype, erase=g.ERASE_ROWS)
    torch.cuda.synchronize()
    return o, ST


def _oracle_rows(inp):
    return oracle.fwd(*[inp[n] for n in TOKENS], S0=inp["S0"], cu_seqlens=inp["cu_seqlens"],
                      erase="rows")


@pytest.mark.parametrize("wl,B,T,H,dk,dv,s0", [
    (0, 1, 256, 2, 64, 64, True), (0, 2, 97, 1, 128, 64, False),
    (1, 2, 200, 2, 128, 128, True), (1, 1, 65, 3, 64, 128, True), (1, 1, 1, 1, 128, 128, True)])
def test_fwd_erase_rows(wl, B, T, H, dk, dv, s0):
    say(f"fwd erase-rows wl={wl} B={B} T={T} H={H} dk={dk} dv={dv} s0={s0}")
    inp = synth.make_fwd(wl, B=B, T=T, H=H, dk=dk, dv=dv, s0=s0)
    ref_o, ref_S, _ = _oracle_rows(inp)
    d = dev_inputs(inp)
    o, ST = _fwd_rows(d, out_dtype=torch.float32)
    if inp["dtype"] == "f32":
        assert_fp32(o, ref_o, "o")
        assert_fp32(ST, ref_S, "S_T")
    else:
        assert_rms(o, ref_o, "o")
        assert_rms(ST, ref_S, "S_T")
        o16, _ = _fwd_rows(d)
        assert np.array_equal(o16.float().cpu().numpy(), bf16_rne(o))
    # the two readings differ on these general gates
    o_read, _ = g.gdn2_fwd(*[d[n] for n in TOKENS], S0=d["S0"], out_dtype=torch.float32)
    assert float((o_read - o).abs().max()) > 1e-3 * float(o.abs().max())


def test_fwd_erase_rows_varlen():
    lengths = [5, 0, 130, 64, 1]
    say(f"fwd erase-rows packed lengths={lengths}")
    inp = synth.make_varlen(lengths=lengths, H=2)
    ref_o, ref_S, _ = _oracle_rows(inp)
    o, ST = _fwd_rows(dev_inputs(inp), out_dtype=torch.float32)
    assert_rms(o, ref_o, "o")
    assert_rms(ST, ref_S, "S_T")


# long sequences with few (sequence, head) pairs: the token-serial forward
# under the chunked forward's segment plan (summary, combine, forward)
@pytest.mark.parametrize("wl,B,T,H,dk,dv", [(1, 1, 2048, 2, 128, 128), (0, 1, 2048, 2, 64, 64),
                                            (0, 1, 1500, 1, 128, 64)])
def test_fwd_erase_rows_segmented(wl, B, T, H, dk, dv):
    say(f"fwd erase-rows segmented wl={wl} B={B} T={T} H={H} dk={dk} dv={dv}")
    inp = synth.make_fwd(wl, B=B, T=T, H=H, dk=dk, dv=dv, s0=True)
    in_code = g.GDN2_F32 if inp["dtype"] == "f32" else g.GDN2_BF16
    assert g.gdn2_fwd_workspace_size(B, T, H, dk, dv, B, in_code) > 0
    ref_o, ref_S, _ = _oracle_rows(inp)
    o, ST = _fwd_rows(dev_inputs(inp), out_dtype=torch.float32)
    if inp["dtype"] == "f32":
        assert_fp32(o, ref_o, "o")
        assert_fp32(ST, ref_S, "S_T")
    else:
        assert_rms(o, ref_o, "o")
        assert_rms(ST, ref_S, "S_T")


def test_fwd_erase_rows_segmented_varlen():
    lengths = [2100, 64, 0, 513]
    say(f"fwd erase-rows segmented packed lengths={lengths}")
    inp = synth.make_varlen(lengths=lengths, H=2)
    rng = np.random.Generator(np.random.PCG64(92))
    inp["S0"] = (0.02 * rng.standard_normal((len(lengths), 2, 128, 128))).astype(np.float32)
    assert g.gdn2_fwd_workspace_size(1, int(inp["T"]), 2, 128, 128, len(lengths),
                                     g.GDN2_BF16) > len(lengths) * 2 * 128 * 128 * 4
    ref_o, ref_S, _ = _oracle_rows(inp)
    o, ST = _fwd_rows(dev_inputs(inp), out_dtype=torch.float32)
    assert_rms(o, ref_o, "o")
    assert_rms(ST, ref_S, "S_T")


def test_fwd_erase_rows_kda_gates_match_default_reading():
    # b = w = beta * 1: both readings are Kimi Delta Attention
    say("fwd erase-rows vs default reading on KDA gates (per-head b, w)")
    inp = synth.make_varlen(4, variant="kda", lengths=[300, 77], H=2)
    ph = {n: np.ascontiguousarray(inp[n][..., 0]) for n in ("b", "w")}
    ref_o, ref_S, _ = _oracle_rows(inp)
    d = dev_inputs(inp)
    from gpu_util import to_dev
    phd = {n: to_dev(x, inp["dtype"]) for n, x in ph.items()}
    o_rows, S_rows = _fwd_rows(d, out_dtype=torch.float32, gates=g.GATES_KDA, ph=phd)
    o_read, S_read = g.gdn2_fwd_gates(*[phd.get(n, d[n]) for n in TOKENS], g.GATES_KDA,
                                      cu_seqlens=d["cu_seqlens"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    for o, S in ((o_rows, S_rows), (o_read, S_read)):
        assert_rms(o, ref_o, "o")
        assert_rms(S, ref_S, "S_T")


def test_fwd_erase_rows_layer_1p3b_full():
    say("fwd erase-rows full 1.3B layer (B=8 T=4096 H=16 d=128)")
    inp = synth.make_fwd(1)
    ref_o, ref_S, _ = _oracle_rows(inp)
    o, ST = _fwd_rows(dev_inputs(inp), out_dtype=torch.float32)
    e1 = assert_rms(o, ref_o, "o")
    e2 = assert_rms(ST, ref_S, "S_T")
    say(f"  max|err|/rms o {e1:.2e} S_T {e2:.2e}")


def _decode_rows(stream, steps, dtype):
    S = torch.from_numpy(stream.S0).cuda()
    outs = []
    for s in range(steps):
        st = stream.step(s)
        d = {n: (torch.from_numpy(st[n].view(np.int16)).view(torch.bfloat16).cuda()
                 if dtype == "bf16" else torch.from_numpy(st[n]).cuda()) for n in TOKENS}
        outs.append(g.gdn2_decode_gates(*[d[n] for n in TOKENS], g.GATES_FULL, S,
                                        out_dtype=torch.float32, erase=g.ERASE_ROWS).cpu().numpy())
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.decode_steps(stream.S0, [stream.step(s) for s in range(steps)],
                                       erase="rows")
    return np.stack(outs), S.cpu().numpy(), np.stack(ref_o), ref_S


@pytest.mark.parametrize("N,H,dk,dv,steps,dtype", [(4, 2, 128, 128, 8, "bf16"),
                                                   (3, 1, 64, 128, 5, "bf16"),
                                                   (3, 2, 64, 64, 6, "f32")])
def test_decode_erase_rows(N, H, dk, dv, steps, dtype):
    say(f"decode erase-rows N={N} H={H} dk={dk} dv={dv} steps={steps} {dtype}")
    ds = synth.DecodeStream(N=N, H=H, dk=dk, dv=dv, dtype=dtype)
    o, S, ro, rS = _decode_rows(ds, steps, dtype)
    if dtype == "f32":
        assert_fp32(o, ro, "o")
        assert_fp32(S, rS, "S")
    else:
        assert_rms(o, ro, "o (pooled over steps)")
        assert_rms(S, rS, "S")


def test_decode_erase_rows_workload3_full():
    say("decode erase-rows workload 3: N=256 H=16 d=128, 128 steps")
    ds = synth.DecodeStream(3)
    o, S, ro, rS = _decode_rows(ds, ds.steps, "bf16")
    e1 = assert_rms(o, ro, "o (pooled over 128 steps)")
    e2 = assert_rms(S, rS, "final S")
    say(f"  max|err|/rms o {e1:.4f} S {e2:.4f}")
