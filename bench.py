"""Throughput of the Gated Delta Rule-2 path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-context]

Timed step: one gdn2_fwd over the 1.3B-model-shaped layer (B=8, T=4096, H=16,
dk=dv=128, bf16 inputs and output, fp32 state, S0 given and S_T written),
inputs resident in HBM.  The same run also times the same forward on the
65536-token context (B=1, H=16) and on the packed varlen batch (32 sequences
of 128..8192 tokens) under "fwd_workloads", the recurrent decode
(gdn2_decode, N=256 sequences, H=16, d=128, fp32 state read and written in
place) and the fp64 CPU oracle on the host cores.  Prints ONE JSON line.
The mean, which the throughput uses, comes from two events around the timed
steps; a second pass with an event after every step gives the median and
minimum step.

Sustained-load timing.  When load starts on an idle MI355X, its power
management holds the shader clock low for roughly the first 15 ms and then
lets it recover: the 1.3B-layer forward takes 0.24 ms per launch for the
first few launches, up to 0.33 ms around launch 10 and 0.235-0.24 ms from
about launch 60 on (--onset-trace prints that sequence).  So each workload's
K timed steps follow a settle phase of at least SETTLE_MS of the same step
back to back, then its W warm-up steps: the timed window measures the
throughput of a job that keeps the GPU busy.  The headline forward is also
timed once at load onset (W warm-up steps after the GPU sat idle, then K
steps) and reported as "onset", next to the settled figures.  As context it also measures a device-to-device
copy's bandwidth and the fp16 MFMA rate of a kernel that does nothing else
(libgdn2_peak.so).

Roofline of the dominant kernel (the fused forward): HBM-bound; algorithmic
bytes per launch = every input read once + o written once + S0 read once +
S_T written once; achieved = those bytes / mean kernel time from HIP events
on the stream the kernel runs on.  HBM traffic measured with rocprofv3
counters is reported when profiles/fwd_counters.json was taken on the current
kernel source (its sha256 matches), else null.
"""
from __future__ import annotations

import argparse
import re
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFS = 2516.6    # MI355X dense bf16 (and fp16) MFMA
FP32_VALU_PEAK_TFS = 157.3     # MI355X fp32 vector
CHUNK = 64
SETTLE_MS = 40.0            # sustained load before each timed window (ms of GPU time)


def fwd_flops(lengths, H, dk, dv, C=CHUNK):
    """Dense chunkwise-WY contraction count, triangles counted dense:
    per sequence and head L*(2C(3dk + 2dv) + 6 dk dv) + ceil(L/C) * C^3/3."""
    tot = 0
    for L in lengths:
        L = int(L)
        tot += H * (L * (2 * C * (3 * dk + 2 * dv) + 6 * dk * dv) + ((L + C - 1) // C) * C ** 3 // 3)
    return tot


def bwd_flops(lengths, H, dk, dv, C=CHUNK):
    """Dense contraction count of the chunk backward (forward recompute and
    gradient products), triangles counted dense: per chunk and head
    12 C^2 dk + 10 C^2 dv + 14 C dk dv + C^3/3."""
    tot = 0
    for L in lengths:
        nch = (int(L) + C - 1) // C
        tot += H * nch * (12 * C * C * dk + 10 * C * C * dv + 14 * C * dk * dv + C ** 3 // 3)
    return tot


def fwd_bytes(B, T, H, dk, dv, in_bytes, out_bytes, s0, sT, N):
    tokens = B * T * H
    b = tokens * (4 * dk + 2 * dv) * in_bytes + tokens * dv * out_bytes
    b += (s0 + sT) * N * H * dk * dv * 4
    return b


def kernel_source_hash():
    """sha256 of the forward kernel sources with comments and blank space
    removed, so that an edit of comments alone keeps the counters valid."""
    h = hashlib.sha256()
    for f in ("gdn2_fwd.hip", "gdn2_common.hpp"):
        with open(os.path.join(HERE, "gated_delta_rule_59_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def measured_traffic(per_launch_alg_bytes):
    path = os.path.join(HERE, "profiles", "fwd_counters.json")
    if not os.path.exists(path):
        return None
    try:
        c = json.load(open(path))
    except (OSError, ValueError):
        return None
    if c.get("source_sha256") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode timing")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the copy-bandwidth and MFMA-rate measurements")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-gates", action="store_true",
                    help="skip the reduced gate forms (KDA, GDN) of the forward")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="run one plain device-to-device copy of this many bytes before the "
                         "timed region (a reference kernel for hardware byte counters)")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-erase", action="store_true",
                    help="skip the erase reading (A) of the forward and decode")
    ap.add_argument("--no-mixer", action="store_true",
                    help="skip the mixer prologue / epilogue timing")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the 65536-token and packed varlen forwards")
    ap.add_argument("--onset-trace", type=int, default=0, metavar="N",
                    help="print the per-launch times (means of 10) of N back-to-back headline "
                         "steps started on an idle GPU, then exit")
    ap.add_argument("--workload", type=int, default=1, choices=(1, 2, 4),
                    help="forward workload: 1 = 1.3B layer (default, the headline), "
                         "2 = 65536-token context, 4 = packed varlen batch")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only; --gpus must be 1 "
              "(sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_59_amd as g
    from gated_delta_rule_59_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---------------- forward ---------------------------------------------------
    wl = synth.WORKLOADS[args.workload]
    progress(f"generating workload {wl['name']}")
    if args.workload == 4:
        inp = synth.make_varlen(4)
        lengths = [int(x) for x in inp["lengths"]]
    else:
        inp = synth.make_fwd(args.workload)
        lengths = [inp["T"]] * inp["B"]
    B, T, H, dk, dv = inp["B"], inp["T"], inp["H"], inp["dk"], inp["dv"]
    N = inp["num_seqs"]

    def to_dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "alpha", "b", "w")}
    S0 = None if inp["S0"] is None else torch.from_numpy(inp["S0"]).to(dev)
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).to(dev)
    args_fwd = [d[n] for n in ("q", "k", "v", "alpha", "b", "w")]

    def step():
        return g.gdn2_fwd(*args_fwd, S0=S0, cu_seqlens=cu)

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        progress(f"reference copy of {args.copy_bytes} bytes done")
        del src, dst
    stream = torch.cuda.current_stream(dev)
    if args.onset_trace > 0:
        # per-launch times of N back-to-back steps on an idle GPU (W warm-up
        # steps first, then a pause): the clock transient at load onset
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        time.sleep(2.0)
        per = _per_step(step, args.onset_trace, stream, torch)
        blocks = [round(1e3 * sum(per[i:i + 10]) / len(per[i:i + 10]), 1)
                  for i in range(0, len(per), 10)]
        print(json.dumps({"onset_trace": wl["name"], "launches": len(per),
                          "us_mean_of_10": blocks}), flush=True)
        return
    # onset: W warm-up steps on the GPU that has sat idle while the inputs
    # were generated, then K timed steps (the clock transient of load onset)
    progress(f"onset: warmup {args.warmup}, timing {args.steps} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    o0.record(stream)
    for i in range(args.steps):
        step()
    o1.record(stream)
    torch.cuda.synchronize()
    ms_onset = o0.elapsed_time(o1) / args.steps
    # settled: SETTLE_MS of sustained load, W warm-up steps, K timed steps
    settle_steps = _settle(step, stream, torch)
    progress(f"settled after {settle_steps} steps; warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    progress(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    step_ms = _per_step(step, args.steps, stream, torch)
    tokens = B * T
    fwd_tok_s = tokens / (ms * 1e-3)
    flops = fwd_flops(lengths, H, dk, dv)
    alg_bytes = fwd_bytes(B, T, H, dk, dv, 2, 2, S0 is not None, 1, N)
    achieved_gbs = alg_bytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic(alg_bytes)
    progress(f"fwd {ms:.3f} ms/step, {fwd_tok_s / 1e6:.1f} M tok/s, {achieved_gbs:.0f} GB/s")

    # ---------------- decode ----------------------------------------------------
    # timed right after the headline forward, after its own settle phase and
    # warm-up steps (measured last, after seconds of backward and long
    # forwards, the same decode once read 91.8 us per step against 85-86 us)
    decode = None
    if not args.no_decode:
        progress("decode workload")
        ds = synth.DecodeStream(3)
        n_steps = args.decode_steps
        Sd = torch.from_numpy(ds.S0).to(dev)
        steps_dev = []
        for s in range(n_steps):
            st = ds.step(s)
            steps_dev.append([to_dev(st[n]) for n in ("q", "k", "v", "alpha", "b", "w")])
        _settle(lambda: g.gdn2_decode(*steps_dev[0], Sd), stream, torch)
        for s in range(min(args.warmup, n_steps)):
            g.gdn2_decode(*steps_dev[s], Sd)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for s in range(n_steps):
            g.gdn2_decode(*steps_dev[s], Sd)
        d1.record(stream)
        torch.cuda.synchronize()
        us = d0.elapsed_time(d1) * 1e3 / n_steps
        it = iter(range(n_steps))
        dstep = sorted(1e3 * t for t in _per_step(lambda: g.gdn2_decode(*steps_dev[next(it)], Sd),
                                                   n_steps, stream, torch))
        Nd, Hd, dkd, dvd = ds.N, ds.H, ds.dk, ds.dv
        dbytes = 2 * Nd * Hd * dkd * dvd * 4 + Nd * Hd * (4 * dkd + 2 * dvd) * 2 + Nd * Hd * dvd * 2
        # the same stream under erase reading (A) (gdn2_decode_ex): one read
        # and one write of the state too
        dec_ex = None
        if not args.no_erase:
            def dstep_ex(s):
                return g.gdn2_decode_gates(*steps_dev[s], g.GATES_FULL, Sd, erase=g.ERASE_ROWS)
            _settle(lambda: dstep_ex(0), stream, torch)
            for s in range(min(args.warmup, n_steps)):
                dstep_ex(s)
            torch.cuda.synchronize()
            x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            x0.record(stream)
            for s in range(n_steps):
                dstep_ex(s)
            x1.record(stream)
            torch.cuda.synchronize()
            us_ex = x0.elapsed_time(x1) * 1e3 / n_steps
            dec_ex = {"us_per_step": round(us_ex, 3), "tokens_per_s": round(Nd / (us_ex * 1e-6), 1),
                      "gbps": round(dbytes / (us_ex * 1e-6) / 1e9, 1),
                      "frac_hbm_peak": round(dbytes / (us_ex * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        decode = {"workload": f"decode N={Nd} H={Hd} dk=dv={dkd} bf16 tokens, fp32 state",
                  "us_per_step": round(us, 3), "us_median": round(dstep[n_steps // 2], 3),
                  "us_min": round(dstep[0], 3), "tokens_per_s": round(Nd / (us * 1e-6), 1),
                  "gbps": round(dbytes / (us * 1e-6) / 1e9, 1),
                  "frac_hbm_peak": round(dbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "bytes_per_step": dbytes, "erase_rows": dec_ex}
        progress(f"decode {us:.2f} us/step, {decode['gbps']} GB/s")
        del steps_dev, Sd
        torch.cuda.empty_cache()

    # ---------------- reduced gate forms of the same forward --------------------
    # b, w (KDA form) and alpha (GDN form) as one value per (token, head): the
    # first channel of the drawn gates.  Algorithmic bytes drop by the gate
    # streams no longer read.
    gate_forms = None
    if not args.no_gates:
        gate_forms = {}
        for name, form in (("kda", g.GATES_KDA), ("gdn", g.GATES_GDN)):
            red = dict(d)
            for n in ("b", "w") + (("alpha",) if form == g.GATES_GDN else ()):
                red[n] = d[n][..., 0].contiguous()
            a_red = [red[n] for n in ("q", "k", "v", "alpha", "b", "w")]
            gms, _, gmin = _time_steps(
                lambda: g.gdn2_fwd_gates(*a_red, form, S0=S0, cu_seqlens=cu), args.steps,
                args.warmup, stream, torch)
            per_tok = (2 * dk + (dk if form == g.GATES_KDA else 1) + 2 + dv) * 2 + dv * 2
            gbytes = tokens * H * per_tok + ((S0 is not None) + 1) * N * H * dk * dv * 4
            gate_forms[name] = {
                "gates": "b, w per (token, head)" if form == g.GATES_KDA
                         else "alpha, b, w per (token, head)",
                "ms_per_step": round(gms, 4), "ms_step_min": round(gmin, 4),
                "tokens_per_s": round(tokens / (gms * 1e-3), 1),
                "alg_bytes": gbytes, "gbps": round(gbytes / (gms * 1e-3) / 1e9, 1),
                "frac_hbm_peak": round(gbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del red, a_red
            progress(f"fwd gates={name} {gms:.3f} ms/step (min {gmin:.3f})")

    # ---------------- erase reading (A) of the same forward -----------------------
    # gdn2_fwd_ex with GDN2_ERASE_ROWS runs the token-serial fp32 recurrence,
    # bound by its fp32 vector arithmetic: 9 dk dv flops per token and head
    # (decay, the two column sums S'^T k and S'^T q, two rank-one updates)
    erase_fwd = None
    if not args.no_erase and args.workload == 1:
        progress("forward, erase reading (A)")
        ems, emed, emin = _time_steps(
            lambda: g.gdn2_fwd_gates(*args_fwd, g.GATES_FULL, S0=S0, cu_seqlens=cu,
                                     erase=g.ERASE_ROWS), args.steps, args.warmup, stream, torch)
        efl = tokens * H * 9 * dk * dv
        erase_fwd = {"workload": f"{wl['name']} fwd, erase reading (A), token-serial fp32 kernel",
                     "ms_per_step": round(ems, 4), "ms_step_median": round(emed, 4),
                     "ms_step_min": round(emin, 4), "tokens_per_s": round(tokens / (ems * 1e-3), 1),
                     "flops_per_step": efl, "tflops": round(efl / (ems * 1e-3) / 1e12, 2),
                     "roofline": {"bound": "alu", "peak": FP32_VALU_PEAK_TFS, "unit": "TFLOP/s",
                                  "frac": round(efl / (ems * 1e-3) / 1e12 / FP32_VALU_PEAK_TFS, 4)}}
        progress(f"fwd erase reading (A) {ems:.3f} ms/step")

    # ---------------- backward on the same layer ---------------------------------
    # gdn2_bwd: checkpoint forward + the backward kernels, bf16 gradients.
    # Algorithmic bytes: the six inputs, dout, the six gradients (bf16), S0,
    # dS_T and dS0 once each.  Flops: the dense contractions of the chunk
    # backward (bwd_flops), on fp32 vector ALUs.
    bwd = None
    if not args.no_bwd and args.workload == 1:
        progress("backward")
        gen = torch.Generator(device=dev)
        gen.manual_seed(1234)
        dout = torch.randn((B, T, H, dv), generator=gen, device=dev).to(torch.bfloat16)
        dST = torch.randn((N, H, dk, dv), generator=gen, device=dev)
        bws = torch.empty(g.gdn2_bwd_workspace_size(B, T, H, dk, dv, N, g.GDN2_BF16),
                          dtype=torch.uint8, device=dev)

        def bstep():
            return g.gdn2_bwd(*args_fwd, dout, S0=S0, dS_T=dST, cu_seqlens=cu, workspace=bws)

        bmean, bmed, bmin = _time_steps(bstep, args.steps, args.warmup, stream, torch)
        bbytes = tokens * H * ((4 * dk + 2 * dv) * 2 + dv * 2 + (4 * dk + 2 * dv) * 2) \
            + ((S0 is not None) + 2) * N * H * dk * dv * 4
        bfl = bwd_flops(lengths, H, dk, dv)
        bwd = {"workload": "layer_1p3b backward, bf16 inputs, dout and gradients, dS_T given",
               "ms_per_step": round(bmean, 4), "ms_step_median": round(bmed, 4),
               "ms_step_min": round(bmin, 4),
               "tokens_per_s": round(tokens / (bmean * 1e-3), 1),
               "alg_bytes": bbytes, "gbps": round(bbytes / (bmean * 1e-3) / 1e9, 1),
               "frac_hbm_peak": round(bbytes / (bmean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "flops_per_step": bfl, "tflops": round(bfl / (bmean * 1e-3) / 1e12, 2),
               "roofline": {"bound": "alu", "peak": FP32_VALU_PEAK_TFS, "unit": "TFLOP/s",
                            "frac": round(bfl / (bmean * 1e-3) / 1e12 / FP32_VALU_PEAK_TFS, 4)},
               "workspace_bytes": int(bws.numel())}
        progress(f"bwd {bmean:.3f} ms/step (min {bmin:.3f})")
        del dout, dST, bws
        torch.cuda.empty_cache()

    # ---------------- mixer prologue and epilogue on the same layer ------------
    # elementwise, HBM-bound: the prologue reads six [B,T,H,d] bf16 streams
    # (the short convolution's earlier rows come back from the L2) and writes
    # six; the epilogue reads o and the output gate and writes y
    mixer = None
    if not args.no_mixer and args.workload == 1:
        progress("mixer prologue / epilogue")
        gen = torch.Generator(device=dev)
        gen.manual_seed(4321)
        pre = [torch.randn((B, T, H, dk if i in (0, 1, 3, 4) else dv), generator=gen,
                           device=dev).to(torch.bfloat16) for i in range(6)]
        Ws = [torch.randn((H * (dk if i < 2 else dv), 4), generator=gen, device=dev) * 0.5
              for i in range(3)]
        pmean, _, pmin = _time_steps(lambda: g.gdn2_prologue(*pre, *Ws), args.steps,
                                     args.warmup, stream, torch)
        pbytes = 2 * tokens * H * (4 * dk + 2 * dv) * 2
        o_in = torch.randn((B, T, H, dv), generator=gen, device=dev).to(torch.bfloat16)
        g_in = torch.randn((B, T, H, dv), generator=gen, device=dev).to(torch.bfloat16)
        gam = torch.ones(dv, device=dev)
        emean, _, emin = _time_steps(lambda: g.gdn2_epilogue(o_in, g_in, gam), args.steps,
                                     args.warmup, stream, torch)
        ebytes = 3 * tokens * H * dv * 2
        mixer = {"prologue": {"ms_per_step": round(pmean, 4), "ms_step_min": round(pmin, 4),
                              "alg_bytes": pbytes, "gbps": round(pbytes / (pmean * 1e-3) / 1e9, 1),
                              "frac_hbm_peak": round(pbytes / (pmean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                 "epilogue": {"ms_per_step": round(emean, 4), "ms_step_min": round(emin, 4),
                              "alg_bytes": ebytes, "gbps": round(ebytes / (emean * 1e-3) / 1e9, 1),
                              "frac_hbm_peak": round(ebytes / (emean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        progress(f"prologue {pmean:.3f} ms, epilogue {emean:.3f} ms")
        del pre, Ws, o_in, g_in
        torch.cuda.empty_cache()

    # ---------------- the other forward workloads -------------------------------
    # 65536-token context (B=1, H=16) and the packed varlen batch (32
    # sequences), each timed like the headline step; their per-token cost next
    # to the 1.3B layer's is the check of near-flat cost in T
    others = None
    if not args.no_others and args.workload == 1:
        del d, args_fwd
        torch.cuda.empty_cache()
        others = {}
        for wid in (2, 4):
            wl2 = synth.WORKLOADS[wid]
            progress(f"generating workload {wl2['name']}")
            inp2 = synth.make_varlen(4) if wid == 4 else synth.make_fwd(wid)
            lengths2 = ([int(x) for x in inp2["lengths"]] if wid == 4
                        else [inp2["T"]] * inp2["B"])
            B2, T2, H2 = inp2["B"], inp2["T"], inp2["H"]
            d2 = [to_dev(inp2[n]) for n in ("q", "k", "v", "alpha", "b", "w")]
            cu2 = (None if inp2["cu_seqlens"] is None
                   else torch.from_numpy(inp2["cu_seqlens"]).to(dev))
            S02 = None if inp2["S0"] is None else torch.from_numpy(inp2["S0"]).to(dev)
            ws2 = g.gdn2_fwd_workspace_size(B2, T2, H2, dk, dv, inp2["num_seqs"], g.GDN2_BF16)
            wsb = torch.empty(max(ws2, 1), dtype=torch.uint8, device=dev)

            def step2():
                return g.gdn2_fwd(*d2, S0=S02, cu_seqlens=cu2, workspace=wsb)

            mean2, med2, min2 = _time_steps(step2, args.steps, args.warmup, stream, torch)
            tok2 = B2 * T2
            by2 = fwd_bytes(B2, T2, H2, dk, dv, 2, 2, S02 is not None, 1, inp2["num_seqs"])
            fl2 = fwd_flops(lengths2, H2, dk, dv)
            others[wl2["name"]] = {
                "workload": (f"B={B2} T={T2} H={H2} d={dk}" if wid == 2 else
                             f"packed N={inp2['num_seqs']} lengths in [128, 8192], "
                             f"{T2} tokens, H={H2} d={dk}") + ", bf16, S0 = 0",
                "ms_per_step": round(mean2, 4), "ms_step_median": round(med2, 4),
                "ms_step_min": round(min2, 4),
                "tokens_per_s": round(tok2 / (mean2 * 1e-3), 1),
                "ns_per_token": round(mean2 * 1e6 / tok2, 3),
                "alg_bytes": by2, "gbps": round(by2 / (mean2 * 1e-3) / 1e9, 1),
                "frac_hbm_peak": round(by2 / (mean2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "tflops": round(fl2 / (mean2 * 1e-3) / 1e12, 2),
                "frac_bf16_peak": round(fl2 / (mean2 * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFS, 4),
                "workspace_bytes": ws2}
            progress(f"fwd {wl2['name']} {mean2:.3f} ms/step (min {min2:.3f})")
            del d2, cu2, S02, wsb, inp2
            torch.cuda.empty_cache()

    # ---------------- context: copy bandwidth and MFMA rate ---------------------
    context = None
    if not args.no_context:
        progress("context: device copy and MFMA rate")
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        best = None
        for _ in range(6):
            c0.record(stream)
            dst.copy_(src)
            c1.record(stream)
            torch.cuda.synchronize()
            t = c0.elapsed_time(c1)
            best = t if best is None else min(best, t)
        copy_gbps = 2 * nbytes / (best * 1e-3) / 1e9
        del src, dst
        mfma_tfs = {}
        peak_so = os.path.join(HERE, "gated_delta_rule_59_amd", "libgdn2_peak.so")
        if os.path.exists(peak_so):
            import ctypes
            pl = ctypes.CDLL(peak_so)
            pl.gdn2_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p]
            groups, iters = 256 * 8, 2048
            outp = torch.empty(groups, dtype=torch.float32, device=dev)
            for kind, name in ((0, "32x32x16_f16"), (1, "16x16x32_f16")):
                tbest = None
                for _ in range(4):
                    c0.record(stream)
                    rc = pl.gdn2_peak_mfma(kind, outp.data_ptr(), groups, iters,
                                           ctypes.c_void_p(stream.cuda_stream))
                    c1.record(stream)
                    torch.cuda.synchronize()
                    if rc != 0:
                        raise RuntimeError(f"gdn2_peak_mfma failed ({rc})")
                    t = c0.elapsed_time(c1)
                    tbest = t if tbest is None else min(tbest, t)
                mfma_tfs[name] = round(groups * 4 * iters * 131072 / (tbest * 1e-3) / 1e12, 1)
        else:
            progress("libgdn2_peak.so not built: MFMA rates not measured")
        context = {"device_copy_gbps": round(copy_gbps, 1),
                   "copy": "1 GiB device-to-device copy (torch), read + write bytes, best of 6",
                   "mfma_f16_tflops_measured": mfma_tfs or None,
                   "mfma": "one MFMA instruction only, 32 KFLOP of independent chains per wave "
                           "per round, 8 workgroups per CU, best of 4; the forward's contractions "
                           "use 16x16x32_f16"}

    # ---------------- CPU baseline: the fp64 oracle -----------------------------
    cpu = None
    if not args.no_cpu:
        import oracle
        nt = oracle.default_threads()
        progress(f"oracle on {nt} host threads (whole {wl['name']} batch)")
        c0 = time.perf_counter()
        _, _, used = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"],
                                S0=inp["S0"], cu_seqlens=inp["cu_seqlens"], nthreads=nt)
        csec = time.perf_counter() - c0
        cpu = {"value": round(tokens / csec, 1), "unit": "tokens/s", "cores": int(used),
               "kind": "oracle",
               "sample": f"whole {wl['name']} batch ({tokens} tokens x {H} heads), fp64 "
                         f"token recurrence, {csec:.2f} s wall",
               "cpu_model": _cpu_model()}
        # one host thread on the small fp32 workload (B=1 T=256 H=2 d=64)
        i0 = synth.make_fwd(0)
        reps, c0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - c0 < 0.2:
            oracle.fwd(i0["q"], i0["k"], i0["v"], i0["alpha"], i0["b"], i0["w"], S0=i0["S0"],
                       nthreads=1)
            reps += 1
        t0 = i0["q"].shape[0] * i0["q"].shape[1]
        cpu["one_thread_small_fp32_tokens_per_s"] = round(reps * t0 / (time.perf_counter() - c0), 1)

    out = {
        "metric": "GDN-2 fwd tokens/s + % bf16 MFMA peak; decode tokens/s + % HBM BW",
        "value": round(fwd_tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_step_median": round(sorted(step_ms)[len(step_ms) // 2], 4),
        "ms_step_min": round(min(step_ms), 4),
        "settle": {"ms": SETTLE_MS, "steps": settle_steps,
                   "note": "the timed steps follow SETTLE_MS of the same step back to back "
                           "and the W warm-up steps"},
        "onset": {"ms_per_step": round(ms_onset, 4),
                  "tokens_per_s": round(tokens / (ms_onset * 1e-3), 1),
                  "frac_hbm_peak": round(alg_bytes / (ms_onset * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "note": "W warm-up + K steps right after the GPU sat idle: the clock "
                          "transient of load onset"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{wl['name']} fwd B={B} T={T} H={H} dk=dv={dk} chunk=64"
                               + (f" varlen N={N}" if cu is not None else "")
                               + ", bf16 inputs and output, fp32 state"
                               + (", S0 given" if S0 is not None else ", S0 = 0"),
                   "global_batch": B, "seq_len": T, "heads": H, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "mfma": {"tflops": round(tflops, 2), "frac_bf16_peak": round(tflops / BF16_MFMA_PEAK_TFS, 4),
                 "flops_per_step": flops},
        "gate_forms": gate_forms,
        "erase_rows_fwd": erase_fwd,
        "bwd": bwd,
        "mixer": mixer,
        "fwd_workloads": others,
        "ns_per_token": round(ms * 1e6 / tokens, 3),
        "decode": decode,
        "context": context,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


def _per_step(fn, steps, stream, torch):
    """ms of each of `steps` further calls, from an event recorded after each.
    Kept out of the timed region: an event between two launches leaves a gap
    of a few microseconds on the GPU (measured: decode 89.4 us per step with
    an event after every launch, 86.5 us without)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def _settle(fn, stream, torch, ms=SETTLE_MS):
    """Runs fn back to back until at least `ms` of GPU time has passed (in
    batches bracketed by two events, sized from the previous batch's mean
    step); returns the number of calls.  Gets the GPU past the clock
    transient of load onset before a timed window."""
    done, n, k = 0.0, 0, 1
    while done < ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        el = a.elapsed_time(b)
        done, n = done + el, n + k
        k = int(min(max((ms - done) / max(el / k, 1e-3), 1), 500)) + 1
    return n


def _time_steps(fn, steps, warmup, stream, torch):
    """Mean ms of `steps` back-to-back calls after SETTLE_MS of sustained load
    and `warmup` untimed calls, from two HIP events on `stream` around them;
    then the median and minimum of a second pass with an event after each
    call."""
    _settle(fn, stream, torch)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(_per_step(fn, steps, stream, torch))
    return e0.elapsed_time(e1) / steps, per[steps // 2], per[0]


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
