"""Throughput of the Gated Delta Rule-2 path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-context]

Timed step: one gdn2_fwd over the 1.3B-model-shaped layer (B=8, T=4096, H=16,
dk=dv=128, bf16 inputs and output, fp32 state, S0 given and S_T written),
inputs resident in HBM.  The same run also times the recurrent decode
(gdn2_decode, N=256 sequences, H=16, d=128, fp32 state read and written in
place) and the fp64 CPU oracle on the host cores.  Prints ONE JSON line.
Per-step times (an event between steps) give the median and minimum beside
the mean the throughput uses.  As context it also measures a device-to-device
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
CHUNK = 64


def fwd_flops(lengths, H, dk, dv, C=CHUNK):
    """Dense chunkwise-WY contraction count, triangles counted dense:
    per sequence and head L*(2C(3dk + 2dv) + 6 dk dv) + ceil(L/C) * C^3/3."""
    tot = 0
    for L in lengths:
        L = int(L)
        tot += H * (L * (2 * C * (3 * dk + 2 * dv) + 6 * dk * dv) + ((L + C - 1) // C) * C ** 3 // 3)
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
    progress(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    progress(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    tokens = B * T
    fwd_tok_s = tokens / (ms * 1e-3)
    flops = fwd_flops(lengths, H, dk, dv)
    alg_bytes = fwd_bytes(B, T, H, dk, dv, 2, 2, S0 is not None, 1, N)
    achieved_gbs = alg_bytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic(alg_bytes)
    progress(f"fwd {ms:.3f} ms/step, {fwd_tok_s / 1e6:.1f} M tok/s, {achieved_gbs:.0f} GB/s")

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
            for _ in range(args.warmup):
                g.gdn2_fwd_gates(*a_red, form, S0=S0, cu_seqlens=cu)
            torch.cuda.synchronize()
            gev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            gev[0].record(stream)
            for i in range(args.steps):
                g.gdn2_fwd_gates(*a_red, form, S0=S0, cu_seqlens=cu)
                gev[i + 1].record(stream)
            torch.cuda.synchronize()
            gms = gev[0].elapsed_time(gev[-1]) / args.steps
            gmin = min(gev[i].elapsed_time(gev[i + 1]) for i in range(args.steps))
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

    # ---------------- decode ----------------------------------------------------
    decode = None
    if not args.no_decode:
        progress("decode workload")
        del d, args_fwd
        torch.cuda.empty_cache()
        ds = synth.DecodeStream(3)
        n_steps = args.decode_steps
        Sd = torch.from_numpy(ds.S0).to(dev)
        steps_dev = []
        for s in range(n_steps):
            st = ds.step(s)
            steps_dev.append([to_dev(st[n]) for n in ("q", "k", "v", "alpha", "b", "w")])
        for s in range(min(3, n_steps)):
            g.gdn2_decode(*steps_dev[s], Sd)
        torch.cuda.synchronize()
        dev_evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
        dev_evs[0].record(stream)
        for s in range(n_steps):
            g.gdn2_decode(*steps_dev[s], Sd)
            dev_evs[s + 1].record(stream)
        torch.cuda.synchronize()
        us = dev_evs[0].elapsed_time(dev_evs[-1]) * 1e3 / n_steps
        dstep = sorted(dev_evs[i].elapsed_time(dev_evs[i + 1]) * 1e3 for i in range(n_steps))
        Nd, Hd, dkd, dvd = ds.N, ds.H, ds.dk, ds.dv
        dbytes = 2 * Nd * Hd * dkd * dvd * 4 + Nd * Hd * (4 * dkd + 2 * dvd) * 2 + Nd * Hd * dvd * 2
        decode = {"workload": f"decode N={Nd} H={Hd} dk=dv={dkd} bf16 tokens, fp32 state",
                  "us_per_step": round(us, 3), "us_median": round(dstep[n_steps // 2], 3),
                  "us_min": round(dstep[0], 3), "tokens_per_s": round(Nd / (us * 1e-6), 1),
                  "gbps": round(dbytes / (us * 1e-6) / 1e9, 1),
                  "frac_hbm_peak": round(dbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "bytes_per_step": dbytes}
        progress(f"decode {us:.2f} us/step, {decode['gbps']} GB/s")

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
        "decode": decode,
        "context": context,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


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
