"""Helpers of the GPU parity tests: host <-> device transfer of the seeded
inputs (same bits for the oracle and the HIP path) and oracle calls."""
import sys

import numpy as np
import torch

import oracle
from gated_delta_rule_59_amd import synth

TOKENS = ("q", "k", "v", "alpha", "b", "w")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_inputs(inp):
    d = {n: to_dev(inp[n], inp["dtype"]) for n in TOKENS}
    d["S0"] = None if inp["S0"] is None else torch.from_numpy(inp["S0"]).cuda()
    d["cu_seqlens"] = (None if inp["cu_seqlens"] is None
                       else torch.from_numpy(inp["cu_seqlens"]).cuda())
    return d


def oracle_fwd(inp, **kw):
    return oracle.fwd(*[inp[n] for n in TOKENS], S0=inp["S0"], cu_seqlens=inp["cu_seqlens"], **kw)


def bf16_rne(t):
    """fp32 torch tensor -> bf16 (round to nearest even), as float32 numpy."""
    return t.to(torch.bfloat16).float().cpu().numpy()
