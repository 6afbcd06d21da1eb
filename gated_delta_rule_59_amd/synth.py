"""Seeded synthetic inputs for the Gated Delta Rule-2 forward and decode.

This module is shared by the tests, the bench and the smoke check, and feeds
both the HIP path and the CPU oracle with the *same host bits*.  It holds none
of the recurrence's arithmetic: only random draws, the input recipe of the
token mixer that sits in front of the recurrence (L2-normalised q/k, gates
through a sigmoid: Gated DeltaNet-2 pages, Japanese article, "architecture"
section) and the round-to-nearest-even cast to bfloat16.

Workloads (all seeded with numpy PCG64, seed = 1000 + workload index):

  0 tiny_fp32   B=1  H=2  T=256    d=64   fp32  S0 = 0
  1 layer_1p3b  B=8  H=16 T=4096   d=128  bf16  S0 ~ N(0, 0.02^2) fp32
  2 long_ctx    B=1  H=16 T=65536  d=128  bf16  alpha = sigmoid(N(5,1)), S0 = 0
  3 decode      N=256 H=16 d=128   bf16 tokens, fp32 state ~ N(0, 0.02^2), 128 steps
  4 varlen      32 sequences, lengths uniform in [128, 8192], H=16, d=128, bf16

Draw order: q, k, v, alpha, b, w, then S0.  Decode: the state first, then per
step q, k, v, alpha, b, w.  Varlen: the lengths first, then q, k, v, alpha, b,
w, then the scalar beta and scalar alpha used by the reduced-gate passes.
"""
from __future__ import annotations

import numpy as np

CHUNK = 64

WORKLOADS = {
    0: dict(name="tiny_fp32", kind="fwd", B=1, H=2, T=256, dk=64, dv=64,
            dtype="f32", alpha_mu=4.0, s0=False),
    1: dict(name="layer_1p3b", kind="fwd", B=8, H=16, T=4096, dk=128, dv=128,
            dtype="bf16", alpha_mu=4.0, s0=True),
    2: dict(name="long_ctx", kind="fwd", B=1, H=16, T=65536, dk=128, dv=128,
            dtype="bf16", alpha_mu=5.0, s0=False),
    3: dict(name="decode", kind="decode", N=256, H=16, dk=128, dv=128,
            dtype="bf16", alpha_mu=4.0, steps=128),
    4: dict(name="varlen", kind="varlen", N=32, Lmin=128, Lmax=8192, H=16,
            dk=128, dv=128, dtype="bf16", alpha_mu=4.0),
}

S0_STD = 0.02


def seed_of(workload: int) -> int:
    return 1000 + int(workload)


# ----------------------------------------------------------------------------
# bfloat16 storage (round to nearest, ties to even)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast fp32 values to the storage dtype: float32 array or bf16 bits."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


# ----------------------------------------------------------------------------
# value recipes
# ----------------------------------------------------------------------------
def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def _l2_unit(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) vectors normalised over the last axis, in fp32, no epsilon."""
    x = rng.standard_normal(shape, dtype=np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _token_draws(rng, lead, H, dk, dv, alpha_mu):
    """q, k, v, alpha, b, w in fp32, in the fixed draw order."""
    q = _l2_unit(rng, lead + (H, dk))
    k = _l2_unit(rng, lead + (H, dk))
    v = rng.standard_normal(lead + (H, dv), dtype=np.float32)
    alpha = _sigmoid(rng.standard_normal(lead + (H, dk), dtype=np.float32)
                     + np.float32(alpha_mu))
    b = _sigmoid(rng.standard_normal(lead + (H, dk), dtype=np.float32))
    w = _sigmoid(rng.standard_normal(lead + (H, dv), dtype=np.float32))
    return q, k, v, alpha, b, w


def make_fwd(workload: int = 1, seed: int | None = None, **over) -> dict:
    """Forward inputs [B, T, H, d] in storage dtype, S0 [B, H, dk, dv] fp32 or None.

    Keyword overrides (B, T, H, dk, dv, dtype, alpha_mu, s0) shrink a workload
    while keeping its value distributions.
    """
    cfg = dict(WORKLOADS[workload])
    if cfg["kind"] != "fwd":
        raise ValueError("workload is not a dense forward")
    cfg.update(over)
    rng = np.random.Generator(np.random.PCG64(seed_of(workload) if seed is None else seed))
    B, T, H, dk, dv = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    draws = _token_draws(rng, (B, T), H, dk, dv, cfg["alpha_mu"])
    out = {n: to_storage(x, cfg["dtype"]) for n, x in zip(("q", "k", "v", "alpha", "b", "w"), draws)}
    del draws
    out["S0"] = (rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(S0_STD)
                 if cfg["s0"] else None)
    out["cu_seqlens"] = None
    out.update(dtype=cfg["dtype"], B=B, T=T, H=H, dk=dk, dv=dv, num_seqs=B)
    return out


def make_varlen(workload: int = 4, seed: int | None = None, variant: str = "general",
                lengths=None, **over) -> dict:
    """Packed variable-length inputs [1, sum(L), H, d] with cu_seqlens int32[N+1].

    variant: "general" per-channel gates; "kda": b = w = beta*1 with per-channel
    alpha; "gdn": b = w = beta*1 and alpha one scalar per (token, head).
    `lengths` overrides the drawn lengths (the draws that follow are unchanged
    in order).
    """
    cfg = dict(WORKLOADS[4])
    cfg.update(over)
    rng = np.random.Generator(np.random.PCG64(seed_of(workload) if seed is None else seed))
    drawn = rng.integers(cfg["Lmin"], cfg["Lmax"], size=cfg["N"], endpoint=True)
    L = np.asarray(drawn if lengths is None else lengths, dtype=np.int64)
    cu = np.zeros(len(L) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(L)
    total = int(cu[-1])
    H, dk, dv = cfg["H"], cfg["dk"], cfg["dv"]
    q, k, v, alpha, b, w = _token_draws(rng, (1, total), H, dk, dv, cfg["alpha_mu"])
    beta = _sigmoid(rng.standard_normal((1, total, H, 1), dtype=np.float32))
    alpha_s = _sigmoid(rng.standard_normal((1, total, H, 1), dtype=np.float32)
                       + np.float32(cfg["alpha_mu"]))
    if variant in ("kda", "gdn"):
        b = np.broadcast_to(beta, b.shape).copy()
        w = np.broadcast_to(beta, w.shape).copy()
    if variant == "gdn":
        alpha = np.broadcast_to(alpha_s, alpha.shape).copy()
    elif variant not in ("general", "kda"):
        raise ValueError(f"unknown variant {variant!r}")
    dt = cfg["dtype"]
    out = {n: to_storage(x, dt) for n, x in
           zip(("q", "k", "v", "alpha", "b", "w"), (q, k, v, alpha, b, w))}
    out.update(S0=None, cu_seqlens=cu, dtype=dt, B=1, T=total, H=H, dk=dk, dv=dv,
               num_seqs=len(L), lengths=L, variant=variant)
    return out


class DecodeStream:
    """Decode workload: the fp32 start state, then the per-step token inputs.

    The state is drawn first; step inputs are drawn lazily, in step order,
    from the same generator, so step s is identical however many steps a
    caller consumes.
    """

    def __init__(self, workload: int = 3, seed: int | None = None, **over):
        cfg = dict(WORKLOADS[workload])
        cfg.update(over)
        self.cfg = cfg
        self.N, self.H, self.dk, self.dv = cfg["N"], cfg["H"], cfg["dk"], cfg["dv"]
        self.dtype = cfg["dtype"]
        self.steps = cfg["steps"]
        self._rng = np.random.Generator(np.random.PCG64(seed_of(workload) if seed is None else seed))
        self.S0 = (self._rng.standard_normal((self.N, self.H, self.dk, self.dv), dtype=np.float32)
                   * np.float32(S0_STD))
        self._drawn = []

    def step(self, s: int) -> dict:
        while len(self._drawn) <= s:
            d = _token_draws(self._rng, (self.N,), self.H, self.dk, self.dv, self.cfg["alpha_mu"])
            self._drawn.append({n: to_storage(x, self.dtype) for n, x in
                                zip(("q", "k", "v", "alpha", "b", "w"), d)})
        return self._drawn[s]

