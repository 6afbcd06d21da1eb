"""fp64 CPU oracle of the Gated Delta Rule-2 recurrence -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The product path (gated_delta_rule_59_amd) never does, and the
two share no code: the only common input is the seeded generator module,
which holds none of the method's arithmetic.

The C library (gdn2_oracle.c) runs the recurrence token by token in fp64;
this wrapper only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
F32, BF16, F64 = 0, 1, 2


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB) or any(
                os.path.getmtime(_build.LIB) < os.path.getmtime(s) for s in _build.SRCS):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.gdn2_oracle_fwd.restype = ctypes.c_int
        lib.gdn2_oracle_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_int, P, P, P, P, i32,
                                        i32, i32, i32, i32, i32, P, i32]
        lib.gdn2_oracle_fwd_ex.restype = ctypes.c_int
        lib.gdn2_oracle_fwd_ex.argtypes = lib.gdn2_oracle_fwd.argtypes + [i32]
        lib.gdn2_oracle_bwd.restype = ctypes.c_int
        lib.gdn2_oracle_bwd.argtypes = [P, P, P, P, P, P, ctypes.c_int, P, P, ctypes.c_int, P,
                                        P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32]
        _LIB = lib
    return _LIB


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs are float32, float64 or bf16 bits (uint16), got {x.dtype}")


def default_threads() -> int:
    """Host threads to use: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fwd(q, k, v, alpha, b, w, S0=None, cu_seqlens=None, pair_mask=None, nthreads=None,
        erase="read"):
    """Token-by-token fp64 recurrence.

    erase: "read" (b gates the key that reads the prediction) or "rows" (b
    gates the erased rows); see gdn2_oracle.c.

    q, k, alpha, b: [B, T, H, dk]; v, w: [B, T, H, dv]; float32 or bf16 bits.
    S0: [N, H, dk, dv] (any float dtype, widened exactly) or None.
    cu_seqlens: int32 [N+1] (then B must be 1) or None.
    Returns (o [B, T, H, dv] float64, S_T [N, H, dk, dv] float64, threads used).
    """
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, alpha, b, w)]
    dt = _dtype_code(arrs[0])
    for x in arrs:
        if _dtype_code(x) != dt:
            raise TypeError("all token inputs must share one dtype")
    B, T, H, dk = arrs[0].shape
    dv = arrs[2].shape[-1]
    for x, d in zip(arrs, (dk, dk, dv, dk, dk, dv)):
        if x.shape != (B, T, H, d):
            raise ValueError(f"shape {x.shape} != {(B, T, H, d)}")
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = len(cu) - 1
        if B != 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("bad cu_seqlens")
    s0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    if s0 is not None and s0.shape != (N, H, dk, dv):
        raise ValueError(f"S0 shape {s0.shape} != {(N, H, dk, dv)}")
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    ST = np.zeros((N, H, dk, dv), dtype=np.float64)
    mask = None
    if pair_mask is not None:
        mask = np.ascontiguousarray(pair_mask, dtype=np.uint8).reshape(N * H)
    nt = default_threads() if nthreads is None else int(nthreads)

    def ptr(a):
        return None if a is None else a.ctypes.data

    if erase not in ("read", "rows"):
        raise ValueError(f"erase must be 'read' or 'rows', got {erase!r}")
    rc = _lib().gdn2_oracle_fwd_ex(*[ptr(x) for x in arrs], dt, ptr(s0), ptr(o), ptr(ST),
                                   ptr(cu), N, B, T, H, dk, dv, ptr(mask), nt,
                                   1 if erase == "rows" else 0)
    if rc < 0:
        raise RuntimeError(f"oracle failed ({rc})")
    return o, ST, rc


def decode_steps(S0, steps, nthreads=None, erase="read"):
    """Iterate single-token steps. steps: iterable of dicts with q, k, v, alpha,
    b, w of shape [N, H, d]. Returns (list of o [N, H, dv] float64, final S)."""
    S = np.ascontiguousarray(S0, dtype=np.float64)
    outs = []
    for st in steps:
        args = [np.ascontiguousarray(st[n])[:, None] for n in ("q", "k", "v", "alpha", "b", "w")]
        o, S, _ = fwd(*args, S0=S, nthreads=nthreads, erase=erase)
        outs.append(o[:, 0])
    return outs, S


def bwd(q, k, v, alpha, b, w, dout, S0=None, dS_T=None, cu_seqlens=None, nthreads=None):
    """Gradients of L = sum <dout, o> + <dS_T, S_T> through the token recurrence,
    by its fp64 adjoint (gdn2_oracle_bwd.c).

    Inputs as for fwd (float32, float64 or bf16 bits); dout [B, T, H, dv] in
    any of those dtypes; dS_T [N, H, dk, dv] (any float dtype) or None.
    Returns a dict of float64 arrays: dq, dk, dalpha, db [B, T, H, dk];
    dv, dw [B, T, H, dv]; dS0 [N, H, dk, dv]; and "threads".
    """
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, alpha, b, w)]
    dt = _dtype_code(arrs[0])
    for x in arrs:
        if _dtype_code(x) != dt:
            raise TypeError("all token inputs must share one dtype")
    B, T, H, dk = arrs[0].shape
    dv = arrs[2].shape[-1]
    for x, d in zip(arrs, (dk, dk, dv, dk, dk, dv)):
        if x.shape != (B, T, H, d):
            raise ValueError(f"shape {x.shape} != {(B, T, H, d)}")
    dout = np.ascontiguousarray(dout)
    if dout.shape != (B, T, H, dv):
        raise ValueError(f"dout shape {dout.shape} != {(B, T, H, dv)}")
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = len(cu) - 1
        if B != 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("bad cu_seqlens")
    s0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    dST = None if dS_T is None else np.ascontiguousarray(dS_T, dtype=np.float64)
    for name, x in (("S0", s0), ("dS_T", dST)):
        if x is not None and x.shape != (N, H, dk, dv):
            raise ValueError(f"{name} shape {x.shape} != {(N, H, dk, dv)}")
    out = {n: np.zeros((B, T, H, dk), np.float64) for n in ("dq", "dk", "dalpha", "db")}
    out.update({n: np.zeros((B, T, H, dv), np.float64) for n in ("dv", "dw")})
    out["dS0"] = np.zeros((N, H, dk, dv), np.float64)
    nt = default_threads() if nthreads is None else int(nthreads)

    def ptr(a):
        return None if a is None else a.ctypes.data

    rc = _lib().gdn2_oracle_bwd(*[ptr(x) for x in arrs], dt, ptr(s0), ptr(dout),
                                _dtype_code(dout), ptr(dST), ptr(out["dq"]), ptr(out["dk"]),
                                ptr(out["dv"]), ptr(out["dalpha"]), ptr(out["db"]),
                                ptr(out["dw"]), ptr(out["dS0"]), ptr(cu), N, B, T, H, dk, dv, nt)
    if rc < 0:
        raise RuntimeError(f"oracle bwd failed ({rc})")
    out["threads"] = rc
    return out
