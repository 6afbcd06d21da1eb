"""MI355X (gfx950) Gated Delta Rule-2: Python face of the C ABI in include/gdn2.h.

Argument marshalling only: every step of the recurrence runs in the HIP
kernels of libgdn2.so (built in-tree by gated_delta_rule_59_amd/build.py).
PyTorch supplies device memory and the current HIP stream.  There is no CPU
fallback: if the library is missing, every call raises.

    gdn2_fwd(q, k, v, alpha, b, w, S0=None, cu_seqlens=None, out_dtype=None,
             final_state=True, workspace=None) -> (o, S_T)
    gdn2_decode(q, k, v, alpha, b, w, S, out_dtype=None) -> o   (S updated in place)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["gdn2_fwd", "gdn2_decode", "gdn2_fwd_workspace_size", "gdn2_status_string",
           "gdn2_version", "lib", "library_path", "GDN2_F32", "GDN2_BF16", "Gdn2Error"]

GDN2_F32, GDN2_BF16 = 0, 1
_DT = {torch.float32: GDN2_F32, torch.bfloat16: GDN2_BF16}
_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))


class Gdn2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {gdn2_status_string(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libgdn2.so")


def lib():
    """The loaded C library (ctypes). Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"HIP library not built: {path} is missing "
                               "(run gated_delta_rule_59_amd/build.py)")
        L = ctypes.CDLL(path)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.gdn2_version.restype = ctypes.c_int
        L.gdn2_version.argtypes = []
        L.gdn2_status_string.restype = ctypes.c_char_p
        L.gdn2_status_string.argtypes = [ctypes.c_int]
        L.gdn2_fwd_workspace_size.restype = sz
        L.gdn2_fwd_workspace_size.argtypes = [i32] * 7
        L.gdn2_fwd.restype = ctypes.c_int
        L.gdn2_fwd.argtypes = [P, P, P, P, P, P, i32, P, P, i32, P, P, i32, i32, i32, i32, i32, i32,
                               P, sz, P]
        L.gdn2_decode.restype = ctypes.c_int
        L.gdn2_decode.argtypes = [P, P, P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, P]
        L.gdn2_fwd_gates.restype = ctypes.c_int
        L.gdn2_fwd_gates.argtypes = [P] * 6 + [i32] + L.gdn2_fwd.argtypes[6:]
        L.gdn2_decode_gates.restype = ctypes.c_int
        L.gdn2_decode_gates.argtypes = [P] * 6 + [i32] + L.gdn2_decode.argtypes[6:]
        _LIB = L
    return _LIB


def gdn2_version() -> int:
    return int(lib().gdn2_version())


def gdn2_status_string(status: int) -> str:
    return lib().gdn2_status_string(int(status)).decode()


def gdn2_fwd_workspace_size(B, T, H, dk, dv, num_seqs, in_dtype) -> int:
    return int(lib().gdn2_fwd_workspace_size(B, T, H, dk, dv, num_seqs, in_dtype))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tokens(names, tensors, shapes):
    dev = tensors[0].device
    dt = tensors[0].dtype
    if dt not in _DT:
        raise TypeError(f"token inputs must be bfloat16 or float32, got {dt}")
    for n, t, s in zip(names, tensors, shapes):
        if t.device != dev or t.dtype != dt:
            raise TypeError(f"{n}: all token inputs must share device and dtype")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
        if tuple(t.shape) != tuple(s):
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {tuple(s)}")
    if dev.type != "cuda":
        raise ValueError("inputs must be GPU tensors")
    return dev, dt


# gate forms (gdn2_gates): per channel; b and w per (token, head) (the Kimi
# Delta Attention form); alpha, b and w per (token, head) (the Gated DeltaNet form)
GATES_FULL, GATES_KDA, GATES_GDN = 0, 1, 2


def _gate_shapes(lead, dk, dv, gates):
    """Expected shapes of alpha, b, w: [*lead, d] per channel, [*lead] per head."""
    if gates not in (GATES_FULL, GATES_KDA, GATES_GDN):
        raise ValueError(f"gates must be GATES_FULL, GATES_KDA or GATES_GDN, got {gates}")
    ph = gates != GATES_FULL
    return ((*lead,) if gates == GATES_GDN else (*lead, dk),
            (*lead,) if ph else (*lead, dk),
            (*lead,) if ph else (*lead, dv))


def gdn2_fwd(q, k, v, alpha, b, w, S0=None, cu_seqlens=None, out_dtype=None,
             final_state=True, workspace=None):
    """Chunkwise-WY forward. q, k, alpha, b: [B, T, H, dk]; v, w: [B, T, H, dv].

    S0: fp32 [N, H, dk, dv] or None (zeros).  cu_seqlens: int32 [N+1] on the
    device (then B must be 1) or None (N = B).  out_dtype: dtype of o (the
    input dtype by default, or torch.float32).  workspace: a contiguous device
    buffer of at least gdn2_fwd_workspace_size(...) bytes, or None (one is
    allocated when needed).  Returns (o, S_T or None).
    """
    return gdn2_fwd_gates(q, k, v, alpha, b, w, GATES_FULL, S0, cu_seqlens, out_dtype,
                          final_state, workspace)


def gdn2_fwd_gates(q, k, v, alpha, b, w, gates, S0=None, cu_seqlens=None, out_dtype=None,
                   final_state=True, workspace=None):
    """gdn2_fwd with a gate form: GATES_KDA takes b, w as [B, T, H] (one value
    per token and head, for every channel), GATES_GDN alpha, b and w."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    sa, sb, sw = _gate_shapes((B, T, H), dk, dv, gates)
    dev, dt = _check_tokens(("q", "k", "v", "alpha", "b", "w"), (q, k, v, alpha, b, w),
                            ((B, T, H, dk), (B, T, H, dk), (B, T, H, dv), sa, sb, sw))
    N = B
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be an int32 vector on the inputs' device")
        if not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous")
        N = cu_seqlens.numel() - 1
    if S0 is not None:
        if S0.dtype != torch.float32 or S0.device != dev or not S0.is_contiguous():
            raise ValueError("S0 must be a contiguous float32 tensor on the inputs' device")
        if tuple(S0.shape) != (N, H, dk, dv):
            raise ValueError(f"S0 has shape {tuple(S0.shape)}, expected {(N, H, dk, dv)}")
    odt = dt if out_dtype is None else out_dtype
    if odt not in _DT:
        raise TypeError(f"out_dtype must be bfloat16 or float32, got {odt}")
    o = torch.empty((B, T, H, dv), dtype=odt, device=dev)
    ST = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if final_state else None
    in_code = _DT[dt]
    need = gdn2_fwd_workspace_size(B, T, H, dk, dv, N, in_code)
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().gdn2_fwd_gates(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), gates,
                              in_code, _ptr(S0), _ptr(o), _DT[odt], _ptr(ST), _ptr(cu_seqlens),
                              N, B, T, H, dk, dv, _ptr(workspace), ws_bytes, _stream(dev))
    if st != 0:
        raise Gdn2Error(st, "gdn2_fwd_gates")
    return o, ST


def gdn2_decode(q, k, v, alpha, b, w, S, out_dtype=None):
    """One recurrent step. q, k, alpha, b: [N, H, dk]; v, w: [N, H, dv];
    S: fp32 [N, H, dk, dv], updated in place.  Returns o [N, H, dv]."""
    return gdn2_decode_gates(q, k, v, alpha, b, w, GATES_FULL, S, out_dtype)


def gdn2_decode_gates(q, k, v, alpha, b, w, gates, S, out_dtype=None):
    """gdn2_decode with a gate form: GATES_KDA takes b, w as [N, H],
    GATES_GDN alpha, b and w."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    sa, sb, sw = _gate_shapes((N, H), dk, dv, gates)
    dev, dt = _check_tokens(("q", "k", "v", "alpha", "b", "w"), (q, k, v, alpha, b, w),
                            ((N, H, dk), (N, H, dk), (N, H, dv), sa, sb, sw))
    if S.dtype != torch.float32 or S.device != dev or not S.is_contiguous() or \
            tuple(S.shape) != (N, H, dk, dv):
        raise ValueError(f"S must be a contiguous float32 [N, H, dk, dv] = {(N, H, dk, dv)} "
                         "tensor on the inputs' device")
    odt = dt if out_dtype is None else out_dtype
    if odt not in _DT:
        raise TypeError(f"out_dtype must be bfloat16 or float32, got {odt}")
    o = torch.empty((N, H, dv), dtype=odt, device=dev)
    st = lib().gdn2_decode_gates(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                 gates, _DT[dt], _ptr(S), _ptr(o), _DT[odt], N, H, dk, dv,
                                 _stream(dev))
    if st != 0:
        raise Gdn2Error(st, "gdn2_decode_gates")
    return o
