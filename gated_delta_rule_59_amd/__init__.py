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
           "gdn2_fwd_noalloc", "gdn2_bwd", "gdn2_bwd_workspace_size", "gdn2_prologue",
           "gdn2_epilogue",
           "gdn2_version", "lib", "library_path", "GDN2_F32", "GDN2_BF16", "Gdn2Error"]

GDN2_F32, GDN2_BF16 = 0, 1
GDN2_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/gdn2.h: scratch of gdn2_fwd_noalloc per GPU
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
        L.gdn2_bwd_workspace_size.restype = sz
        L.gdn2_bwd_workspace_size.argtypes = [i32] * 7
        L.gdn2_bwd.restype = ctypes.c_int
        L.gdn2_bwd.argtypes = [P] * 6 + [i32, P, P, P] + [P] * 6 + [i32, P, P] + [i32] * 6 + \
            [P, sz, P]
        L.gdn2_fwd_ex.restype = ctypes.c_int
        L.gdn2_fwd_ex.argtypes = [P] * 6 + [i32, i32] + L.gdn2_fwd.argtypes[6:]
        L.gdn2_decode_ex.restype = ctypes.c_int
        L.gdn2_decode_ex.argtypes = [P] * 6 + [i32, i32] + L.gdn2_decode.argtypes[6:]
        f32 = ctypes.c_float
        L.gdn2_prologue.restype = ctypes.c_int
        L.gdn2_prologue.argtypes = [P] * 9 + [i32, f32] + [P] * 6 + [P] + [i32] * 7 + [P]
        L.gdn2_epilogue.restype = ctypes.c_int
        L.gdn2_epilogue.argtypes = [P, P, P, f32, P, i32, i32, i32, i32, i32, P]
        L.gdn2_fwd_noalloc.restype = ctypes.c_int
        L.gdn2_fwd_noalloc.argtypes = L.gdn2_fwd_gates.argtypes[:19] + [P]
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


# readings of the erase gate (gdn2_erase): b on the key that reads the
# prediction (every call's default), or b on the erased rows
ERASE_READ, ERASE_ROWS = 0, 1


def gdn2_fwd_gates(q, k, v, alpha, b, w, gates, S0=None, cu_seqlens=None, out_dtype=None,
                   final_state=True, workspace=None, erase=ERASE_READ):
    """gdn2_fwd with a gate form: GATES_KDA takes b, w as [B, T, H] (one value
    per token and head, for every channel), GATES_GDN alpha, b and w.
    erase=ERASE_ROWS takes the other reading of the erase gate (gdn2_fwd_ex:
    token-serial)."""
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
    st = lib().gdn2_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), gates,
                           erase, in_code, _ptr(S0), _ptr(o), _DT[odt], _ptr(ST),
                           _ptr(cu_seqlens), N, B, T, H, dk, dv, _ptr(workspace), ws_bytes,
                           _stream(dev))
    if st != 0:
        raise Gdn2Error(st, "gdn2_fwd_ex")
    return o, ST


def gdn2_fwd_noalloc(q, k, v, alpha, b, w, gates, o, S0=None, S_T=None, cu_seqlens=None):
    """gdn2_fwd_gates into caller-given outputs (o [B, T, H, dv], S_T fp32
    [N, H, dk, dv] or None), with no workspace: the C call allocates nothing
    and uses the library's per-GPU scratch where a workspace would be needed
    (GDN2_NOALLOC_SCRATCH_BYTES at most).  Calls that overlap on one GPU race
    on that scratch."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    sa, sb, sw = _gate_shapes((B, T, H), dk, dv, gates)
    dev, dt = _check_tokens(("q", "k", "v", "alpha", "b", "w"), (q, k, v, alpha, b, w),
                            ((B, T, H, dk), (B, T, H, dk), (B, T, H, dv), sa, sb, sw))
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    for name, t, shape, dts in (("o", o, (B, T, H, dv), tuple(_DT)),
                                ("S0", S0, (N, H, dk, dv), (torch.float32,)),
                                ("S_T", S_T, (N, H, dk, dv), (torch.float32,))):
        if t is None:
            if name == "o":
                raise ValueError("o is required")
            continue
        if t.device != dev or not t.is_contiguous() or t.dtype not in dts or \
                tuple(t.shape) != shape:
            raise ValueError(f"{name} must be a contiguous {dts} {shape} tensor on the "
                             "inputs' device")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev
                                   or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 vector on the inputs' device")
    st = lib().gdn2_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), gates,
                                _DT[dt], _ptr(S0), _ptr(o), _DT[o.dtype], _ptr(S_T),
                                _ptr(cu_seqlens), N, B, T, H, dk, dv, _stream(dev))
    if st != 0:
        raise Gdn2Error(st, "gdn2_fwd_noalloc")
    return o, S_T


def gdn2_bwd_workspace_size(B, T, H, dk, dv, num_seqs, in_dtype) -> int:
    return int(lib().gdn2_bwd_workspace_size(B, T, H, dk, dv, num_seqs, in_dtype))


def gdn2_bwd(q, k, v, alpha, b, w, dout, S0=None, dS_T=None, cu_seqlens=None, grad_dtype=None,
             workspace=None):
    """Gradients of L = sum <dout, o> + <dS_T, S_T> through gdn2_fwd.

    Inputs as for gdn2_fwd (per-channel gates); dout [B, T, H, dv] in the
    input dtype; dS_T fp32 [N, H, dk, dv] or None.  grad_dtype: dtype of
    the token gradients (the input dtype by default, or torch.float32).
    Returns dict dq, dk, dv, dalpha, db, dw, dS0 (fp32)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = _check_tokens(("q", "k", "v", "alpha", "b", "w", "dout"),
                            (q, k, v, alpha, b, w, dout),
                            ((B, T, H, dk), (B, T, H, dk), (B, T, H, dv), (B, T, H, dk),
                             (B, T, H, dk), (B, T, H, dv), (B, T, H, dv)))
    N = B
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or \
                not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous int32 vector on the inputs' device")
        N = cu_seqlens.numel() - 1
    for name, x in (("S0", S0), ("dS_T", dS_T)):
        if x is not None and (x.dtype != torch.float32 or x.device != dev or
                              not x.is_contiguous() or tuple(x.shape) != (N, H, dk, dv)):
            raise ValueError(f"{name} must be a contiguous float32 {(N, H, dk, dv)} tensor")
    gdt = dt if grad_dtype is None else grad_dtype
    if gdt not in _DT:
        raise TypeError(f"grad_dtype must be bfloat16 or float32, got {gdt}")
    out = {n: torch.empty((B, T, H, dk), dtype=gdt, device=dev) for n in ("dq", "dk", "dalpha", "db")}
    out.update({n: torch.empty((B, T, H, dv), dtype=gdt, device=dev) for n in ("dv", "dw")})
    out["dS0"] = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    need = gdn2_bwd_workspace_size(B, T, H, dk, dv, N, _DT[dt])
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib().gdn2_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _DT[dt],
                        _ptr(S0), _ptr(dout), _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]),
                        _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["db"]), _ptr(out["dw"]),
                        _DT[gdt], _ptr(out["dS0"]), _ptr(cu_seqlens), N, B, T, H, dk, dv,
                        _ptr(workspace), workspace.numel() * workspace.element_size(),
                        _stream(dev))
    if st != 0:
        raise Gdn2Error(st, "gdn2_bwd")
    return out


def gdn2_prologue(xq, xk, xv, ga, gb, gw, conv_q, conv_k, conv_v, cu_seqlens=None,
                  l2_eps=1e-6):
    """Mixer prologue: q, k = L2norm(SiLU(conv(x))), v = SiLU(conv(xv)),
    alpha, b, w = sigmoid(ga, gb, gw).  x*, g*: [B, T, H, d] (bf16 or fp32);
    conv_*: fp32 [H*d, K], K <= 4.  Returns (q, k, v, alpha, b, w)."""
    B, T, H, dk = xq.shape
    dv = xv.shape[-1]
    dev, dt = _check_tokens(("xq", "xk", "xv", "ga", "gb", "gw"), (xq, xk, xv, ga, gb, gw),
                            ((B, T, H, dk), (B, T, H, dk), (B, T, H, dv), (B, T, H, dk),
                             (B, T, H, dk), (B, T, H, dv)))
    K = conv_q.shape[-1]
    for name, W, d in (("conv_q", conv_q, dk), ("conv_k", conv_k, dk), ("conv_v", conv_v, dv)):
        if W.dtype != torch.float32 or W.device != dev or not W.is_contiguous() or \
                tuple(W.shape) != (H * d, K):
            raise ValueError(f"{name} must be a contiguous float32 {(H * d, K)} tensor")
    N = B
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or \
                not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous int32 vector on the inputs' device")
        N = cu_seqlens.numel() - 1
    outs = [torch.empty_like(x) for x in (xq, xk, xv, ga, gb, gw)]
    st = lib().gdn2_prologue(*[_ptr(x) for x in (xq, xk, xv, ga, gb, gw, conv_q, conv_k, conv_v)],
                             K, float(l2_eps), *[_ptr(x) for x in outs], _ptr(cu_seqlens), N, B,
                             T, H, dk, dv, _DT[dt], _stream(dev))
    if st != 0:
        raise Gdn2Error(st, "gdn2_prologue")
    return tuple(outs)


def gdn2_epilogue(o, g, gamma=None, eps=1e-6, out_dtype=None):
    """Mixer epilogue: y = RMSNorm(o) * gamma * SiLU(g) over the last axis.
    o, g: [.., H, dv] (bf16 or fp32, same dtype); gamma fp32 [dv] or None."""
    if o.shape != g.shape or o.dtype != g.dtype or o.device != g.device:
        raise ValueError("o and g must share shape, dtype and device")
    if o.dtype not in _DT or not o.is_contiguous() or not g.is_contiguous() or o.dim() < 2:
        raise ValueError("o and g must be contiguous bf16 or fp32 tensors [.., H, dv]")
    H, dv = o.shape[-2], o.shape[-1]
    rows = o.numel() // (H * dv)
    if gamma is not None and (gamma.dtype != torch.float32 or gamma.device != o.device or
                              gamma.numel() != dv or not gamma.is_contiguous()):
        raise ValueError("gamma must be a contiguous float32 [dv] tensor on the same device")
    odt = o.dtype if out_dtype is None else out_dtype
    y = torch.empty(o.shape, dtype=odt, device=o.device)
    st = lib().gdn2_epilogue(_ptr(o), _ptr(g), _ptr(gamma), float(eps), _ptr(y), rows, H, dv,
                             _DT[o.dtype], _DT[odt], _stream(o.device))
    if st != 0:
        raise Gdn2Error(st, "gdn2_epilogue")
    return y


def gdn2_decode(q, k, v, alpha, b, w, S, out_dtype=None):
    """One recurrent step. q, k, alpha, b: [N, H, dk]; v, w: [N, H, dv];
    S: fp32 [N, H, dk, dv], updated in place.  Returns o [N, H, dv]."""
    return gdn2_decode_gates(q, k, v, alpha, b, w, GATES_FULL, S, out_dtype)


def gdn2_decode_gates(q, k, v, alpha, b, w, gates, S, out_dtype=None, erase=ERASE_READ):
    """gdn2_decode with a gate form: GATES_KDA takes b, w as [N, H],
    GATES_GDN alpha, b and w; erase selects the erase gate's reading."""
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
    st = lib().gdn2_decode_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                              gates, erase, _DT[dt], _ptr(S), _ptr(o), _DT[odt], N, H, dk, dv,
                              _stream(dev))
    if st != 0:
        raise Gdn2Error(st, "gdn2_decode_ex")
    return o
