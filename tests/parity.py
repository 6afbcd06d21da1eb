"""Tolerances of the parity tests, written out once.

fp32 inputs : max |x_gpu - x| / max |x| <= 1e-4            (o and S_T separately)
bf16 inputs : max |x_gpu - x| <= 2e-2 * rms(x)             (fp32 output; S_T against
                                                            its own RMS)
bf16 output : |x_gpu - x| <= 2e-2 * rms(x) + half a bf16 ulp of x, elementwise:
              the stored value is the computed one rounded to bf16, and that
              rounding alone reaches 2e-2 * rms(x) on the full 1.3B-layer
              workload for the exact result.
x is the fp64 oracle's value.
"""
import numpy as np

FP32_MAX_REL = 1e-4
BF16_RMS_FRAC = 2e-2


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def err_fp32(got, ref):
    got, ref = _f64(got), _f64(ref)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def err_rms(got, ref):
    """max |got - ref| / rms(ref)"""
    got, ref = _f64(got), _f64(ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref)) / max(rms, 1e-300))


def half_ulp_bf16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def err_rms_bf16_out(got, ref):
    """max over elements of (|got - ref| - half_ulp_bf16(ref)) / rms(ref)."""
    got, ref = _f64(got), _f64(ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref) - half_ulp_bf16(ref)) / max(rms, 1e-300))


def assert_fp32(got, ref, what):
    e = err_fp32(got, ref)
    assert e <= FP32_MAX_REL, f"{what}: max rel error {e:.3e} > {FP32_MAX_REL}"
    return e


def assert_rms(got, ref, what):
    e = err_rms(got, ref)
    assert e <= BF16_RMS_FRAC, f"{what}: max|err|/rms {e:.4f} > {BF16_RMS_FRAC}"
    return e


def assert_rms_bf16_out(got, ref, what):
    e = err_rms_bf16_out(got, ref)
    assert e <= BF16_RMS_FRAC, f"{what}: (max|err| - half ulp)/rms {e:.4f} > {BF16_RMS_FRAC}"
    return e
