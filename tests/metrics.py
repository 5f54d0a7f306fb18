"""Parity measures used by the GPU tests.

fp32 workloads: elementwise relative error with a floor,
  max_i |y_i - r_i| / max(|r_i|, 0.01 * RMS(r))      must be <= 1e-4;
bf16-input workloads (fp32 accumulation):
  max_i |y_i - r_i| / RMS(r)                          must be <= 1e-2.
The floor keeps outputs that are near zero from turning a ratio of two
rounding residues into a failure. The same bf16 bound is applied to runs with
D = 0 (the state-space part alone), judged against that output's own RMS.
"""
import numpy as np

F32_TOL = 1e-4
BF16_TOL = 1e-2


def rel_err_f32(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    if rms == 0.0:
        # an all-zero reference: the largest deviation itself (0 when exact)
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 0.01 * rms)))


def rms_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    if rms == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / rms)


def within(got, ref, dtype):
    if dtype == "f32":
        e = rel_err_f32(got, ref)
        return e, e <= F32_TOL
    e = rms_err(got, ref)
    return e, e <= BF16_TOL


def bf16_rne(v):
    """Exact round-to-nearest-even of float64 values to bfloat16 (8
    significant bits), returned as float64. Normal range only."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def conv_close(got, ref, scale, dtype, rel=2.0 ** -18):
    """Output of the short convolution against the fp64 oracle.

    The kernel evaluates each output in fp32 from exact inputs: a handful of
    fused multiply-adds and one SiLU, so its value before the final rounding
    lies within delta = rel * (scale + |ref|) of the exact one, where
    ``scale`` is the same filter applied to |input|, |weight| and |bias|
    (bounding every partial sum). fp32 outputs must lie within delta; bf16
    outputs (rounded to nearest even, a monotone map) must lie between the
    roundings of ref - delta and ref + delta. Returns (worst excess, ok):
    the largest distance outside the interval in units of delta (0 when
    every element is inside it); ok is exact interval membership.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    delta = rel * (np.asarray(scale, dtype=np.float64) + np.abs(ref))
    if got.size == 0:
        return 0.0, True
    if dtype == "f32":
        lo, hi = ref - delta, ref + delta
    else:
        lo, hi = bf16_rne(ref - delta), bf16_rne(ref + delta)
    outside = np.maximum(np.maximum(lo - got, got - hi), 0.0)
    ok = bool(np.all((got >= lo) & (got <= hi)))
    return float(np.max(outside / np.maximum(delta, 1e-300))), ok
