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
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 0.01 * rms)))


def rms_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(got - ref)) / rms)


def within(got, ref, dtype):
    if dtype == "f32":
        e = rel_err_f32(got, ref)
        return e, e <= F32_TOL
    e = rms_err(got, ref)
    return e, e <= BF16_TOL
