"""Oracle for the step-size preprocessing read by the scan (fp64, CPU).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The mixer the DiffuMamba pages name is Mamba-2, whose step size is
dt = softplus(dt_raw + dt_bias) per head (the pages leave the form open;
this is its plainest reading, no clamping). Evaluated as
max(v, 0) + log1p(exp(-|v|)), exact in fp64 to rounding.

Parity: pinned (tests/test_oracle_pins.py, dt section).
"""
import numpy as np


def _f64(a):
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def softplus(v):
    v = _f64(v)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def preprocess_dt(raw, bias=None):
    """raw [..., H] pre-activations, bias [H] or None -> dt [..., H]."""
    raw = _f64(raw)
    if bias is not None:
        raw = raw + _f64(bias)
    return softplus(raw)
