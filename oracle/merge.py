"""Oracle for the concatenating merge of the two streams (fp64, CPU).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The DiffuMamba blog's bidirectional block ("network architecture")
concatenates the forward output and the flipped-back reverse output along
the channels and applies a Linear layer back to one width:
out = [y_fwd ; y_bwd] W^T + bias, W of shape (cout, 2 cin). One matmul
(numpy) as the step.

Parity: pinned (tests/test_oracle_pins.py, merge section).
"""
import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def merge_linear(y_fwd, y_bwd, weight, bias=None):
    """y_fwd, y_bwd [..., cin]; weight [cout, 2 cin]; bias [cout] or None."""
    yf, yb, w, b = _f64(y_fwd), _f64(y_bwd), _f64(weight), _f64(bias)
    cat = np.concatenate([yf, yb], axis=-1)
    out = cat @ w.T
    if b is not None:
        out = out + b
    return out
