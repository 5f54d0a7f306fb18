"""Oracle for the gated-norm epilogue on the scan's output (fp64, CPU).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the smoke check; never
by the product package, which shares no code with it.

What the pages fix: each direction of the bidirectional block is a whole
Mamba block (DiffuMamba blog, "network architecture"), and the mixer is
Mamba-2 (DiffuMamba summaries, methodology sections). What they leave open,
and the reading taken here: Mamba-2's output gate and normalization, in its
default order -- the scan output y is gated by SiLU of the gate branch z,
then RMS-normalized over groups of ``group_size`` consecutive channels and
scaled per channel:

    v   = y * silu(z),          silu(u) = u / (1 + exp(-u))
    out = v / sqrt(mean_group(v^2) + eps) * weight

Written out with numpy per group; ``torch.nn.functional.rms_norm`` can
therefore pin it independently.

Parity: pinned (tests/test_oracle_pins.py, epilogue section).
"""
import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def silu(u):
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def gated_rmsnorm(y, z, weight, group_size, eps=1e-5):
    """y, z [..., C]; weight [C]; groups of group_size consecutive channels.
    Returns the fp64 output [..., C]."""
    y, z, w = _f64(y), _f64(z), _f64(weight)
    C = y.shape[-1]
    assert z.shape == y.shape and w.shape == (C,) and C % group_size == 0
    v = y * silu(z)
    out = np.empty_like(v)
    for g0 in range(0, C, group_size):
        part = v[..., g0:g0 + group_size]
        ms = np.mean(part * part, axis=-1, keepdims=True)
        out[..., g0:g0 + group_size] = part / np.sqrt(ms + eps) * w[g0:g0 + group_size]
    return out
