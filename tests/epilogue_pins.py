"""Pins of the epilogue oracle (oracle/epilogue.py) against facts that do
not come from it: torch's own RMS norm and SiLU, the unit mean square of a
normalized group, scale invariance, and the independence of groups.

Each pin takes the module under test (the oracle or a copy with a planted
mistake) and returns the worst error it found.
"""
import numpy as np
import torch
import torch.nn.functional as F


def _draw(seed, shape, C):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape + (C,)), rng.standard_normal(shape + (C,)),
            rng.uniform(0.5, 1.5, C))


def pin_torch(mod, seed=90):
    """== torch.nn.functional.rms_norm(y * silu(z)) per group, fp64."""
    worst = 0.0
    for C, gs in ((48, 48), (48, 16), (40, 8)):
        y, z, w = _draw(seed, (3, 5), C)
        got = mod.gated_rmsnorm(y, z, w, gs, eps=1e-5)
        v = torch.from_numpy(y) * F.silu(torch.from_numpy(z))
        v = v.reshape(3, 5, C // gs, gs)
        ref = F.rms_norm(v, (gs,), eps=1e-5).reshape(3, 5, C) * torch.from_numpy(w)
        worst = max(worst, float(np.max(np.abs(got - ref.numpy()))))
    return worst


def pin_unit_mean_square(mod, seed=91):
    """With weight 1 and eps 0, every group of the output has mean square 1."""
    y, z, _ = _draw(seed, (4,), 64)
    out = mod.gated_rmsnorm(y, z, np.ones(64), 16, eps=0.0)
    ms = np.mean(out.reshape(4, 4, 16) ** 2, axis=-1)
    return float(np.max(np.abs(ms - 1.0)))


def pin_scale_invariant(mod, seed=92):
    """With eps 0, scaling y by a positive factor changes nothing."""
    y, z, w = _draw(seed, (6,), 32)
    a = mod.gated_rmsnorm(y, z, w, 32, eps=0.0)
    b = mod.gated_rmsnorm(7.5 * y, z, w, 32, eps=0.0)
    return float(np.max(np.abs(a - b)))


def pin_groups_independent(mod, seed=93):
    """Each group is normalized on its own: a group equals the whole-row
    norm of that group alone."""
    y, z, w = _draw(seed, (2, 3), 24)
    out = mod.gated_rmsnorm(y, z, w, 8, eps=1e-3)
    worst = 0.0
    for g0 in (0, 8, 16):
        alone = mod.gated_rmsnorm(y[..., g0:g0 + 8], z[..., g0:g0 + 8], w[g0:g0 + 8], 8, eps=1e-3)
        worst = max(worst, float(np.max(np.abs(out[..., g0:g0 + 8] - alone))))
    return worst


EPILOGUE_PINS = {
    "epi_torch": (pin_torch, 1e-13),
    "epi_unit_mean_square": (pin_unit_mean_square, 1e-13),
    "epi_scale_invariant": (pin_scale_invariant, 1e-13),
    "epi_groups_independent": (pin_groups_independent, 0.0),
}
