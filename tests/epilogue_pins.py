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


# ---- the step-size preprocessing (oracle/dt.py)

def pin_dt_torch(mod, seed=94):
    """== torch.nn.functional.softplus(raw + bias) in fp64 (its linear region
    starts at 20, where the two differ by less than e^-20)."""
    rng = np.random.default_rng(seed)
    raw = rng.standard_normal((5, 7)) * 6
    bias = rng.uniform(-3, 1, 7)
    got = mod.preprocess_dt(raw, bias)
    ref = F.softplus(torch.from_numpy(raw + bias)).numpy()
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)))


def pin_dt_identities(mod):
    """softplus(0) = ln 2; softplus(v) - softplus(-v) = v; softplus(-40) =
    e^-40 to 1e-17 relative."""
    v = np.linspace(-30, 30, 121)
    worst = abs(float(mod.softplus(np.array([0.0]))[0]) - np.log(2.0))
    worst = max(worst, float(np.max(np.abs(mod.softplus(v) - mod.softplus(-v) - v))))
    small = float(mod.softplus(np.array([-40.0]))[0])
    worst = max(worst, abs(small - np.exp(-40.0)) / np.exp(-40.0))
    return worst


DT_PINS = {
    "dt_torch": (pin_dt_torch, 1e-9),
    "dt_identities": (pin_dt_identities, 1e-14),
}


# ---- the concatenating merge (oracle/merge.py)

def _merge_draw(seed, rows=5, cin=3, cout=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, cin)), rng.standard_normal((rows, cin)),
            rng.standard_normal((cout, 2 * cin)), rng.standard_normal(cout))


def pin_merge_loops(mod, seed=95):
    """Explicit sums: out[t][o] = sum_c W[o][c] y_fwd[t][c] + W[o][cin + c] y_bwd[t][c] + b[o]."""
    yf, yb, w, b = _merge_draw(seed)
    got = mod.merge_linear(yf, yb, w, b)
    worst = 0.0
    for t in range(yf.shape[0]):
        for o in range(w.shape[0]):
            ref = b[o]
            for c in range(yf.shape[1]):
                ref += w[o][c] * yf[t][c] + w[o][yf.shape[1] + c] * yb[t][c]
            worst = max(worst, abs(got[t][o] - ref))
    return worst


def pin_merge_torch(mod, seed=96):
    """== torch.nn.functional.linear(cat(y_fwd, y_bwd), W, b) in fp64."""
    yf, yb, w, b = _merge_draw(seed, rows=7, cin=6, cout=5)
    got = mod.merge_linear(yf, yb, w, b)
    ref = F.linear(torch.cat([torch.from_numpy(yf), torch.from_numpy(yb)], -1),
                   torch.from_numpy(w), torch.from_numpy(b)).numpy()
    return float(np.max(np.abs(got - ref)))


MERGE_PINS = {
    "merge_loops": (pin_merge_loops, 1e-13),
    "merge_torch": (pin_merge_torch, 1e-13),
}
