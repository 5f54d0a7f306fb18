"""Pins of the oracle's gradients (oracle.bissd_bwd, the adjoint recurrence)
against facts that do not come from it: central finite differences of the
forward oracle, torch's autograd through a plain torch recurrence, the flip
definition of the reverse stream, closed forms and exact identities.

Each pin takes an oracle library handle (None: the built one; or a copy
with a planted mistake) and returns the worst error it found.
"""
import numpy as np
import torch

import oracle
from pins import rand_dir

KEYS = oracle.GRAD_KEYS


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / scale


def _inputs(seed, batch=1, L=6, H=2, P=3, N=4, G=1):
    rng = np.random.default_rng(seed)
    f = rand_dir(rng, batch, L, H, P, N, G)
    b = rand_dir(rng, batch, L, H, P, N, G)
    dy = rng.standard_normal((batch, L, H, P))
    return f, b, dy


def pin_finite_differences(lib=None, seed=60):
    """Every gradient entry against a central difference of sum(y * dy)."""
    worst = 0.0
    for dims in (dict(L=6, H=2, P=3, N=4, G=1), dict(L=5, H=4, P=2, N=3, G=2)):
        f, b, dy = _inputs(seed, **dims)
        gf, gb = oracle.bissd_bwd(f, b, dy, lib=lib)

        def loss():
            return float(np.sum(oracle.bissd(f, b, lib=lib) * dy))

        eps = 1e-5
        for d, g in ((f, gf), (b, gb)):
            for k in KEYS:
                a = d[k]
                num = np.empty_like(a)
                for idx in np.ndindex(a.shape):
                    a0 = a[idx]
                    a[idx] = a0 + eps
                    lp = loss()
                    a[idx] = a0 - eps
                    lm = loss()
                    a[idx] = a0
                    num[idx] = (lp - lm) / (2 * eps)
                worst = max(worst, _rel(g[k], num))
    return worst


def _torch_direction(x, dt, A, B, C, D, reverse):
    """Plain torch recurrence of one direction, one row: x [L,H,P]."""
    L, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    cols = []
    for h in range(H):
        g = h // (H // G)
        st = torch.zeros(P, N, dtype=torch.float64)
        ys = [None] * L
        for t in (range(L - 1, -1, -1) if reverse else range(L)):
            st = torch.exp(dt[t, h] * A[h]) * st + dt[t, h] * torch.outer(x[t, h], B[t, g])
            ys[t] = st @ C[t, g] + D[h] * x[t, h]
        cols.append(torch.stack(ys))
    return torch.stack(cols, dim=1)


def pin_autograd(lib=None, seed=61):
    """The adjoint against torch.autograd through a plain torch recurrence
    (fp64, both directions, two rows, grouped heads)."""
    batch, L, H, P, N, G = 2, 24, 4, 5, 6, 2
    f, b, dy = _inputs(seed, batch, L, H, P, N, G)
    gf, gb = oracle.bissd_bwd(f, b, dy, lib=lib)
    tf = {k: torch.tensor(v, requires_grad=True) for k, v in f.items()}
    tb = {k: torch.tensor(v, requires_grad=True) for k, v in b.items()}
    y = torch.stack([
        _torch_direction(tf["x"][r], tf["dt"][r], tf["A"], tf["B"][r], tf["C"][r], tf["D"], False) +
        _torch_direction(tb["x"][r], tb["dt"][r], tb["A"], tb["B"][r], tb["C"][r], tb["D"], True)
        for r in range(batch)])
    (y * torch.from_numpy(dy)).sum().backward()
    worst = 0.0
    for t, g in ((tf, gf), (tb, gb)):
        for k in KEYS:
            worst = max(worst, _rel(g[k], t[k].grad.numpy()))
    return worst


def _flip(d):
    out = dict(d)
    for k in ("x", "dt", "B", "C"):
        out[k] = np.ascontiguousarray(d[k][:, ::-1])
    return out


def pin_reverse_is_flip(lib=None, seed=62):
    """Reverse-stream gradients == flipped forward-stream gradients of the
    flipped inputs and flipped dy, bit for bit."""
    f, b, dy = _inputs(seed, batch=2, L=9, H=2, P=3, N=4)
    _, gb = oracle.bissd_bwd(f, b, dy, lib=lib)
    gflip, _ = oracle.bissd_bwd(_flip(b), None, np.ascontiguousarray(dy[:, ::-1]), lib=lib)
    worst = 0.0
    for k in KEYS:
        ref = gflip[k][:, ::-1] if k in ("x", "dt", "B", "C") else gflip[k]
        worst = max(worst, float(np.max(np.abs(gb[k] - ref))))
    return worst


def pin_dD_closed_form(lib=None, seed=63):
    """dD_h = sum_t x_t . dy_t (each direction its own x)."""
    f, b, dy = _inputs(seed, batch=2, L=7, H=3, P=4, N=2)
    gf, gb = oracle.bissd_bwd(f, b, dy, lib=lib)
    worst = 0.0
    for d, g in ((f, gf), (b, gb)):
        worst = max(worst, _rel(g["D"], np.einsum("blhp,blhp->h", d["x"], dy)))
    return worst


def pin_packed_independent(lib=None, seed=64):
    """Packed sequences (one empty) == each sequence alone, bit for bit."""
    lens = [4, 0, 1, 6, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    f, b, dy = _inputs(seed, batch=1, L=int(cu[-1]), H=2, P=3, N=4)
    gf, gb = oracle.bissd_bwd(f, b, dy, cu_seqlens=cu, lib=lib)
    worst = 0.0
    sum_AD = {("f", "A"): 0.0, ("f", "D"): 0.0, ("b", "A"): 0.0, ("b", "D"): 0.0}
    for j, n in enumerate(lens):
        if n == 0:
            continue
        a = int(cu[j])

        def cut(d):
            return {k: (v[:, a:a + n] if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
        sf, sb = oracle.bissd_bwd(cut(f), cut(b), dy[:, a:a + n], lib=lib)
        for tag, g, s in (("f", gf, sf), ("b", gb, sb)):
            for k in ("x", "dt", "B", "C"):
                worst = max(worst, float(np.max(np.abs(g[k][:, a:a + n] - s[k]))))
            sum_AD[(tag, "A")] = sum_AD[(tag, "A")] + s["A"]
            sum_AD[(tag, "D")] = sum_AD[(tag, "D")] + s["D"]
    for tag, g in (("f", gf), ("b", gb)):
        for k in ("A", "D"):
            worst = max(worst, _rel(g[k], sum_AD[(tag, k)]))
    return worst


def pin_linear_in_dy(lib=None, seed=65):
    """Gradients are linear in dy: doubling dy doubles every gradient exactly."""
    f, b, dy = _inputs(seed, batch=1, L=8, H=2, P=3, N=4)
    g1f, g1b = oracle.bissd_bwd(f, b, dy, lib=lib)
    g2f, g2b = oracle.bissd_bwd(f, b, 2.0 * dy, lib=lib)
    worst = 0.0
    for a, c in ((g1f, g2f), (g1b, g2b)):
        for k in KEYS:
            worst = max(worst, float(np.max(np.abs(2.0 * a[k] - c[k]))))
    return worst


BWD_PINS = {
    "bwd_finite_differences": (pin_finite_differences, 1e-7),
    "bwd_autograd": (pin_autograd, 1e-12),
    "bwd_reverse_is_flip": (pin_reverse_is_flip, 0.0),
    "bwd_dD_closed_form": (pin_dD_closed_form, 1e-14),
    "bwd_packed_independent": (pin_packed_independent, 1e-14),
    "bwd_linear_in_dy": (pin_linear_in_dy, 0.0),
}
