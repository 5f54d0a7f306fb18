"""Pins of the oracle against facts that do not come from the oracle itself.

Each pin returns the worst error it found (0.0 when exact). They are shared
by test_oracle_pins.py (the oracle must pass them all) and
test_oracle_mutants.py (an oracle with a planted mistake must fail at least
one of them).
"""
import json
import os

import numpy as np

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def rand_dir(rng, batch, L, H, P, N, G, with_D=True):
    """A small random direction in the workload's distributions (fp64)."""
    return dict(
        x=rng.standard_normal((batch, L, H, P)),
        dt=np.log1p(np.exp(rng.standard_normal((batch, L, H)) - 2.0)),
        A=-np.exp(rng.uniform(0, np.log(16.0), H)),
        B=rng.standard_normal((batch, L, G, N)) / 4,
        C=rng.standard_normal((batch, L, G, N)) / 4,
        D=rng.standard_normal(H) if with_D else None)


def _golden_dir(d, L, P, N):
    x = np.asarray(d["x"], dtype=np.float64).reshape(1, L, 1, P)
    return dict(x=x,
                dt=np.asarray(d["dt"], dtype=np.float64).reshape(1, L, 1),
                A=np.asarray([d["A"]], dtype=np.float64),
                B=np.asarray(d["B"], dtype=np.float64).reshape(1, L, 1, N),
                C=np.asarray(d["C"], dtype=np.float64).reshape(1, L, 1, N),
                D=np.asarray([d["D"]], dtype=np.float64))


def pin_golden(name, lib=None):
    """Hand-derived fixtures under tests/golden."""
    g = json.load(open(os.path.join(GOLDEN, name)))
    y_ref = np.asarray(g["y"], dtype=np.float64)
    L = y_ref.shape[0]
    P = 1 if y_ref.ndim == 1 else y_ref.shape[1]
    fs_ref = np.asarray(g["final_state_fwd"], dtype=np.float64)
    N = fs_ref.size // P
    f = _golden_dir(g["fwd"], L, P, N)
    b = _golden_dir(g["bwd"], L, P, N)
    y, fs = oracle.bissd(f, b, want_final_state=True, lib=lib)
    y1 = oracle.bissd(f, None, lib=lib)
    err = max(np.max(np.abs(y.reshape(-1) - y_ref.reshape(-1))),
              np.max(np.abs(y1.reshape(-1) -
                            np.asarray(g["y_fwd_only"]).reshape(-1))),
              np.max(np.abs(fs.reshape(-1) - fs_ref.reshape(-1))))
    return float(err)


def pin_brute(lib=None, seed=0):
    """Recurrence == quadratic masked C.B^T form (both directions, groups)."""
    rng = _rng(seed)
    batch, L, H, P, N, G = 2, 13, 4, 3, 5, 2
    f = rand_dir(rng, batch, L, H, P, N, G)
    b = rand_dir(rng, batch, L, H, P, N, G)
    y = oracle.bissd(f, b, lib=lib)
    ref = brute.bissd(f, b)
    y1 = oracle.bissd(f, None, lib=lib)
    ref1 = brute.bissd(f, None)
    scale = np.max(np.abs(ref))
    return float(max(np.max(np.abs(y - ref)), np.max(np.abs(y1 - ref1))) / scale)


def pin_A_zero(lib=None, seed=1):
    """A = 0: the state is a dt-weighted running sum of B x^T (closed form)."""
    rng = _rng(seed)
    batch, L, H, P, N, G = 1, 40, 2, 3, 4, 1
    f = rand_dir(rng, batch, L, H, P, N, G)
    b = rand_dir(rng, batch, L, H, P, N, G)
    f["A"] = np.zeros(H)
    b["A"] = np.zeros(H)
    y = oracle.bissd(f, b, lib=lib)
    ref = np.zeros_like(y)
    for d, rev in ((f, False), (b, True)):
        # outer[t,h,p,n] = dt_t B_t[n] x_t[p]
        outer = (d["dt"][0][:, :, None, None] * d["x"][0][:, :, :, None]
                 * d["B"][0][:, None, None, 0, :].repeat(H, axis=1))
        if rev:
            S = np.cumsum(outer[::-1], axis=0)[::-1]
        else:
            S = np.cumsum(outer, axis=0)
        ref[0] += np.einsum("tn,thpn->thp", d["C"][0][:, 0, :], S)
        ref[0] += d["D"][None, :, None] * d["x"][0]
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def pin_A_neg_inf(lib=None, seed=2):
    """A -> -inf: nothing is carried, y_t = dt_t (C_t.B_t) x_t + D x_t."""
    rng = _rng(seed)
    batch, L, H, P, N, G = 2, 9, 2, 3, 4, 1
    f = rand_dir(rng, batch, L, H, P, N, G)
    b = rand_dir(rng, batch, L, H, P, N, G)
    f["A"] = np.full(H, -np.inf)
    b["A"] = np.full(H, -np.inf)
    y = oracle.bissd(f, b, lib=lib)
    ref = np.zeros_like(y)
    for d in (f, b):
        cb = np.sum(d["C"][:, :, 0, :] * d["B"][:, :, 0, :], axis=-1)  # [b,L]
        ref += (d["dt"] * cb[:, :, None])[..., None] * d["x"]
        ref += d["D"][None, None, :, None] * d["x"]
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def pin_L1(lib=None, seed=3):
    """L = 1: a single token, both directions see only itself."""
    rng = _rng(seed)
    f = rand_dir(rng, 3, 1, 2, 2, 3, 1)
    b = rand_dir(rng, 3, 1, 2, 2, 3, 1)
    y = oracle.bissd(f, b, lib=lib)
    ref = np.zeros_like(y)
    for d in (f, b):
        cb = np.sum(d["C"][:, :, 0, :] * d["B"][:, :, 0, :], axis=-1)
        ref += (d["dt"] * cb[:, :, None])[..., None] * d["x"] + d["D"][None, None, :, None] * d["x"]
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def _flip(d):
    out = {}
    for k, v in d.items():
        out[k] = v[:, ::-1].copy() if k in ("x", "dt", "B", "C") else v
    return out


def pin_time_reversal(lib=None, seed=4):
    """Reverse stream == flip(forward stream(flip(inputs))), bit for bit."""
    rng = _rng(seed)
    batch, L, H, P, N, G = 2, 17, 2, 3, 4, 1
    b = rand_dir(rng, batch, L, H, P, N, G)
    silent = rand_dir(rng, batch, L, H, P, N, G)
    silent["x"] = np.zeros_like(silent["x"])   # forward stream adds exact zeros
    silent["D"] = np.zeros(H)
    y_rev = oracle.bissd(silent, b, lib=lib)
    y_flip = oracle.bissd(_flip(b), None, lib=lib)[:, ::-1]
    return float(np.max(np.abs(y_rev - y_flip)))


def pin_block_exact(lib=None, seed=5):
    """Block-by-block decoding with a carried forward state equals the full
    scan ("Fixed state, long reach", Sec. 1: the cache is exact); the block
    step's reverse part equals the full reverse scan with a reset at every
    block end; the committed state equals the full scan's final state."""
    rng = _rng(seed)
    L, Lb, H, P, N, G = 24, 6, 2, 3, 4, 1
    f = rand_dir(rng, 1, L, H, P, N, G)
    b = rand_dir(rng, 1, L, H, P, N, G)
    y_full_f, fs_full = oracle.bissd(f, None, want_final_state=True, lib=lib)
    cu = list(range(0, L + 1, Lb))
    y_full_b_blocks = oracle.bissd(
        dict(f, x=np.zeros_like(f["x"]), D=np.zeros(H)), b, cu_seqlens=cu, lib=lib)
    state = np.zeros((1, H, P, N))
    silent_f = dict(f, x=np.zeros_like(f["x"]), D=np.zeros(H))
    silent_b = dict(b, x=np.zeros_like(b["x"]), D=np.zeros(H))
    errs = []
    for k in range(L // Lb):
        sl = slice(k * Lb, (k + 1) * Lb)

        def cut(d):
            return {kk: (v[:, sl] if kk in ("x", "dt", "B", "C") else v) for kk, v in d.items()}
        y_fwd = oracle.block_step(state, cut(f), cut(silent_b), lib=lib)[0]
        y_bwd = oracle.block_step(np.zeros_like(state), cut(silent_f), cut(b), lib=lib)[0]
        yk, state = oracle.block_step(state, cut(f), cut(b), commit=True, lib=lib)
        errs.append(np.max(np.abs(y_fwd - y_full_f[:, sl])))
        errs.append(np.max(np.abs(y_bwd - y_full_b_blocks[:, sl])))
        errs.append(np.max(np.abs(yk - (y_fwd + y_bwd))))
    errs.append(np.max(np.abs(state - fs_full)))
    return float(max(errs))


def pin_packed(lib=None, seed=6):
    """Packed sequences (with an empty one) == each sequence run alone."""
    rng = _rng(seed)
    lens = [5, 0, 9, 1, 7]
    L, H, P, N, G = sum(lens), 2, 3, 4, 1
    f = rand_dir(rng, 1, L, H, P, N, G)
    b = rand_dir(rng, 1, L, H, P, N, G)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    y, fs = oracle.bissd(f, b, cu_seqlens=cu, want_final_state=True, lib=lib)
    errs = []
    for i, n in enumerate(lens):
        sl = slice(cu[i], cu[i + 1])
        fi = {k: (v[:, sl] if k in ("x", "dt", "B", "C") else v) for k, v in f.items()}
        bi = {k: (v[:, sl] if k in ("x", "dt", "B", "C") else v) for k, v in b.items()}
        yi, fsi = oracle.bissd(fi, bi, want_final_state=True, lib=lib)
        if n:
            errs.append(np.max(np.abs(yi - y[:, sl])))
        errs.append(np.max(np.abs(fsi[0] - fs[i])))
    return float(max(errs))


def pin_linearity(lib=None, seed=7):
    """y is linear in x (D included) for fixed dt, A, B, C."""
    rng = _rng(seed)
    batch, L, H, P, N, G = 1, 11, 2, 3, 4, 1
    f = rand_dir(rng, batch, L, H, P, N, G)
    b = rand_dir(rng, batch, L, H, P, N, G)
    x2f = rng.standard_normal(f["x"].shape)
    x2b = rng.standard_normal(b["x"].shape)
    y1 = oracle.bissd(f, b, lib=lib)
    y2 = oracle.bissd(dict(f, x=x2f), dict(b, x=x2b), lib=lib)
    y3 = oracle.bissd(dict(f, x=2 * f["x"] - 3 * x2f), dict(b, x=2 * b["x"] - 3 * x2b), lib=lib)
    return float(np.max(np.abs(y3 - (2 * y1 - 3 * y2))) / np.max(np.abs(y3)))


ALL_PINS = {
    "golden_scalar": (lambda lib: pin_golden("scalar_L3.json", lib), 1e-12),
    "golden_2x2": (lambda lib: pin_golden("state2x2_L2.json", lib), 1e-12),
    "brute": (pin_brute, 1e-12),
    "A_zero": (pin_A_zero, 1e-12),
    "A_neg_inf": (pin_A_neg_inf, 1e-12),
    "L1": (pin_L1, 1e-12),
    "time_reversal": (pin_time_reversal, 0.0),
    "block_exact": (pin_block_exact, 0.0),
    "packed": (pin_packed, 0.0),
    "linearity": (pin_linearity, 1e-12),
}
