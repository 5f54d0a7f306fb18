"""Pins of the convolution oracle (oracle/conv.py) against facts that do not
come from it: torch's own depthwise convolution, impulse responses, the flip
definition of the reverse direction, and the carried-context and packing
identities.

Each pin takes the module under test (the oracle, or a copy of it with a
planted mistake) and returns the worst error it found (0.0 when exact).
"""
import numpy as np
import torch
import torch.nn.functional as F


def _rng(seed):
    return np.random.default_rng(seed)


def _draw(rng, batch, L, ch, W):
    return (rng.standard_normal((batch, L, ch)),
            rng.uniform(-0.5, 0.5, (ch, W)),
            rng.uniform(-0.5, 0.5, ch))


def _torch_causal(u, w, b, silu):
    """torch.nn.functional.conv1d, fp64, depthwise, left padding W-1."""
    batch, L, ch = u.shape
    W = w.shape[1]
    ut = torch.from_numpy(u).permute(0, 2, 1)                 # [batch, ch, L]
    wt = torch.from_numpy(w).reshape(ch, 1, W)
    out = F.conv1d(ut, wt, torch.from_numpy(b), padding=W - 1, groups=ch)[..., :L]
    if silu:
        out = F.silu(out)
    return out.permute(0, 2, 1).numpy()


def pin_torch(mod, seed=30):
    """Forward == torch's depthwise conv; reverse == flip(conv(flip(.)))."""
    rng = _rng(seed)
    worst = 0.0
    for W in (4, 3, 2):
        u, w, b = _draw(rng, 2, 37, 24, W)
        for silu in (False, True):
            act = "silu" if silu else "none"
            fwd = mod.conv1d(u, w, b, activation=act)
            worst = max(worst, float(np.max(np.abs(fwd - _torch_causal(u, w, b, silu)))))
            rev = mod.conv1d(u, w, b, reverse=True, activation=act)
            ref = _torch_causal(u[:, ::-1].copy(), w, b, silu)[:, ::-1]
            worst = max(worst, float(np.max(np.abs(rev - ref))))
    return worst


def pin_impulse(mod):
    """A unit impulse at token s of channel c gives bias + w[c, W-1-j] at
    token s+j (forward) or s-j (reverse), j < W, and bias elsewhere."""
    L, ch, W, s = 12, 3, 4, 5
    w = np.arange(1.0, ch * W + 1).reshape(ch, W)
    b = np.array([0.25, -0.5, 2.0])
    worst = 0.0
    for c in range(ch):
        u = np.zeros((1, L, ch))
        u[0, s, c] = 1.0
        for reverse in (False, True):
            out = mod.conv1d(u, w, b, reverse=reverse, activation="none")
            exp = np.tile(b, (L, 1))
            for j in range(W):
                t = s - j if reverse else s + j
                exp[t, c] += w[c, W - 1 - j]
            worst = max(worst, float(np.max(np.abs(out[0] - exp))))
    return worst


def pin_silu(mod):
    """SiLU at points with known values and against scipy's logistic."""
    from scipy.special import expit
    v = np.array([0.0, 1.0, -1.0, 3.5, -7.25, 30.0, -30.0, 800.0, -800.0])
    got = mod.silu(v)
    ref = v * expit(v)
    worst = float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)))
    # silu(0) = 0, silu(ln 3) = ln(3) * 3/4 exactly in real arithmetic
    worst = max(worst, abs(float(mod.silu(np.array([0.0]))[0])))
    worst = max(worst, abs(float(mod.silu(np.array([np.log(3.0)]))[0]) - 0.75 * np.log(3.0)))
    return worst


def pin_context(mod, seed=31):
    """Splitting a row and carrying the forward context reproduces the whole
    row, and the final context is the row's last W-1 inputs (reaching into
    the initial context when the row is shorter than W-1)."""
    rng = _rng(seed)
    worst = 0.0
    W, ch = 4, 16
    u, w, b = _draw(rng, 2, 40, ch, W)
    whole, fin_whole = mod.conv1d(u, w, b, want_final=True)
    worst = max(worst, float(np.max(np.abs(fin_whole - u[:, -(W - 1):]))))
    for s in (1, 2, 3, 17):
        _, ctx = mod.conv1d(u[:, :s], w, b, want_final=True)
        tail, fin = mod.conv1d(u[:, s:], w, b, init_ctx=ctx, want_final=True)
        worst = max(worst, float(np.max(np.abs(tail - whole[:, s:]))))
        worst = max(worst, float(np.max(np.abs(fin - fin_whole))))
    ctx = rng.standard_normal((2, W - 1, ch))
    _, fin = mod.conv1d(u[:, :1], w, b, init_ctx=ctx, want_final=True)
    exp = np.concatenate([ctx[:, 1:], u[:, :1]], axis=1)
    worst = max(worst, float(np.max(np.abs(fin - exp))))
    return worst


def pin_packed(mod, seed=32):
    """Packed sequences (empty and shorter-than-W ones included) == each
    sequence filtered alone, in both directions."""
    rng = _rng(seed)
    lens = [5, 0, 1, 2, 9, 3, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    u, w, b = _draw(rng, 1, int(cu[-1]), 8, 4)
    worst = 0.0
    for reverse in (False, True):
        packed = mod.conv1d(u, w, b, reverse=reverse, cu_seqlens=cu)
        for j, n in enumerate(lens):
            if n == 0:
                continue
            a = int(cu[j])
            alone = mod.conv1d(u[:, a:a + n], w, b, reverse=reverse)
            worst = max(worst, float(np.max(np.abs(packed[:, a:a + n] - alone))))
    return worst


def pin_split(mod, seed=33):
    """x | B | C channel split: x first (head-major), then B, then C."""
    rng = _rng(seed)
    H, P, G, N = 3, 4, 2, 5
    out = rng.standard_normal((2, 6, H * P + 2 * G * N))
    x, B, C = mod.split_xbc(out, H, P, G, N)
    worst = float(np.max(np.abs(x[:, :, 2, 1] - out[:, :, 2 * P + 1])))
    worst = max(worst, float(np.max(np.abs(B[:, :, 1, 3] - out[:, :, H * P + N + 3]))))
    worst = max(worst, float(np.max(np.abs(C[:, :, 0, 4] - out[:, :, H * P + G * N + 4]))))
    return worst


CONV_PINS = {
    "conv_torch": (pin_torch, 1e-12),
    "conv_impulse": (pin_impulse, 0.0),
    "conv_silu": (pin_silu, 1e-14),
    "conv_context": (pin_context, 0.0),
    "conv_packed": (pin_packed, 0.0),
    "conv_split": (pin_split, 0.0),
}
