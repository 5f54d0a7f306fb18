"""Quadratic ("masked C.B^T") form of the bidirectional SSD, in numpy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Unrolling the recurrence of ssd_oracle.c gives, per head h with group g,

  forward : y_t = sum_{s<=t} exp(sum_{k=s+1..t} a_k) (C_t . B_s) dt_s x_s + D x_t
  backward: y_t = sum_{s>=t} exp(sum_{k=t..s-1} a_k) (C_t . B_s) dt_s x_s + D x_t

with a_k = dt_k * A_h. This file evaluates those sums literally (explicit
segment sums, no cumsum differences), so it shares no arithmetic with the
recurrence and is only meant for tiny L. It is the whole-sequence special
case of the SSD block decomposition of Mamba-2 (the mixer the DiffuMamba
pages name).
"""
import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def direction(x, dt, A, B, C, D=None, reverse=False):
    """One direction for one row: x [L,H,P], dt [L,H], A [H], B,C [L,G,N]."""
    x, dt, A, B, C, D = map(_f64, (x, dt, A, B, C, D))
    L, H, P = x.shape
    G = B.shape[1]
    y = np.zeros((L, H, P))
    for h in range(H):
        g = h // (H // G)
        a = dt[:, h] * A[h]
        W = np.zeros((L, L))
        for t in range(L):
            for s in range(L):
                if not reverse and s <= t:
                    lam = np.exp(np.sum(a[s + 1:t + 1]))
                elif reverse and s >= t:
                    lam = np.exp(np.sum(a[t:s]))
                else:
                    continue
                W[t, s] = lam * np.dot(C[t, g], B[s, g]) * dt[s, h]
        y[:, h, :] = W @ x[:, h, :]
        if D is not None:
            y[:, h, :] += D[h] * x[:, h, :]
    return y


def bissd(fwd, bwd=None):
    """Sum of both directions for [b, L, ...] inputs (dicts as in oracle)."""
    batch = fwd["x"].shape[0]
    out = []
    for r in range(batch):
        yr = direction(fwd["x"][r], fwd["dt"][r], fwd["A"], fwd["B"][r],
                       fwd["C"][r], fwd.get("D"), reverse=False)
        if bwd is not None:
            yr = yr + direction(bwd["x"][r], bwd["dt"][r], bwd["A"],
                                bwd["B"][r], bwd["C"][r], bwd.get("D"),
                                reverse=True)
        out.append(yr)
    return np.stack(out)
