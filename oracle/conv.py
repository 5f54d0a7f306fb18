"""Oracle for the short depthwise convolution in front of the scan (fp64, CPU).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the smoke check; never
by the product package, which shares no code with it.

What the pages fix: each direction of the bidirectional block is a whole
Mamba block with its own parameters, and the reverse one runs on the flipped
sequence (DiffuMamba blog, "network architecture": ``backward_mamba`` applied
to ``torch.flip(x)``, result flipped back); the configuration gives the
convolution width ``d_conv = 4`` (same section, ``DiffuMambaConfig``). The
block cache carries what the finalized prefix leaves behind and the reverse
pass sees only the active block ("Fixed state, long reach: constant-size
caches in large-scale block diffusion", Sec. 1).

What the pages leave open, and the reading taken here (Mamba-2's mixer, the
one the pages name): the channels that feed the scan -- x, then B, then C of
one direction, ``nheads*headdim + 2*ngroups*d_state`` of them per token --
each go through their own length-``W`` causal filter with a bias, followed
by SiLU, ``v / (1 + exp(-v))``:

    forward : u_t = bias + sum_{k=0}^{W-1} w[k] * in_{t-(W-1)+k}
    reverse : the same filter on the flipped sequence, i.e.
              u_t = bias + sum_{k=0}^{W-1} w[k] * in_{t+(W-1)-k}

Inputs outside the token's own sequence are zero (a packed sequence never
sees its neighbours), except that the forward filter of a row may start from
``init_ctx``, the W-1 forward inputs that preceded token 0 (oldest first);
``final_ctx`` is the W-1 forward inputs that end the row, in the same order:
the conv part of the block cache. The reverse filter of a block sees zeros
after the block's last token.

Everything is written out per tap with numpy slices; no library convolution
is used, so ``torch.nn.functional.conv1d`` can pin it independently.

Parity: pinned (tests/test_oracle_pins.py, conv section).
"""
import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def silu(v):
    """v * sigmoid(v), written as v / (1 + exp(-v)); exp overflow gives -0."""
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def _filter_row(u, w, bias, reverse, ctx):
    """One sequence: u [T, ch] inputs, w [ch, W], bias [ch] or None, ctx
    [W-1, ch] forward history (zeros if None). Returns the pre-activation
    [T, ch]."""
    T, ch = u.shape
    W = w.shape[1]
    if reverse:
        padded = np.concatenate([u, np.zeros((W - 1, ch))], axis=0)
    else:
        head = np.zeros((W - 1, ch)) if ctx is None else ctx
        padded = np.concatenate([head, u], axis=0)
    out = np.zeros((T, ch)) if bias is None else np.tile(bias, (T, 1))
    for k in range(W):
        if reverse:
            # tap k multiplies the input W-1-k tokens AFTER t
            src = padded[W - 1 - k:W - 1 - k + T]
        else:
            # tap k multiplies the input W-1-k tokens BEFORE t
            src = padded[k:k + T]
        out = out + w[:, k] * src
    return out


def conv1d(xbc, weight, bias=None, reverse=False, cu_seqlens=None,
           init_ctx=None, activation="silu", want_final=False):
    """Depthwise short convolution of one direction.

    xbc [batch, L, ch]; weight [ch, W]; bias [ch] or None; init_ctx
    [batch, W-1, ch] or None (forward only, not with cu_seqlens).
    Returns the fp64 output [batch, L, ch] and, with ``want_final``, the
    forward context after each row [batch, W-1, ch].
    """
    u = _f64(xbc)
    w = _f64(weight)
    b = _f64(bias)
    ctx = _f64(init_ctx)
    batch, L, ch = u.shape
    W = w.shape[1]
    assert w.shape == (ch, W) and W >= 1
    if reverse or cu_seqlens is not None:
        assert ctx is None, "init_ctx is a forward, unpacked-row input"
    out = np.empty_like(u)
    if cu_seqlens is not None:
        assert batch == 1
        cu = [int(v) for v in cu_seqlens]
        for j in range(len(cu) - 1):
            a, e = cu[j], cu[j + 1]
            if e > a:
                out[0, a:e] = _filter_row(u[0, a:e], w, b, reverse, None)
    else:
        for r in range(batch):
            out[r] = _filter_row(u[r], w, b, reverse, None if ctx is None else ctx[r])
    if activation == "silu":
        out = silu(out)
    else:
        assert activation in (None, "none")
    if not want_final:
        return out
    assert cu_seqlens is None
    final = np.empty((batch, W - 1, ch))
    for r in range(batch):
        hist = np.zeros((W - 1, ch)) if ctx is None else ctx[r]
        seq = np.concatenate([hist, u[r]], axis=0)
        final[r] = seq[seq.shape[0] - (W - 1):]
    return out, final


def split_xbc(out, nheads, headdim, ngroups, d_state):
    """[batch, L, ch] -> x [batch, L, H, P], B, C [batch, L, G, N]."""
    batch, L, ch = out.shape
    hp, gn = nheads * headdim, ngroups * d_state
    assert ch == hp + 2 * gn
    return (out[..., :hp].reshape(batch, L, nheads, headdim),
            out[..., hp:hp + gn].reshape(batch, L, ngroups, d_state),
            out[..., hp + gn:].reshape(batch, L, ngroups, d_state))
