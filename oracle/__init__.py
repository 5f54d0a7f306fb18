"""Oracle for the bidirectional Mamba-2 SSD mixer (fp64, CPU).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``; never by the product package, which
shares no code with it.

Two independent formulations live here:

* ``bissd`` / ``block_step`` -- the sequential fp64 recurrence in
  ``ssd_oracle.c`` (one token at a time, see that file's header for the
  equations and the passages they follow);
* ``bissd_bwd`` -- its gradients (the training backward), by the adjoint
  recurrence in the same file;
* ``oracle.brute`` -- the quadratic "masked C.B^T" form of the same operator
  in numpy, used to pin the recurrence on tiny inputs.

Every input is upcast losslessly to float64 before the call, so the oracle
reads exactly the values the GPU reads (bf16 and fp32 embed in fp64).

Parity: pinned (see tests/test_oracle_pins.py). No function here is
unpinned.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def bind(path):
    """Load an oracle shared library built from ssd_oracle.c."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_bissd_f64.argtypes = (
        [ctypes.c_int] * 6 + [dp] * 12 + [ip, ctypes.c_int, dp, dp, dp])
    lib.oracle_bissd_f64.restype = ctypes.c_int
    pp = ctypes.c_void_p * 6
    lib.oracle_bissd_bwd_f64.argtypes = (
        [ctypes.c_int] * 6 + [dp] * 12 + [ip, ctypes.c_int, dp, pp, pp])
    lib.oracle_bissd_bwd_f64.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    return lib


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = bind(_build.LIB)
    return _LIB


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor: exact upcast on the host
        a = a.detach().to("cpu")
        a = a.double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, typ=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(typ))


def num_threads() -> int:
    return int(_lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _lib().oracle_set_num_threads(int(n))


def bissd(fwd, bwd=None, cu_seqlens=None, init_state=None,
          want_final_state=False, lib=None):
    """Bidirectional SSD, fp64 recurrence.

    ``fwd`` / ``bwd`` are dicts with keys x [b,L,H,P], dt [b,L,H], A [H],
    B [b,L,G,N], C [b,L,G,N], D [H] or None (torch tensors or arrays of any
    float dtype). ``bwd=None`` runs the forward direction only.
    ``cu_seqlens`` (ints, nseq+1) packs sequences into the single row.
    Returns y (float64 [b,L,H,P]) and, if asked, the forward final state
    float64 [nseq or b, H, P, N].
    """
    f = {k: _f64(v) for k, v in fwd.items()}
    b = {k: _f64(v) for k, v in bwd.items()} if bwd is not None else None
    batch, L, H, P = f["x"].shape
    G, N = f["B"].shape[2], f["B"].shape[3]
    cu = None
    nseq = batch
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        nseq = len(cu) - 1
    y = np.empty((batch, L, H, P), dtype=np.float64)
    fs = np.empty((nseq, H, P, N), dtype=np.float64) if want_final_state else None
    ist = _f64(init_state)
    if ist is not None:
        assert ist.shape == (nseq, H, P, N), ist.shape
    none = None
    rc = (lib or _lib()).oracle_bissd_f64(
        batch, L, H, P, N, G,
        _ptr(f["x"]), _ptr(f["dt"]), _ptr(f["A"]), _ptr(f["B"]), _ptr(f["C"]),
        _ptr(f.get("D")),
        _ptr(b["x"]) if b else none, _ptr(b["dt"]) if b else none,
        _ptr(b["A"]) if b else none, _ptr(b["B"]) if b else none,
        _ptr(b["C"]) if b else none, _ptr(b.get("D")) if b else none,
        _ptr(cu, ctypes.c_int32), nseq, _ptr(ist), _ptr(fs), _ptr(y))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return (y, fs) if want_final_state else y


def block_step(state, fwd, bwd, commit=False, lib=None):
    """Cached block-diffusion step for nseq independent sequences.

    ``state`` [nseq, H, P, N] is the carried forward SSM state of each
    sequence's finalized prefix; ``fwd``/``bwd`` hold the active block
    ([nseq, Lb, ...]). The forward scan resumes from ``state``; the reverse
    scan is restricted to the block and starts from zero at its end.
    Returns y [nseq, Lb, H, P] and the new state (the forward state at the
    block end) if ``commit`` else the unchanged state.
    """
    y, fs = bissd(fwd, bwd, init_state=state, want_final_state=True, lib=lib)
    new_state = fs if commit else _f64(state).copy()
    return y, new_state


GRAD_KEYS = ("x", "dt", "A", "B", "C", "D")


def bissd_bwd(fwd, bwd, dy, cu_seqlens=None, lib=None):
    """Gradients of ``bissd(fwd, bwd)`` with respect to every input, given
    the output gradient dy [b, L, H, P]. Returns (gfwd, gbwd): dicts with
    keys x, dt, A, B, C, D (float64, shaped like the inputs; D's gradient
    is returned even when D is None). gbwd is None when bwd is None."""
    f = {k: _f64(v) for k, v in fwd.items()}
    b = {k: _f64(v) for k, v in bwd.items()} if bwd is not None else None
    g = _f64(dy)
    batch, L, H, P = f["x"].shape
    G, N = f["B"].shape[2], f["B"].shape[3]
    cu, nseq = None, batch
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        nseq = len(cu) - 1

    def grads():
        return {"x": np.empty((batch, L, H, P)), "dt": np.empty((batch, L, H)),
                "A": np.empty(H), "B": np.empty((batch, L, G, N)),
                "C": np.empty((batch, L, G, N)), "D": np.empty(H)}

    gf = grads()
    gb = grads() if b is not None else None

    def ptrs(gd):
        arr = (ctypes.c_void_p * 6)()
        if gd is not None:
            for i, k in enumerate(GRAD_KEYS):
                arr[i] = gd[k].ctypes.data
        return arr

    none = None
    rc = (lib or _lib()).oracle_bissd_bwd_f64(
        batch, L, H, P, N, G,
        _ptr(f["x"]), _ptr(f["dt"]), _ptr(f["A"]), _ptr(f["B"]), _ptr(f["C"]),
        _ptr(f.get("D")),
        _ptr(b["x"]) if b else none, _ptr(b["dt"]) if b else none,
        _ptr(b["A"]) if b else none, _ptr(b["B"]) if b else none,
        _ptr(b["C"]) if b else none, _ptr(b.get("D")) if b else none,
        _ptr(cu, ctypes.c_int32), nseq, _ptr(g), ptrs(gf), ptrs(gb))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return gf, gb
