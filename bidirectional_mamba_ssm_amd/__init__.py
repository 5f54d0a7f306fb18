"""Bidirectional Mamba-2 SSD mixer on MI355X: thin Python binding.

Every step of the computation runs in libbimamba's HIP kernels; this module
only marshals torch tensors (device memory and the current stream) into the
C ABI declared in include/bimamba.h. It has no compute path of its own and
raises if the library is not built.
"""
import ctypes

import torch

from . import _abi
from ._abi import BimambaError, LibraryMissing  # noqa: F401

DTYPES = {torch.float32: _abi.F32, torch.bfloat16: _abi.BF16}


def lib():
    return _abi.load()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dir(d, dtype):
    for k in ("x", "dt", "B", "C"):
        t = d[k]
        if t.dtype != dtype:
            raise TypeError(f"{k} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{k} must be contiguous")
    for k in ("A", "D"):
        t = d.get(k)
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise TypeError(f"{k} must be a contiguous float32 tensor")
    return _abi.Dir(d["x"].data_ptr(), d["dt"].data_ptr(), d["A"].data_ptr(),
                    d["B"].data_ptr(), d["C"].data_ptr(),
                    d["D"].data_ptr() if d.get("D") is not None else None)


def make_shape(x, B, chunk, seqlen=None):
    """Shape of a problem whose x is [batch, L, H, P] and B [batch, L, G, N]."""
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if x.dtype not in DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    return _abi.Shape(batch, L if seqlen is None else seqlen, H, P, N, G, chunk,
                      DTYPES[x.dtype], 0)


def workspace_size(shape, nseq=0):
    n = ctypes.c_size_t(0)
    _abi.check(lib().bimamba_ssd_workspace_size(ctypes.byref(shape), nseq, ctypes.byref(n)))
    return n.value


def ssd_fwd(fwd, bwd=None, chunk=256, cu_seqlens=None, init_state=None,
            final_state=None, y=None, workspace=None, stream=None):
    """Bidirectional SSD (see include/bimamba.h, bimamba_ssd_fwd).

    fwd/bwd: dicts of device tensors x [b,L,H,P], dt [b,L,H], A [H] f32,
    B/C [b,L,G,N], D [H] f32 or None. cu_seqlens: host list/tensor of
    nseq+1 offsets. Returns y (float32 [b,L,H,P]).
    """
    x = fwd["x"]
    shape = make_shape(x, fwd["B"], chunk)
    dtype = x.dtype
    fd = _dir(fwd, dtype)
    bd = _dir(bwd, dtype) if bwd is not None else None
    cu_arr, nseq = None, 0
    if cu_seqlens is not None:
        vals = [int(v) for v in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        nseq = len(vals) - 1
        cu_arr = (ctypes.c_int32 * len(vals))(*vals)
    if y is None:
        y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    need = workspace_size(shape, nseq)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _abi.check(lib().bimamba_ssd_fwd(
        ctypes.byref(shape), ctypes.byref(fd), ctypes.byref(bd) if bd is not None else None,
        cu_arr, nseq, _ptr(init_state), _ptr(final_state), _ptr(y),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return y


class State:
    """Library-owned forward-state cache: float [nslots, H, P, N] on the GPU."""

    def __init__(self, nslots, nheads, headdim, d_state):
        self._h = ctypes.c_void_p()
        _abi.check(lib().bimamba_state_alloc(ctypes.byref(self._h), nslots, nheads,
                                             headdim, d_state))
        self.shape = (nslots, nheads, headdim, d_state)

    def data_ptr(self):
        return lib().bimamba_state_data(self._h)

    def tensor(self):
        """A zero-copy torch view of the cache (valid while this object lives)."""
        ptr = self.data_ptr()
        shape = self.shape

        class _View:
            __cuda_array_interface__ = {
                "shape": shape, "typestr": "<f4", "data": (ptr, False),
                "version": 2, "strides": None}
        return torch.as_tensor(_View(), device="cuda")

    def reset(self, slots=None, stream=None):
        arr, n = None, 0
        if slots is not None:
            slots = [int(s) for s in slots]
            n = len(slots)
            arr = (ctypes.c_int32 * max(n, 1))(*slots)
        _abi.check(lib().bimamba_state_reset(self._h, arr, n, _stream(stream)))

    def free(self):
        if self._h:
            _abi.check(lib().bimamba_state_free(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h


def block_step(state, fwd, bwd, commit=False, chunk=64, y=None, stream=None):
    """One cached block-diffusion step (bimamba_block_step)."""
    x = fwd["x"]
    shape = make_shape(x, fwd["B"], chunk)
    fd = _dir(fwd, x.dtype)
    bd = _dir(bwd, x.dtype)
    if y is None:
        y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _abi.check(lib().bimamba_block_step(state.handle, ctypes.byref(shape), ctypes.byref(fd),
                                        ctypes.byref(bd), int(bool(commit)), _ptr(y),
                                        _stream(stream)))
    return y


def seq_index(cu_seqlens, device="cuda", stream=None):
    """Per-token packed-sequence index built on the GPU (int32 [total])."""
    vals = [int(v) for v in cu_seqlens]
    total = vals[-1]
    out = torch.empty(max(total, 1), dtype=torch.int32, device=device)
    arr = (ctypes.c_int32 * len(vals))(*vals)
    _abi.check(lib().bimamba_seq_index(arr, len(vals) - 1, total, _ptr(out), _stream(stream)))
    return out[:total]


class profile:
    """Context manager: per-kernel launch counts and summed device time (ms)
    of every library kernel launched from this thread inside the block,
    measured with HIP events on each kernel's stream.

        with bm.profile() as prof:
            bm.ssd_fwd(...)
        prof.kernels  # {name: (launches, total_ms)}
    """

    def __enter__(self):
        _abi.check(lib().bimamba_profile_begin())
        self.kernels = {}
        return self

    def __exit__(self, *exc):
        cap, nl = 64, 64
        names = ctypes.create_string_buffer(cap * nl)
        counts = (ctypes.c_int * cap)()
        ms = (ctypes.c_double * cap)()
        n = lib().bimamba_profile_end(names, nl, counts, ms, cap)
        if n < 0:
            _abi.check(n)
        raw = names.raw
        for i in range(min(n, cap)):
            name = raw[i * nl:(i + 1) * nl].split(b"\0", 1)[0].decode()
            self.kernels[name] = (counts[i], ms[i])
        return False
