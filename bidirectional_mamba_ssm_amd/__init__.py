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


def _check(t, name, shape, dtype, device):
    """The library sees plain pointers: every tensor's device, dtype, shape and
    layout is checked here, before anything is launched."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _cuda_device(x):
    if x.device.type != "cuda":
        raise ValueError(f"tensors must be on a CUDA device, not {x.device}")
    return x.device


def _dims(d):
    x, B = d["x"], d["B"]
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [batch, L, H, P] and B [batch, L, G, N]")
    batch, L, H, P = x.shape
    return batch, L, H, P, B.shape[2], B.shape[3]


def _dir(d, dtype, dims=None, device=None, name="fwd"):
    batch, L, H, P, G, N = dims if dims is not None else _dims(d)
    device = device if device is not None else d["x"].device
    _check(d["x"], f"{name}.x", (batch, L, H, P), dtype, device)
    _check(d["dt"], f"{name}.dt", (batch, L, H), dtype, device)
    _check(d["B"], f"{name}.B", (batch, L, G, N), dtype, device)
    _check(d["C"], f"{name}.C", (batch, L, G, N), dtype, device)
    _check(d["A"], f"{name}.A", (H,), torch.float32, device)
    if d.get("D") is not None:
        _check(d["D"], f"{name}.D", (H,), torch.float32, device)
    if d.get("dt_bias") is not None:
        _check(d["dt_bias"], f"{name}.dt_bias", (H,), torch.float32, device)
    return _abi.Dir(d["x"].data_ptr(), d["dt"].data_ptr(), d["A"].data_ptr(),
                    d["B"].data_ptr(), d["C"].data_ptr(),
                    d["D"].data_ptr() if d.get("D") is not None else None,
                    d["dt_bias"].data_ptr() if d.get("dt_bias") is not None else None)


def make_shape(x, B, chunk, seqlen=None, dt_softplus=False):
    """Shape of a problem whose x is [batch, L, H, P] and B [batch, L, G, N]."""
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if x.dtype not in DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    return _abi.Shape(batch, L if seqlen is None else seqlen, H, P, N, G, chunk,
                      DTYPES[x.dtype], _abi.DT_SOFTPLUS if dt_softplus else 0)


def workspace_size(shape, nseq=0):
    n = ctypes.c_size_t(0)
    _abi.check(lib().bimamba_ssd_workspace_size(ctypes.byref(shape), nseq, ctypes.byref(n)))
    return n.value


def ssd_fwd(fwd, bwd=None, chunk=256, cu_seqlens=None, init_state=None,
            final_state=None, y=None, workspace=None, stream=None, dt_softplus=False):
    """Bidirectional SSD (see include/bimamba.h, bimamba_ssd_fwd).

    fwd/bwd: dicts of device tensors x [b,L,H,P], dt [b,L,H], A [H] f32,
    B/C [b,L,G,N], D [H] f32 or None, and (with dt_softplus, where dt is the
    pre-activation) dt_bias [H] f32 or None. cu_seqlens: host list/tensor
    of nseq+1 offsets. Returns y (float32 [b,L,H,P]).
    """
    x = fwd["x"]
    dims = _dims(fwd)
    batch, L, H, P, G, N = dims
    shape = make_shape(x, fwd["B"], chunk, dt_softplus=dt_softplus)
    dtype = x.dtype
    dev = _cuda_device(x)
    fd = _dir(fwd, dtype, dims, dev, "fwd")
    bd = _dir(bwd, dtype, dims, dev, "bwd") if bwd is not None else None
    cu_arr, nseq = None, 0
    if cu_seqlens is not None:
        vals = [int(v) for v in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        nseq = len(vals) - 1
        cu_arr = (ctypes.c_int32 * len(vals))(*vals)
    units = nseq if cu_seqlens is not None else batch
    for t, name in ((init_state, "init_state"), (final_state, "final_state")):
        if t is not None:
            _check(t, name, (units, H, P, N), torch.float32, dev)
    if y is None:
        y = torch.empty(x.shape, dtype=torch.float32, device=dev)
    _check(y, "y", (batch, L, H, P), torch.float32, dev)
    need = workspace_size(shape, nseq)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _abi.check(lib().bimamba_ssd_fwd(
        ctypes.byref(shape), ctypes.byref(fd), ctypes.byref(bd) if bd is not None else None,
        cu_arr, nseq, _ptr(init_state), _ptr(final_state), _ptr(y),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def bwd_workspace_size(shape, has_bwd=True):
    n = ctypes.c_size_t(0)
    _abi.check(lib().bimamba_ssd_bwd_workspace_size(ctypes.byref(shape), int(bool(has_bwd)),
                                                     ctypes.byref(n)))
    return n.value


def _grads(g, dims, dev, name):
    batch, L, H, P, G, N = dims
    shapes = {"x": (batch, L, H, P), "dt": (batch, L, H), "A": (H,),
              "B": (batch, L, G, N), "C": (batch, L, G, N), "D": (H,)}
    if g is None:
        g = {k: torch.empty(v, dtype=torch.float32, device=dev) for k, v in shapes.items()}
    for k, v in shapes.items():
        if k == "D" and g.get("D") is None:
            continue
        _check(g[k], f"{name}_grad.{k}", v, torch.float32, dev)
    return g, _abi.Grad(g["x"].data_ptr(), g["dt"].data_ptr(), g["A"].data_ptr(),
                        g["B"].data_ptr(), g["C"].data_ptr(),
                        g["D"].data_ptr() if g.get("D") is not None else None)


def ssd_bwd(fwd, bwd, dy, grads=None, workspace=None, stream=None):
    """Training backward of ssd_fwd (bimamba_ssd_bwd): gradients of every
    input of both streams given dy (float32 [b,L,H,P]). Returns (gfwd, gbwd),
    dicts of float32 tensors keyed x, dt, A, B, C, D (gbwd None without bwd).
    grads: optional (gfwd, gbwd) dicts to write into."""
    x = fwd["x"]
    dims = _dims(fwd)
    batch, L, H, P, G, N = dims
    shape = make_shape(x, fwd["B"], 64)
    dev = _cuda_device(x)
    fd = _dir(fwd, x.dtype, dims, dev, "fwd")
    bd = _dir(bwd, x.dtype, dims, dev, "bwd") if bwd is not None else None
    _check(dy, "dy", (batch, L, H, P), torch.float32, dev)
    gl = list(grads) if grads is not None else [None, None]
    gf, gfs = _grads(gl[0], dims, dev, "fwd")
    gb, gbs = _grads(gl[1], dims, dev, "bwd") if bwd is not None else (None, None)
    need = bwd_workspace_size(shape, bwd is not None)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _abi.check(lib().bimamba_ssd_bwd(
        ctypes.byref(shape), ctypes.byref(fd), ctypes.byref(bd) if bd is not None else None,
        _ptr(dy), ctypes.byref(gfs), ctypes.byref(gbs) if gbs is not None else None,
        _ptr(workspace), ws_bytes, _stream(stream)))
    return gf, gb


def ssd_fwd_noalloc(fwd, bwd, y, chunk=256, cu_seqlens=None, init_state=None,
                    final_state=None, stream=None, dt_softplus=False):
    """bimamba_ssd_fwd_noalloc: ssd_fwd with the library's static device
    buffer as its workspace (the call allocates nothing; y is the caller's
    float32 [b,L,H,P]). Returns y."""
    x = fwd["x"]
    dims = _dims(fwd)
    batch, L, H, P, G, N = dims
    shape = make_shape(x, fwd["B"], chunk, dt_softplus=dt_softplus)
    dev = _cuda_device(x)
    fd = _dir(fwd, x.dtype, dims, dev, "fwd")
    bd = _dir(bwd, x.dtype, dims, dev, "bwd") if bwd is not None else None
    cu_arr, nseq = None, 0
    if cu_seqlens is not None:
        vals = [int(v) for v in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        nseq = len(vals) - 1
        cu_arr = (ctypes.c_int32 * len(vals))(*vals)
    units = nseq if cu_seqlens is not None else batch
    for t, name in ((init_state, "init_state"), (final_state, "final_state")):
        if t is not None:
            _check(t, name, (units, H, P, N), torch.float32, dev)
    _check(y, "y", (batch, L, H, P), torch.float32, dev)
    _abi.check(lib().bimamba_ssd_fwd_noalloc(
        ctypes.byref(shape), ctypes.byref(fd), ctypes.byref(bd) if bd is not None else None,
        cu_arr, nseq, _ptr(init_state), _ptr(final_state), _ptr(y), _stream(stream)))
    return y


def ssd_fwd_streams(fwd, bwd, chunk=256, cu_seqlens=None, init_state=None,
                    final_state=None, y_fwd=None, y_bwd=None, workspace=None, stream=None):
    """bimamba_ssd_fwd_streams: the two streams' outputs kept apart.
    Returns (y_fwd, y_bwd), float32 [b,L,H,P] each."""
    x = fwd["x"]
    dims = _dims(fwd)
    batch, L, H, P, G, N = dims
    shape = make_shape(x, fwd["B"], chunk)
    dev = _cuda_device(x)
    fd = _dir(fwd, x.dtype, dims, dev, "fwd")
    bd = _dir(bwd, x.dtype, dims, dev, "bwd")
    cu_arr, nseq = None, 0
    if cu_seqlens is not None:
        vals = [int(v) for v in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        nseq = len(vals) - 1
        cu_arr = (ctypes.c_int32 * len(vals))(*vals)
    units = nseq if cu_seqlens is not None else batch
    for t, name in ((init_state, "init_state"), (final_state, "final_state")):
        if t is not None:
            _check(t, name, (units, H, P, N), torch.float32, dev)
    outs = []
    for t, name in ((y_fwd, "y_fwd"), (y_bwd, "y_bwd")):
        if t is None:
            t = torch.empty(x.shape, dtype=torch.float32, device=dev)
        _check(t, name, (batch, L, H, P), torch.float32, dev)
        outs.append(t)
    need = workspace_size(shape, nseq)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _abi.check(lib().bimamba_ssd_fwd_streams(
        ctypes.byref(shape), ctypes.byref(fd), ctypes.byref(bd), cu_arr, nseq,
        _ptr(init_state), _ptr(final_state), _ptr(outs[0]), _ptr(outs[1]),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return outs[0], outs[1]


def merge_linear(y_fwd, y_bwd, weight, bias=None, out=None, stream=None):
    """bimamba_merge_linear: W [y_fwd ; y_bwd] + bias per token. y_fwd,
    y_bwd float32 [..., cin]; weight bf16 [cout, 2 cin]; bias float32 [cout]
    or None. Returns float32 [..., cout]."""
    dev = _cuda_device(y_fwd)
    cin = y_fwd.shape[-1]
    rows = y_fwd.numel() // cin if cin else 0
    cout = weight.shape[0]
    _check(y_fwd, "y_fwd", tuple(y_fwd.shape), torch.float32, dev)
    _check(y_bwd, "y_bwd", tuple(y_fwd.shape), torch.float32, dev)
    _check(weight, "weight", (cout, 2 * cin), torch.bfloat16, dev)
    if bias is not None:
        _check(bias, "bias", (cout,), torch.float32, dev)
    oshape = tuple(y_fwd.shape[:-1]) + (cout,)
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=dev)
    _check(out, "out", oshape, torch.float32, dev)
    _abi.check(lib().bimamba_merge_linear(rows, cin, cout, _ptr(y_fwd), _ptr(y_bwd), _ptr(weight),
                                          _ptr(bias), _ptr(out), _stream(stream)))
    return out


class State:
    """Library-owned forward-state cache: float [nslots, H, P, N] on the GPU;
    with conv=(ngroups, width, dtype) it also carries the short convolution's
    context, [nslots, width-1, channels] of that dtype (bimamba_state_alloc_conv)."""

    def __init__(self, nslots, nheads, headdim, d_state, conv=None):
        self._h = ctypes.c_void_p()
        self.conv = None
        if conv is None:
            _abi.check(lib().bimamba_state_alloc(ctypes.byref(self._h), nslots, nheads,
                                                 headdim, d_state))
        else:
            ngroups, width, dtype = conv
            if dtype not in DTYPES:
                raise TypeError(f"unsupported dtype {dtype}")
            _abi.check(lib().bimamba_state_alloc_conv(ctypes.byref(self._h), nslots, nheads, headdim,
                                                      d_state, ngroups, width, DTYPES[dtype]))
            ch = conv_channels(nheads, headdim, ngroups, d_state)
            self.conv = (ngroups, width, dtype, ch)
        self.shape = (nslots, nheads, headdim, d_state)

    def ctx_tensor(self):
        """A zero-copy torch view of the convolution context (valid while
        this object lives)."""
        if self.conv is None:
            raise ValueError("this state carries no convolution context")
        ptr = lib().bimamba_state_conv_ctx(self._h)
        _, width, dtype, ch = self.conv
        shape = (self.shape[0], width - 1, ch)
        typestr = "<f4" if dtype == torch.float32 else "<u2"

        class _View:
            __cuda_array_interface__ = {
                "shape": shape, "typestr": typestr, "data": (ptr, False),
                "version": 2, "strides": None}
        t = torch.as_tensor(_View(), device="cuda")
        return t.view(torch.bfloat16) if dtype == torch.bfloat16 else t

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


def block_step(state, fwd, bwd, commit=False, chunk=64, y=None, stream=None, dt_softplus=False):
    """One cached block-diffusion step (bimamba_block_step)."""
    x = fwd["x"]
    dims = _dims(fwd)
    shape = make_shape(x, fwd["B"], chunk, dt_softplus=dt_softplus)
    dev = _cuda_device(x)
    fd = _dir(fwd, x.dtype, dims, dev, "fwd")
    bd = _dir(bwd, x.dtype, dims, dev, "bwd")
    if y is None:
        y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _check(y, "y", tuple(x.shape), torch.float32, x.device)
    _abi.check(lib().bimamba_block_step(state.handle, ctypes.byref(shape), ctypes.byref(fd),
                                        ctypes.byref(bd), int(bool(commit)), _ptr(y),
                                        _stream(stream)))
    return y


def block_step_conv(state, fwd, bwd, conv_fwd, conv_bwd, commit=False, chunk=64, y=None,
                    activation="silu", conv_out=None, stream=None, dt_softplus=False):
    """One cached block step from the block's raw convolution inputs
    (bimamba_block_step_conv) for a State made with conv=...: the short
    convolution of both directions (the forward one from the state's
    context), then the block step; with commit the SSM state and the
    context both move past the block.

    conv_fwd/conv_bwd: dicts xbc [b, L, ch], weight [ch, W] f32, bias [ch] f32
    or None. fwd/bwd: dicts dt, A, D (and optionally dt_bias) of each
    direction; x, B, C are the convolution's outputs (allocated here, or
    given in conv_out as for conv1d). Returns y."""
    if state.conv is None:
        raise ValueError("the state carries no convolution context")
    ngroups, W, cdtype, ch = state.conv
    xbc = conv_fwd["xbc"]
    dev = _cuda_device(xbc)
    if xbc.dim() != 3:
        raise ValueError("xbc must be [batch, L, channels]")
    batch, L, chx = xbc.shape
    _, H, P, N = state.shape
    if chx != ch or conv_fwd["weight"].shape != (ch, W) or xbc.dtype != cdtype:
        raise ValueError("the convolution's inputs do not match the state's context")
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation {activation!r} is not one of {sorted(map(str, ACTIVATIONS))}")
    dims = (batch, L, ch, W)
    outs = list(conv_out) if conv_out is not None else [None, None]
    fo = _conv_out(outs[0], batch, L, H, P, ngroups, N, xbc.dtype, dev, "fwd")
    bo = _conv_out(outs[1], batch, L, H, P, ngroups, N, xbc.dtype, dev, "bwd")
    cfd = _conv_dir(conv_fwd, dims, xbc.dtype, dev, fo, "fwd")
    cbd = _conv_dir(conv_bwd, dims, xbc.dtype, dev, bo, "bwd")
    sf = dict(fwd, x=fo["x"], B=fo["B"], C=fo["C"])
    sb = dict(bwd, x=bo["x"], B=bo["B"], C=bo["C"])
    sdims = _dims(sf)
    shape = make_shape(fo["x"], fo["B"], chunk, dt_softplus=dt_softplus)
    fd = _dir(sf, xbc.dtype, sdims, dev, "fwd")
    bd = _dir(sb, xbc.dtype, sdims, dev, "bwd")
    if y is None:
        y = torch.empty((batch, L, H, P), dtype=torch.float32, device=dev)
    _check(y, "y", (batch, L, H, P), torch.float32, dev)
    cshape = _abi.ConvShape(batch, L, H, P, N, ngroups, W, DTYPES[xbc.dtype], ACTIVATIONS[activation], 0)
    _abi.check(lib().bimamba_block_step_conv(
        state.handle, ctypes.byref(cshape), ctypes.byref(cfd), ctypes.byref(cbd),
        ctypes.byref(shape), ctypes.byref(fd), ctypes.byref(bd), int(bool(commit)), _ptr(y),
        _stream(stream)))
    return y


class BlockStepPlan:
    """A block step with its arguments checked and bound once, for decode
    loops: run() calls bimamba_block_step on the same tensors (and the
    stream current at construction) without checking them again, so a step
    costs the C call and the launch. Write each step's inputs into the
    bound tensors in place; keep them alive and unchanged in shape while the
    plan is used. Same arguments as block_step."""

    def __init__(self, state, fwd, bwd, commit=False, chunk=64, y=None, stream=None,
                 dt_softplus=False):
        x = fwd["x"]
        dims = _dims(fwd)
        self._shape = make_shape(x, fwd["B"], chunk, dt_softplus=dt_softplus)
        dev = _cuda_device(x)
        self._fd = _dir(fwd, x.dtype, dims, dev, "fwd")
        self._bd = _dir(bwd, x.dtype, dims, dev, "bwd")
        if y is None:
            y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
        _check(y, "y", tuple(x.shape), torch.float32, x.device)
        self.y = y
        self._state = state
        self._keep = (fwd, bwd)
        self._fn = lib().bimamba_block_step
        self._args = (ctypes.byref(self._shape), ctypes.byref(self._fd), ctypes.byref(self._bd),
                      int(bool(commit)), _ptr(y), _stream(stream))

    def run(self):
        # the cache's handle is read per call: a freed cache is rejected by
        # the library instead of being used through a stale pointer
        rc = self._fn(self._state.handle, *self._args)
        if rc:
            _abi.check(rc)
        return self.y


ACTIVATIONS = {None: 0, "none": 0, "silu": 1}


def conv_channels(nheads, headdim, ngroups, d_state):
    return nheads * headdim + 2 * ngroups * d_state


def _conv_dir(d, dims, dtype, device, out, name):
    batch, L, ch, W = dims
    _check(d["xbc"], f"{name}.xbc", (batch, L, ch), dtype, device)
    _check(d["weight"], f"{name}.weight", (ch, W), torch.float32, device)
    if d.get("bias") is not None:
        _check(d["bias"], f"{name}.bias", (ch,), torch.float32, device)
    return _abi.ConvDir(d["xbc"].data_ptr(), d["weight"].data_ptr(),
                        d["bias"].data_ptr() if d.get("bias") is not None else None,
                        out["x"].data_ptr(), out["B"].data_ptr(), out["C"].data_ptr())


def _conv_out(out, batch, L, nheads, headdim, ngroups, d_state, dtype, device, name):
    if out is None:
        out = dict(x=torch.empty(batch, L, nheads, headdim, dtype=dtype, device=device),
                   B=torch.empty(batch, L, ngroups, d_state, dtype=dtype, device=device),
                   C=torch.empty(batch, L, ngroups, d_state, dtype=dtype, device=device))
    _check(out["x"], f"{name}_out.x", (batch, L, nheads, headdim), dtype, device)
    _check(out["B"], f"{name}_out.B", (batch, L, ngroups, d_state), dtype, device)
    _check(out["C"], f"{name}_out.C", (batch, L, ngroups, d_state), dtype, device)
    return out


def conv1d(fwd, bwd, nheads, headdim, ngroups, d_state, activation="silu",
           cu_seqlens=None, init_ctx=None, final_ctx=None, out=None, stream=None):
    """Short depthwise convolution of the scan inputs (bimamba_conv1d).

    fwd/bwd: dicts of device tensors xbc [b,L,ch] (x | B | C channels, bf16 or
    fp32), weight [ch,W] f32, bias [ch] f32 or None; bwd may be None.
    init_ctx/final_ctx: [b, W-1, ch] in xbc's dtype (may be the same tensor).
    out: optional (fwd_out, bwd_out) dicts of x, B, C to write.
    Returns (fwd_out, bwd_out), each a dict x [b,L,H,P], B, C [b,L,G,N].
    """
    xbc = fwd["xbc"]
    dev = _cuda_device(xbc)
    if xbc.dim() != 3 or fwd["weight"].dim() != 2:
        raise ValueError("xbc must be [batch, L, channels] and weight [channels, width]")
    batch, L, ch = xbc.shape
    W = fwd["weight"].shape[1]
    if ch != conv_channels(nheads, headdim, ngroups, d_state):
        raise ValueError(f"xbc has {ch} channels, expected nheads*headdim + 2*ngroups*d_state")
    if xbc.dtype not in DTYPES:
        raise TypeError(f"unsupported dtype {xbc.dtype}")
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation {activation!r} is not one of {sorted(map(str, ACTIVATIONS))}")
    dims = (batch, L, ch, W)
    outs = list(out) if out is not None else [None, None]
    fo = _conv_out(outs[0], batch, L, nheads, headdim, ngroups, d_state, xbc.dtype, dev, "fwd")
    fd = _conv_dir(fwd, dims, xbc.dtype, dev, fo, "fwd")
    bo = bd = None
    if bwd is not None:
        bo = _conv_out(outs[1], batch, L, nheads, headdim, ngroups, d_state, xbc.dtype, dev, "bwd")
        bd = _conv_dir(bwd, dims, xbc.dtype, dev, bo, "bwd")
    cu_arr, nseq = None, 0
    if cu_seqlens is not None:
        vals = [int(v) for v in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        nseq = len(vals) - 1
        cu_arr = (ctypes.c_int32 * len(vals))(*vals)
    for t, name in ((init_ctx, "init_ctx"), (final_ctx, "final_ctx")):
        if t is not None:
            _check(t, name, (batch, W - 1, ch), xbc.dtype, dev)
    shape = _abi.ConvShape(batch, L, nheads, headdim, d_state, ngroups, W,
                           DTYPES[xbc.dtype], ACTIVATIONS[activation], 0)
    n = ctypes.c_size_t(0)
    _abi.check(lib().bimamba_conv1d_workspace_size(ctypes.byref(shape), nseq, ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=dev) if n.value else None
    _abi.check(lib().bimamba_conv1d(
        ctypes.byref(shape), ctypes.byref(fd), ctypes.byref(bd) if bd is not None else None,
        cu_arr, nseq, _ptr(init_ctx), _ptr(final_ctx), _ptr(ws), n.value, _stream(stream)))
    return fo, bo


def gated_norm(y, z, weight, group_size=None, eps=1e-5, out=None, stream=None):
    """Gated RMS norm on the scan output (bimamba_gated_norm): y float32
    [..., C], z [..., C] (bf16 or fp32, also the output dtype), weight
    float32 [C]. group_size defaults to C (one group)."""
    dev = _cuda_device(y)
    C = y.shape[-1]
    rows = y.numel() // C if C else 0
    if z.dtype not in DTYPES:
        raise TypeError(f"unsupported dtype {z.dtype}")
    _check(y, "y", tuple(y.shape), torch.float32, dev)
    _check(z, "z", tuple(y.shape), z.dtype, dev)
    _check(weight, "weight", (C,), torch.float32, dev)
    if out is None:
        out = torch.empty(y.shape, dtype=z.dtype, device=dev)
    _check(out, "out", tuple(y.shape), z.dtype, dev)
    _abi.check(lib().bimamba_gated_norm(rows, C, C if group_size is None else int(group_size),
                                        DTYPES[z.dtype], _ptr(y), _ptr(z), _ptr(weight),
                                        float(eps), _ptr(out), _stream(stream)))
    return out


def seq_index(cu_seqlens, device="cuda", stream=None):
    """Per-token packed-sequence index built on the GPU (int32 [total])."""
    vals = [int(v) for v in cu_seqlens]
    total = vals[-1]
    if torch.device(device).type != "cuda":
        raise ValueError(f"device must be a CUDA device, not {device}")
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
