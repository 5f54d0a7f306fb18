"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects malformed arguments on the host before any HIP
call (so no error path launches anything)."""
import ctypes
import os
import re

import pytest

from bidirectional_mamba_ssm_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        from bidirectional_mamba_ssm_amd import build
        build.build()
    return _abi.load()


def header_symbols():
    text = open(os.path.join(ROOT, "include", "bimamba.h")).read()
    return sorted(set(re.findall(r"\b(bimamba_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = header_symbols()
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in bimamba.h but not exported"
    assert set(declared) == set(_abi.EXPORTS)


def test_version_and_status_strings(lib):
    assert lib.bimamba_version() == 2
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.bimamba_status_str(code)
    assert lib.bimamba_status_str(99) == b"unknown status"


def shape(**kw):
    d = dict(batch=1, seqlen=256, nheads=4, headdim=16, d_state=16, ngroups=1,
             chunk=64, dtype=_abi.F32)
    d.update(kw)
    return _abi.Shape(**d)


FAKE = 0x10000  # 16-aligned, never dereferenced: every call below fails validation


def fake_dir(**kw):
    d = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None)
    d.update(kw)
    return _abi.Dir(**d)


def call_fwd(lib, s, f, b=None, cu=None, nseq=0, init=None, final=None, y=FAKE,
             ws=None, wsb=0):
    arr = None
    if cu is not None:
        arr = (ctypes.c_int32 * len(cu))(*cu)
    return lib.bimamba_ssd_fwd(ctypes.byref(s) if s is not None else None,
                               ctypes.byref(f) if f is not None else None,
                               ctypes.byref(b) if b is not None else None,
                               arr, nseq, init, final, y, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _abi.EINVAL),
    (dict(batch=0), _abi.EINVAL),
    (dict(seqlen=-1), _abi.EINVAL),
    (dict(nheads=0), _abi.EINVAL),
    (dict(nheads=4, ngroups=3), _abi.EINVAL),
    (dict(chunk=32), _abi.EUNSUPPORTED),
    (dict(chunk=0), _abi.EUNSUPPORTED),
    (dict(d_state=24), _abi.EUNSUPPORTED),
    (dict(headdim=256), _abi.EUNSUPPORTED),
    (dict(batch=1 << 16, seqlen=1 << 16), _abi.EUNSUPPORTED),
])
def test_shape_rejected(lib, kw, code):
    assert call_fwd(lib, shape(**kw), fake_dir()) == code
    assert lib.bimamba_last_error()


def test_null_arguments(lib):
    assert call_fwd(lib, None, fake_dir()) == _abi.EINVAL
    assert call_fwd(lib, shape(), None) == _abi.EINVAL
    assert call_fwd(lib, shape(), fake_dir(x=None)) == _abi.EINVAL
    assert call_fwd(lib, shape(), fake_dir(A=None)) == _abi.EINVAL
    assert call_fwd(lib, shape(), fake_dir(), y=None) == _abi.EINVAL
    assert call_fwd(lib, shape(), fake_dir(), b=fake_dir(C=None)) == _abi.EINVAL


def test_misaligned(lib):
    assert call_fwd(lib, shape(), fake_dir(x=FAKE + 2)) == _abi.EINVAL
    assert call_fwd(lib, shape(), fake_dir(), y=FAKE + 4) == _abi.EINVAL
    assert call_fwd(lib, shape(), fake_dir(), init=FAKE + 4) == _abi.EINVAL
    assert call_fwd(lib, shape(), fake_dir(), final=FAKE + 8) == _abi.EINVAL


def test_bad_offsets(lib):
    s = shape(seqlen=10)
    assert call_fwd(lib, s, fake_dir(), cu=[0, 4, 3, 10], nseq=3) == _abi.EINVAL  # decreasing
    assert call_fwd(lib, s, fake_dir(), cu=[1, 4, 10], nseq=2) == _abi.EINVAL     # cu[0] != 0
    assert call_fwd(lib, s, fake_dir(), cu=[0, 4, 9], nseq=2) == _abi.EINVAL      # wrong total
    assert call_fwd(lib, shape(seqlen=10, batch=2), fake_dir(), cu=[0, 10], nseq=1) == _abi.EINVAL
    assert call_fwd(lib, s, fake_dir(), cu=None, nseq=2) == _abi.EINVAL           # nseq w/o offsets
    assert call_fwd(lib, s, fake_dir(), cu=[0, 10], nseq=1, init=FAKE) == _abi.EUNSUPPORTED


def test_workspace_checks(lib):
    s = shape(seqlen=10)
    n = ctypes.c_size_t(0)
    assert lib.bimamba_ssd_workspace_size(ctypes.byref(s), 2, ctypes.byref(n)) == 0
    assert n.value > 0
    assert call_fwd(lib, s, fake_dir(), cu=[0, 4, 10], nseq=2, ws=None) == _abi.EWORKSPACE
    assert call_fwd(lib, s, fake_dir(), cu=[0, 4, 10], nseq=2, ws=FAKE * 256,
                    wsb=n.value - 1) == _abi.EWORKSPACE
    assert call_fwd(lib, s, fake_dir(), cu=[0, 4, 10], nseq=2, ws=FAKE * 256 + 16,
                    wsb=n.value) == _abi.EINVAL
    assert lib.bimamba_ssd_workspace_size(ctypes.byref(shape(chunk=48)), 0,
                                          ctypes.byref(n)) == _abi.EUNSUPPORTED


def test_state_and_block_step_validation(lib):
    assert lib.bimamba_state_alloc(None, 1, 1, 1, 1) == _abi.EINVAL
    h = ctypes.c_void_p()
    assert lib.bimamba_state_alloc(ctypes.byref(h), 0, 4, 16, 16) == _abi.EINVAL
    assert lib.bimamba_state_reset(None, None, 0, None) == _abi.EINVAL
    assert lib.bimamba_state_data(None) is None
    assert lib.bimamba_state_free(None) == 0
    s = shape(seqlen=64)
    assert lib.bimamba_block_step(None, ctypes.byref(s), ctypes.byref(fake_dir()),
                                  ctypes.byref(fake_dir()), 0, FAKE, None) == _abi.EINVAL


def test_conv_state_validation(lib):
    """The state with a convolution context and the raw-input block step:
    malformed arguments are rejected before any allocation or launch."""
    h = ctypes.c_void_p()
    assert lib.bimamba_state_alloc_conv(None, 1, 4, 64, 128, 1, 4, _abi.BF16) == _abi.EINVAL
    assert lib.bimamba_state_alloc_conv(ctypes.byref(h), 1, 4, 64, 128, 1, 5, _abi.BF16) == _abi.EINVAL
    assert lib.bimamba_state_alloc_conv(ctypes.byref(h), 1, 4, 64, 128, 1, 1, _abi.BF16) == _abi.EINVAL
    assert lib.bimamba_state_alloc_conv(ctypes.byref(h), 1, 4, 64, 128, 3, 4, _abi.BF16) == _abi.EINVAL
    assert lib.bimamba_state_alloc_conv(ctypes.byref(h), 1, 4, 64, 128, 1, 4, 7) == _abi.EINVAL
    # a slot's context that is not a multiple of 16 bytes: 3 x (3 + 2 * 2) bf16 values
    assert lib.bimamba_state_alloc_conv(ctypes.byref(h), 1, 1, 3, 2, 1, 4, _abi.BF16) == _abi.EUNSUPPORTED
    assert lib.bimamba_state_conv_ctx(None) is None
    cs, s = conv_shape(), shape(seqlen=64)
    rc = lib.bimamba_block_step_conv(None, ctypes.byref(cs), ctypes.byref(fake_conv_dir()),
                                     ctypes.byref(fake_conv_dir()), ctypes.byref(s),
                                     ctypes.byref(fake_dir()), ctypes.byref(fake_dir()), 1, FAKE, None)
    assert rc == _abi.EINVAL
    assert b"state is NULL" in lib.bimamba_last_error()


def test_seq_index_validation(lib):
    arr = (ctypes.c_int32 * 3)(0, 5, 4)
    assert lib.bimamba_seq_index(arr, 2, 4, FAKE, None) == _abi.EINVAL
    assert lib.bimamba_seq_index(None, 2, 4, FAKE, None) == _abi.EINVAL


def conv_shape(**kw):
    d = dict(batch=1, seqlen=64, nheads=4, headdim=16, d_state=16, ngroups=1,
             width=4, dtype=_abi.BF16, activation=1, flags=0)
    d.update(kw)
    return _abi.ConvShape(**d)


def fake_conv_dir(**kw):
    d = dict(xbc=FAKE, weight=FAKE, bias=FAKE, x=FAKE, B=FAKE, C=FAKE)
    d.update(kw)
    return _abi.ConvDir(**d)


def call_conv(lib, s, f, b=None, cu=None, nseq=0, init=None, final=None, ws=None, wsb=0):
    arr = (ctypes.c_int32 * len(cu))(*cu) if cu is not None else None
    return lib.bimamba_conv1d(ctypes.byref(s) if s is not None else None,
                              ctypes.byref(f) if f is not None else None,
                              ctypes.byref(b) if b is not None else None,
                              arr, nseq, init, final, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), _abi.EINVAL),
    (dict(batch=0), _abi.EINVAL),
    (dict(seqlen=-2), _abi.EINVAL),
    (dict(headdim=0), _abi.EINVAL),
    (dict(width=1), _abi.EUNSUPPORTED),
    (dict(width=5), _abi.EUNSUPPORTED),
    (dict(activation=2), _abi.EINVAL),
    (dict(flags=1), _abi.EINVAL),
    (dict(batch=40000), _abi.EUNSUPPORTED),
    (dict(batch=1 << 16, seqlen=1 << 16), _abi.EUNSUPPORTED),
])
def test_conv_shape_rejected(lib, kw, code):
    assert call_conv(lib, conv_shape(**kw), fake_conv_dir()) == code
    n = ctypes.c_size_t(7)
    assert lib.bimamba_conv1d_workspace_size(ctypes.byref(conv_shape(**kw)), 0, ctypes.byref(n)) == code


def test_conv_arguments_rejected(lib):
    s = conv_shape()
    assert call_conv(lib, None, fake_conv_dir()) == _abi.EINVAL
    assert call_conv(lib, s, None) == _abi.EINVAL
    for field in ("xbc", "weight", "x", "B", "C"):
        assert call_conv(lib, s, fake_conv_dir(**{field: None})) == _abi.EINVAL, field
        assert call_conv(lib, s, fake_conv_dir(), fake_conv_dir(**{field: None})) == _abi.EINVAL, field
    for field in ("xbc", "x", "B", "C"):
        assert call_conv(lib, s, fake_conv_dir(**{field: FAKE + 8})) == _abi.EINVAL, field
    assert call_conv(lib, s, fake_conv_dir(weight=FAKE + 2)) == _abi.EINVAL
    assert call_conv(lib, s, fake_conv_dir(bias=FAKE + 1)) == _abi.EINVAL
    assert call_conv(lib, s, fake_conv_dir(), init=FAKE + 4) == _abi.EINVAL
    # contexts that overlap without being the same array
    assert call_conv(lib, s, fake_conv_dir(), init=FAKE, final=FAKE + 16) == _abi.EINVAL
    # packed sequences: bad offsets, batch > 1, contexts, workspace
    assert call_conv(lib, s, fake_conv_dir(), cu=[0, 70], nseq=1) == _abi.EINVAL
    assert call_conv(lib, s, fake_conv_dir(), cu=[0, 40, 30, 64], nseq=3) == _abi.EINVAL
    assert call_conv(lib, conv_shape(batch=2), fake_conv_dir(), cu=[0, 64], nseq=1) == _abi.EINVAL
    assert call_conv(lib, s, fake_conv_dir(), cu=[0, 64], nseq=1, init=FAKE) == _abi.EUNSUPPORTED
    assert call_conv(lib, s, fake_conv_dir(), nseq=2) == _abi.EINVAL
    assert call_conv(lib, s, fake_conv_dir(), cu=[0, 32, 64], nseq=2) == _abi.EWORKSPACE
    n = ctypes.c_size_t(0)
    assert lib.bimamba_conv1d_workspace_size(ctypes.byref(s), 2, ctypes.byref(n)) == _abi.OK
    assert n.value >= 12 and n.value % 256 == 0
    assert call_conv(lib, s, fake_conv_dir(), cu=[0, 32, 64], nseq=2, ws=FAKE,
                     wsb=n.value - 1) == _abi.EWORKSPACE
    assert call_conv(lib, s, fake_conv_dir(), cu=[0, 32, 64], nseq=2, ws=FAKE + 16,
                     wsb=n.value) == _abi.EINVAL
    assert lib.bimamba_conv1d_workspace_size(ctypes.byref(s), 0, ctypes.byref(n)) == _abi.OK
    assert n.value == 0
    assert lib.bimamba_conv1d_workspace_size(ctypes.byref(s), -1, ctypes.byref(n)) == _abi.EINVAL


def test_dt_softplus_flag(lib):
    # defined for the forward and the block step only
    assert call_fwd(lib, shape(flags=2), fake_dir()) == _abi.EINVAL
    s = shape(flags=1)
    n = ctypes.c_size_t(0)
    assert lib.bimamba_ssd_bwd_workspace_size(ctypes.byref(s), 1, ctypes.byref(n)) == _abi.EUNSUPPORTED
    g = _abi.Grad(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    f = fake_dir()
    assert lib.bimamba_ssd_bwd(ctypes.byref(s), ctypes.byref(f), None, FAKE, ctypes.byref(g), None,
                               FAKE, 1 << 30, None) == _abi.EUNSUPPORTED


def test_gated_norm_validation(lib):
    f = lib.bimamba_gated_norm
    ok = dict(rows=4, channels=512, group_size=256, dtype=_abi.BF16, y=FAKE, z=FAKE,
              weight=FAKE, eps=1e-5, out=FAKE)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return f(d["rows"], d["channels"], d["group_size"], d["dtype"], d["y"], d["z"],
                 d["weight"], d["eps"], d["out"], None)
    assert call(dtype=3) == _abi.EINVAL
    assert call(rows=-1) == _abi.EINVAL
    assert call(rows=1 << 31) == _abi.EUNSUPPORTED
    assert call(channels=100) == _abi.EUNSUPPORTED
    assert call(channels=8192 + 256) == _abi.EUNSUPPORTED
    assert call(group_size=128) == _abi.EINVAL
    assert call(group_size=768) == _abi.EINVAL
    assert call(eps=-1.0) == _abi.EINVAL
    assert call(eps=float("nan")) == _abi.EINVAL
    for k in ("y", "z", "weight", "out"):
        assert call(**{k: None}) == _abi.EINVAL, k
        assert call(**{k: FAKE + 4}) == _abi.EINVAL, k
    assert call(rows=0, y=None, z=None, weight=None, out=None) == _abi.OK


def test_streams_validation(lib):
    s, f, b = shape(), fake_dir(), fake_dir()

    def call(s=s, f=f, b=b, yf=FAKE, yb=FAKE + 4096):
        return lib.bimamba_ssd_fwd_streams(ctypes.byref(s) if s is not None else None,
                                           ctypes.byref(f) if f is not None else None,
                                           ctypes.byref(b) if b is not None else None,
                                           None, 0, None, None, yf, yb, None, 0, None)
    assert call(b=None) == _abi.EINVAL
    assert call(s=None) == _abi.EINVAL
    assert call(s=shape(flags=_abi.DT_SOFTPLUS)) == _abi.EUNSUPPORTED
    assert call(yf=None) == _abi.EINVAL
    assert call(yb=None) == _abi.EINVAL
    assert call(yb=FAKE) == _abi.EINVAL
    assert call(yf=FAKE + 4) == _abi.EINVAL
    assert call(yb=FAKE + 4100) == _abi.EINVAL
    assert call(s=shape(dtype=7)) == _abi.EINVAL


def test_merge_validation(lib):
    f = lib.bimamba_merge_linear
    ok = dict(rows=4, cin=64, cout=32, yf=FAKE, yb=FAKE, w=FAKE, bias=None, out=FAKE)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return f(d["rows"], d["cin"], d["cout"], d["yf"], d["yb"], d["w"], d["bias"],
                 d["out"], None)
    assert call(rows=-1) == _abi.EINVAL
    assert call(rows=1 << 31) == _abi.EUNSUPPORTED
    assert call(cin=48) == _abi.EUNSUPPORTED
    assert call(cin=0) == _abi.EUNSUPPORTED
    assert call(cout=24) == _abi.EUNSUPPORTED
    assert call(cout=-16) == _abi.EUNSUPPORTED
    for k in ("yf", "yb", "w", "out"):
        assert call(**{k: None}) == _abi.EINVAL, k
        assert call(**{k: FAKE + 4}) == _abi.EINVAL, k
    assert call(bias=FAKE + 2) == _abi.EINVAL
    assert call(bias=FAKE + 4) == _abi.EINVAL
    assert call(rows=0, yf=None, yb=None, w=None, out=None) == _abi.OK


def _al256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("batch,L,H,chunk,nseg", [
    (1, 131072, 64, 256, 8),    # the long prefill: 16 384-token segments, one round of 256 workgroups
    (1, 148170, 64, 256, 8),    # the packed batch's length: 18 688-token segments (not a power of two)
    (1, 32768, 64, 256, 8),
    (1, 5000, 64, 64, 8),       # 640-token segments
    (8, 1024, 64, 256, 1),      # the training layer: whole rows, no segment states
    (1, 1000, 4, 256, 4),       # few heads: 256-token segments
])
def test_segment_rule_workspace(lib, batch, L, H, chunk, nseg):
    """The workspace the chunked scan asks for holds the segment states of
    the segment count its length rule gives (a multiple of the chunk, the
    shortest for each count, costed in rounds of 256 workgroups)."""
    s = shape(batch=batch, seqlen=L, nheads=H, headdim=64, d_state=128, chunk=chunk, dtype=_abi.BF16)
    n = ctypes.c_size_t(0)
    assert lib.bimamba_ssd_workspace_size(ctypes.byref(s), 0, ctypes.byref(n)) == _abi.OK
    want = 0 if nseg == 1 else (2 * _al256(batch * 2 * nseg * H * 64 * 128 * 4) +
                                _al256(batch * 2 * nseg * H * 4))
    assert n.value == want
