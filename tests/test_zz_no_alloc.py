"""The no-allocation entry point (bimamba_ssd_fwd_noalloc) against
bimamba_ssd_fwd through the C ABI: two calls in a row, the second with a
smaller input, each to the parity bar against the allocating entry point's
output (their segment lengths may differ, so rounding may)."""
import numpy as np
import pytest
import torch

import bidirectional_mamba_ssm_amd as bm
import synth
from metrics import within

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(f, b, chunk, cu=None, init=None):
    batch, L, H, P = f["x"].shape
    N = f["B"].shape[3]
    want = init is not None
    ref_fs = torch.full((batch, H, P, N), float("nan"), device=DEV) if want else None
    got_fs = torch.full((batch, H, P, N), float("nan"), device=DEV) if want else None
    ref = bm.ssd_fwd(f, b, chunk=chunk, cu_seqlens=cu, init_state=init, final_state=ref_fs)
    y = torch.full_like(ref, float("nan"))
    bm.ssd_fwd_noalloc(f, b, y, chunk=chunk, cu_seqlens=cu, init_state=init, final_state=got_fs)
    torch.cuda.synchronize()
    out = [(y, ref)] + ([(got_fs, ref_fs)] if want else [])
    return [(g.double().cpu().numpy(), r.double().cpu().numpy()) for g, r in out]


def test_noalloc_two_calls():
    # 1: a row whose normal segment states (64 MiB) exceed the static buffer,
    #    so the no-allocation call runs longer segments; incoming and outgoing
    #    states, both directions
    f, b = synth.make_inputs(1, 4096, 64, 64, 128, 1, "bf16", 181, device=DEV)
    shape = bm.make_shape(f["x"], f["B"], 256)
    assert bm.workspace_size(shape, 0) > bm._abi.NOALLOC_SCRATCH_BYTES
    g = torch.Generator(device=DEV).manual_seed(182)
    init = torch.randn(1, 64, 64, 128, generator=g, device=DEV) * 0.5
    for got, ref in _both(f, b, 256, init=init):
        assert np.all(np.isfinite(got))
        err, ok = within(got, ref, "bf16")
        print(f"call 1: {err:.3e}", flush=True)
        assert ok, f"call 1: {err:.3e}"
    # 2: a smaller packed batch (the sequence tables live in the same buffer)
    lens = [300, 0, 77, 600, 1]
    cu = synth.cu_seqlens_of(lens)
    f, b = synth.make_inputs(1, cu[-1], 4, 64, 128, 1, "bf16", 183, device=DEV)
    for got, ref in _both(f, b, 64, cu=cu):
        err, ok = within(got, ref, "bf16")
        print(f"call 2: {err:.3e}", flush=True)
        assert ok, f"call 2: {err:.3e}"


def test_noalloc_token_sequential_shape():
    # fp32 and a small head shape: the token-sequential kernels
    f, b = synth.make_inputs(2, 700, 4, 16, 16, 1, "f32", 184, device=DEV)
    for got, ref in _both(f, b, 64):
        err, ok = within(got, ref, "f32")
        print(f"fp32: {err:.3e}", flush=True)
        assert ok, f"fp32: {err:.3e}"


def test_noalloc_rejects_tables_beyond_the_buffer():
    # packed tables larger than the buffer are rejected before any launch
    L = (64 << 20) // 4 + 64
    x = torch.zeros(1, 1, 1, 64, dtype=torch.bfloat16, device=DEV)
    d = dict(x=x, dt=torch.zeros(1, 1, 1, dtype=torch.bfloat16, device=DEV),
             A=torch.zeros(1, device=DEV), B=torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16, device=DEV),
             C=torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16, device=DEV), D=None)
    shape = bm._abi.Shape(1, L, 1, 64, 128, 1, 64, bm._abi.BF16, 0)
    fd = bm._dir(d, torch.bfloat16, (1, 1, 1, 64, 1, 128), x.device)
    cu = (bm.ctypes.c_int32 * 2)(0, L)
    rc = bm.lib().bimamba_ssd_fwd_noalloc(bm.ctypes.byref(shape), bm.ctypes.byref(fd), None, cu, 1,
                                          None, None, bm._ptr(x), None)
    assert rc == bm._abi.EWORKSPACE, rc
    assert b"sequence tables" in bm.lib().bimamba_last_error()
