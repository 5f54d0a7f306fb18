"""GPU parity of the concatenating merge, through the C ABI: the scan with
the two streams kept apart (bimamba_ssd_fwd_streams) against the fp64
oracle's forward-only and reverse-only outputs, and the Linear merge of the
two (bimamba_merge_linear) against oracle/merge.py."""
import numpy as np
import pytest
import torch

import bidirectional_mamba_ssm_amd as bm
import oracle
from oracle import merge as omerge
import synth
from metrics import bf16_rne, within

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _np(t):
    return t.double().cpu().numpy()


def _stream_refs(f, b, cu=None, init=None):
    """(forward stream, reverse stream, final state) from the oracle: the
    forward stream alone, and the reverse one as the bidirectional sum minus
    it (fp64: the difference is exact to far below any tolerance here)."""
    yf, fs = oracle.bissd(f, None, cu_seqlens=cu, init_state=init, want_final_state=True)
    ysum = oracle.bissd(f, b, cu_seqlens=cu, init_state=init)
    return yf, ysum - yf, fs


def _check_streams(f, b, dtype, chunk, cu=None, init=None, tag=""):
    batch, L, H, P = f["x"].shape
    N = f["B"].shape[3]
    # packed sequences carry no states
    final = torch.full((batch, H, P, N), float("nan"), device=DEV) if cu is None else None
    yf, yb = bm.ssd_fwd_streams(f, b, chunk=chunk, cu_seqlens=cu, init_state=init,
                                final_state=final)
    torch.cuda.synchronize()
    rf, rb, rfs = _stream_refs(f, b, cu, init)
    checks = [("y_fwd", yf, rf), ("y_bwd", yb, rb)]
    if final is not None:
        checks.append(("final state", final, rfs))
    for name, got, ref in checks:
        err, ok = within(_np(got), ref, dtype)
        print(f"  {tag} {name} error {err:.3e}", flush=True)
        assert ok, f"{tag} {name}: error {err:.3e}"
    return yf, yb


STREAM_CASES = [
    # name, batch, L, H, P, N, G, dtype, chunk, seed
    ("f32_q64_ragged_groups", 2, 203, 4, 16, 32, 2, "f32", 64, 140),
    ("bf16_q64", 2, 200, 4, 64, 128, 2, "bf16", 64, 141),
    ("bf16_q128", 1, 384, 2, 64, 128, 1, "bf16", 128, 142),
    ("bf16_q256_ragged", 1, 777, 2, 64, 128, 1, "bf16", 256, 143),
    ("bf16_single_chunk", 3, 40, 2, 64, 128, 1, "bf16", 64, 144),
    ("bf16_L1", 2, 1, 2, 64, 128, 1, "bf16", 256, 145),
    # few (row, head) pairs over long rows: the token-sequential path
    ("f32_sequential_ragged", 1, 4001, 1, 16, 16, 1, "f32", 64, 146),
    ("bf16_sequential", 1, 3000, 2, 16, 16, 1, "bf16", 256, 147),
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=[c[0] for c in STREAM_CASES])
@pytest.mark.parametrize("with_init", [False, True], ids=["zero_state", "init_state"])
def test_streams_parity(case, with_init):
    name, batch, L, H, P, N, G, dtype, chunk, seed = case
    print(f"streams {name} init={with_init}", flush=True)
    f, b = synth.make_inputs(batch, L, H, P, N, G, dtype, seed, device=DEV)
    init = None
    if with_init:
        g = torch.Generator(device=DEV).manual_seed(seed + 1000)
        init = torch.randn(batch, H, P, N, generator=g, device=DEV) * 0.5
    _check_streams(f, b, dtype, chunk, init=init, tag=name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 256])
def test_streams_packed(dtype, chunk):
    lens = [100, 0, 1, 257, 64, 30]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    P, N = (16, 16) if dtype == "f32" else (64, 128)
    f, b = synth.make_inputs(1, int(cu[-1]), 4, P, N, 1, dtype, 150 + chunk, device=DEV)
    _check_streams(f, b, dtype, chunk, cu=cu.tolist(), tag=f"packed {dtype} q{chunk}")


def test_streams_sum_equals_fused():
    """The two streams added equal the summed output the fused scan writes
    (the same kernels; only where each stream lands differs)."""
    f, b = synth.make_inputs(2, 300, 4, 64, 128, 1, "bf16", 151, device=DEV)
    yf, yb = bm.ssd_fwd_streams(f, b, chunk=256)
    y = bm.ssd_fwd(f, b, chunk=256)
    torch.cuda.synchronize()
    err = float((yf + yb - y).abs().max()) / float(y.abs().max())
    print(f"  |y_fwd + y_bwd - y| / max|y| = {err:.2e}", flush=True)
    assert err <= 1e-6


def test_streams_layer_full_size_sampled():
    """The training layer (8 x 1024 tokens, 64 heads x 64, d_state 128,
    bf16) in the benchmark's launch; the oracle recomputes a few heads."""
    w = synth.WORKLOADS["layer_1p3b_train"]
    f, b = synth.make_workload(w, device=DEV)
    yf, yb = bm.ssd_fwd_streams(f, b, chunk=w.chunk)
    torch.cuda.synchronize()
    heads = [0, 17, 63]

    def sel(d):
        # the same inputs on a subset of heads (one group: B and C are shared)
        e = dict(d)
        for k in ("x", "dt"):
            e[k] = d[k][:, :, heads].contiguous()
        for k in ("A", "D"):
            e[k] = d[k][heads].contiguous()
        return e
    assert f["B"].shape[2] == 1
    rf, rb, _ = _stream_refs(sel(f), sel(b))
    for name, got, ref in (("y_fwd", yf, rf), ("y_bwd", yb, rb)):
        err, ok = within(_np(got[:, :, heads]), ref, "bf16")
        print(f"  layer {name} error {err:.3e}", flush=True)
        assert ok, f"layer {name}: error {err:.3e}"


# ---- the Linear merge
#
# The kernel rounds y_fwd and y_bwd to bfloat16 (nearest even) as it stages
# them, multiplies with the bf16 weight on the matrix cores and accumulates
# in fp32. Two bars: against the oracle on the bf16-rounded inputs (only fp32
# accumulation error remains: |err| <= 1e-5 * S, S = |y| |W|^T + |bias| on
# the same inputs), and against the oracle on the fp32 inputs (the rounding
# of y adds at most 2^-9 relative per product: |err| <= 2^-8 * S).

def _merge_inputs(rows, cin, cout, seed, bias=True):
    g = torch.Generator(device=DEV).manual_seed(seed)
    yf = torch.randn(rows, cin, generator=g, device=DEV)
    yb = torch.randn(rows, cin, generator=g, device=DEV)
    w = (torch.randn(cout, 2 * cin, generator=g, device=DEV) / (2 * cin) ** 0.5).to(torch.bfloat16)
    b = torch.randn(cout, generator=g, device=DEV) if bias else None
    return yf, yb, w, b


def _check_merge(yf, yb, w, b, out, tag):
    nyf, nyb, nw = _np(yf), _np(yb), _np(w)
    nb = _np(b) if b is not None else None
    got = _np(out).reshape(-1, nw.shape[0])
    nyf, nyb = nyf.reshape(-1, nyf.shape[-1]), nyb.reshape(-1, nyb.shape[-1])
    absb = np.abs(nb) if nb is not None else None
    rf, rb = bf16_rne(nyf), bf16_rne(nyb)
    exact = omerge.merge_linear(rf, rb, nw, nb)
    S = omerge.merge_linear(np.abs(rf), np.abs(rb), np.abs(nw), absb)
    e1 = float(np.max(np.abs(got - exact) / np.maximum(S, 1e-300), initial=0.0))
    ref = omerge.merge_linear(nyf, nyb, nw, nb)
    S0 = omerge.merge_linear(np.abs(nyf), np.abs(nyb), np.abs(nw), absb)
    e2 = float(np.max(np.abs(got - ref) / np.maximum(S0, 1e-300), initial=0.0))
    print(f"  {tag}: |err|/S on rounded inputs {e1:.2e}, on fp32 inputs {e2:.2e}", flush=True)
    assert e1 <= 1e-5, f"{tag}: {e1:.3e}"
    assert e2 <= 2.0 ** -8, f"{tag}: {e2:.3e}"


MERGE_CASES = [
    # name, rows, cin, cout, bias, seed
    ("one_tile", 128, 32, 128, True, 160),
    ("ragged_rows", 1000, 64, 96, True, 161),
    ("cout_16", 77, 32, 16, False, 162),
    ("one_row", 1, 128, 144, True, 163),
    ("ragged_tiles", 515, 160, 272, True, 164),
    ("deep_k", 300, 2048, 128, True, 165),
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=[c[0] for c in MERGE_CASES])
def test_merge_parity(case):
    name, rows, cin, cout, bias, seed = case
    print(f"merge {name}", flush=True)
    yf, yb, w, b = _merge_inputs(rows, cin, cout, seed, bias)
    out = bm.merge_linear(yf, yb, w, b)
    torch.cuda.synchronize()
    _check_merge(yf, yb, w, b, out, name)


def test_merge_empty():
    yf, yb, w, b = _merge_inputs(0, 64, 32, 166)
    out = bm.merge_linear(yf, yb, w, b)
    torch.cuda.synchronize()
    assert out.shape == (0, 32)


def test_merge_deterministic():
    yf, yb, w, b = _merge_inputs(700, 256, 256, 167)
    o1 = bm.merge_linear(yf, yb, w, b)
    o2 = bm.merge_linear(yf, yb, w, b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_merge_layer_full_size_sampled():
    """The layer's merge at its real width (8 x 1024 tokens, d_model 2048 per
    stream into 2048), in the benchmark's launch; the oracle recomputes a
    sample of rows."""
    rows, cin, cout = 8 * 1024, 2048, 2048
    yf, yb, w, b = _merge_inputs(rows, cin, cout, 168)
    out = bm.merge_linear(yf, yb, w, b)
    torch.cuda.synchronize()
    idx = torch.tensor([0, 1, 127, 128, 4095, 5000, rows - 1], device=DEV)
    _check_merge(yf[idx], yb[idx], w, b, out[idx], "layer sample")


def test_streams_then_merge_end_to_end():
    """Scan with the streams apart, each stream laid out as [tokens, H*P],
    then the merge: against the oracle's streams fed to the oracle merge."""
    batch, L, H, P, N = 2, 130, 4, 64, 128
    f, b = synth.make_inputs(batch, L, H, P, N, 1, "bf16", 169, device=DEV)
    yf, yb = bm.ssd_fwd_streams(f, b, chunk=64)
    cin = H * P
    _, _, w, bias = _merge_inputs(1, cin, 192, 170)
    out = bm.merge_linear(yf.reshape(-1, cin), yb.reshape(-1, cin), w, bias)
    torch.cuda.synchronize()
    rf, rb, _ = _stream_refs(f, b)
    ref = omerge.merge_linear(rf.reshape(-1, cin), rb.reshape(-1, cin), _np(w), _np(bias))
    # the scan's error (bf16 bar) carried through W, plus the bf16 staging of y
    err, ok = within(_np(out), ref, "bf16")
    print(f"  streams + merge error {err:.3e}", flush=True)
    assert ok, f"streams + merge: {err:.3e}"


def test_merge_large_tile_ragged():
    """The large-tile launch (256 x 256 workgroup tiles) with a ragged last
    token panel, a ragged last output block and an odd number of 32-channel
    K steps per stream; sampled rows against the oracle."""
    rows, cin, cout = 8192 + 77, 1056, 2048 + 16
    yf, yb, w, b = _merge_inputs(rows, cin, cout, 171)
    out = bm.merge_linear(yf, yb, w, b)
    torch.cuda.synchronize()
    idx = torch.tensor([0, 255, 256, 4097, rows - 78, rows - 77, rows - 2, rows - 1], device=DEV)
    _check_merge(yf[idx], yb[idx], w, b, out[idx], "large ragged sample")
