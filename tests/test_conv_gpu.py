"""GPU parity of the short convolution (bimamba_conv1d, through the C ABI)
against the fp64 oracle in oracle/conv.py, element by element: bf16 outputs
must be a correct rounding of the exact value (up to the fp32 evaluation
bound of tests/metrics.conv_close), fp32 outputs within that bound, carried
contexts bit for bit."""
import numpy as np
import pytest
import torch

import bidirectional_mamba_ssm_amd as bm
import oracle
import synth
from metrics import conv_close, within
from oracle import conv as oconv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _np(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().double().cpu().numpy()


def _scale(d, reverse, cu=None, init=None):
    """The filter on |inputs|, |weights|, |bias|: bounds every partial sum."""
    return oconv.conv1d(np.abs(_np(d["xbc"])), np.abs(_np(d["weight"])),
                        np.abs(_np(d["bias"])) if d.get("bias") is not None else None,
                        reverse=reverse, cu_seqlens=cu,
                        init_ctx=None if init is None else np.abs(_np(init)),
                        activation="none")


def _check_dir(out, d, reverse, dims, dtype, act, cu=None, init=None):
    H, P, G, N = dims
    ref = oconv.conv1d(d["xbc"], d["weight"], d.get("bias"), reverse=reverse,
                       cu_seqlens=cu, init_ctx=init, activation=act)
    scale = _scale(d, reverse, cu, init)
    got = np.concatenate([_np(out["x"]).reshape(ref.shape[0], ref.shape[1], -1),
                          _np(out["B"]).reshape(ref.shape[0], ref.shape[1], -1),
                          _np(out["C"]).reshape(ref.shape[0], ref.shape[1], -1)], axis=-1)
    worst, ok = conv_close(got, ref, scale, dtype)
    # the split itself: the oracle's x | B | C against the kernel's arrays
    rx, rB, rC = oconv.split_xbc(ref, H, P, G, N)
    assert rx.shape == out["x"].shape and rB.shape == out["B"].shape == rC.shape
    return worst, ok


CASES = [
    # name, batch, L, H, P, G, N, W, dtype, act, seed
    ("bf16_layer_slice", 2, 300, 8, 64, 1, 128, 4, "bf16", "silu", 40),
    ("bf16_groups_ragged", 3, 77, 4, 64, 2, 128, 4, "bf16", "silu", 41),
    ("f32_small", 1, 203, 4, 16, 2, 16, 4, "f32", "silu", 42),
    ("bf16_w3_noact", 2, 129, 4, 16, 1, 16, 3, "bf16", "none", 43),
    ("f32_w2", 1, 64, 2, 16, 1, 16, 2, "f32", "silu", 44),
    ("bf16_scalar_path", 2, 90, 3, 5, 1, 3, 4, "bf16", "silu", 45),
    ("f32_scalar_path", 1, 131, 5, 3, 1, 7, 3, "f32", "none", 46),
    ("bf16_L1", 2, 1, 4, 16, 1, 16, 4, "bf16", "silu", 47),
    ("bf16_L2", 1, 2, 4, 16, 1, 16, 4, "bf16", "silu", 48),
    ("bf16_L65", 1, 65, 4, 64, 1, 128, 4, "bf16", "silu", 49),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("bidir", [True, False], ids=["bi", "fwd"])
def test_conv_parity(case, bidir):
    name, batch, L, H, P, G, N, W, dtype, act, seed = case
    print(f"case {name} bidir={bidir}", flush=True)
    ch = bm.conv_channels(H, P, G, N)
    f, b = synth.make_conv_inputs(batch, L, ch, W, dtype, seed, device=DEV, bidirectional=bidir)
    if name.endswith("noact"):
        f["bias"] = None
    fo, bo = bm.conv1d(f, b, H, P, G, N, activation=act)
    torch.cuda.synchronize()
    worst, ok = _check_dir(fo, f, False, (H, P, G, N), dtype, act)
    print(f"  forward excess {worst:.3f}", flush=True)
    assert ok, f"{name} forward: {worst:.3f} delta outside"
    if bidir:
        worst, ok = _check_dir(bo, b, True, (H, P, G, N), dtype, act)
        print(f"  reverse excess {worst:.3f}", flush=True)
        assert ok, f"{name} reverse: {worst:.3f} delta outside"
    else:
        assert bo is None


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_packed(dtype):
    lens = [5, 0, 1, 2, 70, 3, 0, 130, 1]
    cu = synth.cu_seqlens_of(lens)
    H, P, G, N = (4, 64, 1, 128) if dtype == "bf16" else (4, 16, 1, 16)
    ch = bm.conv_channels(H, P, G, N)
    f, b = synth.make_conv_inputs(1, cu[-1], ch, 4, dtype, 50, device=DEV)
    fo, bo = bm.conv1d(f, b, H, P, G, N, cu_seqlens=cu)
    torch.cuda.synchronize()
    for out, d, rev in ((fo, f, False), (bo, b, True)):
        worst, ok = _check_dir(out, d, rev, (H, P, G, N), dtype, "silu", cu=cu)
        assert ok, f"packed reverse={rev}: {worst:.3f} delta outside"


@pytest.mark.parametrize("L", [1, 2, 3, 40, 64, 200])
@pytest.mark.parametrize("inplace", [False, True], ids=["separate", "inplace"])
def test_conv_context(L, inplace):
    """init_ctx in, final_ctx out (bit for bit), updated in place or not."""
    H, P, G, N, W = 4, 64, 1, 128, 4
    ch = bm.conv_channels(H, P, G, N)
    batch = 3
    f, b = synth.make_conv_inputs(batch, L, ch, W, "bf16", 51 + L, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(52)
    init = torch.randn(batch, W - 1, ch, generator=g, device=DEV).to(torch.bfloat16)
    init_np = _np(init)
    final = init if inplace else torch.full_like(init, float("nan"))
    fo, bo = bm.conv1d(f, b, H, P, G, N, init_ctx=init, final_ctx=final)
    torch.cuda.synchronize()
    worst, ok = _check_dir(fo, f, False, (H, P, G, N), "bf16", "silu", init=init_np)
    assert ok, f"forward with context: {worst:.3f} delta outside"
    worst, ok = _check_dir(bo, b, True, (H, P, G, N), "bf16", "silu")
    assert ok, f"reverse: {worst:.3f} delta outside"
    _, ref_final = oconv.conv1d(f["xbc"], f["weight"], f["bias"], init_ctx=init_np,
                                want_final=True)
    assert np.array_equal(_np(final), ref_final), "final context differs"


@pytest.mark.parametrize("with_init", [False, True])
def test_conv_empty_row(with_init):
    H, P, G, N, W = 4, 16, 1, 16, 4
    ch = bm.conv_channels(H, P, G, N)
    f, _ = synth.make_conv_inputs(2, 0, ch, W, "bf16", 53, device=DEV, bidirectional=False)
    init = torch.randn(2, W - 1, ch, device=DEV).to(torch.bfloat16) if with_init else None
    final = torch.full((2, W - 1, ch), 7.0, device=DEV, dtype=torch.bfloat16)
    fo, _ = bm.conv1d(f, None, H, P, G, N, init_ctx=init, final_ctx=final)
    torch.cuda.synchronize()
    assert fo["x"].numel() == 0
    exp = init if with_init else torch.zeros_like(final)
    assert torch.equal(final, exp)


def test_conv_layer_full_size():
    """The benchmarked layer (8 x 1024 tokens, 4352 channels, bf16, width 4,
    both directions) in the launch the benchmark times, every element."""
    c = synth.CONV_LAYER
    H, P, G, N, W = c["nheads"], c["headdim"], c["ngroups"], c["d_state"], c["width"]
    ch = bm.conv_channels(H, P, G, N)
    print(f"layer conv {c['batch']}x{c['seqlen']}x{ch}", flush=True)
    f, b = synth.make_conv_inputs(c["batch"], c["seqlen"], ch, W, c["dtype"], c["seed"], device=DEV)
    fo, bo = bm.conv1d(f, b, H, P, G, N)
    torch.cuda.synchronize()
    for out, d, rev in ((fo, f, False), (bo, b, True)):
        worst, ok = _check_dir(out, d, rev, (H, P, G, N), "bf16", "silu")
        print(f"  reverse={rev} excess {worst:.3f}", flush=True)
        assert ok, f"layer conv reverse={rev}: {worst:.3f} delta outside"


def test_block_step_with_conv():
    """Cached block diffusion with the convolution in front of the scan: a
    prefix is filtered and scanned once (its forward conv context and SSM
    state are kept), then a block resumes from both; the result equals the
    oracle's convolution of the whole sequence (forward) and of the block
    alone (reverse), fed to the oracle's block step."""
    H, P, G, N, W = 4, 64, 1, 128, 4
    ch = bm.conv_channels(H, P, G, N)
    nseq, Lp, Lb = 2, 150, 64
    f, b = synth.make_conv_inputs(nseq, Lp + Lb, ch, W, "bf16", 54, device=DEV)
    ssd_f, ssd_b = synth.make_inputs(nseq, Lp + Lb, H, P, N, G, "bf16", 56, device=DEV)

    def part(d, lo, hi):
        return dict(xbc=d["xbc"][:, lo:hi].contiguous(), weight=d["weight"], bias=d["bias"])

    def ssd_part(d, lo, hi, conv_out):
        return dict(x=conv_out["x"], dt=d["dt"][:, lo:hi].contiguous(), A=d["A"],
                    B=conv_out["B"], C=conv_out["C"], D=d["D"])

    # prefix: forward conv (keeping its context) and forward scan (keeping its state)
    ctx = torch.zeros(nseq, W - 1, ch, device=DEV, dtype=torch.bfloat16)
    pf, _ = bm.conv1d(part(f, 0, Lp), None, H, P, G, N, init_ctx=ctx, final_ctx=ctx)
    st = bm.State(nseq, H, P, N)
    bm.ssd_fwd(ssd_part(ssd_f, 0, Lp, pf), None, chunk=64, init_state=st.tensor(),
               final_state=st.tensor())
    # the block: both directions from the carried context / state
    bf_, bb_ = bm.conv1d(part(f, Lp, Lp + Lb), part(b, Lp, Lp + Lb), H, P, G, N,
                         init_ctx=ctx, final_ctx=ctx)
    y = bm.block_step(st, ssd_part(ssd_f, Lp, Lp + Lb, bf_), ssd_part(ssd_b, Lp, Lp + Lb, bb_),
                      commit=True, chunk=64)
    torch.cuda.synchronize()

    # oracle: forward conv over the whole sequence, reverse conv over the block alone
    whole = oconv.conv1d(f["xbc"], f["weight"], f["bias"])
    blk_rev = oconv.conv1d(part(b, Lp, Lp + Lb)["xbc"], b["weight"], b["bias"], reverse=True)
    # the scan reads the kernel's own bf16 conv outputs; those are checked
    # against the oracle here, then fed to the scan oracle as they are
    got_f = np.concatenate([_np(bf_[k]).reshape(nseq, Lb, -1) for k in ("x", "B", "C")], axis=-1)
    worst, ok = conv_close(got_f, whole[:, Lp:], _scale(f, False)[:, Lp:], "bf16")
    assert ok, f"block forward conv: {worst:.3f} delta outside"
    got_b = np.concatenate([_np(bb_[k]).reshape(nseq, Lb, -1) for k in ("x", "B", "C")], axis=-1)
    worst, ok = conv_close(got_b, blk_rev, _scale(part(b, Lp, Lp + Lb), True), "bf16")
    assert ok, f"block reverse conv: {worst:.3f} delta outside"
    assert np.array_equal(_np(ctx), _np(f["xbc"][:, Lp + Lb - (W - 1):])), "carried context"

    _, st_ref = oracle.bissd(ssd_part(ssd_f, 0, Lp, pf), None, want_final_state=True)
    y_ref, st_new = oracle.block_step(st_ref, ssd_part(ssd_f, Lp, Lp + Lb, bf_),
                                      ssd_part(ssd_b, Lp, Lp + Lb, bb_), commit=True)
    err, ok = within(_np(y), y_ref, "bf16")
    assert ok, f"block step after conv: error {err:.3e}"
    err, ok = within(_np(st.tensor()), st_new, "bf16")
    assert ok, f"committed state: error {err:.3e}"


def test_block_step_conv_state():
    """The convolution's context carried in the state object
    (bimamba_state_alloc_conv, bimamba_block_step_conv): a prefix is filtered
    (into the state's context) and scanned (into its SSM state), then two
    committed blocks and one uncommitted block run from raw inputs. Outputs
    and committed states match the oracle's convolution of the whole
    sequence (forward) and of each block alone (reverse) fed to its block
    step; the context equals the last width-1 raw forward inputs, bit for
    bit; the uncommitted block changes neither the state nor the context."""
    H, P, G, N, W = 4, 64, 1, 128, 4
    ch = bm.conv_channels(H, P, G, N)
    nseq, Lp, Lb = 2, 150, 64
    L = Lp + 3 * Lb
    f, b = synth.make_conv_inputs(nseq, L, ch, W, "bf16", 57, device=DEV)
    ssd_f, ssd_b = synth.make_inputs(nseq, L, H, P, N, G, "bf16", 58, device=DEV)

    def part(d, lo, hi):
        return dict(xbc=d["xbc"][:, lo:hi].contiguous(), weight=d["weight"], bias=d["bias"])

    def scan_part(d, lo, hi, conv_out=None):
        out = dict(dt=d["dt"][:, lo:hi].contiguous(), A=d["A"], D=d["D"])
        if conv_out is not None:
            out.update(x=conv_out["x"], B=conv_out["B"], C=conv_out["C"])
        return out

    st = bm.State(nseq, H, P, N, conv=(G, W, torch.bfloat16))
    ctx = st.ctx_tensor()
    assert tuple(ctx.shape) == (nseq, W - 1, ch) and not bool(ctx.abs().sum())
    # prefix: filtered into the state's context, scanned into its SSM state
    pf, _ = bm.conv1d(part(f, 0, Lp), None, H, P, G, N, init_ctx=ctx, final_ctx=ctx)
    bm.ssd_fwd(scan_part(ssd_f, 0, Lp, pf), None, chunk=64, init_state=st.tensor(),
               final_state=st.tensor())
    torch.cuda.synchronize()
    _, st_ref = oracle.bissd(scan_part(ssd_f, 0, Lp, pf), None, want_final_state=True)

    whole = oconv.conv1d(f["xbc"], f["weight"], f["bias"])
    for k, commit in enumerate((True, True, False)):
        lo, hi = Lp + k * Lb, Lp + (k + 1) * Lb
        state_before = st.tensor().clone()
        ctx_before = ctx.clone()
        outs = ({}, {})
        for o in outs:
            o.update(x=torch.empty(nseq, Lb, H, P, dtype=torch.bfloat16, device=DEV),
                     B=torch.empty(nseq, Lb, G, N, dtype=torch.bfloat16, device=DEV),
                     C=torch.empty(nseq, Lb, G, N, dtype=torch.bfloat16, device=DEV))
        y = bm.block_step_conv(st, scan_part(ssd_f, lo, hi), scan_part(ssd_b, lo, hi),
                               part(f, lo, hi), part(b, lo, hi), commit=commit, chunk=64,
                               conv_out=outs)
        torch.cuda.synchronize()
        # the filtered values: the forward filter continues the whole
        # sequence, the reverse one sees only the block
        got_f = np.concatenate([_np(outs[0][n]).reshape(nseq, Lb, -1) for n in ("x", "B", "C")], axis=-1)
        worst, ok = conv_close(got_f, whole[:, lo:hi], _scale(f, False)[:, lo:hi], "bf16")
        assert ok, f"block {k}: forward conv {worst:.3f} delta outside"
        blk_rev = oconv.conv1d(part(b, lo, hi)["xbc"], b["weight"], b["bias"], reverse=True)
        got_b = np.concatenate([_np(outs[1][n]).reshape(nseq, Lb, -1) for n in ("x", "B", "C")], axis=-1)
        worst, ok = conv_close(got_b, blk_rev, _scale(part(b, lo, hi), True), "bf16")
        assert ok, f"block {k}: reverse conv {worst:.3f} delta outside"
        y_ref, st_next = oracle.block_step(st_ref, scan_part(ssd_f, lo, hi, outs[0]),
                                           scan_part(ssd_b, lo, hi, outs[1]), commit=commit)
        err, ok = within(_np(y), y_ref, "bf16")
        print(f"block {k} (commit={commit}): y {err:.3e}", flush=True)
        assert ok, f"block {k}: y error {err:.3e}"
        if commit:
            err, ok = within(_np(st.tensor()), st_next, "bf16")
            assert ok, f"block {k}: committed state error {err:.3e}"
            assert torch.equal(ctx, f["xbc"][:, hi - (W - 1):hi]), f"block {k}: carried context"
            st_ref = st_next
        else:
            assert torch.equal(st.tensor(), state_before), "uncommitted block changed the state"
            assert torch.equal(ctx, ctx_before), "uncommitted block changed the context"
    # reset zeroes both
    st.reset([1])
    torch.cuda.synchronize()
    assert not bool(ctx[1].float().abs().sum()) and not bool(st.tensor()[1].abs().sum())
    assert bool(ctx[0].float().abs().sum())
    st.free()


def _random_conv_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        H = int(rng.integers(1, 9))
        P = int(rng.choice([3, 4, 8, 16, 64]))
        G = int(rng.choice([1, 2]))
        N = int(rng.choice([4, 5, 16, 128]))
        cases.append(dict(k=k, H=H, P=P, G=G, N=N, W=int(rng.integers(2, 5)),
                          dtype=["bf16", "f32"][k % 2], act=["silu", "none"][k % 3 == 2],
                          batch=int(rng.integers(1, 4)),
                          L=int(rng.choice([1, 2, 15, 16, 17, 64, 65, 100, 257])),
                          bidir=k % 4 != 1, seed=3000 + k))
    return cases


@pytest.mark.parametrize("case", _random_conv_cases(20, 93), ids=lambda c: f"r{c['k']}")
def test_conv_random_shapes(case):
    c = case
    print(f"random case {c}", flush=True)
    ch = bm.conv_channels(c["H"], c["P"], c["G"], c["N"])
    f, b = synth.make_conv_inputs(c["batch"], c["L"], ch, c["W"], c["dtype"], c["seed"],
                                  device=DEV, bidirectional=c["bidir"])
    fo, bo = bm.conv1d(f, b, c["H"], c["P"], c["G"], c["N"], activation=c["act"])
    torch.cuda.synchronize()
    dims = (c["H"], c["P"], c["G"], c["N"])
    worst, ok = _check_dir(fo, f, False, dims, c["dtype"], c["act"])
    assert ok, f"forward: {worst:.3f} delta outside"
    if c["bidir"]:
        worst, ok = _check_dir(bo, b, True, dims, c["dtype"], c["act"])
        assert ok, f"reverse: {worst:.3f} delta outside"
