"""GPU parity of the training backward (bimamba_ssd_bwd, through the C ABI)
against the oracle's adjoint recurrence (fp64), element by element, every
gradient of both streams."""
import numpy as np
import pytest
import torch

import bidirectional_mamba_ssm_amd as bm
import oracle
import synth
from metrics import rel_err_f32, rms_err

pytestmark = pytest.mark.gpu

DEV = "cuda"
KEYS = ("x", "dt", "A", "B", "C", "D")
# fp32 arithmetic from exact inputs. A gradient element is a sum of many
# products of both signs (over the block, the carried state, and for dB and
# dC the heads of a group), so its rounding error follows the size of those
# products, not its own value, which cancellation can make arbitrarily
# small (one token with three heads: dB is C times a sum over heads that
# nearly cancels). The bar is therefore relative to S, the same gradient
# with every contribution taken positive -- the oracle's adjoint on |x|,
# |dy|, |B|, |C|, |D|, step sizes and decays being positive already -- for
# dx, dB, dC, dA and dD: |g - g_ref| <= 1e-5 * S elementwise (fp32 sums
# of up to a few thousand terms, tree- and matrix-core-accumulated, stay
# well inside). ddt mixes a term of each sign by construction (A < 0), so
# S does not bound it; it is held to max|g - g_ref| <= 1e-4 * RMS(g_ref).
# The elementwise relative error with the 1 %-of-RMS floor is printed.
TOL = 1e-4
TOL_SUM = 1e-5


def _dy(batch, L, H, P, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(batch, L, H, P, generator=g, device=DEV)


def _abs_scale(f, b, dy):
    """Gradients with every contribution positive (bounds for all but ddt)."""
    def ab(d):
        if d is None:
            return None
        e = dict(d)
        for k in ("x", "B", "C", "D"):
            if e.get(k) is not None:
                e[k] = e[k].abs()
        return e
    return oracle.bissd_bwd(ab(f), ab(b), dy.abs())


def _compare(gpu, ref, tag, scale=None):
    worst, elem = {}, {}
    for k in KEYS:
        if gpu.get(k) is None:
            continue
        got = gpu[k].double().cpu().numpy()
        elem[k] = rel_err_f32(got, ref[k])
        if k != "dt" and scale is not None:
            # |err| / S against TOL_SUM
            worst[k] = (float(np.max(np.abs(got - ref[k]) / np.maximum(scale[k], 1e-300),
                                     initial=0.0)), TOL_SUM)
            continue
        err = rms_err(got, ref[k]) if np.any(ref[k]) else float(np.max(np.abs(got), initial=0.0))
        worst[k] = (err, TOL)
    print(f"  {tag}: max|err|/S (dt: /RMS) " + ", ".join(f"{k} {v[0]:.2e}" for k, v in worst.items()) +
          " | elementwise " + ", ".join(f"{k} {v:.1e}" for k, v in elem.items()), flush=True)
    bad = {k: v[0] for k, v in worst.items() if not v[0] <= v[1]}
    assert not bad, f"{tag}: {bad}"


CASES = [
    # name, batch, L, H, P, N, G, dtype, seed
    ("f32_tiny_ragged", 1, 130, 4, 16, 16, 1, "f32", 70),
    ("f32_groups_one_block", 2, 64, 4, 16, 128, 2, "f32", 71),
    ("f32_p64_n16", 1, 200, 2, 64, 16, 1, "f32", 72),
    ("bf16_layer_slice", 2, 300, 4, 64, 128, 1, "bf16", 73),
    ("bf16_short", 3, 5, 2, 64, 128, 1, "bf16", 74),
    ("bf16_L1", 2, 1, 2, 16, 16, 1, "bf16", 75),
    ("bf16_groups", 1, 257, 8, 64, 128, 4, "bf16", 76),
    # more than 16 blocks and fewer than 512 (row, stream, head) units: the
    # block-parallel state kernel and the pass over its output
    ("bf16_state_pass", 1, 1100, 2, 64, 128, 1, "bf16", 89),
    ("f32_state_pass", 2, 1090, 2, 16, 16, 1, "f32", 90),
    # 512 units and 21 blocks: the chained kernel over a longer walk
    ("f32_long_chain", 2, 1300, 128, 16, 16, 1, "f32", 92),
    ("bf16_long_chain_groups", 1, 1350, 256, 16, 128, 2, "bf16", 93),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("bidir", [True, False], ids=["bi", "fwd"])
def test_bwd_parity(case, bidir):
    name, batch, L, H, P, N, G, dtype, seed = case
    print(f"case {name} bidir={bidir}", flush=True)
    f, b = synth.make_inputs(batch, L, H, P, N, G, dtype, seed, device=DEV)
    if not bidir:
        b = None
    dy = _dy(batch, L, H, P, seed + 1000)
    gf, gb = bm.ssd_bwd(f, b, dy)
    torch.cuda.synchronize()
    rf, rb = oracle.bissd_bwd(f, b, dy)
    sf, sb = _abs_scale(f, b, dy)
    _compare(gf, rf, "forward stream", sf)
    if bidir:
        _compare(gb, rb, "reverse stream", sb)
    else:
        assert gb is None


def test_bwd_without_D():
    f, b = synth.make_inputs(1, 100, 2, 16, 16, 1, "f32", 77, device=DEV)
    f["D"] = None
    b["D"] = None
    dy = _dy(1, 100, 2, 16, 78)
    gf, gb = bm.ssd_bwd(f, b, dy)
    torch.cuda.synchronize()
    rf, rb = oracle.bissd_bwd(f, b, dy)
    sf, sb = _abs_scale(f, b, dy)
    _compare(gf, rf, "forward stream", sf)
    _compare(gb, rb, "reverse stream", sb)


def test_bwd_empty():
    f, b = synth.make_inputs(2, 0, 2, 16, 16, 1, "bf16", 79, device=DEV)
    dy = torch.empty(2, 0, 2, 16, device=DEV)
    gf, gb = bm.ssd_bwd(f, b, dy)
    torch.cuda.synchronize()
    for g in (gf, gb):
        assert torch.count_nonzero(g["A"]) == 0 and torch.count_nonzero(g["D"]) == 0


def test_bwd_deterministic():
    f, b = synth.make_inputs(2, 200, 4, 64, 128, 1, "bf16", 80, device=DEV)
    dy = _dy(2, 200, 4, 64, 81)
    g1 = bm.ssd_bwd(f, b, dy)
    g2 = bm.ssd_bwd(f, b, dy)
    torch.cuda.synchronize()
    for a, c in zip(g1, g2):
        for k in KEYS:
            assert torch.equal(a[k], c[k]), k


def test_bwd_layer_full_size():
    """The training layer (8 x 1024 tokens, 64 heads x 64, d_state 128, bf16,
    both streams) in the launch the benchmark times, every gradient element
    against the oracle."""
    w = synth.WORKLOADS["layer_1p3b_train"]
    f, b = synth.make_workload(w, device=DEV)
    dy = _dy(w.batch, w.seqlen, w.nheads, w.headdim, 82)
    print("layer backward", flush=True)
    gf, gb = bm.ssd_bwd(f, b, dy)
    torch.cuda.synchronize()
    rf, rb = oracle.bissd_bwd(f, b, dy)
    sf, sb = _abs_scale(f, b, dy)
    _compare(gf, rf, "forward stream", sf)
    _compare(gb, rb, "reverse stream", sb)


def _random_bwd_cases(n, seed):
    """Seeded random backward problems: both supported head shapes, lengths
    with ragged last blocks, grouped heads, one or both streams, D or not."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        P, N = [(64, 128), (16, 16), (64, 16), (16, 128)][k % 4]
        G = int(rng.choice([1, 2]))
        H = G * int(rng.integers(1, 4))
        cases.append(dict(k=k, dtype=["bf16", "f32"][k % 2], P=P, N=N, G=G, H=H,
                          batch=int(rng.integers(1, 3)),
                          L=int(rng.choice([1, 3, 63, 64, 65, 129, 200, 333])),
                          bidir=k % 3 != 2, with_D=k % 4 != 3, seed=2000 + k))
    return cases


@pytest.mark.parametrize("case", _random_bwd_cases(16, 91), ids=lambda c: f"r{c['k']}")
def test_bwd_random_shapes(case):
    c = case
    print(f"random case {c}", flush=True)
    f, b = synth.make_inputs(c["batch"], c["L"], c["H"], c["P"], c["N"], c["G"], c["dtype"],
                             c["seed"], device=DEV)
    if not c["with_D"]:
        f["D"] = None
        b["D"] = None
    if not c["bidir"]:
        b = None
    dy = _dy(c["batch"], c["L"], c["H"], c["P"], c["seed"] + 1)
    gf, gb = bm.ssd_bwd(f, b, dy)
    torch.cuda.synchronize()
    rf, rb = oracle.bissd_bwd(f, b, dy)
    sf, sb = _abs_scale(f, b, dy)
    _compare(gf, rf, "forward stream", sf)
    if b is not None:
        _compare(gb, rb, "reverse stream", sb)


# Shapes with at least 256 (block, row, stream) workgroups take the gradient
# kernel that walks the heads of each group and sums dB, dC over them in
# place; smaller ones keep one workgroup per head and a separate head sum.
HEAD_LOOP_CASES = [
    # name, batch, L, H, P, N, G, dtype, bidir, seed
    ("bf16_groups_ragged_bi", 8, 1000, 4, 64, 128, 2, "bf16", True, 83),
    ("f32_ragged_fwd_only", 16, 1001, 3, 16, 16, 1, "f32", False, 84),
    ("bf16_small_state_fwd_only", 16, 1024, 2, 64, 16, 1, "bf16", False, 87),
    ("f32_p16_n128_bi", 8, 999, 2, 16, 128, 2, "f32", True, 88),
]


@pytest.mark.parametrize("case", HEAD_LOOP_CASES, ids=[c[0] for c in HEAD_LOOP_CASES])
def test_bwd_head_loop(case):
    name, batch, L, H, P, N, G, dtype, bidir, seed = case
    print(f"head-loop case {name}", flush=True)
    f, b = synth.make_inputs(batch, L, H, P, N, G, dtype, seed, device=DEV)
    if not bidir:
        b = None
    dy = _dy(batch, L, H, P, seed + 1000)
    gf, gb = bm.ssd_bwd(f, b, dy)
    torch.cuda.synchronize()
    rf, rb = oracle.bissd_bwd(f, b, dy)
    sf, sb = _abs_scale(f, b, dy)
    _compare(gf, rf, "forward stream", sf)
    if bidir:
        _compare(gb, rb, "reverse stream", sb)


def test_bwd_head_loop_matches_per_head_form():
    """A batch that takes the head-walking gradient kernel against each row
    alone (too few workgroups: one per head and a separate head sum): the
    per-token gradients are the same numbers (both forms add the heads in
    order from zero)."""
    batch, L, H, P, N, G = 8, 1000, 4, 64, 128, 2
    f, b = synth.make_inputs(batch, L, H, P, N, G, "bf16", 85, device=DEV)
    dy = _dy(batch, L, H, P, 86)
    gf, gb = bm.ssd_bwd(f, b, dy)
    for r in (0, 5):
        fr = {k: (v[r:r + 1].contiguous() if v.dim() > 1 else v) for k, v in f.items()}
        br = {k: (v[r:r + 1].contiguous() if v.dim() > 1 else v) for k, v in b.items()}
        sf, sb = bm.ssd_bwd(fr, br, dy[r:r + 1].contiguous())
        torch.cuda.synchronize()
        for whole, one in ((gf, sf), (gb, sb)):
            for k in ("x", "dt", "B", "C"):
                assert torch.equal(whole[k][r:r + 1], one[k]), (r, k)
