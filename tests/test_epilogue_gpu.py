"""GPU parity of the gated-norm epilogue (bimamba_gated_norm, through the C
ABI) against the fp64 oracle in oracle/epilogue.py, element by element:
bf16 outputs a correct rounding of the exact value up to the fp32
evaluation bound, fp32 outputs within it."""
import numpy as np
import pytest
import torch

import bidirectional_mamba_ssm_amd as bm
import synth
from metrics import conv_close
from oracle import epilogue as oepi

pytestmark = pytest.mark.gpu

DEV = "cuda"
# the kernel sums v^2 in fp32 over a short tree (4 per lane, 6 shuffle
# levels, then the group's 256-channel chunks): relative error of the mean
# square a few 2^-24, of the scale half that, plus the gate's and the
# products' few ulps; 2^-18 of |ref| bounds the value before rounding
REL = 2.0 ** -18


def _check(out, y, z, w, gs, eps, dtype):
    ref = oepi.gated_rmsnorm(y, z, w, gs, eps)
    got = out.double().cpu().numpy()
    worst, ok = conv_close(got, ref, np.zeros_like(ref), dtype, rel=REL)
    return worst, ok


CASES = [
    # name, rows, C, group_size, dtype, eps, seed
    ("bf16_layer_row", 64, 4096, 4096, "bf16", 1e-5, 100),
    ("bf16_groups", 33, 4096, 1024, "bf16", 1e-5, 101),
    ("bf16_small", 17, 256, 256, "bf16", 1e-6, 102),
    ("bf16_ragged_passes", 5, 1280, 256, "bf16", 1e-5, 103),
    ("f32_8192", 9, 8192, 2048, "f32", 1e-5, 104),
    ("f32_512", 12, 512, 512, "f32", 0.0, 105),
    ("bf16_5120", 7, 5120, 5120, "bf16", 1e-5, 106),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gated_norm_parity(case):
    name, rows, C, gs, dtype, eps, seed = case
    print(f"case {name}", flush=True)
    y, z, w = synth.make_epilogue_inputs(rows, C, dtype, seed, device=DEV)
    out = bm.gated_norm(y, z, w, group_size=gs, eps=eps)
    torch.cuda.synchronize()
    worst, ok = _check(out, y, z, w, gs, eps, dtype)
    print(f"  excess {worst:.3f}", flush=True)
    assert ok, f"{name}: {worst:.3f} delta outside"


def test_gated_norm_empty():
    y, z, w = synth.make_epilogue_inputs(0, 4096, "bf16", 107, device=DEV)
    out = bm.gated_norm(y, z, w)
    torch.cuda.synchronize()
    assert out.shape == (0, 4096)


def test_gated_norm_layer_full_size():
    """The training layer's epilogue: 8 x 1024 tokens, 4096 channels (64
    heads x 64), one group, bf16 gate and output; every element."""
    rows, C = 8 * 1024, 4096
    y, z, w = synth.make_epilogue_inputs(rows, C, "bf16", 108, device=DEV)
    out = bm.gated_norm(y, z, w)
    torch.cuda.synchronize()
    worst, ok = _check(out, y, z, w, C, 1e-5, "bf16")
    print(f"  layer excess {worst:.3f}", flush=True)
    assert ok, f"layer: {worst:.3f} delta outside"
