"""Seeded synthetic inputs for the bidirectional SSD.

This module holds the workload shapes and the input recipe only -- none of
the method's arithmetic. It is the one module that both the oracle side
(tests, CPU baseline) and the HIP side (tests, bench, smoke) draw inputs
from, so both sides see the very same tensors.

Recipe (per direction, drawn in this order: x, z, B, C; then A_fwd, A_bwd,
D_fwd, D_bwd):

* x ~ N(0, 1)
* dt = softplus(z - 2), z ~ N(0, 1)       (already positive, consumed as is)
* B, C ~ N(0, 1) / 4                      (N(0,1)/sqrt(16), kept at every d_state)
* A_h = -exp(U(0, ln 16))                 (A in [-16, -1])
* D_h ~ N(0, 1)

Half-precision workloads round x, dt, B and C to bf16 (round-to-nearest-
even, torch's conversion); A and D stay fp32. The generator is torch's
seeded generator on the target device, so large workloads are drawn on the
GPU; the oracle receives the exact drawn values after a host copy.
"""
import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    d_state: int
    ngroups: int
    chunk: int
    dtype: str                      # "f32" or "bf16"
    seed: int
    seqlens: Optional[tuple] = None  # packed lengths (then batch == 1)
    note: str = ""

    def tokens(self) -> int:
        return self.batch * self.seqlen


def packed_lengths(nseq: int, lo: int, hi: int, seed: int) -> List[int]:
    """Lengths uniform in [lo, hi] (inclusive), seeded."""
    g = torch.Generator().manual_seed(seed)
    return [int(v) for v in torch.randint(lo, hi + 1, (nseq,), generator=g)]


def _c4_lengths():
    return tuple(packed_lengths(32, 512, 8192, 5))


WORKLOADS = {
    # tiny fp32 parity case
    "tiny_f32": Workload("tiny_f32", 1, 256, 4, 16, 16, 1, 64, "f32", 0,
                         note="fp32, L=256, 4 heads x 16, d_state 16, chunk 64"),
    # one layer of a DiffuMamba-1.3B-shaped mixer at training length 1024
    "layer_1p3b_train": Workload("layer_1p3b_train", 8, 1024, 64, 64, 128, 1,
                                 256, "bf16", 1,
                                 note="d_inner 4096 = 64 heads x 64, d_state 128"),
    "long_32k": Workload("long_32k", 1, 32768, 64, 64, 128, 1, 256, "bf16", 2),
    "long_128k": Workload("long_128k", 1, 131072, 64, 64, 128, 1, 256, "bf16", 3),
    # the same length with the small head shape (token-sequential path)
    "long_128k_small_heads": Workload("long_128k_small_heads", 1, 131072, 4, 16, 16, 1, 256,
                                      "bf16", 3, note="4 heads x 16, d_state 16"),
    # packed variable-length batch with per-sequence resets
    "packed_varlen": Workload("packed_varlen", 1, 0, 64, 64, 128, 1, 256,
                              "bf16", 5, seqlens=None),
}


def packed_workload():
    lens = _c4_lengths()
    return Workload("packed_varlen", 1, sum(lens), 64, 64, 128, 1, 256, "bf16",
                    5, seqlens=lens)


# block-cached decode step: 80 heads x 64 (d_inner 5120), d_state 128, block 64
BLOCK_STEP = dict(nheads=80, headdim=64, d_state=128, ngroups=1, block=64,
                  prefix=262144, seed=4)


def _dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def draw_direction(g, batch, L, H, P, N, G, dtype, device):
    """x, dt, B, C of one direction, drawn in that order."""
    dt_ = _dtype(dtype)
    x = torch.randn(batch, L, H, P, generator=g, device=device).to(dt_)
    z = torch.randn(batch, L, H, generator=g, device=device)
    dt = torch.nn.functional.softplus(z - 2.0).to(dt_)
    B = (torch.randn(batch, L, G, N, generator=g, device=device) / 4.0).to(dt_)
    C = (torch.randn(batch, L, G, N, generator=g, device=device) / 4.0).to(dt_)
    return dict(x=x.contiguous(), dt=dt.contiguous(), B=B.contiguous(),
                C=C.contiguous())


def draw_head_params(g, H, device):
    u = torch.rand(H, generator=g, device=device)
    A = -torch.exp(u * math.log(16.0))
    D = torch.randn(H, generator=g, device=device)
    return A.float().contiguous(), D.float().contiguous()


def make_inputs(batch, L, H, P, N, G, dtype, seed, device="cpu",
                bidirectional=True):
    """Returns (fwd, bwd) dicts with x, dt, A, B, C, D (bwd None if not wanted)."""
    g = torch.Generator(device=device).manual_seed(seed)
    fwd = draw_direction(g, batch, L, H, P, N, G, dtype, device)
    bwd = draw_direction(g, batch, L, H, P, N, G, dtype, device) if bidirectional else None
    Af, Df = draw_head_params(g, H, device)
    fwd["A"], fwd["D"] = Af, Df
    if bwd is not None:
        Ab, Db = draw_head_params(g, H, device)
        bwd["A"], bwd["D"] = Ab, Db
    return fwd, bwd


# Short convolution in front of the scan (d_conv = 4 over the x | B | C
# channels): the layer workload's channels, 64 x 64 + 2 x 128 = 4352.
CONV_LAYER = dict(batch=8, seqlen=1024, nheads=64, headdim=64, ngroups=1,
                  d_state=128, width=4, dtype="bf16", seed=6)


def draw_conv_direction(g, batch, L, ch, width, dtype, device):
    """One direction's convolution inputs, drawn in this order: the pre-
    convolution activations xbc ~ N(0, 1) (rounded to the workload dtype),
    then weight and bias ~ U(-1/sqrt(W), 1/sqrt(W)) (the default initial
    range of a depthwise Conv1d of width W), fp32."""
    bound = 1.0 / math.sqrt(width)
    xbc = torch.randn(batch, L, ch, generator=g, device=device).to(_dtype(dtype))
    weight = (torch.rand(ch, width, generator=g, device=device) * 2 - 1) * bound
    bias = (torch.rand(ch, generator=g, device=device) * 2 - 1) * bound
    return dict(xbc=xbc.contiguous(), weight=weight.float().contiguous(),
                bias=bias.float().contiguous())


def make_conv_inputs(batch, L, ch, width, dtype, seed, device="cpu",
                     bidirectional=True):
    """Returns (fwd, bwd) convolution inputs (bwd None if not wanted)."""
    g = torch.Generator(device=device).manual_seed(seed)
    fwd = draw_conv_direction(g, batch, L, ch, width, dtype, device)
    bwd = draw_conv_direction(g, batch, L, ch, width, dtype, device) if bidirectional else None
    return fwd, bwd


def make_epilogue_inputs(rows, C, dtype, seed, device="cpu"):
    """Inputs of the gated-norm epilogue, drawn in this order: the scan's
    output y ~ N(0, 1) (fp32), the gate branch z ~ N(0, 1) (rounded to the
    workload dtype), the per-channel weight ~ U(0.5, 1.5) (fp32)."""
    g = torch.Generator(device=device).manual_seed(seed)
    y = torch.randn(rows, C, generator=g, device=device)
    z = torch.randn(rows, C, generator=g, device=device).to(_dtype(dtype))
    w = torch.rand(C, generator=g, device=device) + 0.5
    return y.contiguous(), z.contiguous(), w.float().contiguous()


def make_workload(w: Workload, device="cpu"):
    return make_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.d_state,
                       w.ngroups, w.dtype, w.seed, device)


def cu_seqlens_of(lengths):
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return cu
