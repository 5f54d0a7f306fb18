"""The Python binding's argument checks (CPU only: every rejection happens
before anything reaches the library or the GPU)."""
import pytest
import torch

import bidirectional_mamba_ssm_amd as bm


def _direction(batch=1, L=8, H=2, P=16, N=16, G=1, dtype=torch.float32, device="cpu"):
    return {"x": torch.zeros(batch, L, H, P, dtype=dtype, device=device),
            "dt": torch.zeros(batch, L, H, dtype=dtype, device=device),
            "A": torch.zeros(H, dtype=torch.float32, device=device),
            "B": torch.zeros(batch, L, G, N, dtype=dtype, device=device),
            "C": torch.zeros(batch, L, G, N, dtype=dtype, device=device),
            "D": torch.zeros(H, dtype=torch.float32, device=device)}


def test_host_tensors_rejected():
    with pytest.raises(ValueError, match="CUDA"):
        bm.ssd_fwd(_direction(), None, chunk=64)


def test_check_shape_dtype_layout():
    dev = torch.device("cpu")
    t = torch.zeros(2, 3)
    bm._check(t, "t", (2, 3), torch.float32, dev)
    with pytest.raises(ValueError, match="shape"):
        bm._check(t, "t", (3, 2), torch.float32, dev)
    with pytest.raises(TypeError, match="dtype"):
        bm._check(t, "t", (2, 3), torch.bfloat16, dev)
    with pytest.raises(ValueError, match="contiguous"):
        bm._check(t.t(), "t", (3, 2), torch.float32, dev)
    with pytest.raises(TypeError):
        bm._check([0.0], "t", (1,), torch.float32, dev)


def test_direction_accepted():
    d = _direction()
    bm._dir(d, torch.float32, bm._dims(d), torch.device("cpu"), "fwd")


@pytest.mark.parametrize("bad", ["dt", "B", "C", "A", "D"])
def test_direction_shapes_checked(bad):
    d = _direction()
    d[bad] = torch.zeros(*(s + 1 for s in d[bad].shape), dtype=d[bad].dtype)
    with pytest.raises(ValueError, match="shape"):
        bm._dir(d, torch.float32, bm._dims(_direction()), torch.device("cpu"), "fwd")


def test_direction_dtype_checked():
    d = _direction()
    d["dt"] = d["dt"].to(torch.bfloat16)
    with pytest.raises(TypeError, match="dtype"):
        bm._dir(d, torch.float32, bm._dims(d), torch.device("cpu"), "fwd")
