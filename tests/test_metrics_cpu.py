"""The test-side rounding helper against torch's own fp32 -> bf16 rounding."""
import numpy as np
import torch

from metrics import bf16_rne, conv_close


def test_bf16_rne_matches_torch():
    v = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 3
    # exact ties between two bf16 values, both parities
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.75 + 2 ** -9, 0.0],
                    dtype=np.float32)
    v = np.concatenate([v, ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_rne(v.astype(np.float64)), ref)


def test_conv_close_interval():
    ref = np.array([1.0 + 2 ** -9, 2.0, -0.5])
    scale = np.zeros(3)
    # bf16 spacing at 1 is 2^-7, so 1 + 2^-9 rounds to 1; with a tiny delta
    # only 1 is allowed
    assert conv_close(np.array([1.0, 2.0, -0.5]), ref, scale, "bf16", rel=2 ** -20)[1]
    assert not conv_close(np.array([1.0 + 2 ** -7, 2.0, -0.5]), ref, scale, "bf16", rel=2 ** -20)[1]
    # fp32: inside / outside the absolute bound
    assert conv_close(ref + 1e-7, ref, np.ones(3), "f32", rel=2 ** -18)[1]
    assert not conv_close(ref + 1e-5, ref, np.ones(3), "f32", rel=2 ** -18)[1]


def test_errors_of_an_all_zero_reference_are_finite():
    from metrics import rel_err_f32, rms_err
    z = np.zeros(8)
    assert rel_err_f32(z, z) == 0.0 and rms_err(z, z) == 0.0
    got = np.array([0.0, 1e-9, -2e-9, 0.0])
    assert rel_err_f32(got, np.zeros(4)) == 2e-9
    assert rms_err(got, np.zeros(4)) == 2e-9
