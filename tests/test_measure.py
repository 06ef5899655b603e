"""The parity measure itself: exact results rounded for storage score zero, and an error
of the size the bars guard against is reported."""
import numpy as np

import synth
from common import head_err, half_ulp


def test_rounding_alone_scores_zero_and_errors_are_seen():
    rng = np.random.default_rng(1)
    want = rng.standard_normal((2, 3, 500, 16)) * np.array([1.0, 30.0, 900.0])[None, :, None, None]
    bf = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(want.astype(np.float32)))
    assert head_err(bf, want, "bf16") == 0.0
    f32 = want.astype(np.float32)
    assert head_err(f32, want, "f32") == 0.0
    # without the half-ulp allowance the same bf16 rounding exceeds a 2e-2 bar on heavy-tailed data
    heavy = want * np.abs(rng.standard_normal(want.shape)) ** 3
    bfh = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(heavy.astype(np.float32)))
    rms = np.sqrt(np.mean(heavy[0, 0] ** 2))
    assert np.abs(bfh[0, 0] - heavy[0, 0]).max() / rms > 2e-2
    assert head_err(bfh, heavy, "bf16") == 0.0
    # a 3% error on one element of one head is caught
    bad = bf.copy()
    bad[1, 2, 7, 3] += 0.03 * np.sqrt(np.mean(want[1, 2] ** 2))
    assert head_err(bad, want, "bf16") > 2e-2


def test_half_ulp_values():
    assert half_ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -8
    assert half_ulp(np.array([1.99]), "bf16")[0] == 2.0 ** -8
    assert half_ulp(np.array([-3.0]), "bf16")[0] == 2.0 ** -7
    assert half_ulp(np.array([1.0]), "f32")[0] == 2.0 ** -24
    assert half_ulp(np.array([0.0]), "bf16")[0] == 0.0
