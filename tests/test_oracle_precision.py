"""Pins for the oracle's storage rounding (CPU only)."""

import numpy as np
import torch

from oracle.precision import round_to


def test_bf16_matches_torch_on_fp32_values():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8), 2.0**-130]   # ties and a subnormal
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to(x.astype(np.float64), "bf16"), ref)


def test_bf16_is_nearest_representable_with_ties_to_even():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, size=20000))
    r = round_to(x, "bf16")
    bits = r.view(np.uint64)
    assert np.all(bits & np.uint64((1 << 45) - 1) == 0)           # bf16-representable
    e = np.floor(np.log2(np.abs(x)))
    ulp = np.exp2(e - 7)
    assert np.all(np.abs(x - r) <= ulp / 2)
    assert round_to(np.array([1.0 + 2.0**-8]), "bf16")[0] == 1.0                     # tie to even (down)
    assert round_to(np.array([1.0 + 3 * 2.0**-8]), "bf16")[0] == 1.0 + 2.0**-6      # tie to even (up)
    assert round_to(np.array([1.0 + 2.0**-8 + 2.0**-40]), "bf16")[0] == 1.0 + 2.0**-7


def test_f32_and_identity():
    x = np.array([1.0 + 2.0**-30, np.pi])
    assert np.array_equal(round_to(x, "f32"), x.astype(np.float32).astype(np.float64))
    assert np.array_equal(round_to(x, None), x)
