"""The GPU acceptance check's bf16 floor: half the bf16 spacing at a value
bounds the error of rounding that value to bf16 (checked against torch's
conversion), and is attained at the midpoint of two neighbours."""
import numpy as np
import torch

from tests.harness import bf16_half_ulp, within_tol


def test_half_spacing_bounds_bf16_rounding():
    rng = np.random.default_rng(5)
    # fp32-exact values: fp32 -> bf16 is one round-to-nearest-even
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, size=200000))).astype(np.float32)
    r = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    x = x.astype(np.float64)
    assert np.all(np.abs(r - x) <= bf16_half_ulp(x))
    # exact values: spacing 2^-7 on [1, 2), 2^-6 on [2, 4)
    assert bf16_half_ulp(np.array([1.0, 1.999, 2.0, 3.5, -2.0853]))[0] == 2.0 ** -8
    assert list(bf16_half_ulp(np.array([1.999, 2.0, 3.5, -2.0853]))) == [2.0 ** -8, 2.0 ** -7, 2.0 ** -7, 2.0 ** -7]
    mid = 1.0 + 2.0 ** -8  # halfway between 1 and its bf16 successor
    r = torch.tensor([mid], dtype=torch.float64).to(torch.bfloat16).double().item()
    assert abs(r - mid) == bf16_half_ulp(np.array([mid]))[0]


def test_within_tol_is_the_bar_plus_the_floor():
    ref = np.array([0.1, -0.2, 0.3, 2.0853])
    bound = 2e-2 * np.sqrt(np.mean(ref ** 2))
    ok, err, b = within_tol(ref + bound * 0.99, ref)
    assert ok and abs(b - bound) < 1e-15
    # a small element's floor is small (2^-12 at 0.1): 5 % over the bar fails
    ok, _, _ = within_tol(ref + np.array([bound * 1.05, 0, 0, 0]), ref)
    assert not ok
    # the large element may miss by the bar plus half its spacing, no more
    ok, _, _ = within_tol(ref + np.array([0, 0, 0, bound + 2.0 ** -7 * 0.99]), ref)
    assert ok
    ok, _, _ = within_tol(ref + np.array([0, 0, 0, bound + 2.0 ** -7 * 1.01]), ref)
    assert not ok
    ok, _, _ = within_tol(np.array([np.nan, 0, 0, 0]), ref)
    assert not ok
