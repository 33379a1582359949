"""Host checks of the GPU-parity comparators (no GPU): the bf16 unit in the last place and the
elementwise output tolerance built on it."""
import numpy as np
import pytest
import torch

from tests import _compare as cmp


def test_bf16_ulp_matches_torch_rounding_steps():
    # the gap from each bfloat16 value to the next one above it, from torch's own bf16 encoding
    xs = torch.tensor([0.3, 1.0, 1.99, 2.0, 3.7, 4.0, 4.1036, 7.9, 8.0, 100.0, 1e-3],
                      dtype=torch.bfloat16)
    nxt = (xs.view(torch.int16) + 1).view(torch.bfloat16)
    step = (nxt.double() - xs.double()).numpy()
    assert np.array_equal(cmp.bf16_ulp(xs.double().numpy()), step)
    assert np.array_equal(cmp.bf16_ulp(-xs.double().numpy()), step)


def test_bf16_ulp_closed_form():
    assert cmp.bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert cmp.bf16_ulp(np.array([4.1036]))[0] == 2.0 ** -5
    assert cmp.bf16_ulp(np.array([-3.99]))[0] == 2.0 ** -6
    assert cmp.bf16_ulp(np.array([0.3]))[0] == 2.0 ** -9


def test_output_tolerance_is_the_stated_bound_below_magnitude_four():
    ref = np.array([0.0, -1.5, 3.99, 4.0, -4.1036, 9.0])
    tol = cmp.out_tolerance(ref, "bf16")
    assert np.all(tol[:3] == 2e-2)
    assert tol[3] == 2.0 ** -5 and tol[4] == 2.0 ** -5 and tol[5] == 2.0 ** -4
    assert np.all(cmp.out_tolerance(ref, "f32") == 1e-4)
    # one bf16 step at magnitude >= 4 passes, two fail
    out = ref.copy()
    out[4] += 2.0 ** -5
    cmp.check_attention(out, np.zeros(1), ref, np.zeros(1), "bf16")
    out[4] += 2.0 ** -5
    with pytest.raises(AssertionError):
        cmp.check_attention(out, np.zeros(1), ref, np.zeros(1), "bf16")
