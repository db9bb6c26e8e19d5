"""The per-element bar on the bf16 output (msa_testlib.out_tolerance): it is
attainable by a correctly rounded bf16 output at every magnitude, it is the
plain 1e-2 absolute bar below |out| = 4, and it rejects a result two bf16
units away from the exact value (CPU)."""
import numpy as np
import torch

import msa_testlib as TL


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def test_ulp_at_known_points():
    x = np.array([1.0, 1.5, 2.0, 3.99, 4.0, 7.5, 0.25, -3.0])
    want = np.array([2.0**-7, 2.0**-7, 2.0**-6, 2.0**-6, 2.0**-5, 2.0**-5, 2.0**-9, 2.0**-6])
    np.testing.assert_array_equal(TL.bf16_ulp(x), want)
    # the spacing is the gap between consecutive bf16 numbers
    for v in (1.0, 2.0, 4.0, 0.25):
        nxt = torch.nextafter(torch.tensor(v, dtype=torch.bfloat16), torch.tensor(10.0, dtype=torch.bfloat16))
        assert float(nxt) - v == float(TL.bf16_ulp(v))


def test_round_to_nearest_always_passes():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-6, 6, size=200000))
    assert np.all(np.abs(_bf16(x) - x) <= TL.out_tolerance(x))


def test_plain_bar_below_four_and_one_unit_above():
    x = np.linspace(-3.999, 3.999, 8001)
    assert np.all(TL.out_tolerance(x) == 1e-2)
    assert float(TL.out_tolerance(5.0)) == 2.0**-5 and float(TL.out_tolerance(-4.0)) == 2.0**-5
    assert float(TL.out_tolerance(8.5)) == 2.0**-4


def test_plain_bar_on_two_to_four_rejects_one_unit():
    # on [2, 4) one bf16 unit (2^-6) exceeds the 1e-2 bar: a result one unit
    # away from a representable exact value fails there
    ref = np.array([[3.0, 0.0]])
    off = ref + np.array([[2.0**-6, 0.0]])
    lse = np.zeros((1, 2))
    try:
        TL.assert_out_lse(torch.from_numpy(off), torch.from_numpy(lse), ref, lse)
    except AssertionError:
        return
    raise AssertionError("an error of 2^-6 at |out| = 3 passed")


def test_two_units_off_fails():
    ref = np.array([[4.0106, 0.5, -2.3]])
    off = _bf16(ref) + np.array([[2 * 2.0**-5, 0.0, 0.0]])
    lse = np.zeros((1, 3))
    try:
        TL.assert_out_lse(torch.from_numpy(off), torch.from_numpy(lse), ref, lse)
    except AssertionError:
        pass
    else:
        raise AssertionError("a result two bf16 units off passed")
    TL.assert_out_lse(torch.from_numpy(_bf16(ref)), torch.from_numpy(lse), ref, lse)
    # 0.5 is held to the plain 1e-2 bar
    near = _bf16(ref).copy()
    near[0, 1] += 0.011
    try:
        TL.assert_out_lse(torch.from_numpy(near), torch.from_numpy(lse), ref, lse)
    except AssertionError:
        return
    raise AssertionError("an error of 0.011 at |out| = 0.5 passed")
