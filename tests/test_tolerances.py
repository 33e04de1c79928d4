"""CPU checks of the bf16 output bound the parity tests use for o (tests.helpers.o_bound)."""
import numpy as np

from masked_attention_eagle_amd.inputs import round_to_bf16
from tests.helpers import TOL_O, o_bound


def test_bound_is_the_stated_one_below_four():
    a = np.linspace(-3.999, 3.999, 10001)
    assert (o_bound(a) == TOL_O).all()
    # there the output rounding alone takes at most half of 2^-6: room is left for arithmetic
    r = np.abs(round_to_bf16(a.astype(np.float32)).astype(np.float64) - a)
    assert r.max() <= 2.0 ** -7


def test_bound_holds_the_output_rounding_from_four_on():
    rng = np.random.default_rng(7)
    a = np.exp(rng.uniform(np.log(4.0), np.log(64.0), 200000)) * rng.choice([-1.0, 1.0], 200000)
    r = np.abs(round_to_bf16(a.astype(np.float32)).astype(np.float64) - a)
    b = o_bound(a)
    # the rounding of the reference itself fits, with 2^-9 |ref| to spare for P's rounding
    # (through fp32 first, as the kernel's result: that step adds at most 2^-24 |ref|)
    assert (r <= b - np.abs(a) * 2.0 ** -9 + np.abs(a) * 2.0 ** -24).all()
    assert (b > TOL_O).all()
    # and the bound is not wider than that: half a step at the top of each binade
    assert np.isclose(o_bound(np.array([4.0]))[0], 2.0 ** -6 + 4 * 2.0 ** -9)
    assert np.isclose(o_bound(np.array([7.999]))[0], 2.0 ** -6 + 7.999 * 2.0 ** -9)
    assert np.isclose(o_bound(np.array([8.0]))[0], 2.0 ** -5 + 8 * 2.0 ** -9)
