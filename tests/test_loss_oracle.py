"""Pins for the CPU oracle of the in-place masked softmax-loss gradient.

* a hand-derived fixture of the review's formulas (tests/golden/loss_grad_hand.txt);
* torch's cross entropy with probability targets (a library routine) and its autograd;
* central finite differences of sum_n g_n L_n;
* closed forms and invariants: one-hot targets, shift invariance, zero row sums, masked rows.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from masked_attention_eagle_amd import inputs
from oracle import loss_oracle as LO

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(tok):
    """A fixture token: an exact fraction, 'lnX', or a sum/difference like 'ln4-ln3/2'."""
    tok = tok.strip()
    if "ln" in tok:
        total, sign, i = 0.0, 1.0, 0
        for part in tok.replace("-", " -").split():
            neg = part.startswith("-")
            part = part.lstrip("-")
            assert part.startswith("ln")
            arg = part[2:]
            if "/" in arg:
                a, d = arg.split("/")
                val = math.log(float(a)) / float(d)
            else:
                val = math.log(float(arg))
            total += -val if neg else val
        return total
    return float(Fraction(tok))


def _rows():
    with open(os.path.join(GOLDEN, "loss_grad_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            z, p, g, L, gr = (x.split() for x in line.split("|"))
            yield (np.array([_num(t) for t in z]), np.array([_num(t) for t in p]),
                   _num(g[0]), _num(L[0]), np.array([_num(t) for t in gr]))


def test_hand_fixture():
    n = 0
    for z, p, g, L, gr in _rows():
        l, grad = LO.loss_and_grad(z[None], p[None], np.array([g]))
        assert abs(l[0] - L) < 1e-14, (z, l, L)
        np.testing.assert_allclose(grad[0], gr, atol=1e-14)
        n += 1
    assert n == 4


def _rand_case(seed, N=7, V=13):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((N, V)) * 3
    p = rng.gamma(0.3, size=(N, V))
    p /= p.sum(axis=1, keepdims=True)
    p *= rng.uniform(0.5, 1.0, size=(N, 1))  # targets that do not sum to one
    g = rng.uniform(-1, 2, size=N)
    g[0] = 0.0
    return z, p, g


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_against_torch_cross_entropy_and_autograd(seed):
    z, p, g = _rand_case(seed)
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    pt = torch.tensor(p, dtype=torch.float64)
    Lt = torch.nn.functional.cross_entropy(zt, pt, reduction="none")
    (Lt * torch.tensor(g, dtype=torch.float64)).sum().backward()
    L, grad = LO.loss_and_grad(z, p, g)
    np.testing.assert_allclose(L, Lt.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(grad, zt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_finite_differences():
    z, p, g = _rand_case(5, N=3, V=6)
    f = lambda zz: float((LO.loss_rows(zz, p) * g).sum())
    num = np.zeros_like(z)
    h = 1e-6
    for idx in np.ndindex(*z.shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += h
        zm[idx] -= h
        num[idx] = (f(zp) - f(zm)) / (2 * h)
    np.testing.assert_allclose(LO.grad_inplace(z, p, g), num, rtol=1e-6, atol=1e-8)


def test_one_hot_closed_form():
    rng = np.random.default_rng(9)
    z = rng.standard_normal((5, 11))
    y = rng.integers(0, 11, size=5)
    p = np.eye(11)[y]
    g = rng.uniform(0.1, 1, size=5)
    L, grad = LO.loss_and_grad(z, p, g)
    lse = np.log(np.exp(z).sum(axis=1))
    np.testing.assert_allclose(L, lse - z[np.arange(5), y], rtol=1e-13)
    pi = np.exp(z - lse[:, None])
    np.testing.assert_allclose(grad, g[:, None] * (pi - p), atol=1e-14)


def test_invariants():
    z, p, g = _rand_case(3)
    L, grad = LO.loss_and_grad(z, p, g)
    c = np.arange(z.shape[0])[:, None] * 7.5 - 20  # a different constant per row
    L2, grad2 = LO.loss_and_grad(z + c, p, g)
    np.testing.assert_allclose(L2, L, rtol=1e-12)
    np.testing.assert_allclose(grad2, grad, atol=1e-14)
    np.testing.assert_allclose(grad.sum(axis=1), 0.0, atol=1e-14)   # sum_i pi_i = 1
    assert not grad[0].any()                                      # masked row (g = 0)
    # large logits do not overflow
    Lb, gb = LO.loss_and_grad(z * 1e3, p, g)
    assert np.isfinite(Lb).all() and np.isfinite(gb).all()


def test_generated_workload_shapes():
    z, p, g = inputs.loss_case(4, 16, 256, "bf16")
    assert z.shape == p.shape == (16, 256) and g.shape == (16,)
    assert (p >= 0).all() and np.allclose(p.sum(axis=1), 1.0, atol=0.05)
    assert (g == 0).any() and np.isclose(g.sum(), 1.0)
    np.testing.assert_array_equal(inputs.round_to_bf16(z), z)
