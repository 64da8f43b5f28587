"""Pins for the oracle's RMSNorm (the pre-pass ahead of gemm1).

Each pin is a value the definition fixes without re-evaluating its formula:

* a constant row c with eps = 0 normalises to sign(c) * w exactly, whatever
  c and H (catches a missing square root, a divisor other than H, the weight
  applied before the scale);
* a constant row c with eps = 3c^2 gives sign(c) * w / 2 (eps sits inside
  the root, added to the mean of squares, not to the sum);
* a row with H/4 entries c and the rest 0 gives 2 sign(c) w on the non-zero
  entries (the mean runs over all H entries, zeros included);
* scaling a row by 2^k with eps = 0 leaves every output bit unchanged;
* exact rational arithmetic (fractions, with a 40-digit square root) on small
  random rows agrees with the oracle's double result to 1e-15;
* permuting the columns of x and w permutes the output; a transposed x (last
  dim stride T) gives the same bits as the contiguous copy.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import bits


def _bf16_bits(v):
    return bits(torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.bfloat16))


@pytest.mark.parametrize("c", [0.5, -3.0, 7.25, -1.0e-3, 96.0])
@pytest.mark.parametrize("H", [8, 64, 4096])
def test_constant_row_eps0_gives_sign_times_weight(orc, c, H):
    rng = np.random.default_rng(H)
    w = rng.uniform(0.0, 2.0, H)
    x = _bf16_bits(np.full((3, H), c))
    acc, out = orc.rmsnorm(x, w, 0.0)
    cb = float(torch.tensor(c).to(torch.bfloat16))
    want = np.sign(cb) * w
    assert np.allclose(acc, want, rtol=1e-15, atol=0)
    assert (out == _bf16_bits(want.astype(np.float32))[None, :]).all()


def test_eps_inside_the_root(orc):
    H = 64
    w = np.linspace(0.25, 4.0, H)
    x = _bf16_bits(np.full((2, H), 2.0))
    acc, _ = orc.rmsnorm(x, w, 12.0)          # 1 / sqrt(4 + 12) = 1/4
    assert np.array_equal(acc[0], w / 2.0)
    x = _bf16_bits(np.full((1, H), -2.0))
    acc, _ = orc.rmsnorm(x, w, 12.0)
    assert np.array_equal(acc[0], -w / 2.0)


def test_mean_runs_over_all_entries(orc):
    H = 256
    w = np.ones(H)
    row = np.zeros(H)
    row[::4] = 3.0                              # mean of squares 9/4, scale 2/3
    acc, _ = orc.rmsnorm(_bf16_bits(row[None, :]), w, 0.0)
    assert np.allclose(acc[0, ::4], 2.0, rtol=1e-15)
    assert (acc[0, 1::4] == 0).all()


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_scale_by_power_of_two_leaves_bits(orc, k):
    rng = np.random.default_rng(7)
    H = 512
    x = torch.randn(4, H, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    w = rng.uniform(0.0, 1.0, H)
    _, a = orc.rmsnorm(bits(x), w, 0.0)
    _, b = orc.rmsnorm(bits(x * (2.0 ** k)), w, 0.0)
    assert np.array_equal(a, b)


def test_exact_rational_brute_force(orc):
    getcontext().prec = 40
    rng = np.random.default_rng(11)
    H, T = 16, 5
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    w = rng.uniform(0.0, 1.0, H)
    eps = 1e-6
    acc, _ = orc.rmsnorm(bits(x), w, eps)
    xf = x.to(torch.float64).numpy()
    for t in range(T):
        ss = sum(Fraction(float(v)) ** 2 for v in xf[t])
        ms = ss / H + Fraction(eps)
        r = Decimal(1) / (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
        for h in range(H):
            exact = Decimal(float(xf[t, h])) * r * Decimal(float(w[h]))
            assert abs(Decimal(float(acc[t, h])) - exact) <= abs(exact) * Decimal("1e-15")


def test_column_permutation_and_transposed_layout(orc):
    rng = np.random.default_rng(2)
    T, H = 9, 128
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    w = rng.uniform(0.0, 1.0, H)
    _, out = orc.rmsnorm(bits(x), w, 1e-6)
    perm = rng.permutation(H)
    _, outp = orc.rmsnorm(bits(x[:, perm].contiguous()), w[perm], 1e-6)
    assert np.array_equal(outp, out[:, perm])
    xt = x.t().contiguous().t()                 # [T, H] with strides (1, T)
    assert xt.stride() == (1, T)
    _, outt = orc.rmsnorm(bits(xt), w, 1e-6)
    assert np.array_equal(outt, out)
