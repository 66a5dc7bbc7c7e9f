"""Order-independence of the Stage-0 block sums (the condition the pooling
kernels, the cache append and the oracle rely on to agree bit for bit).

A bf16 value has 8 significant bits; the sum of 64 of them needs at most 6
more bits of carry, so while a block's non-zero magnitudes lie within 2^39
of each other every partial sum fits the 53 bits of a double exactly and
the order of summation cannot change the result.  Checked against exact
rational arithmetic; outside the range a constructed case shows the order
does matter.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle


def _bf16_values(rng, n, lo_exp, hi_exp):
    """n random bf16-representable values with binary exponents in [lo_exp, hi_exp]."""
    mant = rng.integers(128, 256, size=n)  # 8 significant bits
    exps = rng.integers(lo_exp, hi_exp + 1, size=n)
    sign = rng.choice([-1.0, 1.0], size=n)
    return sign * np.ldexp(mant.astype(np.float64), exps - 7)


def _orders(x):
    """Sums of x in float64 in several orders: sequential, reversed, the
    lane-split order of the pooling kernel (16 partial sums then a butterfly),
    numpy's pairwise sum."""
    seq = 0.0
    for v in x:
        seq += v
    rev = 0.0
    for v in x[::-1]:
        rev += v
    parts = [0.0] * 16
    for i, v in enumerate(x):
        parts[i % 16] += v
    while len(parts) > 1:
        parts = [parts[i] + parts[i + len(parts) // 2] for i in range(len(parts) // 2)]
    return [seq, rev, parts[0], float(np.sum(x))]


@pytest.mark.parametrize("span", [0, 8, 20, 38])
def test_block_sum_exact_within_range(span):
    rng = np.random.default_rng(span)
    for trial in range(200):
        lo = int(rng.integers(-60, 40))
        x = _bf16_values(rng, 64, lo, lo + span)
        exact = sum((Fraction(v) for v in x), Fraction(0))
        sums = _orders(x)
        assert all(Fraction(s) == exact for s in sums), (span, trial)
        # the oracle's pooled mean is the exact mean rounded once
        k = x.reshape(64, 1)
        got = oracle.pool_blocks(k, 64, "bf16")[0, 0]
        want = oracle.round_bf16(np.float64(exact / 64))
        assert got == want


def test_block_sum_order_matters_outside_range():
    # magnitudes 2^60 apart: 2^60 + 1 - 2^60 in float64 depends on the order
    x = np.zeros(64)
    x[0], x[1], x[2] = 2.0 ** 60, 1.0, -(2.0 ** 60)
    sums = _orders(x)
    assert Fraction(sums[0]) != sum((Fraction(v) for v in x), Fraction(0))
    assert len(set(sums)) > 1
