"""Pins for the oracle's alpha-entmax (CPU only).

Every check compares the bisection in ``oracle.entmax`` with something other
than itself: a library routine (softmax), a closed form derived in this file
from the definition (sparsemax, the sort-based 1.5-entmax), brute force over
all supports, invariants of the definition, finite differences, and the
worked example printed on the DashAttention pages.
"""

import itertools
import json
import os

import numpy as np
import pytest
import scipy.special
from scipy.optimize import brentq

from oracle import entmax, entmax_jvp, entmax_threshold

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, n, scale=1.0):
    return np.random.default_rng(seed).normal(size=n) * scale


# --------------------------------------------------------------------- closed forms


def sparsemax_closed(z):
    """Sparsemax by sorting (Martins & Astudillo, 2016): k(z) = max{k : 1 + k z_(k) > sum_{j<=k} z_(j)}."""
    zs = np.sort(z)[::-1]
    cs = np.cumsum(zs)
    ks = np.arange(1, z.size + 1)
    k = ks[1 + ks * zs > cs].max()
    tau = (cs[k - 1] - 1.0) / k
    return np.maximum(z - tau, 0.0), tau


def entmax15_sort(z):
    """Exact 1.5-entmax by sorting (Peters, Niculae & Martins, 2019).

    With u = z/2 sorted decreasingly, a support of the top k gives the
    quadratic sum_{j<=k} (u_j - t)^2 = 1, whose smaller root is
    t_k = mean_k - sqrt((1 - k var_k) / k); the support size is the largest
    k with t_k <= u_(k).
    """
    u = np.sort(z / 2.0)[::-1]
    best = None
    for k in range(1, u.size + 1):
        top = u[:k]
        mean = top.mean()
        var = ((top - mean) ** 2).mean()
        disc = 1.0 - k * var
        if disc < 0:
            continue
        t = mean - np.sqrt(disc / k)
        if t <= u[k - 1]:
            best = t
    p = np.maximum(z / 2.0 - best, 0.0) ** 2
    return p, best


@pytest.mark.parametrize("seed,n,scale", [(0, 1, 1.0), (1, 5, 1.0), (2, 37, 3.0), (3, 256, 0.3), (4, 1000, 5.0)])
def test_alpha1_is_softmax(seed, n, scale):
    z = _rand(seed, n, scale)
    p, tau, sup = entmax(z, 1.0)
    np.testing.assert_allclose(p, scipy.special.softmax(z), rtol=0, atol=1e-12)
    assert abs(tau - scipy.special.logsumexp(z)) < 1e-12 * max(1.0, abs(tau))
    assert sup.all()


@pytest.mark.parametrize("seed,n,scale", [(0, 2, 1.0), (1, 8, 1.0), (2, 64, 2.0), (3, 300, 0.5), (5, 1535, 4.0)])
def test_alpha2_is_sparsemax(seed, n, scale):
    z = _rand(seed, n, scale)
    p, tau, sup = entmax(z, 2.0)
    pc, tc = sparsemax_closed(z)
    np.testing.assert_allclose(p, pc, rtol=0, atol=1e-12)
    assert abs(tau - tc) < 1e-12
    np.testing.assert_array_equal(sup, pc > 0)


@pytest.mark.parametrize("seed,n,scale", [(0, 3, 1.0), (1, 16, 2.0), (2, 128, 1.0), (3, 777, 3.0), (6, 1024, 0.2)])
def test_alpha15_matches_sort_based(seed, n, scale):
    z = _rand(seed, n, scale)
    p, tau, sup = entmax(z, 1.5)
    pc, tc = entmax15_sort(z)
    np.testing.assert_allclose(p, pc, rtol=0, atol=1e-12)
    assert abs(tau - tc) < 1e-12
    np.testing.assert_array_equal(sup, pc > 0)


def _brute_force_support(u, alpha):
    """All supports S whose exact threshold t_S is self-consistent.

    For each non-empty S, t_S solves sum_{b in S} (u_b - t)^(1/(alpha-1)) = 1
    with t < min_S u (a 1-D root found by Brent's method); S is consistent
    when every u outside S is <= t_S.
    """
    m = 1.0 / (alpha - 1.0)
    n = u.size
    found = []
    for r in range(1, n + 1):
        for S in itertools.combinations(range(n), r):
            us = u[list(S)]
            lo, hi = us.min() - 2.0, us.min()
            g = lambda t: np.sum((us - t) ** m) - 1.0  # noqa: E731
            if g(lo) < 0 or g(hi) >= 0:
                continue  # no root below min_S u: S cannot be the support
            t = brentq(g, lo, hi, xtol=1e-15, rtol=1e-15)
            rest = np.delete(u, list(S))
            if rest.size == 0 or rest.max() <= t + 1e-12:
                found.append((set(S), t))
    return found


@pytest.mark.parametrize("alpha", [1.25, 1.5, 1.75, 2.0])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_supports(alpha, seed):
    n = 9
    z = _rand(100 + seed, n, 2.0)
    u = (alpha - 1.0) * z
    found = _brute_force_support(u, alpha)
    assert len(found) == 1, found
    S, t = found[0]
    p, tau, sup = entmax(z, alpha)
    assert set(np.flatnonzero(sup)) == S
    assert abs(tau - t) < 1e-10


@pytest.mark.parametrize("alpha", [1.0, 1.25, 1.5, 2.0])
def test_invariants(alpha):
    rng = np.random.default_rng(7)
    for n in [1, 2, 10, 255, 1535]:
        z = rng.normal(size=n) * 2.0
        p, tau, sup = entmax(z, alpha)
        assert abs(p.sum() - 1.0) < 1e-14
        assert (p >= 0).all()
        # exact zeros exactly where u <= tau
        if alpha > 1:
            u = (alpha - 1.0) * z
            np.testing.assert_array_equal(p > 0, u > tau)
            assert (p[u <= tau] == 0.0).all()
        # permutation equivariance
        perm = rng.permutation(n)
        pp, tp, _ = entmax(z[perm], alpha)
        np.testing.assert_allclose(pp, p[perm], atol=1e-14)
        # shift invariance
        ps, _, _ = entmax(z + 3.25, alpha)
        np.testing.assert_allclose(ps, p, atol=1e-12)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_one_hot_when_gap_at_least_one(alpha):
    z = np.array([0.3, -1.0, 0.1, -2.0])
    u_gap = 1.0 / (alpha - 1.0)  # a gap of 1 in u-units
    z[0] = z[2] + u_gap + 1e-9
    p, tau, sup = entmax(z, alpha)
    np.testing.assert_array_equal(p, [1.0, 0.0, 0.0, 0.0])
    assert sup.sum() == 1


def test_near_one_is_close_to_softmax():
    z = _rand(11, 50, 1.0)
    p, _, _ = entmax(z, 1.0 + 1e-4)
    np.testing.assert_allclose(p, scipy.special.softmax(z), atol=2e-3)


def test_worked_example_from_pages():
    d = json.load(open(os.path.join(GOLDEN, "entmax_worked_example.json")))
    z = np.array(d["scores"])
    ps, _, _ = entmax(z, 1.0)
    np.testing.assert_allclose(ps, d["expected"]["softmax"], atol=1e-12)
    p, tau, sup = entmax(z, d["alpha"])
    np.testing.assert_array_equal(p, d["expected"]["entmax15_p"])
    assert tau == d["expected"]["entmax15_tau"]
    # the pages' qualitative claim: the bottom two scores get exactly zero
    assert all(p[i] == 0.0 for i in d["expected"]["zero_indices"])


def test_threshold_rejects_bad_input():
    with pytest.raises(ValueError):
        entmax_threshold(np.zeros(0), 1.5)
    with pytest.raises(ValueError):
        entmax_threshold(np.zeros(3), 2.5)


# --------------------------------------------------------------------- Jacobian


def _fd_jacobian(z, alpha, h=1e-6):
    n = z.size
    J = np.zeros((n, n))
    for c in range(n):
        e = np.zeros(n)
        e[c] = h
        J[:, c] = (entmax(z + e, alpha)[0] - entmax(z - e, alpha)[0]) / (2 * h)
    return J


@pytest.mark.parametrize("alpha", [1.0, 1.25, 1.5, 2.0])
def test_jvp_matches_finite_differences(alpha):
    rng = np.random.default_rng(3)
    z = rng.normal(size=12) * 1.5
    p, tau, sup = entmax(z, alpha)
    if alpha > 1:
        u = (alpha - 1) * z
        assert np.min(np.abs(u - tau)) > 1e-4  # away from support changes
    J = _fd_jacobian(z, alpha)
    for _ in range(4):
        g = rng.normal(size=12)
        np.testing.assert_allclose(entmax_jvp(p, g, alpha), J.T @ g, atol=1e-7)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_jvp_structure(alpha):
    rng = np.random.default_rng(5)
    z = rng.normal(size=20) * 2.0
    p, tau, sup = entmax(z, alpha)
    n = z.size
    J = np.stack([entmax_jvp(p, np.eye(n)[b], alpha) for b in range(n)])  # rows: dz for g = e_b
    np.testing.assert_allclose(J, J.T, atol=1e-14)  # symmetric
    np.testing.assert_allclose(J.sum(axis=1), 0.0, atol=1e-14)  # sum_b dz_b = 0
    assert np.all(J[:, ~sup] == 0.0) and np.all(J[~sup, :] == 0.0)  # zero off the support
    if alpha == 2.0:
        one = sup.astype(float)
        np.testing.assert_allclose(J, np.diag(one) - np.outer(one, one) / one.sum(), atol=1e-14)
