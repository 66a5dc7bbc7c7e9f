"""Pins for the oracle's backward (CPU only): central finite differences.

The loss is L = <dO, O>.  The oracle's analytic gradients (through Stage 2,
log p, the alpha-entmax Jacobian, the block scores and mean pooling) must
match central differences of its own float64 forward along random
directions.  Inputs are chosen away from support changes (every candidate
score is at least 1e-4 from tau in u-units), where the forward is smooth.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import Params


def _inputs(seed, T, D, causal, spread=1.5):
    rng = np.random.default_rng(seed)
    nb = T // 64
    k = rng.normal(size=(T, D))
    v = rng.normal(size=(T, D))
    kb = k.reshape(nb, 64, D).mean(axis=1)
    unit = kb / np.linalg.norm(kb, axis=1, keepdims=True)
    q = 0.5 * rng.normal(size=(T, D))
    for i in range(T):
        c = i // 64 if causal else nb
        if c:
            pick = rng.choice(c, size=min(c, rng.integers(1, 3)), replace=False)
            q[i] += spread * unit[pick].sum(axis=0)
    dout = rng.normal(size=(T, D))
    return [x[None, None] for x in (q, k, v, dout)]


def _loss(q, k, v, dout, prm):
    return float(np.sum(oracle.forward(q, k, v, prm)["o"] * dout))


def _min_gap(q, k, v, prm):
    """Smallest |u - tau| over all candidate scores (u-units)."""
    res = oracle.forward(q, k, v, prm)
    T = q.shape[2]
    gap = np.inf
    rows = oracle.forward_rows(q, k, v, prm, [(0, 0, i) for i in range(T)])
    for r in rows:
        if r["cand"].size == 0:
            continue
        u = (prm.alpha - 1.0) * r["z"]
        gap = min(gap, np.min(np.abs(u - r["tau"])))
    return gap, res


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("alpha", [1.0, 1.25, 1.5, 2.0])
def test_gradients_match_finite_differences(causal, alpha):
    T, D = 320, 16
    prm = Params(causal=causal, alpha=alpha, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    ncand = sum((i // 64 if causal else T // 64) for i in range(T))
    for seed in range(10, 30):  # first seed whose scores all sit away from tau
        q, k, v, dout = _inputs(seed, T, D, causal)
        if alpha == 1.0:
            break
        gap, res = _min_gap(q, k, v, prm)
        if gap > 1e-4:
            break
    if alpha > 1:
        assert gap > 1e-4, gap
        assert 0 < res["mask"].sum() < ncand  # the support is a strict subset
    g = oracle.backward(q, k, v, dout, prm)
    rng = np.random.default_rng(99)
    h = 1e-6
    for name in ["q", "k", "v"]:
        for _ in range(2):
            e = rng.normal(size=q.shape)
            args = dict(q=q, k=k, v=v)
            plus = dict(args)
            minus = dict(args)
            plus[name] = args[name] + h * e
            minus[name] = args[name] - h * e
            fd = (_loss(plus["q"], plus["k"], plus["v"], dout, prm)
                  - _loss(minus["q"], minus["k"], minus["v"], dout, prm)) / (2 * h)
            an = float(np.sum(g["d" + name] * e))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("alpha", [1.25, 1.5])
def test_summary_gradient_matches_finite_differences(alpha):
    T, D = 256, 16
    q, k, v, dout = _inputs(30, T, D, True)
    prm = Params(causal=True, alpha=alpha, storage="fp64", coarse_scale=4.0 / math.sqrt(D))
    g = oracle.backward(q, k, v, dout, prm)
    kb = oracle.pool_blocks(k[0, 0], 64, "fp64")[None, None]
    rows = [(0, 0, i) for i in range(T)]

    def loss_kbar(kbar):
        rs = oracle.forward_rows(q, k, v, prm, rows, kbar=kbar)
        return float(sum(np.dot(r["o"], dout[0, 0, i]) for i, r in enumerate(rs)))

    rng = np.random.default_rng(7)
    h = 1e-6
    for _ in range(3):
        e = rng.normal(size=kb.shape)
        fd = (loss_kbar(kb + h * e) - loss_kbar(kb - h * e)) / (2 * h)
        an = float(np.sum(g["dkbar"] * e))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)
    # dk contains the pooling path dkbar / 64 on every key of the block
    g_no_pool = g["dk"] - np.repeat(g["dkbar"][0, 0], 64, axis=0)[None, None] / 64
    assert np.abs(g_no_pool).max() > 0


def test_backward_rows_matches_full_backward():
    T, D = 256, 16
    q, k, v, dout = _inputs(40, T, D, True)
    prm = Params(causal=True, alpha=1.5, storage="bf16", coarse_scale=4.0 / math.sqrt(D))
    full = oracle.backward(q, k, v, dout, prm)
    rows = [(0, 0, i) for i in range(128, T)]  # every row that attends blocks 2 and 3
    part = oracle.backward_rows(q, k, v, dout, prm, rows)
    np.testing.assert_allclose(part["dq"][0, 0, 128:], full["dq"][0, 0, 128:], atol=1e-13)
    for name in ["dk", "dv"]:
        np.testing.assert_allclose(part[name][0, 0, 128:], full[name][0, 0, 128:], atol=1e-13)
    np.testing.assert_allclose(part["dkbar"][0, 0, 2:], full["dkbar"][0, 0, 2:], atol=1e-13)
