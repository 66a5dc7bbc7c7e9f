"""Pins for the oracle's learned Stage-0 summariser (CPU only).

pool_attention at w = 0 is mean pooling bit for bit (every weight is
exactly 1/64), and so are the forward and the gradients into q, k, v and the
summaries; its gradient (pool_attention_vjp) and the full backward's dw
match central finite differences of the float64 forward; a large w turns
the summary into the block's highest-scoring key (hard attention); the
summary is invariant to the order of the keys in a block and lies in their
convex hull.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import Params

from test_oracle_backward import _inputs


def _bf16(x):
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("storage", ["bf16", "fp32", "fp64"])
def test_zero_head_is_mean_pooling(storage):
    rng = np.random.default_rng(41)
    k = _bf16(rng.normal(size=(512, 128)))
    got = oracle.pool_attention(k, np.zeros(128), 64, storage)
    np.testing.assert_array_equal(got, oracle.pool_blocks(k, 64, storage))
    dkbar = rng.normal(size=(8, 128))
    dk, dw = oracle.pool_attention_vjp(k, np.zeros(128), dkbar, 64)
    np.testing.assert_array_equal(dk, np.repeat(dkbar, 64, axis=0) / 64)
    assert np.abs(dw).max() > 0  # the head still gets a gradient at zero


@pytest.mark.parametrize("scale", [0.0, 0.3])
def test_pool_attention_vjp_matches_finite_differences(scale):
    rng = np.random.default_rng(42)
    T, D = 192, 16
    k = rng.normal(size=(T, D))
    w = scale * rng.normal(size=D)
    dkbar = rng.normal(size=(T // 64, D))
    f = lambda kk, ww: float(np.sum(oracle.pool_attention(kk, ww, 64, "fp64") * dkbar))  # noqa: E731
    dk, dw = oracle.pool_attention_vjp(k, w, dkbar, 64)
    h = 1e-6
    for _ in range(3):
        e = rng.normal(size=k.shape)
        fd = (f(k + h * e, w) - f(k - h * e, w)) / (2 * h)
        assert abs(fd - np.sum(dk * e)) <= 1e-7 * max(1.0, abs(fd)), (fd, np.sum(dk * e))
        u = rng.normal(size=D)
        fd = (f(k, w + h * u) - f(k, w - h * u)) / (2 * h)
        assert abs(fd - dw @ u) <= 1e-7 * max(1.0, abs(fd)), (fd, dw @ u)


def test_large_head_picks_the_top_key():
    rng = np.random.default_rng(43)
    k = rng.normal(size=(256, 32))
    u = rng.normal(size=32)
    got = oracle.pool_attention(k, 1e5 * u, 64, "fp64")
    for b in range(4):
        blk = k[64 * b:64 * b + 64]
        np.testing.assert_allclose(got[b], blk[np.argmax(blk @ u)], rtol=0, atol=1e-12)


def test_order_invariance_and_convex_hull():
    rng = np.random.default_rng(44)
    k = rng.normal(size=(128, 32))
    w = 0.5 * rng.normal(size=32)
    base = oracle.pool_attention(k, w, 64, "fp64")
    perm = np.concatenate([rng.permutation(64), 64 + rng.permutation(64)])
    np.testing.assert_allclose(oracle.pool_attention(k[perm], w, 64, "fp64"), base, rtol=0, atol=1e-14)
    for b in range(2):
        blk = k[64 * b:64 * b + 64]
        assert np.all(base[b] <= blk.max(axis=0) + 1e-15) and np.all(base[b] >= blk.min(axis=0) - 1e-15)
    # not the mean once w is away from zero
    assert np.abs(base - oracle.pool_blocks(k, 64, "fp64")).max() > 1e-3


@pytest.mark.parametrize("causal", [True, False])
def test_zero_head_forward_and_backward_equal_mean_pooling(causal):
    T, D = 256, 16
    prm = Params(causal=causal, alpha=1.5, storage="bf16", coarse_scale=8.0 / math.sqrt(D))
    q, k, v, dout = _inputs(45, T, D, causal)
    w0 = np.zeros((1, D))
    a = oracle.forward(q, k, v, prm)
    b = oracle.forward(q, k, v, prm, w=w0)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    ga = oracle.backward(q, k, v, dout, prm)
    gb = oracle.backward(q, k, v, dout, prm, w=w0)
    for key in ("dq", "dk", "dv", "dkbar"):
        np.testing.assert_array_equal(ga[key], gb[key], err_msg=key)


@pytest.mark.parametrize("scale", [0.0, 0.2])
def test_head_gradient_matches_finite_differences(scale):
    T, D = 320, 16
    prm = Params(causal=True, alpha=1.5, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    rng = np.random.default_rng(46)
    for seed in range(50, 70):  # first seed whose scores all sit away from tau
        q, k, v, dout = _inputs(seed, T, D, True)
        w = scale * rng.normal(size=(1, D))
        gap = min(np.min(np.abs((prm.alpha - 1) * r["z"] - r["tau"]))
                  for r in oracle.forward_rows(q, k, v, prm, [(0, 0, i) for i in range(64, T)], w=w))
        if gap > 1e-4:
            break
    assert gap > 1e-4
    g = oracle.backward(q, k, v, dout, prm, w=w)
    loss = lambda ww, kk: float(np.sum(oracle.forward(q, kk, v, prm, w=ww)["o"] * dout))  # noqa: E731
    h = 1e-6
    for _ in range(2):
        u = rng.normal(size=w.shape)
        fd = (loss(w + h * u, k) - loss(w - h * u, k)) / (2 * h)
        assert abs(fd - np.sum(g["dw"] * u)) <= 2e-6 * max(1.0, abs(fd)), (fd, np.sum(g["dw"] * u))
        e = rng.normal(size=k.shape)
        fd = (loss(w, k + h * e) - loss(w, k - h * e)) / (2 * h)
        assert abs(fd - np.sum(g["dk"] * e)) <= 2e-6 * max(1.0, abs(fd)), (fd, np.sum(g["dk"] * e))


def test_backward_rows_carries_the_head_gradient():
    T, D = 256, 16
    prm = Params(causal=True, alpha=1.5, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    q, k, v, dout = _inputs(47, T, D, True)
    w = 0.2 * np.random.default_rng(48).normal(size=(1, D))
    full = oracle.backward(q, k, v, dout, prm, w=w)
    rows = oracle.backward_rows(q, k, v, dout, prm, [(0, 0, i) for i in range(T)], w=w)
    for key in ("dq", "dk", "dv", "dkbar", "dw"):
        np.testing.assert_allclose(rows[key], full[key], rtol=0, atol=1e-12, err_msg=key)
