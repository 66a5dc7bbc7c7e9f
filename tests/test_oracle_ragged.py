"""Pins for the oracle's causal prefill of a length T that is not a multiple of 64 (CPU only).

Only the complete blocks get summaries; the partial last block is the own
block of its queries.  Checked against torch's float64
scaled_dot_product_attention over the T tokens (the prior as additive mask),
against the same computation on the sequence padded to whole blocks (the
padding values and the padded rows must not matter), and, for the gradients,
against central finite differences.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import Params

from test_oracle_backward import _inputs


def _ragged(seed, T, D):
    Tp = 64 * ((T + 63) // 64)
    q, k, v, dout = _inputs(seed, Tp, D, True)
    return q[:, :, :T].copy(), k[:, :, :T].copy(), v[:, :, :T].copy(), dout[:, :, :T].copy()


@pytest.mark.parametrize("T", [65, 100, 127, 200, 255])
def test_ragged_forward_matches_library_routine(T):
    D = 16
    prm = Params(causal=True, alpha=1.5, storage="bf16", coarse_scale=8.0 / math.sqrt(D))
    q, k, v, _ = _ragged(101 + T, T, D)
    res = oracle.forward(q, k, v, prm)
    nbf = T // 64
    assert res["kbar"].shape[2] == nbf and res["mask"].shape[3] == nbf
    M = np.full((T, T), -np.inf)
    for i in range(T):
        for b in np.flatnonzero(res["mask"][0, 0, i]):
            M[i, 64 * b:64 * b + 64] = np.log(res["p"][0, 0, i, b])
        M[i, 64 * (i // 64):i + 1] = 0.0
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))  # noqa: E731
    ref = F.scaled_dot_product_attention(t(q[0, 0]), t(k[0, 0]), t(v[0, 0]), attn_mask=t(M),
                                         scale=1 / math.sqrt(D)).numpy()
    np.testing.assert_allclose(res["o"][0, 0], ref, rtol=0, atol=1e-12)
    # rows of the partial block select among all complete blocks
    if nbf:
        assert res["nsel"][0, 0, 64 * nbf:].min() >= 1


@pytest.mark.parametrize("T", [100, 200])
def test_ragged_equals_padded_prefix(T):
    D = 16
    prm = Params(causal=True, alpha=1.5, storage="bf16", coarse_scale=8.0 / math.sqrt(D))
    q, k, v, dout = _ragged(111 + T, T, D)
    rng = np.random.default_rng(112)
    Tp = 64 * ((T + 63) // 64)
    pad = lambda x, val=None: np.concatenate(  # noqa: E731
        [x, rng.normal(size=x.shape[:2] + (Tp - T,) + x.shape[3:]) if val is None else np.zeros(x.shape[:2] + (Tp - T,) + x.shape[3:])], axis=2)
    qp, kp, vp, dp = pad(q), pad(k), pad(v), pad(dout, 0.0)
    a = oracle.forward(q, k, v, prm)
    b = oracle.forward(qp, kp, vp, prm)
    nbf = T // 64
    np.testing.assert_array_equal(a["o"], b["o"][:, :, :T])
    np.testing.assert_array_equal(a["lse"], b["lse"][:, :, :T])
    np.testing.assert_array_equal(a["mask"], b["mask"][:, :, :T, :nbf])
    assert not b["mask"][:, :, :T, nbf:].any()  # the padded block is nobody's candidate
    ga = oracle.backward(q, k, v, dout, prm)
    gb = oracle.backward(qp, kp, vp, dp, prm)
    for n, sl in (("dq", np.s_[:, :, :T]), ("dv", np.s_[:, :, :T]), ("dk", np.s_[:, :, :T])):
        np.testing.assert_allclose(ga[n], gb[n][sl], rtol=0, atol=1e-12, err_msg=n)
    np.testing.assert_allclose(ga["dkbar"], gb["dkbar"][:, :, :nbf], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(gb["dkbar"][:, :, nbf:], 0.0)


def test_ragged_gradients_match_finite_differences():
    T, D = 200, 16
    prm = Params(causal=True, alpha=1.5, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    for seed in range(120, 140):
        q, k, v, dout = _ragged(seed, T, D)
        rows = oracle.forward_rows(q, k, v, prm, [(0, 0, i) for i in range(64, T)])
        gap = min(np.min(np.abs(0.5 * r["z"] - r["tau"])) for r in rows)
        if gap > 1e-4:
            break
    assert gap > 1e-4
    g = oracle.backward(q, k, v, dout, prm)
    loss = lambda qq, kk, vv: float(np.sum(oracle.forward(qq, kk, vv, prm)["o"] * dout))  # noqa: E731
    rng = np.random.default_rng(141)
    h = 1e-6
    for name, x in (("q", q), ("k", k), ("v", v)):
        e = rng.normal(size=x.shape)
        args = dict(q=q, k=k, v=v)
        plus, minus = dict(args), dict(args)
        plus[name] = x + h * e
        minus[name] = x - h * e
        fd = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / (2 * h)
        an = float(np.sum(g["d" + name] * e))
        assert abs(fd - an) <= 2e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_non_causal_needs_whole_blocks():
    prm = Params(causal=False)
    x = np.zeros((1, 1, 100, 8))
    with pytest.raises(ValueError):
        oracle.forward(x, x, x, prm)
