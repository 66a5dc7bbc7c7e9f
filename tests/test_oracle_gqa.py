"""Pins for the oracle's grouped-query attention with entmax head aggregation (CPU only).

One head per group is the per-head (MHA) oracle bit for bit; a group of
identical query heads reduces to one head's selection; every head's output
equals torch's float64 scaled_dot_product_attention with the group's log
pbar as an additive mask over its KV head; the gradients match central
finite differences; the shared support is the union of the heads' supports.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import Params


def _inputs(seed, B, H, Hkv, T, D, causal=True, spread=1.5):
    rng = np.random.default_rng(seed)
    nb = T // 64
    k = rng.normal(size=(B, Hkv, T, D))
    v = rng.normal(size=(B, Hkv, T, D))
    q = 0.5 * rng.normal(size=(B, H, T, D))
    G = H // Hkv
    for b in range(B):
        for h in range(H):
            kb = k[b, h // G].reshape(nb, 64, D).mean(axis=1)
            unit = kb / np.linalg.norm(kb, axis=1, keepdims=True)
            for i in range(T):
                c = i // 64 if causal else nb
                if c:
                    pick = rng.choice(c, size=min(c, rng.integers(1, 3)), replace=False)
                    q[b, h, i] += spread * unit[pick].sum(axis=0)
    dout = rng.normal(size=(B, H, T, D))
    return q, k, v, dout


@pytest.mark.parametrize("causal", [True, False])
def test_one_head_per_group_is_per_head_attention(causal):
    T, D = 256, 16
    prm = Params(causal=causal, alpha=1.5, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    q, k, v, dout = _inputs(61, 1, 2, 2, T, D, causal)
    a = oracle.forward_gqa(q, k, v, prm)
    b = oracle.forward(q, k, v, prm)
    np.testing.assert_array_equal(a["o"], b["o"])
    np.testing.assert_array_equal(a["lse"], b["lse"])
    np.testing.assert_array_equal(a["union"], b["mask"])
    ga = oracle.backward_gqa(q, k, v, dout, prm)
    gb = oracle.backward(q, k, v, dout, prm)
    for n in ("dq", "dk", "dv", "dkbar"):
        np.testing.assert_array_equal(ga[n], gb[n], err_msg=n)


@pytest.mark.parametrize("G", [2, 4])
def test_identical_heads_reduce_to_one_head(G):
    T, D = 256, 16
    prm = Params(causal=True, alpha=1.5, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    q1, k, v, d1 = _inputs(62, 1, 1, 1, T, D)
    q = np.repeat(q1, G, axis=1)
    dout = np.repeat(d1, G, axis=1)
    a = oracle.forward_gqa(q, k, v, prm)
    b = oracle.forward(q1, k, v, prm)
    for h in range(G):
        np.testing.assert_array_equal(a["o"][:, h], b["o"][:, 0])
        np.testing.assert_array_equal(a["union"][:, h], b["mask"][:, 0])
    ga = oracle.backward_gqa(q, k, v, dout, prm)
    gb = oracle.backward(q1, k, v, d1, prm)
    for h in range(G):
        np.testing.assert_array_equal(ga["dq"][:, h], gb["dq"][:, 0])
    for n in ("dk", "dv", "dkbar"):
        np.testing.assert_allclose(ga[n], G * gb[n], rtol=1e-12, atol=1e-12, err_msg=n)


def test_matches_library_routine_with_the_group_prior():
    T, D, H, Hkv = 256, 16, 4, 2
    prm = Params(causal=True, alpha=1.5, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    q, k, v, _ = _inputs(63, 1, H, Hkv, T, D)
    res = oracle.forward_gqa(q, k, v, prm)
    sf = 1 / math.sqrt(D)
    G = H // Hkv
    for h in range(H):
        M = np.full((T, T), -np.inf)
        for i in range(T):
            own = i // 64
            for b in np.flatnonzero(res["union"][0, h, i]):
                M[i, 64 * b:64 * b + 64] = np.log(res["pbar"][0, h, i, b])
            M[i, 64 * own:i + 1] = 0.0
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x))  # noqa: E731
        ref = F.scaled_dot_product_attention(t(q[0, h]), t(k[0, h // G]), t(v[0, h // G]), attn_mask=t(M),
                                             scale=sf).numpy()
        np.testing.assert_allclose(res["o"][0, h], ref, rtol=0, atol=1e-12)


def test_union_support_and_normalisation():
    T, D, H, Hkv = 320, 16, 4, 1
    prm = Params(causal=True, alpha=1.5, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    q, k, v, _ = _inputs(64, 1, H, Hkv, T, D)
    rows = [(0, h, i) for h in range(H) for i in range(64, T)]
    res = oracle.forward_rows_gqa(q, k, v, prm, rows)
    differ = 0
    for i in range(64, T):
        group = [res[h * (T - 64) + (i - 64)] for h in range(H)]
        union = group[0]["union"]
        for r in group:
            np.testing.assert_array_equal(r["union"], union)
            assert np.all(union[r["mask"]])  # every head's own support is inside the union
            np.testing.assert_allclose(r["pbar"].sum(), 1.0, rtol=0, atol=1e-12)
            assert np.all((r["pbar"] > 0) == union)
        masks = np.stack([r["mask"] for r in group])
        assert np.array_equal(masks.any(axis=0), union)
        differ += int((masks != masks[0]).any())
    assert differ > 0  # the heads do select differently, so the union is not trivial


@pytest.mark.parametrize("alpha", [1.25, 1.5])
def test_gradients_match_finite_differences(alpha):
    T, D, H, Hkv = 256, 8, 4, 2
    prm = Params(causal=True, alpha=alpha, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    for seed in range(70, 90):  # first seed whose scores all sit away from tau
        q, k, v, dout = _inputs(seed, 1, H, Hkv, T, D)
        rows = [(0, h, i) for h in range(H) for i in range(64, T)]
        gap = min(np.min(np.abs((alpha - 1) * r["z"] - r["tau"])) for r in oracle.forward_rows_gqa(q, k, v, prm, rows))
        if gap > 1e-4:
            break
    assert gap > 1e-4
    g = oracle.backward_gqa(q, k, v, dout, prm)
    loss = lambda qq, kk, vv: float(np.sum(oracle.forward_gqa(qq, kk, vv, prm)["o"] * dout))  # noqa: E731
    rng = np.random.default_rng(91)
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


def test_heads_must_divide():
    prm = Params()
    q = np.zeros((1, 3, 64, 8))
    k = np.zeros((1, 2, 64, 8))
    with pytest.raises(ValueError):
        oracle.forward_rows_gqa(q, k, k, prm, [(0, 0, 0)])


def test_gqa_decode_is_the_last_prefill_row():
    rng = np.random.default_rng(92)
    S, H, Hkv, C, D = 3, 4, 2, 256, 16
    prm = Params(causal=True, alpha=1.5, storage="bf16", coarse_scale=8.0 / math.sqrt(D))
    lens = np.array([64, 150, 256])
    kc = rng.normal(size=(S, Hkv, C, D))
    vc = rng.normal(size=(S, Hkv, C, D))
    q = rng.normal(size=(S, H, D))
    for s in range(S):
        for h in range(H):
            kb = kc[s, h // 2, :64].mean(axis=0)
            q[s, h] += 1.5 * kb / np.linalg.norm(kb)
    dec = oracle.decode_gqa(q, kc, vc, lens, prm)
    for s, n in enumerate(lens):
        Tp = 64 * ((n + 63) // 64)
        qq = np.zeros((1, H, Tp, D))
        qq[0, :, n - 1] = q[s]
        kk = np.zeros((1, Hkv, Tp, D))
        vv = np.zeros((1, Hkv, Tp, D))
        kk[0, :, :n], vv[0, :, :n] = kc[s, :, :n], vc[s, :, :n]
        rows = oracle.forward_rows_gqa(qq, kk, vv, prm, [(0, h, n - 1) for h in range(H)])
        for h, r in enumerate(rows):
            np.testing.assert_array_equal(dec["o"][s, h], r["o"])
            assert dec["lse"][s, h] == r["lse"]
            np.testing.assert_array_equal(dec["union"][s, h, : (n - 1) // 64], r["union"][: (n - 1) // 64])
    # one KV head per query head: the per-head decode
    kc1 = np.repeat(kc, 2, axis=1)
    vc1 = np.repeat(vc, 2, axis=1)
    a = oracle.decode_gqa(q, kc1, vc1, lens, prm)
    b = oracle.decode_varlen(q, kc1, vc1, lens, prm)
    np.testing.assert_array_equal(a["o"], b["o"])
    np.testing.assert_array_equal(a["nsel"], b["nsel"])
