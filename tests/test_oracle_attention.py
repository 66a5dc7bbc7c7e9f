"""Pins for the oracle's Stage 0, Stage 2 and decode (CPU only).

Stage 2 is checked against torch's float64 scaled_dot_product_attention (a
library routine) in the special cases the pages fix, and against the same
routine with an additive mask that carries the oracle's own Stage-1 weights
(so only the gathering, the prior and the causal own block are under test).
The non-dispersive property from the pages is checked bit for bit.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import Params


def _sdpa(q, k, v, scale, mask=None, is_causal=False):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))  # noqa: E731
    m = None if mask is None else t(mask)
    return F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale,
                                          is_causal=is_causal).numpy()


def _planted(rng, T, D, nb, blk=64, causal=True, spread=1.0):
    k = rng.normal(size=(T, D))
    v = rng.normal(size=(T, D))
    kb = k.reshape(nb, blk, D).mean(axis=1)
    unit = kb / np.linalg.norm(kb, axis=1, keepdims=True)
    q = 0.5 * rng.normal(size=(T, D))
    for i in range(T):
        c = i // blk if causal else nb
        if c == 0:
            continue
        pick = rng.choice(c, size=min(c, rng.integers(1, 4)), replace=False)
        q[i] += spread * unit[pick].sum(axis=0)
    return q, k, v


# --------------------------------------------------------------------- Stage 0


def test_round_bf16_matches_library_and_handles_double_rounding():
    rng = np.random.default_rng(0)
    x32 = rng.normal(size=10000).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()  # RNE from float32
    np.testing.assert_array_equal(oracle.round_bf16(x32.astype(np.float64)), ref)
    # ties go to even
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above a tie: one-step rounding goes up, a float32 detour would tie to even
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.round_bf16(x) == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(-x) == -(1.0 + 2.0 ** -7)


@pytest.mark.parametrize("storage", ["bf16", "fp32", "fp64"])
def test_pool_is_exact_mean(storage):
    rng = np.random.default_rng(1)
    k = rng.normal(size=(256, 32)).astype(np.float32)
    if storage == "bf16":
        k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
    kb = oracle.pool_blocks(k.astype(np.float64), 64, storage)
    for b in range(4):
        for d in range(32):
            exact = math.fsum(float(x) for x in k[b * 64:(b + 1) * 64, d]) / 64
            assert kb[b, d] == oracle.round_storage(np.array([exact]), storage)[0]


# --------------------------------------------------------------------- Stage 2 special cases


def test_all_equal_prior_is_dense_softmax():
    rng = np.random.default_rng(2)
    T, D, nb = 256, 32, 4
    q, k, v = rng.normal(size=(3, T, D))
    prm = Params(causal=False, storage="fp64")
    sf = 1 / math.sqrt(D)
    ref = _sdpa(q, k, v, sf)
    for i in [0, 17, 255]:
        sel = dict(cand=np.arange(nb), p=np.full(nb, 1 / nb), support=np.ones(nb, bool))
        o, lse, _ = oracle.attend_row(q[i], k, v, i, sel, prm, D)
        np.testing.assert_allclose(o, ref[i], atol=1e-13)
        # the common log-prior -log(nb) shifts the log-sum-exp
        assert abs(lse - (np.log(np.exp(sf * k @ q[i]).sum()) - np.log(nb))) < 1e-12


def test_common_prior_shift_leaves_output_unchanged():
    rng = np.random.default_rng(3)
    T, D, nb = 256, 16, 4
    q, k, v = rng.normal(size=(3, T, D))
    prm = Params(causal=False, storage="fp64")
    p = np.array([0.5, 0.0, 0.3, 0.2])
    sup = p > 0
    sel = dict(cand=np.arange(nb), p=p, support=sup)
    sel2 = dict(cand=np.arange(nb), p=p * math.exp(2.5), support=sup)
    o1, l1, _ = oracle.attend_row(q[5], k, v, 5, sel, prm, D)
    o2, l2, _ = oracle.attend_row(q[5], k, v, 5, sel2, prm, D)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    assert abs((l2 - l1) - 2.5) < 1e-12


def test_single_selected_block_is_softmax_over_its_keys():
    rng = np.random.default_rng(4)
    T, D, nb = 320, 32, 5
    q, k, v = rng.normal(size=(3, T, D))
    prm = Params(causal=False, storage="fp64")
    sel = dict(cand=np.arange(nb), p=np.array([0, 0, 1.0, 0, 0]), support=np.array([0, 0, 1, 0, 0], bool))
    o, _, _ = oracle.attend_row(q[7], k, v, 7, sel, prm, D)
    ref = _sdpa(q[7:8], k[128:192], v[128:192], 1 / math.sqrt(D))[0]
    np.testing.assert_allclose(o, ref, atol=1e-13)


def test_causal_first_block_rows_are_causal_softmax():
    rng = np.random.default_rng(5)
    T, D = 192, 16
    q, k, v = (rng.normal(size=(1, 1, T, D)) for _ in range(3))
    prm = Params(causal=True, storage="fp64", alpha=1.5)
    res = oracle.forward(q, k, v, prm)
    ref = _sdpa(q[0, 0, :64], k[0, 0, :64], v[0, 0, :64], 1 / math.sqrt(D), is_causal=True)
    np.testing.assert_allclose(res["o"][0, 0, :64], ref, atol=1e-13)
    assert (res["nsel"][0, 0, :64] == 0).all()


def _prior_mask(res, T, causal, blk=64):
    """Additive mask from the oracle's Stage-1 weights: log p on selected blocks, 0 on the own block."""
    M = np.full((T, T), -np.inf)
    p = res["p"][0, 0]
    for i in range(T):
        for b in np.flatnonzero(res["mask"][0, 0, i]):
            M[i, b * blk:(b + 1) * blk] = np.log(p[i, b])
        if causal:
            s = (i // blk) * blk
            M[i, s:i + 1] = 0.0
    return M


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("alpha", [1.0, 1.5, 2.0])
def test_forward_equals_masked_library_attention(causal, alpha):
    rng = np.random.default_rng(6)
    T, D = 320, 32
    nb = T // 64
    q, k, v = _planted(rng, T, D, nb, causal=causal)
    q, k, v = (x[None, None] for x in (q, k, v))
    prm = Params(causal=causal, alpha=alpha, storage="fp64", coarse_scale=8.0 / math.sqrt(D))
    res = oracle.forward(q, k, v, prm)
    M = _prior_mask(res, T, causal)
    sf = 1 / math.sqrt(D)
    ref = _sdpa(q[0, 0], k[0, 0], v[0, 0], sf, mask=M)
    np.testing.assert_allclose(res["o"][0, 0], ref, atol=1e-12)
    logits = sf * q[0, 0] @ k[0, 0].T + M
    mx = logits.max(axis=1, keepdims=True)
    lse = (mx + np.log(np.exp(logits - mx).sum(axis=1, keepdims=True)))[:, 0]
    np.testing.assert_allclose(res["lse"][0, 0], lse, atol=1e-12)
    ncand = sum((i // 64 if causal else nb) for i in range(T))
    if alpha > 1:
        assert 0 < res["mask"].sum() < ncand  # some candidate blocks dropped, some kept


def test_forward_rows_matches_forward():
    rng = np.random.default_rng(7)
    T, D = 256, 16
    q, k, v = (rng.normal(size=(1, 2, T, D)) for _ in range(3))
    prm = Params(causal=True, alpha=1.25, storage="bf16")
    res = oracle.forward(q, k, v, prm)
    rows = [(0, 1, 0), (0, 0, 63), (0, 1, 64), (0, 0, 255)]
    for (b, h, i), r in zip(rows, oracle.forward_rows(q, k, v, prm, rows)):
        np.testing.assert_array_equal(r["o"], res["o"][b, h, i])
        np.testing.assert_array_equal(r["mask"], res["mask"][b, h, i])
        assert r["nsel"] == res["nsel"][b, h, i]


# --------------------------------------------------------------------- non-dispersive invariance


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_irrelevant_blocks_change_nothing(alpha):
    """Page "DashAttention: Making Sparse Attention...", "Key Concepts": the weights
    do not depend on the number of irrelevant tokens added to the context."""
    rng = np.random.default_rng(8)
    T, D, nb = 256, 32, 4
    e = np.zeros(D)
    e[0] = 1.0
    q, k, v = _planted(rng, T, D, nb, causal=False)
    q = q + 2.0 * e  # every query leans along e
    prm = Params(causal=False, alpha=alpha, storage="fp64")
    base = oracle.forward(q[None, None], k[None, None], v[None, None], prm)
    extra_k = -10.0 * e + 0.1 * rng.normal(size=(128, D))  # two blocks pointing away from every query
    extra_v = rng.normal(size=(128, D))
    k2 = np.concatenate([k, extra_k])
    v2 = np.concatenate([v, extra_v])
    rows = [(0, 0, i) for i in range(T)]
    big = oracle.forward_rows(q[None, None], k2[None, None], v2[None, None], prm, rows)
    for i, r in enumerate(big):
        assert not r["mask"][nb:].any()
        np.testing.assert_array_equal(r["mask"][:nb], base["mask"][0, 0, i])
        np.testing.assert_array_equal(r["o"], base["o"][0, 0, i])
        assert r["lse"] == base["lse"][0, 0, i]
        assert r["tau"] == base["tau"][0, 0, i]


# --------------------------------------------------------------------- decode


def test_decode_is_last_row_of_causal_prefill():
    rng = np.random.default_rng(9)
    S, H, N, D = 2, 2, 512, 32
    kc, vc = rng.normal(size=(2, S, H, N, D))
    q = rng.normal(size=(S, H, D)) + 1.5 * kc[:, :, 64:128].mean(axis=2)
    prm = Params(causal=True, alpha=1.5, storage="bf16", coarse_scale=10.0 / math.sqrt(D))
    dec = oracle.decode(q, kc, vc, prm)
    sf = 1 / math.sqrt(D)
    for s in range(S):
        for h in range(H):
            qq = np.zeros((N, D))
            qq[-1] = q[s, h]
            res = oracle.forward_rows(qq[None, None], kc[s, h][None, None], vc[s, h][None, None], prm,
                                      [(0, 0, N - 1)])[0]
            np.testing.assert_array_equal(dec["o"][s, h], res["o"])
            np.testing.assert_array_equal(dec["mask"][s, h], res["mask"])
            # and against the library routine with the prior as an additive mask
            M = np.full((1, N), -np.inf)
            for b in np.flatnonzero(res["mask"]):
                M[0, b * 64:(b + 1) * 64] = np.log(res["p"][b])
            M[0, N - 64:] = 0.0
            ref = _sdpa(q[s, h][None], kc[s, h], vc[s, h], sf, mask=M)[0]
            np.testing.assert_allclose(dec["o"][s, h], ref, atol=1e-12)
            assert 0 < dec["nsel"][s, h] < N // 64 - 1
