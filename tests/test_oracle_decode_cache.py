"""Pins for the oracle's decode cache maintenance and per-sequence cache lengths (CPU only).

``decode_varlen`` is checked against torch's float64 scaled_dot_product_attention
over the first n cached tokens (the library routine; the additive mask carries
the oracle's own Stage-1 weights, so the length handling, the gathering, the
prior and the partial own block are under test), against a dense causal
softmax where the query's own block is the only one, and against a causal
prefill row on a cache truncated to n tokens.  ``cache_append`` is checked
against the exact block means (math.fsum) of the keys appended one by one.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import Params


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _sdpa_row(q, k, v, scale, mask):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))  # noqa: E731
    return F.scaled_dot_product_attention(t(q[None]), t(k), t(v), attn_mask=t(mask[None]), scale=scale).numpy()[0]


def _cache(rng, S, H, C, D, lens, spread=1.5):
    kc = _bf16(rng.normal(size=(S, H, C, D)))
    vc = _bf16(rng.normal(size=(S, H, C, D)))
    q = rng.normal(size=(S, H, D))
    for s in range(S):
        nc = (int(lens[s]) - 1) // 64
        for h in range(H):
            if nc:
                b = rng.integers(0, nc)
                kb = kc[s, h, 64 * b:64 * b + 64].mean(axis=0)
                q[s, h] += spread * kb / np.linalg.norm(kb)
    return _bf16(q), kc, vc


LENS = [1, 2, 63, 64, 65, 127, 128, 129, 200, 255, 256]


@pytest.mark.parametrize("alpha", [1.5, 1.25])
def test_decode_varlen_matches_library_routine(alpha):
    rng = np.random.default_rng(21)
    S, H, C, D = len(LENS), 2, 256, 32
    lens = np.array(LENS)
    q, kc, vc = _cache(rng, S, H, C, D, lens)
    prm = Params(causal=True, alpha=alpha, storage="bf16", coarse_scale=12.0 / math.sqrt(D))
    dec = oracle.decode_varlen(q, kc, vc, lens, prm)
    sf = 1 / math.sqrt(D)
    for s, n in enumerate(LENS):
        own = (n - 1) // 64
        for h in range(H):
            sel = oracle.select_row(q[s, h], oracle.pool_blocks(kc[s, h, :64 * own], 64, "bf16"), n - 1, prm, D)
            M = np.full(n, -np.inf)
            for b, p in zip(sel["cand"][sel["support"]], sel["p"][sel["support"]]):
                M[64 * b:64 * b + 64] = np.log(p)
            M[64 * own:n] = 0.0
            ref = _sdpa_row(q[s, h], kc[s, h, :n], vc[s, h, :n], sf, M)
            np.testing.assert_allclose(dec["o"][s, h], ref, atol=1e-12, err_msg=f"n={n}")
            assert dec["nsel"][s, h] == int(sel["support"].sum())
            np.testing.assert_array_equal(np.flatnonzero(dec["mask"][s, h]), sel["cand"][sel["support"]])
            if own == 0:
                # only the own block: a dense causal softmax over the n tokens
                assert dec["nsel"][s, h] == 0 and math.isnan(dec["tau"][s, h])
                dense = _sdpa_row(q[s, h], kc[s, h, :n], vc[s, h, :n], sf, np.zeros(n))
                np.testing.assert_allclose(dec["o"][s, h], dense, atol=1e-12)
            else:
                assert dec["nsel"][s, h] >= 1


def test_decode_varlen_is_prefill_row_of_truncated_cache():
    rng = np.random.default_rng(22)
    S, H, C, D = len(LENS), 2, 256, 32
    lens = np.array(LENS)
    q, kc, vc = _cache(rng, S, H, C, D, lens)
    prm = Params(causal=True, alpha=1.5, storage="bf16", coarse_scale=12.0 / math.sqrt(D))
    dec = oracle.decode_varlen(q, kc, vc, lens, prm)
    for s, n in enumerate(LENS):
        Tp = 64 * ((n + 63) // 64)
        for h in range(H):
            # the first n tokens, padded with fresh values the row must not see
            kk = np.concatenate([kc[s, h, :n], _bf16(rng.normal(size=(Tp - n, D)))])
            vv = np.concatenate([vc[s, h, :n], _bf16(rng.normal(size=(Tp - n, D)))])
            qq = np.zeros((Tp, D))
            qq[n - 1] = q[s, h]
            r = oracle.forward_rows(qq[None, None], kk[None, None], vv[None, None], prm, [(0, 0, n - 1)])[0]
            np.testing.assert_array_equal(dec["o"][s, h], r["o"])
            assert dec["lse"][s, h] == r["lse"]
            assert dec["nsel"][s, h] == r["nsel"]
    # a full last block: the fixed-length decode (R7) on the truncated cache
    for s, n in enumerate(LENS):
        if n % 64 == 0:
            full = oracle.decode(q[s:s + 1], kc[s:s + 1, :, :n], vc[s:s + 1, :, :n], prm)
            np.testing.assert_array_equal(dec["o"][s], full["o"][0])


def test_decode_varlen_never_reads_beyond_the_length():
    rng = np.random.default_rng(23)
    S, H, C, D = len(LENS), 2, 256, 32
    lens = np.array(LENS)
    q, kc, vc = _cache(rng, S, H, C, D, lens)
    prm = Params(causal=True, alpha=1.5, storage="bf16", coarse_scale=12.0 / math.sqrt(D))
    kbar = np.stack([[oracle.pool_blocks(kc[s, h], 64, "bf16") for h in range(H)] for s in range(S)])
    base = oracle.decode_varlen(q, kc, vc, lens, prm, kbar=kbar)
    kn, vn, kbn = kc.copy(), vc.copy(), kbar.copy()
    for s, n in enumerate(LENS):
        kn[s, :, n:] = np.nan
        vn[s, :, n:] = np.nan
        kbn[s, :, (n - 1) // 64:] = np.nan  # the own block and later: never candidates
    poisoned = oracle.decode_varlen(q, kn, vn, lens, prm, kbar=kbn)
    for key in ("o", "lse", "nsel", "mask"):
        np.testing.assert_array_equal(poisoned[key], base[key])


def test_cache_append_builds_the_block_means():
    rng = np.random.default_rng(24)
    S, H, C, D = 2, 2, 256, 16
    prm = Params(causal=True, storage="bf16")
    kc = np.full((S, H, C, D), 7.0)
    vc = np.full((S, H, C, D), 7.0)
    kbar = np.full((S, H, C // 64, D), -3.0)  # sentinel: untouched until a block completes
    lens = np.array([0, 37])
    start = lens.copy()
    keys, vals = [], []
    for step in range(150):
        kn = _bf16(rng.normal(size=(S, H, D)))
        vn = _bf16(rng.normal(size=(S, H, D)))
        keys.append(kn)
        vals.append(vn)
        kc2, vc2, kbar2, lens2 = oracle.cache_append(kc, vc, kbar, lens, kn, vn, prm)
        np.testing.assert_array_equal(lens2, lens + 1)
        for s in range(S):
            n = int(lens[s])
            np.testing.assert_array_equal(kc2[s, :, n], kn[s])
            np.testing.assert_array_equal(vc2[s, :, n], vn[s])
            others = np.ones(C, dtype=bool)
            others[n] = False
            np.testing.assert_array_equal(kc2[s, :, others], kc[s, :, others])
            done = n % 64 == 63
            for b in range(C // 64):
                if done and b == n // 64:
                    continue
                np.testing.assert_array_equal(kbar2[s, :, b], kbar[s, :, b])
        kc, vc, kbar, lens = kc2, vc2, kbar2, lens2
    # every block completed by appends holds the exact mean of its keys, rounded once
    for s in range(S):
        for b in range(C // 64):
            lo, hi = 64 * b, 64 * b + 64
            complete_by_append = start[s] <= hi - 1 < lens[s]  # its last token was appended
            for h in range(H):
                if complete_by_append:
                    for d in range(D):
                        exact = math.fsum(float(x) for x in kc[s, h, lo:hi, d]) / 64
                        assert kbar[s, h, b, d] == oracle.round_bf16(np.array([exact]))[0]
                else:
                    assert np.all(kbar[s, h, b] == -3.0)
    # the appended tokens sit at their positions
    for t in range(150):
        for s in range(S):
            np.testing.assert_array_equal(kc[s, :, start[s] + t], keys[t][s])
            np.testing.assert_array_equal(vc[s, :, start[s] + t], vals[t][s])


def test_append_then_decode_equals_decode_of_the_grown_cache():
    rng = np.random.default_rng(25)
    S, H, C, D = 3, 2, 192, 32
    prm = Params(causal=True, alpha=1.5, storage="bf16", coarse_scale=8.0 / math.sqrt(D))
    lens = np.array([60, 64, 130])
    q, kc, vc = _cache(rng, S, H, C, D, lens + 1)
    kbar = np.stack([[oracle.pool_blocks(kc[s, h], 64, "bf16") for h in range(H)] for s in range(S)])
    kn = _bf16(rng.normal(size=(S, H, D)))
    vn = _bf16(rng.normal(size=(S, H, D)))
    kc2, vc2, kbar2, lens2 = oracle.cache_append(kc, vc, kbar, lens, kn, vn, prm)
    a = oracle.decode_varlen(q, kc2, vc2, lens2, prm, kbar=kbar2)
    b = oracle.decode_varlen(q, kc2, vc2, lens2, prm)  # summaries pooled from the grown cache
    for key in ("o", "lse", "nsel", "mask"):
        np.testing.assert_array_equal(a[key], b[key])


def test_lengths_out_of_range_are_rejected():
    prm = Params(causal=True)
    kc = np.zeros((1, 1, 64, 8))
    with pytest.raises(ValueError):
        oracle.decode_varlen(np.zeros((1, 1, 8)), kc, kc, np.array([0]), prm)
    with pytest.raises(ValueError):
        oracle.decode_varlen(np.zeros((1, 1, 8)), kc, kc, np.array([65]), prm)
    with pytest.raises(ValueError):
        oracle.cache_append(kc, kc, np.zeros((1, 1, 1, 8)), np.array([64]), np.zeros((1, 1, 8)), np.zeros((1, 1, 8)), prm)
