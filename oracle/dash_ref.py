"""DashAttention forward, decode and backward in plain float64 (test infrastructure only).

One query row at a time, gathering only the tokens the row attends, so that
the arithmetic of a row does not depend on blocks it does not select.  This
is slow by design; it is the reference the HIP library is checked against.

Method, as the pages state it:

* Stage 0 (page "DashAttention and the year sparse attention became a
  field", section "What alpha-entmax changes"): each block of keys gets a
  summary; the learned summariser starts at zero, i.e. from mean pooling.
  Here the summary is the mean of the block's keys.
* Stage 1 (page "DashAttention: Making Sparse Attention Fully
  Differentiable...", sections "Core Mechanism" and its pipeline figure):
  coarse score q . summary for each block, then alpha-entmax gives sparse
  block weights p.
* Stage 2 (same sections): for the selected blocks, fine logits q . k plus
  log p of the key's block, one softmax, weighted sum of V.
* Gradients flow from Stage 2 through log p into the entmax and on to the
  summaries (same sections; "What alpha-entmax changes").

Readings taken where the pages are silent:

* R1 entmax parameterisation u = (alpha-1) z, p = [u - tau]_+^(1/(alpha-1)).
* R2 one joint softmax over all attended tokens with log p added to the logits.
* R4 causal: the candidates of query i are the blocks strictly before its
  own block; its own block is always attended under the causal mask with
  log-prior 0.  Queries of block 0 attend only their own block.
* R5 the summary is the exact mean of the block's keys, rounded once
  (round-to-nearest-even) to the storage dtype of K.
* R7 decode: the new token is the last cached token; the decode output is
  row N-1 of a causal prefill over the cache.
* R18 decode cache maintenance: appending token n writes it at position n;
  when that completes a block, the block's summary is its Stage-0 mean.
* R20 the learned summariser: per head a vector w (initialised at zero);
  a block's summary is sum_j softmax_j(w . k_j) k_j over its keys, which is
  mean pooling at w = 0.
* R22 a causal prefill of T tokens, T not a multiple of the block: the
  last block is partial; it is the own block of its queries and never a
  candidate of any query, so only the complete blocks get summaries.
  Non-causal attention needs whole blocks (every block is a candidate).
* R19 a cache of n tokens (any n >= 1): the query is at position n-1, its
  candidates are the complete blocks before its own, and its own block is
  attended over its cached tokens only (row n-1 of a causal prefill over
  the first n tokens).
* R9 separate fine scale (logits) and coarse scale (block scores).
* Backward treats the rounding of the summary to its storage dtype as the
  identity (straight-through).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .entmax import entmax, entmax_jvp


@dataclass(frozen=True)
class Params:
    block: int = 64
    alpha: float = 1.5
    causal: bool = True
    fine_scale: float | None = None  # default 1/sqrt(D)
    coarse_scale: float | None = None  # default 1/sqrt(D)
    storage: str = "bf16"  # dtype the summaries are stored in: bf16 | fp32 | fp64

    def scales(self, D: int) -> tuple[float, float]:
        sf = self.fine_scale if self.fine_scale is not None else 1.0 / np.sqrt(D)
        sc = self.coarse_scale if self.coarse_scale is not None else 1.0 / np.sqrt(D)
        return float(sf), float(sc)


# ----------------------------------------------------------------------------- rounding


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even, in one step.

    bfloat16 keeps 8 significant bits.  With x = m * 2**e and 0.5 <= |m| < 1
    (``frexp``), the rounded value is rint(m * 2**8) * 2**(e - 8), where
    ``rint`` rounds half to even.  Rounding straight from float64 avoids the
    double rounding of a float64 -> float32 -> bfloat16 chain.  Values here
    are far from the bfloat16 overflow and subnormal ranges.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_storage(x, storage: str):
    if storage == "bf16":
        return round_bf16(x)
    if storage == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if storage == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown storage {storage!r}")


# ----------------------------------------------------------------------------- Stage 0


def pool_blocks(k_head, block: int, storage: str):
    """Stage 0: mean of each block's keys, rounded once to the storage dtype.

    ``k_head`` is [T, D] (T a multiple of ``block``); returns [T/block, D].
    The sum of 64 bfloat16 (or float32) values of ordinary magnitude is exact
    in float64, so the mean is exact before the single rounding (R5).
    """
    k_head = np.asarray(k_head, dtype=np.float64)
    T, D = k_head.shape
    if T % block:
        raise ValueError("T must be a multiple of the block size")
    mean = k_head.reshape(T // block, block, D).sum(axis=1) / block
    return round_storage(mean, storage)


def pool_attention(k_head, w, block: int, storage: str):
    """Stage 0 with the learned summariser (R20): attention pooling per block.

    The montana-research page ("What alpha-entmax changes") has Stage 0
    summarise each block with a small learned attention head that starts
    at zero, so training starts from mean pooling.  Here the head is one
    vector ``w`` [D] per attention head: block b's keys get scores
    e_j = w . k_j, weights a = softmax(e) over the block, and the summary is
    sum_j a_j k_j, rounded once to the storage dtype.  At w = 0 every
    a_j = 1/block exactly, so this is :func:`pool_blocks` bit for bit.
    """
    k_head = np.asarray(k_head, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, D = k_head.shape
    if T % block:
        raise ValueError("T must be a multiple of the block size")
    kb = k_head.reshape(T // block, block, D)
    e = kb @ w  # [nb, block]
    a = np.exp(e - e.max(axis=1, keepdims=True))
    a = a / a.sum(axis=1, keepdims=True)
    return round_storage((a[:, :, None] * kb).sum(axis=1), storage)


def pool_attention_vjp(k_head, w, dkbar, block: int):
    """Gradient of sum_b <dkbar_b, summary_b> through :func:`pool_attention`.

    The rounding of the summary is taken as the identity.  With a the block
    weights, m_b the exact summary and c_j = k_j . dkbar_b - m_b . dkbar_b
    (the softmax Jacobian applied to the scores' gradient k_j . dkbar_b):

        dk_j = a_j dkbar_b + a_j c_j w,        dw = sum_b sum_j a_j c_j k_j.

    Returns (dk [T, D], dw [D]).  At w = 0 the first term is dkbar_b / block,
    the mean-pooling gradient.
    """
    k_head = np.asarray(k_head, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dkbar = np.asarray(dkbar, dtype=np.float64)
    T, D = k_head.shape
    kb = k_head.reshape(T // block, block, D)
    e = kb @ w
    a = np.exp(e - e.max(axis=1, keepdims=True))
    a = a / a.sum(axis=1, keepdims=True)
    m = (a[:, :, None] * kb).sum(axis=1)  # [nb, D]
    c = kb @ dkbar[:, :, None]  # [nb, block, 1]
    c = c[:, :, 0] - (m * dkbar).sum(axis=1)[:, None]
    de = a * c  # gradient of the scores
    dk = a[:, :, None] * dkbar[:, None, :] + de[:, :, None] * w[None, None, :]
    dw = (de[:, :, None] * kb).sum(axis=(0, 1))
    return dk.reshape(T, D), dw


def summarise(k_head, prm: "Params", w_h=None):
    """Stage 0 of one head: mean pooling, or the learned summariser when ``w_h`` is given.

    Summaries of the complete blocks only: with a partial last block
    (causal attention, R22) the partial block gets none.
    """
    T = k_head.shape[0]
    if T % prm.block:
        if not prm.causal:
            raise ValueError("non-causal attention needs T to be a multiple of the block size")
        k_head = k_head[: (T // prm.block) * prm.block]
    if w_h is None:
        return pool_blocks(k_head, prm.block, prm.storage)
    return pool_attention(k_head, w_h, prm.block, prm.storage)


# ----------------------------------------------------------------------------- Stage 1


def candidate_blocks(i: int, nb: int, block: int, causal: bool):
    """Blocks query ``i`` scores in Stage 1: all blocks, or those before its own (R4)."""
    return np.arange(i // block) if causal else np.arange(nb)


def select_row(q_i, kbar, i: int, prm: Params, D: int):
    """Stage 1 for one query row: coarse scores, alpha-entmax, support.

    Returns a dict with the candidate block ids, z, p (over the candidates),
    tau (u-units for alpha > 1, z-units for alpha = 1; NaN with no
    candidates) and the boolean support.
    """
    _, sc = prm.scales(D)
    nb = kbar.shape[0]
    cand = candidate_blocks(i, nb, prm.block, prm.causal)
    if cand.size == 0:
        return dict(cand=cand, z=np.zeros(0), p=np.zeros(0), tau=np.nan,
                    support=np.zeros(0, dtype=bool))
    # Row-wise dot products, reduced along the contiguous feature axis, so
    # each score depends only on its own summary.
    z = sc * (kbar[cand] * q_i[None, :]).sum(axis=1)
    p, tau, support = entmax(z, prm.alpha)
    return dict(cand=cand, z=z, p=p, tau=tau, support=support)


# ----------------------------------------------------------------------------- Stage 2


def attend_row(q_i, k_head, v_head, i: int, sel, prm: Params, D: int):
    """Stage 2 for one query row.

    Attended tokens: every token of every selected candidate block (prior
    log p_b) and, when causal, the tokens j <= i of the row's own block
    (prior 0).  One softmax over logits fine_scale * q . k_j + prior_j, then
    the weighted sum of V.  Returns (o, lse, ctx) where ctx holds what the
    backward needs.
    """
    sf, _ = prm.scales(D)
    blk = prm.block
    chosen = sel["cand"][sel["support"]]
    logp = np.log(sel["p"][sel["support"]])
    idx_parts = [np.arange(b * blk, (b + 1) * blk) for b in chosen]
    prior_parts = [np.full(blk, lp) for lp in logp]
    if prm.causal:
        start = (i // blk) * blk
        idx_parts.append(np.arange(start, i + 1))
        prior_parts.append(np.zeros(i + 1 - start))
    idx = np.concatenate(idx_parts) if idx_parts else np.zeros(0, dtype=np.int64)
    prior = np.concatenate(prior_parts) if prior_parts else np.zeros(0)
    if idx.size == 0:
        # Non-causal row whose support is empty cannot happen (entmax always
        # selects at least one block); keep the shape honest anyway.
        return np.zeros(D), -np.inf, dict(idx=idx, a=np.zeros(0), prior=prior,
                                          chosen=chosen, logp=logp)
    ks = k_head[idx]
    logits = sf * (ks @ q_i) + prior
    mx = logits.max()
    w = np.exp(logits - mx)
    den = w.sum()
    a = w / den
    o = a @ v_head[idx]
    lse = mx + np.log(den)
    return o, lse, dict(idx=idx, a=a, prior=prior, chosen=chosen, logp=logp)


# ----------------------------------------------------------------------------- forward


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def forward_rows(q, k, v, prm: Params, rows, kbar=None, w=None):
    """Forward for selected rows only.

    ``q, k, v``: [B, H, T, D]; ``rows``: iterable of (b, h, i).  Returns a
    list of dicts (o, lse, tau, nsel, mask over all nb blocks, p over all nb
    blocks).  ``kbar`` may be passed to avoid re-pooling ([B, H, nb, D]);
    ``w`` ([H, D]) selects the learned summariser (R20).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    D = q.shape[-1]
    nb = k.shape[2] // prm.block
    cache = {}
    out = []
    for (b, h, i) in rows:
        if kbar is not None:
            kb = _as64(kbar[b, h])
        else:
            if (b, h) not in cache:
                cache[(b, h)] = summarise(k[b, h], prm, None if w is None else w[h])
            kb = cache[(b, h)]
        sel = select_row(q[b, h, i], kb, i, prm, D)
        o, lse, _ = attend_row(q[b, h, i], k[b, h], v[b, h], i, sel, prm, D)
        mask = np.zeros(nb, dtype=bool)
        mask[sel["cand"][sel["support"]]] = True
        pfull = np.zeros(nb)
        pfull[sel["cand"]] = sel["p"]
        out.append(dict(o=o, lse=lse, tau=sel["tau"], nsel=int(sel["support"].sum()),
                        mask=mask, p=pfull, z=sel["z"], cand=sel["cand"]))
    return out


def forward(q, k, v, prm: Params, w=None):
    """Full forward over every row: summaries, selection and attention.

    ``w`` ([H, D]) selects the learned summariser (R20); None is mean pooling.

    Returns a dict of arrays: kbar [B,H,nb,D], tau [B,H,T], nsel [B,H,T],
    mask [B,H,T,nb] (bool), p [B,H,T,nb], o [B,H,T,D], lse [B,H,T].
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, T, D = q.shape
    nb = T // prm.block
    kbar = np.zeros((B, H, nb, D))
    tau = np.full((B, H, T), np.nan)
    nsel = np.zeros((B, H, T), dtype=np.int64)
    mask = np.zeros((B, H, T, nb), dtype=bool)
    p = np.zeros((B, H, T, nb))
    o = np.zeros((B, H, T, D))
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            kb = summarise(k[b, h], prm, None if w is None else w[h])
            kbar[b, h] = kb
            for i in range(T):
                sel = select_row(q[b, h, i], kb, i, prm, D)
                oi, li, _ = attend_row(q[b, h, i], k[b, h], v[b, h], i, sel, prm, D)
                tau[b, h, i] = sel["tau"]
                nsel[b, h, i] = int(sel["support"].sum())
                mask[b, h, i, sel["cand"][sel["support"]]] = True
                p[b, h, i, sel["cand"]] = sel["p"]
                o[b, h, i] = oi
                lse[b, h, i] = li
    return dict(kbar=kbar, tau=tau, nsel=nsel, mask=mask, p=p, o=o, lse=lse)


# ----------------------------------------------------------------------------- backward


def _backward_row(q, k, v, dout, prm: Params, b, h, i, kb, grads):
    """Accumulate the gradient contributions of query row (b, h, i) into ``grads``.

    Per row (notation of the forward): a = softmax weights over the attended
    tokens, D_i = dout_i . o_i,

        dl_j   = a_j (dout_i . v_j - D_i)           (gradient of the logit)
        dv_j  += a_j dout_i
        dq_i  += fine_scale * sum_j dl_j k_j
        dk_j  += fine_scale * dl_j q_i
        G_b    = sum_{j in block b} dl_j              (gradient of log p_b)

    then through log p (dp_b = G_b / p_b) and alpha-entmax
    (:func:`oracle.entmax.entmax_jvp`) to dz, and through
    z_b = coarse_scale * q_i . kbar_b:

        dq_i    += coarse_scale * sum_b dz_b kbar_b
        dkbar_b += coarse_scale * dz_b q_i
    """
    D = q.shape[-1]
    blk = prm.block
    sf, sc = prm.scales(D)
    dq, dk, dv, dkbar = grads["dq"], grads["dk"], grads["dv"], grads["dkbar"]
    kh, vh = k[b, h], v[b, h]
    qi = q[b, h, i]
    sel = select_row(qi, kb, i, prm, D)
    oi, _, ctx = attend_row(qi, kh, vh, i, sel, prm, D)
    idx, a = ctx["idx"], ctx["a"]
    if idx.size == 0:
        return
    gi = dout[b, h, i]
    Di = gi @ oi
    dl = a * (vh[idx] @ gi - Di)
    dv[b, h, idx] += np.outer(a, gi)
    dq[b, h, i] += sf * (dl @ kh[idx])
    dk[b, h, idx] += sf * np.outer(dl, qi)
    chosen = ctx["chosen"]
    if chosen.size == 0:
        return
    # G over the selected candidate blocks (the causal own block carries
    # prior 0 and no gradient into Stage 1).
    G = dl[: chosen.size * blk].reshape(chosen.size, blk).sum(axis=1)
    pc = sel["p"]
    sup = sel["support"]
    g = np.zeros_like(pc)
    g[sup] = G / pc[sup]
    dz = entmax_jvp(pc, g, prm.alpha)
    cand = sel["cand"]
    dq[b, h, i] += sc * (dz @ kb[cand])
    dkbar[b, h, cand] += sc * np.outer(dz, qi)


def _grad_arrays(q):
    B, H, T, D = q.shape
    return dict(dq=np.zeros_like(q), dk=np.zeros_like(q), dv=np.zeros_like(q),
                dkbar=np.zeros((B, H, T // 64, D)))


def _pool_backward(k, prm: Params, w, grads, b, h):
    """Send dkbar of head (b, h) through Stage 0 into dk (and dw); keys of a
    partial last block (R22) have no summary and get nothing here."""
    nk = grads["dkbar"].shape[2] * prm.block
    if w is None:
        grads["dk"][b, h, :nk] += np.repeat(grads["dkbar"][b, h], prm.block, axis=0) / prm.block
        return
    dk, dw = pool_attention_vjp(k[b, h, :nk], w[h], grads["dkbar"][b, h], prm.block)
    grads["dk"][b, h, :nk] += dk
    grads["dw"][h] += dw


def backward(q, k, v, dout, prm: Params, w=None):
    """Gradients of the scalar <dout, O> with respect to q, k, v and the summaries.

    Sums the per-row contributions of :func:`_backward_row` over every row,
    then Stage 0 sends dkbar into dk: dkbar_b / block to every key of block
    b for mean pooling, :func:`pool_attention_vjp` for the learned
    summariser ``w`` ([H, D], R20), which also gives dw.
    Returns dict(dq, dk, dv, dkbar[, dw]) (dk includes the pooling path).
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, H, T, D = q.shape
    grads = _grad_arrays(q)
    if w is not None:
        grads["dw"] = np.zeros((H, D))
    for b in range(B):
        for h in range(H):
            kb = summarise(k[b, h], prm, None if w is None else w[h])
            for i in range(T):
                _backward_row(q, k, v, dout, prm, b, h, i, kb, grads)
            _pool_backward(k, prm, w, grads, b, h)
    return grads


def backward_rows(q, k, v, dout, prm: Params, rows, w=None):
    """The contributions of the given query rows (b, h, i) only.

    Returns the same dict as :func:`backward` but summed over ``rows``: dq
    is complete for those rows; dk, dv and dkbar are complete for any key
    block attended only by rows in ``rows`` (e.g. the last blocks of a causal
    head when ``rows`` holds every row from some position on).  dk includes
    the pooling path of the accumulated dkbar (and, with the learned
    summariser ``w``, dw from those rows).
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    grads = _grad_arrays(q)
    if w is not None:
        grads["dw"] = np.zeros((q.shape[1], q.shape[3]))
    pooled = {}
    for (b, h, i) in rows:
        if (b, h) not in pooled:
            pooled[(b, h)] = summarise(k[b, h], prm, None if w is None else w[h])
        _backward_row(q, k, v, dout, prm, b, h, i, pooled[(b, h)], grads)
    for (b, h) in pooled:
        _pool_backward(k, prm, w, grads, b, h)
    return grads


# ----------------------------------------------------------------------------- decode


def decode(q, kc, vc, prm: Params, kbar=None):
    """Decode: one new query per (sequence, head) against a KV cache.

    ``q``: [S, H, D]; ``kc, vc``: [S, H, N, D] with the new token already
    appended at position N-1 (R7).  The output equals row N-1 of a causal
    prefill over the cache: candidates are blocks 0..N/block-2, the last
    block is attended causally (all of it) with prior 0.  ``kbar`` may be
    given ([S, H, N/block, D]); by default it is pooled here.
    Returns dict(o [S,H,D], lse [S,H], nsel [S,H], mask [S,H,nb], tau [S,H]).
    """
    if not prm.causal:
        raise ValueError("decode is defined as the last row of a causal prefill")
    q, kc, vc = _as64(q), _as64(kc), _as64(vc)
    S, H, N, D = kc.shape
    nb = N // prm.block
    o = np.zeros((S, H, D))
    lse = np.zeros((S, H))
    nsel = np.zeros((S, H), dtype=np.int64)
    mask = np.zeros((S, H, nb), dtype=bool)
    tau = np.zeros((S, H))
    for s in range(S):
        for h in range(H):
            kb = _as64(kbar[s, h]) if kbar is not None else pool_blocks(kc[s, h], prm.block, prm.storage)
            sel = select_row(q[s, h], kb, N - 1, prm, D)
            oi, li, _ = attend_row(q[s, h], kc[s, h], vc[s, h], N - 1, sel, prm, D)
            o[s, h], lse[s, h], tau[s, h] = oi, li, sel["tau"]
            nsel[s, h] = int(sel["support"].sum())
            mask[s, h, sel["cand"][sel["support"]]] = True
    return dict(o=o, lse=lse, nsel=nsel, mask=mask, tau=tau)


# ----------------------------------------------------------------------------- decode cache maintenance


def cache_append(kc, vc, kbar, lens, k_new, v_new, prm: Params):
    """Append one token per (sequence, head) to a decode cache (R18).

    ``kc, vc``: [S, H, C, D] caches of capacity C (a multiple of the block);
    ``kbar``: [S, H, C/block, D] their summaries; ``lens``: [S] tokens
    already cached per sequence (each < C); ``k_new, v_new``: [S, H, D].
    Sequence s's token goes to position lens[s].  If that position is the
    last of its block, the block is now complete and its summary becomes the
    Stage-0 mean of its keys (the decoding path keeps one summary per chunk
    of the cache: the chunk-summarise stage among the code samples that the
    codewithpapers.app entry "DashAttention: Differentiable and Adaptive
    Sparse Hierarchical Attention" lists).  Summaries of incomplete blocks
    are left as they are.  Returns new arrays (kc, vc, kbar, lens + 1); the inputs are
    not modified.
    """
    kc, vc, kbar = _as64(kc).copy(), _as64(vc).copy(), _as64(kbar).copy()
    lens = np.asarray(lens, dtype=np.int64)
    S, H, C, D = kc.shape
    blk = prm.block
    if np.any(lens < 0) or np.any(lens >= C):
        raise ValueError("every length must lie in [0, capacity)")
    for s in range(S):
        n = int(lens[s])
        kc[s, :, n] = _as64(k_new[s])
        vc[s, :, n] = _as64(v_new[s])
        if n % blk == blk - 1:
            b = n // blk
            for h in range(H):
                kbar[s, h, b] = pool_blocks(kc[s, h, b * blk:(b + 1) * blk], blk, prm.storage)[0]
    return kc, vc, kbar, lens + 1


def decode_varlen(q, kc, vc, lens, prm: Params, kbar=None):
    """Decode with a cache length per sequence (R19).

    ``q``: [S, H, D]; ``kc, vc``: [S, H, C, D] with sequence s holding
    ``lens[s]`` tokens (1 <= lens[s] <= C), the new one last.  Entries beyond
    a sequence's length are never read.  The output of (s, h) is row
    lens[s]-1 of a causal prefill over the first lens[s] tokens: candidates
    are the complete blocks before the query's own block, which is attended
    over its cached tokens with prior 0.  ``kbar`` ([S, H, C/block, D]) may
    be given; only the entries of complete blocks before the query's own
    block are read.  By default they are pooled here.
    Returns dict(o [S,H,D], lse [S,H], nsel [S,H], mask [S,H,C/block], tau [S,H]).
    """
    if not prm.causal:
        raise ValueError("decode is defined as the last row of a causal prefill")
    q = _as64(q)
    S, H, C, D = kc.shape
    blk = prm.block
    lens = np.asarray(lens, dtype=np.int64)
    if np.any(lens < 1) or np.any(lens > C):
        raise ValueError("every length must lie in [1, capacity]")
    nbc = C // blk
    o = np.zeros((S, H, D))
    lse = np.zeros((S, H))
    nsel = np.zeros((S, H), dtype=np.int64)
    mask = np.zeros((S, H, nbc), dtype=bool)
    tau = np.zeros((S, H))
    for s in range(S):
        n = int(lens[s])
        i = n - 1
        ncand = i // blk  # complete blocks before the query's own block
        for h in range(H):
            k_head = _as64(kc[s, h, :n])
            v_head = _as64(vc[s, h, :n])
            if kbar is not None:
                kb = _as64(kbar[s, h, :ncand])
            else:
                kb = pool_blocks(k_head[:ncand * blk], blk, prm.storage)
            sel = select_row(q[s, h], kb, i, prm, D)
            oi, li, _ = attend_row(q[s, h], k_head, v_head, i, sel, prm, D)
            o[s, h], lse[s, h], tau[s, h] = oi, li, sel["tau"]
            nsel[s, h] = int(sel["support"].sum())
            mask[s, h, sel["cand"][sel["support"]]] = True
    return dict(o=o, lse=lse, nsel=nsel, mask=mask, tau=tau)
