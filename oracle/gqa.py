"""Grouped-query attention with entmax head aggregation, in plain float64 (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
may use this module; the HIP library shares no code with it.

Reading R21 (the pages are not explicit).  The montana-research page
("Non-dispersive attention at long context") contrasts methods that
aggregate the heads' block distributions with softmax before their top-k
cut (dispersive) with entmax head aggregation (not dispersive while each
head's support grows sublinearly), and the codewithpapers.app entry lists a
``repeat_kv`` step in the prefill block selection.  Here, with H query heads
sharing H_kv key/value heads (G = H / H_kv consecutive query heads per KV
head, as ``repeat_kv`` expands them):

* Stage 0 summarises each KV head's blocks (mean pooling);
* Stage 1 gives every query head h its own alpha-entmax p_h over the
  candidate blocks (scores against its KV head's summaries), and the group
  shares their mean pbar = (1/G) sum_h p_h: a distribution whose support is
  the union of the heads' supports;
* Stage 2: every head of the group attends the blocks of pbar's support
  with prior log pbar (its own block causally, prior 0), against its KV
  head's keys and values.

Gradients: G_b = sum over the group's heads of sum_{j in b} dS_ij is the
gradient of log pbar_b; dL/dp_h = G / (G_heads * pbar) for every head; then
each head's entmax Jacobian (entmax_jvp) gives dz_h, which reaches q_h and
the KV head's summaries.  dK and dV of a KV head sum its query heads' terms.
"""

from __future__ import annotations

import numpy as np

from .dash_ref import Params, _as64, attend_row, pool_blocks, select_row
from .entmax import entmax_jvp


def select_row_group(q_rows, kbar, i: int, prm: Params, D: int):
    """Stage 1 of one position for the G query heads of a group (R21).

    ``q_rows``: [G, D].  Returns dict(cand, p = pbar over the candidates,
    support = pbar > 0, heads = each head's :func:`select_row` result); the
    dict can be passed to :func:`attend_row` as the row's selection.
    """
    heads = [select_row(q_rows[g], kbar, i, prm, D) for g in range(q_rows.shape[0])]
    cand = heads[0]["cand"]
    if cand.size == 0:
        pbar = np.zeros(0)
    else:
        pbar = np.stack([h["p"] for h in heads]).mean(axis=0)
    return dict(cand=cand, p=pbar, support=pbar > 0, heads=heads)


def _group(H: int, Hkv: int) -> int:
    if Hkv < 1 or H % Hkv:
        raise ValueError("the query heads must split evenly over the KV heads")
    return H // Hkv


def forward_rows_gqa(q, k, v, prm: Params, rows, kbar=None):
    """Forward of rows (b, h, i) of a grouped-query layer (R21).

    ``q``: [B, H, T, D]; ``k, v``: [B, Hkv, T, D].  Returns a list of dicts:
    o, lse, pbar and union (over all nb blocks), and the head's own tau,
    nsel, mask, z and p (over its candidates).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, T, D = q.shape
    G = _group(H, k.shape[1])
    nb = T // prm.block
    pooled = {}
    out = []
    for (b, h, i) in rows:
        kv = h // G
        if kbar is not None:
            kb = _as64(kbar[b, kv])
        else:
            if (b, kv) not in pooled:
                pooled[(b, kv)] = pool_blocks(k[b, kv], prm.block, prm.storage)
            kb = pooled[(b, kv)]
        grp = select_row_group(q[b, kv * G:(kv + 1) * G, i], kb, i, prm, D)
        o, lse, _ = attend_row(q[b, h, i], k[b, kv], v[b, kv], i, grp, prm, D)
        own = grp["heads"][h - kv * G]
        cand = grp["cand"]
        mask = np.zeros(nb, dtype=bool)
        mask[cand[own["support"]]] = True
        union = np.zeros(nb, dtype=bool)
        union[cand[grp["support"]]] = True
        pbar = np.zeros(nb)
        pbar[cand] = grp["p"]
        out.append(dict(o=o, lse=lse, tau=own["tau"], nsel=int(own["support"].sum()), mask=mask, z=own["z"],
                        p=own["p"], cand=cand, union=union, pbar=pbar))
    return out


def forward_gqa(q, k, v, prm: Params):
    """Every row of a grouped-query layer: dict(kbar [B,Hkv,nb,D], o [B,H,T,D], lse [B,H,T],
    union [B,H,T,nb] (pbar's support), pbar [B,H,T,nb])."""
    q = _as64(q)
    B, H, T, D = q.shape
    Hkv = k.shape[1]
    nb = T // prm.block
    kbar = np.stack([[pool_blocks(_as64(k[b, kv]), prm.block, prm.storage) for kv in range(Hkv)] for b in range(B)])
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(T)]
    res = forward_rows_gqa(q, k, v, prm, rows, kbar=kbar)
    o = np.stack([r["o"] for r in res]).reshape(B, H, T, D)
    lse = np.array([r["lse"] for r in res]).reshape(B, H, T)
    union = np.stack([r["union"] for r in res]).reshape(B, H, T, nb)
    pbar = np.stack([r["pbar"] for r in res]).reshape(B, H, T, nb)
    return dict(kbar=kbar, o=o, lse=lse, union=union, pbar=pbar)


def backward_gqa(q, k, v, dout, prm: Params):
    """Gradients of <dout, O> for a grouped-query layer (R21).

    Returns dict(dq [B,H,T,D], dk, dv [B,Hkv,T,D], dkbar [B,Hkv,nb,D]); dk
    includes the mean-pooling path.
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, H, T, D = q.shape
    Hkv = k.shape[1]
    G = _group(H, Hkv)
    blk = prm.block
    sf, sc = prm.scales(D)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dkbar = np.zeros((B, Hkv, T // blk, D))
    for b in range(B):
        for kv in range(Hkv):
            kh, vh = k[b, kv], v[b, kv]
            kb = pool_blocks(kh, blk, prm.storage)
            for i in range(T):
                qg = q[b, kv * G:(kv + 1) * G, i]
                grp = select_row_group(qg, kb, i, prm, D)
                chosen = grp["cand"][grp["support"]]
                Gsum = np.zeros(chosen.size)
                for g in range(G):
                    h = kv * G + g
                    oi, _, ctx = attend_row(qg[g], kh, vh, i, grp, prm, D)
                    idx, a = ctx["idx"], ctx["a"]
                    gi = dout[b, h, i]
                    dl = a * (vh[idx] @ gi - gi @ oi)
                    dv[b, kv, idx] += np.outer(a, gi)
                    dq[b, h, i] += sf * (dl @ kh[idx])
                    dk[b, kv, idx] += sf * np.outer(dl, qg[g])
                    if chosen.size:
                        Gsum += dl[: chosen.size * blk].reshape(chosen.size, blk).sum(axis=1)
                if chosen.size == 0:
                    continue
                cand = grp["cand"]
                gp = np.zeros(cand.size)
                gp[grp["support"]] = Gsum / (G * grp["p"][grp["support"]])
                for g in range(G):
                    h = kv * G + g
                    dz = entmax_jvp(grp["heads"][g]["p"], gp, prm.alpha)
                    dq[b, h, i] += sc * (dz @ kb[cand])
                    dkbar[b, kv, cand] += sc * np.outer(dz, qg[g])
            dk[b, kv] += np.repeat(dkbar[b, kv], blk, axis=0) / blk
    return dict(dq=dq, dk=dk, dv=dv, dkbar=dkbar)


def decode_gqa(q, kc, vc, lens, prm: Params):
    """Decode for grouped-query heads (R21 applied to the decode row, R19 lengths).

    ``q``: [S, H, D]; ``kc, vc``: [S, Hkv, C, D] holding ``lens[s]`` tokens of
    sequence s (the new one last; lens None: all C).  Each query head attends
    its KV head's cache with the group's aggregated selection: row lens[s]-1
    of a grouped-query causal prefill over the first lens[s] tokens.
    Returns dict(o [S,H,D], lse [S,H], nsel [S,H] (each head's own support),
    union [S,H,C/block] (the group's), tau [S,H]).
    """
    q = _as64(q)
    S, H, D = q.shape
    Hkv, C = kc.shape[1], kc.shape[2]
    G = _group(H, Hkv)
    blk = prm.block
    lens = np.full(S, C) if lens is None else np.asarray(lens, dtype=np.int64)
    if np.any(lens < 1) or np.any(lens > C):
        raise ValueError("every length must lie in [1, capacity]")
    o = np.zeros((S, H, D))
    lse = np.zeros((S, H))
    nsel = np.zeros((S, H), dtype=np.int64)
    union = np.zeros((S, H, C // blk), dtype=bool)
    tau = np.zeros((S, H))
    for s in range(S):
        n = int(lens[s])
        i = n - 1
        for kv in range(Hkv):
            kh = _as64(kc[s, kv, :n])
            vh = _as64(vc[s, kv, :n])
            kb = pool_blocks(kh[: (i // blk) * blk], blk, prm.storage)
            grp = select_row_group(q[s, kv * G:(kv + 1) * G], kb, i, prm, D)
            for g in range(G):
                h = kv * G + g
                o[s, h], lse[s, h], _ = attend_row(q[s, h], kh, vh, i, grp, prm, D)
                own = grp["heads"][g]
                nsel[s, h] = int(own["support"].sum())
                tau[s, h] = own["tau"]
                union[s, h, grp["cand"][grp["support"]]] = True
    return dict(o=o, lse=lse, nsel=nsel, union=union, tau=tau)
