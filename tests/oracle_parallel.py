"""The float64 oracle over many query rows at once, in worker processes.

Test infrastructure only: it splits rows of one (batch, head) over spawned
processes (one BLAS thread each) and gathers the oracle's own results.  Rows
are independent in the forward, and the backward's contributions of disjoint
row sets add up, so the results are the oracle's, unchanged.
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

_STATE = {}


def default_workers() -> int:
    # the GPU machines give a process 16 CPUs whatever os.cpu_count() reports
    return max(1, min(16, os.cpu_count() or 1))


def _bits(t):
    """A bf16 torch tensor as uint16 bit patterns (compact to ship to workers)."""
    import torch

    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _f64(x):
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _init(arrays, prm):
    _STATE["x"] = {k: _f64(v)[None, None] for k, v in arrays.items()}
    _STATE["prm"] = prm


def _forward_job(rows):
    import oracle

    x = _STATE["x"]
    kb = x.get("kbar")
    return oracle.forward_rows(x["q"], x["k"], x["v"], _STATE["prm"], [(0, 0, i) for i in rows],
                               kbar=kb)


def _backward_job(rows):
    import oracle

    x = _STATE["x"]
    g = oracle.backward_rows(x["q"], x["k"], x["v"], x["dout"], _STATE["prm"], [(0, 0, i) for i in rows])
    return {k: v[0, 0] for k, v in g.items()}


def _select_job(rows):
    import oracle

    x = _STATE["x"]
    D = x["q"].shape[-1]
    return [oracle.select_row(x["q"][0, 0, i], x["kbar"][0, 0], i, _STATE["prm"], D) for i in rows]


def _run(job, arrays, prm, rows, workers):
    workers = workers or default_workers()
    chunks = [rows[w::workers] for w in range(workers)]
    chunks = [c for c in chunks if c]
    keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in keep:
        os.environ[k] = "1"
    try:
        with mp.get_context("spawn").Pool(len(chunks), initializer=_init, initargs=(arrays, prm)) as pool:
            res = pool.map(job, chunks)
    finally:
        for k, v in keep.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return chunks, res


def _arrays(**tensors):
    out = {}
    for k, t in tensors.items():
        if t is None:
            continue
        import torch

        out[k] = _bits(t) if t.dtype == torch.bfloat16 else t.detach().double().cpu().numpy()
    return out


def forward_rows(q, k, v, prm, rows, kbar=None, workers=None):
    """oracle.forward_rows of one head's rows (q, k, v: [T, D] torch tensors);
    returns the per-row dicts in the order of ``rows``."""
    chunks, res = _run(_forward_job, _arrays(q=q, k=k, v=v, kbar=kbar), prm, list(rows), workers)
    by_row = {}
    for c, r in zip(chunks, res):
        by_row.update(zip(c, r))
    return [by_row[i] for i in rows]


def select_rows(q, kbar, prm, rows, workers=None):
    """oracle.select_row of one head's rows (q [T, D], kbar [nb, D])."""
    chunks, res = _run(_select_job, _arrays(q=q, kbar=kbar), prm, list(rows), workers)
    by_row = {}
    for c, r in zip(chunks, res):
        by_row.update(zip(c, r))
    return [by_row[i] for i in rows]


def backward_head(q, k, v, dout, prm, workers=None):
    """oracle.backward of one head (q, k, v, dout: [T, D] torch tensors), every
    row: dict(dq, dk, dv, dkbar) as [T, D] / [nb, D] float64 arrays."""
    T = q.shape[0]
    _, res = _run(_backward_job, _arrays(q=q, k=k, v=v, dout=dout), prm, list(range(T)), workers)
    out = {}
    for r in res:
        for n, a in r.items():
            out[n] = a.copy() if n not in out else out[n] + a
    return out
