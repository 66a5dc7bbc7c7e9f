"""Seeded synthetic workloads for the DashAttention hot path.

This module only draws random tensors and builds the planted queries; it
holds none of the method's arithmetic.  Both the HIP path and the oracle
consume the tensors it returns, bit for bit.

Workload recipe (the pages measure on model checkpoints and benchmark suites
that are not used here; these seeded tensors stand in for their 16K-96K
prefill and 96K decode workloads):

* keys, values and output gradients are iid N(0, 1), drawn in float32 and
  rounded to the tensor dtype;
* planted queries: q_i = 0.5 * g_i + sum_{b in P_i} kbar_b / |kbar_b| with
  g_i iid N(0, 1) and kbar_b the exact float64 mean of block b's (rounded)
  keys, i.e. the unit direction of that block's key sum; P_i is a uniformly
  drawn set of min(U{lo..hi}, c_i) distinct candidate blocks of query i
  (c_i = own block index when causal, else all blocks); then rounded;
* seeds: 1000 + config number for the inputs, + 100 for dO.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK = 64


@dataclass
class Workload:
    name: str
    kind: str  # "prefill" or "decode"
    dtype: str  # "bf16" or "fp32"
    alpha: float | tuple
    causal: bool
    coarse_scale: float
    fine_scale: float
    shape: dict
    planted: tuple | None
    seed: int
    note: str = ""
    extra: dict = field(default_factory=dict)


def _cfg(name, kind, dtype, alpha, causal, cs_mult, shape, planted, seed, note=""):
    D = shape["D"]
    return Workload(name, kind, dtype, alpha, causal, cs_mult / math.sqrt(D), 1.0 / math.sqrt(D),
                    shape, planted, seed, note)


CONFIGS = {
    # tiny non-causal forward + backward, float32
    "tiny512": _cfg("tiny512", "prefill", "fp32", 1.5, False, 1.0, dict(B=1, H=2, T=512, D=64), None,
                    1001),
    # same inputs with a 16x larger coarse scale, so the masks are exercised
    "tiny512_sc16": _cfg("tiny512_sc16", "prefill", "fp32", 1.5, False, 16.0, dict(B=1, H=2, T=512, D=64),
                         None, 1001),
    # causal prefill at 16K
    "prefill16k": _cfg("prefill16k", "prefill", "bf16", 1.5, True, 1.0, dict(B=1, H=32, T=16384, D=128),
                       (1, 8), 1002),
    # causal prefill at 64K, coarse scale 2/sqrt(128)
    "prefill64k": _cfg("prefill64k", "prefill", "bf16", 1.5, True, 2.0, dict(B=1, H=32, T=65536, D=128),
                       (1, 8), 1003),
    # the same at a coarse scale that gives about 8% selected pairs
    "prefill64k_sc7": _cfg("prefill64k_sc7", "prefill", "bf16", 1.5, True, 7.0,
                           dict(B=1, H=32, T=65536, D=128), (1, 8), 1003, "calibrated coarse scale 7/sqrt(128)"),
    # causal prefill at 96K (the longest prefill the pages quote), coarse scale 2/sqrt(128)
    "prefill96k": _cfg("prefill96k", "prefill", "bf16", 1.5, True, 2.0, dict(B=1, H=32, T=98304, D=128),
                       (1, 8), 1006),
    # decode: 16 sequences x 32 heads, 98304-token bf16 cache
    "decode96k": _cfg("decode96k", "decode", "bf16", 1.5, True, 1.0, dict(S=16, H=32, N=98304, D=128),
                      (1, 16), 1004),
    "decode96k_sc5": _cfg("decode96k_sc5", "decode", "bf16", 1.5, True, 5.0,
                          dict(S=16, H=32, N=98304, D=128), (1, 16), 1004, "calibrated coarse scale 5/sqrt(128)"),
    # training step (forward + backward), alpha swept over {1.25, 1.5}
    "train16k": _cfg("train16k", "prefill", "bf16", (1.25, 1.5), True, 1.0,
                     dict(B=2, H=16, T=16384, D=128), (1, 8), 1005),
}


def torch_dtype(dtype: str):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, dtype, device, chunk_rows=None):
    """iid N(0,1) drawn in float32, rounded to ``dtype``; drawn along dim 0 in chunks."""
    out = torch.empty(shape, dtype=dtype, device=device)
    n0 = shape[0]
    step = chunk_rows or n0
    for s in range(0, n0, step):
        e = min(n0, s + step)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=g, dtype=torch.float32,
                               device=device).to(dtype)
    return out


def _planted_rows(kh, rows_pos, causal, lo, hi, g, device):
    """Planted query directions for one head.

    ``kh``: [T, D] keys of the head (already rounded); ``rows_pos``: int64
    positions of the queries.  Returns the float64 sum of unit block
    directions for each row ([len(rows_pos), D]).
    """
    T, D = kh.shape
    nb = T // BLOCK
    kb = kh.double().view(nb, BLOCK, D).sum(dim=1)
    unit = kb / kb.norm(dim=1, keepdim=True)
    R = rows_pos.numel()
    c = (rows_pos // BLOCK) if causal else torch.full((R,), nb, device=device, dtype=torch.int64)
    cnt = torch.randint(lo, hi + 1, (R,), generator=g, device=device)
    cnt = torch.minimum(cnt, c)
    kmax = min(hi, nb)
    out = torch.zeros((R, D), dtype=torch.float64, device=device)
    step = max(1, (1 << 24) // max(nb, 1))
    for s in range(0, R, step):
        e = min(R, s + step)
        r = torch.rand((e - s, nb), generator=g, device=device)
        bidx = torch.arange(nb, device=device)[None, :]
        r = torch.where(bidx < c[s:e, None], r, torch.full_like(r, 2.0))
        pick = torch.topk(r, kmax, dim=1, largest=False).indices  # [e-s, kmax]
        valid = torch.arange(kmax, device=device)[None, :] < cnt[s:e, None]
        out[s:e] = (unit[pick] * valid[..., None].double()).sum(dim=1)
    return out


def make_prefill(B, H, T, D, dtype="bf16", causal=True, planted=(1, 8), seed=0, device="cpu",
                 with_dout=True, kv_heads=None):
    """Q, K, V (and dO): q and dO [B, H, T, D], k and v [B, kv_heads, T, D]
    (kv_heads defaults to H; query head h is planted toward the blocks of
    KV head h // (H / kv_heads)).

    ``planted=None`` gives iid N(0,1) queries; otherwise (lo, hi) plants each
    query toward lo..hi earlier blocks as described in the module docstring.
    """
    if T % BLOCK:
        raise ValueError("T must be a multiple of 64")
    Hkv = H if kv_heads is None else kv_heads
    if Hkv < 1 or H % Hkv:
        raise ValueError("kv_heads must divide H")
    G = H // Hkv
    td = torch_dtype(dtype)
    g = _gen(seed, device)
    k = _randn((B * Hkv, T, D), g, td, device, chunk_rows=4).view(B, Hkv, T, D)
    v = _randn((B * Hkv, T, D), g, td, device, chunk_rows=4).view(B, Hkv, T, D)
    if planted is None:
        q = _randn((B * H, T, D), g, td, device, chunk_rows=4).view(B, H, T, D)
    else:
        lo, hi = planted
        q = torch.empty((B, H, T, D), dtype=td, device=device)
        pos = torch.arange(T, device=device)
        for b in range(B):
            for h in range(H):
                noise = torch.randn((T, D), generator=g, dtype=torch.float32, device=device).double()
                qp = 0.5 * noise + _planted_rows(k[b, h // G], pos, causal, lo, hi, g, device)
                q[b, h] = qp.float().to(td)
    out = dict(q=q, k=k, v=v)
    if with_dout:
        g2 = _gen(seed + 100, device)
        out["dout"] = _randn((B * H, T, D), g2, td, device, chunk_rows=4).view(B, H, T, D)
    return out


def make_decode(S, H, N, D, dtype="bf16", planted=(1, 16), seed=0, device="cpu", lens=None, beyond=None,
                kv_heads=None):
    """Decode workload: q [S, H, D] and caches k, v [S, H, N, D].

    The new token is the last cached token: position N-1, or lens[s]-1 when
    a list of per-sequence lengths is given (N is then the capacity).
    Planted blocks are drawn among the query's candidates, the complete
    blocks before its own.  ``beyond`` (a float, e.g. NaN) overwrites the
    cache entries at positions >= lens[s] after everything is drawn.
    ``kv_heads`` (default H) gives caches of that many heads, query head h
    planted toward KV head h // (H / kv_heads).
    """
    if N % BLOCK:
        raise ValueError("N must be a multiple of 64")
    if lens is not None and (len(lens) != S or min(lens) < 1 or max(lens) > N):
        raise ValueError("lens must hold S lengths in [1, N]")
    Hkv = H if kv_heads is None else kv_heads
    if Hkv < 1 or H % Hkv:
        raise ValueError("kv_heads must divide H")
    G = H // Hkv
    td = torch_dtype(dtype)
    g = _gen(seed, device)
    kc = torch.empty((S, Hkv, N, D), dtype=td, device=device)
    vc = torch.empty((S, Hkv, N, D), dtype=td, device=device)
    for s in range(S):
        kc[s] = _randn((Hkv, N, D), g, td, device, chunk_rows=4)
    for s in range(S):
        vc[s] = _randn((Hkv, N, D), g, td, device, chunk_rows=4)
    q = torch.empty((S, H, D), dtype=td, device=device)
    for s in range(S):
        pos = torch.tensor([(N if lens is None else int(lens[s])) - 1], device=device)
        for h in range(H):
            noise = torch.randn((1, D), generator=g, dtype=torch.float32, device=device).double()
            if planted is None:
                qp = noise
            else:
                qp = 0.5 * noise + _planted_rows(kc[s, h // G], pos, True, planted[0], planted[1], g, device)
            q[s, h] = qp[0].float().to(td)
    if lens is not None and beyond is not None:
        for s in range(S):
            kc[s, :, int(lens[s]):] = beyond
            vc[s, :, int(lens[s]):] = beyond
    return dict(q=q, k=kc, v=vc)


def make_config(name: str, device="cpu", with_dout=True):
    """Inputs of a named workload (see ``CONFIGS``)."""
    w = CONFIGS[name]
    sh = w.shape
    if w.kind == "decode":
        return w, make_decode(sh["S"], sh["H"], sh["N"], sh["D"], w.dtype, w.planted, w.seed, device)
    return w, make_prefill(sh["B"], sh["H"], sh["T"], sh["D"], w.dtype, w.causal, w.planted, w.seed,
                           device, with_dout)
