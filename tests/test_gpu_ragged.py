"""GPU parity of a causal prefill whose length is not a multiple of 64.

dash_fwd and dash_bwd (through the C ABI) with a partial last block against
the float64 oracle (summaries of the complete blocks only): every row and
gradient of small cases, sampled rows of a 16K prefill, and the identity with
the whole-block path on zero-padded inputs.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from differentiable_adaptive_block_amd import inputs
from parity import check_rows, rel_l2, unpack_mask

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.double().cpu().numpy()


def _make(B, H, T, D, dtype, planted, seed, with_dout=True):
    Tp = 64 * ((T + 63) // 64)
    w = inputs.make_prefill(B, H, Tp, D, dtype, True, planted, seed=seed, device="cpu", with_dout=with_dout)
    return {k: v[:, :, :T].contiguous().to(DEV) for k, v in w.items()}


def _gpu(r, T):
    nbf = T // 64
    sel = r["sel"]
    mask = unpack_mask(sel.mask, -(-T // 64))
    assert not mask[:, :, :T, nbf:].any(), "the partial block was selected"
    return dict(o=r["o"].float().cpu().numpy(), lse=r["lse"].cpu().numpy(), tau=sel.tau[:, :, :T].cpu().numpy(),
                nsel=sel.nsel[:, :, :T].cpu().numpy(), mask=mask[:, :, :T, :nbf])


CASES = [
    # name, B, H, T, D, dtype, alpha, coarse multiple, planted
    ("bf16-T10", 1, 2, 10, 128, "bf16", 1.5, 4.0, (1, 3)),
    ("bf16-T65", 1, 2, 65, 128, "bf16", 1.5, 4.0, (1, 3)),
    ("bf16-T100-d64", 1, 2, 100, 64, "bf16", 1.25, 4.0, (1, 3)),
    ("bf16-T1000", 1, 2, 1000, 128, "bf16", 1.5, 4.0, (1, 4)),
    ("bf16-T1089-a2", 1, 1, 1089, 128, "bf16", 2.0, 4.0, (1, 4)),
    ("fp32-T200-d64", 1, 2, 200, 64, "fp32", 1.5, 4.0, (1, 3)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ragged_forward_and_backward_small(case):
    from differentiable_adaptive_block_amd import api
    name, B, H, T, D, dtype, alpha, csm, planted = case
    _say(f"[ragged] {name} B{B} H{H} T{T} D{D} {dtype} alpha={alpha}")
    w = _make(B, H, T, D, dtype, planted, 91 + T)
    cs = csm / math.sqrt(D)
    r = api.forward(w["q"], w["k"], w["v"], alpha=alpha, causal=True, coarse_scale=cs)
    g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"])
    torch.cuda.synchronize()
    prm = oracle.Params(alpha=alpha, causal=True, coarse_scale=cs, storage=dtype)
    q64, k64, v64, d64 = (_np64(w[x]) for x in ("q", "k", "v", "dout"))
    nbf = T // 64
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(_np64(r["kbar"][b, h, :nbf]), oracle.summarise(k64[b, h], prm))
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(T)]
    ora = oracle.forward_rows(q64, k64, v64, prm, rows)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    st = check_rows(_gpu(r, T), ora, rows, tdt, alpha, name)
    ref = oracle.backward(q64, k64, v64, d64, prm)
    errs = {n: rel_l2(_np64(g[n]), ref[n]) for n in ("dq", "dk", "dv")}
    errs["dkbar"] = rel_l2(_np64(g["dkbar"][:, :, :nbf]), ref["dkbar"]) if nbf else 0.0
    _say(f"  forward {st}; rel-L2 {errs}")
    for n, e in errs.items():
        assert e <= 5e-2, (name, n, e)
    assert not g["dkbar"][:, :, nbf:].any()  # the partial block has no summary


def test_ragged_equals_zero_padded_whole_blocks():
    from differentiable_adaptive_block_amd import api
    B, H, T, D = 1, 2, 1000, 128
    w = _make(B, H, T, D, "bf16", (1, 4), 95)
    Tp = 1024
    pad = lambda x: torch.nn.functional.pad(x, (0, 0, 0, Tp - T)).contiguous()  # noqa: E731
    cs = 4.0 / math.sqrt(D)
    r = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=cs)
    g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"])
    rp = api.forward(pad(w["q"]), pad(w["k"]), pad(w["v"]), alpha=1.5, causal=True, coarse_scale=cs)
    lsep = rp["lse"].clone()
    lsep[:, :, T:] = float("inf")
    gp = api.backward(pad(w["q"]), pad(w["k"]), pad(w["v"]), rp["o"], lsep, pad(w["dout"]), rp["kbar"], rp["sel"],
                      rp["params"])
    torch.cuda.synchronize()
    assert torch.equal(r["o"], rp["o"][:, :, :T]) and torch.equal(r["lse"], rp["lse"][:, :, :T])
    assert torch.equal(r["kbar"], rp["kbar"])
    for n in ("dq", "dk", "dv"):
        assert torch.equal(g[n], gp[n][:, :, :T]), n
    assert torch.equal(g["dkbar"], gp["dkbar"])


def test_ragged_16k_sampled():
    from differentiable_adaptive_block_amd import api
    B, H, T, D = 1, 32, 16384 - 37, 128
    _say(f"[ragged] 16K prefill T{T}")
    w = inputs.make_prefill(B, H, 16384, D, "bf16", True, (1, 8), seed=96, device=DEV, with_dout=False)
    q, k, v = (w[x][:, :, :T].contiguous() for x in ("q", "k", "v"))
    cs = 1.0 / math.sqrt(D)
    r = api.forward(q, k, v, alpha=1.5, causal=True, coarse_scale=cs)
    torch.cuda.synchronize()
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=cs, storage="bf16")
    rng = np.random.default_rng(97)
    rows = [(0, int(h), int(i)) for h, i in zip(rng.integers(0, H, 8), rng.integers(64, T, 8))]
    rows += [(0, 3, T - 1), (0, 17, T - 30), (0, 9, 64 * (T // 64))]
    heads = sorted({h for _, h, _ in rows})
    q64 = np.zeros((1, H, T, D))
    k64 = np.zeros((1, H, T, D))
    v64 = np.zeros((1, H, T, D))
    for h in heads:
        q64[0, h], k64[0, h], v64[0, h] = _np64(q[0, h]), _np64(k[0, h]), _np64(v[0, h])
    ora = oracle.forward_rows(q64, k64, v64, prm, rows)
    st = check_rows(_gpu(r, T), ora, rows, torch.bfloat16, 1.5, "ragged 16K")
    _say(f"  ok {st}")


def test_ragged_autograd():
    from differentiable_adaptive_block_amd import api
    w = _make(1, 2, 300, 128, "bf16", (1, 3), 98)
    q, k, v = (w[x].clone().requires_grad_(True) for x in ("q", "k", "v"))
    cs = 4 / math.sqrt(128)
    o = api.dash_attention(q, k, v, 1.5, True, None, cs)
    (o.float() * w["dout"].float()).sum().backward()
    r = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=cs)
    g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"])
    torch.cuda.synchronize()
    assert o.shape == w["q"].shape
    for t, n in ((q, "dq"), (k, "dk"), (v, "dv")):
        assert torch.equal(t.grad, g[n]), n
