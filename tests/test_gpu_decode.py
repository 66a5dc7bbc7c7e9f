"""GPU decode parity: dash_pool + dash_decode against the float64 oracle."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from differentiable_adaptive_block_amd import inputs
from parity import check_mask_row, tau_tol, tol_out

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.double().cpu().numpy()


def _check(rows, q, kc, vc, kbar_gpu, out, prm, what):
    """Oracle rows (s, h) vs GPU decode outputs."""
    max_abs, mean_abs = tol_out(torch.bfloat16)
    errs = []
    for (s, h) in rows:
        k64 = _np64(kc[s, h])
        kb = oracle.pool_blocks(k64, 64, "bf16")
        np.testing.assert_array_equal(_np64(kbar_gpu[s, h]), kb, err_msg=f"{what} kbar {(s, h)}")
        N = k64.shape[0]
        qq = _np64(q[s, h])
        sel = oracle.select_row(qq, kb, N - 1, prm, qq.size)
        o, lse, _ = oracle.attend_row(qq, k64, _np64(vc[s, h]), N - 1, sel, prm, qq.size)
        errs.append(np.abs(out["o"][s, h].double().cpu().numpy() - o))
        assert abs(float(out["lse"][s, h]) - lse) <= 1e-3, (what, s, h, float(out["lse"][s, h]), lse)
        # the selected set, bit for bit outside the tie band; the count agrees with it
        flips = check_mask_row(out["mask"][s, h], sel, prm.alpha, f"{what} {(s, h)}")
        ns = int(out["nsel"][s, h])
        assert ns == int(sel["support"].sum()) if flips == 0 else abs(ns - int(sel["support"].sum())) <= flips
        assert ns == int(np.unpackbits(out["mask"][s, h].cpu().numpy().view(np.uint8)).sum())
        if sel["cand"].size:
            assert abs(float(out["tau"][s, h]) - sel["tau"]) <= tau_tol(sel["tau"])
    E = np.stack(errs)
    assert E.max() <= max_abs and E.mean() <= mean_abs, (what, E.max(), E.mean())
    return float(E.max()), float(E.mean())


@pytest.mark.parametrize("N,cs_mult", [(1024, 4.0), (64, 1.0), (4096, 1.0), (4096, 5.0)])
def test_decode_small(N, cs_mult):
    from differentiable_adaptive_block_amd import api
    S, H, D = 2, 3, 128
    _say(f"[decode] S{S} H{H} N{N} coarse {cs_mult}/sqrt(D)")
    w = inputs.make_decode(S, H, N, D, "bf16", (1, 4), seed=N + int(cs_mult), device="cpu")
    q, kc, vc = (w[x].to(DEV) for x in ("q", "k", "v"))
    kbar = api.pool(kc.view(1, S * H, N, D)).view(S, H, N // 64, D)
    cs = cs_mult / math.sqrt(D)
    out = api.decode(q, kc, vc, kbar, alpha=1.5, coarse_scale=cs)
    torch.cuda.synchronize()
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=cs, storage="bf16")
    st = _check([(s, h) for s in range(S) for h in range(H)], q, kc, vc, kbar, out, prm, f"N{N}")
    _say(f"  ok max/mean abs {st}")


def test_decode_equals_last_prefill_row():
    from differentiable_adaptive_block_amd import api
    S, H, N, D = 1, 4, 2048, 128
    w = inputs.make_decode(S, H, N, D, "bf16", (1, 4), seed=5, device="cpu")
    q, kc, vc = (w[x].to(DEV) for x in ("q", "k", "v"))
    kbar = api.pool(kc)
    cs = 3.0 / math.sqrt(D)
    dec = api.decode(q, kc, vc, kbar, alpha=1.5, coarse_scale=cs)
    qp = torch.zeros_like(kc)
    qp[:, :, N - 1] = q
    pre = api.forward(qp, kc, vc, alpha=1.5, causal=True, coarse_scale=cs)
    torch.cuda.synchronize()
    assert torch.equal(pre["kbar"], kbar)
    diff = (dec["o"].float() - pre["o"][:, :, N - 1].float()).abs().max().item()
    assert diff <= 1e-2, diff
    # the prefill normaliser sums the weights as rounded to bf16 (each within
    # 2^-8 relative), decode sums them in fp32: logs within -ln(1 - 2^-8)
    assert torch.allclose(dec["lse"], pre["lse"][:, :, N - 1], atol=4e-3)


@pytest.mark.parametrize("name", ["decode96k", "decode96k_sc5"])
def test_decode_96k_sampled(name):
    from differentiable_adaptive_block_amd import api
    wl = inputs.CONFIGS[name]
    sh = wl.shape
    _say(f"[decode] {name} full size {sh}")
    w = inputs.make_decode(sh["S"], sh["H"], sh["N"], sh["D"], wl.dtype, wl.planted, wl.seed, device=DEV)
    q, kc, vc = w["q"], w["k"], w["v"]
    S, H, N, D = kc.shape
    kbar = api.pool(kc.view(1, S * H, N, D)).view(S, H, N // 64, D)
    out = api.decode(q, kc, vc, kbar, alpha=wl.alpha, coarse_scale=wl.coarse_scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = [(int(s), int(h)) for s, h in zip(rng.integers(0, S, 6), rng.integers(0, H, 6))]
    prm = oracle.Params(alpha=wl.alpha, causal=True, coarse_scale=wl.coarse_scale, storage="bf16")
    st = _check(rows, q, kc, vc, kbar, out, prm, name)
    sparsity = 1.0 - float(out["nsel"].double().mean()) / (N // 64 - 1)
    _say(f"  ok max/mean abs {st}; block sparsity {sparsity:.4f}")
