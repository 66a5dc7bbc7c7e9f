"""GPU parity of the low-density Stage-2 schedule (dash_fwd_attend_lowdens).

The schedule computes the same attention as the dense walk by another route
(per (row, block) partials merged per row), so it is held to the same bar:
O and LSE against the float64 oracle (tests/parity.py tolerances) on every
row of small cases that span several tiles, and on sampled rows of the
calibrated 64K prefill, where the whole output is also compared with the
dense walk's.  The cases cover every tile taken (ratio 0), a mix decided by
the ratio, a workspace too small for every qualifying tile (the rest fall
back to the dense walk in the same call), head dim 64 and 128, a last tile
of a single block, the longest prefill (98304 tokens) with every tile
through the schedule, dash_fwd's own choice with a workspace, and reruns
(bit-identical).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle_parallel
from differentiable_adaptive_block_amd import inputs
from parity import check_out_rows, check_rows, unpack_mask, tol_out

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _api():
    from differentiable_adaptive_block_amd import api
    return api


def _lib():
    from differentiable_adaptive_block_amd import _lib as L
    return L


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.double().cpu().numpy()


def _lowdens(w, cs, ratio, pairs=None, alpha=1.5, extra_bytes=0):
    """Selection, then Stage 2 through dash_fwd_attend_lowdens with room for
    ``pairs`` pairs (None: all the qualifying tiles' pairs), plus ``extra_bytes``."""
    api, L = _api(), _lib()
    q, k, v = w["q"], w["k"], w["v"]
    B, H, T, D = q.shape
    p = api.make_params(q, alpha, True, None, cs)
    sel = api.alloc_selection(p, q.device, want_mask=True)
    csel = sel.as_c()
    kbar = torch.empty((B, H, T // 64, D), dtype=q.dtype, device=q.device)
    st = torch.cuda.current_stream().cuda_stream
    L.fwd_select(p, q.data_ptr(), k.data_ptr(), kbar.data_ptr(), csel, st)
    need = api.lowdens_pairs(sel, p, ratio)
    n = need if pairs is None else pairs
    wsb = L.fwd_lowdens_workspace_bytes(p, n) + extra_bytes
    ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    L.fwd_attend_lowdens(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), kbar.data_ptr(), csel, ratio, o.data_ptr(),
                         lse.data_ptr(), ws.data_ptr(), wsb, st)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, kbar=kbar, sel=sel, p=p, need=need)


def _dense(w, cs, alpha=1.5):
    r = _api().forward(w["q"], w["k"], w["v"], alpha=alpha, causal=True, coarse_scale=cs, want_mask=True)
    torch.cuda.synchronize()
    return r


SMALL = [
    # name, B, H, T, D, coarse multiple of 1/sqrt(D), planted, ratio, share of the pairs the workspace holds
    ("all-tiles-d128", 1, 2, 2048, 128, 7.0, (1, 8), 0.0, 1.0),
    ("all-tiles-d64", 2, 1, 1600, 64, 7.0, (1, 4), 0.0, 1.0),
    ("ratio-mix", 1, 2, 6144, 128, 16.0, (1, 8), 4.0, 1.0),
    ("half-workspace", 1, 2, 2048, 128, 7.0, (1, 8), 0.0, 0.5),
    ("dense-scale-all-tiles", 1, 1, 1088, 128, 1.0, (1, 8), 0.0, 1.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_lowdens_small_full_oracle(case):
    name, B, H, T, D, csm, planted, ratio, share = case
    _say(f"[lowdens] {name} B{B} H{H} T{T} D{D} coarse {csm}/sqrt(D) ratio {ratio} workspace share {share}")
    w = inputs.make_prefill(B, H, T, D, "bf16", True, planted, seed=91 + T + D, device="cpu", with_dout=False)
    w = {k: v.to(DEV) for k, v in w.items()}
    cs = csm / math.sqrt(D)
    full = int(w["q"].shape[0] * w["q"].shape[1] * T + _dense(w, cs)["sel"].nsel.long().sum())
    pairs = None if share == 1.0 else int(share * full)
    r = _lowdens(w, cs, ratio, pairs)
    if ratio == 0.0:
        assert r["need"] == full, (r["need"], full)
    elif share == 1.0:
        assert 0 < r["need"] < full, (r["need"], full)  # some tiles each way
    _say(f"  pairs: qualifying {r['need']} of {full}, workspace for {pairs if pairs is not None else r['need']}")
    sel = r["sel"]
    g = dict(o=r["o"].float().cpu().numpy(), lse=r["lse"].cpu().numpy(), tau=sel.tau.cpu().numpy(),
             nsel=sel.nsel.cpu().numpy(), mask=unpack_mask(sel.mask, T // 64))
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=cs, storage="bf16")
    q, k, v = _np64(w["q"]), _np64(w["k"]), _np64(w["v"])
    kb_o = np.stack([np.stack([oracle.pool_blocks(k[b, h], 64, "bf16") for h in range(H)]) for b in range(B)])
    np.testing.assert_array_equal(r["kbar"].double().cpu().numpy(), kb_o)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(T)]
    ora = oracle.forward_rows(q, k, v, prm, rows, kbar=kb_o)
    st = check_rows(g, ora, rows, torch.bfloat16, 1.5, name)
    _say(f"  ok {st}")


def test_lowdens_deterministic_and_close_to_dense():
    w = inputs.make_prefill(1, 2, 4096, 128, "bf16", True, (1, 8), seed=17, device=DEV, with_dout=False)
    cs = 7.0 / math.sqrt(128)
    a = _lowdens(w, cs, 0.0)
    b = _lowdens(w, cs, 0.0)
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])
    d = _dense(w, cs)
    diff = (a["o"].float() - d["o"].float()).abs()
    mx, mn = tol_out(torch.bfloat16)
    assert float(diff.max()) <= mx and float(diff.mean()) <= mn, (float(diff.max()), float(diff.mean()))
    assert float((a["lse"] - d["lse"]).abs().max()) <= 4e-3
    _say(f"[lowdens] vs dense walk: O max {float(diff.max()):.3e} mean {float(diff.mean()):.3e}")


def test_lowdens_exact_workspace_takes_every_qualifying_tile():
    """A workspace sized for exactly the qualifying tiles' pairs holds all of them: the
    result equals (bit for bit) the one with a much larger workspace, so no tile fell back
    to the dense walk, whose rounding differs."""
    w = inputs.make_prefill(1, 2, 4096, 128, "bf16", True, (1, 8), seed=29, device=DEV, with_dout=False)
    cs = 7.0 / math.sqrt(128)
    a = _lowdens(w, cs, 0.0)
    b = _lowdens(w, cs, 0.0, extra_bytes=64 << 20)
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])


def test_lowdens_api_forward_switch():
    """api.forward(low_density=True) takes the schedule and sizes its workspace."""
    w = inputs.make_prefill(1, 2, 2048, 128, "bf16", True, (1, 8), seed=23, device=DEV, with_dout=False)
    cs = 7.0 / math.sqrt(128)
    r = _api().forward(w["q"], w["k"], w["v"], coarse_scale=cs, low_density=True, ratio=0.0)
    torch.cuda.synchronize()
    assert r["lowdens_pairs"] == 2 * 2048 + int(r["sel"].nsel.long().sum())
    a = _lowdens(w, cs, 0.0)
    assert torch.equal(r["o"], a["o"]) and torch.equal(r["lse"], a["lse"])


def test_lowdens_64k_calibrated_prefill_sampled():
    """The calibrated 64K prefill (coarse scale 7/sqrt(128)) through the schedule with
    its default ratio: sampled rows of two heads against the oracle, and every row of
    every head against the dense walk."""
    wl = inputs.CONFIGS["prefill64k_sc7"]
    sh = wl.shape
    _say(f"[lowdens] prefill64k_sc7 full size {sh}")
    w = inputs.make_prefill(sh["B"], sh["H"], sh["T"], sh["D"], wl.dtype, True, wl.planted, wl.seed, device=DEV,
                            with_dout=False)
    api = _api()
    r = _lowdens(w, wl.coarse_scale, api.LOWDENS_RATIO)
    total = sh["B"] * sh["H"] * sh["T"] + int(r["sel"].nsel.long().sum())
    _say(f"  qualifying pairs {r['need']} of {total}")
    assert r["need"] > 0.9 * total  # nearly every tile takes the schedule at this density
    d = _dense(w, wl.coarse_scale)
    assert torch.equal(d["sel"].mask, r["sel"].mask)
    diff = (r["o"].float() - d["o"].float()).abs()
    mx, mn = tol_out(torch.bfloat16)
    _say(f"  vs dense walk: O max {float(diff.max()):.3e} mean {float(diff.mean()):.3e}, "
         f"lse max {float((r['lse'] - d['lse']).abs().max()):.3e}")
    assert float(diff.max()) <= mx and float(diff.mean()) <= mn
    assert float((r["lse"] - d["lse"]).abs().max()) <= 4e-3
    del d
    rng = np.random.default_rng(5)
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=wl.coarse_scale, storage="bf16")
    T = sh["T"]
    for h in sorted(rng.choice(sh["H"], size=2, replace=False).tolist()):
        rows = sorted(set(rng.choice(T, size=256, replace=False).tolist() + [0, 63, 64, 127, 128, T - 1]))
        qh, kh, vh = (w[x][0, h] for x in ("q", "k", "v"))
        ora = oracle_parallel.forward_rows(qh, kh, vh, prm, rows, kbar=r["kbar"][0, h])
        st = check_out_rows(r["o"][0, h].float().cpu().numpy(), r["lse"][0, h].cpu().numpy(), ora, rows,
                            torch.bfloat16, f"lowdens 64K head {h}")
        _say(f"  head {h}: {st}")


def test_dash_fwd_with_workspace_takes_the_schedule():
    """dash_fwd given a low-density workspace runs Stages 0-2 with the schedule at
    DASH_LOWDENS_RATIO: the same bits as dash_fwd_select + dash_fwd_attend_lowdens; with no
    workspace it runs the dense walk (the same bits as api.forward)."""
    api, L = _api(), _lib()
    # a sparse selection (coarse scale 16/sqrt(128): a few blocks per row), so that most
    # tiles' dense walk exceeds the default ratio times their pairs
    w = inputs.make_prefill(1, 2, 8192, 128, "bf16", True, (1, 8), seed=31, device=DEV, with_dout=False)
    cs = 16.0 / math.sqrt(128)
    ref = _lowdens(w, cs, api.LOWDENS_RATIO)
    q, k, v = w["q"], w["k"], w["v"]
    B, H, T, D = q.shape
    p = api.make_params(q, 1.5, True, None, cs)
    sel = api.alloc_selection(p, q.device, want_mask=True)
    kbar = torch.empty((B, H, T // 64, D), dtype=q.dtype, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    wsb = L.fwd_lowdens_workspace_bytes(p, ref["need"])
    ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    st = torch.cuda.current_stream().cuda_stream
    L.fwd(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), kbar.data_ptr(), sel.as_c(),
          ws.data_ptr(), wsb, st)
    torch.cuda.synchronize()
    assert ref["need"] > 0
    assert torch.equal(o, ref["o"]) and torch.equal(lse, ref["lse"])
    d = _dense(w, cs)
    L.fwd(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), kbar.data_ptr(), sel.as_c(),
          0, 0, st)
    torch.cuda.synchronize()
    assert torch.equal(o, d["o"]) and torch.equal(lse, d["lse"])


def test_lowdens_96k_every_tile():
    """The longest prefill (98304 tokens, 1536 blocks: 48 mask words per row, the fill's row
    buffers flushed more than once, twelve 8192-row ranges) with every tile through the
    schedule (ratio 0), two heads at coarse scale 7/sqrt(128): every row against the dense
    walk, sampled rows against the oracle."""
    B, H, T, D = 1, 2, 98304, 128
    cs = 7.0 / math.sqrt(D)
    _say(f"[lowdens] B{B} H{H} T{T} D{D}, every tile, coarse 7/sqrt(D)")
    w = inputs.make_prefill(B, H, T, D, "bf16", True, (1, 8), seed=97, device=DEV, with_dout=False)
    r = _lowdens(w, cs, 0.0)
    total = B * H * T + int(r["sel"].nsel.long().sum())
    assert r["need"] == total, (r["need"], total)
    d = _dense(w, cs)
    assert torch.equal(d["sel"].mask, r["sel"].mask)
    diff = (r["o"].float() - d["o"].float()).abs()
    mx, mn = tol_out(torch.bfloat16)
    _say(f"  pairs {total}; vs dense walk: O max {float(diff.max()):.3e} mean {float(diff.mean()):.3e}")
    assert float(diff.max()) <= mx and float(diff.mean()) <= mn
    assert float((r["lse"] - d["lse"]).abs().max()) <= 4e-3
    del d
    rng = np.random.default_rng(11)
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=cs, storage="bf16")
    h = 1
    rows = sorted(set(rng.choice(T, size=128, replace=False).tolist() + [0, 63, 8191, 8192, T - 1]))
    qh, kh, vh = (w[x][0, h] for x in ("q", "k", "v"))
    ora = oracle_parallel.forward_rows(qh, kh, vh, prm, rows, kbar=r["kbar"][0, h])
    st = check_out_rows(r["o"][0, h].float().cpu().numpy(), r["lse"][0, h].cpu().numpy(), ora, rows,
                        torch.bfloat16, "lowdens 96K head 1")
    _say(f"  head {h}: {st}")
