"""GPU parity of grouped-query heads with entmax head aggregation.

dash_fwd_gqa and dash_bwd_gqa (through the C ABI) against the float64
oracle's forward_rows_gqa and backward_gqa: each head's own selection
(tau, counts, masks) and the outputs to the usual tolerances, the gradients
to 5e-2 relative L2, the summaries of the KV heads bit for bit; one KV head
per query head is dash_fwd / dash_bwd bit for bit.
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


def _gpu(r, nb):
    sel = r["sel"]
    return dict(o=r["o"].float().cpu().numpy(), lse=r["lse"].cpu().numpy(), tau=sel.tau.cpu().numpy(),
                nsel=sel.nsel.cpu().numpy(), mask=unpack_mask(sel.mask, nb))


CASES = [
    # name, B, H, Hkv, T, D, causal, alpha, coarse multiple, planted
    ("h4-kv2-causal-ragged", 1, 4, 2, 1088, 128, True, 1.5, 4.0, (1, 4)),
    ("h4-kv1-noncausal-d64", 1, 4, 1, 576, 64, False, 1.25, 4.0, (1, 3)),
    ("b2-h8-kv2-causal", 2, 8, 2, 512, 128, True, 1.5, 6.0, (1, 3)),
    ("h2-kv1-causal-a1", 1, 2, 1, 640, 128, True, 1.0, 2.0, (1, 3)),
    ("h4-kv2-causal-a2", 1, 4, 2, 576, 128, True, 2.0, 6.0, (1, 3)),
    ("h4-kv1-causal-T2048", 1, 4, 1, 2048, 128, True, 1.5, 6.0, (1, 4)),
    # eight query heads per KV head: a wave's 32 columns are 8 heads x 4 rows
    ("h8-kv1-causal-ragged", 1, 8, 1, 1088, 128, True, 1.5, 4.0, (1, 4)),
    ("h8-kv1-noncausal-d64", 1, 8, 1, 512, 64, False, 1.25, 4.0, (1, 3)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gqa_forward_and_backward_small(case):
    from differentiable_adaptive_block_amd import api
    name, B, H, Hkv, T, D, causal, alpha, csm, planted = case
    _say(f"[gqa] {name} B{B} H{H} Hkv{Hkv} T{T} D{D} causal={causal} alpha={alpha}")
    w = inputs.make_prefill(B, H, T, D, "bf16", causal, planted, seed=81 + T, device="cpu", with_dout=True,
                            kv_heads=Hkv)
    w = {k: v.to(DEV) for k, v in w.items()}
    cs = csm / math.sqrt(D)
    r = api.forward(w["q"], w["k"], w["v"], alpha=alpha, causal=causal, coarse_scale=cs)
    g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"])
    torch.cuda.synchronize()
    prm = oracle.Params(alpha=alpha, causal=causal, coarse_scale=cs, storage="bf16")
    q64, k64, v64, d64 = (_np64(w[x]) for x in ("q", "k", "v", "dout"))
    for b in range(B):
        for kv in range(Hkv):
            np.testing.assert_array_equal(_np64(r["kbar"][b, kv]), oracle.pool_blocks(k64[b, kv], 64, "bf16"))
    nb = T // 64
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(T)]
    ora = oracle.forward_rows_gqa(q64, k64, v64, prm, rows)
    st = check_rows(_gpu(r, nb), ora, rows, torch.bfloat16, alpha, name)
    ref = oracle.backward_gqa(q64, k64, v64, d64, prm)
    errs = {n: rel_l2(_np64(g[n]), ref[n]) for n in ("dq", "dk", "dv", "dkbar")}
    _say(f"  forward {st}; rel-L2 {errs}")
    for n, e in errs.items():
        assert e <= 5e-2, (name, n, e)
    # the group's heads share one block list per tile: the union of their masks
    ntile = (T + 127) // 128
    cnt = r["sel"].tile_cnt.view(B, H, ntile).cpu()
    G = H // Hkv
    for kv in range(Hkv):
        for h in range(kv * G + 1, (kv + 1) * G):
            assert torch.equal(cnt[:, h], cnt[:, kv * G])


def test_one_kv_head_per_query_head_is_the_per_head_path():
    from differentiable_adaptive_block_amd import _lib, api
    B, H, T, D = 1, 2, 1024, 128
    w = inputs.make_prefill(B, H, T, D, "bf16", True, (1, 4), seed=85, device="cpu", with_dout=True)
    w = {k: v.to(DEV) for k, v in w.items()}
    cs = 4.0 / math.sqrt(D)
    r = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=cs)
    p = r["params"]
    o = torch.empty_like(w["q"])
    lse = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    kbar = torch.empty((B, H, T // 64, D), dtype=torch.bfloat16, device=DEV)
    sel = api.alloc_selection(p, DEV, True)
    st = torch.cuda.current_stream().cuda_stream
    _lib.fwd_gqa(p, H, w["q"].data_ptr(), w["k"].data_ptr(), w["v"].data_ptr(), o.data_ptr(), lse.data_ptr(),
                 kbar.data_ptr(), sel.as_c(), st)
    g0 = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], p)
    dq, dk, dv = (torch.empty_like(w[x]) for x in ("q", "k", "v"))
    dkbar = torch.empty((B, H, T // 64, D), dtype=torch.float32, device=DEV)
    wsb = _lib.bwd_gqa_workspace_bytes(p, H)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    _lib.bwd_gqa(p, H, w["q"].data_ptr(), w["k"].data_ptr(), w["v"].data_ptr(), r["o"].data_ptr(),
                 r["lse"].data_ptr(), w["dout"].data_ptr(), r["kbar"].data_ptr(), r["sel"].as_c(), dq.data_ptr(),
                 dk.data_ptr(), dv.data_ptr(), dkbar.data_ptr(), ws.data_ptr(), wsb, st)
    torch.cuda.synchronize()
    assert torch.equal(o, r["o"]) and torch.equal(lse, r["lse"]) and torch.equal(kbar, r["kbar"])
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dkbar", dkbar)):
        assert torch.equal(t, g0[n]), n


def test_gqa_deterministic():
    from differentiable_adaptive_block_amd import api
    w = inputs.make_prefill(1, 4, 1024, 128, "bf16", True, (1, 4), seed=86, device="cpu", with_dout=True, kv_heads=1)
    w = {k: v.to(DEV) for k, v in w.items()}
    outs = []
    for _ in range(2):
        r = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=4 / math.sqrt(128))
        g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"])
        outs.append((r["o"], g["dq"], g["dk"], g["dv"], g["dkbar"]))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_gqa_16k_sampled():
    from differentiable_adaptive_block_amd import api
    B, H, Hkv, T, D = 1, 32, 8, 16384, 128
    _say(f"[gqa] 16K prefill B{B} H{H} Hkv{Hkv} T{T} D{D}")
    w = inputs.make_prefill(B, H, T, D, "bf16", True, (1, 8), seed=87, device=DEV, with_dout=False, kv_heads=Hkv)
    cs = 1.0 / math.sqrt(D)
    r = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=cs)
    torch.cuda.synchronize()
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=cs, storage="bf16")
    rng = np.random.default_rng(88)
    rows = [(0, int(h), int(i)) for h, i in zip(rng.integers(0, H, 8), rng.integers(64, T, 8))]
    rows += [(0, 5, T - 1), (0, 30, 70)]
    # the oracle reads only the rows' own KV heads and positions up to the row
    q64 = np.zeros((B, H, T, D))
    for (_, h, i) in rows:
        q64[0, (h // 4) * 4:(h // 4) * 4 + 4, i] = _np64(w["q"][0, (h // 4) * 4:(h // 4) * 4 + 4, i])
    k64, v64 = _np64(w["k"]), _np64(w["v"])
    ora = oracle.forward_rows_gqa(q64, k64, v64, prm, rows)
    gpu = _gpu(r, T // 64)
    st = check_rows({k: v for k, v in gpu.items()}, ora, rows, torch.bfloat16, 1.5, "gqa 16K")
    _say(f"  ok {st}")


def _head_sel(q, kc, lens, prm, s, h, G):
    """The oracle's Stage-1 row of query head h of sequence s over its KV head's cache."""
    C = kc.shape[2]
    n = C if lens is None else int(lens[s])
    own = (n - 1) // 64
    kb = oracle.pool_blocks(_np64(kc[s, h // G, :64 * own]), 64, "bf16")
    return oracle.select_row(_np64(q[s, h]), kb, n - 1, prm, q.shape[-1])


def _decode_check(out, ora, rows, prm, what, sel_of):
    """GPU grouped decode vs the oracle on rows ((s, h) in out, (s, h) in ora):
    outputs, each head's own tau and selected set (bit for bit outside the tie
    band), and the group's union = the OR of its heads' sets."""
    from parity import check_mask_row, tau_tol, tol_lse, tol_out
    max_abs, mean_abs = tol_out(torch.bfloat16)
    errs = []
    for (s, h), (os_, oh) in rows:
        errs.append(np.abs(_np64(out["o"][s, h]) - ora["o"][os_, oh]))
        assert abs(float(out["lse"][s, h]) - ora["lse"][os_, oh]) <= tol_lse(torch.bfloat16), (what, s, h)
        sel = sel_of(s, h)
        flips = check_mask_row(out["mask"][s, h], sel, prm.alpha, f"{what} {(s, h)}")
        ns, nso = int(out["nsel"][s, h]), int(ora["nsel"][os_, oh])
        assert ns == nso if flips == 0 else abs(ns - nso) <= flips, (what, s, h)
        t, to = float(out["tau"][s, h]), float(ora["tau"][os_, oh])
        assert (math.isnan(t) and math.isnan(to)) or abs(t - to) <= tau_tol(to), (what, s, h, t, to)
        if flips == 0:
            # the union the group walks: every head's selected set lies in it
            bits = ((out["mask"][s, h].cpu().numpy().astype(np.int64)[:, None] >> np.arange(32)) & 1).reshape(-1)
            nbc = ora["union"].shape[-1]
            assert not (bits[:nbc].astype(bool) & ~ora["union"][os_, oh]).any(), (what, s, h)
    E = np.stack(errs)
    assert E.max() <= max_abs and E.mean() <= mean_abs, (what, E.max(), E.mean())
    return float(E.max()), float(E.mean())


@pytest.mark.parametrize("heads", [(4, 2), (8, 2), (8, 1)], ids=["G2", "G4", "G8"])
@pytest.mark.parametrize("lens", [None, [1, 65, 700]], ids=["full", "lengths"])
def test_gqa_decode_small(lens, heads):
    """2, 4 and 8 query heads per KV head: the register-streamed walk (2, 4)
    and the LDS-staged one (8), with each group size's selection kernel."""
    from differentiable_adaptive_block_amd import api
    H, Hkv = heads
    S, C, D = 3, 1024, 128
    _say(f"[gqa decode] S{S} H{H} Hkv{Hkv} C{C} lens {lens}")
    w = inputs.make_decode(S, H, C, D, "bf16", (1, 4), seed=98, device="cpu", lens=lens, kv_heads=Hkv)
    q, kc, vc = (w[x].to(DEV) for x in ("q", "k", "v"))
    kbar = api.pool(kc.view(1, S * Hkv, C, D)).view(S, Hkv, C // 64, D)
    cs = 4.0 / math.sqrt(D)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = api.decode_gqa(q, kc, vc, kbar, lt, coarse_scale=cs)
    torch.cuda.synchronize()
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=cs, storage="bf16")
    ora = oracle.decode_gqa(_np64(q), _np64(kc), _np64(vc), lens, prm)
    st = _decode_check(out, ora, [((s, h), (s, h)) for s in range(S) for h in range(H)], prm, "gqa decode",
                       lambda s, h: _head_sel(q, kc, lens, prm, s, h, H // Hkv))
    # the OR of the group's heads' masks is the oracle's union (no tie-band candidates here)
    G = H // Hkv
    m = out["mask"].cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    bits = ((m[..., None] >> np.arange(32)) & 1).reshape(S, H, -1)[..., :C // 64].astype(bool)
    for s in range(S):
        for kv in range(Hkv):
            gu = bits[s, kv * G:(kv + 1) * G].any(axis=0)
            np.testing.assert_array_equal(gu, ora["union"][s, kv * G], err_msg=f"union {(s, kv)}")
    _say(f"  ok {st}")


def test_gqa_decode_one_kv_head_per_query_head_is_dash_decode():
    from differentiable_adaptive_block_amd import api
    S, H, C, D = 2, 4, 2048, 128
    w = inputs.make_decode(S, H, C, D, "bf16", (1, 4), seed=99, device="cpu")
    q, kc, vc = (w[x].to(DEV) for x in ("q", "k", "v"))
    kbar = api.pool(kc.view(1, S * H, C, D)).view(S, H, C // 64, D)
    a = {k: v.clone() for k, v in api.decode(q, kc, vc, kbar, coarse_scale=3 / math.sqrt(D)).items()}
    b = api.decode_gqa(q, kc, vc, kbar, None, coarse_scale=3 / math.sqrt(D))
    torch.cuda.synchronize()
    assert torch.equal(a["nsel"], b["nsel"]) and torch.equal(a["tau"], b["tau"]) and torch.equal(a["mask"], b["mask"])
    assert (a["o"].float() - b["o"].float()).abs().max().item() <= 1e-2
    assert (a["lse"] - b["lse"]).abs().max().item() <= 1e-4


def test_gqa_decode_96k_sampled():
    from differentiable_adaptive_block_amd import api
    wl = inputs.CONFIGS["decode96k_sc5"]
    S, H, Hkv, C, D = 4, 32, 8, wl.shape["N"], wl.shape["D"]
    _say(f"[gqa decode] 96K cache S{S} H{H} Hkv{Hkv}")
    w = inputs.make_decode(S, H, C, D, "bf16", wl.planted, wl.seed, device=DEV, kv_heads=Hkv)
    q, kc, vc = w["q"], w["k"], w["v"]
    kbar = api.pool(kc.view(1, S * Hkv, C, D)).view(S, Hkv, C // 64, D)
    out = api.decode_gqa(q, kc, vc, kbar, None, coarse_scale=wl.coarse_scale)
    torch.cuda.synchronize()
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=wl.coarse_scale, storage="bf16")
    G = H // Hkv
    for (s, kv) in [(0, 0), (3, 5)]:
        ora = oracle.decode_gqa(_np64(q[s:s + 1, kv * G:(kv + 1) * G]), _np64(kc[s:s + 1, kv:kv + 1]),
                                _np64(vc[s:s + 1, kv:kv + 1]), None, prm)
        st = _decode_check(out, ora, [((s, kv * G + g), (0, g)) for g in range(G)], prm, f"gqa decode {s} {kv}",
                           lambda s_, h_: _head_sel(q, kc, None, prm, s_, h_, G))
        _say(f"  ok group ({s}, {kv}): {st}")


def test_gqa_autograd():
    from differentiable_adaptive_block_amd import api
    w = inputs.make_prefill(1, 4, 512, 128, "bf16", True, (1, 3), seed=89, device="cpu", with_dout=True, kv_heads=2)
    w = {k: v.to(DEV) for k, v in w.items()}
    q, k, v = (w[x].clone().requires_grad_(True) for x in ("q", "k", "v"))
    cs = 4 / math.sqrt(128)
    o = api.dash_attention(q, k, v, 1.5, True, None, cs)
    (o.float() * w["dout"].float()).sum().backward()
    r = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=cs)
    g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"])
    torch.cuda.synchronize()
    assert k.grad.shape == k.shape and v.grad.shape == v.shape
    for t, n in ((q, "dq"), (k, "dk"), (v, "dv")):
        assert torch.equal(t.grad, g[n]), n
