"""GPU parity of the learned Stage-0 summariser (zero-initialised attention pooling).

dash_pool_attn, dash_select, dash_bwd_learned (dash_bwd_no_pool and
dash_pool_attn_bwd composed, dK rounded once)
(through the C ABI) against the float64 oracle: the summaries bit for bit
(mean pooling at w = 0), the forward to the usual output tolerances, the
gradients (dw included) to 5e-2 relative L2.
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


def _head(H, D, scale, seed):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn((H, D), generator=g) / math.sqrt(D)).float()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64)])
def test_zero_head_equals_mean_pooling(dtype, D):
    from differentiable_adaptive_block_amd import api
    w = inputs.make_prefill(2, 3, 1024, D, dtype, False, None, seed=51, device="cpu", with_dout=False)
    k = w["k"].to(DEV)
    a = api.pool_attn(k, torch.zeros((3, D), dtype=torch.float32, device=DEV))
    b = api.pool(k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,D,scale", [("bf16", 128, 1.0), ("bf16", 128, 4.0), ("fp32", 64, 2.0)])
def test_pool_attn_matches_oracle(dtype, D, scale):
    from differentiable_adaptive_block_amd import api
    B, H, T = 1, 4, 1024
    w = inputs.make_prefill(B, H, T, D, dtype, False, None, seed=52, device="cpu", with_dout=False)
    head = _head(H, D, scale, 53)
    kbar = api.pool_attn(w["k"].to(DEV), head.to(DEV))
    torch.cuda.synchronize()
    k64 = _np64(w["k"])
    for h in range(H):
        ref = oracle.pool_attention(k64[0, h], head[h].double().numpy(), 64, dtype)
        np.testing.assert_array_equal(_np64(kbar[0, h]), ref, err_msg=f"head {h}")
    # away from zero the summaries are not the means
    assert not torch.equal(kbar, api.pool(w["k"].to(DEV)))


CASES = [
    # name, B, H, T, D, dtype, causal, alpha, coarse multiple, planted, head scale
    ("bf16-causal", 1, 2, 1088, 128, "bf16", True, 1.5, 4.0, (1, 4), 2.0),
    ("bf16-noncausal-a125", 1, 2, 512, 128, "bf16", False, 1.25, 4.0, (1, 3), 2.0),
    ("fp32-noncausal", 1, 2, 512, 64, "fp32", False, 1.5, 16.0, None, 2.0),
    ("bf16-causal-zero-head", 1, 2, 576, 128, "bf16", True, 1.5, 4.0, (1, 3), 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_and_backward_with_learned_summariser(case):
    from differentiable_adaptive_block_amd import api
    name, B, H, T, D, dtype, causal, alpha, csm, planted, scale = case
    _say(f"[summariser] {name} B{B} H{H} T{T} D{D} {dtype} causal={causal} alpha={alpha} head scale {scale}")
    w = inputs.make_prefill(B, H, T, D, dtype, causal, planted, seed=54 + T, device="cpu", with_dout=True)
    w = {k: v.to(DEV) for k, v in w.items()}
    head = _head(H, D, scale, 55).to(DEV)
    cs = csm / math.sqrt(D)
    r = api.forward(w["q"], w["k"], w["v"], alpha=alpha, causal=causal, coarse_scale=cs, summariser_w=head)
    g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"],
                     summariser_w=head)
    torch.cuda.synchronize()
    prm = oracle.Params(alpha=alpha, causal=causal, coarse_scale=cs, storage=dtype)
    q64, k64, v64, d64 = (_np64(w[x]) for x in ("q", "k", "v", "dout"))
    h64 = _np64(head)
    for h in range(H):
        np.testing.assert_array_equal(_np64(r["kbar"][0, h]), oracle.pool_attention(k64[0, h], h64[h], 64, dtype))
    nb = T // 64
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(T)]
    ora = oracle.forward_rows(q64, k64, v64, prm, rows, w=h64)
    sel = r["sel"]
    gpu = dict(o=r["o"].float().cpu().numpy(), lse=r["lse"].cpu().numpy(), tau=sel.tau.cpu().numpy(),
               nsel=sel.nsel.cpu().numpy(), mask=unpack_mask(sel.mask, nb))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    st = check_rows(gpu, ora, rows, tdt, alpha, name)
    ref = oracle.backward(q64, k64, v64, d64, prm, w=h64)
    errs = {n: rel_l2(_np64(g[n]), ref[n]) for n in ("dq", "dk", "dv", "dkbar", "dw")}
    _say(f"  forward {st}; rel-L2 {errs}")
    for n, e in errs.items():
        assert e <= 5e-2, (name, n, e)


def test_autograd_head_gradient():
    from differentiable_adaptive_block_amd import api
    B, H, T, D = 1, 2, 512, 128
    w = inputs.make_prefill(B, H, T, D, "bf16", True, (1, 3), seed=56, device="cpu", with_dout=True)
    w = {k: v.to(DEV) for k, v in w.items()}
    head = _head(H, D, 2.0, 57).to(DEV).requires_grad_(True)
    cs = 4.0 / math.sqrt(D)
    o = api.dash_attention(w["q"], w["k"], w["v"], 1.5, True, None, cs, summariser_w=head)
    (o.float() * w["dout"].float()).sum().backward()
    r = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=cs, summariser_w=head.detach())
    g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"],
                     summariser_w=head.detach())
    torch.cuda.synchronize()
    assert head.grad is not None and torch.equal(head.grad, g["dw"])


def test_zero_head_gradients_match_mean_pooling_path():
    from differentiable_adaptive_block_amd import api
    B, H, T, D = 1, 2, 1024, 128
    w = inputs.make_prefill(B, H, T, D, "bf16", True, (1, 4), seed=58, device="cpu", with_dout=True)
    w = {k: v.to(DEV) for k, v in w.items()}
    cs = 4.0 / math.sqrt(D)
    zero = torch.zeros((H, D), dtype=torch.float32, device=DEV)
    r = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=cs)
    g0 = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"])
    r1 = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=cs, summariser_w=zero)
    g1 = api.backward(w["q"], w["k"], w["v"], r1["o"], r1["lse"], w["dout"], r1["kbar"], r1["sel"], r1["params"],
                      summariser_w=zero)
    torch.cuda.synchronize()
    assert torch.equal(r["o"], r1["o"]) and torch.equal(r["kbar"], r1["kbar"])
    # every gradient, dk included: the summariser's share of dk is added to the
    # unrounded other terms and rounded once, as the mean-pooling path does
    for n in ("dq", "dk", "dv", "dkbar"):
        assert torch.equal(g0[n], g1[n]), n
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=cs, storage="bf16")
    ref = oracle.backward(*(_np64(w[x]) for x in ("q", "k", "v", "dout")), prm, w=np.zeros((H, D)))
    assert rel_l2(_np64(g1["dw"]), ref["dw"]) <= 5e-2


def test_summariser_training_16k_sampled():
    """The 16K training shape (B2 H16 T16384) with a non-zero summariser head: dQ on sampled
    rows, dK, dV and the summary gradient of the last key blocks (attended only by the last
    rows), against the oracle over those rows; dw needs every row and is checked at small sizes."""
    from differentiable_adaptive_block_amd import api
    wl = inputs.CONFIGS["train16k"]
    sh = wl.shape
    _say(f"[summariser] train16k full size {sh} (sampled)")
    w = inputs.make_prefill(sh["B"], sh["H"], sh["T"], sh["D"], wl.dtype, True, wl.planted, wl.seed, device=DEV,
                            with_dout=True)
    head = _head(sh["H"], sh["D"], 2.0, 59).to(DEV)
    r = api.forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=wl.coarse_scale,
                    summariser_w=head, want_mask=False)
    g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"],
                     summariser_w=head)
    torch.cuda.synchronize()
    T = sh["T"]
    nb = T // 64
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=wl.coarse_scale, storage="bf16")
    rng = np.random.default_rng(3)
    for (b, h) in [(0, int(rng.integers(sh["H"]))), (1, int(rng.integers(sh["H"])))]:
        x = {n: _np64(w[n][b:b + 1, h:h + 1]) for n in ("q", "k", "v", "dout")}
        hw = _np64(head[h:h + 1])
        np.testing.assert_array_equal(_np64(r["kbar"][b, h]), oracle.pool_attention(x["k"][0, 0], hw[0], 64, "bf16"))
        tail = 4 * 64
        rows = [(0, 0, i) for i in range(T - tail, T)]
        rows += [(0, 0, int(i)) for i in rng.choice(T - tail, size=24, replace=False)]
        ref = oracle.backward_rows(x["q"], x["k"], x["v"], x["dout"], prm, rows, w=hw)
        ridx = np.array([i for (_, _, i) in rows])
        e_dq = rel_l2(_np64(g["dq"][b, h])[ridx], ref["dq"][0, 0][ridx])
        e_dk = rel_l2(_np64(g["dk"][b, h])[T - tail:], ref["dk"][0, 0][T - tail:])
        e_dv = rel_l2(_np64(g["dv"][b, h])[T - tail:], ref["dv"][0, 0][T - tail:])
        e_kb = rel_l2(_np64(g["dkbar"][b, h])[nb - 4:nb - 1], ref["dkbar"][0, 0][nb - 4:nb - 1])
        _say(f"  (b={b}, h={h}) rel-L2 dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e} dkbar {e_kb:.2e}")
        assert max(e_dq, e_dk, e_dv, e_kb) <= 5e-2
