"""GPU forward parity: libdash.so (through the C ABI) against the float64 oracle.

Small cases run the oracle over every row; the full-size workloads (the
16K and 64K causal prefills) compare sampled rows.  Tolerances are in
tests/parity.py.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from differentiable_adaptive_block_amd import inputs
import oracle_parallel
from parity import check_out_rows, check_rows, check_stage1_head, unpack_mask

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _api():
    from differentiable_adaptive_block_amd import api
    return api


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu_forward(w, alpha, causal, coarse_scale):
    api = _api()
    r = api.forward(w["q"], w["k"], w["v"], alpha=alpha, causal=causal, coarse_scale=coarse_scale, want_mask=True)
    torch.cuda.synchronize()
    nb = w["q"].shape[2] // 64
    sel = r["sel"]
    return r, dict(o=r["o"].float().cpu().numpy(), lse=r["lse"].cpu().numpy(), tau=sel.tau.cpu().numpy(),
                   nsel=sel.nsel.cpu().numpy(), mask=unpack_mask(sel.mask, nb))


def _np64(t):
    return t.double().cpu().numpy()


SMALL = [
    # name, B, H, T, D, dtype, causal, alpha, coarse multiple of 1/sqrt(D), planted
    ("tiny512", 1, 2, 512, 64, "fp32", False, 1.5, 1.0, None),
    ("tiny512_sc16", 1, 2, 512, 64, "fp32", False, 1.5, 16.0, None),
    ("tiny512-a1", 1, 2, 512, 64, "fp32", False, 1.0, 1.0, None),
    ("tiny512-a125", 1, 2, 512, 64, "fp32", False, 1.25, 16.0, None),
    ("tiny512-a2", 1, 2, 512, 64, "fp32", False, 2.0, 16.0, None),
    ("fp32-causal", 1, 2, 320, 128, "fp32", True, 1.5, 4.0, (1, 3)),
    ("bf16-causal-ragged", 1, 2, 1088, 128, "bf16", True, 1.5, 4.0, (1, 4)),
    ("bf16-causal-dense", 2, 1, 576, 128, "bf16", True, 1.5, 1.0, (1, 8)),
    ("bf16-noncausal-d64", 1, 2, 576, 64, "bf16", False, 1.25, 4.0, (1, 3)),
    ("bf16-noncausal-tile-tail", 2, 2, 1088, 128, "bf16", False, 1.5, 4.0, (1, 4)),
    ("bf16-causal-a1", 1, 1, 512, 128, "bf16", True, 1.0, 1.0, (1, 3)),
    ("bf16-causal-a2", 1, 1, 512, 64, "bf16", True, 2.0, 4.0, (1, 3)),
    ("bf16-one-block", 1, 2, 64, 128, "bf16", True, 1.5, 1.0, None),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_forward_small_full_oracle(case):
    name, B, H, T, D, dtype, causal, alpha, csm, planted = case
    _say(f"[forward] {name} B{B} H{H} T{T} D{D} {dtype} causal={causal} alpha={alpha}")
    w = inputs.make_prefill(B, H, T, D, dtype, causal, planted, seed=7 + T + D, device="cpu", with_dout=False)
    w = {k: v.to(DEV) for k, v in w.items()}
    cs = csm / math.sqrt(D)
    r, g = _gpu_forward(w, alpha, causal, cs)
    prm = oracle.Params(alpha=alpha, causal=causal, coarse_scale=cs, storage=dtype)
    q, k, v = _np64(w["q"]), _np64(w["k"]), _np64(w["v"])
    # summaries bit-exact
    kb_o = np.stack([np.stack([oracle.pool_blocks(k[b, h], 64, dtype) for h in range(H)]) for b in range(B)])
    np.testing.assert_array_equal(r["kbar"].double().cpu().numpy(), kb_o)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(T)]
    ora = oracle.forward_rows(q, k, v, prm, rows, kbar=kb_o)
    st = check_rows(g, ora, rows, w["q"].dtype, alpha, name)
    _say(f"  ok {st}")


def test_forward_deterministic():
    w = inputs.make_prefill(1, 2, 1024, 128, "bf16", True, (1, 4), seed=3, device="cpu", with_dout=False)
    w = {k: v.to(DEV) for k, v in w.items()}
    api = _api()
    a = api.forward(w["q"], w["k"], w["v"], coarse_scale=3 / math.sqrt(128))
    b = api.forward(w["q"], w["k"], w["v"], coarse_scale=3 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])
    assert torch.equal(a["sel"].mask, b["sel"].mask)


def _prefill_head_checks(w, r, h, prm, dtype, n_rows, rng, what, all_rows_out=False):
    """One head (batch 0) of a GPU forward against the oracle: the summaries
    bit for bit, Stage 1 (mask, count, tau) on every row, O and LSE on
    ``n_rows`` uniformly drawn rows plus the first, block-edge and last rows
    (every row with ``all_rows_out``).  The oracle runs over worker processes."""
    T = w["q"].shape[2]
    qh, kh, vh = (w[x][0, h] for x in ("q", "k", "v"))
    kb = oracle.pool_blocks(_np64(kh), 64, dtype)
    np.testing.assert_array_equal(r["kbar"][0, h].double().cpu().numpy(), kb)
    sel = r["sel"]
    sels = oracle_parallel.select_rows(qh, r["kbar"][0, h], prm, list(range(T)))
    flips, tau_w = check_stage1_head(sel.mask[0, h].cpu().numpy(), sel.tau[0, h].cpu().numpy(),
                                     sel.nsel[0, h].cpu().numpy(), sels, prm.alpha, f"{what} head {h}")
    if all_rows_out:
        rows = list(range(T))
    else:
        rows = sorted(set(rng.choice(T, size=n_rows, replace=False).tolist() + [0, 63, 64, T - 1]))
    ora = oracle_parallel.forward_rows(qh, kh, vh, prm, rows, kbar=r["kbar"][0, h])
    st = check_out_rows(r["o"][0, h].float().cpu().numpy(), r["lse"][0, h].cpu().numpy(), ora, rows,
                        w["q"].dtype, f"{what} head {h}")
    st.update(flips=flips, tau_over_bound=tau_w)
    return st


def _sampled(name, n_heads=3, n_rows=512, full_head=False):
    """A named full-size prefill workload: heads drawn at random get the
    per-head checks; with ``full_head`` the first of them compares O and LSE
    on every row."""
    wl = inputs.CONFIGS[name]
    sh = wl.shape
    _say(f"[forward] {name} full size {sh}")
    w = inputs.make_prefill(sh["B"], sh["H"], sh["T"], sh["D"], wl.dtype, wl.causal, wl.planted, wl.seed,
                            device=DEV, with_dout=False)
    alpha = wl.alpha if not isinstance(wl.alpha, tuple) else wl.alpha[-1]
    r = _api().forward(w["q"], w["k"], w["v"], alpha=alpha, causal=wl.causal, coarse_scale=wl.coarse_scale,
                       want_mask=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    B, H, T = sh["B"], sh["H"], sh["T"]
    heads = sorted(rng.choice(H, size=n_heads, replace=False).tolist())
    prm = oracle.Params(alpha=alpha, causal=wl.causal, coarse_scale=wl.coarse_scale, storage=wl.dtype)
    for n, h in enumerate(heads):
        st = _prefill_head_checks(w, r, h, prm, wl.dtype, n_rows, rng, name, all_rows_out=full_head and n == 0)
        _say(f"  head {h}: {st}")
    density = float(r["sel"].nsel.double().sum()) / float(sum((i // 64) for i in range(T)) * B * H)
    _say(f"  ok; selected-pair density {density:.4f}")
    return density


def test_forward_16k_causal_prefill_sampled():
    _sampled("prefill16k", full_head=True)


def test_forward_64k_causal_prefill_sampled():
    _sampled("prefill64k", n_heads=2, n_rows=384)


def test_forward_64k_calibrated_prefill_sampled():
    """The 64K prefill at coarse scale 7/sqrt(128) (about 8% of the candidate pairs selected)."""
    d = _sampled("prefill64k_sc7", n_heads=2, n_rows=384)
    assert d < 0.12, d


def test_forward_96k_causal_prefill_sampled():
    """The longest prefill (98304 tokens, 1536 blocks: the Stage-1 shape with 96
    candidates per lane and six 256-block chunks)."""
    _sampled("prefill96k", n_heads=1, n_rows=256)


@pytest.mark.parametrize("T", [8192, 32768])
def test_forward_stage1_kernel_sizes(T):
    """Sequence lengths that take the other Stage-1 kernel shapes: 128 blocks
    (8 candidates per lane of a 16-lane row group) and 512 blocks (two
    256-block chunks of the staged score tile)."""
    B, H, D = 1, 2, 128
    _say(f"[forward] B{B} H{H} T{T} D{D} bf16 causal, coarse 4/sqrt(D)")
    w = inputs.make_prefill(B, H, T, D, "bf16", True, (1, 8), seed=50 + T // 1024, device=DEV, with_dout=False)
    cs = 4.0 / math.sqrt(D)
    r = _api().forward(w["q"], w["k"], w["v"], alpha=1.5, causal=True, coarse_scale=cs, want_mask=True)
    torch.cuda.synchronize()
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=cs, storage="bf16")
    rng = np.random.default_rng(T)
    for h in range(H):
        st = _prefill_head_checks(w, r, h, prm, "bf16", 384, rng, f"T{T}")
        _say(f"  head {h}: {st}")
