"""GPU backward parity: dash_bwd (through the C ABI) against the float64 oracle.

Gradients must match within 5e-2 relative L2 (tests/parity.py).  Small
cases compare every gradient; the full-size training workload
(B2 H16 T16384 D128, alpha in {1.25, 1.5}) compares dQ on sampled rows and
dK, dV and the summary gradient on the last key blocks of sampled heads,
which only the rows from those blocks on attend.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from differentiable_adaptive_block_amd import inputs
import oracle_parallel
from parity import rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 5e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.double().cpu().numpy()


def _run(w, alpha, causal, cs):
    from differentiable_adaptive_block_amd import api
    r = api.forward(w["q"], w["k"], w["v"], alpha=alpha, causal=causal, coarse_scale=cs, want_mask=False)
    g = api.backward(w["q"], w["k"], w["v"], r["o"], r["lse"], w["dout"], r["kbar"], r["sel"], r["params"])
    torch.cuda.synchronize()
    return r, g


SMALL = [
    ("tiny512", 1, 2, 512, 64, "fp32", False, 1.5, 1.0, None),
    ("tiny512_sc16", 1, 2, 512, 64, "fp32", False, 1.5, 16.0, None),
    ("fp32-causal-a125", 1, 1, 320, 128, "fp32", True, 1.25, 4.0, (1, 3)),
    ("bf16-causal-ragged", 1, 2, 1088, 128, "bf16", True, 1.5, 4.0, (1, 4)),
    ("bf16-causal-dense", 1, 1, 1024, 128, "bf16", True, 1.25, 1.0, (1, 8)),
    ("bf16-causal-d64", 1, 2, 576, 64, "bf16", True, 1.25, 4.0, (1, 3)),
    ("bf16-noncausal-a2", 1, 2, 512, 128, "bf16", False, 2.0, 4.0, (1, 3)),
    ("bf16-noncausal-d64-tile-tail", 2, 1, 1088, 64, "bf16", False, 1.5, 4.0, (1, 4)),
    ("bf16-causal-a1", 1, 1, 512, 128, "bf16", True, 1.0, 1.0, (1, 3)),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_small_full_oracle(case):
    name, B, H, T, D, dtype, causal, alpha, csm, planted = case
    _say(f"[backward] {name} B{B} H{H} T{T} D{D} {dtype} causal={causal} alpha={alpha}")
    w = inputs.make_prefill(B, H, T, D, dtype, causal, planted, seed=17 + T + D, device="cpu", with_dout=True)
    w = {k: v.to(DEV) for k, v in w.items()}
    cs = csm / math.sqrt(D)
    _, g = _run(w, alpha, causal, cs)
    prm = oracle.Params(alpha=alpha, causal=causal, coarse_scale=cs, storage=dtype)
    ref = oracle.backward(*(_np64(w[x]) for x in ("q", "k", "v", "dout")), prm)
    errs = {n: rel_l2(_np64(g[n]), ref[n]) for n in ("dq", "dk", "dv", "dkbar")}
    _say(f"  rel-L2 {errs}")
    for n, e in errs.items():
        assert e <= TOL, (name, n, e)


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("fp32", False), ("fp32", True)])
def test_backward_deterministic(dtype, causal):
    """Bitwise-equal gradients on a rerun (no floating-point atomics on any path)."""
    D = 128 if dtype == "bf16" else 64
    w = inputs.make_prefill(1, 2, 1024 if dtype == "bf16" else 512, D, dtype, causal, (1, 4) if causal else None,
                            seed=4, device="cpu", with_dout=True)
    w = {k: v.to(DEV) for k, v in w.items()}
    _, g1 = _run(w, 1.5, causal, 3 / math.sqrt(D))
    g1 = {k: v.clone() for k, v in g1.items()}
    _, g2 = _run(w, 1.5, causal, 3 / math.sqrt(D))
    for n in ("dq", "dk", "dv", "dkbar"):
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("alpha", [1.25, 1.5])
def test_backward_training_16k_sampled(alpha):
    wl = inputs.CONFIGS["train16k"]
    sh = wl.shape
    _say(f"[backward] train16k full size {sh} alpha={alpha} (sampled)")
    w = inputs.make_prefill(sh["B"], sh["H"], sh["T"], sh["D"], wl.dtype, True, wl.planted, wl.seed, device=DEV,
                            with_dout=True)
    _, g = _run(w, alpha, True, wl.coarse_scale)
    T = sh["T"]
    nb = T // 64
    prm = oracle.Params(alpha=alpha, causal=True, coarse_scale=wl.coarse_scale, storage="bf16")
    rng = np.random.default_rng(2)
    for (b, h) in [(0, int(rng.integers(sh["H"]))), (1, int(rng.integers(sh["H"])))]:
        x = {n: _np64(w[n][b:b + 1, h:h + 1]) for n in ("q", "k", "v", "dout")}
        tail = 4 * 64  # rows attending the last 4 key blocks
        rows = [(0, 0, i) for i in range(T - tail, T)]
        rows += [(0, 0, int(i)) for i in rng.choice(T - tail, size=24, replace=False)]
        ref = oracle.backward_rows(x["q"], x["k"], x["v"], x["dout"], prm, rows)
        ridx = np.array([i for (_, _, i) in rows])
        e_dq = rel_l2(_np64(g["dq"][b, h])[ridx], ref["dq"][0, 0][ridx])
        e_dk = rel_l2(_np64(g["dk"][b, h])[T - tail:], ref["dk"][0, 0][T - tail:])
        e_dv = rel_l2(_np64(g["dv"][b, h])[T - tail:], ref["dv"][0, 0][T - tail:])
        e_kb = rel_l2(_np64(g["dkbar"][b, h])[nb - 4:nb - 1], ref["dkbar"][0, 0][nb - 4:nb - 1])
        _say(f"  (b={b}, h={h}) rel-L2 dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e} dkbar {e_kb:.2e}")
        assert max(e_dq, e_dk, e_dv, e_kb) <= TOL


def test_backward_training_16k_full_head():
    """One (batch, head) slice of the 16K training workload at alpha 1.5, launched
    at full size: dQ of every row and dK, dV, dkbar of every key block against
    oracle.backward over all 16384 rows (run over worker processes)."""
    wl = inputs.CONFIGS["train16k"]
    sh = wl.shape
    _say(f"[backward] train16k full size {sh} alpha=1.5, one head compared whole")
    w = inputs.make_prefill(sh["B"], sh["H"], sh["T"], sh["D"], wl.dtype, True, wl.planted, wl.seed, device=DEV,
                            with_dout=True)
    _, g = _run(w, 1.5, True, wl.coarse_scale)
    b, h = 1, 5
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=wl.coarse_scale, storage="bf16")
    ref = oracle_parallel.backward_head(*(w[n][b, h] for n in ("q", "k", "v", "dout")), prm)
    errs = {n: rel_l2(_np64(g[n][b, h]), ref[n]) for n in ("dq", "dk", "dv", "dkbar")}
    # the first key blocks collect terms from up to 16K query rows: check them on their own too
    nb = sh["T"] // 64
    first = slice(0, 8 * 64)
    errs["dk_first8"] = rel_l2(_np64(g["dk"][b, h])[first], ref["dk"][first])
    errs["dv_first8"] = rel_l2(_np64(g["dv"][b, h])[first], ref["dv"][first])
    errs["dkbar_first8"] = rel_l2(_np64(g["dkbar"][b, h])[:8], ref["dkbar"][:8])
    # per key block: the worst block's relative error
    dkb = np.linalg.norm((_np64(g["dk"][b, h]) - ref["dk"]).reshape(nb, -1), axis=1) / np.maximum(
        np.linalg.norm(ref["dk"].reshape(nb, -1), axis=1), 1e-30)
    errs["dk_worst_block"] = float(dkb.max())
    _say(f"  rel-L2 {errs}")
    for n, e in errs.items():
        assert e <= TOL, (n, e)


@pytest.mark.parametrize("T,csm", [(65536, 2.0), (65536, 7.0), (98304, 2.0)], ids=["64k-literal", "64k-calibrated", "96k"])
def test_backward_long_sampled(T, csm):
    """Long prefills (T 65536 and 98304: tile lists of up to 1024 / 1536 blocks,
    the coarse kernel's summaries in 16 / 24 chunks, the dK/dV walk over up to
    1024 / 1536 query chunks), at the 64K workload's coarse scales: dQ on
    sampled rows and dK, dV and dkbar of the last key blocks (which only the
    last 256 rows attend) against oracle.backward_rows."""
    B, H, D = 1, 2, 128
    cs = csm / math.sqrt(D)
    _say(f"[backward] B{B} H{H} T{T} D{D} coarse {csm}/sqrt(D) (sampled)")
    w = inputs.make_prefill(B, H, T, D, "bf16", True, (1, 8), seed=1100 + int(csm) + T // 1024, device=DEV,
                            with_dout=True)
    _, g = _run(w, 1.5, True, cs)
    nb = T // 64
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=cs, storage="bf16")
    rng = np.random.default_rng(int(csm))
    for h in range(H):
        x = {n: _np64(w[n][0:1, h:h + 1]) for n in ("q", "k", "v", "dout")}
        tail = 4 * 64
        rows = [(0, 0, i) for i in range(T - tail, T)]
        rows += [(0, 0, int(i)) for i in rng.choice(T - tail, size=16, replace=False)]
        ref = oracle.backward_rows(x["q"], x["k"], x["v"], x["dout"], prm, rows)
        ridx = np.array([i for (_, _, i) in rows])
        e_dq = rel_l2(_np64(g["dq"][0, h])[ridx], ref["dq"][0, 0][ridx])
        e_dk = rel_l2(_np64(g["dk"][0, h])[T - tail:], ref["dk"][0, 0][T - tail:])
        e_dv = rel_l2(_np64(g["dv"][0, h])[T - tail:], ref["dv"][0, 0][T - tail:])
        e_kb = rel_l2(_np64(g["dkbar"][0, h])[nb - 4:nb - 1], ref["dkbar"][0, 0][nb - 4:nb - 1])
        _say(f"  h={h} rel-L2 dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e} dkbar {e_kb:.2e}")
        assert max(e_dq, e_dk, e_dv, e_kb) <= TOL
