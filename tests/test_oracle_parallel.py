"""The worker-process runner of the oracle returns the oracle's own results (CPU)."""

import numpy as np
import torch

import oracle
import oracle_parallel
from differentiable_adaptive_block_amd import inputs


def _case():
    w = inputs.make_prefill(1, 1, 320, 64, "bf16", True, (1, 3), seed=61, device="cpu", with_dout=True)
    prm = oracle.Params(alpha=1.5, causal=True, coarse_scale=4 / 8.0, storage="bf16")
    return w, prm


def test_parallel_backward_equals_serial():
    w, prm = _case()
    ref = oracle.backward(*(w[n].double().numpy() for n in ("q", "k", "v", "dout")), prm)
    par = oracle_parallel.backward_head(*(w[n][0, 0] for n in ("q", "k", "v", "dout")), prm, workers=3)
    for n in ("dq", "dk", "dv", "dkbar"):
        np.testing.assert_allclose(par[n], ref[n][0, 0], rtol=0, atol=1e-12)


def test_parallel_forward_and_select_equal_serial():
    w, prm = _case()
    q, k, v = (w[n].double().numpy() for n in ("q", "k", "v"))
    rows = [0, 5, 64, 130, 319]
    ref = oracle.forward_rows(q, k, v, prm, [(0, 0, i) for i in rows])
    par = oracle_parallel.forward_rows(w["q"][0, 0], w["k"][0, 0], w["v"][0, 0], prm, rows, workers=2)
    for a, b in zip(ref, par):
        np.testing.assert_array_equal(a["o"], b["o"])
        assert a["lse"] == b["lse"] and a["nsel"] == b["nsel"]
    kb = torch.from_numpy(oracle.pool_blocks(k[0, 0], 64, "bf16")).to(torch.bfloat16)
    sels = oracle_parallel.select_rows(w["q"][0, 0], kb, prm, rows, workers=2)
    for i, s in zip(rows, sels):
        r = oracle.select_row(q[0, 0, i], oracle.pool_blocks(k[0, 0], 64, "bf16"), i, prm, 64)
        np.testing.assert_array_equal(s["support"], r["support"])
        assert (np.isnan(s["tau"]) and np.isnan(r["tau"])) or s["tau"] == r["tau"]
