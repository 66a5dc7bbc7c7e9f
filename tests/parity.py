"""Helpers shared by the GPU parity tests: tolerances and comparisons against the oracle.

Tolerances (the numerical bar of the forward, backward and decode paths):

* outputs O: bf16 tensors max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 tensors
  max-abs <= 1e-4;
* gradients: relative L2 error <= 5e-2;
* summaries kbar: bit-exact (both sides round the exact mean once);
* selection masks and selected counts: bit-exact, except for candidate
  blocks whose oracle score lies within 1e-6 (u-units) of the oracle tau;
* tau: |tau_gpu - tau_oracle| <= 1e-6 * max(1, |tau|), i.e. 1e-6 in u-units
  for the thresholds of order 1 these workloads have (the tie band's own
  width; fp32 resolves tau to about 1e-7 there);
* log-sum-exp: max-abs <= 4e-3 for bf16 and 1e-4 for fp32.  The bf16 bound
  follows from the kernel's arithmetic: the Stage-2 normaliser sums the
  weights as they are rounded to bf16 for the PV product, each within 2^-8
  relative of the exact weight, so its log lies within -ln(1 - 2^-8) =
  3.91e-3 of the exact log-sum-exp.
"""

from __future__ import annotations

import numpy as np
import torch

TIE_BAND = 1e-6


def tol_out(dtype):
    return (2e-2, 2e-3) if dtype == torch.bfloat16 else (1e-4, 1e-4)


def tol_lse(dtype):
    # bf16: the normaliser is the sum of the weights as rounded to bf16 for
    # the PV product (relative error <= 2^-8 each), so its log is within
    # -ln(1 - 2^-8) = 3.91e-3 of the exact one; fp32 keeps 1e-4
    return 4e-3 if dtype == torch.bfloat16 else 1e-4


def tau_tol(tau: float) -> float:
    return 1e-6 * max(1.0, abs(tau))


def unpack_mask(words: torch.Tensor, nb: int) -> np.ndarray:
    """int32 words [..., nbw] -> bool [..., nb] (bit b of word b//32)."""
    w = words.cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    bits = (w[..., :, None] >> np.arange(32)) & 1
    return bits.reshape(*w.shape[:-1], -1)[..., :nb].astype(bool)


def check_rows(gpu, ora_rows, rows, dtype, alpha, what=""):
    """Compare GPU forward outputs with oracle rows.

    ``gpu``: dict of numpy arrays o [B,H,T,D], lse [B,H,T], tau, nsel, mask
    (bool [B,H,T,nb]); ``ora_rows``: list of oracle dicts for ``rows``.
    Returns a dict of error statistics.
    """
    max_out, mean_out = tol_out(dtype)
    errs = []
    lse_err = 0.0
    tau_err = 0.0
    flips = 0
    for (b, h, i), r in zip(rows, ora_rows):
        e = np.abs(gpu["o"][b, h, i].astype(np.float64) - r["o"])
        errs.append(e)
        lse_err = max(lse_err, abs(float(gpu["lse"][b, h, i]) - r["lse"]))
        cand = r["cand"]
        if cand.size:
            gm = gpu["mask"][b, h, i][cand]
            om = r["mask"][cand]
            u = (alpha - 1.0) * r["z"] if alpha != 1.0 else r["z"]
            diff = gm != om
            if diff.any():
                near = np.abs(u - r["tau"]) <= TIE_BAND
                assert np.all(near[diff]), f"{what} row {(b, h, i)}: mask differs outside the tie band at blocks {cand[diff & ~near]}"
                flips += int(diff.sum())
            else:
                assert int(gpu["nsel"][b, h, i]) == r["nsel"], f"{what} row {(b, h, i)}: nsel {gpu['nsel'][b, h, i]} vs {r['nsel']}"
            assert not gpu["mask"][b, h, i][cand.size:].any(), "bits set beyond the candidate blocks"
            t = float(gpu["tau"][b, h, i])
            tau_err = max(tau_err, abs(t - r["tau"]) / tau_tol(r["tau"]))
        else:
            assert int(gpu["nsel"][b, h, i]) == 0
            assert not gpu["mask"][b, h, i].any()
    E = np.stack(errs)
    stats = dict(max_abs=float(E.max()), mean_abs=float(E.mean()), lse=lse_err, tau=tau_err, flips=flips)
    assert stats["max_abs"] <= max_out, f"{what}: O max-abs {stats}"
    assert stats["mean_abs"] <= mean_out, f"{what}: O mean-abs {stats}"
    assert stats["lse"] <= tol_lse(dtype), f"{what}: lse {stats}"
    assert stats["tau"] <= 1.0, f"{what}: tau error over its bound {stats}"
    return stats


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def check_mask_row(words, sel, alpha, what=""):
    """One row's selection bits from the GPU (32-bit words, any integer
    storage) against the oracle's Stage-1 result ``sel`` of the same row
    (``oracle.select_row``): equal on every candidate block whose oracle
    score lies outside the tie band, and no bit set past the candidates.
    Returns the number of candidates that differ inside the band."""
    w = np.asarray(words.cpu().numpy() if isinstance(words, torch.Tensor) else words).astype(np.int64) & 0xFFFFFFFF
    bits = ((w[:, None] >> np.arange(32)) & 1).reshape(-1).astype(bool)
    cand = sel["cand"]
    n = cand.size
    assert not bits[n:].any(), f"{what}: bits set past the {n} candidate blocks"
    if n == 0:
        return 0
    diff = bits[cand] != sel["support"]
    if not diff.any():
        return 0
    u = (alpha - 1.0) * sel["z"] if alpha != 1.0 else sel["z"]
    near = np.abs(u - sel["tau"]) <= TIE_BAND
    assert np.all(near[diff]), f"{what}: selection differs outside the tie band at blocks {cand[diff & ~near]}"
    return int(diff.sum())


def check_stage1_head(words, tau, nsel, sels, alpha, what=""):
    """Stage-1 outputs of every row of one head (mask words [T, nbw], tau [T],
    nsel [T], as numpy arrays) against the oracle's select_row results
    ``sels`` (one per row, in row order).  Returns (flips in the tie band,
    largest tau error over its bound)."""
    flips = 0
    worst = 0.0
    for i, sel in enumerate(sels):
        f = check_mask_row(words[i], sel, alpha, f"{what} row {i}")
        flips += f
        ns, nso = int(nsel[i]), int(sel["support"].sum())
        assert ns == nso if f == 0 else abs(ns - nso) <= f, f"{what} row {i}: nsel {ns} vs {nso}"
        if sel["cand"].size:
            worst = max(worst, abs(float(tau[i]) - sel["tau"]) / tau_tol(sel["tau"]))
        else:
            assert ns == 0
    assert worst <= 1.0, f"{what}: tau error {worst} x its bound"
    return flips, worst


def check_out_rows(o, lse, ora, rows, dtype, what=""):
    """Stage-2 outputs of one head (o [T, D], lse [T] numpy) on ``rows``
    against the oracle's forward_rows dicts ``ora`` (same order)."""
    max_out, mean_out = tol_out(dtype)
    E = np.stack([np.abs(o[i].astype(np.float64) - r["o"]) for i, r in zip(rows, ora)])
    lerr = max(abs(float(lse[i]) - r["lse"]) for i, r in zip(rows, ora))
    st = dict(max_abs=float(E.max()), mean_abs=float(E.mean()), lse=lerr, rows=len(rows))
    assert st["max_abs"] <= max_out and st["mean_abs"] <= mean_out, f"{what}: O {st}"
    assert lerr <= tol_lse(dtype), f"{what}: lse {st}"
    return st
