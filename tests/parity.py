"""Helpers shared by the GPU parity tests: tolerances and comparisons against the oracle.

Tolerances (the numerical bar of the forward, backward and decode paths):

* outputs O: bf16 tensors max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 tensors
  max-abs <= 1e-4;
* gradients: relative L2 error <= 5e-2;
* summaries kbar: bit-exact (both sides round the exact mean once);
* selection masks and selected counts: bit-exact, except for candidate
  blocks whose oracle score lies within 1e-6 (u-units) of the oracle tau;
* tau: |tau_gpu - tau_oracle| <= 4e-6 * max(1, |tau|) (fp32 arithmetic on
  values of order 1, a few ulp);
* log-sum-exp: max-abs <= 1e-3 for bf16 and 1e-4 for fp32 (fp32 sums of
  exactly-rounded bf16 products; the bf16 rounding of P does not enter it).
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
            tau_err = max(tau_err, abs(t - r["tau"]) / max(1.0, abs(r["tau"])))
        else:
            assert int(gpu["nsel"][b, h, i]) == 0
            assert not gpu["mask"][b, h, i].any()
    E = np.stack(errs)
    stats = dict(max_abs=float(E.max()), mean_abs=float(E.mean()), lse=lse_err, tau=tau_err, flips=flips)
    assert stats["max_abs"] <= max_out, f"{what}: O max-abs {stats}"
    assert stats["mean_abs"] <= mean_out, f"{what}: O mean-abs {stats}"
    assert stats["lse"] <= tol_lse(dtype), f"{what}: lse {stats}"
    assert stats["tau"] <= 4e-6, f"{what}: tau {stats}"
    return stats


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))
