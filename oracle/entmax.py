"""alpha-entmax by bisection on the threshold tau (float64).  Test infrastructure only.

Definition followed (page "DashAttention: Making Sparse Attention Fully
Differentiable...", section "Key Concepts", alpha-entmax bullet; page
"DashAttention and the year sparse attention became a field", section "What
alpha-entmax changes"): alpha-entmax maps scores to a probability vector that
is exactly zero below a data-dependent threshold; alpha = 1 is softmax and
alpha = 2 is sparsemax; larger alpha is sparser.

Reading (the pages print no formula): the standard parameterisation

    u = (alpha - 1) * z,   p_b = [u_b - tau]_+ ** (1 / (alpha - 1)),
    tau chosen so that sum_b p_b = 1,

which gives sparsemax at alpha = 2 and softmax as alpha -> 1.  For
alpha = 1 the oracle uses p_b = exp(z_b - tau), tau = log-sum-exp(z).
"""

from __future__ import annotations

import numpy as np


def entmax_threshold(z, alpha: float, max_iter: int = 400) -> float:
    """Threshold tau of alpha-entmax over the 1-D score vector ``z`` (n >= 1).

    tau is returned in the units of ``p``: u-units ((alpha-1) z) for
    alpha > 1, z-units for alpha = 1.

    Bisection on the decreasing function f(t) = sum_b p_b(t) - 1:

    * alpha > 1: bracket [max u - 1, max u].  f(max u - 1) >= 0 because the
      largest term alone is 1; f(max u) = -1.  The bracket does not depend on
      n, and f sums only the terms with u_b > t, so adding scores far below
      tau changes nothing (the non-dispersive property).
    * alpha = 1: bracket [max z, max z + log n].

    The loop halves the bracket until no float64 lies strictly inside it,
    keeping f(lo) >= 0 > f(hi); ``lo`` is returned, so a score equal to tau
    gets weight exactly zero.
    """
    z = np.asarray(z, dtype=np.float64).ravel()
    n = z.size
    if n == 0:
        raise ValueError("entmax over an empty candidate set")
    if alpha < 1.0 or alpha > 2.0:
        raise ValueError("alpha must lie in [1, 2]")
    if alpha == 1.0:
        lo = float(z.max())
        hi = lo + float(np.log(n))

        def f(t):
            return float(np.sum(np.exp(z - t))) - 1.0
    else:
        u = (alpha - 1.0) * z
        m = 1.0 / (alpha - 1.0)
        hi = float(u.max())
        lo = hi - 1.0

        def f(t):
            return float(np.sum((u[u > t] - t) ** m)) - 1.0

    if hi == lo:  # alpha = 1, n = 1
        return lo
    for _ in range(max_iter):
        mid = 0.5 * (lo + hi)
        if not (lo < mid < hi):
            break
        if f(mid) >= 0.0:
            lo = mid
        else:
            hi = mid
    return lo


def entmax(z, alpha: float):
    """alpha-entmax of the score vector ``z``.

    Returns ``(p, tau, support)``: probabilities (renormalised to sum 1 in
    float64, as the bisection leaves sum p within a few ulp of 1), the
    threshold in p's units (see :func:`entmax_threshold`) and the boolean
    support {b : p_b > 0}.
    """
    z = np.asarray(z, dtype=np.float64).ravel()
    tau = entmax_threshold(z, alpha)
    if alpha == 1.0:
        p = np.exp(z - tau)
        support = np.ones(z.size, dtype=bool)
    else:
        u = (alpha - 1.0) * z
        support = u > tau
        p = np.zeros_like(z)
        p[support] = (u[support] - tau) ** (1.0 / (alpha - 1.0))
    p = p / p.sum()
    return p, tau, support


def entmax_jvp(p, g, alpha: float):
    """Vector-Jacobian product of alpha-entmax with respect to z.

    With s = p ** (2 - alpha) on the support (0 elsewhere), the Jacobian of
    p with respect to z is diag(s) - s s^T / sum(s) (derived by
    differentiating sum_b [(alpha-1) z_b - tau]^(1/(alpha-1)) = 1 in tau), so

        dz = s * g - s * <s, g> / sum(s).

    At alpha = 1, s = p (the softmax Jacobian).  Page "DashAttention: Making
    Sparse Attention Fully Differentiable...", section "Core Mechanism":
    gradients flow from Stage 2 back through the log into the entmax.
    """
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    s = np.zeros_like(p)
    nz = p > 0
    s[nz] = p[nz] ** (2.0 - alpha)
    ssum = s.sum()
    if ssum == 0.0:
        return np.zeros_like(p)
    return s * g - s * (np.dot(s, g) / ssum)
