"""Plain float64 CPU oracle for the DashAttention hot path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
reference that the HIP library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``differentiable_adaptive_block_amd``) never
imports it and shares no code with it.

Sources (the DashAttention pages; no line numbers, section names only):

* "DashAttention: Making Sparse Attention Fully Differentiable with Adaptive
  Block Selection" (alanhou.org blog), sections "Core Mechanism" and
  "Key Concepts": two stages, block scores q . summary, alpha-entmax with
  exact zeros, alpha=1 softmax / alpha=2 sparsemax, log of the coarse
  weights added to the fine logits, gradients through both stages.
* "DashAttention and the year sparse attention became a field"
  (montana-research blog), section "What alpha-entmax changes": Stage 0
  mean-pooling summaries, Stage 1 entmax routing, Stage 2 softmax with the
  routing weights as a prior on the logits; alpha 1.5 at inference, 1.25
  early in training.
* AdaSplash-2 abstract (thelatestinai.com page): the entmax normaliser tau is
  the expensive part; here it is found by plain bisection.

Readings where the pages are silent are listed in each function's docstring.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library routines, brute force, invariants or finite
differences.  The speed numbers on the pages are not pinned (they carry no
absolute values).
"""

from .entmax import entmax, entmax_threshold, entmax_jvp  # noqa: F401
from .gqa import select_row_group, forward_rows_gqa, forward_gqa, backward_gqa, decode_gqa  # noqa: F401
from .dash_ref import (  # noqa: F401
    Params,
    round_bf16,
    round_storage,
    pool_blocks,
    pool_attention,
    pool_attention_vjp,
    summarise,
    candidate_blocks,
    select_row,
    attend_row,
    forward,
    forward_rows,
    backward,
    backward_rows,
    decode,
    cache_append,
    decode_varlen,
)
