"""DashAttention hot path for AMD Instinct MI355X (gfx950).

The compute lives in ``libdash.so`` (HIP kernels behind the C ABI of
``include/dash.h``); :mod:`.api` marshals PyTorch tensors into it.
"""

from . import inputs  # noqa: F401
