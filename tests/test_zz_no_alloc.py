"""dash_decode_static (the decode that takes its workspace from the library's
static device scratch) against dash_decode with a caller workspace, through
the C ABI: two calls in a row, the second smaller, each bit for bit equal."""

import math

import pytest
import torch

from differentiable_adaptive_block_amd import _lib, api, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outputs(p, q):
    S, H, D = q.shape
    nbw = (p.N // 64 + 31) // 32
    return dict(o=torch.empty((S, H, D), dtype=q.dtype, device=DEV),
                lse=torch.empty((S, H), dtype=torch.float32, device=DEV),
                nsel=torch.empty((S, H), dtype=torch.int32, device=DEV),
                tau=torch.empty((S, H), dtype=torch.float32, device=DEV),
                mask=torch.empty((S, H, nbw), dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("first,second", [((4, 8, 8192, 5.0), (2, 3, 2048, 3.0))])
def test_decode_static_equals_workspace_decode(first, second):
    st = torch.cuda.current_stream().cuda_stream
    for n, (S, H, N, csm) in enumerate((first, second)):
        w = inputs.make_decode(S, H, N, 128, "bf16", (1, 8), seed=70 + n, device=DEV)
        q, kc, vc = w["q"], w["k"], w["v"]
        kbar = api.pool(kc.view(1, S * H, N, 128)).view(S, H, N // 64, 128)
        p = api.make_decode_params(q, kc, 1.5, None, csm / math.sqrt(128))
        assert _lib.decode_workspace_bytes(p) <= _lib.decode_static_max_bytes()
        ref = api.decode(q, kc, vc, kbar, alpha=1.5, coarse_scale=p.coarse_scale)
        ref = {k: v.clone() for k, v in ref.items()}
        got = _outputs(p, q)
        _lib.decode_static(p, q.data_ptr(), kc.data_ptr(), vc.data_ptr(), kbar.data_ptr(), got["o"].data_ptr(),
                           got["lse"].data_ptr(), got["nsel"].data_ptr(), got["tau"].data_ptr(),
                           got["mask"].data_ptr(), st)
        torch.cuda.synchronize()
        for k in ("o", "lse", "nsel", "tau", "mask"):
            assert torch.equal(got[k], ref[k]), (n, k)
        assert int(got["nsel"].sum()) > 0
