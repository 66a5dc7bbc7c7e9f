"""The C ABI on the host (no GPU needed): exports and argument validation.

Every call here fails validation, which happens before anything is launched,
so no device work is enqueued.  Fake device pointers are 16-byte aligned
integers that are never dereferenced.
"""

import ctypes
import os
import re

import pytest

from differentiable_adaptive_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dash.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from differentiable_adaptive_block_amd import build
        build.build()
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dash_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTS)


def _params(**kw):
    p = _lib.DashParams()
    p.B, p.H, p.T, p.D, p.block = 1, 2, 256, 128, 64
    p.alpha, p.causal, p.fine_scale, p.coarse_scale, p.dtype = 1.5, 1, 0.088, 0.088, _lib.DASH_BF16
    for k, v in kw.items():
        setattr(p, k, v)
    return p


FAKE = 0x10000  # aligned, never dereferenced


def _sel(**kw):
    s = _lib.DashSel()
    for f, _ in s._fields_:
        setattr(s, f, FAKE)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _fwd(L, p, **ptrs):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, kbar=FAKE)
    a.update(ptrs)
    return L.dash_fwd(ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["lse"], a["kbar"],
                      ctypes.byref(_sel()), None, 0, None)


@pytest.mark.parametrize("field,value,status", [
    ("T", 0, _lib.DASH_EINVAL),
    ("B", 0, _lib.DASH_EINVAL),
    ("alpha", 2.5, _lib.DASH_EINVAL),
    ("alpha", 0.5, _lib.DASH_EINVAL),
    ("alpha", float("nan"), _lib.DASH_EINVAL),
    ("fine_scale", 0.0, _lib.DASH_EINVAL),
    ("coarse_scale", float("inf"), _lib.DASH_EINVAL),
    ("causal", 2, _lib.DASH_EINVAL),
    ("dtype", 7, _lib.DASH_EINVAL),
    ("block", 32, _lib.DASH_EUNSUPPORTED),
    ("D", 96, _lib.DASH_EUNSUPPORTED),
    ("T", 98304 + 64, _lib.DASH_EUNSUPPORTED),
])
def test_fwd_rejects_bad_params(L, field, value, status):
    p = _params(**{field: value})
    assert _fwd(L, p) == status
    assert L.dash_last_error().decode() != ""


def test_fwd_rejects_null_and_misaligned_pointers(L):
    p = _params()
    assert _fwd(L, p, q=None) == _lib.DASH_EINVAL
    assert _fwd(L, p, o=FAKE + 2) == _lib.DASH_EINVAL
    bad = _sel(tau=None)
    assert L.dash_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(bad), None, 0,
                      None) == _lib.DASH_EINVAL
    assert L.dash_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0,
                      None) == _lib.DASH_EINVAL


def test_bwd_checks_workspace_size(L):
    p = _params()
    need = L.dash_bwd_workspace_bytes(ctypes.byref(p))
    assert need > 0
    st = L.dash_bwd(ctypes.byref(p), *([FAKE] * 7), ctypes.byref(_sel()), FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                    None)
    assert st == _lib.DASH_EWORKSPACE
    assert "workspace" in L.dash_last_error().decode()


def test_sel_sizes(L):
    p = _params(T=1088)
    sizes = _lib.sel_sizes(p)
    nb, nbw, nt = 17, 1, 9
    assert sizes == [2 * 1088, 2 * 1088, 2 * 1088, 2 * 1088 * nbw, 2 * nt, 2 * nt * nb, 2 * nt * nbw, 2 * 1088]
    assert _lib.query_tile() == 128
    with pytest.raises(_lib.DashError) as e:
        _lib.sel_sizes(_params(D=32))
    assert e.value.status == _lib.DASH_EUNSUPPORTED


def test_decode_validation(L):
    p = _lib.DashDecodeParams()
    p.S, p.H, p.N, p.D, p.block = 2, 2, 1024, 128, 64
    p.alpha, p.fine_scale, p.coarse_scale, p.dtype = 1.5, 0.088, 0.088, _lib.DASH_BF16
    need = L.dash_decode_workspace_bytes(ctypes.byref(p))
    assert need > 0
    # q, kc, vc, kbar, o, lse, nsel, tau, mask, ws
    args = [FAKE] * 5 + [None, None, None, None, FAKE]
    assert L.dash_decode(ctypes.byref(p), *args, need - 1, None) == _lib.DASH_EWORKSPACE
    bad = list(args)
    bad[8] = FAKE + 4  # a mask that is not 16-byte aligned
    assert L.dash_decode(ctypes.byref(p), *bad, need, None) == _lib.DASH_EINVAL
    assert "mask" in L.dash_last_error().decode()
    p.N = 1000
    assert L.dash_decode(ctypes.byref(p), *args, need, None) == _lib.DASH_EINVAL
    p.N, p.dtype = 1024, _lib.DASH_F32
    assert L.dash_decode(ctypes.byref(p), *args, need, None) == _lib.DASH_EUNSUPPORTED
    p.dtype, p.D = _lib.DASH_BF16, 64
    assert L.dash_decode(ctypes.byref(p), *args, need, None) == _lib.DASH_EUNSUPPORTED
    p.D, p.N = 128, 64 * 4096
    assert L.dash_decode(ctypes.byref(p), *args, need, None) == _lib.DASH_EUNSUPPORTED


def test_pool_accepts_long_sequences_in_validation(L):
    p = _params(T=98304)
    # null k is rejected after the shape checks pass (no 65536 limit for pooling)
    assert L.dash_pool(ctypes.byref(p), None, FAKE, None) == _lib.DASH_EINVAL
    assert "k and kbar" in L.dash_last_error().decode()


def _dparams(**kw):
    p = _lib.DashDecodeParams()
    p.S, p.H, p.N, p.D, p.block = 2, 2, 1024, 128, 64
    p.alpha, p.fine_scale, p.coarse_scale, p.dtype = 1.5, 0.088, 0.088, _lib.DASH_BF16
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_cache_append_validation(L):
    p = _dparams()
    # k_new, v_new, len, kc, vc, kbar
    assert L.dash_cache_append(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == _lib.DASH_EINVAL
    assert "len" in L.dash_last_error().decode()
    assert L.dash_cache_append(ctypes.byref(p), FAKE, FAKE, FAKE + 2, FAKE, FAKE, FAKE, None) == _lib.DASH_EINVAL
    assert L.dash_cache_append(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.DASH_EINVAL
    assert L.dash_cache_append(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, None) == _lib.DASH_EINVAL
    assert L.dash_cache_append(ctypes.byref(_dparams(N=1000)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.DASH_EINVAL
    assert L.dash_cache_append(ctypes.byref(_dparams(dtype=_lib.DASH_F32)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None) == _lib.DASH_EUNSUPPORTED


def test_decode_varlen_and_step_validation(L):
    p = _dparams()
    need = L.dash_decode_workspace_bytes(ctypes.byref(p))
    # q, kc, vc, kbar, len, o, lse, nsel, tau, mask, ws
    args = [FAKE] * 6 + [None, None, None, None, FAKE]
    assert L.dash_decode_varlen(ctypes.byref(p), *args, need - 1, None) == _lib.DASH_EWORKSPACE
    bad = list(args)
    bad[4] = None
    assert L.dash_decode_varlen(ctypes.byref(p), *bad, need, None) == _lib.DASH_EINVAL
    assert "len" in L.dash_last_error().decode()
    assert L.dash_decode_varlen(ctypes.byref(_dparams(N=64 * 4096)), *args, need, None) == _lib.DASH_EUNSUPPORTED
    # q, k_new, v_new, len, kc, vc, kbar, o, lse, nsel, tau, mask, ws
    sargs = [FAKE] * 8 + [None, None, None, None, FAKE]
    assert L.dash_decode_step(ctypes.byref(p), *sargs, need - 1, None) == _lib.DASH_EWORKSPACE
    bad = list(sargs)
    bad[1] = None
    assert L.dash_decode_step(ctypes.byref(p), *bad, need, None) == _lib.DASH_EINVAL
    bad = list(sargs)
    bad[7] = None
    assert L.dash_decode_step(ctypes.byref(p), *bad, need, None) == _lib.DASH_EINVAL
    assert L.dash_decode_step(ctypes.byref(_dparams(D=64)), *sargs, need, None) == _lib.DASH_EUNSUPPORTED


def test_summariser_entry_validation(L):
    p = _params(T=98304)
    # pooling accepts long sequences (no 65536 limit), rejects null pointers
    assert L.dash_pool_attn(ctypes.byref(p), FAKE, None, FAKE, None) == _lib.DASH_EINVAL
    assert L.dash_pool_attn(ctypes.byref(_params(T=100)), FAKE, FAKE, FAKE, None) == _lib.DASH_EINVAL
    p = _params()
    assert L.dash_select(ctypes.byref(p), FAKE, None, ctypes.byref(_sel()), None) == _lib.DASH_EINVAL
    assert L.dash_select(ctypes.byref(p), FAKE, FAKE, ctypes.byref(_sel(tau=None)), None) == _lib.DASH_EINVAL
    need = L.dash_pool_attn_bwd_workspace_bytes(ctypes.byref(p))
    assert need == 1 * 2 * (256 // 64) * 128 * 4
    args = [FAKE] * 5
    assert L.dash_pool_attn_bwd(ctypes.byref(p), *args, FAKE, need - 1, None) == _lib.DASH_EWORKSPACE
    assert L.dash_pool_attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, need, None) == _lib.DASH_EINVAL
    wsb = L.dash_bwd_workspace_bytes(ctypes.byref(p))
    bargs = [FAKE] * 7 + [ctypes.byref(_sel())] + [FAKE] * 5
    assert L.dash_bwd_no_pool(ctypes.byref(p), *bargs, wsb - 1, None) == _lib.DASH_EWORKSPACE
    assert L.dash_bwd_no_pool(ctypes.byref(_params(D=96)), *bargs, wsb, None) != _lib.DASH_OK


def test_gqa_entry_validation(L):
    p = _params(H=4)
    # q, k, v, o, lse, kbar, sel
    args = [FAKE] * 6 + [ctypes.byref(_sel())]
    assert L.dash_fwd_gqa(ctypes.byref(p), 3, *args, None) == _lib.DASH_EINVAL
    assert "kv_heads" in L.dash_last_error().decode()
    assert L.dash_fwd_gqa(ctypes.byref(p), 0, *args, None) == _lib.DASH_EINVAL
    assert L.dash_fwd_gqa(ctypes.byref(_params(H=4, dtype=_lib.DASH_F32, D=64)), 2, *args, None) == _lib.DASH_EUNSUPPORTED
    assert L.dash_bwd_gqa_workspace_bytes(ctypes.byref(p), 3) == 0
    need = L.dash_bwd_gqa_workspace_bytes(ctypes.byref(p), 2)
    assert need > L.dash_bwd_workspace_bytes(ctypes.byref(p)) > 0
    assert L.dash_bwd_gqa_workspace_bytes(ctypes.byref(p), 4) == L.dash_bwd_workspace_bytes(ctypes.byref(p))
    bargs = [FAKE] * 7 + [ctypes.byref(_sel())] + [FAKE] * 5
    assert L.dash_bwd_gqa(ctypes.byref(p), 2, *bargs, need - 1, None) == _lib.DASH_EWORKSPACE
    assert L.dash_bwd_gqa(ctypes.byref(p), 3, *bargs, need, None) == _lib.DASH_EINVAL


def test_partial_last_block_validation(L):
    # a T that is not a multiple of 64: causal only, through dash_fwd / dash_bwd with a workspace
    assert _fwd(L, _params(T=100, causal=0)) == _lib.DASH_EINVAL
    assert "causal" in L.dash_last_error().decode()
    p = _params(T=100)
    # the forward handles the partial block inside its kernels: no workspace
    assert L.dash_fwd_workspace_bytes(ctypes.byref(p)) == 0
    assert L.dash_fwd_workspace_bytes(ctypes.byref(_params())) == 0
    assert _fwd(L, p, lse=FAKE + 4) == _lib.DASH_EINVAL  # validated before any launch
    assert L.dash_bwd_workspace_bytes(ctypes.byref(p)) > L.dash_bwd_workspace_bytes(ctypes.byref(_params(T=128)))
    sizes = (ctypes.c_size_t * 8)()
    assert L.dash_sel_sizes(ctypes.byref(p), sizes) == _lib.DASH_OK
    assert sizes[0] == 1 * 2 * 128  # rows laid out as whole blocks
    # the stage entry points keep whole blocks
    assert L.dash_fwd_select(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(_sel()), None) == _lib.DASH_EINVAL
    assert L.dash_pool(ctypes.byref(p), FAKE, FAKE, None) == _lib.DASH_EINVAL
    assert L.dash_fwd_gqa(ctypes.byref(p), 2, *([FAKE] * 6), ctypes.byref(_sel()), None) == _lib.DASH_EINVAL


def test_gqa_decode_validation(L):
    p = _dparams(H=4)
    need = L.dash_decode_workspace_bytes(ctypes.byref(p))
    # q, kc, vc, kbar, len, o, lse, nsel, tau, mask, ws
    args = [FAKE] * 4 + [None, FAKE, None, None, None, None, FAKE]
    assert L.dash_decode_gqa(ctypes.byref(p), 3, *args, need, None) == _lib.DASH_EINVAL
    assert L.dash_decode_gqa(ctypes.byref(p), 2, *args, need - 1, None) == _lib.DASH_EWORKSPACE
    bad = list(args)
    bad[4] = FAKE + 2
    assert L.dash_decode_gqa(ctypes.byref(p), 2, *bad, need, None) == _lib.DASH_EINVAL
    p16 = _dparams(H=16)
    need16 = L.dash_decode_workspace_bytes(ctypes.byref(p16))
    assert L.dash_decode_gqa(ctypes.byref(p16), 1, *args, need16, None) == _lib.DASH_EUNSUPPORTED


def test_decode_static_rejects_sizes_beyond_its_scratch(L):
    """Validation runs before anything touches the GPU: a decode whose workspace
    exceeds the static scratch is refused with DASH_EWORKSPACE."""
    assert L.dash_decode_static_max_bytes() == 32 << 20
    p = _dparams(S=16, H=64, N=131072)
    assert L.dash_decode_workspace_bytes(ctypes.byref(p)) > L.dash_decode_static_max_bytes()
    args = [FAKE] * 5 + [None, None, None, None]
    assert L.dash_decode_static(ctypes.byref(p), *args, None) == _lib.DASH_EWORKSPACE
    assert "static scratch" in L.dash_last_error().decode()
    assert L.dash_decode_static(ctypes.byref(_dparams(N=1000)), *args, None) == _lib.DASH_EINVAL


def _lowdens(L, p, sel=None, ratio=4.0, ws=FAKE, wsb=1 << 40):
    return L.dash_fwd_attend_lowdens(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ctypes.byref(sel or _sel()),
                                     ratio, FAKE, FAKE, ws, wsb, None)


def test_lowdens_workspace_grows_by_pair(L):
    for D in (64, 128):
        p = _params(D=D, B=2, H=4, T=4096)
        base = L.dash_fwd_lowdens_workspace_bytes(ctypes.byref(p), 0)
        assert base > 8 * 2 * 4 * 4096  # the per-row (first pair, count) table at least
        n = 1 << 20
        grow = L.dash_fwd_lowdens_workspace_bytes(ctypes.byref(p), n) - base
        per = 20 + 2 * D
        assert per * n <= grow <= per * n + n // 128 * 16 + 8 * 256
        assert L.dash_fwd_lowdens_workspace_bytes(ctypes.byref(p), -1) == 0
        assert L.dash_fwd_lowdens_workspace_bytes(ctypes.byref(p), 1 << 31) == 0  # pair indices are int32


def test_lowdens_entry_validation(L):
    p = _params()
    base = L.dash_fwd_lowdens_workspace_bytes(ctypes.byref(p), 0)
    assert _lowdens(L, p, ratio=float("nan")) == _lib.DASH_EINVAL
    assert _lowdens(L, p, ratio=-1.0) == _lib.DASH_EINVAL
    assert _lowdens(L, _params(dtype=_lib.DASH_F32)) == _lib.DASH_EUNSUPPORTED
    assert _lowdens(L, _params(causal=0)) == _lib.DASH_EUNSUPPORTED
    assert _lowdens(L, p, sel=_sel(mask=None)) == _lib.DASH_EUNSUPPORTED
    assert _lowdens(L, p, wsb=base - 1) == _lib.DASH_EWORKSPACE
    assert "workspace" in L.dash_last_error().decode()
    assert _lowdens(L, p, ws=None, wsb=base) == _lib.DASH_EINVAL
    assert _lowdens(L, _params(T=300)) == _lib.DASH_EINVAL  # whole blocks only


def test_lowdens_workspace_sizes_are_monotone(L):
    """dash_fwd_lowdens_workspace_bytes grows with the pair count (the library derives the
    capacity of a workspace by searching these sizes; that an exactly sized workspace holds
    every pair is checked on the GPU, tests/test_gpu_lowdens.py)."""
    p = _params(T=4096)
    for n in (1, 127, 128, 100003, 7 << 20):
        need = L.dash_fwd_lowdens_workspace_bytes(ctypes.byref(p), n)
        assert L.dash_fwd_lowdens_workspace_bytes(ctypes.byref(p), n - 1) <= need
        assert L.dash_fwd_lowdens_workspace_bytes(ctypes.byref(p), n + 1024) > need
