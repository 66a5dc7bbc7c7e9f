"""ctypes binding of libdash.so (argument marshalling only).

Every entry point mirrors a declaration of include/dash.h.  Nothing here
computes any part of the method; when the library is missing the import of
this module fails loudly.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdash.so")

DASH_OK, DASH_EINVAL, DASH_EUNSUPPORTED, DASH_EWORKSPACE, DASH_EHIP = range(5)
DASH_F32, DASH_BF16 = 0, 1
STATUS_NAMES = {0: "DASH_OK", 1: "DASH_EINVAL", 2: "DASH_EUNSUPPORTED", 3: "DASH_EWORKSPACE", 4: "DASH_EHIP"}

EXPORTS = [
    "dash_query_tile",
    "dash_sel_sizes",
    "dash_fwd_workspace_bytes",
    "dash_bwd_workspace_bytes",
    "dash_pool",
    "dash_fwd",
    "dash_fwd_select",
    "dash_fwd_attend",
    "dash_fwd_lowdens_workspace_bytes",
    "dash_fwd_attend_lowdens",
    "dash_bwd",
    "dash_fwd_gqa",
    "dash_bwd_gqa_workspace_bytes",
    "dash_bwd_gqa",
    "dash_pool_attn",
    "dash_select",
    "dash_bwd_no_pool",
    "dash_pool_attn_bwd_workspace_bytes",
    "dash_pool_attn_bwd",
    "dash_bwd_learned_workspace_bytes",
    "dash_bwd_learned",
    "dash_decode_workspace_bytes",
    "dash_decode",
    "dash_cache_append",
    "dash_decode_varlen",
    "dash_decode_step",
    "dash_decode_gqa",
    "dash_decode_static_max_bytes",
    "dash_decode_static",
    "dash_last_error",
]


class DashParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
        ("block", ctypes.c_int32), ("alpha", ctypes.c_float), ("causal", ctypes.c_int32),
        ("fine_scale", ctypes.c_float), ("coarse_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
    ]


class DashSel(ctypes.Structure):
    _fields_ = [
        ("tau", ctypes.c_void_p), ("lognorm", ctypes.c_void_p), ("nsel", ctypes.c_void_p),
        ("mask", ctypes.c_void_p), ("tile_cnt", ctypes.c_void_p), ("tile_blk", ctypes.c_void_p),
        ("tile_bits", ctypes.c_void_p), ("passes", ctypes.c_void_p),
    ]


class DashDecodeParams(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
        ("block", ctypes.c_int32), ("alpha", ctypes.c_float), ("fine_scale", ctypes.c_float),
        ("coarse_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
    ]


class DashError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libdash.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m differentiable_adaptive_block_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    L.dash_query_tile.restype = ctypes.c_int32
    L.dash_query_tile.argtypes = []
    L.dash_sel_sizes.restype = ctypes.c_int
    L.dash_sel_sizes.argtypes = [P(DashParams), P(ctypes.c_size_t)]
    L.dash_fwd_workspace_bytes.restype = ctypes.c_size_t
    L.dash_fwd_workspace_bytes.argtypes = [P(DashParams)]
    L.dash_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.dash_bwd_workspace_bytes.argtypes = [P(DashParams)]
    L.dash_pool.restype = ctypes.c_int
    L.dash_pool.argtypes = [P(DashParams), vp, vp, vp]
    L.dash_fwd.restype = ctypes.c_int
    L.dash_fwd.argtypes = [P(DashParams), vp, vp, vp, vp, vp, vp, P(DashSel), vp, ctypes.c_size_t, vp]
    L.dash_fwd_select.restype = ctypes.c_int
    L.dash_fwd_select.argtypes = [P(DashParams), vp, vp, vp, P(DashSel), vp]
    L.dash_fwd_attend.restype = ctypes.c_int
    L.dash_fwd_attend.argtypes = [P(DashParams), vp, vp, vp, vp, P(DashSel), vp, vp, vp]
    L.dash_fwd_lowdens_workspace_bytes.restype = ctypes.c_size_t
    L.dash_fwd_lowdens_workspace_bytes.argtypes = [P(DashParams), ctypes.c_int64]
    L.dash_fwd_attend_lowdens.restype = ctypes.c_int
    L.dash_fwd_attend_lowdens.argtypes = [P(DashParams), vp, vp, vp, vp, P(DashSel), ctypes.c_float, vp, vp, vp,
                                          ctypes.c_size_t, vp]
    L.dash_bwd.restype = ctypes.c_int
    L.dash_bwd.argtypes = [P(DashParams), vp, vp, vp, vp, vp, vp, vp, P(DashSel), vp, vp, vp, vp, vp,
                           ctypes.c_size_t, vp]
    i32 = ctypes.c_int32
    L.dash_fwd_gqa.restype = ctypes.c_int
    L.dash_fwd_gqa.argtypes = [P(DashParams), i32, vp, vp, vp, vp, vp, vp, P(DashSel), vp]
    L.dash_bwd_gqa_workspace_bytes.restype = ctypes.c_size_t
    L.dash_bwd_gqa_workspace_bytes.argtypes = [P(DashParams), i32]
    L.dash_bwd_gqa.restype = ctypes.c_int
    L.dash_bwd_gqa.argtypes = [P(DashParams), i32, vp, vp, vp, vp, vp, vp, vp, P(DashSel), vp, vp, vp, vp, vp,
                               ctypes.c_size_t, vp]
    L.dash_pool_attn.restype = ctypes.c_int
    L.dash_pool_attn.argtypes = [P(DashParams), vp, vp, vp, vp]
    L.dash_select.restype = ctypes.c_int
    L.dash_select.argtypes = [P(DashParams), vp, vp, P(DashSel), vp]
    L.dash_bwd_no_pool.restype = ctypes.c_int
    L.dash_bwd_no_pool.argtypes = [P(DashParams), vp, vp, vp, vp, vp, vp, vp, P(DashSel), vp, vp, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    L.dash_pool_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.dash_pool_attn_bwd_workspace_bytes.argtypes = [P(DashParams)]
    L.dash_pool_attn_bwd.restype = ctypes.c_int
    L.dash_pool_attn_bwd.argtypes = [P(DashParams), vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.dash_bwd_learned_workspace_bytes.restype = ctypes.c_size_t
    L.dash_bwd_learned_workspace_bytes.argtypes = [P(DashParams)]
    L.dash_bwd_learned.restype = ctypes.c_int
    L.dash_bwd_learned.argtypes = [P(DashParams), vp, vp, vp, vp, vp, vp, vp, P(DashSel), vp, vp, vp, vp, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    L.dash_decode_workspace_bytes.restype = ctypes.c_size_t
    L.dash_decode_workspace_bytes.argtypes = [P(DashDecodeParams)]
    L.dash_decode.restype = ctypes.c_int
    L.dash_decode.argtypes = [P(DashDecodeParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.dash_cache_append.restype = ctypes.c_int
    L.dash_cache_append.argtypes = [P(DashDecodeParams), vp, vp, vp, vp, vp, vp, vp]
    L.dash_decode_varlen.restype = ctypes.c_int
    L.dash_decode_varlen.argtypes = [P(DashDecodeParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
    L.dash_decode_step.restype = ctypes.c_int
    L.dash_decode_step.argtypes = [P(DashDecodeParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    L.dash_decode_gqa.restype = ctypes.c_int
    L.dash_decode_gqa.argtypes = [P(DashDecodeParams), ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  vp, ctypes.c_size_t, vp]
    L.dash_decode_static_max_bytes.restype = ctypes.c_size_t
    L.dash_decode_static_max_bytes.argtypes = []
    L.dash_decode_static.restype = ctypes.c_int
    L.dash_decode_static.argtypes = [P(DashDecodeParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.dash_last_error.restype = ctypes.c_char_p
    L.dash_last_error.argtypes = []
    _lib = L
    return L


def check(status: int) -> None:
    if status != DASH_OK:
        raise DashError(status, load().dash_last_error().decode())


def query_tile() -> int:
    return int(load().dash_query_tile())


def sel_sizes(p: DashParams):
    out = (ctypes.c_size_t * 8)()
    check(load().dash_sel_sizes(ctypes.byref(p), out))
    return list(out)


def fwd_workspace_bytes(p: DashParams) -> int:
    return int(load().dash_fwd_workspace_bytes(ctypes.byref(p)))


def bwd_workspace_bytes(p: DashParams) -> int:
    return int(load().dash_bwd_workspace_bytes(ctypes.byref(p)))


def decode_workspace_bytes(p: DashDecodeParams) -> int:
    return int(load().dash_decode_workspace_bytes(ctypes.byref(p)))


def pool(p: DashParams, k, kbar, stream) -> None:
    check(load().dash_pool(ctypes.byref(p), k, kbar, stream))


def fwd(p: DashParams, q, k, v, o, lse, kbar, sel: DashSel, ws, ws_bytes, stream) -> None:
    check(load().dash_fwd(ctypes.byref(p), q, k, v, o, lse, kbar, ctypes.byref(sel), ws, ws_bytes, stream))


def fwd_select(p: DashParams, q, k, kbar, sel: DashSel, stream) -> None:
    check(load().dash_fwd_select(ctypes.byref(p), q, k, kbar, ctypes.byref(sel), stream))


def fwd_attend(p: DashParams, q, k, v, kbar, sel: DashSel, o, lse, stream) -> None:
    check(load().dash_fwd_attend(ctypes.byref(p), q, k, v, kbar, ctypes.byref(sel), o, lse, stream))


def fwd_lowdens_workspace_bytes(p: DashParams, max_pairs: int) -> int:
    return int(load().dash_fwd_lowdens_workspace_bytes(ctypes.byref(p), int(max_pairs)))


def fwd_attend_lowdens(p: DashParams, q, k, v, kbar, sel: DashSel, ratio, o, lse, ws, ws_bytes, stream) -> None:
    check(load().dash_fwd_attend_lowdens(ctypes.byref(p), q, k, v, kbar, ctypes.byref(sel), float(ratio), o, lse,
                                         ws, ws_bytes, stream))


def bwd(p: DashParams, q, k, v, o, lse, dout, kbar, sel: DashSel, dq, dk, dv, dkbar, ws, ws_bytes, stream) -> None:
    check(load().dash_bwd(ctypes.byref(p), q, k, v, o, lse, dout, kbar, ctypes.byref(sel), dq, dk, dv, dkbar, ws,
                          ws_bytes, stream))


def fwd_gqa(p: DashParams, kv_heads: int, q, k, v, o, lse, kbar, sel: DashSel, stream) -> None:
    check(load().dash_fwd_gqa(ctypes.byref(p), kv_heads, q, k, v, o, lse, kbar, ctypes.byref(sel), stream))


def bwd_gqa_workspace_bytes(p: DashParams, kv_heads: int) -> int:
    return int(load().dash_bwd_gqa_workspace_bytes(ctypes.byref(p), kv_heads))


def bwd_gqa(p: DashParams, kv_heads: int, q, k, v, o, lse, dout, kbar, sel: DashSel, dq, dk, dv, dkbar, ws, ws_bytes,
            stream) -> None:
    check(load().dash_bwd_gqa(ctypes.byref(p), kv_heads, q, k, v, o, lse, dout, kbar, ctypes.byref(sel), dq, dk, dv,
                              dkbar, ws, ws_bytes, stream))


def pool_attn(p: DashParams, k, w, kbar, stream) -> None:
    check(load().dash_pool_attn(ctypes.byref(p), k, w, kbar, stream))


def select(p: DashParams, q, kbar, sel: DashSel, stream) -> None:
    check(load().dash_select(ctypes.byref(p), q, kbar, ctypes.byref(sel), stream))


def bwd_no_pool(p: DashParams, q, k, v, o, lse, dout, kbar, sel: DashSel, dq, dk, dv, dkbar, ws, ws_bytes,
                stream) -> None:
    check(load().dash_bwd_no_pool(ctypes.byref(p), q, k, v, o, lse, dout, kbar, ctypes.byref(sel), dq, dk, dv, dkbar,
                                  ws, ws_bytes, stream))


def pool_attn_bwd_workspace_bytes(p: DashParams) -> int:
    return int(load().dash_pool_attn_bwd_workspace_bytes(ctypes.byref(p)))


def pool_attn_bwd(p: DashParams, k, w, dkbar, dk, dw, ws, ws_bytes, stream) -> None:
    check(load().dash_pool_attn_bwd(ctypes.byref(p), k, w, dkbar, dk, dw, ws, ws_bytes, stream))


def decode(p: DashDecodeParams, q, kc, vc, kbar, o, lse, nsel, tau, mask, ws, ws_bytes, stream) -> None:
    check(load().dash_decode(ctypes.byref(p), q, kc, vc, kbar, o, lse, nsel, tau, mask, ws, ws_bytes, stream))


def cache_append(p: DashDecodeParams, k_new, v_new, lens, kc, vc, kbar, stream) -> None:
    check(load().dash_cache_append(ctypes.byref(p), k_new, v_new, lens, kc, vc, kbar, stream))


def decode_varlen(p: DashDecodeParams, q, kc, vc, kbar, lens, o, lse, nsel, tau, mask, ws, ws_bytes,
                  stream) -> None:
    check(load().dash_decode_varlen(ctypes.byref(p), q, kc, vc, kbar, lens, o, lse, nsel, tau, mask, ws, ws_bytes,
                                    stream))


def decode_step(p: DashDecodeParams, q, k_new, v_new, lens, kc, vc, kbar, o, lse, nsel, tau, mask, ws,
                ws_bytes, stream) -> None:
    check(load().dash_decode_step(ctypes.byref(p), q, k_new, v_new, lens, kc, vc, kbar, o, lse, nsel, tau, mask,
                                  ws, ws_bytes, stream))


def decode_gqa(p: DashDecodeParams, kv_heads: int, q, kc, vc, kbar, lens, o, lse, nsel, tau, mask, ws,
               ws_bytes, stream) -> None:
    check(load().dash_decode_gqa(ctypes.byref(p), kv_heads, q, kc, vc, kbar, lens, o, lse, nsel, tau, mask, ws,
                                 ws_bytes, stream))


def decode_static_max_bytes() -> int:
    return int(load().dash_decode_static_max_bytes())


def decode_static(p: DashDecodeParams, q, kc, vc, kbar, o, lse, nsel, tau, mask, stream) -> None:
    check(load().dash_decode_static(ctypes.byref(p), q, kc, vc, kbar, o, lse, nsel, tau, mask, stream))


def bwd_learned_workspace_bytes(p: DashParams) -> int:
    return int(load().dash_bwd_learned_workspace_bytes(ctypes.byref(p)))


def bwd_learned(p: DashParams, q, k, v, o, lse, dout, kbar, sel: DashSel, w, dq, dk, dv, dkbar, dw, ws, ws_bytes,
                stream) -> None:
    check(load().dash_bwd_learned(ctypes.byref(p), q, k, v, o, lse, dout, kbar, ctypes.byref(sel), w, dq, dk, dv,
                                  dkbar, dw, ws, ws_bytes, stream))
