"""PyTorch-facing entry points of the DashAttention hot path.

PyTorch provides device memory and the current HIP stream; every step of the
method runs in libdash.so (see include/dash.h).  Tensors must live on a ROCm
device; there is no CPU fallback.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import _lib

BLOCK = 64
QTILE = 128  # query rows per Stage-2 tile (dash_query_tile())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.DASH_BF16
    if t.dtype == torch.float32:
        return _lib.DASH_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(t: torch.Tensor, name: str, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def make_params(q: torch.Tensor, alpha: float, causal: bool, fine_scale=None, coarse_scale=None):
    B, H, T, D = q.shape
    p = _lib.DashParams()
    p.B, p.H, p.T, p.D, p.block = B, H, T, D, BLOCK
    p.alpha = float(alpha)
    p.causal = int(bool(causal))
    p.fine_scale = float(fine_scale if fine_scale is not None else 1.0 / math.sqrt(D))
    p.coarse_scale = float(coarse_scale if coarse_scale is not None else 1.0 / math.sqrt(D))
    p.dtype = _dtype_code(q)
    return p


@dataclass
class Selection:
    """Stage-1 outputs (device tensors), see dash_sel in include/dash.h."""
    tau: torch.Tensor
    lognorm: torch.Tensor
    nsel: torch.Tensor | None
    mask: torch.Tensor | None
    tile_cnt: torch.Tensor
    tile_blk: torch.Tensor
    tile_bits: torch.Tensor
    passes: torch.Tensor | None = None

    def as_c(self) -> _lib.DashSel:
        s = _lib.DashSel()
        s.tau, s.lognorm = _ptr(self.tau), _ptr(self.lognorm)
        s.nsel, s.mask = _ptr(self.nsel), _ptr(self.mask)
        s.tile_cnt, s.tile_blk, s.tile_bits = _ptr(self.tile_cnt), _ptr(self.tile_blk), _ptr(self.tile_bits)
        s.passes = _ptr(self.passes)
        return s


def alloc_selection(p: _lib.DashParams, device, want_mask: bool = True) -> Selection:
    n = _lib.sel_sizes(p)
    B, H = p.B, p.H
    T = -(-p.T // BLOCK) * BLOCK  # rows laid out as whole blocks
    nb = T // BLOCK
    nbw = (nb + 31) // 32
    ntile = n[4] // (B * H)
    e = lambda m, dt: torch.empty(m, dtype=dt, device=device)  # noqa: E731
    return Selection(
        tau=e(n[0], torch.float32).view(B, H, T),
        lognorm=e(n[1], torch.float32).view(B, H, T),
        nsel=e(n[2], torch.int32).view(B, H, T) if want_mask else None,
        # the library writes 32-bit words; torch has no uint32 arithmetic, so int32 storage
        mask=e(n[3], torch.int32).view(B, H, T, nbw) if want_mask else None,
        tile_cnt=e(n[4], torch.int32).view(B, H, ntile),
        tile_blk=e(n[5], torch.int32).view(B, H, ntile, nb),
        tile_bits=e(n[6], torch.int32).view(B, H, ntile, nbw),
        passes=e(n[7], torch.int32).view(B, H, T) if want_mask else None,
    )


def pool(k: torch.Tensor) -> torch.Tensor:
    """Stage 0: block summaries kbar [B,H,T/64,D] of k [B,H,T,D]."""
    _require(k, "k")
    p = make_params(k, 1.5, True)
    kbar = torch.empty((p.B, p.H, p.T // BLOCK, p.D), dtype=k.dtype, device=k.device)
    _lib.pool(p, _ptr(k), _ptr(kbar), _stream(k.device))
    return kbar


def pool_attn(k: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """Stage 0 with the learned summariser: kbar [B,H,T/64,D] of k [B,H,T,D], head vectors w [H,D] (f32)."""
    _require(k, "k")
    p = make_params(k, 1.5, True)
    _require(w, "w", (p.H, p.D), torch.float32)
    kbar = torch.empty((p.B, p.H, p.T // BLOCK, p.D), dtype=k.dtype, device=k.device)
    _lib.pool_attn(p, _ptr(k), _ptr(w), _ptr(kbar), _stream(k.device))
    return kbar


LOWDENS_RATIO = 4.0  # DASH_LOWDENS_RATIO of include/dash.h


def lowdens_pairs(sel: Selection, p: _lib.DashParams, ratio: float = LOWDENS_RATIO) -> int:
    """(row, block) pairs of the query tiles that take the low-density Stage-2 schedule
    (dash_fwd_attend_lowdens): a tile qualifies when its block-list length x rows exceeds
    ratio x the sum over its rows of (selected blocks + 1).  Needs sel.nsel; reads one
    number back from the device."""
    if sel.nsel is None:
        raise ValueError("the low-density schedule needs the selection counts (want_mask=True)")
    B, H, T = sel.nsel.shape
    ntile = sel.tile_cnt.shape[-1]
    per_row = sel.nsel.to(torch.int64) + 1
    per_row = torch.nn.functional.pad(per_row, (0, ntile * QTILE - T))
    tile_pairs = per_row.view(B, H, ntile, QTILE).sum(-1)
    rows = torch.clamp(T - QTILE * torch.arange(ntile, device=per_row.device), max=QTILE)
    walked = sel.tile_cnt.to(torch.int64) * rows
    take = walked.double() > ratio * tile_pairs.double()
    return int(tile_pairs[take].sum())


def forward(q, k, v, alpha=1.5, causal=True, fine_scale=None, coarse_scale=None, want_mask=True,
            summariser_w=None, low_density=False, ratio=LOWDENS_RATIO):
    """Stages 0-2.  Returns dict(o, lse, kbar, sel, params).

    ``summariser_w`` ([H, D] f32) switches Stage 0 to the learned summariser;
    None is mean pooling.  k and v may have fewer heads than q (grouped-query
    heads with entmax head aggregation, bf16): then kbar has k's heads.

    ``low_density`` lets query tiles whose rows select few blocks take the
    block-stationary Stage-2 schedule (causal bf16 prefill with whole blocks and
    one KV head per query head; other cases ignore it): the selection is made
    first, the pairs of the qualifying tiles are counted (``lowdens_pairs``, one
    read-back) and the workspace is sized for them."""
    _require(q, "q")
    B, H, T, D = q.shape
    Hkv = k.shape[1] if k.dim() == 4 else -1
    for name, t in (("k", k), ("v", v)):
        _require(t, name, (B, Hkv, T, D), q.dtype)
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"k has {Hkv} heads, which must divide q's {H}")
    if Hkv != H and summariser_w is not None:
        raise ValueError("the learned summariser is built for one KV head per query head")
    p = make_params(q, alpha, causal, fine_scale, coarse_scale)
    if summariser_w is not None:
        _require(summariser_w, "summariser_w", (p.H, p.D), torch.float32)
    use_ld = bool(low_density) and q.dtype == torch.bfloat16 and causal and T % BLOCK == 0 and Hkv == H
    if use_ld:
        want_mask = True  # the schedule's lists come from the masks
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((p.B, p.H, p.T), dtype=torch.float32, device=dev)
    kbar = torch.empty((p.B, Hkv, -(-p.T // BLOCK), p.D), dtype=q.dtype, device=dev)
    sel = alloc_selection(p, dev, want_mask)
    wsb = _lib.fwd_workspace_bytes(p)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    csel = sel.as_c()
    if use_ld:
        if summariser_w is None:
            _lib.fwd_select(p, _ptr(q), _ptr(k), _ptr(kbar), csel, _stream(dev))
        else:
            _lib.pool_attn(p, _ptr(k), _ptr(summariser_w), _ptr(kbar), _stream(dev))
            _lib.select(p, _ptr(q), _ptr(kbar), csel, _stream(dev))
        npairs = lowdens_pairs(sel, p, ratio)
        wsb = _lib.fwd_lowdens_workspace_bytes(p, npairs)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        _lib.fwd_attend_lowdens(p, _ptr(q), _ptr(k), _ptr(v), _ptr(kbar), csel, ratio, _ptr(o), _ptr(lse),
                                _ptr(ws), wsb, _stream(dev))
        return dict(o=o, lse=lse, kbar=kbar, sel=sel, params=p, lowdens_pairs=npairs)
    if Hkv != H:
        _lib.fwd_gqa(p, Hkv, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(kbar), csel, _stream(dev))
    elif summariser_w is None:
        _lib.fwd(p, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(kbar), csel, _ptr(ws), wsb, _stream(dev))
    else:
        _lib.pool_attn(p, _ptr(k), _ptr(summariser_w), _ptr(kbar), _stream(dev))
        _lib.select(p, _ptr(q), _ptr(kbar), csel, _stream(dev))
        _lib.fwd_attend(p, _ptr(q), _ptr(k), _ptr(v), _ptr(kbar), csel, _ptr(o), _ptr(lse), _stream(dev))
    return dict(o=o, lse=lse, kbar=kbar, sel=sel, params=p)


def backward(q, k, v, o, lse, dout, kbar, sel: Selection, p: _lib.DashParams, summariser_w=None):
    """Gradients of <dout, O>: dict(dq, dk, dv, dkbar), plus dw [H,D] with the learned summariser.
    With fewer KV heads than query heads, dk, dv and dkbar have k's heads."""
    _require(dout, "dout", q.shape, q.dtype)
    dev = q.device
    Hkv = k.shape[1]
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dkbar = torch.empty((p.B, Hkv, -(-p.T // BLOCK), p.D), dtype=torch.float32, device=dev)
    if Hkv != p.H:
        wsb = _lib.bwd_gqa_workspace_bytes(p, Hkv)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        _lib.bwd_gqa(p, Hkv, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(kbar), sel.as_c(),
                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dkbar), _ptr(ws), wsb, _stream(dev))
        return dict(dq=dq, dk=dk, dv=dv, dkbar=dkbar)
    if summariser_w is None:
        wsb = _lib.bwd_workspace_bytes(p)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        _lib.bwd(p, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(kbar), sel.as_c(), _ptr(dq),
                 _ptr(dk), _ptr(dv), _ptr(dkbar), _ptr(ws), wsb, _stream(dev))
        return dict(dq=dq, dk=dk, dv=dv, dkbar=dkbar)
    _require(summariser_w, "summariser_w", (p.H, p.D), torch.float32)
    dw = torch.empty((p.H, p.D), dtype=torch.float32, device=dev)
    wsb = _lib.bwd_learned_workspace_bytes(p)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _lib.bwd_learned(p, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(kbar), sel.as_c(),
                     _ptr(summariser_w), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dkbar), _ptr(dw), _ptr(ws), wsb,
                     _stream(dev))
    return dict(dq=dq, dk=dk, dv=dv, dkbar=dkbar, dw=dw)


def make_decode_params(q, kc, alpha, fine_scale=None, coarse_scale=None):
    S, H, N, D = kc.shape
    p = _lib.DashDecodeParams()
    p.S, p.H, p.N, p.D, p.block = S, H, N, D, BLOCK
    p.alpha = float(alpha)
    p.fine_scale = float(fine_scale if fine_scale is not None else 1.0 / math.sqrt(D))
    p.coarse_scale = float(coarse_scale if coarse_scale is not None else 1.0 / math.sqrt(D))
    p.dtype = _dtype_code(q)
    return p


class DecodeBuffers:
    """Outputs and workspace of one decode step, allocated once and reused."""

    def __init__(self, p: _lib.DashDecodeParams, dtype, device):
        self.o = torch.empty((p.S, p.H, p.D), dtype=dtype, device=device)
        self.lse = torch.empty((p.S, p.H), dtype=torch.float32, device=device)
        self.nsel = torch.empty((p.S, p.H), dtype=torch.int32, device=device)
        self.tau = torch.empty((p.S, p.H), dtype=torch.float32, device=device)
        # selected candidate blocks of each row as 32-bit words (int32 storage)
        self.mask = torch.empty((p.S, p.H, (p.N // BLOCK + 31) // 32), dtype=torch.int32, device=device)
        self.ws_bytes = _lib.decode_workspace_bytes(p)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)


def decode(q, kc, vc, kbar, alpha=1.5, fine_scale=None, coarse_scale=None, bufs: DecodeBuffers | None = None):
    """One decode step: q [S,H,D] against caches kc, vc [S,H,N,D] and summaries kbar."""
    S, H, N, D = kc.shape
    _require(q, "q", (S, H, D), kc.dtype)
    _require(vc, "vc", kc.shape, kc.dtype)
    _require(kbar, "kbar", (S, H, N // BLOCK, D), kc.dtype)
    p = make_decode_params(q, kc, alpha, fine_scale, coarse_scale)
    if bufs is None:
        bufs = DecodeBuffers(p, q.dtype, q.device)
    _lib.decode(p, _ptr(q), _ptr(kc), _ptr(vc), _ptr(kbar), _ptr(bufs.o), _ptr(bufs.lse), _ptr(bufs.nsel),
                _ptr(bufs.tau), _ptr(bufs.mask), _ptr(bufs.ws), bufs.ws_bytes, _stream(q.device))
    return dict(o=bufs.o, lse=bufs.lse, nsel=bufs.nsel, tau=bufs.tau, mask=bufs.mask)


def _require_lens(lens, S, device):
    if not (isinstance(lens, torch.Tensor) and lens.dtype == torch.int32 and lens.shape == (S,)
            and lens.device == device and lens.is_contiguous()):
        raise ValueError(f"lens must be a contiguous int32 tensor of shape ({S},) on {device}")


def cache_append(kc, vc, kbar, lens, k_new, v_new):
    """Write k_new, v_new [S,H,D] at position lens[s] of caches kc, vc [S,H,C,D]
    and, for blocks the token completes, their summaries in kbar.  lens is not advanced."""
    S, H, C, D = kc.shape
    _require(vc, "vc", kc.shape, kc.dtype)
    _require(kbar, "kbar", (S, H, C // BLOCK, D), kc.dtype)
    _require(k_new, "k_new", (S, H, D), kc.dtype)
    _require(v_new, "v_new", (S, H, D), kc.dtype)
    _require_lens(lens, S, kc.device)
    p = make_decode_params(k_new, kc, 1.5)
    _lib.cache_append(p, _ptr(k_new), _ptr(v_new), _ptr(lens), _ptr(kc), _ptr(vc), _ptr(kbar), _stream(kc.device))


def decode_varlen(q, kc, vc, kbar, lens, alpha=1.5, fine_scale=None, coarse_scale=None,
                  bufs: DecodeBuffers | None = None):
    """Decode with lens[s] tokens cached for sequence s (the new one last) in caches of capacity C."""
    S, H, C, D = kc.shape
    _require(q, "q", (S, H, D), kc.dtype)
    _require(vc, "vc", kc.shape, kc.dtype)
    _require(kbar, "kbar", (S, H, C // BLOCK, D), kc.dtype)
    _require_lens(lens, S, q.device)
    p = make_decode_params(q, kc, alpha, fine_scale, coarse_scale)
    if bufs is None:
        bufs = DecodeBuffers(p, q.dtype, q.device)
    _lib.decode_varlen(p, _ptr(q), _ptr(kc), _ptr(vc), _ptr(kbar), _ptr(lens), _ptr(bufs.o), _ptr(bufs.lse),
                       _ptr(bufs.nsel), _ptr(bufs.tau), _ptr(bufs.mask), _ptr(bufs.ws), bufs.ws_bytes, _stream(q.device))
    return dict(o=bufs.o, lse=bufs.lse, nsel=bufs.nsel, tau=bufs.tau, mask=bufs.mask)


def decode_step(q, k_new, v_new, kc, vc, kbar, lens, alpha=1.5, fine_scale=None, coarse_scale=None,
                bufs: DecodeBuffers | None = None):
    """Append (k_new, v_new) at lens[s], then decode over lens[s] + 1 tokens.  lens is not advanced."""
    S, H, C, D = kc.shape
    _require(q, "q", (S, H, D), kc.dtype)
    _require(k_new, "k_new", (S, H, D), kc.dtype)
    _require(v_new, "v_new", (S, H, D), kc.dtype)
    _require(vc, "vc", kc.shape, kc.dtype)
    _require(kbar, "kbar", (S, H, C // BLOCK, D), kc.dtype)
    _require_lens(lens, S, q.device)
    p = make_decode_params(q, kc, alpha, fine_scale, coarse_scale)
    if bufs is None:
        bufs = DecodeBuffers(p, q.dtype, q.device)
    _lib.decode_step(p, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(lens), _ptr(kc), _ptr(vc), _ptr(kbar),
                     _ptr(bufs.o), _ptr(bufs.lse), _ptr(bufs.nsel), _ptr(bufs.tau), _ptr(bufs.mask), _ptr(bufs.ws),
                     bufs.ws_bytes, _stream(q.device))
    return dict(o=bufs.o, lse=bufs.lse, nsel=bufs.nsel, tau=bufs.tau, mask=bufs.mask)


def decode_gqa(q, kc, vc, kbar, lens=None, alpha=1.5, fine_scale=None, coarse_scale=None,
               bufs: DecodeBuffers | None = None):
    """Decode for grouped-query heads: q [S,H,D] over caches kc, vc [S,Hkv,C,D] (Hkv divides H);
    lens: None (full caches) or int32 [S] device lengths."""
    S, Hkv, C, D = kc.shape
    H = q.shape[1]
    _require(q, "q", (S, H, D), kc.dtype)
    _require(vc, "vc", kc.shape, kc.dtype)
    _require(kbar, "kbar", (S, Hkv, C // BLOCK, D), kc.dtype)
    if lens is not None:
        _require_lens(lens, S, q.device)
    p = make_decode_params(q, kc, alpha, fine_scale, coarse_scale)
    p.H = H
    if bufs is None:
        bufs = DecodeBuffers(p, q.dtype, q.device)
    _lib.decode_gqa(p, Hkv, _ptr(q), _ptr(kc), _ptr(vc), _ptr(kbar), None if lens is None else _ptr(lens),
                    _ptr(bufs.o), _ptr(bufs.lse), _ptr(bufs.nsel), _ptr(bufs.tau), _ptr(bufs.mask), _ptr(bufs.ws),
                    bufs.ws_bytes, _stream(q.device))
    return dict(o=bufs.o, lse=bufs.lse, nsel=bufs.nsel, tau=bufs.tau, mask=bufs.mask)


class DashAttentionFn(torch.autograd.Function):
    """DashAttention as an autograd function (forward: Stages 0-2; backward through all of them)."""

    @staticmethod
    def forward(ctx, q, k, v, alpha, causal, fine_scale, coarse_scale, summariser_w=None):
        r = forward(q, k, v, alpha, causal, fine_scale, coarse_scale, want_mask=False, summariser_w=summariser_w)
        ctx.save_for_backward(q, k, v, r["o"], r["lse"], r["kbar"])
        ctx.w = summariser_w
        ctx.sel = r["sel"]
        ctx.p = r["params"]
        return r["o"]

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse, kbar = ctx.saved_tensors
        g = backward(q, k, v, o, lse, dout.contiguous(), kbar, ctx.sel, ctx.p, summariser_w=ctx.w)
        return g["dq"], g["dk"], g["dv"], None, None, None, None, g.get("dw")


def dash_attention(q, k, v, alpha=1.5, causal=True, fine_scale=None, coarse_scale=None, summariser_w=None):
    """DashAttention with autograd; ``summariser_w`` ([H, D] f32, a leaf that may require grad)
    selects the learned Stage-0 summariser."""
    return DashAttentionFn.apply(q, k, v, alpha, causal, fine_scale, coarse_scale, summariser_w)
