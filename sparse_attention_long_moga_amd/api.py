"""Torch-facing binding of libmoga.so.

Argument marshalling only: each function checks device, dtype, shape and
contiguity, allocates outputs (and a workspace unless one is passed) with
torch, and calls the C entry point of the same name on the current HIP stream.
Every step of the computation runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _capi
from ._capi import MogaDims, MogaGrads, MogaInputs, MogaOutputs, MogaSaved, StgaLayout, check

__all__ = ["make_dims", "make_stga_layout", "moga_workspace_bytes", "workspace", "moga_route",
           "moga_permute", "moga_unpermute", "moga_group_attn", "moga_group_attn_noalloc",
           "stga_group_attn",
           "moga_balance_loss", "moga_forward", "moga_forward_fused", "moga_backward",
           "moga_hybrid_backward", "moga_attention", "MoGALayer"]


def _lib():
    return _capi.load()


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_dims(n_tokens: int, d_model: int, n_heads: int, head_dim: int, n_groups: int,
              alpha: float = 0.1, softmax_scale: float = 0.0) -> MogaDims:
    return MogaDims(n_tokens, d_model, n_heads, head_dim, n_groups, softmax_scale, alpha)


class _Layout:
    """An stga_layout plus the host array it points into (kept alive here)."""

    def __init__(self, frames, height, width, shot_start: Sequence[int], win_h, win_w, t_group,
                 aug_frames):
        self.shots = (ctypes.c_int32 * len(shot_start))(*[int(s) for s in shot_start])
        self.c = StgaLayout(frames, height, width, len(shot_start) - 1,
                            ctypes.cast(self.shots, ctypes.POINTER(ctypes.c_int32)), win_h, win_w,
                            t_group, aug_frames)

    def ref(self):
        return ctypes.byref(self.c)


def make_stga_layout(frames: int, height: int, width: int, shot_start: Sequence[int], win_h: int,
                     win_w: int, t_group: int, aug_frames: int) -> _Layout:
    return _Layout(frames, height, width, shot_start, win_h, win_w, t_group, aug_frames)


def moga_workspace_bytes(dims: MogaDims, stga: Optional[_Layout] = None) -> int:
    n = _lib().moga_workspace_bytes(ctypes.byref(dims), stga.ref() if stga else None)
    if n == 0:
        check(_capi.MOGA_ERR_ARG)
    return int(n)


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _ws(ws: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    if ws is None:
        return workspace(nbytes, device)
    _need(ws, "ws", torch.uint8)
    return ws


def moga_route(x: torch.Tensor, w: torch.Tensor, n_groups: int, pin: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None) -> dict:
    """Router: group_id [N] int32, p_sel [N] f32, counts [M] int32, prob_sum [M] f64."""
    _need(x, "x", ndim=2)
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    n, d = x.shape
    _need(w, "w", torch.float32, 2, x.device)
    if tuple(w.shape) != (d, n_groups):
        raise ValueError(f"w must be [{d}, {n_groups}]")
    if pin is not None:
        _need(pin, "pin", torch.int32, 1, x.device)
    dims = make_dims(n, d, 1, 64, n_groups)
    dev = x.device
    out = dict(group_id=torch.empty(n, dtype=torch.int32, device=dev),
               p_sel=torch.empty(n, dtype=torch.float32, device=dev),
               counts=torch.empty(n_groups, dtype=torch.int32, device=dev),
               prob_sum=torch.empty(n_groups, dtype=torch.float64, device=dev))
    nb = moga_workspace_bytes(dims)
    ws = _ws(ws, nb, dev)
    check(_lib().moga_route(_ptr(x), _capi.MOGA_BF16 if x.dtype == torch.bfloat16 else _capi.MOGA_F32,
                            _ptr(w), _ptr(pin), ctypes.byref(dims), _ptr(out["group_id"]),
                            _ptr(out["p_sel"]), _ptr(out["counts"]), _ptr(out["prob_sum"]),
                            _ptr(ws), ws.numel(), _stream()))
    return out


def _heads_shape(ts: Sequence[torch.Tensor]):
    h, n, hd = ts[0].shape
    for i, t in enumerate(ts):
        _need(t, f"tensor {i}", torch.bfloat16, 3, ts[0].device)
        if tuple(t.shape) != (h, n, hd):
            raise ValueError("all tensors must share one [H, N, head_dim] shape")
    return h, n, hd


def moga_permute(group_id: torch.Tensor, tensors: Sequence[torch.Tensor], n_groups: int,
                 p_sel: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Stable permute into groups: returns (cu_seqlens, perm, permuted tensors, p_perm)."""
    _need(group_id, "group_id", torch.int32, 1)
    n = group_id.shape[0]
    dev = group_id.device
    if tensors:
        h, nn, hd = _heads_shape(tensors)
        if nn != n:
            raise ValueError("tensors must have N rows per head")
    else:
        h, hd = 1, 64
    dims = make_dims(n, 1, h, hd, n_groups)
    cu = torch.empty(n_groups + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    outs = [torch.empty_like(t) for t in tensors]
    p_perm = None
    if p_sel is not None:
        _need(p_sel, "p_sel", torch.float32, 1, dev)
        p_perm = torch.empty_like(p_sel)
    src = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in tensors])
    dst = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in outs])
    ws = _ws(ws, moga_workspace_bytes(dims), dev)
    check(_lib().moga_permute(0, _ptr(group_id), ctypes.byref(dims), _ptr(cu), _ptr(perm), src, dst,
                              len(tensors), _ptr(p_sel), _ptr(p_perm), _ptr(ws), ws.numel(),
                              _stream()))
    return cu, perm, outs, p_perm


def moga_unpermute(perm: torch.Tensor, tensors: Sequence[torch.Tensor], n_groups: int = 1,
                   ws: Optional[torch.Tensor] = None):
    """Inverse permute: out[h][perm[j]] = t[h][j] for each tensor."""
    _need(perm, "perm", torch.int32, 1)
    h, n, hd = _heads_shape(tensors)
    dims = make_dims(n, 1, h, hd, n_groups)
    outs = [torch.empty_like(t) for t in tensors]
    src = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in tensors])
    dst = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in outs])
    ws = _ws(ws, moga_workspace_bytes(dims), perm.device)
    check(_lib().moga_permute(1, None, ctypes.byref(dims), None, _ptr(perm), src, dst, len(tensors),
                              None, None, _ptr(ws), ws.numel(), _stream()))
    return outs


def _group_attn_args(q, k, v, cu_q, cu_k, row_scale, out):
    _need(q, "q", torch.bfloat16, 3)
    h, lq, hd = q.shape
    _need(k, "k", torch.bfloat16, 3, q.device)
    _need(v, "v", torch.bfloat16, 3, q.device)
    if k.shape != v.shape or k.shape[0] != h or k.shape[2] != hd:
        raise ValueError("k and v must be [H, Lk, head_dim] matching q")
    _need(cu_q, "cu_q", torch.int32, 1, q.device)
    _need(cu_k, "cu_k", torch.int32, 1, q.device)
    if cu_q.shape != cu_k.shape:
        raise ValueError("cu_q and cu_k must have the same length")
    if row_scale is not None:
        _need(row_scale, "row_scale", torch.float32, 1, q.device)
        if row_scale.shape[0] != lq:
            raise ValueError("row_scale must have len_q entries")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 3, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    return h, lq, hd, k.shape[1], cu_q.shape[0] - 1, out


def moga_group_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_q: torch.Tensor,
                    cu_k: torch.Tensor, row_scale: Optional[torch.Tensor] = None,
                    softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Varlen group attention: q [H, Lq, hd], k/v [H, Lk, hd] bf16; cu_q/cu_k int32 [S+1]."""
    h, lq, hd, lk, n_seg, out = _group_attn_args(q, k, v, cu_q, cu_k, row_scale, out)
    dims = make_dims(max(lq, 1), 1, h, hd, 1, softmax_scale=softmax_scale)
    nb = _lib().moga_group_attn_workspace_bytes(ctypes.byref(dims), n_seg, lq)
    if nb == 0:
        check(_capi.MOGA_ERR_ARG)
    ws = _ws(ws, nb, q.device)
    check(_lib().moga_group_attn(_ptr(q), _ptr(k), _ptr(v), lq, lk, n_seg, _ptr(cu_q), _ptr(cu_k),
                                 _ptr(row_scale), ctypes.byref(dims), _ptr(out), _ptr(ws),
                                 ws.numel(), _stream()))
    return out


def moga_group_attn_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            cu_q: torch.Tensor, cu_k: torch.Tensor,
                            row_scale: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moga_group_attn with the library's static scratch instead of a workspace (pass `out`
    to allocate nothing at all).  Calls that overlap on one device race."""
    h, lq, hd, lk, n_seg, out = _group_attn_args(q, k, v, cu_q, cu_k, row_scale, out)
    dims = make_dims(max(lq, 1), 1, h, hd, 1, softmax_scale=softmax_scale)
    check(_lib().moga_group_attn_noalloc(_ptr(q), _ptr(k), _ptr(v), lq, lk, n_seg, _ptr(cu_q),
                                         _ptr(cu_k), _ptr(row_scale), ctypes.byref(dims),
                                         _ptr(out), _stream()))
    return out


def stga_group_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: _Layout,
                    temporal: bool = True, frame: bool = True, softmax_scale: float = 0.0,
                    ws: Optional[torch.Tensor] = None):
    """STGA branches in token order: returns (o_temporal or None, o_frame or None)."""
    h, n, hd = _heads_shape([q, k, v])
    dims = make_dims(n, 1, h, hd, 1, softmax_scale=softmax_scale)
    o_t = torch.empty_like(q) if temporal else None
    o_f = torch.empty_like(q) if frame else None
    ws = _ws(ws, moga_workspace_bytes(dims, layout), q.device)
    check(_lib().stga_group_attn(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(dims), layout.ref(),
                                 _ptr(o_t), _ptr(o_f), _ptr(ws), ws.numel(), _stream()))
    return o_t, o_f


def moga_balance_loss(counts: torch.Tensor, prob_sum: torch.Tensor, n_tokens: int,
                      alpha: float = 0.1):
    """L_gb with F and P: returns (loss [1] f64, F [M] f64, P [M] f64) on the device."""
    _need(counts, "counts", torch.int32, 1)
    _need(prob_sum, "prob_sum", torch.float64, 1, counts.device)
    m = counts.shape[0]
    dims = make_dims(n_tokens, 1, 1, 64, m, alpha=alpha)
    dev = counts.device
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    F = torch.empty(m, dtype=torch.float64, device=dev)
    P = torch.empty(m, dtype=torch.float64, device=dev)
    check(_lib().moga_balance_loss(_ptr(counts), _ptr(prob_sum), ctypes.byref(dims), _ptr(loss),
                                   _ptr(F), _ptr(P), _stream()))
    return loss, F, P


def moga_forward(x: torch.Tensor, w: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                 v: torch.Tensor, n_groups: int, alpha: float = 0.1,
                 pin: Optional[torch.Tensor] = None, stga: Optional[_Layout] = None,
                 softmax_scale: float = 0.0, ws: Optional[torch.Tensor] = None,
                 out: Optional[dict] = None, fused: bool = False, with_lse: bool = False) -> dict:
    """Whole forward.  Returns a dict with out, loss and the routing tensors
    (group_id, p_sel, cu_seqlens, perm, counts, prob_sum), plus lse ([H, N] f32, what
    moga_backward needs) when with_lse is set; with a STGA layout with_lse returns the
    three branches' state moga_hybrid_backward needs instead: lse [3, H, N] and o_branches
    [3, H, N, head_dim] (MoGA row scaled by p, temporal row, per-frame row).  Pass `out` (a
    dict of preallocated tensors with those keys) and `ws` to run without allocating.
    fused=True calls moga_forward_fused (rows read through perm inside the attention kernel;
    bitwise identical results)."""
    _need(x, "x", ndim=2)
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    n, d = x.shape
    _need(w, "w", torch.float32, 2, x.device)
    h, nn, hd = _heads_shape([q, k, v])
    if nn != n or tuple(w.shape) != (d, n_groups):
        raise ValueError("shape mismatch between x, w and q/k/v")
    if pin is not None:
        _need(pin, "pin", torch.int32, 1, x.device)
    dims = make_dims(n, d, h, hd, n_groups, alpha=alpha, softmax_scale=softmax_scale)
    dev = x.device
    if out is None:
        out = dict(out=torch.empty_like(q), loss=torch.empty(1, dtype=torch.float64, device=dev),
                   group_id=torch.empty(n, dtype=torch.int32, device=dev),
                   p_sel=torch.empty(n, dtype=torch.float32, device=dev),
                   cu_seqlens=torch.empty(n_groups + 1, dtype=torch.int32, device=dev),
                   perm=torch.empty(n, dtype=torch.int32, device=dev),
                   counts=torch.empty(n_groups, dtype=torch.int32, device=dev),
                   prob_sum=torch.empty(n_groups, dtype=torch.float64, device=dev))
        if with_lse and stga is not None:
            out["lse"] = torch.empty(3, h, n, dtype=torch.float32, device=dev)
            out["o_branches"] = torch.empty((3,) + tuple(q.shape), dtype=q.dtype, device=dev)
        elif with_lse:
            out["lse"] = torch.empty(h, n, dtype=torch.float32, device=dev)
    ws = _ws(ws, moga_workspace_bytes(dims, stga), dev)
    ins = MogaInputs(x.data_ptr(), _capi.MOGA_BF16 if x.dtype == torch.bfloat16 else _capi.MOGA_F32,
                     w.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                     pin.data_ptr() if pin is not None else None)
    g = lambda key: out[key].data_ptr() if out.get(key) is not None else None
    outs = MogaOutputs(g("out"), g("loss"), g("group_id"), g("p_sel"), g("cu_seqlens"), g("perm"),
                       g("counts"), g("prob_sum"), g("lse"), g("o_branches"))
    fn = _lib().moga_forward_fused if fused else _lib().moga_forward
    check(fn(ctypes.byref(ins), ctypes.byref(dims), stga.ref() if stga else None,
             ctypes.byref(outs), _ptr(ws), ws.numel(), _stream()))
    return out


def moga_forward_fused(*args, **kwargs) -> dict:
    """moga_forward with the permutation applied inside the attention kernel."""
    return moga_forward(*args, fused=True, **kwargs)


def _backward(x, w, q, k, v, saved, d_out, d_loss, alpha, softmax_scale, ws, grads, stga):
    _need(x, "x", ndim=2)
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    n, d = x.shape
    _need(w, "w", torch.float32, 2, x.device)
    m = w.shape[1]
    h, nn, hd = _heads_shape([q, k, v, d_out])
    if nn != n or w.shape[0] != d:
        raise ValueError("shape mismatch between x, w and q/k/v")
    hybrid = stga is not None
    out_key = "o_branches" if hybrid else "out"
    lse_shape = (3, h, n) if hybrid else (h, n)
    for key, dt, shape in (("group_id", torch.int32, (n,)), ("p_sel", torch.float32, (n,)),
                           ("counts", torch.int32, (m,)), ("cu_seqlens", torch.int32, (m + 1,)),
                           ("perm", torch.int32, (n,)), ("lse", torch.float32, lse_shape),
                           (out_key, q.dtype, ((3,) if hybrid else ()) + tuple(q.shape))):
        if saved.get(key) is None:
            raise ValueError(f"saved['{key}'] is missing (run moga_forward with with_lse=True"
                             + (" and this stga layout)" if hybrid else ")"))
        _need(saved[key], f"saved['{key}']", dt, len(shape), x.device)
        if tuple(saved[key].shape) != shape:
            raise ValueError(f"saved['{key}'] must be {shape}")
    dims = make_dims(n, d, h, hd, m, alpha=alpha, softmax_scale=softmax_scale)
    dev = x.device
    if grads is None:
        grads = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                     dx=torch.empty(n, d, dtype=torch.float32, device=dev),
                     dw=torch.empty(d, m, dtype=torch.float32, device=dev),
                     dp=torch.empty(n, dtype=torch.float32, device=dev))
    if hybrid:
        nb = _lib().moga_hybrid_backward_workspace_bytes(ctypes.byref(dims), stga.ref())
    else:
        nb = _lib().moga_backward_workspace_bytes(ctypes.byref(dims))
    if nb == 0:
        check(_capi.MOGA_ERR_ARG)
    ws = _ws(ws, nb, dev)
    ins = MogaInputs(x.data_ptr(), _capi.MOGA_BF16 if x.dtype == torch.bfloat16 else _capi.MOGA_F32,
                     w.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), None)
    sv = lambda key: saved[key].data_ptr()
    sav = MogaSaved(sv("group_id"), sv("p_sel"), sv("counts"), sv("cu_seqlens"), sv("perm"),
                    sv(out_key), sv("lse"))
    g = lambda key: grads[key].data_ptr() if grads.get(key) is not None else None
    gr = MogaGrads(g("dq"), g("dk"), g("dv"), g("dx"), g("dw"), g("dp"))
    if hybrid:
        check(_lib().moga_hybrid_backward(ctypes.byref(ins), ctypes.byref(sav), stga.ref(),
                                          _ptr(d_out), float(d_loss), ctypes.byref(dims),
                                          ctypes.byref(gr), _ptr(ws), ws.numel(), _stream()))
    else:
        check(_lib().moga_backward(ctypes.byref(ins), ctypes.byref(sav), _ptr(d_out),
                                   float(d_loss), ctypes.byref(dims), ctypes.byref(gr), _ptr(ws),
                                   ws.numel(), _stream()))
    return grads


def moga_backward(x: torch.Tensor, w: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                  v: torch.Tensor, saved: dict, d_out: torch.Tensor, d_loss: float = 0.0,
                  alpha: float = 0.1, softmax_scale: float = 0.0,
                  ws: Optional[torch.Tensor] = None, grads: Optional[dict] = None) -> dict:
    """Gradients of moga_forward (stga None, routing held fixed).  saved: the dict
    moga_forward returned with with_lse=True; d_out: bf16 [H, N, head_dim], the gradient
    with respect to out; d_loss: the gradient with respect to the balance loss.  Returns
    dq, dk, dv (bf16, like q), dx ([N, d] f32), dw ([d, M] f32) and dp ([N] f32)."""
    return _backward(x, w, q, k, v, saved, d_out, d_loss, alpha, softmax_scale, ws, grads, None)


def moga_hybrid_backward(x: torch.Tensor, w: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                         v: torch.Tensor, saved: dict, d_out: torch.Tensor, stga: _Layout,
                         d_loss: float = 0.0, alpha: float = 0.1, softmax_scale: float = 0.0,
                         ws: Optional[torch.Tensor] = None, grads: Optional[dict] = None) -> dict:
    """Gradients of the hybrid forward (moga_forward with this stga layout, routing held
    fixed): out is the mean of the MoGA, temporal and per-frame rows.  saved: the dict
    moga_forward returned with with_lse=True and stga (o_branches and the [3, H, N] lse);
    otherwise as moga_backward."""
    if stga is None:
        raise ValueError("moga_hybrid_backward needs the forward's stga layout")
    return _backward(x, w, q, k, v, saved, d_out, d_loss, alpha, softmax_scale, ws, grads, stga)


_SAVED_KEYS = ("group_id", "p_sel", "counts", "cu_seqlens", "perm", "lse")


class _MogaAttention(torch.autograd.Function):
    """The layer as one autograd node: moga_forward (with the state its backward needs) on the
    way in, moga_backward or moga_hybrid_backward on the way out."""

    @staticmethod
    def forward(ctx, x, w, q, k, v, n_groups, alpha, stga, softmax_scale, pin, fused):
        fwd = moga_forward(x, w, q, k, v, n_groups, alpha=alpha, pin=pin, stga=stga,
                           softmax_scale=softmax_scale, fused=fused, with_lse=True)
        rows = fwd["o_branches"] if stga is not None else fwd["out"]
        ctx.save_for_backward(x, w, q, k, v, rows, *(fwd[key] for key in _SAVED_KEYS))
        ctx.stga, ctx.alpha, ctx.softmax_scale = stga, alpha, softmax_scale
        return fwd["out"], fwd["loss"].view(())

    @staticmethod
    def backward(ctx, g_out, g_loss):
        x, w, q, k, v, rows, *state = ctx.saved_tensors
        saved = dict(zip(_SAVED_KEYS, state))
        saved["o_branches" if ctx.stga is not None else "out"] = rows
        d_out = torch.zeros_like(q) if g_out is None else g_out.to(q.dtype).contiguous()
        # the loss's gradient enters the library as a host scalar (one device synchronisation)
        d_loss = 0.0 if g_loss is None else float(g_loss)
        grads = _backward(x, w, q, k, v, saved, d_out, d_loss, ctx.alpha, ctx.softmax_scale,
                          None, None, ctx.stga)
        return (grads["dx"].to(x.dtype), grads["dw"], grads["dq"], grads["dk"], grads["dv"],
                None, None, None, None, None, None)


def moga_attention(x: torch.Tensor, w: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                   v: torch.Tensor, n_groups: int, alpha: float = 0.1,
                   stga: Optional[_Layout] = None, softmax_scale: float = 0.0,
                   pin: Optional[torch.Tensor] = None, fused: bool = True):
    """Differentiable MoGA layer (the hybrid MoGA + STGA mean with a layout): returns out
    ([H, N, head_dim] bf16, token order) and the balance loss (fp64 scalar), both tracked by
    autograd.  The backward is moga_backward / moga_hybrid_backward with the routing held
    fixed: gradients reach x and w through p(g|x) and the loss, and q, k, v through the
    attention; none flows through the group choice."""
    return _MogaAttention.apply(x, w, q, k, v, n_groups, alpha, stga, softmax_scale, pin, fused)


class MoGALayer(torch.nn.Module):
    """The MoGA attention layer as a module (the drop-in layer of the xugj520.cn blog on MoGA,
    §8): it owns the router weight W [d_model, n_groups] (fp32, the group centres the router
    scores tokens against) and, with a STGA layout, forms the mean with the two static
    branches.  forward(x, q, k, v) returns (out, balance loss)
    through moga_attention; the Q/K/V projections and the output projection stay with the
    caller's model."""

    def __init__(self, d_model: int, n_groups: int, alpha: float = 0.1,
                 stga: Optional[_Layout] = None, softmax_scale: float = 0.0, device=None):
        super().__init__()
        self.n_groups, self.alpha, self.stga, self.softmax_scale = n_groups, alpha, stga, softmax_scale
        self.weight = torch.nn.Parameter(
            torch.empty(d_model, n_groups, dtype=torch.float32, device=device))
        torch.nn.init.normal_(self.weight, std=d_model ** -0.5)

    def forward(self, x: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                pin: Optional[torch.Tensor] = None):
        return moga_attention(x, self.weight, q, k, v, self.n_groups, alpha=self.alpha,
                              stga=self.stga, softmax_scale=self.softmax_scale, pin=pin)
