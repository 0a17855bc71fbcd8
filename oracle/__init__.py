"""CPU oracle for the MoGA + STGA forward path (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and the library never calls it.

Two independent implementations live here:

* ``moga_oracle.c`` (this module's ctypes wrapper): the plain, per-row
  definitions in fp64 with OpenMP over rows.  This is the oracle the GPU path
  is compared with.
* ``bruteforce.py``: dense N x N masks built from predicates and NumPy
  matrix products, for tiny inputs only.  It pins the C oracle.

Every function cites the page and section it follows (see the header of
``moga_oracle.c`` for the citation keys).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moga_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (OpenMP, -O2)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    c_i64, c_int, c_dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    vp = ctypes.c_void_p
    lib.oracle_route.argtypes = [_f32p, _f32p, c_i64, c_int, c_int, vp, _i32p, _f64p, _f64p,
                                 _f64p, _i64p, vp]
    lib.oracle_route.restype = c_int
    lib.oracle_groups.argtypes = [_i32p, c_i64, c_int, _i64p, _i64p]
    lib.oracle_groups.restype = c_int
    lib.oracle_balance_loss.argtypes = [_i64p, _f64p, c_i64, c_int, c_dbl, _f64p, _f64p]
    lib.oracle_balance_loss.restype = c_dbl
    lib.oracle_moga_attn.argtypes = [_f32p, _f32p, _f32p, c_i64, c_int, _i32p, c_int, vp, c_dbl,
                                     c_i64, _i32p, _i64p, _f64p]
    lib.oracle_moga_attn.restype = c_i64
    lib.oracle_stga_attn.argtypes = [_f32p, _f32p, _f32p, c_int, c_int, c_int, c_int, c_int,
                                     _i32p, c_int, c_int, c_int, c_int, c_int, c_dbl, c_i64,
                                     _i32p, _i64p, _f64p]
    lib.oracle_stga_attn.restype = c_i64
    lib.oracle_stga_pairs.argtypes = [c_int, c_int, c_int, c_int, _i32p, c_int, c_int, c_int,
                                      c_int, c_int]
    lib.oracle_stga_pairs.restype = c_i64
    lib.oracle_stga_key_list.argtypes = [c_int, c_int, c_int, c_int, _i32p, c_int, c_int, c_int,
                                         c_int, c_int, c_i64, _i64p]
    lib.oracle_stga_key_list.restype = c_i64
    lib.oracle_varlen_attn.argtypes = [_f32p, _f32p, _f32p, c_i64, c_i64, c_int, c_int, _i64p,
                                       _i64p, vp, c_dbl, c_i64, _i32p, _i64p, _f64p]
    lib.oracle_varlen_attn.restype = c_i64
    lib.oracle_moga_backward.argtypes = [_f32p, _f32p, c_i64, c_int, c_int, c_int, c_int, _f32p,
                                         _f32p, _f32p, _i32p, _f32p, c_dbl, c_dbl, c_dbl, _f64p,
                                         _f64p, _f64p, _f64p, _f64p, _f64p, _f64p]
    lib.oracle_moga_backward.restype = c_int
    lib.oracle_moga_dq_rows.argtypes = [_f32p, _f32p, _f32p, _f32p, c_i64, c_int, _i32p, c_int,
                                        _f64p, c_dbl, c_i64, _i32p, _i64p, _f64p, _f64p, _f64p]
    lib.oracle_moga_dq_rows.restype = c_int
    lib.oracle_moga_dkdv_rows.argtypes = [_f32p, _f32p, _f32p, _f32p, c_i64, c_int, _i32p, c_int,
                                          _f64p, c_dbl, c_i64, _i32p, _i64p, _f64p, _f64p]
    lib.oracle_moga_dkdv_rows.restype = c_int
    lib.oracle_stga_backward.argtypes = [_f32p, _f32p, _f32p, _f32p, c_int, c_int, c_int, c_int,
                                         c_int, c_int, _i32p, c_int, c_int, c_int, c_int, c_int,
                                         c_dbl, _f64p, _f64p, _f64p, _f64p]
    lib.oracle_stga_backward.restype = c_int
    lib.oracle_stga_bwd_rows.argtypes = [_f32p, _f32p, _f32p, _f32p, c_int, c_int, c_int, c_int,
                                         c_int, _i32p, c_int, c_int, c_int, c_int, c_int, c_dbl,
                                         c_i64, _i32p, _i64p, _f64p, _f64p, _f64p, _f64p]
    lib.oracle_stga_bwd_rows.restype = c_int
    lib.oracle_router_bwd_rows.argtypes = [_f32p, _f32p, c_i64, c_int, c_int, _i32p, _f64p,
                                           _i64p, c_i64, c_dbl, c_dbl, _f64p, _f64p]
    lib.oracle_router_bwd_rows.restype = c_int
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor (bf16 upcasts exactly)
        a = a.detach().float().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# Router, groups, loss (papernotes.org MoGA note, 关键设计 1-3)
# --------------------------------------------------------------------------
def route(x, w, pin=None, want_probs: bool = False) -> dict:
    """r = x W, p = softmax(r), g = argmax (first max; pins override), p_sel = p[g].

    Returns group_id (int32), p_sel (f64), gap = top-1 minus top-2 logit (f64),
    prob_sum = sum_t p(i|x_t) (f64 [M]), counts (int64 [M]) and optionally the
    full probability matrix.
    """
    x, w = _f32(x), _f32(w)
    n, d = x.shape
    m = w.shape[1]
    assert w.shape[0] == d
    pin_a = None if pin is None else np.ascontiguousarray(pin, dtype=np.int32)
    out = dict(group_id=np.empty(n, np.int32), p_sel=np.empty(n), gap=np.empty(n),
               prob_sum=np.empty(m), counts=np.empty(m, np.int64))
    probs = np.empty((n, m)) if want_probs else None
    rc = _load().oracle_route(x, w, n, d, m, _ptr(pin_a), out["group_id"], out["p_sel"],
                              out["gap"], out["prob_sum"], out["counts"], _ptr(probs))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc})")
    if want_probs:
        out["probs"] = probs
    return out


def near_tie_pins(r: dict, threshold: float = 1e-5) -> np.ndarray:
    """Pin list for tokens whose top-2 logit gap is below `threshold`: -1 = free,
    else the oracle's own choice."""
    pin = np.full(r["group_id"].shape, -1, np.int32)
    tie = r["gap"] < threshold
    pin[tie] = r["group_id"][tie]
    return pin


def groups(group_id, m: int):
    """cu_seqlens [M+1] and the stable permutation (grouped row -> token)."""
    g = np.ascontiguousarray(group_id, dtype=np.int32)
    n = g.shape[0]
    cu = np.empty(m + 1, np.int64)
    perm = np.empty(n, np.int64)
    rc = _load().oracle_groups(g, n, m, cu, perm)
    if rc != 0:
        raise ValueError(f"oracle_groups failed ({rc})")
    return cu, perm


def balance_loss(counts, prob_sum, n: int, alpha: float):
    """L_gb = alpha * M * sum_i F_i P_i with F_i = n_i/N, P_i = prob_sum_i/N."""
    c = np.ascontiguousarray(counts, dtype=np.int64)
    ps = np.ascontiguousarray(prob_sum, dtype=np.float64)
    m = c.shape[0]
    F, P = np.empty(m), np.empty(m)
    loss = _load().oracle_balance_loss(c, ps, n, m, float(alpha), F, P)
    return loss, F, P


# --------------------------------------------------------------------------
# Attention rows
# --------------------------------------------------------------------------
def _rows(rows_h, rows_t):
    rh = np.ascontiguousarray(rows_h, dtype=np.int32)
    rt = np.ascontiguousarray(rows_t, dtype=np.int64)
    assert rh.shape == rt.shape
    return rh, rt


def moga_attn(q, k, v, group_id, m: int, p_sel, scale: float, rows_h, rows_t):
    """MoGA output rows p(g|x) * SA(q_t, K_g, V_g) in fp64.

    q, k, v: [Hs][N][hd] (rows_h indexes the Hs heads given).  p_sel None -> no
    scale.  Returns (out [rows][hd] f64, pair count).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    _, n, hd = q.shape
    g = np.ascontiguousarray(group_id, dtype=np.int32)
    ps = None if p_sel is None else np.ascontiguousarray(p_sel, dtype=np.float64)
    rh, rt = _rows(rows_h, rows_t)
    out = np.empty((rh.shape[0], hd))
    pairs = _load().oracle_moga_attn(q, k, v, n, hd, g, m, _ptr(ps), float(scale), rh.shape[0],
                                     rh, rt, out)
    if pairs < 0:
        raise ValueError("oracle_moga_attn failed")
    return out, int(pairs)


def moga_backward(x, w, q, k, v, group_id, d_out, d_loss: float, alpha: float,
                  scale: float) -> dict:
    """Gradients of the MoGA forward (papernotes.org MoGA note, 关键设计 1 and 3) with the
    routing held fixed: given d_out for out = p(g|x) * SA(q, K_g, V_g) and d_loss for L_gb,
    returns dq, dk, dv ([H][N][hd]), dx ([N][d]), dw ([d][M]), dp ([N], gradient with respect
    to p(g_t|x_t) from the attention output) and lse ([H][N]) in fp64."""
    x, w = _f32(x), _f32(w)
    q, k, v, go = _f32(q), _f32(k), _f32(v), _f32(d_out)
    h, n, hd = q.shape
    d, m = w.shape
    g = np.ascontiguousarray(group_id, dtype=np.int32)
    out = dict(dq=np.empty((h, n, hd)), dk=np.empty((h, n, hd)), dv=np.empty((h, n, hd)),
               dx=np.empty((n, d)), dw=np.empty((d, m)), dp=np.empty(n), lse=np.empty((h, n)))
    rc = _load().oracle_moga_backward(x, w, n, d, m, h, hd, q, k, v, g, go, float(d_loss),
                                      float(alpha), float(scale), out["dq"], out["dk"],
                                      out["dv"], out["dx"], out["dw"], out["dp"], out["lse"])
    if rc != 0:
        raise ValueError(f"oracle_moga_backward failed ({rc})")
    return out


def moga_dq_rows(q, k, v, d_out, group_id, m: int, p_sel, scale: float, rows_h, rows_t):
    """dq, D = <dO', O'> and lse of selected (head, token) rows, same definitions as
    moga_backward.  Returns (dq [rows][hd], D [rows], lse [rows])."""
    q, k, v, go = _f32(q), _f32(k), _f32(v), _f32(d_out)
    _, n, hd = q.shape
    g = np.ascontiguousarray(group_id, dtype=np.int32)
    ps = np.ascontiguousarray(p_sel, dtype=np.float64)
    rh, rt = _rows(rows_h, rows_t)
    dq, D, lse = np.empty((rh.shape[0], hd)), np.empty(rh.shape[0]), np.empty(rh.shape[0])
    rc = _load().oracle_moga_dq_rows(q, k, v, go, n, hd, g, m, ps, float(scale), rh.shape[0],
                                     rh, rt, dq, D, lse)
    if rc != 0:
        raise ValueError(f"oracle_moga_dq_rows failed ({rc})")
    return dq, D, lse


def moga_dkdv_rows(q, k, v, d_out, group_id, m: int, p_sel, scale: float, rows_h, rows_t):
    """dk and dv of selected (head, key token) rows, same definitions as moga_backward (each
    needs the softmax rows of every query of the key's group).  Returns (dk, dv), each
    [rows][hd]."""
    q, k, v, go = _f32(q), _f32(k), _f32(v), _f32(d_out)
    _, n, hd = q.shape
    g = np.ascontiguousarray(group_id, dtype=np.int32)
    ps = np.ascontiguousarray(p_sel, dtype=np.float64)
    rh, rt = _rows(rows_h, rows_t)
    dk, dv = np.empty((rh.shape[0], hd)), np.empty((rh.shape[0], hd))
    rc = _load().oracle_moga_dkdv_rows(q, k, v, go, n, hd, g, m, ps, float(scale), rh.shape[0],
                                       rh, rt, dk, dv)
    if rc != 0:
        raise ValueError(f"oracle_moga_dkdv_rows failed ({rc})")
    return dk, dv


def router_backward_rows(x_rows, w, group_rows, dp_rows, counts, n: int, d_loss: float,
                         alpha: float):
    """Router part of moga_backward for selected tokens: given their x rows, groups and
    dp_t, and the whole problem's counts and N, returns (dr [rows][M], dx [rows][d])."""
    x, w = _f32(x_rows), _f32(w)
    r, d = x.shape
    m = w.shape[1]
    g = np.ascontiguousarray(group_rows, dtype=np.int32)
    dp = np.ascontiguousarray(dp_rows, dtype=np.float64)
    c = np.ascontiguousarray(counts, dtype=np.int64)
    dr, dx = np.empty((r, m)), np.empty((r, d))
    rc = _load().oracle_router_bwd_rows(x, w, r, d, m, g, dp, c, int(n), float(d_loss),
                                        float(alpha), dr, dx)
    if rc != 0:
        raise ValueError(f"oracle_router_bwd_rows failed ({rc})")
    return dr, dx


def varlen_attn(q, k, v, cu_q, cu_k, scale: float, rows_h, rows_i, row_scale=None):
    """Segment attention: q row i of segment s attends to key rows [cu_k[s], cu_k[s+1]).

    q: [Hs][Lq][hd], k/v: [Hs][Lk][hd].  Returns (out [rows][hd] f64, pair count).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    _, lq, hd = q.shape
    lk = k.shape[1]
    cq = np.ascontiguousarray(cu_q, dtype=np.int64)
    ck = np.ascontiguousarray(cu_k, dtype=np.int64)
    rs = None if row_scale is None else np.ascontiguousarray(row_scale, dtype=np.float64)
    rh, ri = _rows(rows_h, rows_i)
    out = np.empty((rh.shape[0], hd))
    pairs = _load().oracle_varlen_attn(q, k, v, lq, lk, hd, cq.shape[0] - 1, cq, ck, _ptr(rs),
                                       float(scale), rh.shape[0], rh, ri, out)
    if pairs < 0:
        raise ValueError("oracle_varlen_attn: bad segments")
    return out, int(pairs)


def _grid_args(grid: dict):
    ss = np.ascontiguousarray(grid["shot_start"], dtype=np.int32)
    return (int(grid["frames"]), int(grid["height"]), int(grid["width"]), ss.shape[0] - 1, ss,
            int(grid["win_h"]), int(grid["win_w"]), int(grid["t_group"]),
            int(grid["aug_frames"]))


def stga_attn(q, k, v, grid: dict, mode: str, scale: float, rows_h, rows_t):
    """STGA output rows, mode 'temporal' or 'frame'.  Returns (out, pairs)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    hd = q.shape[2]
    rh, rt = _rows(rows_h, rows_t)
    out = np.empty((rh.shape[0], hd))
    f, hh, ww, ns, ss, wh, wws, tg, aug = _grid_args(grid)
    pairs = _load().oracle_stga_attn(q, k, v, hd, f, hh, ww, ns, ss, wh, wws, tg, aug,
                                     {"temporal": 0, "frame": 1}[mode], float(scale),
                                     rh.shape[0], rh, rt, out)
    if pairs < 0:
        raise ValueError("oracle_stga_attn failed (bad geometry)")
    return out, int(pairs)


def stga_backward(q, k, v, d_out, grid: dict, mode: str, scale: float) -> dict:
    """Gradients of sum <d_out, O> for one STGA branch ('temporal' or 'frame') on whole tensors
    [H][N][hd]: dq, dk, dv (dk, dv add over every query whose key set holds the key) and lse."""
    q, k, v, go = _f32(q), _f32(k), _f32(v), _f32(d_out)
    h, n, hd = q.shape
    f, hh, ww, ns, ss, wh, wws, tg, aug = _grid_args(grid)
    out = {name: np.empty((h, n, hd)) for name in ("dq", "dk", "dv")}
    out["lse"] = np.empty((h, n))
    rc = _load().oracle_stga_backward(q, k, v, go, h, hd, f, hh, ww, ns, ss, wh, wws, tg, aug,
                                      {"temporal": 0, "frame": 1}[mode], float(scale),
                                      out["dq"], out["dk"], out["dv"], out["lse"])
    if rc != 0:
        raise ValueError(f"oracle_stga_backward failed ({rc})")
    return out


def stga_bwd_rows(q, k, v, d_out, grid: dict, mode: str, scale: float, rows_h, rows_t):
    """stga_backward's dq and lse (the token as a query) and dk, dv (as a key) of selected
    (head, token) rows.  Returns (dq, dk, dv, lse)."""
    q, k, v, go = _f32(q), _f32(k), _f32(v), _f32(d_out)
    hd = q.shape[2]
    rh, rt = _rows(rows_h, rows_t)
    f, hh, ww, ns, ss, wh, wws, tg, aug = _grid_args(grid)
    r = rh.shape[0]
    dq, dk, dv, lse = np.empty((r, hd)), np.empty((r, hd)), np.empty((r, hd)), np.empty(r)
    rc = _load().oracle_stga_bwd_rows(q, k, v, go, hd, f, hh, ww, ns, ss, wh, wws, tg, aug,
                                      {"temporal": 0, "frame": 1}[mode], float(scale), r, rh, rt,
                                      dq, dk, dv, lse)
    if rc != 0:
        raise ValueError(f"oracle_stga_bwd_rows failed ({rc})")
    return dq, dk, dv, lse


def hybrid_backward(x, w, q, k, v, group_id, grid: dict, d_out, d_loss: float, alpha: float,
                    scale: float) -> dict:
    """Gradients of <d_out, out> + d_loss * L_gb for the hybrid layer out = (O_moga + O_temporal
    + O_frame) / 3 (papernotes.org MoGA note, 关键设计 4: each token takes the mean of its three
    outputs), routing held fixed: each branch receives d_out / 3, the MoGA branch's gradients
    (router included) come from moga_backward, and dq, dk, dv add over the three branches."""
    # every gradient is linear in d_out, and the loss term does not depend on it: the
    # d_out / 3 share is formed by dividing gradients in fp64 (d_out itself stays exact)
    att = moga_backward(x, w, q, k, v, group_id, d_out, 0.0, alpha, scale)
    los = moga_backward(x, w, q, k, v, group_id, np.zeros_like(_f32(d_out)), d_loss, alpha,
                        scale)
    out = {name: att[name] / 3.0 + los[name] for name in ("dq", "dk", "dv", "dx", "dw", "dp")}
    out["lse"] = att["lse"]
    for mode in ("temporal", "frame"):
        st = stga_backward(q, k, v, d_out, grid, mode, scale)
        for name in ("dq", "dk", "dv"):
            out[name] = out[name] + st[name] / 3.0
        out["lse_" + mode] = st["lse"]
    return out


def stga_pairs(grid: dict, mode: str) -> int:
    f, hh, ww, ns, ss, wh, wws, tg, aug = _grid_args(grid)
    r = _load().oracle_stga_pairs(f, hh, ww, ns, ss, wh, wws, tg, aug,
                                  {"temporal": 0, "frame": 1}[mode])
    if r < 0:
        raise ValueError("bad geometry")
    return int(r)


def stga_key_list(grid: dict, mode: str, t: int) -> np.ndarray:
    f, hh, ww, ns, ss, wh, wws, tg, aug = _grid_args(grid)
    buf = np.empty(hh * ww * (tg + 2 * aug) + hh * ww, np.int64)
    nk = _load().oracle_stga_key_list(f, hh, ww, ns, ss, wh, wws, tg, aug,
                                      {"temporal": 0, "frame": 1}[mode], int(t), buf)
    if nk < 0:
        raise ValueError("bad geometry")
    return buf[:nk].copy()


def grid_of(wl) -> dict:
    """STGA geometry dict of a workloads.Workload."""
    return dict(frames=wl.frames, height=wl.height, width=wl.width,
                shot_start=list(wl.shot_start), win_h=wl.win_h, win_w=wl.win_w,
                t_group=wl.t_group, aug_frames=wl.aug_frames)
