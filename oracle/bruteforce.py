"""Dense brute force for tiny inputs (TEST INFRASTRUCTURE).

A second, independent formulation of what the C oracle computes: every
grouping is written as a dense N x N boolean predicate on per-token attributes
and attention is a masked softmax over full matrix products in fp64.  It pins
the list-based C oracle on small cases.  Only tests import it.

Citations: papernotes.org MoGA note, 关键设计 1 (router, group attention) and
4 (STGA); xugj520.cn MoGA blog §2.3 (router form), §3.2 (two boundary frames
from each neighbouring shot, keys/values only).
"""
from __future__ import annotations

import numpy as np


def router(x, w):
    """logits = x W; p = softmax(logits); g = first argmax of p."""
    logits = np.asarray(x, np.float64) @ np.asarray(w, np.float64)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    return logits, p, np.argmax(p, axis=1)


def masked_attention(q, k, v, mask, scale):
    """softmax(scale Q K^T restricted to mask) V for one head, fp64, dense."""
    s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(s), 0.0)
    return (e / e.sum(axis=1, keepdims=True)) @ np.asarray(v, np.float64)


def moga_mask(group_id):
    g = np.asarray(group_id)
    return g[:, None] == g[None, :]


def token_attrs(grid):
    """Per-token (frame, y, x, window-y, window-x, shot, chunk) for a frame-major grid."""
    f_all, hh, ww = grid["frames"], grid["height"], grid["width"]
    t = np.arange(f_all * hh * ww)
    f = t // (hh * ww)
    y = (t % (hh * ww)) // ww
    x = t % ww
    starts = np.asarray(grid["shot_start"])
    shot = np.searchsorted(starts, f, side="right") - 1
    chunk = (f - starts[shot]) // grid["t_group"]
    return dict(f=f, wy=y // grid["win_h"], wx=x // grid["win_w"], shot=shot, chunk=chunk)


def stga_mask(grid, mode):
    """Dense key predicate for STGA: mode 'frame' or 'temporal'."""
    a = token_attrs(grid)
    if mode == "frame":
        return a["f"][:, None] == a["f"][None, :]
    starts = np.asarray(grid["shot_start"])
    n_shots = len(starts) - 1
    lengths = np.diff(starts)
    last_chunk = (lengths - 1) // grid["t_group"]
    aug = grid["aug_frames"]
    T = lambda k: a[k][:, None]  # query attribute as a column
    U = lambda k: a[k][None, :]  # key attribute as a row
    same_win = (T("wy") == U("wy")) & (T("wx") == U("wx"))
    own = same_win & (T("shot") == U("shot")) & (T("chunk") == U("chunk"))
    s_t = a["shot"][:, None]
    first_of_shot = (T("chunk") == 0) & (s_t > 0)
    prev = (same_win & first_of_shot & (U("shot") == s_t - 1)
            & (U("f") >= starts[s_t] - aug))
    last_of_shot = (T("chunk") == last_chunk[a["shot"]][:, None]) & (s_t < n_shots - 1)
    nxt = (same_win & last_of_shot & (U("shot") == s_t + 1)
           & (U("f") < starts[np.minimum(s_t + 1, n_shots)] + aug))
    return own | prev | nxt


def moga_forward(x, w, q, k, v, scale, stga_grid=None):
    """Whole forward on tiny inputs: MoGA output, or the mean of MoGA and both
    STGA branches.  q, k, v: [H][N][hd]."""
    _, p, g = router(x, w)
    p_sel = p[np.arange(len(g)), g]
    mm = moga_mask(g)
    out = np.stack([p_sel[:, None] * masked_attention(q[h], k[h], v[h], mm, scale)
                    for h in range(q.shape[0])])
    if stga_grid is None:
        return out, g, p
    mt, mf = stga_mask(stga_grid, "temporal"), stga_mask(stga_grid, "frame")
    ot = np.stack([masked_attention(q[h], k[h], v[h], mt, scale) for h in range(q.shape[0])])
    of = np.stack([masked_attention(q[h], k[h], v[h], mf, scale) for h in range(q.shape[0])])
    return (out + ot + of) / 3.0, g, p
