"""Parity of the hybrid forward's saved state (o_branches, the three lse planes) and of
moga_hybrid_backward with the CPU oracle.

The hybrid layer's output is the mean of the MoGA, temporal-window and per-frame rows; its
gradient gives each branch a third of d_out, and a key row that a temporal group borrows from
the adjacent shot passes its dK, dV back to the token it came from.  Small cases compare every
element with oracle.hybrid_backward (geometries with ragged chunks, a shot shorter than the
borrowed frames and a single shot without borrowing).  The full-size case (the 30 s hybrid
workload) compares sampled rows the oracle computes one by one: dq of tokens of every group and
of the frames on either side of each shot cut, dk and dv of tokens of the two smallest groups
(the MoGA part needs the softmax of every query of the key's group), including tokens in the
borrowed frames, whose temporal dK, dV add over every group that holds them.

The floating-point bar is the one the MoGA backward tests use (bf16 operands, fp32
accumulation, results rounded to bf16 once per branch and once more after the sum)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from sparse_attention_long_moga_amd import api
from tests.helpers import assert_close_bf16, host
from tests.test_gpu_backward import LSE_ABS, assert_grad_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

GEOMS = {
    # 5-, 4- and 3-frame shots in chunks of 3 (ragged last chunks), two borrowed frames
    "ragged_chunks": dict(frames=12, height=8, width=16, shot_start=[0, 5, 9, 12], win_h=4,
                          win_w=8, t_group=3, aug_frames=2, heads=2, m=4, seed=61),
    # a one-frame shot: both neighbours borrow fewer frames than aug_frames
    "short_shot": dict(frames=10, height=4, width=16, shot_start=[0, 1, 4, 10], win_h=4,
                       win_w=8, t_group=2, aug_frames=2, heads=2, m=5, seed=62),
    # one shot, nothing borrowed; temporal groups of a whole frame window
    "one_shot": dict(frames=6, height=8, width=8, shot_start=[0, 6], win_h=8, win_w=8,
                     t_group=4, aug_frames=0, heads=1, m=3, seed=63),
    # head_dim 64 (rows widened to the 128-channel kernels), three shots
    "hd64": dict(frames=9, height=6, width=8, shot_start=[0, 4, 7, 9], win_h=3, win_w=4,
                 t_group=2, aug_frames=2, heads=2, m=4, seed=64, hd=64),
}


def _announce(what, **kw):
    print(f"[case] {what} {kw}", flush=True)


def _setup(geom):
    c = dict(geom)
    h, m, seed, hd = c.pop("heads"), c.pop("m"), c.pop("seed"), c.pop("hd", 128)
    n = c["frames"] * c["height"] * c["width"]
    wl = workloads.small(f"hyb_{n}_{m}", n, 256, h, hd, m, seed=seed)
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    q, k, v = workloads.make_qkv(wl, DEV)
    dout = workloads.make_dout(wl, DEV)
    return wl, c, x, w, q, k, v, dout


@pytest.mark.parametrize("name", sorted(GEOMS))
def test_hybrid_backward_parity(name):
    _announce("hybrid backward", name=name)
    wl, grid, x, w, q, k, v, dout = _setup(GEOMS[name])
    n, m, hd = wl.n_tokens, wl.n_groups, wl.head_dim
    scale = 1.0 / math.sqrt(hd)
    r = oracle.route(host(x), host(w))
    pin = torch.from_numpy(oracle.near_tie_pins(r)).to(DEV)
    lay = api.make_stga_layout(**grid)
    d_loss = 0.7
    fwd = api.moga_forward(x, w, q, k, v, m, alpha=wl.alpha, pin=pin, stga=lay, fused=True,
                           with_lse=True)
    explicit = api.moga_forward(x, w, q, k, v, m, alpha=wl.alpha, pin=pin, stga=lay,
                                with_lse=True)
    plain = api.moga_forward(x, w, q, k, v, m, alpha=wl.alpha, pin=pin, stga=lay)
    grads = api.moga_hybrid_backward(x, w, q, k, v, fwd, dout, lay, d_loss=d_loss,
                                     alpha=wl.alpha)
    again = api.moga_hybrid_backward(x, w, q, k, v, fwd, dout, lay, d_loss=d_loss,
                                     alpha=wl.alpha)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(fwd["group_id"]), r["group_id"])
    # saving the branches does not change out, both forward variants save the same state, and
    # the backward is reproducible
    assert torch.equal(fwd["out"], plain["out"])
    for key in ("out", "o_branches", "lse"):
        assert torch.equal(fwd[key], explicit[key]), key
    for key in grads:
        assert torch.equal(grads[key], again[key]), key

    # forward state: each branch's rows and normaliser
    h = q.shape[0]
    rows_h, rows_t = np.repeat(np.arange(h), n), np.tile(np.arange(n), h)
    qh, kh, vh, gh = host(q), host(k), host(v), host(dout)
    ob = host(fwd["o_branches"]).reshape(3, -1, hd)
    ref_m, _ = oracle.moga_attn(qh, kh, vh, r["group_id"], m, r["p_sel"], scale, rows_h, rows_t)
    assert_close_bf16(ob[0], ref_m, f"{name} MoGA branch rows")
    for i, mode in ((1, "temporal"), (2, "frame")):
        ref, _ = oracle.stga_attn(qh, kh, vh, grid, mode, scale, rows_h, rows_t)
        assert_close_bf16(ob[i], ref, f"{name} {mode} branch rows")

    ref = oracle.hybrid_backward(host(x), host(w), qh, kh, vh, r["group_id"], grid, gh, d_loss,
                                 wl.alpha, scale)
    lse = host(fwd["lse"])
    for i, key in ((0, "lse"), (1, "lse_temporal"), (2, "lse_frame")):
        err = np.abs(lse[i] - ref[key]).max()
        assert err <= LSE_ABS, f"{name} {key} error {err:.3e}"
    for key in ("dq", "dk", "dv", "dp", "dx", "dw"):
        assert_grad_close(host(grads[key]), ref[key], f"{name} {key}")


def test_hybrid_backward_loss_only():
    """d_out = 0: nothing reaches q, k, v or p (bitwise zero); dx and dW are the balance
    loss's alone."""
    _announce("hybrid backward loss only")
    wl, grid, x, w, q, k, v, _ = _setup(GEOMS["ragged_chunks"])
    dout = torch.zeros_like(q)
    r = oracle.route(host(x), host(w))
    pin = torch.from_numpy(oracle.near_tie_pins(r)).to(DEV)
    lay = api.make_stga_layout(**grid)
    fwd = api.moga_forward(x, w, q, k, v, wl.n_groups, alpha=wl.alpha, pin=pin, stga=lay,
                           with_lse=True)
    grads = api.moga_hybrid_backward(x, w, q, k, v, fwd, dout, lay, d_loss=1.0, alpha=wl.alpha)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dp"):
        assert torch.count_nonzero(grads[key]) == 0, key
    ref = oracle.moga_backward(host(x), host(w), host(q), host(k), host(v), r["group_id"],
                               host(dout), 1.0, wl.alpha, 1.0 / math.sqrt(128))
    assert_grad_close(host(grads["dx"]), ref["dx"], "loss-only dx", rrms=1e-4, rmax=1e-3)
    assert_grad_close(host(grads["dw"]), ref["dw"], "loss-only dw", rrms=1e-4, rmax=1e-3)


def test_full_size_hybrid_backward():
    wl = workloads.WAN30S_HYBRID
    _announce("full-size hybrid backward", name=wl.name)
    n, m, hd, nh = wl.n_tokens, wl.n_groups, wl.head_dim, wl.n_heads
    grid = oracle.grid_of(wl)
    lay = api.make_stga_layout(**grid)
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    q, k, v = workloads.make_qkv(wl, DEV)
    dout = workloads.make_dout(wl, DEV)
    xh, wh = host(x), host(w)
    r = oracle.route(xh, wh)
    pin = torch.from_numpy(oracle.near_tie_pins(r)).to(DEV)
    d_loss = 0.8
    fwd = api.moga_forward(x, w, q, k, v, m, alpha=wl.alpha, pin=pin, stga=lay, fused=True,
                           with_lse=True)
    grads = api.moga_hybrid_backward(x, w, q, k, v, fwd, dout, lay, d_loss=d_loss,
                                     alpha=wl.alpha)
    torch.cuda.synchronize()
    del x
    g = r["group_id"]
    np.testing.assert_array_equal(host(fwd["group_id"]), g)
    scale = 1.0 / math.sqrt(hd)
    hw = wl.height * wl.width
    rng = np.random.Generator(np.random.PCG64(wl.seed + 93))
    cut_frames = sorted({f for s in wl.shot_start[1:-1] for f in range(s - 2, s + 2)})
    in_cut = np.isin(np.arange(n) // hw, cut_frames)

    # dq rows: tokens of every group and of the frames around every cut, first and last head
    toks = [rng.choice(np.flatnonzero(g == gi), size=min(8, int(np.sum(g == gi))), replace=False)
            for gi in range(m) if np.any(g == gi)]
    toks.append(rng.choice(np.flatnonzero(in_cut), size=48, replace=False))
    t = np.unique(np.concatenate(toks))
    heads = np.array([0, nh - 1])
    rows_h = np.repeat(heads, t.size).astype(np.int32)
    rows_t = np.tile(t, heads.size).astype(np.int64)
    qh, kh, vh, gh = (np.stack([host(a[i]) for i in heads]) for a in (q, k, v, dout))
    rh_local = np.repeat(np.arange(heads.size), t.size).astype(np.int32)
    dq_m, D_m, lse_m = oracle.moga_dq_rows(qh, kh, vh, gh, g, m, r["p_sel"], scale, rh_local,
                                           rows_t)
    dq_t, _, _, lse_t = oracle.stga_bwd_rows(qh, kh, vh, gh, grid, "temporal", scale, rh_local,
                                             rows_t)
    dq_f, _, _, lse_f = oracle.stga_bwd_rows(qh, kh, vh, gh, grid, "frame", scale, rh_local,
                                             rows_t)
    hi = torch.from_numpy(rows_h.astype(np.int64)).to(DEV)
    ti = torch.from_numpy(rows_t).to(DEV)
    assert_grad_close(host(grads["dq"][hi, ti]), (dq_m + dq_t + dq_f) / 3.0, "30 s hybrid dq rows")
    for i, want in enumerate((lse_m, lse_t, lse_f)):
        err = np.abs(host(fwd["lse"][i][hi, ti]) - want).max()
        assert err <= LSE_ABS, f"lse plane {i} error {err:.3e}"

    # dk, dv rows: tokens of the two smallest groups, half of them in the borrowed frames
    sizes = np.bincount(g, minlength=m)
    small = [int(i) for i in np.argsort(sizes) if sizes[i] > 0][:2]
    kt = []
    for gi in small:
        mem = np.flatnonzero(g == gi)
        cut = mem[in_cut[mem]]
        kt.append(rng.choice(mem, size=min(6, mem.size), replace=False))
        if cut.size:
            kt.append(rng.choice(cut, size=min(6, cut.size), replace=False))
    kt = np.unique(np.concatenate(kt))
    krows_h = np.repeat(np.arange(heads.size), kt.size).astype(np.int32)
    krows_t = np.tile(kt, heads.size).astype(np.int64)
    dk_m, dv_m = oracle.moga_dkdv_rows(qh, kh, vh, gh, g, m, r["p_sel"], scale, krows_h, krows_t)
    _, dk_t, dv_t, _ = oracle.stga_bwd_rows(qh, kh, vh, gh, grid, "temporal", scale, krows_h,
                                            krows_t)
    _, dk_f, dv_f, _ = oracle.stga_bwd_rows(qh, kh, vh, gh, grid, "frame", scale, krows_h,
                                            krows_t)
    khi = torch.from_numpy(heads[krows_h].astype(np.int64)).to(DEV)
    kti = torch.from_numpy(krows_t).to(DEV)
    assert_grad_close(host(grads["dk"][khi, kti]), (dk_m + dk_t + dk_f) / 3.0,
                      "30 s hybrid dk rows")
    assert_grad_close(host(grads["dv"][khi, kti]), (dv_m + dv_t + dv_f) / 3.0,
                      "30 s hybrid dv rows")

    # dp and dx of the dq tokens: the MoGA share of d_out is a third
    qfull, kfull, vfull, gfull = host(q), host(k), host(v), host(dout)
    rows_all_h = np.repeat(np.arange(nh), t.size).astype(np.int32)
    rows_all_t = np.tile(t, nh).astype(np.int64)
    _, D_all, _ = oracle.moga_dq_rows(qfull, kfull, vfull, gfull, g, m, r["p_sel"], scale,
                                      rows_all_h, rows_all_t)
    del qfull, kfull, vfull, gfull
    dp_ref = D_all.reshape(nh, t.size).sum(0) / r["p_sel"][t] / 3.0
    tt = torch.from_numpy(t).to(DEV)
    assert_grad_close(host(grads["dp"][tt]), dp_ref, "30 s hybrid dp rows")
    _, dx_ref = oracle.router_backward_rows(xh[t], wh, g[t], dp_ref, r["counts"], n, d_loss,
                                            wl.alpha)
    assert_grad_close(host(grads["dx"][tt]), dx_ref, "30 s hybrid dx rows")
