"""Parity at the full sizes of the five workloads and of the group-count sweep (M = 1..16 at the
10 s shape), in the launch configuration the benchmark times (one moga_forward call through the
C ABI).

Routing, cu_seqlens, perm, counts (F_i), P_i and the loss are compared on every token.
Attention outputs are compared on seeded samples of output rows, which the oracle computes
one by one: two heads and up to 64 tokens per group (and, for the hybrid workloads, tokens
in the frames on either side of every shot boundary, where keys/values borrow frames)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from sparse_attention_long_moga_amd import api
from tests.helpers import assert_close_bf16, assert_close_per_group, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _sample_rows(wl, group_id, heads, per_group, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    toks = []
    for gidx in range(wl.n_groups):
        members = np.flatnonzero(group_id == gidx)
        if members.size:
            toks.append(rng.choice(members, size=min(per_group, members.size), replace=False))
    if wl.hybrid:
        hw = wl.height * wl.width
        for s in wl.shot_start[1:-1]:  # last frame before and first frame after each cut
            for f in (s - 1, s):
                toks.append(f * hw + rng.choice(hw, size=4, replace=False))
    t = np.unique(np.concatenate(toks))
    rows_h = np.repeat(np.arange(len(heads)), t.size)
    rows_t = np.tile(t, len(heads))
    return rows_h, rows_t


ALL = workloads.CONFIGS + workloads.MSWEEP


@pytest.mark.parametrize("wl", ALL, ids=[w.name for w in ALL])
def test_full_size_forward(wl):
    print(f"[case] full-size forward {wl.name}", flush=True)
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    q, k, v = workloads.make_qkv(wl, DEV)
    n, m, hd = wl.n_tokens, wl.n_groups, wl.head_dim
    xh = host(x)
    ref = oracle.route(xh, host(w))
    del xh
    pin = torch.from_numpy(oracle.near_tie_pins(ref)).to(DEV)
    lay = None
    grid = None
    if wl.hybrid:
        grid = oracle.grid_of(wl)
        lay = api.make_stga_layout(**grid)
    got = api.moga_forward(x, w, q, k, v, m, alpha=wl.alpha, pin=pin, stga=lay)
    torch.cuda.synchronize()
    x_all = x if wl.hybrid else None  # the hybrid check runs the MoGA-only forward again
    del x

    # routing, groups, loss: every token
    np.testing.assert_array_equal(host(got["group_id"]), ref["group_id"])
    np.testing.assert_array_equal(host(got["counts"]), ref["counts"])
    cu_ref, perm_ref = oracle.groups(ref["group_id"], m)
    np.testing.assert_array_equal(host(got["cu_seqlens"]), cu_ref)
    np.testing.assert_array_equal(host(got["perm"]), perm_ref)
    assert np.abs(host(got["prob_sum"]) / n - ref["prob_sum"] / n).max() < 1e-6
    loss_ref = oracle.balance_loss(ref["counts"], ref["prob_sum"], n, wl.alpha)[0]
    assert abs(float(got["loss"].item()) - loss_ref) < 1e-6

    # attention: sampled rows of two heads
    heads = [0, wl.n_heads - 1]
    rows_h, rows_t = _sample_rows(wl, ref["group_id"], heads, 64 if m <= 5 else 16, wl.seed + 7)
    qh = np.stack([host(q[i]) for i in heads])
    kh = np.stack([host(k[i]) for i in heads])
    vh = np.stack([host(v[i]) for i in heads])
    scale = 1.0 / math.sqrt(hd)
    want_m, _ = oracle.moga_attn(qh, kh, vh, ref["group_id"], m, ref["p_sel"], scale, rows_h,
                                 rows_t)
    want = want_m
    if wl.hybrid:
        wt, _ = oracle.stga_attn(qh, kh, vh, grid, "temporal", scale, rows_h, rows_t)
        wf, _ = oracle.stga_attn(qh, kh, vh, grid, "frame", scale, rows_h, rows_t)
        want = (want_m + wt + wf) / 3.0
    gh = torch.tensor([heads[i] for i in rows_h], device=DEV)
    gt = torch.from_numpy(rows_t).to(DEV)
    what = f"{wl.name} sampled rows ({rows_t.size // len(heads)} tokens x 2 heads)"
    assert_close_bf16(host(got["out"][gh, gt]), want, what)
    # the MoGA rows per (head, group): in the hybrid mean the larger STGA rows would hide an
    # error confined to the MoGA branch, so there the MoGA-only forward of the same inputs and
    # the two STGA branches are checked on their own
    label = rows_h * m + ref["group_id"][rows_t]
    if wl.hybrid:
        del got
        moga = api.moga_forward(x_all, w, q, k, v, m, alpha=wl.alpha, pin=pin)["out"]
        o_t, o_f = api.stga_group_attn(q, k, v, lay)
        torch.cuda.synchronize()
        assert_close_per_group(host(moga[gh, gt]), want_m, label, what + " MoGA branch")
        del moga
        assert_close_bf16(host(o_t[gh, gt]), wt, what + " temporal branch")
        assert_close_bf16(host(o_f[gh, gt]), wf, what + " per-frame branch")
    else:
        assert_close_per_group(host(got["out"][gh, gt]), want_m, label, what)


@pytest.mark.parametrize("wl", workloads.CONFIGS, ids=[w.name for w in workloads.CONFIGS])
def test_full_size_fused_forward_is_bitwise_the_explicit_one(wl):
    """The permute-free forward (rows read through perm inside the attention kernel) gives the
    same bits as the explicit one at every workload's full size."""
    print(f"[case] full-size fused forward {wl.name}", flush=True)
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    q, k, v = workloads.make_qkv(wl, DEV)
    lay = api.make_stga_layout(**oracle.grid_of(wl)) if wl.hybrid else None
    a = api.moga_forward(x, w, q, k, v, wl.n_groups, alpha=wl.alpha, stga=lay)
    b = api.moga_forward_fused(x, w, q, k, v, wl.n_groups, alpha=wl.alpha, stga=lay)
    torch.cuda.synchronize()
    for key in ("out", "group_id", "perm", "cu_seqlens", "p_sel", "prob_sum", "counts", "loss"):
        assert torch.equal(a[key], b[key]), key
