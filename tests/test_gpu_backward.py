"""Parity of moga_backward (and the forward's lse output) with the CPU oracle.

Small cases compare every gradient element with oracle.moga_backward.  The full-size cases
run the backward at the workload sizes and compare sampled rows the oracle computes one by
one (dq, D and lse per (head, token); dp and dx per token), plus properties that hold at any
size: the sum of dv over a group equals the sum of p * d_out over it, the sum of dk over a
group vanishes, and every row of dW sums to zero (softmax backward rows sum to zero).

Floating-point bar (bf16 operands, fp32 accumulation): each gradient element is a sum of
products whose factors were rounded to bf16 once or twice (dO' = p d_out, P or dS) and the
result is rounded to bf16 once more, so its error is a few units of 2^-9 relative to the
typical size of the terms.  The tests bound the relative RMS error of every tensor by GRAD_RMS
and the largest error by GRAD_MAX times the RMS of the reference tensor."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from sparse_attention_long_moga_amd import api
from tests.helpers import host, rel_rms

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

GRAD_RMS = 1e-2      # relative RMS error of dq, dk, dv, dp, dx, dw
GRAD_MAX = 8e-2      # largest error / RMS of the reference tensor
LSE_ABS = 2.5e-3     # the forward sums bf16-rounded probabilities: |d lse| <= 2^-9 (+ fp32)


def _announce(what, **kw):
    print(f"[case] {what} {kw}", flush=True)


def assert_grad_close(got, ref, what, rrms=GRAD_RMS, rmax=GRAD_MAX):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    scale = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    r = rel_rms(got, ref)
    print(f"  {what}: rel_rms={r:.2e} max_err/rms={err / scale if scale else err:.2e}", flush=True)
    assert r <= rrms, f"{what}: relative RMS {r:.3e} > {rrms}"
    assert err <= rmax * scale, f"{what}: max error {err:.3e} > {rmax} x RMS {scale:.3e}"


def _case(n, h, m, seed, d=256, x_dtype="bf16", hd=128):
    wl = workloads.small(f"bwd_{n}_{m}", n, d, h, hd, m, seed=seed, x_dtype=x_dtype)
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    q, k, v = workloads.make_qkv(wl, DEV)
    dout = workloads.make_dout(wl, DEV)
    return wl, x, w, q, k, v, dout


def _forward_backward(wl, x, w, q, k, v, dout, d_loss, pin=None, fused=True):
    fwd = api.moga_forward(x, w, q, k, v, wl.n_groups, alpha=wl.alpha, pin=pin, fused=fused,
                           with_lse=True)
    grads = api.moga_backward(x, w, q, k, v, fwd, dout, d_loss=d_loss, alpha=wl.alpha)
    torch.cuda.synchronize()
    return fwd, grads


def _check_all(wl, x, w, q, k, v, dout, d_loss, fwd, grads, group_id, what):
    """Every element against oracle.moga_backward (routing taken from the oracle's router)."""
    ref = oracle.moga_backward(host(x), host(w), host(q), host(k), host(v), group_id,
                               host(dout), d_loss, wl.alpha, 1.0 / math.sqrt(wl.head_dim))
    err = np.abs(host(fwd["lse"]) - ref["lse"]).max()
    assert err <= LSE_ABS, f"{what}: lse error {err:.3e}"
    for name in ("dq", "dk", "dv", "dp", "dx", "dw"):
        assert_grad_close(host(grads[name]), ref[name], f"{what} {name}")
    return ref


@pytest.mark.parametrize("n, h, m, seed, x_dtype, hd", [
    (1000, 2, 5, 51, "bf16", 128),    # ragged groups (none a multiple of 128)
    (2600, 2, 3, 52, "f32", 128),     # several 128-row tiles per group, fp32 router input
    (777, 3, 8, 53, "bf16", 128),
    (1300, 2, 4, 58, "f32", 64),      # head_dim 64 (rows widened to the 128-channel kernels)
    (333, 1, 3, 59, "bf16", 64),
])
def test_backward_parity(n, h, m, seed, x_dtype, hd):
    _announce("backward", n=n, h=h, m=m, x_dtype=x_dtype, hd=hd)
    wl, x, w, q, k, v, dout = _case(n, h, m, seed, x_dtype=x_dtype, hd=hd)
    r = oracle.route(host(x), host(w))
    pin = torch.from_numpy(oracle.near_tie_pins(r)).to(DEV)
    fwd, grads = _forward_backward(wl, x, w, q, k, v, dout, 1.3, pin=pin)
    np.testing.assert_array_equal(host(fwd["group_id"]), r["group_id"])
    _check_all(wl, x, w, q, k, v, dout, 1.3, fwd, grads, r["group_id"], f"n={n} m={m}")


def test_backward_edge_groups():
    """Pinned routing: an empty group, a group of one token, a group of exactly 128 tokens
    (one full tile) and the rest in a ragged group."""
    _announce("backward_edges")
    n, m = 700, 5
    wl, x, w, q, k, v, dout = _case(n, 2, m, 54)
    pin_np = np.full(n, 3, np.int32)
    pin_np[::7] = 1                      # 100 tokens
    pin_np[5] = 4                        # a group of one
    pin_np[np.arange(200, 700, 2)[:128]] = 2  # exactly 128 tokens
    assert np.sum(pin_np == 0) == 0
    pin = torch.from_numpy(pin_np).to(DEV)
    fwd, grads = _forward_backward(wl, x, w, q, k, v, dout, 0.4, pin=pin)
    counts = np.bincount(pin_np, minlength=m)
    assert host(fwd["counts"]).tolist() == counts.tolist()
    assert counts[0] == 0 and counts[4] == 1 and counts[2] == 128
    _check_all(wl, x, w, q, k, v, dout, 0.4, fwd, grads, pin_np, "edges")


def test_backward_single_group_collapse():
    _announce("backward_collapse")
    n = 900
    wl, x, w, q, k, v, dout = _case(n, 1, 4, 55)
    pin_np = np.zeros(n, np.int32)
    fwd, grads = _forward_backward(wl, x, w, q, k, v, dout, 2.0,
                                   pin=torch.from_numpy(pin_np).to(DEV))
    assert host(fwd["cu_seqlens"]).tolist() == [0, n, n, n, n]
    _check_all(wl, x, w, q, k, v, dout, 2.0, fwd, grads, pin_np, "collapse")


def test_backward_loss_only_is_exact_zero_through_attention():
    """d_out = 0: no gradient reaches q, k, v or p (bitwise zero), and dx, dW come from the
    balance loss alone (fp32 against fp64)."""
    _announce("backward_loss_only")
    wl, x, w, q, k, v, _ = _case(1500, 2, 6, 56)
    dout = torch.zeros_like(q)
    r = oracle.route(host(x), host(w))
    pin = torch.from_numpy(oracle.near_tie_pins(r)).to(DEV)
    fwd, grads = _forward_backward(wl, x, w, q, k, v, dout, 1.0, pin=pin)
    for name in ("dq", "dk", "dv", "dp"):
        assert torch.count_nonzero(grads[name]) == 0, name
    ref = oracle.moga_backward(host(x), host(w), host(q), host(k), host(v), r["group_id"],
                               host(dout), 1.0, wl.alpha, 1.0 / math.sqrt(128))
    assert_grad_close(host(grads["dx"]), ref["dx"], "loss-only dx", rrms=1e-4, rmax=1e-3)
    assert_grad_close(host(grads["dw"]), ref["dw"], "loss-only dw", rrms=1e-4, rmax=1e-3)


def test_backward_fused_and_explicit_forward_agree_and_repeat():
    """lse from both forward variants is bitwise equal, so the backward is too; two backward
    calls give bitwise equal gradients (no atomics, fixed orders)."""
    _announce("backward_determinism")
    wl, x, w, q, k, v, dout = _case(3000, 2, 5, 57)
    fa, ga = _forward_backward(wl, x, w, q, k, v, dout, 0.5, fused=False)
    fb, gb = _forward_backward(wl, x, w, q, k, v, dout, 0.5, fused=True)
    assert torch.equal(fa["lse"], fb["lse"])
    assert torch.equal(fa["out"], fb["out"])
    for name in ga:
        assert torch.equal(ga[name], gb[name]), name


FULL = [workloads.WAN5S, workloads.WAN30S_SKEW]


@pytest.mark.parametrize("wl", FULL, ids=[w.name for w in FULL])
def test_full_size_backward(wl):
    _announce("full-size backward", name=wl.name)
    n, m, hd, nh = wl.n_tokens, wl.n_groups, wl.head_dim, wl.n_heads
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    q, k, v = workloads.make_qkv(wl, DEV)
    dout = workloads.make_dout(wl, DEV)
    xh, wh = host(x), host(w)
    r = oracle.route(xh, wh)
    pin = torch.from_numpy(oracle.near_tie_pins(r)).to(DEV)
    d_loss = 0.8
    fwd, grads = _forward_backward(wl, x, w, q, k, v, dout, d_loss, pin=pin)
    g = r["group_id"]
    np.testing.assert_array_equal(host(fwd["group_id"]), g)
    scale = 1.0 / math.sqrt(hd)

    # sampled tokens, every head: dq, D, lse rows; dp and dx of those tokens
    toks = []
    rng = np.random.Generator(np.random.PCG64(wl.seed + 91))
    for gi in range(m):
        mem = np.flatnonzero(g == gi)
        if mem.size:
            toks.append(rng.choice(mem, size=min(6, mem.size), replace=False))
    t = np.unique(np.concatenate(toks))
    rows_h = np.repeat(np.arange(nh), t.size).astype(np.int32)
    rows_t = np.tile(t, nh).astype(np.int64)
    # the oracle reads whole heads; pass host copies of all heads once
    qh, kh, vh, gh = host(q), host(k), host(v), host(dout)
    dq_ref, D_ref, lse_ref = oracle.moga_dq_rows(qh, kh, vh, gh, g, m, r["p_sel"], scale,
                                                 rows_h, rows_t)
    del qh, kh, vh, gh
    ti = torch.from_numpy(rows_t).to(DEV)
    hi = torch.from_numpy(rows_h.astype(np.int64)).to(DEV)
    assert_grad_close(host(grads["dq"][hi, ti]), dq_ref, f"{wl.name} dq rows")
    err = np.abs(host(fwd["lse"][hi, ti]) - lse_ref).max()
    assert err <= LSE_ABS, f"lse error {err:.3e}"
    dp_ref = D_ref.reshape(nh, t.size).sum(0) / r["p_sel"][t]
    assert_grad_close(host(grads["dp"][torch.from_numpy(t).to(DEV)]), dp_ref, f"{wl.name} dp rows")
    _, dx_ref = oracle.router_backward_rows(xh[t], wh, g[t], dp_ref, r["counts"], n, d_loss,
                                            wl.alpha)
    assert_grad_close(host(grads["dx"][torch.from_numpy(t).to(DEV)]), dx_ref,
                      f"{wl.name} dx rows")

    # dk and dv of sampled key rows of the two smallest groups, last head (the oracle needs the
    # softmax row of every query of a key's group: |G|^2 hd per (head, group))
    sizes = np.bincount(g, minlength=m)
    smallest = [int(i) for i in np.argsort(sizes, kind="stable") if sizes[i] > 0][:2]
    krows_t = np.concatenate([rng.choice(np.flatnonzero(g == gi), size=min(6, int(sizes[gi])),
                                         replace=False) for gi in smallest]).astype(np.int64)
    hl = nh - 1
    qh, kh, vh, gh = (host(t[hl:hl + 1]) for t in (q, k, v, dout))
    dk_ref, dv_ref = oracle.moga_dkdv_rows(qh, kh, vh, gh, g, m, r["p_sel"], scale,
                                           np.zeros(krows_t.size, np.int32), krows_t)
    del qh, kh, vh, gh
    kt = torch.from_numpy(krows_t).to(DEV)
    assert_grad_close(host(grads["dk"][hl][kt]), dk_ref, f"{wl.name} dk rows (groups {smallest})")
    assert_grad_close(host(grads["dv"][hl][kt]), dv_ref, f"{wl.name} dv rows (groups {smallest})")

    # group sums at full size, two heads
    gd = torch.from_numpy(g.astype(np.int64)).to(DEV)
    psel = fwd["p_sel"]
    for hh in (0, nh - 1):
        dv_sum = torch.zeros(m, hd, dtype=torch.float64, device=DEV).index_add_(
            0, gd, grads["dv"][hh].double())
        want = torch.zeros(m, hd, dtype=torch.float64, device=DEV).index_add_(
            0, gd, psel.double()[:, None] * dout[hh].double())
        assert_grad_close(host(dv_sum), host(want), f"{wl.name} head {hh} group sums of dv")
        dk_sum = torch.zeros(m, hd, dtype=torch.float64, device=DEV).index_add_(
            0, gd, grads["dk"][hh].double())
        dk_abs = torch.zeros(m, hd, dtype=torch.float64, device=DEV).index_add_(
            0, gd, grads["dk"][hh].double().abs())
        ratio = float((dk_sum.abs() / dk_abs.clamp_min(1e-30)).max())
        print(f"  head {hh}: |sum dk| / sum |dk| = {ratio:.2e}", flush=True)
        assert ratio < 2e-2, f"group sum of dk is not ~0 ({ratio:.3e})"
    row = grads["dw"].double().sum(1).abs().max().item()
    scale_w = grads["dw"].double().abs().sum(1).max().item()
    assert row <= 1e-3 * scale_w, f"dW rows do not sum to zero ({row:.3e} vs {scale_w:.3e})"
