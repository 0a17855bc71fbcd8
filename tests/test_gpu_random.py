"""Seeded sweep of small random configurations through the C ABI, against the oracle: the
whole forward (explicit and fused) and the backward, with group counts from 1 to 9, router
widths, head counts and head sizes, bf16 and fp32 router inputs, forced groups for a random
subset of tokens, and (for the hybrid layer) random frame grids, windows, shot cuts, temporal
group sizes and borrowed-frame counts; and the varlen group attention on random segment lists.
Every configuration is drawn from a fixed seed, so a failure names a reproducible case."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from sparse_attention_long_moga_amd import api
from tests.helpers import assert_close_bf16, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (height, width, win_h, win_w): windows that tile the frame, from one window per frame down to
# single-row windows
GRIDS = [(4, 6, 2, 3), (6, 8, 3, 4), (8, 12, 4, 6), (5, 10, 5, 5), (3, 16, 3, 8), (10, 16, 5, 8),
         (4, 4, 1, 4), (7, 9, 7, 3)]


def _config(seed: int) -> dict:
    rng = np.random.default_rng(1000 + seed)
    h_, w_, wh, ww = GRIDS[rng.integers(len(GRIDS))]
    frames = int(rng.integers(2, 15))
    n_shots = int(rng.integers(1, min(frames, 5) + 1))
    cuts = sorted(rng.choice(np.arange(1, frames), size=n_shots - 1, replace=False).tolist())
    f32 = bool(rng.integers(2))
    return dict(
        seed=seed, frames=frames, height=h_, width=w_, win_h=wh, win_w=ww,
        shot_start=[0] + cuts + [frames], t_group=int(rng.integers(1, 5)),
        aug_frames=int(rng.integers(0, 4)), m=int(rng.integers(1, 10)),
        d=int(rng.choice([32, 64, 128, 200] if not f32 else [36, 64, 100])),
        heads=int(rng.integers(1, 4)), hd=int(rng.choice([64, 128])),
        hybrid=bool(rng.integers(2)), fused=bool(rng.integers(2)), f32=f32,
        pin_frac=float(rng.choice([0.0, 0.05, 0.5])))


def _inputs(c):
    n = c["frames"] * c["height"] * c["width"]
    wl = workloads.small(f"rand_{c['seed']}", n, c["d"], c["heads"], c["hd"], c["m"],
                         seed=500 + c["seed"], x_dtype="f32" if c["f32"] else "bf16",
                         mixture="normal" if c["f32"] else "gaussian")
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    q, k, v = workloads.make_qkv(wl, DEV)
    grid = {kk: c[kk] for kk in ("frames", "height", "width", "shot_start", "win_h", "win_w",
                                 "t_group", "aug_frames")}
    # forced groups for a random subset of tokens, plus the oracle's choice on near ties
    rng = np.random.default_rng(2000 + c["seed"])
    r0 = oracle.route(host(x), host(w))
    pin = oracle.near_tie_pins(r0)
    forced = rng.random(n) < c["pin_frac"]
    pin[forced] = rng.integers(0, c["m"], size=int(forced.sum()))
    return wl, x, w, q, k, v, grid, pin


@pytest.mark.parametrize("seed", range(48))
def test_random_forward(seed):
    c = _config(seed)
    print(f"[case] random forward {c}", flush=True)
    wl, x, w, q, k, v, grid, pin = _inputs(c)
    n, m, hd, h = wl.n_tokens, c["m"], c["hd"], c["heads"]
    lay = api.make_stga_layout(**grid) if c["hybrid"] else None
    got = api.moga_forward(x, w, q, k, v, m, alpha=0.1, pin=torch.from_numpy(pin).to(DEV),
                           stga=lay, fused=c["fused"])
    torch.cuda.synchronize()
    ref_r = oracle.route(host(x), host(w), pin=pin)
    np.testing.assert_array_equal(host(got["group_id"]), ref_r["group_id"])
    np.testing.assert_array_equal(host(got["counts"]), ref_r["counts"])
    np.testing.assert_allclose(host(got["p_sel"]), ref_r["p_sel"], rtol=0, atol=2e-6)
    np.testing.assert_allclose(host(got["prob_sum"]) / n, ref_r["prob_sum"] / n, rtol=0,
                               atol=1e-6)
    cu_ref, perm_ref = oracle.groups(ref_r["group_id"], m)
    np.testing.assert_array_equal(host(got["cu_seqlens"]), cu_ref)
    np.testing.assert_array_equal(host(got["perm"]), perm_ref)
    loss_ref, _, _ = oracle.balance_loss(ref_r["counts"], ref_r["prob_sum"], n, 0.1)
    assert abs(float(got["loss"].item()) - loss_ref) < 1e-6
    scale = 1 / math.sqrt(hd)
    rows_h, rows_t = np.repeat(np.arange(h), n), np.tile(np.arange(n), h)
    qh, kh, vh = host(q), host(k), host(v)
    ref, _ = oracle.moga_attn(qh, kh, vh, ref_r["group_id"], m, ref_r["p_sel"], scale, rows_h,
                              rows_t)
    if c["hybrid"]:
        rt, _ = oracle.stga_attn(qh, kh, vh, grid, "temporal", scale, rows_h, rows_t)
        rf, _ = oracle.stga_attn(qh, kh, vh, grid, "frame", scale, rows_h, rows_t)
        ref = (ref + rt + rf) / 3.0
    assert_close_bf16(host(got["out"]).reshape(-1, hd), ref, f"random forward {c}")


def _grad_close(got, ref, what, rrms=1e-2, rmax=8e-2):
    """Relative RMS within rrms and the largest error within rmax times the reference's RMS
    (the bar of the backward parity tests)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    scale = float(np.sqrt(np.mean(ref * ref)))
    r = float(np.sqrt(np.mean((got - ref) ** 2)) / scale) if scale > 0 else 0.0
    err = float(np.abs(got - ref).max())
    assert r <= rrms, f"{what}: relative RMS {r:.3e} > {rrms}"
    assert err <= rmax * scale, f"{what}: max error {err:.3e} > {rmax} x RMS {scale:.3e}"


@pytest.mark.parametrize("seed", range(16))
def test_random_backward(seed):
    c = _config(100 + seed)
    c["f32"], c["d"] = False, 64
    print(f"[case] random backward {c}", flush=True)
    wl, x, w, q, k, v, grid, pin = _inputs(c)
    m, hd = c["m"], c["hd"]
    scale = 1 / math.sqrt(hd)
    lay = api.make_stga_layout(**grid) if c["hybrid"] else None
    saved = api.moga_forward(x, w, q, k, v, m, alpha=0.1, pin=torch.from_numpy(pin).to(DEV),
                             stga=lay, with_lse=True, fused=c["fused"])
    d_out = workloads.make_dout(wl, DEV)
    if c["hybrid"]:
        grads = api.moga_hybrid_backward(x, w, q, k, v, saved, d_out, lay, d_loss=0.7, alpha=0.1)
    else:
        grads = api.moga_backward(x, w, q, k, v, saved, d_out, d_loss=0.7, alpha=0.1)
    torch.cuda.synchronize()
    gid = oracle.route(host(x), host(w), pin=pin)["group_id"]
    np.testing.assert_array_equal(host(saved["group_id"]), gid)
    args = (host(x), host(w), host(q), host(k), host(v), gid)
    if c["hybrid"]:
        ref = oracle.hybrid_backward(*args, grid, host(d_out), 0.7, 0.1, scale)
    else:
        ref = oracle.moga_backward(*args, host(d_out), 0.7, 0.1, scale)
    for key in ("dq", "dk", "dv", "dp", "dx", "dw"):
        _grad_close(host(grads[key]), ref[key], f"random backward {key} {c}")


@pytest.mark.parametrize("seed", range(24))
def test_random_group_attn(seed):
    """Varlen group attention on random segment lists (empty segments, segments with queries
    and no keys, query and key lengths that differ), with and without a per-row factor and at
    a given or the default softmax scale; the allocation-free entry point gives the same bits."""
    rng = np.random.default_rng(4000 + seed)
    n_seg = int(rng.integers(1, 13))
    hd, h = int(rng.choice([64, 128])), int(rng.integers(1, 4))
    top = 1500 if rng.random() < 0.3 else 300
    ql = rng.integers(0, top, n_seg)
    ql[0] = max(int(ql[0]), 1)
    kl = ql.copy() if rng.random() < 0.5 else rng.integers(0, top, n_seg)
    cu_q = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(kl)]).astype(np.int32)
    lq, lk = int(cu_q[-1]), max(int(cu_k[-1]), 1)
    softmax_scale = float(rng.choice([0.0, 0.05, 0.2]))
    print(f"[case] random group_attn seed={seed} ql={ql.tolist()} kl={kl.tolist()} hd={hd} h={h} "
          f"scale={softmax_scale}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(5000 + seed)
    q = torch.randn((h, lq, hd), generator=g, device=DEV, dtype=torch.bfloat16)
    k = torch.randn((h, lk, hd), generator=g, device=DEV, dtype=torch.bfloat16)
    v = torch.randn((h, lk, hd), generator=g, device=DEV, dtype=torch.bfloat16)
    rs = (torch.rand(lq, generator=g, device=DEV) + 0.5) if rng.random() < 0.5 else None
    cq, ck = torch.from_numpy(cu_q).to(DEV), torch.from_numpy(cu_k).to(DEV)
    out = api.moga_group_attn(q, k, v, cq, ck, row_scale=rs, softmax_scale=softmax_scale)
    out2 = api.moga_group_attn_noalloc(q, k, v, cq, ck, row_scale=rs,
                                       softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    scale = softmax_scale if softmax_scale > 0 else 1 / math.sqrt(hd)
    rows_h, rows_i = np.repeat(np.arange(h), lq), np.tile(np.arange(lq), h)
    ref, _ = oracle.varlen_attn(host(q), host(k), host(v), cu_q, cu_k, scale, rows_h, rows_i,
                                row_scale=None if rs is None else host(rs))
    assert_close_bf16(host(out).reshape(-1, hd), ref, f"random group_attn seed={seed}")


@pytest.mark.parametrize("hybrid", [False, True])
@pytest.mark.parametrize("fused", [False, True])
def test_forward_without_optional_outputs(hybrid, fused):
    """The routing outputs are optional (the library keeps them in the workspace when the
    caller passes NULL): out and loss are the same bits with and without them."""
    c = _config(7)
    c.update(hybrid=hybrid, fused=fused, hd=128, f32=False, d=64)
    print(f"[case] forward without optional outputs {c}", flush=True)
    wl, x, w, q, k, v, grid, pin = _inputs(c)
    lay = api.make_stga_layout(**grid) if hybrid else None
    full = api.moga_forward(x, w, q, k, v, c["m"], alpha=0.1, stga=lay, fused=fused)
    bare = dict(out=torch.empty_like(q), loss=torch.empty(1, dtype=torch.float64, device=DEV))
    api.moga_forward(x, w, q, k, v, c["m"], alpha=0.1, stga=lay, fused=fused, out=bare)
    torch.cuda.synchronize()
    assert torch.equal(full["out"], bare["out"])
    assert torch.equal(full["loss"], bare["loss"])


DEGENERATE = {
    # one token; one group
    "n1_m1": dict(frames=1, height=1, width=1, win_h=1, win_w=1, shot_start=[0, 1], t_group=1,
                  aug_frames=0, m=1, hybrid=False),
    # more groups than tokens: most groups empty
    "n6_m9": dict(frames=1, height=2, width=3, win_h=1, win_w=3, shot_start=[0, 1], t_group=1,
                  aug_frames=0, m=9, hybrid=False),
    # hybrid layer on a 1x1x1 grid: every segment holds the one token
    "hybrid_n1": dict(frames=1, height=1, width=1, win_h=1, win_w=1, shot_start=[0, 1],
                      t_group=1, aug_frames=2, m=3, hybrid=True),
    # one frame per shot, single-token windows, more borrowed frames than the shots hold
    "hybrid_1frame_shots": dict(frames=4, height=2, width=2, win_h=1, win_w=1,
                                shot_start=[0, 1, 2, 3, 4], t_group=3, aug_frames=3, m=2,
                                hybrid=True),
}


@pytest.mark.parametrize("name", sorted(DEGENERATE))
@pytest.mark.parametrize("hd", [64, 128])
def test_forward_degenerate(name, hd):
    c = _config(3)
    c.update(DEGENERATE[name], hd=hd, heads=2, f32=False, d=64, fused=False, pin_frac=0.0)
    print(f"[case] degenerate forward {name} {c}", flush=True)
    wl, x, w, q, k, v, grid, pin = _inputs(c)
    n, m = wl.n_tokens, c["m"]
    lay = api.make_stga_layout(**grid) if c["hybrid"] else None
    got = api.moga_forward(x, w, q, k, v, m, alpha=0.1, pin=torch.from_numpy(pin).to(DEV),
                           stga=lay)
    fused = api.moga_forward(x, w, q, k, v, m, alpha=0.1, pin=torch.from_numpy(pin).to(DEV),
                             stga=lay, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(got["out"], fused["out"])
    ref_r = oracle.route(host(x), host(w), pin=pin)
    np.testing.assert_array_equal(host(got["group_id"]), ref_r["group_id"])
    np.testing.assert_array_equal(host(got["counts"]), ref_r["counts"])
    cu_ref, _ = oracle.groups(ref_r["group_id"], m)
    np.testing.assert_array_equal(host(got["cu_seqlens"]), cu_ref)
    scale = 1 / math.sqrt(hd)
    h = c["heads"]
    rows_h, rows_t = np.repeat(np.arange(h), n), np.tile(np.arange(n), h)
    qh, kh, vh = host(q), host(k), host(v)
    ref, _ = oracle.moga_attn(qh, kh, vh, ref_r["group_id"], m, ref_r["p_sel"], scale, rows_h,
                              rows_t)
    if c["hybrid"]:
        rt, _ = oracle.stga_attn(qh, kh, vh, grid, "temporal", scale, rows_h, rows_t)
        rf, _ = oracle.stga_attn(qh, kh, vh, grid, "frame", scale, rows_h, rows_t)
        ref = (ref + rt + rf) / 3.0
    assert_close_bf16(host(got["out"]).reshape(-1, hd), ref, f"degenerate {name} hd={hd}")
    loss_ref, _, _ = oracle.balance_loss(ref_r["counts"], ref_r["prob_sum"], n, 0.1)
    assert abs(float(got["loss"].item()) - loss_ref) < 1e-6


@pytest.mark.parametrize("hybrid", [False, True])
def test_autograd_layer_matches_the_backward_calls(hybrid):
    """moga_attention under autograd: out and loss are moga_forward's, and the gradients of
    <G, out> + 0.7 loss are bitwise those of moga_backward / moga_hybrid_backward."""
    c = _config(11)
    c.update(hybrid=hybrid, hd=128, f32=False, d=64, m=5, pin_frac=0.0)
    print(f"[case] autograd layer {c}", flush=True)
    wl, x, w, q, k, v, grid, _ = _inputs(c)
    lay = api.make_stga_layout(**grid) if hybrid else None
    leaves = [t.detach().clone().requires_grad_(True) for t in (x, w, q, k, v)]
    out, loss = api.moga_attention(*leaves, c["m"], alpha=0.1, stga=lay)
    g = workloads.make_dout(wl, DEV)
    ((out.float() * g.float()).sum() + 0.7 * loss).backward()
    saved = api.moga_forward(x, w, q, k, v, c["m"], alpha=0.1, stga=lay, fused=True,
                             with_lse=True)
    if hybrid:
        ref = api.moga_hybrid_backward(x, w, q, k, v, saved, g, lay, d_loss=0.7, alpha=0.1)
    else:
        ref = api.moga_backward(x, w, q, k, v, saved, g, d_loss=0.7, alpha=0.1)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), saved["out"])
    assert torch.equal(loss.detach(), saved["loss"].view(()))
    for leaf, key in zip(leaves, ("dx", "dw", "dq", "dk", "dv")):
        assert torch.equal(leaf.grad, ref[key].to(leaf.dtype)), key


def test_layer_module_is_the_autograd_layer():
    """MoGALayer holds W as a parameter and runs moga_attention: same outputs, and W's
    gradient is the one moga_attention gives."""
    c = _config(12)
    c.update(hybrid=True, hd=128, f32=False, d=64, m=4, pin_frac=0.0)
    print(f"[case] layer module {c}", flush=True)
    wl, x, w, q, k, v, grid, _ = _inputs(c)
    lay = api.make_stga_layout(**grid)
    layer = api.MoGALayer(c["d"], c["m"], alpha=0.1, stga=lay, device=DEV)
    with torch.no_grad():
        layer.weight.copy_(w)
    out, loss = layer(x, q, k, v)
    (out.float().sum() + loss).backward()
    w2 = w.detach().clone().requires_grad_(True)
    out2, loss2 = api.moga_attention(x, w2, q, k, v, c["m"], alpha=0.1, stga=lay)
    (out2.float().sum() + loss2).backward()
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(loss, loss2)
    assert torch.equal(layer.weight.grad, w2.grad)


@pytest.mark.parametrize("n, d, m, x_dtype", [
    (3000, 512, 5, "bf16"),    # W image in LDS
    (2500, 5120, 20, "bf16"),  # the image streamed through LDS in chunks (a pre-pass)
    (1500, 1024, 32, "bf16"),  # W fragments from L2 (a pre-pass and a work queue)
    (2000, 256, 8, "f32"),     # the vector router
])
def test_route_replays_from_a_hip_graph(n, d, m, x_dtype):
    """Every router path, captured into a HIP graph with a caller workspace: each replay, with
    new x between replays, gives the bits of an eager call."""
    print(f"[case] route graph replay n={n} d={d} m={m} {x_dtype}", flush=True)
    wl = workloads.small(f"route_graph_{d}_{m}", n, d, 1, 64, m, seed=d + m, x_dtype=x_dtype)
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    x2 = workloads.make_x(workloads.small("route_graph_b", n, d, 1, 64, m, seed=d + m + 1,
                                          x_dtype=x_dtype), DEV)
    dims = api.make_dims(n, d, 1, 64, m)
    ws = api.workspace(api.moga_workspace_bytes(dims), DEV)
    api.moga_route(x, w, m, ws=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = api.moga_route(x, w, m, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        if rep == 2:
            x.copy_(x2)
        graph.replay()
        torch.cuda.synchronize()
        eager = api.moga_route(x, w, m)
        torch.cuda.synchronize()
        for key in ("group_id", "p_sel", "counts", "prob_sum"):
            assert torch.equal(got[key], eager[key]), (rep, key)


@pytest.mark.parametrize("hybrid", [False, True])
def test_forward_replays_from_a_hip_graph(hybrid):
    """moga_forward allocates, clears and synchronises nothing itself, so with a caller
    workspace and preallocated outputs it can be captured into a HIP graph: every replay (with
    eager work and synchronisations between replays, and new input values copied into the
    captured tensors) gives the bits of an eager call on the same inputs."""
    c = _config(13)
    c.update(hybrid=hybrid, hd=128, f32=False, d=64, m=5, pin_frac=0.0)
    print(f"[case] graph replay {c}", flush=True)
    wl, x, w, q, k, v, grid, _ = _inputs(c)
    lay = api.make_stga_layout(**grid) if hybrid else None
    n, m = wl.n_tokens, c["m"]
    dims = api.make_dims(n, c["d"], c["heads"], c["hd"], m, alpha=0.1)
    ws = api.workspace(api.moga_workspace_bytes(dims, lay), DEV)

    def outputs():
        return dict(out=torch.empty_like(q), loss=torch.empty(1, dtype=torch.float64, device=DEV),
                    group_id=torch.empty(n, dtype=torch.int32, device=DEV),
                    p_sel=torch.empty(n, dtype=torch.float32, device=DEV),
                    cu_seqlens=torch.empty(m + 1, dtype=torch.int32, device=DEV),
                    perm=torch.empty(n, dtype=torch.int32, device=DEV),
                    counts=torch.empty(m, dtype=torch.int32, device=DEV),
                    prob_sum=torch.empty(m, dtype=torch.float64, device=DEV))

    captured = outputs()
    api.moga_forward(x, w, q, k, v, m, alpha=0.1, stga=lay, ws=ws, out=captured)  # warm
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        api.moga_forward(x, w, q, k, v, m, alpha=0.1, stga=lay, ws=ws, out=captured)
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV)
    for rep in range(4):
        if rep >= 2:  # new input values in the captured tensors
            gen.manual_seed(600 + rep)
            q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
            k.copy_(torch.randn(k.shape, generator=gen, device=DEV).to(k.dtype))
        graph.replay()
        torch.cuda.synchronize()
        eager_ws = api.workspace(api.moga_workspace_bytes(dims, lay), DEV)
        eager = api.moga_forward(x, w, q, k, v, m, alpha=0.1, stga=lay, ws=eager_ws,
                                 out=outputs())
        _ = (q.float() * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        for key in captured:
            assert torch.equal(captured[key], eager[key]), (rep, key)


def test_backward_replays_from_a_hip_graph():
    """The hybrid backward, with a caller workspace and preallocated gradients, captured into a
    HIP graph: every replay gives the bits of an eager call."""
    c = _config(14)
    c.update(hybrid=True, hd=128, f32=False, d=64, m=5, pin_frac=0.0)
    print(f"[case] backward graph replay {c}", flush=True)
    wl, x, w, q, k, v, grid, _ = _inputs(c)
    lay = api.make_stga_layout(**grid)
    n, m, d = wl.n_tokens, c["m"], c["d"]
    saved = api.moga_forward(x, w, q, k, v, m, alpha=0.1, stga=lay, with_lse=True)
    d_out = workloads.make_dout(wl, DEV)
    import ctypes
    from sparse_attention_long_moga_amd import _capi
    dims = api.make_dims(n, d, c["heads"], c["hd"], m, alpha=0.1)
    nb = _capi.load().moga_hybrid_backward_workspace_bytes(ctypes.byref(dims), lay.ref())
    ws = api.workspace(nb, DEV)

    def grads():
        return dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                    dx=torch.empty(n, d, dtype=torch.float32, device=DEV),
                    dw=torch.empty(d, m, dtype=torch.float32, device=DEV),
                    dp=torch.empty(n, dtype=torch.float32, device=DEV))

    captured = grads()
    api.moga_hybrid_backward(x, w, q, k, v, saved, d_out, lay, d_loss=0.7, ws=ws, grads=captured)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        api.moga_hybrid_backward(x, w, q, k, v, saved, d_out, lay, d_loss=0.7, ws=ws,
                                 grads=captured)
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        eager = api.moga_hybrid_backward(x, w, q, k, v, saved, d_out, lay, d_loss=0.7)
        _ = (d_out.float() * 3).sum()
        torch.cuda.synchronize()
        for key in captured:
            assert torch.equal(captured[key], eager[key]), (rep, key)


def test_concurrent_forwards_on_two_streams():
    """Two forwards on two streams at once, each with its own workspace and outputs, give the
    bits of the same calls made one after the other."""
    outs = []
    cases = []
    for seed in (15, 16):
        c = _config(seed)
        c.update(hd=128, f32=False, d=64, pin_frac=0.0)
        cases.append((c, _inputs(c)))
    ref = []
    for c, (wl, x, w, q, k, v, grid, _) in cases:
        lay = api.make_stga_layout(**grid) if c["hybrid"] else None
        ref.append(api.moga_forward(x, w, q, k, v, c["m"], alpha=0.1, stga=lay))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s, (c, (wl, x, w, q, k, v, grid, _)) in zip(streams, cases):
        with torch.cuda.stream(s):
            lay = api.make_stga_layout(**grid) if c["hybrid"] else None
            outs.append(api.moga_forward(x, w, q, k, v, c["m"], alpha=0.1, stga=lay))
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        for key in ("out", "group_id", "perm", "loss"):
            assert torch.equal(a[key], b[key]), key
