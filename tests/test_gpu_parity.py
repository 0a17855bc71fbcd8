"""GPU parity of every entry point against the CPU oracle, on seeded inputs that span
several tiles and a ragged tail, plus edge cases.  All calls go through the C ABI."""
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


def _announce(what, **kw):
    print(f"[case] {what} {kw}", flush=True)


def _router_case(n, d, m, seed, x_dtype="bf16", dirichlet=None):
    wl = workloads.small(f"route_{n}_{d}_{m}", n, d, 1, 64, m, seed=seed, x_dtype=x_dtype,
                         mixture="normal" if x_dtype == "f32" else "gaussian",
                         dirichlet=dirichlet)
    return wl, workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)


# ------------------------------------------------------------------------------- router
@pytest.mark.parametrize("n, d, m, x_dtype, seed", [
    (4096, 256, 4, "f32", 1),        # the tiny workload's router shape
    (5000, 384, 5, "bf16", 2),       # several blocks and a ragged tail
    (3001, 1536, 5, "bf16", 3),
    (2500, 512, 20, "bf16", 4),
    (700, 512, 64, "bf16", 5),       # W larger than the LDS budget: chunked over d
    (1234, 200, 37, "bf16", 8),      # d not a multiple of 32: a partial last k-step
    (1, 64, 3, "bf16", 6),           # a single token
    (333, 128, 1, "f32", 7),         # one group: p == 1
    (2000, 1024, 8, "bf16", 9),      # two 512-column stripes, eight groups
    (999, 1000, 7, "bf16", 10),      # a partial last stripe (columns 512..999)
    (4099, 1536, 4, "bf16", 11),     # fewer groups than the kernel's slots; a 3-token tail
    (70000, 1536, 5, "bf16", 12),    # many waves, each over a range of 16-token tiles
    (3000, 512, 16, "bf16", 13),     # sixteen groups: every lane of the row-contiguous kernel
    (500, 768, 1, "bf16", 14),       # one group in bf16: p == 1
    # bf16 x whose three-term W image exceeds the LDS budget: W streamed through LDS in chunks
    # of 256 columns (the Wan2.1-14B width, 5120, with the pages' M = 5, 16 and 20)
    (3000, 5120, 5, "bf16", 21),
    (2000, 5120, 16, "bf16", 22),
    (4000, 5120, 20, "bf16", 32),
    (2100, 1000, 30, "bf16", 33),    # the most groups two chunk buffers hold; a partial chunk
    (37, 2048, 20, "bf16", 34),      # one block, most of its waves without a tile
    (1, 5120, 5, "bf16", 35),        # a single token
    (300, 10240, 1, "bf16", 36),     # one group: p == 1
    (70000, 2048, 12, "bf16", 37),   # every CU, a partial last tile group per block
    (1234, 200, 20, "bf16", 39),     # one partial chunk (the image would fit in LDS, M > 16)
    (999, 1000, 17, "bf16", 40),     # one group past the first group tile
    # bf16 x with 31 or 32 groups and a large image: W fragments streamed from L2
    (1500, 1024, 32, "bf16", 38),
    # f32 x at every group-count instantiation of the vector router
    (2500, 256, 5, "f32", 23),
    (2500, 256, 8, "f32", 24),
    (1500, 512, 16, "f32", 25),
    (1500, 300, 20, "f32", 26),
    (1000, 256, 32, "f32", 27),
    (700, 128, 64, "f32", 28),
    # f32 x with W^T larger than the LDS budget: W staged in chunks of columns (a partial last
    # chunk for d = 4100)
    (600, 5120, 5, "f32", 29),
    (500, 4100, 20, "f32", 30),
    (400, 1024, 64, "f32", 31),
])
def test_route_parity(n, d, m, x_dtype, seed):
    _announce("route", n=n, d=d, m=m, x_dtype=x_dtype)
    wl, x, w = _router_case(n, d, m, seed, x_dtype)
    ref = oracle.route(host(x), host(w))
    pin = torch.from_numpy(oracle.near_tie_pins(ref)).to(DEV)
    got = api.moga_route(x, w, m, pin=pin)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got["group_id"]), ref["group_id"])
    np.testing.assert_array_equal(host(got["counts"]), ref["counts"])  # F_i exact
    np.testing.assert_allclose(host(got["p_sel"]), ref["p_sel"], rtol=0, atol=2e-6)
    P_gpu, P_ref = host(got["prob_sum"]) / n, ref["prob_sum"] / n
    assert np.abs(P_gpu - P_ref).max() < 1e-6
    if m == 1:
        assert np.all(host(got["p_sel"]) == 1.0)


def test_route_pins_force_groups():
    _announce("route_pins")
    wl, x, w = _router_case(1000, 256, 4, 9)
    pin = torch.full((1000,), -1, dtype=torch.int32, device=DEV)
    pin[::7] = 2
    got = api.moga_route(x, w, 4, pin=pin)
    ref = oracle.route(host(x), host(w), pin=host(pin))
    free = ref["gap"] >= 1e-5
    gid = host(got["group_id"])
    assert np.all(gid[::7] == 2)
    np.testing.assert_array_equal(gid[free], ref["group_id"][free])
    np.testing.assert_allclose(host(got["p_sel"])[::7], ref["p_sel"][::7], atol=2e-6)


# ------------------------------------------------------------------------------- permute
@pytest.mark.parametrize("n, m, hd, case", [
    (5000, 5, 128, "random"), (4097, 7, 64, "empty_group"), (2048, 1, 128, "one_group"),
    (3000, 4, 64, "collapse"), (1, 3, 64, "single"), (6000, 64, 64, "random"),
    # many index blocks: runs of one group longer than a block (most groups absent from most
    # blocks, so every block's prefix adds many zeros), and a skewed mixture over 64 groups
    (200001, 64, 64, "runs"), (150000, 64, 64, "skewed"),
])
def test_permute_parity_and_round_trip(n, m, hd, case):
    _announce("permute", n=n, m=m, hd=hd, case=case)
    rng = np.random.Generator(np.random.PCG64(n + m))
    g = rng.integers(0, m, n).astype(np.int32)
    if case == "empty_group":
        g[g == 3] = 4
    if case == "collapse":
        g[:] = 2
    if case == "runs":
        g = np.repeat(rng.integers(0, m, n // 5000 + 1), 5000)[:n].astype(np.int32)
    if case == "skewed":
        g = rng.choice(m, n, p=rng.dirichlet(np.full(m, 0.2))).astype(np.int32)
    gid = torch.from_numpy(g).to(DEV)
    h = 3
    q = torch.randn((h, n, hd), device=DEV, dtype=torch.bfloat16)
    k = torch.randn((h, n, hd), device=DEV, dtype=torch.bfloat16)
    p = torch.rand(n, device=DEV, dtype=torch.float32)
    cu, perm, (qp, kp), pp = api.moga_permute(gid, [q, k], m, p_sel=p)
    torch.cuda.synchronize()
    cu_ref, perm_ref = oracle.groups(g, m)
    np.testing.assert_array_equal(host(cu), cu_ref)
    np.testing.assert_array_equal(host(perm), perm_ref)
    pl = perm.long()
    assert torch.equal(qp, q[:, pl]) and torch.equal(kp, k[:, pl])
    assert torch.equal(pp, p[pl])
    back = api.moga_unpermute(perm, [qp, kp], m)
    torch.cuda.synchronize()
    assert torch.equal(back[0], q) and torch.equal(back[1], k)


@pytest.mark.parametrize("n, m, case", [
    (1048576, 64, "random"),   # 512 index blocks: the largest table the scatter scans itself
    (1048577, 64, "random"),   # 513 blocks: the scan runs as its own launch
    (1200001, 64, "runs"),     # the scan launch with most groups absent from most blocks
    (4000000, 5, "skewed"),    # five groups over 1954 blocks: the scan launch
])
def test_index_build_large(n, m, case):
    """cu_seqlens and perm alone (no rows moved) on both sides of the in-scatter scan's bound."""
    _announce("index build", n=n, m=m, case=case)
    rng = np.random.Generator(np.random.PCG64(n + 7 * m))
    if case == "runs":
        g = np.repeat(rng.integers(0, m, n // 5000 + 1), 5000)[:n].astype(np.int32)
    elif case == "skewed":
        g = rng.choice(m, n, p=rng.dirichlet(np.full(m, 0.5))).astype(np.int32)
    else:
        g = rng.integers(0, m, n).astype(np.int32)
    cu, perm, _, _ = api.moga_permute(torch.from_numpy(g).to(DEV), [], m)
    torch.cuda.synchronize()
    cu_ref, perm_ref = oracle.groups(g, m)
    np.testing.assert_array_equal(host(cu), cu_ref)
    np.testing.assert_array_equal(host(perm), perm_ref)


# ------------------------------------------------------------------------------- varlen attention
def _segments(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("case", ["mixed", "q_ne_k", "tiny_segments"])
def test_group_attn_parity(hd, case):
    _announce("group_attn", hd=hd, case=case)
    rng = np.random.Generator(np.random.PCG64(hd * 7 + len(case)))
    if case == "mixed":
        ql = np.array([700, 0, 1, 129, 64, 1000, 33])
        kl = ql.copy()
    elif case == "q_ne_k":
        ql = np.array([780, 195, 300, 1, 77])
        kl = np.array([1560, 585, 0, 5, 64])   # one segment with queries but no keys
    else:
        ql = rng.integers(0, 5, 40)
        kl = rng.integers(1, 6, 40)
    cu_q, cu_k = _segments(ql), _segments(kl)
    h = 2
    lq, lk = int(cu_q[-1]), int(cu_k[-1])
    q = torch.randn((h, lq, hd), device=DEV, dtype=torch.bfloat16)
    k = torch.randn((h, lk, hd), device=DEV, dtype=torch.bfloat16)
    v = torch.randn((h, lk, hd), device=DEV, dtype=torch.bfloat16)
    rs = torch.rand(lq, device=DEV, dtype=torch.float32) + 0.5
    out = api.moga_group_attn(q, k, v, torch.from_numpy(cu_q).to(DEV),
                              torch.from_numpy(cu_k).to(DEV), row_scale=rs)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(hd)
    rows_h, rows_i = np.repeat(np.arange(h), lq), np.tile(np.arange(lq), h)
    ref, pairs = oracle.varlen_attn(host(q), host(k), host(v), cu_q, cu_k, scale, rows_h, rows_i,
                                    row_scale=host(rs))
    assert_close_bf16(host(out).reshape(-1, hd), ref, f"group_attn {case} hd={hd}")


def test_group_attn_head_beyond_32bit_offsets():
    """K/V heads of more than 2^31 bytes (over 8.4 M rows at head_dim 128) leave the
    direct-load kernel's 32-bit buffer offsets and take the register-staged kernel: 65,568
    segments of 128 keys and 8 queries, compared on every query of sampled segments,
    including the last ones, whose keys lie beyond byte 2^31 of the head."""
    _announce("group_attn beyond 32-bit head", hd=128)
    n_seg, kper, qper, hd = 65568, 128, 8, 128
    assert n_seg * kper * hd * 2 > (1 << 31)
    cu_k = _segments(np.full(n_seg, kper))
    cu_q = _segments(np.full(n_seg, qper))
    g = torch.Generator(device=DEV)
    g.manual_seed(4242)
    q = torch.randn((1, n_seg * qper, hd), generator=g, device=DEV, dtype=torch.bfloat16)
    k = torch.randn((1, n_seg * kper, hd), generator=g, device=DEV, dtype=torch.bfloat16)
    v = torch.randn((1, n_seg * kper, hd), generator=g, device=DEV, dtype=torch.bfloat16)
    out = api.moga_group_attn(q, k, v, torch.from_numpy(cu_q).to(DEV),
                              torch.from_numpy(cu_k).to(DEV))
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(4243))
    segs = np.unique(np.concatenate([rng.choice(n_seg, 40, replace=False),
                                     np.arange(n_seg - 8, n_seg)]))
    # the sampled segments' rows alone, as a smaller varlen problem for the oracle
    qi = np.concatenate([np.arange(cu_q[s], cu_q[s + 1]) for s in segs])
    ki = np.concatenate([np.arange(cu_k[s], cu_k[s + 1]) for s in segs])
    sub_q = host(q[:, torch.from_numpy(qi).to(DEV)])
    sub_k = host(k[:, torch.from_numpy(ki).to(DEV)])
    sub_v = host(v[:, torch.from_numpy(ki).to(DEV)])
    scq = _segments(np.full(segs.size, qper))
    sck = _segments(np.full(segs.size, kper))
    ref, _ = oracle.varlen_attn(sub_q, sub_k, sub_v, scq, sck, 1 / math.sqrt(hd),
                                np.zeros(qi.size, np.int64), np.arange(qi.size))
    got = host(out[0, torch.from_numpy(qi).to(DEV)])
    assert_close_bf16(got, ref, "group_attn beyond 32-bit head offsets")


def test_group_attn_leaves_rows_outside_segments():
    _announce("group_attn_untouched")
    h, hd = 1, 64
    cu = torch.tensor([10, 200, 300], dtype=torch.int32, device=DEV)  # rows 0-9, 300+ untouched
    q = torch.randn((h, 400, hd), device=DEV, dtype=torch.bfloat16)
    k = torch.randn((h, 400, hd), device=DEV, dtype=torch.bfloat16)
    out = torch.full_like(q, 7.0)
    api.moga_group_attn(q, k, k, cu, cu, out=out)
    torch.cuda.synchronize()
    assert torch.all(out[:, :10] == 7.0) and torch.all(out[:, 300:] == 7.0)
    assert not torch.any(out[:, 10:300] == 7.0)


def _split_tail(kl, n_q_tiles, heads, slots, cap):
    """The planner's key-range split, restated: items run longest key range first (ties by
    segment), head-major within a segment; the last n_items mod slots items are split when
    they are at most half of min(slots, cap) and the first of them has at least 2048 keys.
    Returns ([(segment, head, q tile)] of the split items, parts)."""
    order = sorted(range(len(kl)), key=lambda s: (-kl[s], s))
    items = [(s, hh, t) for s in order for hh in range(heads) for t in range(n_q_tiles[s])]
    cap = min(slots, cap)
    r = len(items) % slots
    if r == 0 or 2 * r > cap or kl[items[len(items) - r][0]] < 2048:
        return [], 1
    return items[len(items) - r:], min(8, cap // r)


@pytest.mark.parametrize("case", ["mixed_segments", "many_segments"])
def test_group_attn_split_tail(case):
    """The last items of a launch split into key ranges and merged: every row of those items
    and a sample of the others against the oracle, including a segment with queries but no
    keys (every part empty), q != k lengths and ragged last query and key tiles."""
    _announce("group_attn_split_tail", case=case)
    rng = np.random.Generator(np.random.PCG64(31 if case == "mixed_segments" else 37))
    hd = 128
    if case == "mixed_segments":  # the tail: a 2500-key segment's items, then a keyless one's
        h = 2
        ql = np.array([20000, 9000, 3000, 1300, 300])
        kl = np.array([20000, 9050, 3000, 2500, 0])
    else:                         # thirty segments of 2100 rows, one head: eight parts
        h = 1
        ql = np.full(30, 2100)
        kl = ql + rng.integers(0, 40, 30)
    cu_q, cu_k = _segments(ql), _segments(kl)
    lq, lk = int(cu_q[-1]), int(cu_k[-1])
    waves = 8 if lq // len(ql) >= 1024 else 4
    bq = 32 * waves
    slots = torch.cuda.get_device_properties(0).multi_processor_count * (8 // waves)
    split, parts = _split_tail(list(kl), [-(-int(x) // bq) for x in ql], h, slots,
                               min(256, h * lq // 256))
    assert split and parts >= 2, "the shape no longer splits on this device"
    q = torch.randn((h, lq, hd), device=DEV, dtype=torch.bfloat16)
    k = torch.randn((h, lk, hd), device=DEV, dtype=torch.bfloat16)
    v = torch.randn((h, lk, hd), device=DEV, dtype=torch.bfloat16)
    rs = torch.rand(lq, device=DEV, dtype=torch.float32) + 0.5
    out = api.moga_group_attn(q, k, v, torch.from_numpy(cu_q).to(DEV),
                              torch.from_numpy(cu_k).to(DEV), row_scale=rs)
    torch.cuda.synchronize()
    rows = set()
    for s_, hh, t in split:
        for i in range(cu_q[s_] + t * bq, min(cu_q[s_] + (t + 1) * bq, cu_q[s_ + 1])):
            rows.add((hh, int(i)))
    for s_ in range(len(ql)):
        if ql[s_]:
            for i in rng.choice(np.arange(cu_q[s_], cu_q[s_ + 1]), size=min(8, int(ql[s_])),
                                replace=False):
                rows.add((int(rng.integers(0, h)), int(i)))
    rows = sorted(rows)
    rows_h = np.array([r[0] for r in rows])
    rows_i = np.array([r[1] for r in rows])
    ref, _ = oracle.varlen_attn(host(q), host(k), host(v), cu_q, cu_k, 1 / math.sqrt(hd),
                                rows_h, rows_i, row_scale=host(rs))
    have = host(out[torch.from_numpy(rows_h).to(DEV), torch.from_numpy(rows_i).to(DEV)])
    assert_close_bf16(have, ref, f"group_attn split tail {case} ({len(split)} items x {parts})")


# ------------------------------------------------------------------------------- STGA
STGA_CASES = {
    "small_hd64": dict(frames=10, height=6, width=8, shot_start=[0, 3, 4, 8, 10], win_h=3,
                       win_w=4, t_group=2, aug_frames=2, heads=2, hd=64),
    "multi_tile_hd128": dict(frames=12, height=10, width=16, shot_start=[0, 5, 9, 12], win_h=5,
                             win_w=8, t_group=4, aug_frames=2, heads=2, hd=128),
    "one_shot_no_aug": dict(frames=6, height=4, width=8, shot_start=[0, 6], win_h=4, win_w=8,
                            t_group=3, aug_frames=0, heads=1, hd=64),
}


@pytest.mark.parametrize("name", sorted(STGA_CASES))
def test_stga_parity(name):
    c = dict(STGA_CASES[name])
    h, hd = c.pop("heads"), c.pop("hd")
    _announce("stga", name=name)
    n = c["frames"] * c["height"] * c["width"]
    lay = api.make_stga_layout(**c)
    q, k, v = (torch.randn((h, n, hd), device=DEV, dtype=torch.bfloat16) for _ in range(3))
    o_t, o_f = api.stga_group_attn(q, k, v, lay)
    torch.cuda.synchronize()
    rows_h, rows_t = np.repeat(np.arange(h), n), np.tile(np.arange(n), h)
    scale = 1 / math.sqrt(hd)
    for mode, o in (("temporal", o_t), ("frame", o_f)):
        ref, _ = oracle.stga_attn(host(q), host(k), host(v), c, mode, scale, rows_h, rows_t)
        assert_close_bf16(host(o).reshape(-1, hd), ref, f"stga {name} {mode}")


# ------------------------------------------------------------------------------- whole forward
def _forward_case(n_frames, h, hd, m, seed, hybrid, d=256):
    n = n_frames * 8 * 12
    wl = workloads.small(f"fwd_{n}", n, d, h, hd, m, seed=seed)
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    q, k, v = workloads.make_qkv(wl, DEV)
    grid = dict(frames=n_frames, height=8, width=12,
                shot_start=workloads.even_shots(n_frames, 3), win_h=4, win_w=6, t_group=2,
                aug_frames=2) if hybrid else None
    return wl, x, w, q, k, v, grid


@pytest.mark.parametrize("hybrid", [False, True])
@pytest.mark.parametrize("hd", [64, 128])
def test_forward_parity(hybrid, hd):
    _announce("forward", hybrid=hybrid, hd=hd)
    wl, x, w, q, k, v, grid = _forward_case(20, 2, hd, 5, 11 + hd, hybrid)
    n, m = wl.n_tokens, wl.n_groups
    ref_r = oracle.route(host(x), host(w))
    pin_np = oracle.near_tie_pins(ref_r)
    pin = torch.from_numpy(pin_np).to(DEV)
    lay = api.make_stga_layout(**grid) if hybrid else None
    got = api.moga_forward(x, w, q, k, v, m, alpha=0.1, pin=pin, stga=lay)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got["group_id"]), ref_r["group_id"])
    cu_ref, perm_ref = oracle.groups(ref_r["group_id"], m)
    np.testing.assert_array_equal(host(got["cu_seqlens"]), cu_ref)
    np.testing.assert_array_equal(host(got["perm"]), perm_ref)
    loss_ref, F_ref, P_ref = oracle.balance_loss(ref_r["counts"], ref_r["prob_sum"], n, 0.1)
    assert abs(float(got["loss"].item()) - loss_ref) < 1e-6
    scale = 1 / math.sqrt(hd)
    h = q.shape[0]
    rows_h, rows_t = np.repeat(np.arange(h), n), np.tile(np.arange(n), h)
    qh, kh, vh = host(q), host(k), host(v)
    ref_m, _ = oracle.moga_attn(qh, kh, vh, ref_r["group_id"], m, ref_r["p_sel"], scale, rows_h,
                                rows_t)
    ref = ref_m
    if hybrid:
        rt, _ = oracle.stga_attn(qh, kh, vh, grid, "temporal", scale, rows_h, rows_t)
        rf, _ = oracle.stga_attn(qh, kh, vh, grid, "frame", scale, rows_h, rows_t)
        ref = (ref_m + rt + rf) / 3.0
    assert_close_bf16(host(got["out"]).reshape(-1, hd), ref, f"forward hybrid={hybrid}")
    # per (head, group), on the MoGA output alone (in the hybrid mean the STGA rows dominate)
    moga = got["out"] if not hybrid else api.moga_forward(x, w, q, k, v, m, alpha=0.1, pin=pin)["out"]
    torch.cuda.synchronize()
    assert_close_per_group(host(moga).reshape(-1, hd), ref_m, rows_h * m + ref_r["group_id"][rows_t],
                           f"forward hybrid={hybrid} MoGA rows per (head, group)")


def test_forward_collapse_and_single_group():
    _announce("forward_collapse")
    wl, x, w, q, k, v, _ = _forward_case(6, 1, 64, 4, 21, False)
    n = wl.n_tokens
    pin = torch.zeros(n, dtype=torch.int32, device=DEV)  # every token forced into group 0
    got = api.moga_forward(x, w, q, k, v, 4, pin=pin)
    torch.cuda.synchronize()
    ref_r = oracle.route(host(x), host(w), pin=np.zeros(n, np.int32))
    assert host(got["cu_seqlens"]).tolist() == [0, n, n, n, n]
    rows = np.arange(n)
    ref, _ = oracle.moga_attn(host(q), host(k), host(v), ref_r["group_id"], 4, ref_r["p_sel"],
                              1 / 8, np.zeros(n), rows)
    assert_close_bf16(host(got["out"])[0], ref, "collapse")
    loss_ref = 0.1 * 4 * ref_r["prob_sum"][0] / n
    assert abs(float(got["loss"].item()) - loss_ref) < 1e-6


def test_forward_is_deterministic():
    _announce("determinism")
    wl, x, w, q, k, v, grid = _forward_case(12, 2, 128, 5, 31, True)
    lay = api.make_stga_layout(**grid)
    a = api.moga_forward(x, w, q, k, v, 5, stga=lay)
    b = api.moga_forward(x, w, q, k, v, 5, stga=lay)
    torch.cuda.synchronize()
    for key in ("out", "group_id", "perm", "cu_seqlens", "p_sel", "prob_sum", "loss"):
        assert torch.equal(a[key], b[key]), key


def test_balance_loss_parity():
    _announce("balance_loss")
    counts = torch.tensor([10, 0, 30, 60], dtype=torch.int32, device=DEV)
    ps = torch.tensor([20.5, 3.25, 30.0, 46.25], dtype=torch.float64, device=DEV)
    loss, F, P = api.moga_balance_loss(counts, ps, 100, alpha=0.1)
    l_ref, F_ref, P_ref = oracle.balance_loss(host(counts), host(ps), 100, 0.1)
    assert float(loss.item()) == pytest.approx(l_ref, abs=1e-15)
    np.testing.assert_array_equal(host(F), F_ref)
    np.testing.assert_allclose(host(P), P_ref, atol=1e-16)


@pytest.mark.parametrize("hybrid", [False, True])
@pytest.mark.parametrize("hd", [64, 128])
def test_fused_forward_is_bitwise_the_explicit_one(hybrid, hd):
    _announce("fused_vs_explicit", hybrid=hybrid, hd=hd)
    wl, x, w, q, k, v, grid = _forward_case(18, 2, hd, 5, 41 + hd, hybrid)
    lay = api.make_stga_layout(**grid) if hybrid else None
    a = api.moga_forward(x, w, q, k, v, 5, stga=lay)
    b = api.moga_forward_fused(x, w, q, k, v, 5, stga=lay)
    torch.cuda.synchronize()
    for key in ("out", "group_id", "perm", "cu_seqlens", "p_sel", "prob_sum", "counts", "loss"):
        assert torch.equal(a[key], b[key]), key
    # and against the oracle
    n, m = wl.n_tokens, wl.n_groups
    ref_r = oracle.route(host(x), host(w))
    scale = 1 / math.sqrt(hd)
    rows_h, rows_t = np.repeat(np.arange(2), n), np.tile(np.arange(n), 2)
    qh, kh, vh = host(q), host(k), host(v)
    ref, _ = oracle.moga_attn(qh, kh, vh, ref_r["group_id"], m, ref_r["p_sel"], scale, rows_h,
                              rows_t)
    if hybrid:
        ref = (ref + oracle.stga_attn(qh, kh, vh, grid, "temporal", scale, rows_h, rows_t)[0]
               + oracle.stga_attn(qh, kh, vh, grid, "frame", scale, rows_h, rows_t)[0]) / 3.0
    assert_close_bf16(host(b["out"]).reshape(-1, hd), ref, f"fused hybrid={hybrid}")


def test_fused_forward_is_bitwise_the_explicit_one_with_split_tail():
    """At the 5 s size the last 24 items are split into key ranges: the fused forward (rows
    read through perm) must still equal the explicit one bit for bit, lse included."""
    wl = workloads.WAN5S
    _announce("fused_vs_explicit_split", name=wl.name)
    x, w = workloads.make_x(wl, DEV), workloads.make_w(wl, DEV)
    q, k, v = workloads.make_qkv(wl, DEV)
    a = api.moga_forward(x, w, q, k, v, wl.n_groups, alpha=wl.alpha, with_lse=True)
    b = api.moga_forward_fused(x, w, q, k, v, wl.n_groups, alpha=wl.alpha, with_lse=True)
    torch.cuda.synchronize()
    for key in ("out", "lse", "perm", "cu_seqlens", "p_sel"):
        assert torch.equal(a[key], b[key]), key
