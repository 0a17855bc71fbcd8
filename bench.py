#!/usr/bin/env python3
"""Benchmark of the MoGA forward on one MI355X.

A step is one whole forward (route -> histogram/scan/permute -> balance loss -> varlen group
attention scaled by p(g|x), whose epilogue writes each row back to its token; for the hybrid
workloads the two STGA branches run before it and its epilogue stores the 3-way mean) over one
synthetic batch already resident in HBM.  The default
workload is the 30 s, 282,360-token, M = 5 layer with Dirichlet(0.5)-skewed routing.

Prints one JSON line: tokens/s of the whole forward (value), the group-attention
TFLOP/s, per-stage times, the roofline fraction of the dominant kernel (the attention
kernel, measured with HIP events on the stream it runs on) and the CPU oracle's rate on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
DEFAULT_WORKLOAD = "wan1.3b_30s_skewed_N282360_M5"
METRIC = "MoGA fwd tokens/s + group-attn TFLOP/s (% bf16 MFMA peak) at N=282k, M=5"

# HBM bytes per launch of the attention kernel on the default workload: rocprofv3 FETCH_SIZE
# and WRITE_SIZE (KiB per dispatch, one pass each), scaled by what the same counters read for a
# plain 1 GiB device copy (FETCH 2.0x, WRITE 1.0x); the summary with the commands is under
# profiles/.  The figure belongs to one version of the kernel source: any other attn.hip
# reports null until the counters are taken again.
STAGE_REPS = 20  # timed calls per short stage and pass in the stage breakdown
FLUSH_BYTES = 512 << 20  # scratch read before every timed stage call
ATTN_TRAFFIC = {"bytes": 10_717_284 * 1024 * 2 + 850_790 * 1024, "attn_hip_sha256_16": "29b5f1f97824537d",
                "workload": "wan1.3b_30s_skewed_N282360_M5"}


def attn_traffic_bytes(workload: str):
    """HBM bytes per launch of the group-attention kernel from the counter runs, for the
    workload and kernel source they were taken on; None for any other."""
    import hashlib
    if workload != ATTN_TRAFFIC["workload"]:
        return None
    src = os.path.join(ROOT, "sparse_attention_long_moga_amd", "csrc", "attn.hip")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    return ATTN_TRAFFIC["bytes"] if digest == ATTN_TRAFFIC["attn_hip_sha256_16"] else None


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-stages", action="store_true")
    p.add_argument("--msweep", action="store_true",
                   help="only run the group-count sweep (M = 1, 2, 4, 8, 16 at the 10 s shape) "
                        "and print one JSON line per M")
    p.add_argument("--backward", action="store_true",
                   help="only time moga_backward (moga_hybrid_backward on a STGA workload) "
                        "after one forward that saves its state, and print one JSON line")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (calibrates the HBM byte "
                        "counters against a known size) and exit")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the multi-GPU (sequence-parallel) "
                          "path is a design, not an implementation; run --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n_bytes = args.copy_calibration << 20
        src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n_bytes, "copy_bytes_written": n_bytes}))
        return

    import workloads
    from sparse_attention_long_moga_amd import api, metrics

    if not os.path.exists(os.path.join(ROOT, "sparse_attention_long_moga_amd", "libmoga.so")):
        from sparse_attention_long_moga_amd import build
        build.build()

    if args.msweep:
        msweep(args)
        return
    if args.backward:
        backward(args)
        return

    wl = workloads.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n, h, hd, m = wl.n_tokens, wl.n_heads, wl.head_dim, wl.n_groups
    log(f"workload {wl.name}: generating inputs on {dev}")
    x, w = workloads.make_x(wl, dev), workloads.make_w(wl, dev)
    q, k, v = workloads.make_qkv(wl, dev)
    lay = None
    if wl.hybrid:
        lay = api.make_stga_layout(wl.frames, wl.height, wl.width, wl.shot_start, wl.win_h,
                                   wl.win_w, wl.t_group, wl.aug_frames)
    dims = api.make_dims(n, wl.d_model, h, hd, m, alpha=wl.alpha)
    ws = api.workspace(api.moga_workspace_bytes(dims, lay), dev)
    out = dict(out=torch.empty_like(q), loss=torch.empty(1, dtype=torch.float64, device=dev),
               group_id=torch.empty(n, dtype=torch.int32, device=dev),
               p_sel=torch.empty(n, dtype=torch.float32, device=dev),
               cu_seqlens=torch.empty(m + 1, dtype=torch.int32, device=dev),
               perm=torch.empty(n, dtype=torch.int32, device=dev),
               counts=torch.empty(m, dtype=torch.int32, device=dev),
               prob_sum=torch.empty(m, dtype=torch.float64, device=dev))
    torch.cuda.synchronize()

    def step():
        api.moga_forward(x, w, q, k, v, m, alpha=wl.alpha, stga=lay, ws=ws, out=out)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    tokens_per_s = n / (ms_per_step / 1e3)
    log(f"{ms_per_step:.3f} ms/step  ({wall / args.steps * 1e3:.3f} ms wall)  "
        f"{tokens_per_s / 1e6:.3f} M tokens/s")

    counts = out["counts"].cpu().numpy().astype(np.int64)
    pairs_moga = metrics.moga_pairs(counts)
    attn_flops = metrics.attention_flops(pairs_moga, h, hd)
    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": dict(wl.describe(), group_sizes=counts.tolist(),
                       sum_n_sq_over_n_sq=pairs_moga / float(n) ** 2, parallelism="single-gpu"),
    }

    if not args.no_stages:
        result.update(stage_breakdown(args, wl, x, w, q, k, v, lay, ws, dims, counts, attn_flops))
        if lay:
            result.update(hybrid_overhead(args, wl, x, w, q, k, v, lay, ws, out, step))

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x, w, q, k, v, args.cpu_seconds)

    print(json.dumps(result), flush=True)


def stage_breakdown(args, wl, x, w, q, k, v, lay, ws, dims, counts, attn_flops):
    """Time each stage through its own C-ABI call (the same kernels moga_forward
    launches), with HIP events on the stream the kernels run on.  Every timed call is
    preceded by a read of a FLUSH_BYTES scratch buffer (so L2 and the 256 MB MALL hold none
    of its inputs; a read rather than a write, whose dirty lines would be written back
    during the timed call: +54 us on the router) and bracketed alone by its two events; the
    flush also keeps the device busy while the host prepares the call, so the host's
    argument marshalling does not show up as idle device time.  Short stages run STAGE_REPS
    such calls per pass, the attention stages one; the median over all passes is reported."""
    import numpy as np
    import torch

    from sparse_attention_long_moga_amd import api, metrics

    n, h, hd, m = wl.n_tokens, wl.n_heads, wl.head_dim, wl.n_groups
    stream = torch.cuda.current_stream()
    # (no inverse-permute stage: the attention epilogue of moga_forward writes token order)
    names = ["route", "histogram", "permute", "group_attn", "loss"] + (["stga"] if lay else [])
    acc = {s: [] for s in names}
    log(f"stage breakdown over {args.steps} passes")
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=x.device)
    # one pass of the whole path for the later stages' inputs
    r = api.moga_route(x, w, m, ws=ws)
    cu, perm, (qp, kp, vp), pp = api.moga_permute(r["group_id"], [q, k, v], m,
                                                  p_sel=r["p_sel"], ws=ws)
    op = api.moga_group_attn(qp, kp, vp, cu, cu, row_scale=pp, ws=ws)
    torch.cuda.synchronize()
    calls = {
        "route": (lambda: api.moga_route(x, w, m, ws=ws), STAGE_REPS),
        # the index build alone (histogram, scan, stable scatter of perm): no tensors moved
        "histogram": (lambda: api.moga_permute(r["group_id"], [], m, ws=ws), STAGE_REPS),
        "permute": (lambda: api.moga_permute(r["group_id"], [q, k, v], m, p_sel=r["p_sel"], ws=ws),
                    STAGE_REPS),
        "group_attn": (lambda: api.moga_group_attn(qp, kp, vp, cu, cu, row_scale=pp, ws=ws), 1),
        "loss": (lambda: api.moga_balance_loss(r["counts"], r["prob_sum"], n, wl.alpha), STAGE_REPS),
    }
    if lay:
        calls["stga"] = (lambda: api.stga_group_attn(q, k, v, lay, ws=ws), 1)
    for it in range(args.steps + 1):
        for s in names:
            fn, reps = calls[s]
            evs = []
            for i in range(reps):
                flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                evs.append((e0, e1))
            torch.cuda.synchronize()
            if it > 0:  # the first pass warms the allocator
                acc[s].extend(e0.elapsed_time(e1) for e0, e1 in evs)
    del r, cu, perm, qp, kp, vp, pp, op, flush
    ms = {s: float(np.median(v)) for s, v in acc.items()}
    e_bytes = h * n * hd * 2
    x_bytes = n * wl.d_model * (2 if wl.x_dtype == "bf16" else 4)
    route_bytes = x_bytes + wl.d_model * m * 4 + n * 8
    permute_bytes = 6 * e_bytes + n * 4 * 2 + n * 8
    histogram_bytes = n * 4 + n * 4 + (m + 1) * 4  # group ids read, perm and cu_seqlens written
    attn_tflops = attn_flops / (ms["group_attn"] / 1e3) / 1e12
    stages = {
        "stage_ms": ms,
        "attn_tflops": attn_tflops,
        "attn_frac_of_bf16_peak": attn_tflops / MFMA_BF16_PEAK_TFLOPS,
        "route_gbs": route_bytes / (ms["route"] / 1e3) / 1e9,
        "histogram_gbs": histogram_bytes / (ms["histogram"] / 1e3) / 1e9,
        "permute_gbs": permute_bytes / (ms["permute"] / 1e3) / 1e9,
    }
    stages["route_frac_of_hbm"] = stages["route_gbs"] / HBM_PEAK_GBS
    stages["histogram_frac_of_hbm"] = stages["histogram_gbs"] / HBM_PEAK_GBS
    stages["permute_frac_of_hbm"] = stages["permute_gbs"] / HBM_PEAK_GBS
    stages["roofline"] = {
        "bound": "mfma", "kernel": "attn_kernel_direct<8, false, false> (group_attn stage)",
        "achieved": attn_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": attn_traffic_bytes(wl.name),
        "algorithmic_flops_per_launch": attn_flops,
        "launch_ms": ms["group_attn"],
    }
    if lay:
        g = dict(frames=wl.frames, height=wl.height, width=wl.width,
                 shot_start=list(wl.shot_start), win_h=wl.win_h, win_w=wl.win_w,
                 t_group=wl.t_group, aug_frames=wl.aug_frames)
        pt = stga_pairs_closed_form(g)
        stages["stga_tflops"] = metrics.attention_flops(pt, h, hd) / (ms["stga"] / 1e3) / 1e12
        stages["stga_frac_of_bf16_peak"] = stages["stga_tflops"] / MFMA_BF16_PEAK_TFLOPS
    log(f"stages (ms): {ms}  attn {attn_tflops:.1f} TFLOP/s")
    return stages


def hybrid_overhead(args, wl, x, w, q, k, v, lay, ws, out, step):
    """What the two STGA branches add to the forward: each pass times the hybrid forward and
    the same forward without them (its MoGA epilogue then stores its rows without the mean),
    back to back, each enqueued whole by one library call; the median difference is the
    branches' launches plus the mean's extra reads in the MoGA epilogue.  (The stage
    breakdown times the branches alone, after the flush and an idle gap, where these
    few-millisecond launches start at a lower engine clock than inside a forward.)"""
    import numpy as np
    import torch

    from sparse_attention_long_moga_amd import api

    stream = torch.cuda.current_stream()
    evs = []
    for it in range(args.steps + 1):
        ea, eb, ec = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        ea.record(stream)
        step()
        eb.record(stream)
        api.moga_forward(x, w, q, k, v, wl.n_groups, alpha=wl.alpha, ws=ws, out=out)
        ec.record(stream)
        if it > 0:  # the first pair warms the plain forward's allocations
            evs.append((ea, eb, ec))
    torch.cuda.synchronize()
    d = [ea.elapsed_time(eb) - eb.elapsed_time(ec) for ea, eb, ec in evs]
    ms = float(np.median(d))
    log(f"hybrid forward over the MoGA-only forward: {ms:.3f} ms")
    return {"hybrid_over_moga_forward_ms": ms}


# The pages' group-count ablation for Wan2.1-1.3B at 10 s (papernotes.org MoGA note,
# 消融实验表格): sparsity and whole-model forward PFLOPs per M.
PAGES_MSWEEP = {1: (0.0, 0.88), 2: (0.4125, 0.59), 4: (0.6625, 0.42), 8: (0.7875, 0.36),
                16: (0.8125, 0.35)}
# Whole-model FLOPs in the pages' convention (their full-attention figures are reproduced by
# it): 30 attention layers at 4*hd*H FLOPs per (query, key) pair plus 2 * 1.3e9 parameters per
# token (Wan2.1-1.3B public sizes; the layer count and parameter count are not on the pages).
WAN13B_LAYERS, WAN13B_PARAMS = 30, 1.3e9


def backward(args):
    """Time moga_backward: D and dp, the row gathers, the dQ and dK/dV attention kernels, the
    inverse gathers and the router backward, with inputs and the forward's saved state
    resident in HBM.  On a STGA workload, moga_hybrid_backward: the same plus the per-frame
    and temporal branches' backward and the per-token sum of the three.  Attention FLOPs are
    counted two ways: the five products of the standard attention backward (S recomputed,
    dP, dV, dQ, dK: 10 hd per query-key pair and head) and what the two kernels execute (both
    compute S and dP: 14 hd)."""
    import numpy as np
    import torch

    import workloads
    from sparse_attention_long_moga_amd import api, metrics

    wl = workloads.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n, h, hd, m = wl.n_tokens, wl.n_heads, wl.head_dim, wl.n_groups
    log(f"backward {wl.name}: generating inputs")
    x, w = workloads.make_x(wl, dev), workloads.make_w(wl, dev)
    q, k, v = workloads.make_qkv(wl, dev)
    dout = workloads.make_dout(wl, dev)
    lay = None
    if wl.hybrid:
        lay = api.make_stga_layout(wl.frames, wl.height, wl.width, wl.shot_start, wl.win_h,
                                   wl.win_w, wl.t_group, wl.aug_frames)
    saved = api.moga_forward(x, w, q, k, v, m, alpha=wl.alpha, fused=True, with_lse=True,
                             stga=lay)
    dims = api.make_dims(n, wl.d_model, h, hd, m, alpha=wl.alpha)
    import ctypes
    from sparse_attention_long_moga_amd import _capi
    if lay:
        nb = _capi.load().moga_hybrid_backward_workspace_bytes(ctypes.byref(dims), lay.ref())
    else:
        nb = _capi.load().moga_backward_workspace_bytes(ctypes.byref(dims))
    ws = api.workspace(nb, dev)
    grads = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                 dx=torch.empty(n, wl.d_model, dtype=torch.float32, device=dev),
                 dw=torch.empty(wl.d_model, m, dtype=torch.float32, device=dev),
                 dp=torch.empty(n, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()

    def step():
        if lay:
            api.moga_hybrid_backward(x, w, q, k, v, saved, dout, lay, d_loss=1.0, alpha=wl.alpha,
                                     ws=ws, grads=grads)
        else:
            api.moga_backward(x, w, q, k, v, saved, dout, d_loss=1.0, alpha=wl.alpha, ws=ws,
                              grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} backward steps")
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    counts = saved["counts"].cpu().numpy().astype(np.int64)
    pairs = metrics.moga_pairs(counts)
    if lay:  # plus the temporal and per-frame branches' (query, key) pairs
        pairs += stga_pairs_closed_form(dict(
            frames=wl.frames, height=wl.height, width=wl.width, shot_start=list(wl.shot_start),
            win_h=wl.win_h, win_w=wl.win_w, t_group=wl.t_group, aug_frames=wl.aug_frames))
    fwd_flops = metrics.attention_flops(pairs, h, hd)  # 4 hd per pair and head
    algo, executed = 2.5 * fwd_flops, 3.5 * fwd_flops
    line = {
        "mode": "hybrid_backward" if lay else "backward", "workload": wl.name, "n_tokens": n,
        "n_groups": m,
        "group_sizes": counts.tolist(), "steps": args.steps, "warmup": args.warmup,
        "backward_ms": ms, "tokens_per_s": n / (ms / 1e3),
        "attn_bwd_tflop_algorithmic": algo / 1e12, "attn_bwd_tflop_executed": executed / 1e12,
        "whole_backward_tflops_algorithmic": algo / (ms / 1e3) / 1e12,
        "whole_backward_tflops_executed": executed / (ms / 1e3) / 1e12,
        "dtype": "bf16", "data": "synthetic",
    }
    print(json.dumps(line), flush=True)


def msweep(args):
    """Group-count sweep at the 10 s shape: for each M one JSON line with the routing's
    sparsity (1 - sum n_i^2 / N^2), attention FLOPs, forward and attention-stage times."""
    import numpy as np
    import torch

    import workloads
    from sparse_attention_long_moga_amd import api, metrics

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    for wl in workloads.MSWEEP:
        n, h, hd, m = wl.n_tokens, wl.n_heads, wl.head_dim, wl.n_groups
        log(f"msweep {wl.name}")
        x, w = workloads.make_x(wl, dev), workloads.make_w(wl, dev)
        q, k, v = workloads.make_qkv(wl, dev)
        dims = api.make_dims(n, wl.d_model, h, hd, m, alpha=wl.alpha)
        ws = api.workspace(api.moga_workspace_bytes(dims, None), dev)
        out = dict(out=torch.empty_like(q), loss=torch.empty(1, dtype=torch.float64, device=dev),
                   counts=torch.empty(m, dtype=torch.int32, device=dev))

        def fwd():
            api.moga_forward(x, w, q, k, v, m, alpha=wl.alpha, ws=ws, out=out)

        r = api.moga_route(x, w, m, ws=ws)
        cu, perm, (qp, kp, vp), pp = api.moga_permute(r["group_id"], [q, k, v], m,
                                                      p_sel=r["p_sel"], ws=ws)
        op = torch.empty_like(qp)

        def attn():
            api.moga_group_attn(qp, kp, vp, cu, cu, row_scale=pp, out=op, ws=ws)

        res = {}
        for name, fn in (("forward", fwd), ("attn", attn)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / args.steps
        counts = out["counts"].cpu().numpy().astype(np.int64)
        pairs = metrics.moga_pairs(counts)
        flops = metrics.attention_flops(pairs, h, hd)
        full = metrics.attention_flops(float(n) ** 2, h, hd)
        sparsity = 1.0 - pairs / float(n) ** 2
        model_pf = (WAN13B_LAYERS * flops + 2.0 * WAN13B_PARAMS * n) / 1e15
        page_sp, page_pf = PAGES_MSWEEP[m]
        line = {
            "mode": "msweep", "workload": wl.name, "n_tokens": n, "n_groups": m,
            "group_sizes": counts.tolist(), "sparsity": sparsity,
            "attn_tflop_per_layer": flops / 1e12, "full_attn_tflop_per_layer": full / 1e12,
            "model_pflops_estimate": model_pf,
            "pages": {"sparsity": page_sp, "pflops": page_pf},
            "steps": args.steps, "warmup": args.warmup,
            "forward_ms": res["forward"], "tokens_per_s": n / (res["forward"] / 1e3),
            "attn_ms": res["attn"], "attn_tflops": flops / (res["attn"] / 1e3) / 1e12,
            "attn_frac_of_bf16_peak": flops / (res["attn"] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "dtype": "bf16", "data": "synthetic",
        }
        print(json.dumps(line), flush=True)
        del x, w, q, k, v, ws, out, r, cu, perm, qp, kp, vp, pp, op
        torch.cuda.empty_cache()


def stga_pairs_closed_form(g):
    """Temporal + per-frame (query, key) pairs per head from the geometry."""
    starts = g["shot_start"]
    wt = g["win_h"] * g["win_w"]
    nwin = (g["height"] // g["win_h"]) * (g["width"] // g["win_w"])
    pairs = 0
    S = len(starts) - 1
    for s in range(S):
        length = starts[s + 1] - starts[s]
        nch = -(-length // g["t_group"])
        ap = min(g["aug_frames"], starts[s] - starts[s - 1]) if s > 0 else 0
        an = min(g["aug_frames"], starts[s + 2] - starts[s + 1]) if s + 1 < S else 0
        for c in range(nch):
            tf = min(g["t_group"], length - c * g["t_group"])
            kf = tf + (ap if c == 0 else 0) + (an if c == nch - 1 else 0)
            pairs += nwin * (tf * wt) * (kf * wt)
    hw = g["height"] * g["width"]
    return pairs + g["frames"] * hw * hw


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, x, w, q, k, v, target_s):
    """Oracle rate on a bounded sample: routing, groups and loss on every token, MoGA
    attention on seeded (head, token) rows, extrapolated by row count."""
    import numpy as np

    import oracle
    import workloads

    n, h, hd, m = wl.n_tokens, wl.n_heads, wl.head_dim, wl.n_groups
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    log(f"cpu baseline: oracle with {threads} threads")
    xh = x.float().cpu().numpy()
    wh = w.cpu().numpy()
    t0 = time.perf_counter()
    r = oracle.route(xh, wh)
    cu, perm = oracle.groups(r["group_id"], m)
    oracle.balance_loss(r["counts"], r["prob_sum"], n, wl.alpha)
    t_route = time.perf_counter() - t0
    del xh
    heads = [0, h - 1] if h > 1 else [0]
    qh = np.stack([q[i].float().cpu().numpy() for i in heads])
    kh = np.stack([k[i].float().cpu().numpy() for i in heads])
    vh = np.stack([v[i].float().cpu().numpy() for i in heads])
    scale = 1.0 / np.sqrt(hd)
    # calibrate on a few rows, then size the sample to the CPU-time target
    rows = 64
    used = 0.0
    timed_rows = 0
    seed = 0
    while True:
        rt = workloads.random_rows(n, rows, 1000 + seed)
        rh = np.arange(rt.shape[0]) % len(heads)
        t1 = time.perf_counter()
        oracle.moga_attn(qh, kh, vh, r["group_id"], m, r["p_sel"], scale, rh, rt)
        dt = time.perf_counter() - t1
        used += dt
        timed_rows += rt.shape[0]
        seed += 1
        remaining = target_s - t_route - used
        if remaining <= 0.5 or timed_rows >= n:
            break
        rows = int(min(n, max(64, rows * remaining / max(dt, 1e-3) * 0.8)))
    per_row = used / timed_rows
    total = t_route + per_row * h * n
    return {
        "value": n / total, "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"route + groups + loss on all {n} tokens ({t_route:.1f} s); MoGA attention "
                   f"on {timed_rows} seeded (head, token) rows of {h * n} ({used:.1f} s), "
                   f"extrapolated by row count to {total:.0f} s for the whole forward"),
        "measured_s": t_route + used,
    }


if __name__ == "__main__":
    main()
