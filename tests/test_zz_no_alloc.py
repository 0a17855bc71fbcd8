"""moga_group_attn_noalloc: the group attention with its plan in the library's static scratch
instead of a caller workspace.  Two calls in a row through the C ABI (the second smaller, so it
runs on whatever the first left in the scratch) must give bitwise the outputs moga_group_attn
gives on the same inputs; sizes beyond the scratch are refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_attention_long_moga_amd import _capi, api
from sparse_attention_long_moga_amd.api import make_dims

DEV = "cuda:0"


def _segments(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _inputs(ql, kl, h, hd, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    cu_q, cu_k = _segments(ql), _segments(kl)
    lq, lk = int(cu_q[-1]), int(cu_k[-1])
    q = torch.randn((h, lq, hd), generator=g, device=DEV, dtype=torch.bfloat16)
    k = torch.randn((h, lk, hd), generator=g, device=DEV, dtype=torch.bfloat16)
    v = torch.randn((h, lk, hd), generator=g, device=DEV, dtype=torch.bfloat16)
    rs = torch.rand(lq, generator=g, device=DEV, dtype=torch.float32) + 0.5
    return (q, k, v, torch.from_numpy(cu_q).to(DEV), torch.from_numpy(cu_k).to(DEV), rs)


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point():
    rng = np.random.Generator(np.random.PCG64(5))
    cases = [
        # long segments (256-row items); the last items of the launch split into key ranges,
        # so the split parts' rows live in the scratch too; one segment has no keys
        ("split_tail", np.array([20000, 9000, 3000, 1300, 300]),
         np.array([20000, 9050, 3000, 2500, 0]), 2, 128),
        # the smaller second call: short segments (128-row items), q != k lengths
        ("short", rng.integers(0, 700, 30), rng.integers(1, 900, 30), 1, 128),
    ]
    got, inputs = [], []
    for name, ql, kl, h, hd in cases:
        print(f"[case] noalloc {name} h={h} rows={int(ql.sum())}", flush=True)
        args = _inputs(ql, kl, h, hd, seed=len(name))
        out = torch.full_like(args[0], 3.0)
        api.moga_group_attn_noalloc(*args[:5], row_scale=args[5], out=out)
        got.append(out)
        inputs.append(args)
    torch.cuda.synchronize()
    for (name, *_), args, out in zip(cases, inputs, got):
        ref = api.moga_group_attn(*args[:5], row_scale=args[5])
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{name}: noalloc output differs from moga_group_attn"
        assert torch.isfinite(out.float()).all()


def test_noalloc_refuses_sizes_beyond_its_scratch():
    lib = _capi.load()
    d = make_dims(1 << 30, 1, 64, 128, 1)
    p = ctypes.c_void_p(256)
    st = lib.moga_group_attn_noalloc(p, p, p, 1 << 30, 1 << 30, 1, p, p, None, ctypes.byref(d), p,
                                     None)
    assert st == _capi.MOGA_ERR_WORKSPACE
    assert "static scratch" in lib.moga_last_error().decode()
    # and the ordinary argument checks still come first
    st = lib.moga_group_attn_noalloc(None, p, p, 10, 10, 1, p, p, None, ctypes.byref(d), p, None)
    assert st == _capi.MOGA_ERR_ARG
