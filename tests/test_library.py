"""The C-ABI library: it builds, loads, exports what include/moga.h declares, and its
argument checks return the documented status before touching a GPU (CPU only)."""
import ctypes
import os
import re

import pytest

from sparse_attention_long_moga_amd import _capi
from sparse_attention_long_moga_amd.api import make_dims, make_stga_layout, moga_workspace_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_capi.LIB_PATH):
        from sparse_attention_long_moga_amd import build
        build.build(verbose=False)
    return _capi.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "moga.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:moga|stga)_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree(lib):
    names = declared_functions()
    assert names == sorted(_capi.EXPORTS)
    for n in names:
        assert hasattr(lib, n), f"libmoga.so does not export {n}"


def test_exports_are_c_symbols(lib):
    for n in _capi.EXPORTS:
        ctypes.cast(getattr(lib, n), ctypes.c_void_p)  # resolvable by its plain C name


def _dims(**kw):
    base = dict(n_tokens=4096, d_model=256, n_heads=4, head_dim=64, n_groups=4)
    base.update(kw)
    return make_dims(**base)


@pytest.mark.parametrize("kw, msg", [
    (dict(n_tokens=0), "n_tokens"), (dict(n_tokens=1 << 31), "n_tokens"),
    (dict(head_dim=96), "head_dim"), (dict(n_groups=0), "n_groups"),
    (dict(n_groups=65), "n_groups"), (dict(n_heads=0), "n_heads"), (dict(d_model=0), "d_model"),
    (dict(d_model=(1 << 20) + 8), "d_model"),
    (dict(n_tokens=1 << 30, n_heads=256), "work items"),
])
def test_bad_dims_rejected(lib, kw, msg):
    d = _dims(**kw)
    st = lib.moga_route(ctypes.c_void_p(16), 0, ctypes.c_void_p(16), None, ctypes.byref(d),
                        ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                        ctypes.c_void_p(16), ctypes.c_void_p(256), 1 << 30, None)
    assert st == _capi.MOGA_ERR_ARG
    assert msg in lib.moga_last_error().decode()
    assert lib.moga_workspace_bytes(ctypes.byref(d), None) == 0


def test_null_and_workspace_errors(lib):
    d = _dims()
    p = ctypes.c_void_p(256)
    assert lib.moga_route(None, 0, p, None, ctypes.byref(d), p, p, p, p, p, 1 << 30, None) == \
        _capi.MOGA_ERR_ARG
    assert lib.moga_route(p, 0, p, None, ctypes.byref(d), p, p, p, p, None, 0, None) == \
        _capi.MOGA_ERR_WORKSPACE
    assert lib.moga_route(p, 0, p, None, ctypes.byref(d), p, p, p, p, p, 16, None) == \
        _capi.MOGA_ERR_WORKSPACE
    assert "workspace" in lib.moga_last_error().decode()
    # misaligned x, odd d_model for bf16
    assert lib.moga_route(ctypes.c_void_p(258), 0, p, None, ctypes.byref(d), p, p, p, p, p,
                          1 << 30, None) == _capi.MOGA_ERR_ARG
    d2 = _dims(d_model=260)
    assert lib.moga_route(p, 1, p, None, ctypes.byref(d2), p, p, p, p, p, 1 << 30, None) == \
        _capi.MOGA_ERR_UNSUPPORTED
    # permute: too many tensors, aliasing
    src = (ctypes.c_void_p * 4)(256, 512, 768, 1024)
    assert lib.moga_permute(0, p, ctypes.byref(d), p, p, src, src, 5, None, None, p, 1 << 30,
                            None) == _capi.MOGA_ERR_ARG
    assert lib.moga_permute(0, p, ctypes.byref(d), p, p, src, src, 1, None, None, p, 1 << 30,
                            None) == _capi.MOGA_ERR_ARG
    assert "aliases" in lib.moga_last_error().decode()
    # group attention: no segments
    assert lib.moga_group_attn(p, p, p, 10, 10, 0, p, p, None, ctypes.byref(d), p, p, 1 << 20,
                               None) == _capi.MOGA_ERR_ARG


def test_stga_geometry_checks(lib):
    n = 4 * 6 * 8
    d = _dims(n_tokens=n)
    ok = make_stga_layout(4, 6, 8, [0, 2, 4], 3, 4, 2, 2)
    assert moga_workspace_bytes(d, ok) > moga_workspace_bytes(d)
    bad = [make_stga_layout(4, 6, 8, [0, 2, 3], 3, 4, 2, 2),   # does not end at frames
           make_stga_layout(4, 6, 8, [0, 2, 2, 4], 3, 4, 2, 2),  # not strictly increasing
           make_stga_layout(4, 6, 8, [0, 4], 4, 4, 2, 2),        # window does not tile 6 rows
           make_stga_layout(4, 6, 8, [0, 4], 3, 4, 0, 2),        # t_group < 1
           make_stga_layout(4, 6, 8, [0, 4], 3, 4, 2, -1),       # aug < 0
           make_stga_layout(5, 6, 8, [0, 5], 3, 4, 2, 2)]        # 5*6*8 != n_tokens
    p = ctypes.c_void_p(256)
    for lay in bad:
        assert lib.moga_workspace_bytes(ctypes.byref(d), lay.ref()) == 0
        assert lib.stga_group_attn(p, p, p, ctypes.byref(d), lay.ref(), p, p, p, 1 << 40,
                                   None) == _capi.MOGA_ERR_ARG


def test_stga_work_list_bound(lib):
    # one-token windows and one-frame chunks make every token its own group: with two heads
    # the attention work list would pass 2^31 items, so the layout is refused up front
    f, h, w = 1 << 14, 256, 256
    d = _dims(n_tokens=f * h * w, n_heads=2)
    lay = make_stga_layout(f, h, w, [0, f], 1, 1, 1, 0)
    assert lib.moga_workspace_bytes(ctypes.byref(d), lay.ref()) == 0
    assert "work items" in lib.moga_last_error().decode()
    assert lib.moga_workspace_bytes(ctypes.byref(d), None) > 0


def test_workspace_sizes_scale_with_problem(lib):
    small = moga_workspace_bytes(_dims())
    big = moga_workspace_bytes(_dims(n_tokens=8192))
    assert big > small > 3 * 4 * 4096 * 64 * 2  # at least the permuted Q/K/V


def test_no_device_reported_as_unsupported(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    d = _dims()
    p = ctypes.c_void_p(256)
    st = lib.moga_balance_loss(p, p, ctypes.byref(d), p, None, None, None)
    assert st == _capi.MOGA_ERR_UNSUPPORTED


def test_backward_argument_checks(lib):
    """moga_backward validates before touching a GPU: NULL pointers, alignment, workspace."""
    from sparse_attention_long_moga_amd._capi import MogaGrads, MogaInputs, MogaSaved
    p = 256
    ins = MogaInputs(p, 1, p, p, p, p, None)
    sav = MogaSaved(p, p, p, p, p, p, p)
    gr = MogaGrads(p, p, p, None, None, None)
    d128 = _dims(head_dim=128)
    ws = lib.moga_backward_workspace_bytes(ctypes.byref(d128))
    assert ws > lib.moga_workspace_bytes(ctypes.byref(d128), None)  # seven group-order tensors
    call = lambda d, i=ins, s=sav, g=gr, dout=p, w=ws, wsp=p: lib.moga_backward(
        ctypes.byref(i) if i else None, ctypes.byref(s) if s else None, dout, 0.5,
        ctypes.byref(d), ctypes.byref(g) if g else None, wsp, w, None)
    # head_dim 64 runs on the same 128-channel buffers
    assert lib.moga_backward_workspace_bytes(ctypes.byref(_dims(head_dim=64))) == ws
    assert call(d128, s=None) == _capi.MOGA_ERR_ARG
    assert call(d128, dout=None) == _capi.MOGA_ERR_ARG
    assert call(d128, s=MogaSaved(p, p, p, p, p, p, None)) == _capi.MOGA_ERR_ARG  # no lse
    assert "saved" in lib.moga_last_error().decode()
    assert call(d128, g=MogaGrads(p, None, p, None, None, None)) == _capi.MOGA_ERR_ARG
    assert call(d128, dout=258) == _capi.MOGA_ERR_ARG  # misaligned
    assert call(d128, w=16) == _capi.MOGA_ERR_WORKSPACE
    assert call(d128, wsp=None) == _capi.MOGA_ERR_WORKSPACE
    assert lib.moga_backward_workspace_bytes(ctypes.byref(_dims(n_groups=0))) == 0


def test_hybrid_forward_lse_needs_branches(lib):
    """With a STGA layout lse holds the three branches' normalisers, which pair with the
    branch rows: asked for without o_branches the forward is refused before any launch, and
    o_branches without a STGA layout is an argument error."""
    from sparse_attention_long_moga_amd._capi import MogaInputs, MogaOutputs
    n = 4 * 6 * 8
    d = _dims(n_tokens=n)
    lay = make_stga_layout(4, 6, 8, [0, 2, 4], 3, 4, 2, 2)
    p = 256
    ins = MogaInputs(p, 1, p, p, p, p, None)
    outs = MogaOutputs(p, p, None, None, None, None, None, None, p, None)
    branches_only = MogaOutputs(p, p, None, None, None, None, None, None, None, p)
    for fn in (lib.moga_forward, lib.moga_forward_fused):
        st = fn(ctypes.byref(ins), ctypes.byref(d), lay.ref(), ctypes.byref(outs),
                ctypes.c_void_p(256), 1 << 40, None)
        assert st == _capi.MOGA_ERR_UNSUPPORTED
        assert "o_branches" in lib.moga_last_error().decode()
        st = fn(ctypes.byref(ins), ctypes.byref(d), None, ctypes.byref(branches_only),
                ctypes.c_void_p(256), 1 << 40, None)
        assert st == _capi.MOGA_ERR_ARG
        assert "STGA" in lib.moga_last_error().decode()


def test_hybrid_backward_argument_checks(lib):
    """moga_hybrid_backward validates before touching a GPU: the layout, NULL
    pointers, workspace; its workspace covers the temporal branch's borrowed key rows."""
    from sparse_attention_long_moga_amd._capi import MogaGrads, MogaInputs, MogaSaved
    n = 6 * 8 * 16
    lay = make_stga_layout(6, 8, 16, [0, 3, 6], 4, 8, 2, 2)
    p = 256
    ins = MogaInputs(p, 1, p, p, p, p, None)
    sav = MogaSaved(p, p, p, p, p, p, p)
    gr = MogaGrads(p, p, p, None, None, None)
    d128 = _dims(n_tokens=n, head_dim=128)
    ws = lib.moga_hybrid_backward_workspace_bytes(ctypes.byref(d128), lay.ref())
    assert ws > lib.moga_backward_workspace_bytes(ctypes.byref(d128))
    assert lib.moga_hybrid_backward_workspace_bytes(ctypes.byref(_dims(n_tokens=n)), lay.ref()) == ws
    assert lib.moga_hybrid_backward_workspace_bytes(ctypes.byref(d128), None) == 0
    call = lambda d, i=ins, s=sav, g=gr, dout=p, w=ws, wsp=p, st=lay.ref(): \
        lib.moga_hybrid_backward(ctypes.byref(i) if i else None, ctypes.byref(s) if s else None,
                                 st, dout, 0.5, ctypes.byref(d), ctypes.byref(g) if g else None,
                                 wsp, w, None)
    assert call(d128, st=None) == _capi.MOGA_ERR_ARG
    assert "stga" in lib.moga_last_error().decode()
    bad = make_stga_layout(6, 8, 16, [0, 3, 6], 3, 8, 2, 2)  # 3 rows do not tile 8
    assert call(d128, st=bad.ref()) == _capi.MOGA_ERR_ARG
    assert call(d128, s=MogaSaved(p, p, p, p, p, None, p)) == _capi.MOGA_ERR_ARG  # no branches
    assert call(d128, dout=None) == _capi.MOGA_ERR_ARG
    assert call(d128, w=ws - 1) == _capi.MOGA_ERR_WORKSPACE
