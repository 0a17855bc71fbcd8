"""Shared helpers for the parity tests."""
import numpy as np
import torch

# Floating-point bar for bf16 attention outputs against the fp64 oracle.
MAX_ABS = 2e-2
REL_RMS = 1e-2


def rel_rms(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.sqrt(np.mean(ref * ref))
    return float(np.sqrt(np.mean((a - ref) ** 2)) / den) if den > 0 else float(
        np.sqrt(np.mean(a * a)))


def assert_close_bf16(out, ref, what="", max_abs=MAX_ABS, rrms=REL_RMS):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref).max() if out.size else 0.0
    r = rel_rms(out, ref)
    assert err <= max_abs, f"{what}: max-abs error {err:.3e} > {max_abs}"
    assert r <= rrms, f"{what}: relative RMS {r:.3e} > {rrms}"
    return err, r


def assert_close_per_group(out, ref, keys, what="", rrms=REL_RMS, min_rows=1):
    """Relative RMS per label of `keys` (one label per row, e.g. (head, group) pairs encoded
    as integers): the outputs of a large group are small (a softmax over many keys averages
    the values down), so a global figure can hide an error confined to one group."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    keys = np.asarray(keys)
    worst = 0.0
    for key in np.unique(keys):
        sel = keys == key
        if sel.sum() < min_rows:
            continue
        r = rel_rms(out[sel], ref[sel])
        worst = max(worst, r)
        assert r <= rrms, f"{what}: relative RMS {r:.3e} > {rrms} for label {key}"
    return worst


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()
