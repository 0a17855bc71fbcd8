"""Seeded synthetic inputs for the MoGA / STGA forward path.

This module only draws random tensors of the shapes, dtypes and structure of
the workloads; it holds none of the method's arithmetic.  Both the HIP path
(through the package) and the CPU oracle consume what it returns, so it is the
one piece of code the two sides share.

Recipe (the sizes come from the MoGA pages: 1560 tokens per latent frame at
480p after the (4,8,8) VAE and (1,2,2) patchify, xugj520.cn MoGA blog §3.1;
Wan2.1-like widths; 1-minute MMDiT scale from the papernotes.org MoGA note,
实验关键数据):

* x is a mixture of Gaussians around unit-norm centres c_1..c_M with sigma 0.5,
  and the router weight W is [c_1 ... c_M].  The pages describe the router's
  weights as implicit cluster centres (papernotes.org note, 核心 idea; blog
  §2.3), so this is the plainest synthetic stand-in for a trained router.
* Mixture weights are uniform, or Dirichlet(0.5) for the skewed workload.
* Q, K, V ~ N(0, 1), stored bf16, layout [H][N][hd].
* The tiny workload draws x ~ N(0,1) fp32 and W ~ N(0, 1/d) instead.

Small parameters (centres, mixture weights, W) are drawn on the host with
NumPy PCG64; large tensors are drawn with a seeded torch.Generator on the
target device.  The oracle never regenerates: it is given host copies of the
exact tensors the device consumed.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

TOKENS_PER_FRAME = 30 * 52  # 480x832 latent grid after VAE (8x) and patchify (2x)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int
    d_model: int
    n_heads: int
    head_dim: int
    n_groups: int
    alpha: float = 0.1
    x_dtype: str = "bf16"          # "f32" or "bf16"
    mixture: str = "gaussian"      # "gaussian" (W = centres) or "normal" (x, W iid normal)
    dirichlet: Optional[float] = None  # concentration for skewed mixture weights
    sigma: float = 0.5
    seed: int = 0
    # STGA geometry (None -> MoGA only)
    frames: Optional[int] = None
    height: Optional[int] = None
    width: Optional[int] = None
    shot_start: Optional[tuple] = None
    win_h: int = 0
    win_w: int = 0
    t_group: int = 0
    aug_frames: int = 0

    @property
    def hybrid(self) -> bool:
        return self.shot_start is not None

    def describe(self) -> dict:
        d = {"workload": self.name, "n_tokens": self.n_tokens, "d_model": self.d_model,
             "n_heads": self.n_heads, "head_dim": self.head_dim, "n_groups": self.n_groups,
             "x_dtype": self.x_dtype, "seed": self.seed}
        if self.dirichlet is not None:
            d["mixture_weights"] = f"Dirichlet({self.dirichlet})"
        if self.hybrid:
            d.update(grid=[self.frames, self.height, self.width],
                     shots=len(self.shot_start) - 1, window=[self.win_h, self.win_w],
                     t_group=self.t_group, aug_frames=self.aug_frames)
        return d


def even_shots(frames: int, n_shots: int) -> tuple:
    """Shot s covers latent frames [floor(frames*s/S), floor(frames*(s+1)/S))."""
    return tuple((frames * s) // n_shots for s in range(n_shots + 1))


# The five workloads.  Seeds are fixed here once and never re-chosen.
TINY = Workload("tiny_fp32_N4096_M4", 4096, 256, 4, 64, 4, x_dtype="f32", mixture="normal",
                seed=1)
WAN5S = Workload("wan1.3b_5s_N32760_M5", 21 * TOKENS_PER_FRAME, 1536, 12, 128, 5, seed=2,
                 frames=None)
WAN30S_SKEW = Workload("wan1.3b_30s_skewed_N282360_M5", 181 * TOKENS_PER_FRAME, 1536, 12, 128,
                       5, dirichlet=0.5, seed=3)
WAN30S_HYBRID = dataclasses.replace(
    WAN30S_SKEW, name="wan1.3b_30s_hybrid_N282360_M5_stga",
    frames=181, height=30, width=52, shot_start=even_shots(181, 9),
    win_h=15, win_w=13, t_group=4, aug_frames=2)
MMDIT60S = Workload("mmdit_60s_N563160_M20_stga", 361 * TOKENS_PER_FRAME, 5120, 40, 128, 20,
                    seed=5, frames=361, height=30, width=52, shot_start=even_shots(361, 18),
                    win_h=15, win_w=13, t_group=4, aug_frames=2)

CONFIGS: List[Workload] = [TINY, WAN5S, WAN30S_SKEW, WAN30S_HYBRID, MMDIT60S]

# Group-count sweep at the 10 s shape (40 latent frames, N = 62,400) of the pages' M ablation
# (papernotes.org MoGA note, 消融实验表格): MoGA only, uniform mixture, one seed per M.
MSWEEP_M = (1, 2, 4, 8, 16)
MSWEEP: List[Workload] = [
    Workload(f"wan1.3b_10s_N62400_M{m}", 40 * TOKENS_PER_FRAME, 1536, 12, 128, m, seed=100 + m)
    for m in MSWEEP_M]

BY_NAME = {w.name: w for w in CONFIGS + MSWEEP}


def small(name: str, n_tokens: int, d_model: int, n_heads: int, head_dim: int, n_groups: int,
          seed: int, **kw) -> Workload:
    """A reduced workload with the same recipe, for parity tests."""
    return Workload(name, n_tokens, d_model, n_heads, head_dim, n_groups, seed=seed, **kw)


def router_params(wl: Workload):
    """Host-side small parameters: (W [d][M] fp32, centres [M][d] or None, weights [M])."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    if wl.mixture == "normal":
        w = rng.standard_normal((wl.d_model, wl.n_groups)) / np.sqrt(wl.d_model)
        return w.astype(np.float32), None, None
    c = rng.standard_normal((wl.n_groups, wl.d_model))
    c /= np.linalg.norm(c, axis=1, keepdims=True)
    if wl.dirichlet is not None:
        weights = rng.dirichlet(np.full(wl.n_groups, wl.dirichlet))
    else:
        weights = np.full(wl.n_groups, 1.0 / wl.n_groups)
    return np.ascontiguousarray(c.T).astype(np.float32), c.astype(np.float32), weights


def make_x(wl: Workload, device="cpu") -> torch.Tensor:
    """Router input x [N][d] (fp32 or bf16) on `device`."""
    w, centres, weights = router_params(wl)
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000 + 11)
    n, d = wl.n_tokens, wl.d_model
    if wl.mixture == "normal":
        x = torch.randn((n, d), generator=g, device=device, dtype=torch.float32)
    else:
        wt = torch.tensor(weights, dtype=torch.float64, device=device)
        z = torch.multinomial(wt, n, replacement=True, generator=g)
        c = torch.tensor(centres, device=device)
        x = torch.empty((n, d), device=device, dtype=torch.float32)
        step = 1 << 16
        for a in range(0, n, step):
            b = min(n, a + step)
            x[a:b] = c[z[a:b]] + wl.sigma * torch.randn((b - a, d), generator=g, device=device)
    return x if wl.x_dtype == "f32" else x.to(torch.bfloat16)


def make_w(wl: Workload, device="cpu") -> torch.Tensor:
    return torch.from_numpy(router_params(wl)[0]).to(device)


def make_qkv(wl: Workload, device="cpu", n_heads: Optional[int] = None):
    """Q, K, V ~ N(0,1) as bf16 [H][N][hd] on `device`."""
    h = wl.n_heads if n_heads is None else n_heads
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000 + 23)
    shape = (h, wl.n_tokens, wl.head_dim)
    return tuple(torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)
                 for _ in range(3))


def make_dout(wl: Workload, device="cpu", n_heads: Optional[int] = None) -> torch.Tensor:
    """Gradient arriving at the attention output: N(0,1) as bf16 [H][N][hd] on `device`."""
    h = wl.n_heads if n_heads is None else n_heads
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000 + 37)
    return torch.randn((h, wl.n_tokens, wl.head_dim), generator=g, device=device,
                       dtype=torch.bfloat16)


def random_rows(n: int, k: int, seed: int) -> np.ndarray:
    """k distinct sorted indices in [0, n), seeded (for sampled parity checks)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(n, size=min(k, n), replace=False)).astype(np.int64)
