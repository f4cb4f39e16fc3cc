"""Seeded synthetic inputs for the VSA attention path.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds none of the method's arithmetic: no cube tiling, no pooling,
no scoring, no top-k and no attention. It only draws q, k, v in the natural
(T, H, W) token order, in the layout (B, T*H*W, NH, D), and rounds them to bf16.
Each side tiles them with its own code.

What the draws stand in for: the Wan2.2 Production Values dataset card ("VSA
Block-Sparse Attention Inputs + Reference") benchmarks the fine stage on four
captured Wan2.2-A14B attention calls of shape (1, 39936, 40, 128), one of them
an outlier head whose logits overflow a softmax computed without row-max
subtraction. Those captures are not available, so these generators reproduce
their shapes, dtype and the structure the card asks for instead: heavy-tailed
q/k rather than small-magnitude N(0,1), per-head distinct spatially local
selections (a smooth field shared by q and k of a head), partial cubes at the
grid edges, and one head whose logits reach about +-2000.

The recipe (all choices of this implementation; the pages fix none of them):

* numpy PCG64 ``default_rng(seed)``; everything drawn in float32, then rounded
  to bf16 with round-to-nearest-even.
* ``field``: per head, M = 16 modes with wavevector n_m uniform over
  {-2..2}^3 without 0 (cycles per grid extent) and phase U[0, 2pi):
  g_m(t, y, x) = cos(2pi (n_t t/T + n_y y/H + n_x x/W) + phi_m);
  f_h = W_h g with W_h in R^{D x M} ~ N(0, 1); each channel rescaled to peak
  |f| = 2. q and k of a head share f_h and get independent N(0, 1) noise.
* ``heavy``: every (tensor in {q, k}, head, channel) is multiplied by an
  independent |t_3| (Student-t, nu = 3).
* ``outlier``: one head h* = rng.integers(NH) has q and k scaled by
  alpha = sqrt(2000 / max|logit|), the max taken over a 4096 x 4096 sample of
  that head's logits q.k/sqrt(D), so its logits reach about +-2000.
* v ~ N(0, 1) everywhere.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Case",
    "CONFIGS",
    "bf16_bits_from_f32",
    "make_case",
    "tiny",
    "small",
    "wan",
    "hy720",
]


@dataclasses.dataclass
class Case:
    """One seeded input set in natural token order.

    q, k, v are uint16 arrays holding bf16 bit patterns, shape (B, T*H*W, NH, D).
    """

    name: str
    B: int
    T: int
    H: int
    W: int
    NH: int
    D: int
    topk: int
    seed: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    outlier_head: int = -1
    outlier_alpha: float = 1.0

    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return bits.

    torch's CPU float32 -> bfloat16 conversion rounds to nearest even; inputs
    are finite by construction.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _field(rng: np.random.Generator, T: int, H: int, W: int, D: int,
           modes: int = 16, amplitude: float = 2.0) -> np.ndarray:
    """Smooth low-frequency 3D field for one head, shape (T*H*W, D), float32."""
    n = rng.integers(-2, 3, size=(modes, 3))
    bad = ~np.any(n != 0, axis=1)
    while bad.any():  # redraw zero wavevectors only
        n[bad] = rng.integers(-2, 3, size=(int(bad.sum()), 3))
        bad = ~np.any(n != 0, axis=1)
    phi = rng.uniform(0.0, 2.0 * math.pi, size=modes)
    t = np.arange(T, dtype=np.float64)[:, None, None] / T
    y = np.arange(H, dtype=np.float64)[None, :, None] / H
    x = np.arange(W, dtype=np.float64)[None, None, :] / W
    g = np.empty((modes, T * H * W), dtype=np.float64)
    for m in range(modes):
        arg = 2.0 * math.pi * (n[m, 0] * t + n[m, 1] * y + n[m, 2] * x) + phi[m]
        g[m] = np.cos(arg).reshape(-1)
    Wm = rng.standard_normal((D, modes))
    f = Wm @ g  # (D, N)
    peak = np.max(np.abs(f), axis=1, keepdims=True)
    peak[peak == 0] = 1.0
    f *= amplitude / peak
    return np.ascontiguousarray(f.T.astype(np.float32))


def make_case(name: str, *, B: int, T: int, H: int, W: int, NH: int, D: int,
              topk: int, seed: int, qk: str, heavy: bool, outlier: bool) -> Case:
    """Draw one input set.

    qk = "normal": q, k ~ N(0, 1); qk = "field": field + N(0, 1) noise.
    """
    rng = np.random.default_rng(seed)
    N = T * H * W
    q = np.empty((B, N, NH, D), dtype=np.float32)
    k = np.empty((B, N, NH, D), dtype=np.float32)
    for b in range(B):
        if qk == "normal":
            q[b] = rng.standard_normal((N, NH, D), dtype=np.float32)
            k[b] = rng.standard_normal((N, NH, D), dtype=np.float32)
        elif qk == "field":
            for h in range(NH):
                f = _field(rng, T, H, W, D)
                q[b, :, h, :] = f + rng.standard_normal((N, D), dtype=np.float32)
                k[b, :, h, :] = f + rng.standard_normal((N, D), dtype=np.float32)
        else:
            raise ValueError(qk)
    if heavy:
        sq = np.abs(rng.standard_t(3, size=(B, 1, NH, D))).astype(np.float32)
        sk = np.abs(rng.standard_t(3, size=(B, 1, NH, D))).astype(np.float32)
        q *= sq
        k *= sk
    h_star, alpha = -1, 1.0
    if outlier:
        h_star = int(rng.integers(NH))
        rows = min(4096, N)
        iq = rng.choice(N, size=rows, replace=False)
        ik = rng.choice(N, size=rows, replace=False)
        qs = q[0, iq, h_star, :].astype(np.float64)
        ks = k[0, ik, h_star, :].astype(np.float64)
        peak = float(np.max(np.abs(qs @ ks.T))) / math.sqrt(D)
        alpha = math.sqrt(2000.0 / peak)
        q[:, :, h_star, :] *= np.float32(alpha)
        k[:, :, h_star, :] *= np.float32(alpha)
    v = rng.standard_normal((B, N, NH, D), dtype=np.float32)
    return Case(name=name, B=B, T=T, H=H, W=W, NH=NH, D=D, topk=topk, seed=seed,
                q=bf16_bits_from_f32(q), k=bf16_bits_from_f32(k),
                v=bf16_bits_from_f32(v), outlier_head=h_star,
                outlier_alpha=alpha)


# The five workloads: a tiny case for exhaustive checks, the 12-head smooth-field
# case, the Wan2.2-A14B shape (the dataset card's "Shapes" table: q,k,v
# (1, 39936, 40, 128), topk 78 of 624 cubes, grid 21x30x52), and the 720p
# HunyuanVideo-like grid 30x48x80 (115,200 tokens; FastVideo STA guide,
# "The 115K Token Sequence Wall").
CONFIGS = {
    "tiny": dict(B=1, T=5, H=6, W=7, NH=2, D=64, topk=3, seed=0,
                 qk="normal", heavy=False, outlier=False),
    "small": dict(B=1, T=21, H=30, W=52, NH=12, D=128, topk=187, seed=1,
                  qk="field", heavy=False, outlier=False),
    "wan": dict(B=1, T=21, H=30, W=52, NH=40, D=128, topk=78, seed=2,
                qk="field", heavy=True, outlier=True),
    "hy720": dict(B=1, T=30, H=48, W=80, NH=24, D=128, topk=192, seed=4,
                  qk="field", heavy=True, outlier=True),
}

# top-k values of the sparsity sweep on the Wan shape: 0/50/70/87.5/95 % sparse
SWEEP_TOPK = (624, 312, 187, 78, 31)


def tiny() -> Case:
    return make_case("tiny", **CONFIGS["tiny"])


def small() -> Case:
    return make_case("small", **CONFIGS["small"])


def wan() -> Case:
    return make_case("wan", **CONFIGS["wan"])


def hy720() -> Case:
    return make_case("hy720", **CONFIGS["hy720"])
