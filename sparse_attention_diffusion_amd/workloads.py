"""Seeded synthetic workloads shaped like the attention layers the MC-Sparse pages evaluate.

This module only draws random inputs and describes workload shapes; it contains
none of the method's arithmetic (no grouping, selection or attention).  Both the
fp64 oracle tests and the GPU path take their inputs from here.

Recipe (the pages give no data, so these stand in for DiT latents of the video
models named in the MC-Sparse summary page, results paragraphs; see the
workload table below):

* Tokens sit on a (T, Y, X) latent grid, token id n = (t*Y + y)*X + x, with
  integer grid coordinates.
* Per head h: W_h ~ N(0, sigma^-2) of shape (3, D) with sigma = 1 grid unit,
  b_h ~ U[0, 2*pi) of shape (D,), features f = sqrt(2) * cos(coords @ W_h + b_h)
  (random Fourier features: unit variance per component, RBF kernel in space).
* Q = f + N(0, 0.5^2), K = f + N(0, 0.5^2) (same f, independent noise),
  V ~ N(0, 1).  Q/K are stored unscaled; the softmax scale is 1/sqrt(D).
* Drift across denoising steps is a cumulative random walk
  X_t = X_{t-1} + N(0, sigma_d^2) for X in {Q, K, V}, applied before rounding.
* Storage: fp32, or rounded once (round-to-nearest-even) to bf16.

Host arrays come from numpy PCG64 streams keyed by
SeedSequence([seed, layer, head, tensor, step]); tensor 0 = features,
1 = Q noise, 2 = K noise, 3 = V.  Large workloads are drawn on the GPU with a
torch generator instead (same distributions, different streams), see
``make_qkv_torch``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

TENSOR_FEAT, TENSOR_QNOISE, TENSOR_KNOISE, TENSOR_V = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    grid: tuple          # (T, Y, X)
    heads: int
    head_dim: int
    dtype: str           # "f32" | "bf16"
    group: int           # C
    densities: tuple     # rho values
    seed: int
    drift_sigma: float
    reuse_steps: int
    layers: int = 1
    steps: int = 1
    notes: str = ""

    @property
    def n(self) -> int:
        t, y, x = self.grid
        return t * y * x

    @property
    def groups(self) -> int:
        return -(-self.n // self.group)

    def topk(self, rho: float) -> int:
        """Keys kept per group: K = round(rho * N), at least 1, at most N."""
        return int(min(self.n, max(1, int(math.floor(rho * self.n + 0.5)))))


# The five workloads: a tiny single-head case, three single-layer shapes after the
# Wan2.1-1.3B 480p / Wan2.1-14B 720p / HunyuanVideo-13B 720p attention layers the
# pages report on, and a 40-layer, 50-step trajectory of the last shape.
WORKLOADS = {
    "tiny": Workload("tiny", (8, 8, 16), 1, 64, "f32", 64, (0.2,), 0, 0.05, 1,
                     notes="1,024 tokens, one head, fp32; anchor + one reuse"),
    "wan13b_480p": Workload("wan13b_480p", (21, 30, 52), 12, 128, "bf16", 64, (0.2,), 1, 0.03, 4,
                            notes="32,760 tokens; anchor + 4 reuse steps"),
    "wan14b_720p": Workload("wan14b_720p", (21, 45, 80), 40, 128, "bf16", 64,
                            (0.1, 0.15, 0.2, 0.25, 1.0), 2, 0.0, 0,
                            notes="75,600 tokens; kernel-only sparse vs dense"),
    "hunyuan13b_720p": Workload("hunyuan13b_720p", (33, 45, 80), 24, 128, "bf16", 64, (0.15, 0.25),
                                3, 0.0, 0, notes="118,800 tokens; selection and grouping timed"),
    "hunyuan_trajectory": Workload("hunyuan_trajectory", (33, 45, 80), 24, 128, "bf16", 64, (0.15,),
                                   4, 0.02, 0, layers=40, steps=50,
                                   notes="5 dense warm-up steps, anchor every 5 steps"),
}


def grid_coords(grid) -> np.ndarray:
    """(N, 3) float64 integer coordinates, token n = (t*Y + y)*X + x."""
    t, y, x = grid
    tt, yy, xx = np.meshgrid(np.arange(t), np.arange(y), np.arange(x), indexing="ij")
    return np.stack([tt.ravel(), yy.ravel(), xx.ravel()], axis=1).astype(np.float64)


def _rng(seed, layer, head, tensor, step):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, head, tensor, step])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even); returned as float32 holding exact bf16 values."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of an array already holding exact bf16 values (see round_bf16)."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage dtype; float32 array holding the stored values exactly."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


def head_base(grid, d, seed, layer, head, noise=0.5):
    """Un-rounded fp64 (q, k, v) of one head at step 0."""
    coords = grid_coords(grid)
    n = coords.shape[0]
    r = _rng(seed, layer, head, TENSOR_FEAT, 0)
    w = r.standard_normal((3, d))  # sigma = 1 grid unit
    b = r.uniform(0.0, 2.0 * np.pi, d)
    f = np.sqrt(2.0) * np.cos(coords @ w + b)
    q = f + noise * _rng(seed, layer, head, TENSOR_QNOISE, 0).standard_normal((n, d))
    k = f + noise * _rng(seed, layer, head, TENSOR_KNOISE, 0).standard_normal((n, d))
    v = _rng(seed, layer, head, TENSOR_V, 0).standard_normal((n, d))
    return q, k, v


def head_drift(q, k, v, sigma, seed, layer, head, step):
    """Advance one head's (q, k, v) by one random-walk step (step >= 1)."""
    n, d = q.shape
    return (q + sigma * _rng(seed, layer, head, TENSOR_QNOISE, step).standard_normal((n, d)),
            k + sigma * _rng(seed, layer, head, TENSOR_KNOISE, step).standard_normal((n, d)),
            v + sigma * _rng(seed, layer, head, TENSOR_V, step).standard_normal((n, d)))


def make_qkv(wl: Workload, step: int = 0, layer: int = 0, heads=None, noise: float = 0.5):
    """Stored (H, N, D) float32 arrays (values exactly representable in wl.dtype) at a step."""
    hs = range(wl.heads) if heads is None else heads
    out = [[], [], []]
    for h in hs:
        q, k, v = head_base(wl.grid, wl.head_dim, wl.seed, layer, h, noise)
        for s in range(1, step + 1):
            q, k, v = head_drift(q, k, v, wl.drift_sigma, wl.seed, layer, h, s)
        for i, t in enumerate((q, k, v)):
            out[i].append(store(t, wl.dtype))
    return tuple(np.stack(o) for o in out)


def _torch_gen(device, *key):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence(list(key)).generate_state(1)[0]))
    return g


def base_qkv_torch(wl: Workload, device, layer: int = 0, noise: float = 0.5, heads=None):
    """Un-rounded float32 (H, N, D) Q, K, V of one layer at step 0, drawn on a torch
    device (same recipe as ``make_qkv``; per head one torch.Generator stream seeded
    from (seed, layer, head, 0))."""
    import torch

    coords = torch.from_numpy(grid_coords(wl.grid)).to(device=device, dtype=torch.float32)
    n, d = coords.shape[0], wl.head_dim
    hs = list(range(wl.heads)) if heads is None else list(heads)
    out = [torch.empty((len(hs), n, d), device=device, dtype=torch.float32) for _ in range(3)]
    for i, h in enumerate(hs):
        g = _torch_gen(device, wl.seed, layer, h, 0)
        w = torch.randn((3, d), generator=g, device=device)
        b = torch.rand((d,), generator=g, device=device) * (2.0 * math.pi)
        f = math.sqrt(2.0) * torch.cos(coords @ w + b)
        out[0][i] = f + noise * torch.randn((n, d), generator=g, device=device)
        out[1][i] = f + noise * torch.randn((n, d), generator=g, device=device)
        out[2][i] = torch.randn((n, d), generator=g, device=device)
    return tuple(out)


def drift_torch_(q, k, v, wl: Workload, layer: int, step: int, heads=None):
    """Advance float32 (H, N, D) Q, K, V of one layer in place by the random-walk
    step `step` (>= 1): per head one generator seeded from (seed, layer, head, step)."""
    import torch

    hs = list(range(q.shape[0])) if heads is None else list(heads)
    n, d = q.shape[1], q.shape[2]
    for i, h in enumerate(hs):
        gs = _torch_gen(q.device, wl.seed, layer, h, step)
        for t in (q, k, v):
            t[i] += wl.drift_sigma * torch.randn((n, d), generator=gs, device=q.device)


def storage_dtype_torch(wl: Workload):
    import torch
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def make_qkv_torch(wl: Workload, device, step: int = 0, layer: int = 0, noise: float = 0.5,
                   heads=None):
    """Draw (H, N, D) Q, K, V directly on a torch device (large workloads).

    Same recipe as ``make_qkv`` with torch.Generator streams seeded from
    (seed, layer, head, step): the float32 base (``base_qkv_torch``), then the
    drift of steps 1..step (``drift_torch_``) before the single rounding to the
    storage dtype (float32 / bfloat16).
    """
    q, k, v = base_qkv_torch(wl, device, layer, noise, heads)
    for s in range(1, step + 1):
        drift_torch_(q, k, v, wl, layer, s, heads)
    dt = storage_dtype_torch(wl)
    return tuple(t.to(dt) for t in (q, k, v))
