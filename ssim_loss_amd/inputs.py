"""Seeded synthetic image pairs shared by the tests, the smoke check and the
benchmark.

This module holds no SSIM arithmetic: it only draws pixels.  Conventions: the
generator is ``numpy.random.default_rng(seed)`` (PCG64); values are drawn in
fp64, clamped to [0, 1] and cast to fp32 once; img1 (field and noise) is drawn
before img2's noise.  Both the HIP path and the oracle consume the same fp32
arrays.

The workloads stand in for render-vs-ground-truth frames of a Gaussian
splatting train step (the pages measure "1080p" frames and name no dataset).
The volume workload has the shape of the 3-D usage example of "Fully Fused
Differentiable SSIM" (3D data): 2 x 3 x 96^3, uniform voxels; the second
volume is a noisy copy of the first, as for the images.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    shape: tuple[int, ...]            # N, C, H, W (images) or N, C, D, H, W (volumes)
    padding: str                      # "valid" | "same"
    kind: str                         # "uniform" | "field"
    noise: float                      # std of the Gaussian noise added to img1 to form img2
    seed: int
    per_image_seed: bool = False      # image n of the batch uses seed + n

    @property
    def pixels(self) -> int:
        """N*H*W for images, N*D*H*W (voxels) for volumes."""
        n = self.shape[0]
        return n * int(np.prod(self.shape[2:]))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny-64", (1, 1, 64, 64), "valid", "uniform", 0.05, 0),
        Workload("small-256", (1, 3, 256, 256), "valid", "uniform", 0.10, 0),
        Workload("1080p-valid", (1, 3, 1080, 1920), "valid", "field", 0.03, 0),
        Workload("1080p-same", (1, 3, 1080, 1920), "same", "field", 0.03, 0),
        Workload("4k-batch8", (8, 3, 2160, 3840), "valid", "uniform", 0.05, 0, True),
        Workload("vol-96", (2, 3, 96, 96, 96), "same", "uniform", 0.05, 0),
    ]
}


def smooth_field(rng: np.random.Generator, C: int, H: int, W: int, components: int = 32,
                 texture: float = 0.02) -> np.ndarray:
    """Sum of random 2-D sinusoids per channel, min-max rescaled to [0, 1],
    plus U(-texture, +texture) noise, clamped to [0, 1].  fp64.

    Per component: amplitude U[0.5, 1]; frequency log-uniform in [0.5, 50]
    cycles per image height; orientation U[0, pi); phase U[0, 2 pi).
    """
    yy = np.arange(H, dtype=np.float64)[:, None]
    xx = np.arange(W, dtype=np.float64)[None, :]
    out = np.empty((C, H, W), np.float64)
    for c in range(C):
        amp = rng.uniform(0.5, 1.0, components)
        freq = np.exp(rng.uniform(np.log(0.5), np.log(50.0), components))
        theta = rng.uniform(0.0, np.pi, components)
        phase = rng.uniform(0.0, 2.0 * np.pi, components)
        acc = np.zeros((H, W), np.float64)
        for k in range(components):
            kx = 2.0 * np.pi * freq[k] * np.cos(theta[k]) / H
            ky = 2.0 * np.pi * freq[k] * np.sin(theta[k]) / H
            # sin(kx*x + ky*y + phase) as an outer product of 1-D factors
            ax = kx * xx + phase[k]
            by = ky * yy
            acc += amp[k] * (np.sin(ax) * np.cos(by) + np.cos(ax) * np.sin(by))
        lo, hi = acc.min(), acc.max()
        out[c] = (acc - lo) / (hi - lo) if hi > lo else 0.5
    out += rng.uniform(-texture, texture, out.shape)
    np.clip(out, 0.0, 1.0, out=out)
    return out


# Flat levels of the "objects" and "flat" kinds: dark and bright values whose
# offset from 1/2 is not exact in fp32 arithmetic, two 8-bit codes, and
# mid-grey ones.
FLAT_LEVELS = (0.05, 13 / 255, 0.3, 0.7, 242 / 255, 0.95)


def flat_objects(rng: np.random.Generator, C: int, H: int, W: int, count: int = 6) -> np.ndarray:
    """A black background with `count` axis-aligned flat rectangles per
    channel, each at a level drawn from FLAT_LEVELS (later ones cover earlier
    ones).  fp64."""
    out = np.zeros((C, H, W), np.float64)
    for c in range(C):
        for _ in range(count):
            h = int(rng.integers(max(1, H // 8), max(2, H // 2)))
            w = int(rng.integers(max(1, W // 8), max(2, W // 2)))
            i = int(rng.integers(0, H - h + 1))
            j = int(rng.integers(0, W - w + 1))
            out[c, i:i + h, j:j + w] = FLAT_LEVELS[int(rng.integers(len(FLAT_LEVELS)))]
    return out


def _one_image(rng: np.random.Generator, C: int, H: int, W: int, kind: str,
               noise: float) -> tuple[np.ndarray, np.ndarray]:
    """kinds: "uniform" U[0,1); "field" the smooth field; "constant" one
    value; "objects" flat rectangles on black (flat_objects); "dark-field" a
    low-contrast dark field, 0.02 + 0.04 * smooth field.
    img2 = clamp(img1 + N(0, noise^2))."""
    if kind == "uniform":
        a = rng.random((C, H, W))
    elif kind == "field":
        a = smooth_field(rng, C, H, W)
    elif kind == "constant":
        a = np.full((C, H, W), rng.random())
    elif kind == "objects":
        a = flat_objects(rng, C, H, W)
    elif kind == "dark-field":
        a = 0.02 + 0.04 * smooth_field(rng, C, H, W, texture=0.0)
    else:
        raise ValueError(f"unknown kind {kind!r}")
    b = np.clip(a + rng.normal(0.0, noise, a.shape), 0.0, 1.0) if noise > 0 else a.copy()
    return a.astype(np.float32), b.astype(np.float32)


def make_pair(shape, kind: str = "uniform", noise: float = 0.05, seed: int = 0,
              per_image_seed: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """img1, img2 as contiguous fp32 NCHW arrays (or NCDHW volumes, for which
    only the "uniform" and "constant" kinds exist)."""
    if len(shape) == 5:
        rng = np.random.default_rng(seed)
        if kind == "uniform":
            a = rng.random(shape)
        elif kind == "constant":
            a = np.broadcast_to(rng.random((shape[0], shape[1], 1, 1, 1)), shape).copy()
        else:
            raise ValueError(f"volumes have no kind {kind!r}")
        b = np.clip(a + rng.normal(0.0, noise, a.shape), 0.0, 1.0) if noise > 0 else a.copy()
        return np.ascontiguousarray(a.astype(np.float32)), np.ascontiguousarray(b.astype(np.float32))
    N, C, H, W = shape
    if not per_image_seed:
        rng = np.random.default_rng(seed)
        if kind == "uniform":
            a = rng.random((N, C, H, W))
            b = np.clip(a + rng.normal(0.0, noise, a.shape), 0.0, 1.0) if noise > 0 else a.copy()
            return a.astype(np.float32), b.astype(np.float32)
        pairs = [_one_image(rng, C, H, W, kind, noise) for _ in range(N)]
    else:
        pairs = [_one_image(np.random.default_rng(seed + n), C, H, W, kind, noise)
                 for n in range(N)]
    x = np.stack([p[0] for p in pairs])
    y = np.stack([p[1] for p in pairs])
    return np.ascontiguousarray(x), np.ascontiguousarray(y)


def flat_pair(shape, level: float, noise: float, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """img1 = `level` everywhere, img2 = clamp(img1 + N(0, noise^2)), fp32,
    any rank (a render that is flat where the other image has texture)."""
    rng = np.random.default_rng(seed)
    a = np.full(shape, float(level))
    b = np.clip(a + rng.normal(0.0, noise, a.shape), 0.0, 1.0)
    return np.ascontiguousarray(a.astype(np.float32)), np.ascontiguousarray(b.astype(np.float32))


def make_workload(name: str) -> tuple[np.ndarray, np.ndarray]:
    w = WORKLOADS[name]
    return make_pair(w.shape, w.kind, w.noise, w.seed, w.per_image_seed)
