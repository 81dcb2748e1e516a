"""Helpers for the GPU tests: run the HIP path through the C ABI and compare
with the oracle at the tolerances of the method's contract:
    |loss_gpu - loss_oracle| <= 1e-5 * |loss_oracle|
    max |grad_gpu - grad_oracle| <= 1e-4 * max |grad_oracle|  (each image)
"""
from __future__ import annotations

import sys

import numpy as np

LOSS_RTOL = 1e-5
GRAD_RTOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(x: np.ndarray, y: np.ndarray, padding: str, dloss: float = 1.0, grad1: bool = True,
            grad2: bool = True, train: bool = True, keep_on_device: bool = False):
    """Forward (+ backward) through the C ABI on torch's current stream."""
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    t1 = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    t2 = torch.from_numpy(np.ascontiguousarray(y)).to(dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    maps = S.alloc_saved_maps(t1, padding) if train else None
    S.ssim_forward(t1, t2, padding, loss, maps, S.workspace_for(dev))
    g1 = g2 = None
    if train and (grad1 or grad2):
        dl = torch.tensor(dloss, dtype=torch.float32, device=dev)
        g1 = torch.empty_like(t1) if grad1 else None
        g2 = torch.empty_like(t2) if grad2 else None
        S.ssim_backward(dl, t1, t2, padding, maps, g1, g2)
    torch.cuda.synchronize()
    lv = float(loss.item())
    if keep_on_device:
        return lv, g1, g2
    return (lv, None if g1 is None else g1.cpu().numpy(), None if g2 is None else g2.cpu().numpy())


def check_loss(gl: float, ol: float, what: str = ""):
    err = abs(gl - ol)
    assert err <= LOSS_RTOL * abs(ol), f"{what}: loss {gl!r} vs oracle {ol!r} (|d|={err:.3e})"


def check_grad(g: np.ndarray, og: np.ndarray, what: str = ""):
    scale = float(np.abs(og).max())
    err = float(np.abs(g.astype(np.float64) - og).max())
    assert err <= GRAD_RTOL * scale, f"{what}: max|dgrad| {err:.3e} > 1e-4 * {scale:.3e}"
    return err / scale if scale > 0 else 0.0
