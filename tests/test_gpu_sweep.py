"""Seeded random sweeps through every entry point against the fp64 oracle, at
the bars of the other GPU tests: |dloss| <= 1e-5 |loss|, max |dgrad| <=
1e-4 max |grad| per image (plus the storage rounding for half types, and the
absolute loss floor of the one degenerate volume class).

Shapes lean towards the places where the kernels' work splits: widths around
the one-launch kernel's 236-column strips and its packing of planes side by
side, images narrower or shorter than the window (same padding), a few 4-row
batches, and volumes around the 32 x 16 output tile.  Each case prints its
shape before it runs."""
import numpy as np
import pytest

import oracle
from ssim_loss_amd.inputs import make_pair

from gpu_util import check_grad, check_loss, say
from test_gpu_half import _check_half_grad, _loss_scale, _round
from test_gpu_vol import vol_run

pytestmark = pytest.mark.gpu

STRIP_WIDTHS = [236, 237, 246, 247, 256, 472, 482, 483, 492, 708]


def _shape_2d(rng):
    N, C = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    pick = rng.random()
    if pick < 0.3:
        W = int(rng.choice(STRIP_WIDTHS)) + int(rng.integers(-3, 4))
    elif pick < 0.6:
        W = int(rng.integers(1, 64))
    else:
        W = int(rng.integers(1, 900))
    H = int(rng.integers(1, 40)) if rng.random() < 0.5 else int(rng.integers(1, 260))
    padding = "valid" if rng.random() < 0.5 and min(H, W) >= 11 else "same"
    return (N, C, H, W), padding


def _every_entry_point(t1, t2, padding, dloss):
    """(name, loss, grad_img1, grad_img2 or None) of the saved-maps pair, the
    recomputing backward, the one-launch step and the cached-reference step."""
    import torch

    import ssim_loss_amd as S

    dev = t1.device
    ws = S.workspace_for(dev)
    dl = torch.tensor(dloss, dtype=torch.float32, device=dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    g1, g2 = torch.empty_like(t1), torch.empty_like(t2)
    out = []
    maps = S.alloc_saved_maps(t1, padding)
    S.ssim_forward(t1, t2, padding, loss, maps, ws)
    S.ssim_backward(dl, t1, t2, padding, maps, g1, g2)
    torch.cuda.synchronize()
    out.append(("saved maps", float(loss.item()), g1.clone(), g2.clone()))
    S.ssim_forward(t1, t2, padding, loss, None, ws)
    S.ssim_backward_recompute(dl, t1, t2, padding, g1, g2)
    torch.cuda.synchronize()
    out.append(("recompute", float(loss.item()), g1.clone(), g2.clone()))
    S.ssim_loss_and_grad(t1, t2, padding, dl, loss, ws, g1, g2)
    torch.cuda.synchronize()
    out.append(("one launch", float(loss.item()), g1.clone(), g2.clone()))
    ref = S.reference_stats(t2, padding)
    S.ssim_loss_and_grad_ref(t1, t2, ref, padding, dl, loss, ws, g1)
    torch.cuda.synchronize()
    out.append(("cached reference", float(loss.item()), g1.clone(), None))
    return out


def test_sweep_2d_fp32_every_entry_point():
    import torch

    dev = torch.device("cuda")
    rng = np.random.default_rng(7000)
    for k in range(150):
        shape, padding = _shape_2d(rng)
        kind = ["uniform", "field"][int(rng.integers(2))] if min(shape[2:]) >= 4 else "uniform"
        noise = float(rng.uniform(0.01, 0.3))
        dloss = float(rng.choice([1.0, -0.5, 2.5]))
        say(f"[sweep 2d] {k}: {shape} {padding} {kind} noise {noise:.3f} dloss {dloss}")
        x, y = make_pair(shape, kind, noise, seed=7000 + k)
        ol, o1, o2 = oracle.ssim_loss(x, y, padding, dloss=dloss)
        t1, t2 = torch.from_numpy(x).to(dev), torch.from_numpy(y).to(dev)
        for name, gl, g1, g2 in _every_entry_point(t1, t2, padding, dloss):
            what = f"case {k} {name}"
            check_loss(gl, ol, what)
            check_grad(g1.cpu().numpy(), o1, what + " grad_img1")
            if g2 is not None:
                check_grad(g2.cpu().numpy(), o2, what + " grad_img2")


def test_sweep_2d_half_every_entry_point():
    import torch

    dev = torch.device("cuda")
    rng = np.random.default_rng(7100)
    for k in range(60):
        dtype = ["float16", "bfloat16"][k % 2]
        shape, padding = _shape_2d(rng)
        say(f"[sweep 2d half] {k}: {shape} {padding} {dtype}")
        x, y = make_pair(shape, "uniform", float(rng.uniform(0.01, 0.3)), seed=7100 + k)
        xh, yh = _round(x, dtype), _round(y, dtype)
        ol, o1, o2 = oracle.ssim_loss(xh, yh, padding)
        s = _loss_scale((o1, o2))
        td = getattr(torch, dtype)
        t1, t2 = torch.from_numpy(xh).to(dev).to(td), torch.from_numpy(yh).to(dev).to(td)
        for name, gl, g1, g2 in _every_entry_point(t1, t2, padding, s):
            what = f"case {k} {name}"
            check_loss(gl, ol, what)
            _check_half_grad(g1, o1 * s, dtype, what + " grad_img1")
            if g2 is not None:
                _check_half_grad(g2, o2 * s, dtype, what + " grad_img2")


def test_sweep_volumes():
    rng = np.random.default_rng(7200)
    for k in range(80):
        dtype = ["float32", "float16", "bfloat16"][k % 3]
        N, C = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        # depths, rows and columns around the 11-voxel window, the 32 x 16
        # output tile and a few depth ranges
        D, H, W = (int(rng.integers(1, 48)) for _ in range(3))
        padding = "valid" if rng.random() < 0.5 and min(D, H, W) >= 11 else "same"
        shape = (N, C, D, H, W)
        dloss = float(rng.choice([1.0, -0.5]))
        say(f"[sweep vol] {k}: {shape} {padding} {dtype} dloss {dloss}")
        x, y = make_pair(shape, "uniform", float(rng.uniform(0.01, 0.3)), seed=7200 + k)
        if dtype != "float32":
            x, y = _round(x, dtype), _round(y, dtype)
        ol, o1, o2 = oracle.ssim3_loss(x, y, padding, dloss=dloss)
        if dtype != "float32":
            s = _loss_scale((o1, o2))
            dloss, o1, o2 = dloss * s, o1 * s, o2 * s
        gl, g1, g2 = vol_run(x, y, padding, dloss=dloss, dtype=dtype, keep_on_device=True)
        check_loss(gl, ol, f"case {k}")
        if dtype == "float32":
            check_grad(g1.cpu().numpy(), o1, f"case {k} grad_vol1")
            check_grad(g2.cpu().numpy(), o2, f"case {k} grad_vol2")
        else:
            _check_half_grad(g1, o1, dtype, f"case {k} grad_vol1")
            _check_half_grad(g2, o2, dtype, f"case {k} grad_vol2")
