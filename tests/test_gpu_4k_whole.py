"""8x3x2160x3840 valid, whole gradients: every path's gradients compared
element by element with the oracle's, at the launch configuration the
benchmark times.

The oracle runs one image at a time.  Each image holds the same number of map
entries M_n = C*(H-10)*(W-10) of the batch's M = N*M_n, so the batch loss is
the mean of the per-image losses and the batch gradient of image n is the
per-image gradient scaled by M_n / M: the oracle is called with dloss / N.
Bars as everywhere: |dloss| <= 1e-5 |loss|, max |dgrad| <= 1e-4 max |grad| per
image.
"""
import numpy as np
import pytest

import oracle
from ssim_loss_amd.inputs import WORKLOADS, make_workload

from gpu_util import check_grad, check_loss, say

pytestmark = pytest.mark.gpu


def test_4k_batch8_whole_gradients_every_path():
    import torch

    import ssim_loss_amd as S

    name = "4k-batch8"
    w = WORKLOADS[name]
    say(f"[whole] {name} {w.shape} generating inputs")
    x, y = make_workload(name)
    N = x.shape[0]
    dloss = 0.75
    dev = torch.device("cuda")
    t1 = torch.from_numpy(x).to(dev)
    t2 = torch.from_numpy(y).to(dev)
    dl = torch.tensor(dloss, dtype=torch.float32, device=dev)
    ws = S.workspace_for(dev)
    paths = {}

    say("  saved maps: ssim_forward + ssim_backward")
    loss = torch.empty((), dtype=torch.float32, device=dev)
    maps = S.alloc_saved_maps(t1, w.padding)
    S.ssim_forward(t1, t2, w.padding, loss, maps, ws)
    g1, g2 = torch.empty_like(t1), torch.empty_like(t2)
    S.ssim_backward(dl, t1, t2, w.padding, maps, g1, g2)
    torch.cuda.synchronize()
    paths["saved"] = (float(loss.item()), g1, g2)
    del maps

    say("  recompute: inference ssim_forward + ssim_backward_recompute")
    loss = torch.empty((), dtype=torch.float32, device=dev)
    S.ssim_forward(t1, t2, w.padding, loss, None, ws)
    g1, g2 = torch.empty_like(t1), torch.empty_like(t2)
    S.ssim_backward_recompute(dl, t1, t2, w.padding, g1, g2)
    torch.cuda.synchronize()
    paths["recompute"] = (float(loss.item()), g1, g2)

    say("  one launch: ssim_loss_and_grad, both gradients")
    loss, g1, g2 = S.loss_and_grad(t1, t2, w.padding, dloss, True, True)
    torch.cuda.synchronize()
    paths["one-launch"] = (float(loss.item()), g1, g2)

    say("  one launch, grad_x alone (grad_img2 NULL)")
    loss, g1, _ = S.loss_and_grad(t1, t2, w.padding, dloss, True, False)
    torch.cuda.synchronize()
    paths["one-launch grad_x"] = (float(loss.item()), g1, None)

    say("  recompute, grad_y alone (grad_img1 NULL)")
    g2 = torch.empty_like(t2)
    S.ssim_backward_recompute(dl, t1, t2, w.padding, None, g2)
    torch.cuda.synchronize()
    paths["recompute grad_y"] = (paths["recompute"][0], None, g2)

    say("  cached reference: ssim_reference_stats + ssim_loss_and_grad_ref")
    ref = S.reference_stats(t2, w.padding)
    loss, g1 = S.loss_and_grad_ref(t1, t2, ref, w.padding, dloss, True)
    torch.cuda.synchronize()
    paths["reference"] = (float(loss.item()), g1, None)
    del ref

    losses = []
    worst = {p: [0.0, 0.0] for p in paths}
    for n in range(N):
        say(f"  oracle image {n}")
        ol, og1, og2 = oracle.ssim_loss(x[n:n + 1], y[n:n + 1], w.padding, dloss=dloss / N)
        losses.append(ol)
        for p, (_, g1, g2) in paths.items():
            if g1 is not None:
                r = check_grad(g1[n:n + 1].cpu().numpy(), og1, f"{p} image {n} grad_img1")
                worst[p][0] = max(worst[p][0], r)
            if g2 is not None:
                r = check_grad(g2[n:n + 1].cpu().numpy(), og2, f"{p} image {n} grad_img2")
                worst[p][1] = max(worst[p][1], r)
        del og1, og2
    ol = float(np.mean(losses))
    for p, (gl, _, _) in paths.items():
        check_loss(gl, ol, f"{p} loss")
        say(f"  {p}: loss {gl:.9f} (oracle {ol:.9f}); worst grad err/max "
            f"{worst[p][0]:.2e} {worst[p][1]:.2e}")


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
def test_4k_batch8_half_images_whole_gradients(dtype):
    """The same batch stored as half-precision images (the kernels that
    stream 16-bit tensors of this size): the one-launch and recomputing steps
    (both gradients) and the cached reference (grad_img1), every element
    against the oracle on the half values, with
    the storage rounding in the bar (tests/test_gpu_half.py).  The upstream
    gradient is a power of two that brings the largest gradient near 1 (loss
    scaling; float16 would flush these gradients, of order 1/M, to zero)."""
    import torch

    import ssim_loss_amd as S
    from test_gpu_half import _check_half_grad, _loss_scale, _round

    name = "4k-batch8"
    w = WORKLOADS[name]
    say(f"[whole-{dtype}] {name} {w.shape} generating inputs")
    x, y = make_workload(name)
    xh, yh = _round(x, dtype), _round(y, dtype)
    del x, y
    N = xh.shape[0]
    say("  oracle image 0 (for the loss scale)")
    first = oracle.ssim_loss(xh[:1], yh[:1], w.padding, dloss=1.0 / N)
    scale = _loss_scale((first[1], first[2]))
    dev = torch.device("cuda")
    td = getattr(torch, dtype)
    t1 = torch.from_numpy(xh).to(dev).to(td)
    t2 = torch.from_numpy(yh).to(dev).to(td)
    paths = {}
    say(f"  one launch (dloss {scale:g})")
    loss, g1, g2 = S.loss_and_grad(t1, t2, w.padding, scale, True, True)
    torch.cuda.synchronize()
    paths["one-launch"] = (float(loss.item()), g1, g2)
    say("  inference forward + recomputing backward")
    loss = torch.empty((), dtype=torch.float32, device=dev)
    S.ssim_forward(t1, t2, w.padding, loss, None, S.workspace_for(dev))
    dl = torch.tensor(scale, dtype=torch.float32, device=dev)
    g1, g2 = torch.empty_like(t1), torch.empty_like(t2)
    S.ssim_backward_recompute(dl, t1, t2, w.padding, g1, g2)
    torch.cuda.synchronize()
    paths["recompute"] = (float(loss.item()), g1, g2)
    say("  cached reference")
    ref = S.reference_stats(t2, w.padding)
    loss, g1 = S.loss_and_grad_ref(t1, t2, ref, w.padding, scale, True)
    torch.cuda.synchronize()
    paths["reference"] = (float(loss.item()), g1, None)
    del ref

    losses = []
    worst = {p: 0.0 for p in paths}
    for n in range(N):
        say(f"  oracle image {n}")
        ol, og1, og2 = first if n == 0 else oracle.ssim_loss(xh[n:n + 1], yh[n:n + 1], w.padding,
                                                             dloss=1.0 / N)
        losses.append(ol)
        og1, og2 = og1 * scale, og2 * scale
        for p, (_, g1, g2) in paths.items():
            worst[p] = max(worst[p],
                           _check_half_grad(g1[n:n + 1], og1, dtype, f"{p} image {n} grad_img1"))
            if g2 is not None:
                worst[p] = max(worst[p], _check_half_grad(g2[n:n + 1], og2, dtype,
                                                          f"{p} image {n} grad_img2"))
    ol = float(np.mean(losses))
    for p, (gl, _, _) in paths.items():
        check_loss(gl, ol, f"{p} loss")
        say(f"  {p}: loss {gl:.9f} (oracle {ol:.9f}); worst grad err/max {worst[p]:.2e}")
