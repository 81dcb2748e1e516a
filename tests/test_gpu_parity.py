"""Parity of the HIP path with the fp64 oracle on the benchmark workloads, at
their full sizes and in the launch configuration the benchmark times (the same
C entry points with the same grid logic)."""
import numpy as np
import pytest

import oracle
from ssim_loss_amd.inputs import WORKLOADS, make_workload

from gpu_util import check_grad, check_loss, gpu_run, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny-64", "small-256", "1080p-valid", "1080p-same"])
def test_workload_full_parity(name):
    w = WORKLOADS[name]
    say(f"[parity] {name} {w.shape} {w.padding}")
    x, y = make_workload(name)
    gl, g1, g2 = gpu_run(x, y, w.padding)
    ol, og1, og2 = oracle.ssim_loss(x, y, w.padding)
    check_loss(gl, ol, name)
    r1 = check_grad(g1, og1, name + " grad_img1")
    r2 = check_grad(g2, og2, name + " grad_img2")
    say(f"  loss gpu {gl:.9f} oracle {ol:.9f}; grad err/max {r1:.2e} {r2:.2e}")


def test_4k_batch8_parity_loss_and_sampled_grads():
    """8x3x2160x3840 valid: the whole loss against the oracle's whole loss;
    gradients at sampled pixels (every corner and edge of several planes plus
    random interior points), each computed one by one by the oracle."""
    import torch

    name = "4k-batch8"
    w = WORKLOADS[name]
    say(f"[parity] {name} {w.shape} generating inputs")
    x, y = make_workload(name)
    N, C, H, W = x.shape
    Ho, Wo = H - 10, W - 10
    M = N * C * Ho * Wo
    dloss = 0.75
    say("  gpu forward+backward")
    gl, g1, g2 = gpu_run(x, y, w.padding, dloss=dloss, keep_on_device=True)
    rng = np.random.default_rng(42)
    pts = []
    for plane in [0, 5, 23]:
        n, c = divmod(plane, C)
        for (u, v) in [(0, 0), (0, W - 1), (H - 1, 0), (H - 1, W - 1), (5, 5), (9, 10), (10, 9),
                       (H - 11, W - 11), (H // 2, 0), (0, W // 2), (H // 2, W - 1),
                       (H - 1, W // 2), (1000, 243), (1000, 244), (1000, 245), (777, 488)]:
            pts.append((n, c, u, v))
    for _ in range(600):
        pts.append((int(rng.integers(N)), int(rng.integers(C)), int(rng.integers(H)),
                    int(rng.integers(W))))
    idx = torch.tensor(pts, dtype=torch.long, device=g1.device)
    s1 = g1[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].cpu().numpy().astype(np.float64)
    s2 = g2[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].cpu().numpy().astype(np.float64)
    del g1, g2
    say("  oracle samples")
    o1 = np.zeros(len(pts))
    o2 = np.zeros(len(pts))
    for k, (n, c, u, v) in enumerate(pts):
        o1[k], o2[k] = oracle.sample_grad(x[n, c], y[n, c], "valid", M, dloss, u, v)
    # The bar is relative to the largest gradient over the whole image; the
    # samples' own maximum bounds it from below, so this check is stricter.
    check_grad(s1, o1, name + " grad_img1 samples")
    check_grad(s2, o2, name + " grad_img2 samples")
    say("  oracle whole loss")
    ol, _, _ = oracle.ssim_loss(x, y, "valid", grads=False)
    check_loss(gl, ol, name)
    say(f"  loss gpu {gl:.9f} oracle {ol:.9f}")
