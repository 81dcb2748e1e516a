"""Cached reference statistics: ssim_reference_stats once per reference,
then ssim_loss_and_grad_ref per step (loss and grad_img1), against the fp64
oracle at the contract's bars, and against the one-launch kernel that forms
the same statistic itself."""
import numpy as np
import pytest

import oracle
from ssim_loss_amd.inputs import WORKLOADS, make_pair, make_workload

from gpu_util import check_grad, check_loss, say
from test_gpu_half import _check_half_grad, _loss_scale, _round
from test_gpu_recompute import SHAPES, run_loss_and_grad

pytestmark = pytest.mark.gpu


def run_ref(x, y, padding, dloss=1.0, dtype="float32", grad1=True, keep_on_device=False):
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    td = getattr(torch, dtype)
    t1 = torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(td)
    t2 = torch.from_numpy(np.ascontiguousarray(y)).to(dev).to(td)
    ref = S.reference_stats(t2, padding)
    loss, g1 = S.loss_and_grad_ref(t1, t2, ref, padding, dloss, grad1)
    torch.cuda.synchronize()
    lv = float(loss.item())
    if keep_on_device:
        return lv, g1
    return lv, None if g1 is None else g1.float().cpu().numpy()


@pytest.mark.parametrize("name", ["tiny-64", "small-256", "1080p-valid", "1080p-same"])
def test_ref_workload_parity(name):
    w = WORKLOADS[name]
    say(f"[ref] {name} {w.shape} {w.padding}")
    x, y = make_workload(name)
    gl, g1 = run_ref(x, y, w.padding, dloss=0.6)
    ol, og1, _ = oracle.ssim_loss(x, y, w.padding, dloss=0.6)
    check_loss(gl, ol, name)
    r1 = check_grad(g1, og1, name + " grad_img1")
    say(f"  loss gpu {gl:.9f} oracle {ol:.9f}; grad err/max {r1:.2e}")


@pytest.mark.parametrize("name", ["small-256", "1080p-same"])
def test_ref_matches_the_one_launch_kernel(name):
    """The cached statistic is formed by the same blur, in the same order, as
    the one-launch kernel forms it, so the two agree far inside the oracle
    bar (and are expected to agree bit for bit)."""
    w = WORKLOADS[name]
    x, y = make_workload(name)
    la, a1, _ = run_loss_and_grad(x, y, w.padding, dloss=0.6, grad2=False)
    lb, b1 = run_ref(x, y, w.padding, dloss=0.6)
    assert abs(la - lb) <= 1e-7 * abs(la)
    assert float(np.abs(a1 - b1).max()) <= 1e-6 * float(np.abs(a1).max())
    say(f"  {name}: loss equal {la == lb}; gradient identical at {float((a1 == b1).mean()):.6f}")


@pytest.mark.parametrize("shape,padding", SHAPES)
def test_ref_edge_shapes(shape, padding):
    say(f"[ref] {shape} {padding}")
    x, y = make_pair(shape, "uniform", 0.1, seed=sum(shape) + 17)
    gl, g1 = run_ref(x, y, padding, dloss=1.5)
    ol, og1, _ = oracle.ssim_loss(x, y, padding, dloss=1.5)
    check_loss(gl, ol, f"{shape}/{padding}")
    check_grad(g1, og1, f"{shape}/{padding} grad_img1")


def test_ref_random_shapes():
    rng = np.random.default_rng(77)
    for case in range(20):
        padding = "valid" if case % 2 == 0 else "same"
        lo = 11 if padding == "valid" else 1
        shape = (int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(lo, 160)),
                 int(rng.integers(lo, 700)))
        say(f"  case {case}: {shape} {padding}")
        x, y = make_pair(shape, "uniform", float(rng.uniform(0.01, 0.3)), seed=100 + case)
        gl, g1 = run_ref(x, y, padding)
        ol, og1, _ = oracle.ssim_loss(x, y, padding)
        check_loss(gl, ol, f"case {case}")
        check_grad(g1, og1, f"case {case} grad_img1")


def test_ref_reused_across_steps():
    """One reference, its statistics computed once, several different first
    images (the steps of a training run on one view)."""
    import torch

    import ssim_loss_amd as S

    _, y = make_pair((1, 3, 200, 300), "field", 0.0, seed=50)
    dev = torch.device("cuda")
    t2 = torch.from_numpy(y).to(dev)
    ref = S.reference_stats(t2, "same")
    for step in range(4):
        x = np.clip(y + np.random.default_rng(step).normal(0, 0.05 / (step + 1), y.shape), 0,
                    1).astype(np.float32)
        t1 = torch.from_numpy(x).to(dev)
        loss, g1 = S.loss_and_grad_ref(t1, t2, ref, "same", 0.8)
        ol, og1, _ = oracle.ssim_loss(x, y, "same", dloss=0.8)
        check_loss(float(loss.item()), ol, f"step {step}")
        check_grad(g1.cpu().numpy(), og1, f"step {step} grad_img1")


def test_ref_4k_batch8_loss_and_sampled_grads():
    import torch

    name = "4k-batch8"
    w = WORKLOADS[name]
    say(f"[ref] {name} {w.shape}")
    x, y = make_workload(name)
    N, C, H, W = x.shape
    M = N * C * (H - 10) * (W - 10)
    dloss = 0.75
    gl, g1 = run_ref(x, y, w.padding, dloss=dloss, keep_on_device=True)
    rng = np.random.default_rng(44)
    pts = [(0, 0, 0, 0), (7, 2, H - 1, W - 1), (3, 1, 10, 235), (5, 0, 1079, 472)]
    pts += [(int(rng.integers(N)), int(rng.integers(C)), int(rng.integers(H)),
             int(rng.integers(W))) for _ in range(300)]
    idx = torch.tensor(pts, dtype=torch.long, device=g1.device)
    s1 = g1[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].cpu().numpy().astype(np.float64)
    o1 = np.array([oracle.sample_grad(x[n, c], y[n, c], "valid", M, dloss, u, v)[0]
                   for (n, c, u, v) in pts])
    check_grad(s1, o1, "4k ref grad_img1 samples")
    ol, _, _ = oracle.ssim_loss(x, y, "valid", grads=False)
    check_loss(gl, ol, name)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_ref_half_precision(dtype):
    x, y = make_pair((2, 2, 130, 277), "field", 0.1, seed=61)
    xh, yh = _round(x, dtype), _round(y, dtype)
    ol, og1, og2 = oracle.ssim_loss(xh, yh, "valid")
    dloss = _loss_scale((og1, og2))
    gl, g1 = run_ref(xh, yh, "valid", dloss=dloss, dtype=dtype, keep_on_device=True)
    check_loss(gl, ol, dtype)
    _check_half_grad(g1, og1 * dloss, dtype, "grad_img1")


def test_ref_identity_and_loss_only():
    x, _ = make_pair((1, 2, 70, 90), "field", 0.1, seed=3)
    gl, g1 = run_ref(x, x, "same")
    assert gl == 0.0 and (g1 == 0).all()
    _, y = make_pair((1, 2, 70, 90), "field", 0.1, seed=4)
    la, _ = run_ref(x, y, "same", grad1=False)
    lb, _ = run_ref(x, y, "same")
    assert la == lb
