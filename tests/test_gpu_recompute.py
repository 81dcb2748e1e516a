"""The recomputing kernels against the fp64 oracle: the backward without
saved maps (after an inference forward) and the one-pass loss and gradients.
Same bars as the two-kernel path: |dloss| <= 1e-5 |loss|, max |dgrad| <=
1e-4 max |grad| per image; half-precision images as in test_gpu_half."""
import numpy as np
import pytest

import oracle
from ssim_loss_amd.inputs import WORKLOADS, make_pair, make_workload

from gpu_util import check_grad, check_loss, gpu_run, say
from test_gpu_half import _check_half_grad, _loss_scale, _round

pytestmark = pytest.mark.gpu


def _dev():
    import torch

    return torch.device("cuda")


def run_recompute(x, y, padding, dloss=1.0, dtype="float32", grad1=True, grad2=True,
                  keep_on_device=False):
    """Inference forward, then the backward without saved maps."""
    import torch

    import ssim_loss_amd as S

    dev = _dev()
    td = getattr(torch, dtype)
    t1 = torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(td)
    t2 = torch.from_numpy(np.ascontiguousarray(y)).to(dev).to(td)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    S.ssim_forward(t1, t2, padding, loss, None, S.workspace_for(dev))
    dl = torch.tensor(dloss, dtype=torch.float32, device=dev)
    g1 = torch.empty_like(t1) if grad1 else None
    g2 = torch.empty_like(t2) if grad2 else None
    S.ssim_backward_recompute(dl, t1, t2, padding, g1, g2)
    torch.cuda.synchronize()
    return _out(float(loss.item()), g1, g2, keep_on_device)


def run_loss_and_grad(x, y, padding, dloss=1.0, dtype="float32", grad1=True, grad2=True,
                      keep_on_device=False):
    import torch

    import ssim_loss_amd as S

    dev = _dev()
    td = getattr(torch, dtype)
    t1 = torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(td)
    t2 = torch.from_numpy(np.ascontiguousarray(y)).to(dev).to(td)
    loss, g1, g2 = S.loss_and_grad(t1, t2, padding, dloss, grad1, grad2)
    torch.cuda.synchronize()
    return _out(float(loss.item()), g1, g2, keep_on_device)


def _out(lv, g1, g2, keep):
    if keep:
        return lv, g1, g2
    f = lambda g: None if g is None else g.float().cpu().numpy()
    return lv, f(g1), f(g2)


RUNNERS = {"recompute": run_recompute, "loss_and_grad": run_loss_and_grad}


@pytest.mark.parametrize("path", list(RUNNERS))
@pytest.mark.parametrize("name", ["tiny-64", "small-256", "1080p-valid", "1080p-same"])
def test_recompute_workload_parity(name, path):
    w = WORKLOADS[name]
    say(f"[recompute] {path} {name} {w.shape} {w.padding}")
    x, y = make_workload(name)
    gl, g1, g2 = RUNNERS[path](x, y, w.padding)
    ol, og1, og2 = oracle.ssim_loss(x, y, w.padding)
    check_loss(gl, ol, name)
    r1 = check_grad(g1, og1, name + " grad_img1")
    r2 = check_grad(g2, og2, name + " grad_img2")
    say(f"  loss gpu {gl:.9f} oracle {ol:.9f}; grad err/max {r1:.2e} {r2:.2e}")


@pytest.mark.parametrize("name", ["small-256", "1080p-same"])
def test_recompute_matches_saved_maps_path(name):
    """The recomputing kernels form the same statistics, partials and adjoint
    in the same order as the two-kernel path, so the gradients agree far
    inside the oracle bar (and are expected to agree bit for bit)."""
    w = WORKLOADS[name]
    x, y = make_workload(name)
    _, s1, s2 = gpu_run(x, y, w.padding, dloss=0.7)
    for path, run in RUNNERS.items():
        _, r1, r2 = run(x, y, w.padding, dloss=0.7)
        for a, b in ((r1, s1), (r2, s2)):
            scale = float(np.abs(b).max())
            assert float(np.abs(a - b).max()) <= 1e-6 * scale
            say(f"  {name} {path}: identical to the saved-maps gradient at "
                f"{float((a == b).mean()):.6f} of entries")


def test_recompute_4k_batch8_loss_and_sampled_grads():
    """8x3x2160x3840 valid: both recomputing paths, the one-pass loss against
    the oracle's whole loss, and gradients at the sampled pixels of the
    two-kernel test, each computed one by one by the oracle."""
    import torch

    name = "4k-batch8"
    w = WORKLOADS[name]
    say(f"[recompute] {name} {w.shape}")
    x, y = make_workload(name)
    N, C, H, W = x.shape
    M = N * C * (H - 10) * (W - 10)
    dloss = 0.75
    rng = np.random.default_rng(43)
    pts = []
    for plane in [0, 7, 23]:
        n, c = divmod(plane, C)
        for (u, v) in [(0, 0), (0, W - 1), (H - 1, 0), (H - 1, W - 1), (10, 10), (9, 236),
                       (10, 235), (H - 11, W - 11), (H // 2, 0), (0, W // 2), (H // 2, W - 1),
                       (H - 1, W // 2), (1000, 471), (1000, 472), (1080, 707), (540, 3539)]:
            pts.append((n, c, u, v))
    for _ in range(600):
        pts.append((int(rng.integers(N)), int(rng.integers(C)), int(rng.integers(H)),
                    int(rng.integers(W))))
    idx = torch.tensor(pts, dtype=torch.long, device=_dev())
    samples = {}
    for path, run in RUNNERS.items():
        say(f"  gpu {path}")
        gl, g1, g2 = run(x, y, w.padding, dloss=dloss, keep_on_device=True)
        s1 = g1[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].cpu().numpy().astype(np.float64)
        s2 = g2[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].cpu().numpy().astype(np.float64)
        samples[path] = (gl, s1, s2)
        del g1, g2
        torch.cuda.empty_cache()
    say("  oracle samples")
    o1 = np.zeros(len(pts))
    o2 = np.zeros(len(pts))
    for k, (n, c, u, v) in enumerate(pts):
        o1[k], o2[k] = oracle.sample_grad(x[n, c], y[n, c], "valid", M, dloss, u, v)
    for path, (gl, s1, s2) in samples.items():
        check_grad(s1, o1, f"{name} {path} grad_img1 samples")
        check_grad(s2, o2, f"{name} {path} grad_img2 samples")
    say("  oracle whole loss")
    ol, _, _ = oracle.ssim_loss(x, y, "valid", grads=False)
    for path, (gl, _, _) in samples.items():
        check_loss(gl, ol, f"{name} {path}")
        say(f"  {path}: loss gpu {gl:.9f} oracle {ol:.9f}")


# shapes around the window (11), the strip (236 gradient / 256 image
# columns), the 4-wide groups, the 40-row minimum range, many planes (whole
# strip-columns per workgroup) and images smaller than the window (same)
SHAPES = [((1, 1, 11, 11), "valid"), ((1, 1, 1, 1), "same"), ((1, 1, 3, 7), "same"),
          ((1, 2, 67, 133), "valid"), ((2, 1, 40, 245), "same"), ((1, 1, 300, 517), "valid"),
          ((1, 3, 129, 500), "same"), ((1, 1, 16, 1000), "valid"), ((3, 1, 23, 254), "same"),
          ((1, 1, 130, 236), "valid"), ((1, 1, 81, 237), "same"), ((1, 1, 41, 472), "valid"),
          ((300, 1, 24, 480), "valid"), ((2, 2, 260, 96), "same"),
          # many planes side by side: widths around the 246-column pitch floor,
          # odd widths (per-column stores), planes narrower than a strip
          ((5, 2, 30, 247), "same"), ((4, 3, 20, 13), "valid"), ((7, 1, 15, 246), "valid"),
          ((3, 3, 12, 1921), "same")]


@pytest.mark.parametrize("path", list(RUNNERS))
@pytest.mark.parametrize("shape,padding", SHAPES)
def test_recompute_edge_shapes(shape, padding, path):
    say(f"[recompute] {path} {shape} {padding}")
    x, y = make_pair(shape, "uniform", 0.1, seed=sum(shape) + 3 * len(padding))
    gl, g1, g2 = RUNNERS[path](x, y, padding, dloss=1.5)
    ol, og1, og2 = oracle.ssim_loss(x, y, padding, dloss=1.5)
    check_loss(gl, ol, f"{shape}/{padding}")
    check_grad(g1, og1, f"{shape}/{padding} grad_img1")
    check_grad(g2, og2, f"{shape}/{padding} grad_img2")


def test_recompute_random_shapes():
    rng = np.random.default_rng(2024)
    for case in range(24):
        padding = "valid" if case % 2 == 0 else "same"
        lo = 11 if padding == "valid" else 1
        shape = (int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(lo, 160)),
                 int(rng.integers(lo, 700)))
        path = list(RUNNERS)[(case // 2) % 2]  # both paths meet both paddings
        say(f"  case {case}: {path} {shape} {padding}")
        x, y = make_pair(shape, "uniform", float(rng.uniform(0.01, 0.3)), seed=case)
        gl, g1, g2 = RUNNERS[path](x, y, padding)
        ol, og1, og2 = oracle.ssim_loss(x, y, padding)
        check_loss(gl, ol, f"case {case}")
        check_grad(g1, og1, f"case {case} grad_img1")
        check_grad(g2, og2, f"case {case} grad_img2")


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
@pytest.mark.parametrize("path", list(RUNNERS))
@pytest.mark.parametrize("shape,padding", [((1, 3, 1080, 1920), "valid"),
                                           ((1, 2, 67, 133), "same"), ((2, 1, 130, 500), "valid")])
def test_recompute_half_images(shape, padding, path, dtype):
    say(f"[recompute] {path} {shape} {padding} {dtype}")
    if shape == (1, 3, 1080, 1920):
        x, y = make_workload("1080p-valid")
    else:
        x, y = make_pair(shape, "field", 0.1, seed=sum(shape))
    xh, yh = _round(x, dtype), _round(y, dtype)
    ol, og1, og2 = oracle.ssim_loss(xh, yh, padding)
    dloss = _loss_scale((og1, og2))
    gl, g1, g2 = RUNNERS[path](xh, yh, padding, dloss=dloss, dtype=dtype, keep_on_device=True)
    check_loss(gl, ol, f"{shape}/{dtype}")
    _check_half_grad(g1, og1 * dloss, dtype, "grad_img1")
    _check_half_grad(g2, og2 * dloss, dtype, "grad_img2")


@pytest.mark.parametrize("path", list(RUNNERS))
def test_recompute_identical_images_give_exact_zero(path):
    x, _ = make_pair((2, 3, 70, 300), "field", 0.1, seed=9)
    gl, g1, g2 = RUNNERS[path](x, x, "same")
    assert gl == 0.0
    assert (g1 == 0).all() and (g2 == 0).all()


@pytest.mark.parametrize("path", list(RUNNERS))
def test_recompute_null_grads_scaling_and_determinism(path):
    x, y = make_pair((1, 3, 150, 400), "uniform", 0.1, seed=21)
    run = RUNNERS[path]
    l1, a1, a2 = run(x, y, "valid", dloss=1.0)
    l2, b1, b2 = run(x, y, "valid", dloss=1.0)
    assert l1 == l2 and (a1 == b1).all() and (a2 == b2).all()  # deterministic
    _, c1, c2 = run(x, y, "valid", dloss=0.25)                 # a power of two scales exactly
    assert (c1 == 0.25 * a1).all() and (c2 == 0.25 * a2).all()
    _, n1, d2 = run(x, y, "valid", grad1=False)
    assert n1 is None and (d2 == a2).all()
    _, d1, n2 = run(x, y, "valid", grad2=False)
    assert n2 is None and (d1 == a1).all()


def test_recompute_autograd_and_workspace_interleaving():
    """ssim_loss(recompute=True) through autograd; the one-pass kernel and the
    two-kernel forward share one workspace in turn (each leaves its
    completion counter reset)."""
    import torch

    import ssim_loss_amd as S

    x, y = make_pair((2, 3, 120, 333), "field", 0.05, seed=4)
    ol, og1, og2 = oracle.ssim_loss(x, y, "same", dloss=2.0)
    dev = _dev()
    for k in range(3):
        t1 = torch.from_numpy(x).to(dev).requires_grad_(True)
        t2 = torch.from_numpy(y).to(dev).requires_grad_(True)
        loss = S.ssim_loss(t1, t2, "same", recompute=True)
        (2.0 * loss).backward()
        check_loss(float(loss.item()), ol, f"autograd {k}")
        check_grad(t1.grad.cpu().numpy(), og1, "autograd grad_img1")
        check_grad(t2.grad.cpu().numpy(), og2, "autograd grad_img2")
        lv, g1, g2 = S.loss_and_grad(t1.detach(), t2.detach(), "same", 2.0)
        check_loss(float(lv.item()), ol, f"one-pass {k}")
        check_grad(g1.cpu().numpy(), og1, "one-pass grad_img1")
        lf = S.ssim_loss(t1.detach(), t2.detach(), "same", train=False)
        check_loss(float(lf.item()), ol, f"forward {k}")


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "float16"])
@pytest.mark.parametrize("path", list(RUNNERS))
def test_one_gradient_kernels_match_the_two_gradient_kernel(path, dtype):
    """With one gradient pointer NULL the step runs a kernel that skips the
    other gradient's partial and adjoint blur.  The gradient it forms, and the
    loss, are bit for bit those of the kernel that forms both (the same
    arithmetic in the same order), over planes side by side, widths that are
    and are not a strip's multiple, and both paddings."""
    for shape, padding, seed in (((2, 3, 70, 300), "valid", 31), ((1, 2, 45, 516), "same", 32),
                                 ((3, 1, 33, 236), "valid", 33), ((1, 1, 12, 12), "same", 34)):
        say(f"[one-gradient] {path} {dtype} {shape} {padding}")
        x, y = make_pair(shape, "uniform", 0.1, seed=seed)
        lb, a1, a2 = RUNNERS[path](x, y, padding, dloss=0.75, dtype=dtype)
        lx, b1, nb = RUNNERS[path](x, y, padding, dloss=0.75, dtype=dtype, grad2=False)
        ly, nc, c2 = RUNNERS[path](x, y, padding, dloss=0.75, dtype=dtype, grad1=False)
        assert nb is None and nc is None
        assert np.array_equal(b1, a1) and np.array_equal(c2, a2)
        if path == "loss_and_grad":
            assert lx == lb and ly == lb
