"""Volume SSIM ("Fully Fused Differentiable SSIM", 3D data) on the GPU against
the fp64 volume oracle, at the contract's bars: |dloss| <= 1e-5 |loss|,
max |dgrad| <= 1e-4 max |grad| per volume; half-precision volumes as in
test_gpu_half (the fp32 bar plus the storage rounding)."""
import numpy as np
import pytest

import oracle
from ssim_loss_amd.inputs import WORKLOADS, flat_pair, make_pair, make_workload

from gpu_util import check_grad, check_loss, say
from test_gpu_edge import constant_grad_bar
from test_gpu_half import _check_half_grad, _loss_scale, _round

pytestmark = pytest.mark.gpu


def vol_run(x, y, padding, dloss=1.0, dtype="float32", grad1=True, grad2=True, train=True,
            keep_on_device=False):
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    td = getattr(torch, dtype)
    t1 = torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(td)
    t2 = torch.from_numpy(np.ascontiguousarray(y)).to(dev).to(td)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    maps = S.alloc_saved_maps3d(t1, padding) if train else None
    S.ssim3d_forward(t1, t2, padding, loss, maps, S.workspace_for(dev))
    g1 = g2 = None
    if train and (grad1 or grad2):
        dl = torch.tensor(dloss, dtype=torch.float32, device=dev)
        g1 = torch.empty_like(t1) if grad1 else None
        g2 = torch.empty_like(t2) if grad2 else None
        S.ssim3d_backward(dl, t1, t2, padding, maps, g1, g2)
    torch.cuda.synchronize()
    lv = float(loss.item())
    if keep_on_device:
        return lv, g1, g2
    f = lambda g: None if g is None else g.float().cpu().numpy()
    return lv, f(g1), f(g2)


# around the window (11), the 32 x 16 (rows x columns) output tile, several
# depth ranges per tile-column, and volumes smaller than the window (same)
SHAPES = [((1, 1, 11, 11, 11), "valid"), ((1, 1, 1, 1, 1), "same"), ((1, 1, 3, 5, 7), "same"),
          ((1, 2, 20, 17, 33), "valid"), ((2, 1, 13, 16, 16), "same"), ((1, 1, 50, 12, 40), "same"),
          ((1, 3, 26, 27, 15), "valid"), ((3, 2, 9, 31, 18), "same"),
          ((1, 1, 40, 70, 35), "same"), ((1, 2, 33, 34, 17), "same"), ((2, 1, 30, 43, 40), "valid"),
          ((1, 1, 24, 100, 200), "same")]


@pytest.mark.parametrize("shape,padding", SHAPES)
def test_volume_parity(shape, padding):
    say(f"[vol] {shape} {padding}")
    x, y = make_pair(shape, "uniform", 0.1, seed=sum(shape) + len(padding))
    gl, g1, g2 = vol_run(x, y, padding, dloss=0.9)
    ol, og1, og2 = oracle.ssim3_loss(x, y, padding, dloss=0.9)
    check_loss(gl, ol, f"{shape}/{padding}")
    r1 = check_grad(g1, og1, f"{shape}/{padding} grad_vol1")
    r2 = check_grad(g2, og2, f"{shape}/{padding} grad_vol2")
    say(f"  loss gpu {gl:.9f} oracle {ol:.9f}; grad err/max {r1:.2e} {r2:.2e}")


def test_volume_workload_loss_and_grads():
    """The 2 x 3 x 96^3 volumes of the page's 3-D example (same padding): the
    whole loss and both whole gradients against the oracle's, every volume's
    gradients element by element; and gradients at sampled voxels (every
    corner of several volumes, tile and window borders, random interior
    points), each computed one by one by the oracle's single-voxel routine."""
    import torch

    w = WORKLOADS["vol-96"]
    say(f"[vol] {w.name} {w.shape}")
    x, y = make_workload("vol-96")
    N, C, D, H, W = x.shape
    M = float(N * C * D * H * W)
    dloss = 1.25
    gl, g1, g2 = vol_run(x, y, w.padding, dloss=dloss, keep_on_device=True)
    rng = np.random.default_rng(7)
    pts = []
    for vol in [0, 4]:
        n, c = divmod(vol, C)
        for (t, u, v) in [(0, 0, 0), (D - 1, H - 1, W - 1), (0, H - 1, 0), (D - 1, 0, W - 1),
                          (5, 15, 16), (47, 16, 15), (24, 31, 32), (90, 80, 5), (23, 24, 25)]:
            pts.append((n, c, t, u, v))
    for _ in range(150):
        pts.append(tuple(int(rng.integers(k)) for k in (N, C, D, H, W)))
    idx = torch.tensor(pts, dtype=torch.long, device=g1.device)
    s1 = g1[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3], idx[:, 4]].cpu().numpy().astype(np.float64)
    s2 = g2[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3], idx[:, 4]].cpu().numpy().astype(np.float64)
    say("  oracle samples")
    o1 = np.zeros(len(pts))
    o2 = np.zeros(len(pts))
    for k, (n, c, t, u, v) in enumerate(pts):
        o1[k], o2[k] = oracle.sample_grad3(x[n, c], y[n, c], w.padding, M, dloss, t, u, v)
    check_grad(s1, o1, "vol-96 grad_vol1 samples")
    check_grad(s2, o2, "vol-96 grad_vol2 samples")
    say("  oracle whole loss and gradients")
    ol, og1, og2 = oracle.ssim3_loss(x, y, w.padding, dloss=dloss)
    check_loss(gl, ol, "vol-96")
    g1h, g2h = g1.cpu().numpy(), g2.cpu().numpy()
    worst = 0.0
    for n in range(N):
        for c in range(C):
            worst = max(worst, check_grad(g1h[n, c], og1[n, c], f"vol-96 ({n},{c}) grad_vol1"),
                        check_grad(g2h[n, c], og2[n, c], f"vol-96 ({n},{c}) grad_vol2"))
    say(f"  loss gpu {gl:.9f} oracle {ol:.9f}; worst grad err/max per volume {worst:.2e}")


def test_volume_random_shapes():
    rng = np.random.default_rng(99)
    for case in range(16):
        padding = "valid" if case % 2 == 0 else "same"
        lo = 11 if padding == "valid" else 1
        shape = (1, int(rng.integers(1, 3)), int(rng.integers(lo, 40)), int(rng.integers(lo, 40)),
                 int(rng.integers(lo, 40)))
        say(f"  case {case}: {shape} {padding}")
        x, y = make_pair(shape, "uniform", float(rng.uniform(0.01, 0.3)), seed=case)
        gl, g1, g2 = vol_run(x, y, padding)
        ol, og1, og2 = oracle.ssim3_loss(x, y, padding)
        check_loss(gl, ol, f"case {case}")
        check_grad(g1, og1, f"case {case} grad_vol1")
        check_grad(g2, og2, f"case {case} grad_vol2")


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_volume_half_precision(dtype):
    x, y = make_pair((1, 2, 18, 21, 20), "uniform", 0.1, seed=31)
    xh, yh = _round(x, dtype), _round(y, dtype)
    ol, og1, og2 = oracle.ssim3_loss(xh, yh, "same")
    dloss = _loss_scale((og1, og2))
    gl, g1, g2 = vol_run(xh, yh, "same", dloss=dloss, dtype=dtype, keep_on_device=True)
    check_loss(gl, ol, dtype)
    _check_half_grad(g1, og1 * dloss, dtype, "grad_vol1")
    _check_half_grad(g2, og2 * dloss, dtype, "grad_vol2")


def test_volume_inference_identity_null_grads_and_autograd():
    import torch

    import ssim_loss_amd as S

    x, y = make_pair((1, 2, 20, 19, 18), "uniform", 0.1, seed=41)
    lt, a1, a2 = vol_run(x, y, "same")
    li, _, _ = vol_run(x, y, "same", train=False)
    assert li == lt
    l2, b1, b2 = vol_run(x, y, "same")
    assert l2 == lt and (b1 == a1).all() and (b2 == a2).all()  # deterministic
    _, n1, c2 = vol_run(x, y, "same", grad1=False)
    assert n1 is None and (c2 == a2).all()
    l0, z1, z2 = vol_run(x, x, "same")
    assert l0 == 0.0 and (z1 == 0).all() and (z2 == 0).all()
    dev = torch.device("cuda")
    t1 = torch.from_numpy(x).to(dev).requires_grad_(True)
    t2 = torch.from_numpy(y).to(dev)
    s = S.fused_ssim3d(t1, t2)
    (-2.0 * s).backward()
    ol, og1, _ = oracle.ssim3_loss(x, y, "same", dloss=2.0)
    assert abs(float(s.item()) - (1 - ol)) <= 1e-5 * abs(ol)
    check_grad(t1.grad.cpu().numpy(), og1, "autograd grad_vol1")
    assert t2.grad is None


def test_volume_at_the_size_limit():
    """One 512^3 volume pair (2^27 voxels, the documented limit; 512 MiB per
    tensor), valid padding.  The volumes are constant along depth, so the
    whole loss is the 2-D oracle's loss of one slice (the reduction the
    volume oracle's pins establish); gradients at sampled voxels come from
    the volume oracle one by one."""
    import torch

    n = 512
    x2, y2 = make_pair((1, 1, n, n), "uniform", 0.05, seed=512)
    x = np.ascontiguousarray(np.broadcast_to(x2[:, :, None], (1, 1, n, n, n)))
    y = np.ascontiguousarray(np.broadcast_to(y2[:, :, None], (1, 1, n, n, n)))
    say(f"[vol] size limit {x.shape}")
    dloss = 1.1
    gl, g1, g2 = vol_run(x, y, "valid", dloss=dloss, keep_on_device=True)
    ol, _, _ = oracle.ssim_loss(x2, y2, "valid", grads=False)
    check_loss(gl, ol, "512^3 volume")
    M = float((n - 10) ** 3)
    rng = np.random.default_rng(6)
    pts = [(t, u, v) for t in (0, 5, n - 1) for u in (0, n - 1) for v in (0, 15, 16, n - 1)]
    pts += [tuple(int(rng.integers(n)) for _ in range(3)) for _ in range(40)]
    idx = torch.tensor(pts, dtype=torch.long, device=g1.device)
    s1 = g1[0, 0, idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy().astype(np.float64)
    s2 = g2[0, 0, idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy().astype(np.float64)
    o = np.array([oracle.sample_grad3(x[0, 0], y[0, 0], "valid", M, dloss, t, u, v) for t, u, v in pts])
    check_grad(s1, o[:, 0], "512^3 grad_vol1 samples")
    check_grad(s2, o[:, 1], "512^3 grad_vol2 samples")


@pytest.mark.parametrize("padding", ["valid", "same"])
@pytest.mark.parametrize("level", [0.05, 0.3, 0.95, 13 / 255])
def test_flat_volume_against_noisy_one(level, padding):
    """One volume flat at a level, the other a noisy copy, each way round: a
    misrounded mean of the flat volume would bias the covariance of every
    window alike (before the passes were taken by parts, levels 0.05 and 0.95
    missed the loss bar by about 2.5e-5)."""
    x, y = flat_pair((1, 2, 24, 26, 28), level, 0.01, seed=int(level * 1000) + 1)
    for a, b in ((x, y), (y, x)):
        say(f"[vol flat] {level:.4f} {padding}")
        gl, g1, g2 = vol_run(a, b, padding, dloss=0.5)
        ol, og1, og2 = oracle.ssim3_loss(a, b, padding, dloss=0.5)
        check_loss(gl, ol, f"flat {level} {padding}")
        check_grad(g1, og1, "grad_vol1")
        check_grad(g2, og2, "grad_vol2")


@pytest.mark.parametrize("padding", ["valid", "same"])
@pytest.mark.parametrize("a,b", [(0.3, 0.8), (0.05, 0.95), (1.0, 0.98), (0.3, 0.31)])
def test_constant_volumes(a, b, padding):
    """Constant volumes: the loss at the contract's bar (the variances
    vanish, so any rounding bias in the means or in B((x - y)^2) would be
    divided by C2), the gradients at the cancellation bound of the images'
    constant test (test_gpu_edge.constant_grad_bar)."""
    say(f"[vol const] {a} {b} {padding}")
    x = np.full((1, 1, 20, 21, 22), a, np.float32)
    y = np.full((1, 1, 20, 21, 22), b, np.float32)
    gl, g1, g2 = vol_run(x, y, padding)
    ol, og1, og2 = oracle.ssim3_loss(x, y, padding)
    check_loss(gl, ol, f"constant {a} {b} {padding}")
    bar = constant_grad_bar(a, b)
    for g, og in ((g1, og1), (g2, og2)):
        err = float(np.abs(g.astype(np.float64) - og).max())
        assert err <= bar * float(np.abs(og).max()), (err, bar)
