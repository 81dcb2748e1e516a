"""Half-precision image I/O (float16 and bfloat16 images and gradients, fp32
arithmetic inside the kernels) against the fp64 oracle.

The oracle sees the images as the GPU does: the half values, widened exactly.
The loss is held to the fp32 contract (1e-5 relative).  A gradient is the fp32
result rounded once to the storage type, so each element may differ from the
oracle by the fp32 bar (1e-4 of the largest gradient) plus half a unit in the
last place of the storage type: 2^-11 |g| for float16, 2^-8 |g| for bfloat16,
plus half the float16 subnormal spacing (2^-25) where the value is subnormal.

Gradients of SSIM are of order 1/M (M = number of SSIM-map pixels), far below
the float16 normal range at 1080p, so the float16 runs scale the upstream
gradient by a power of two (loss scaling, which is how float16 training uses
it); the scale is exact and the oracle is scaled by the same factor.
"""
import numpy as np
import pytest

import oracle
from ssim_loss_amd.inputs import WORKLOADS, make_pair, make_workload

from gpu_util import LOSS_RTOL, GRAD_RTOL, check_loss, say

pytestmark = pytest.mark.gpu

UNIT = {"float16": 2.0 ** -11, "bfloat16": 2.0 ** -8}
SUBNORMAL_HALF_SPACING = {"float16": 2.0 ** -25, "bfloat16": 0.0}


def _round(a, dtype):
    """The half value of each element (round to nearest even), widened to fp32."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(getattr(torch, dtype)).float().numpy()


def _loss_scale(og_unit):
    """A power of two that brings the largest gradient near 1."""
    m = max(float(np.abs(g).max()) for g in og_unit)
    return 2.0 ** int(np.floor(-np.log2(m))) if m > 0 else 1.0


def _run(xh, yh, padding, dtype, dloss, grad1=True, grad2=True):
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    td = getattr(torch, dtype)
    t1 = torch.from_numpy(xh).to(dev).to(td)
    t2 = torch.from_numpy(yh).to(dev).to(td)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    maps = S.alloc_saved_maps(t1, padding)
    S.ssim_forward(t1, t2, padding, loss, maps, S.workspace_for(dev))
    dl = torch.tensor(dloss, dtype=torch.float32, device=dev)
    g1 = torch.empty_like(t1) if grad1 else None
    g2 = torch.empty_like(t2) if grad2 else None
    S.ssim_backward(dl, t1, t2, padding, maps, g1, g2)
    torch.cuda.synchronize()
    return float(loss.item()), g1, g2


def _check_half_grad(g, og, dtype, what):
    """g: the GPU gradient (a half tensor), og: the oracle's fp64 gradient."""
    gv = g.float().cpu().numpy().astype(np.float64)
    scale = float(np.abs(og).max())
    tol = (GRAD_RTOL * scale * (1 + UNIT[dtype]) + UNIT[dtype] * np.abs(og)
           + SUBNORMAL_HALF_SPACING[dtype])
    err = np.abs(gv - og)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements over the bar; worst "
                           f"|d|={float(err[bad].max()):.3e} at scale {scale:.3e}")
    return float(err.max()) / scale if scale > 0 else 0.0


def _half_case(x, y, padding, dtype, what, scaled=True):
    xh, yh = _round(x, dtype), _round(y, dtype)
    ol, og1, og2 = oracle.ssim_loss(xh, yh, padding)
    dloss = _loss_scale((og1, og2)) if scaled else 1.0
    gl, g1, g2 = _run(xh, yh, padding, dtype, dloss)
    check_loss(gl, ol, what)
    r1 = _check_half_grad(g1, og1 * dloss, dtype, what + " grad_img1")
    r2 = _check_half_grad(g2, og2 * dloss, dtype, what + " grad_img2")
    say(f"  {what}: loss gpu {gl:.9f} oracle {ol:.9f}; dloss {dloss:g}; "
        f"grad err/max {r1:.2e} {r2:.2e}")
    return xh, yh, dloss, g1, g2


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
@pytest.mark.parametrize("name", ["tiny-64", "small-256", "1080p-valid", "1080p-same"])
def test_half_workload_parity(name, dtype):
    w = WORKLOADS[name]
    say(f"[half] {name} {w.shape} {w.padding} {dtype}")
    x, y = make_workload(name)
    _half_case(x, y, w.padding, dtype, f"{name}/{dtype}")


# ragged widths take the scalar-load kernel (W not a multiple of 4); the rest
# cover one and several strips, tails of every residue and both paddings
SHAPES = [((1, 1, 11, 11), "valid"), ((1, 1, 1, 1), "same"), ((1, 2, 67, 133), "valid"),
          ((2, 1, 40, 245), "same"), ((1, 1, 300, 517), "valid"), ((1, 3, 129, 500), "same"),
          ((1, 1, 16, 1000), "valid"), ((3, 1, 23, 254), "same")]


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
@pytest.mark.parametrize("shape,padding", SHAPES)
def test_half_edge_shapes(shape, padding, dtype):
    say(f"[half] {shape} {padding} {dtype}")
    x, y = make_pair(shape, "field", 0.1, seed=sum(shape) * 7 + len(padding))
    _half_case(x, y, padding, dtype, f"{shape}/{padding}/{dtype}")


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_half_gradient_is_the_fp32_gradient_rounded(dtype):
    """The half kernels do the fp32 kernels' arithmetic and round only the
    stored gradient: on the same (half-valued) images, each half gradient lies
    within one unit in the last place of the fp32 gradient rounded to the
    storage type, and the loss is the same."""
    import torch

    say(f"[half] fp32 vs {dtype} on the same values")
    x, y = make_pair((2, 3, 200, 333), "field", 0.1, seed=5)
    xh, yh = _round(x, dtype), _round(y, dtype)
    gl_h, g1_h, g2_h = _run(xh, yh, "same", dtype, 1024.0)
    gl_f, g1_f, g2_f = _run(xh, yh, "same", "float32", 1024.0)
    assert gl_h == gl_f
    td = getattr(torch, dtype)
    for gh, gf in ((g1_h, g1_f), (g2_h, g2_f)):
        ref = gf.to(td).float()
        # one unit in the last place of ref, and the float16 subnormal spacing
        ulp = 2 * UNIT[dtype] * ref.abs() + 4 * SUBNORMAL_HALF_SPACING[dtype]
        assert bool(((gh.float() - ref).abs() <= ulp).all())
        frac = float((gh.float() == ref).float().mean())
        say(f"  identical to the rounded fp32 gradient: {frac:.6f}")


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_half_autograd_and_null_grads(dtype):
    import torch

    import ssim_loss_amd as S

    say(f"[half] autograd {dtype}")
    x, y = make_pair((1, 3, 96, 130), "field", 0.1, seed=11)
    xh, yh = _round(x, dtype), _round(y, dtype)
    dev = torch.device("cuda")
    td = getattr(torch, dtype)
    t1 = torch.from_numpy(xh).to(dev).to(td).requires_grad_(True)
    t2 = torch.from_numpy(yh).to(dev).to(td)
    loss = S.ssim_loss(t1, t2, "valid")
    assert loss.dtype == torch.float32
    (loss * 1024.0).backward()
    assert t1.grad.dtype == td and t2.grad is None
    ol, og1, _ = oracle.ssim_loss(xh, yh, "valid")
    check_loss(float(loss.item()), ol, "autograd")
    _check_half_grad(t1.grad, og1 * 1024.0, dtype, "autograd grad_img1")
    # inference mode gives the same loss
    with torch.no_grad():
        li = S.ssim_loss(t1.detach(), t2, "valid", train=False)
    assert float(li.item()) == float(loss.item())
    # only grad_img2 requested through the C entry point
    _, g1, g2 = _run(xh, yh, "valid", dtype, 1024.0, grad1=False)
    assert g1 is None
    _, _, og2 = oracle.ssim_loss(xh, yh, "valid")
    _check_half_grad(g2, og2 * 1024.0, dtype, "grad_img2 only")


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_half_identical_images_give_exact_zero(dtype):
    import torch

    x, _ = make_pair((1, 2, 70, 90), "field", 0.1, seed=3)
    xh = _round(x, dtype)
    gl, g1, g2 = _run(xh, xh, "same", dtype, 1.0)
    assert gl == 0.0
    assert bool((g1.float() == 0).all()) and bool((g2.float() == 0).all())


def test_half_rejects_mixed_dtypes():
    import torch

    import ssim_loss_amd as S

    a = torch.zeros(1, 1, 16, 16, device="cuda", dtype=torch.float16)
    b = torch.zeros(1, 1, 16, 16, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        S.ssim_loss(a, b)
    with pytest.raises(TypeError):
        S.ssim_loss(a, a.float())
