"""Pins for the oracle's volume SSIM ("Fully Fused Differentiable SSIM", 3D
data: the 2-D computation on each XY slice plus a Z-axis pass of the same
window): each test ties it to something other than itself -- scipy's N-D
correlation, the already pinned 2-D oracle (a volume constant along z reduces
to it exactly), plain-torch conv3d with autograd, finite differences, closed
forms and invariants.
"""

import numpy as np
import pytest
import scipy.ndimage
import scipy.signal.windows
import torch

import oracle

C1, C2 = 1e-4, 9e-4


def _pair(shape, seed, noise=0.1):
    rng = np.random.default_rng(seed)
    x = rng.random(shape)
    y = np.clip(x + rng.normal(0, noise, shape), 0, 1)
    return x, y


def _scipy_window3():
    g = scipy.signal.windows.gaussian(11, 1.5)
    g = g / g.sum()
    return np.einsum("a,b,c->abc", g, g, g)


@pytest.mark.parametrize("D,H,W", [(11, 11, 11), (13, 17, 12), (20, 14, 16)])
def test_out_shape3(D, H, W):
    assert oracle.out_shape3(D, H, W, "valid") == (D - 10, H - 10, W - 10)
    assert oracle.out_shape3(D, H, W, "same") == (D, H, W)


@pytest.mark.parametrize("shape", [(12, 13, 14), (16, 11, 15), (5, 7, 9)])
def test_blur3_matches_scipy_correlate(shape):
    rng = np.random.default_rng(sum(shape))
    v = rng.random(shape)
    ref = scipy.ndimage.correlate(v, _scipy_window3(), mode="constant", cval=0.0)
    np.testing.assert_allclose(oracle.blur3(v, "same"), ref, rtol=0, atol=1e-14)
    if min(shape) >= 11:
        np.testing.assert_allclose(oracle.blur3(v, "valid"), ref[5:-5, 5:-5, 5:-5], rtol=0,
                                   atol=1e-14)


def test_z_constant_volume_reduces_to_the_2d_oracle():
    """A volume whose slices are all the same image, valid padding: every Z
    window covers 11 equal slices and the taps sum to 1, so each map slice is
    the 2-D SSIM map and the loss is the 2-D loss.  A voxel at depth z feeds
    the map slices k with 0 <= z - k <= 10, each with tap g[z - k], so its
    gradient is the 2-D gradient times c(z) / Do, c(z) = sum of those taps."""
    x2, y2 = _pair((1, 1, 19, 23), 3)
    D = 16
    x3 = np.repeat(x2[:, :, None], D, axis=2)
    y3 = np.repeat(y2[:, :, None], D, axis=2)
    l2, gx2, gy2 = oracle.ssim_loss(x2, y2, "valid")
    l3, gx3, gy3 = oracle.ssim3_loss(x3, y3, "valid")
    assert abs(l3 - l2) < 1e-13
    g = scipy.signal.windows.gaussian(11, 1.5)
    g = g / g.sum()
    Do = D - 10
    for z in range(D):
        cz = sum(g[z - k] for k in range(Do) if 0 <= z - k <= 10)
        np.testing.assert_allclose(gx3[0, 0, z], gx2[0, 0] * cz / Do, rtol=0,
                                   atol=1e-13 * np.abs(gx2).max())
        np.testing.assert_allclose(gy3[0, 0, z], gy2[0, 0] * cz / Do, rtol=0,
                                   atol=1e-13 * np.abs(gy2).max())


def _torch_ssim3_loss(x, y, padding):
    """Independent plain-torch fp64 volume SSIM loss (depthwise conv3d with
    the scipy window), differentiated by autograd."""
    C = x.shape[1]
    w = torch.tensor(_scipy_window3(), dtype=torch.float64).expand(C, 1, 11, 11, 11).contiguous()
    pad = 0 if padding == "valid" else 5

    def blur(t):
        return torch.nn.functional.conv3d(t, w, padding=pad, groups=C)

    mx, my = blur(x), blur(y)
    vx = blur(x * x) - mx * mx
    vy = blur(y * y) - my * my
    cxy = blur(x * y) - mx * my
    s = ((2 * mx * my + C1) * (2 * cxy + C2)) / ((mx * mx + my * my + C1) * (vx + vy + C2))
    return 1 - s.mean()


# (valid padding needs at least 11 voxels per axis, so the small volume is same only)
@pytest.mark.parametrize("shape,padding", [((1, 1, 12, 12, 12), "valid"), ((1, 1, 12, 12, 12), "same"),
                                           ((2, 2, 11, 14, 13), "valid"), ((2, 2, 11, 14, 13), "same"),
                                           ((1, 1, 7, 9, 8), "same")])
def test_volume_loss_and_grads_match_torch_autograd(shape, padding):
    x, y = _pair(shape, 5)
    dloss = 0.7
    loss, gx, gy = oracle.ssim3_loss(x, y, padding, dloss=dloss)
    tx = torch.tensor(x, requires_grad=True)
    ty = torch.tensor(y, requires_grad=True)
    tl = _torch_ssim3_loss(tx, ty, padding)
    (tl * dloss).backward()
    assert abs(loss - tl.item()) < 1e-12
    np.testing.assert_allclose(gx, tx.grad.numpy(), rtol=0, atol=1e-12 * np.abs(gx).max())
    np.testing.assert_allclose(gy, ty.grad.numpy(), rtol=0, atol=1e-12 * np.abs(gy).max())


@pytest.mark.parametrize("padding", ["valid", "same"])
def test_volume_gradient_matches_finite_differences(padding):
    shape = (1, 1, 11, 12, 11) if padding == "valid" else (1, 1, 6, 7, 5)
    x, y = _pair(shape, 6)
    dloss = 1.7
    _, gx, gy = oracle.ssim3_loss(x, y, padding, dloss=dloss)

    def f(a, b):
        return oracle.ssim3_loss(a, b, padding, grads=False)[0]

    h = 1e-6
    rng = np.random.default_rng(7)
    idxs = [(0, 0, 0, 0, 0), tuple([0, 0] + [n - 1 for n in shape[2:]]),
            tuple([0, 0] + [n // 2 for n in shape[2:]]),
            (0, 0, 0, 3, 1)]
    idxs += [tuple([0, 0] + [int(rng.integers(n)) for n in shape[2:]]) for _ in range(10)]
    scale = max(np.abs(gx).max(), np.abs(gy).max())
    for idx in idxs:
        for g, which in ((gx, 0), (gy, 1)):
            p = [x.copy(), y.copy()]
            m = [x.copy(), y.copy()]
            p[which][idx] += h
            m[which][idx] -= h
            fd = dloss * (f(*p) - f(*m)) / (2 * h)
            assert abs(g[idx] - fd) < 1e-6 * scale, (idx, which, g[idx], fd)


def test_constant_volumes_closed_form():
    """Constant volumes a and b, valid padding: every variance vanishes, so
    S = (2ab + C1)/(a^2 + b^2 + C1) everywhere."""
    a, b = 0.3, 0.6
    x = np.full((1, 1, 12, 11, 13), a)
    y = np.full((1, 1, 12, 11, 13), b)
    loss, _, _ = oracle.ssim3_loss(x, y, "valid", grads=False)
    s = (2 * a * b + C1) / (a * a + b * b + C1)
    assert abs(loss - (1 - s)) < 1e-11


def test_volume_swap_symmetry_and_identity():
    x, y = _pair((1, 2, 9, 8, 10), 11)
    l1, gx1, gy1 = oracle.ssim3_loss(x, y, "same")
    l2, gx2, gy2 = oracle.ssim3_loss(y, x, "same")
    assert abs(l1 - l2) < 1e-15
    np.testing.assert_allclose(gx1, gy2, rtol=0, atol=1e-18)
    np.testing.assert_allclose(gy1, gx2, rtol=0, atol=1e-18)
    l0, g0x, g0y = oracle.ssim3_loss(x, x, "same")
    assert abs(l0) < 1e-15
    assert np.abs(g0x).max() < 1e-15 and np.abs(g0y).max() < 1e-15


def test_volume_float32_entry_equals_float64_entry_on_same_values():
    x, y = _pair((1, 2, 9, 10, 8), 12)
    x32, y32 = x.astype(np.float32), y.astype(np.float32)
    l32, gx32, gy32 = oracle.ssim3_loss(x32, y32, "same")
    l64, gx64, gy64 = oracle.ssim3_loss(x32.astype(np.float64), y32.astype(np.float64), "same")
    assert abs(l32 - l64) < 1e-15
    np.testing.assert_allclose(gx32, gx64, rtol=0, atol=1e-18)
    np.testing.assert_allclose(gy32, gy64, rtol=0, atol=1e-18)


@pytest.mark.parametrize("padding", ["valid", "same"])
def test_volume_point_samples_agree_with_whole_volume(padding):
    rng = np.random.default_rng(13)
    x = rng.random((1, 1, 14, 13, 15)).astype(np.float32)
    y = np.clip(x + rng.normal(0, 0.1, x.shape), 0, 1).astype(np.float32)
    dloss = 1.5
    _, gx, gy = oracle.ssim3_loss(x, y, padding, dloss=dloss)
    M = float(np.prod(oracle.out_shape3(14, 13, 15, padding)))
    for (t, u, v) in [(0, 0, 0), (13, 12, 14), (7, 6, 7), (0, 12, 3), (10, 1, 14)]:
        a, b = oracle.sample_grad3(x[0, 0], y[0, 0], padding, M, dloss, t, u, v)
        assert abs(a - gx[0, 0, t, u, v]) < 1e-16 + 1e-13 * np.abs(gx).max()
        assert abs(b - gy[0, 0, t, u, v]) < 1e-16 + 1e-13 * np.abs(gy).max()
