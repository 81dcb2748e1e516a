"""Edge, ragged, random and degenerate cases of the HIP path against the
oracle (and against closed forms where the oracle's answer is known)."""
import numpy as np
import pytest

import oracle
from ssim_loss_amd.inputs import FLAT_LEVELS, flat_pair, make_pair

from gpu_util import GRAD_RTOL, check_grad, check_loss, gpu_run, say

pytestmark = pytest.mark.gpu

# sizes around the window (11), the strip (244 outputs / 256 inputs), the
# 4-wide output groups and the 4-row batches
EDGE_HW = [(11, 11), (12, 13), (13, 12), (20, 21), (21, 20), (31, 64), (63, 65), (64, 64),
           (65, 63), (127, 129), (254, 11), (11, 254), (255, 256), (256, 257), (257, 255),
           (100, 498), (60, 499), (33, 500), (14, 1001), (1001, 14)]


@pytest.mark.parametrize("padding", ["valid", "same"])
@pytest.mark.parametrize("hw", EDGE_HW, ids=lambda hw: f"{hw[0]}x{hw[1]}")
def test_edge_shapes(hw, padding):
    H, W = hw
    say(f"[edge] {H}x{W} {padding}")
    x, y = make_pair((1, 2, H, W), "uniform", 0.1, seed=H * 1000 + W)
    gl, g1, g2 = gpu_run(x, y, padding, dloss=1.7)
    ol, o1, o2 = oracle.ssim_loss(x, y, padding, dloss=1.7)
    check_loss(gl, ol)
    check_grad(g1, o1, "grad_img1")
    check_grad(g2, o2, "grad_img2")


@pytest.mark.parametrize("H,W", [(1, 1), (1, 7), (5, 1), (3, 3), (10, 10)])
def test_same_padding_images_smaller_than_window(H, W):
    say(f"[edge] tiny same {H}x{W}")
    x, y = make_pair((2, 1, H, W), "uniform", 0.2, seed=H + 7 * W)
    gl, g1, g2 = gpu_run(x, y, "same")
    ol, o1, o2 = oracle.ssim_loss(x, y, "same")
    check_loss(gl, ol)
    check_grad(g1, o1, "grad_img1")
    check_grad(g2, o2, "grad_img2")


def _random_cases(n=40):
    rng = np.random.default_rng(2024)
    cases = []
    for k in range(n):
        N = int(rng.integers(1, 4))
        C = int(rng.integers(1, 5))
        H = int(rng.integers(11, 300))
        W = int(rng.integers(11, 600))
        cases.append((k, N, C, H, W, "valid" if rng.random() < 0.5 else "same",
                      ["uniform", "field"][int(rng.integers(2))], float(rng.uniform(0.01, 0.3))))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"r{c[0]}")
def test_random_shapes(case):
    k, N, C, H, W, padding, kind, noise = case
    say(f"[random] {k}: {N}x{C}x{H}x{W} {padding} {kind} noise {noise:.3f}")
    x, y = make_pair((N, C, H, W), kind, noise, seed=100 + k)
    dloss = [1.0, -0.5, 3.0][k % 3]
    gl, g1, g2 = gpu_run(x, y, padding, dloss=dloss)
    ol, o1, o2 = oracle.ssim_loss(x, y, padding, dloss=dloss)
    check_loss(gl, ol)
    check_grad(g1, o1, "grad_img1")
    check_grad(g2, o2, "grad_img2")


@pytest.mark.parametrize("padding", ["valid", "same"])
def test_identical_images_give_exact_zero(padding):
    """x = y: SSIM is exactly 1 and both gradients vanish (oracle pins).  The
    kernels form 1 - S and every partial from x - y, mu_x - mu_y and
    var(x - y), which are exactly zero here, so the fp32 result is exact."""
    say(f"[stability] identical {padding}")
    x, _ = make_pair((1, 3, 96, 80), "field", 0.05, seed=3)
    gl, g1, g2 = gpu_run(x, x, padding)
    assert gl == 0.0
    assert not g1.any() and not g2.any()
    for v in (0.0, 1.0):
        c = np.full((2, 1, 32, 32), v, np.float32)
        gl, g1, g2 = gpu_run(c, c, padding)
        assert gl == 0.0 and not g1.any() and not g2.any()


def constant_grad_bar(a, b):
    """The gradient bar for images constant at levels a and b: the contract's
    1e-4 of the largest gradient, or the fp32 error of the chain rule's
    cancellation if that is larger.  With zero variance and different means,
    the mean path (B^T of the mu_x partial) and the second-moment path
    ((x - y) B^T of the R partial) each carry about S B1 / B2 times the
    gradient they add up to (B1 = a^2 + b^2 + C1, B2 = C2), so their fp32
    rounding, a few units of 2^-24 of each, shows at 2^-24 B1 / C2 of the
    result; 32 units of that bound it.  Every separable adjoint in fp32 has
    this cancellation; the loss itself keeps the contract's bar."""
    b1 = a * a + b * b + 1e-4
    return max(GRAD_RTOL, 32 * 2.0 ** -24 * b1 / 9e-4)


@pytest.mark.parametrize("padding", ["valid", "same"])
@pytest.mark.parametrize("a,b", [(0.25, 0.75), (0.0, 1.0), (0.9, 0.1), (0.5, 0.5), (0.05, 0.95),
                                 (0.3, 0.31), (13 / 255, 14 / 255), (1.0, 0.98)])
def test_constant_images(a, b, padding):
    """Constant images against the oracle: the loss at the contract's bar (and
    in valid padding against S = (2ab + C1)/(a^2 + b^2 + C1)), the gradients
    at constant_grad_bar.  The variances vanish, so a rounding bias in a
    blurred mean or in B((x - y)^2) would be divided by C2 = 9e-4: the
    forward blurs by parts, which gives a constant window's value exactly."""
    say(f"[stability] constant {a} {b} {padding}")
    x = np.full((1, 2, 40, 50), a, np.float32)
    y = np.full((1, 2, 40, 50), b, np.float32)
    gl, g1, g2 = gpu_run(x, y, padding)
    if a == b:  # identical images: exactly zero (the oracle shows fp64 noise here)
        assert gl == 0.0 and not g1.any() and not g2.any()
        return
    ol, o1, o2 = oracle.ssim_loss(x, y, padding)
    check_loss(gl, ol, f"constant {a} {b} {padding}")
    if padding == "valid":
        af, bf = float(np.float32(a)), float(np.float32(b))
        S = (2 * af * bf + 1e-4) / (af * af + bf * bf + 1e-4)
        assert abs(gl - (1 - S)) <= 1e-5 * abs(1 - S)
    bar = constant_grad_bar(a, b)
    for g, og in ((g1, o1), (g2, o2)):
        err = float(np.abs(g.astype(np.float64) - og).max())
        assert err <= bar * float(np.abs(og).max()), (err, bar)


def test_zero_against_one():
    say("[stability] zeros vs ones")
    z = np.zeros((1, 1, 32, 32), np.float32)
    o = np.ones((1, 1, 32, 32), np.float32)
    gl, g1, g2 = gpu_run(z, o, "same")
    ol, o1, o2 = oracle.ssim_loss(z, o, "same")
    check_loss(gl, ol, "zeros vs ones")
    bar = constant_grad_bar(0.0, 1.0)
    for g, og in ((g1, o1), (g2, o2)):
        assert float(np.abs(g - og).max()) <= bar * float(np.abs(og).max())


def _flat_case(a, b, padding, what):
    """a, b through the saved-maps pair and the one-launch step, against the
    oracle at the contract's bars (upstream gradient 0.5)."""
    import torch

    import ssim_loss_amd as S

    ol, o1, o2 = oracle.ssim_loss(a, b, padding, dloss=0.5)
    gl, g1, g2 = gpu_run(a, b, padding, dloss=0.5)
    check_loss(gl, ol, f"{what} saved maps")
    check_grad(g1, o1, f"{what} grad_img1")
    check_grad(g2, o2, f"{what} grad_img2")
    dev = torch.device("cuda")
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    lo, h1, h2 = S.loss_and_grad(ta, tb, padding, weight=0.5)
    check_loss(float(lo.item()), ol, f"{what} one launch")
    check_grad(h1.cpu().numpy(), o1, f"{what} one launch grad_img1")
    check_grad(h2.cpu().numpy(), o2, f"{what} one launch grad_img2")


@pytest.mark.parametrize("padding", ["valid", "same"])
@pytest.mark.parametrize("level", FLAT_LEVELS)
def test_flat_image_against_noisy_one(level, padding):
    """One image flat at a level, the other a noisy copy, each way round (a
    render flat where the reference has texture).  At 0.05 and 0.95 the
    offset from 1/2 is inexact in fp32, and a blur of the flat image that
    misrounded its mean would bias the covariance of every window by the same
    amount: the loss would miss the bar by about 3e-5."""
    for noise in (0.01, 0.001):
        x, y = flat_pair((1, 2, 150, 190), level, noise, seed=int(level * 1000))
        for a, b in ((x, y), (y, x)):
            say(f"[flat] level {level:.4f} noise {noise} {padding}")
            _flat_case(a, b, padding, f"flat {level:.4f}")


@pytest.mark.parametrize("padding", ["valid", "same"])
@pytest.mark.parametrize("kind,noise", [("objects", 0.01), ("objects", 0.003),
                                        ("dark-field", 0.005), ("dark-field", 0.002)])
def test_objects_and_dark_fields(kind, noise, padding):
    """Flat rectangles on a black background, and dark low-contrast fields,
    with the noise on the second image -- and swapped."""
    for seed in range(2):
        x, y = make_pair((1, 3, 150, 190), kind, noise, seed=400 + seed)
        for a, b in ((x, y), (y, x)):
            say(f"[flat] {kind} noise {noise} {padding} seed {seed}")
            _flat_case(a, b, padding, kind)


@pytest.mark.parametrize("padding", ["valid", "same"])
@pytest.mark.parametrize("lo,hi", [(-0.5, 1.5), (-1.0, 2.0), (0.0, 4.0), (0.0, 255.0)])
def test_values_outside_the_unit_range(lo, hi, padding):
    """The pages take images in [0, 1], and C1 and C2 assume that range, but
    the formula is defined for any values: uniform images on [lo, hi] against
    a copy with noise of 5% of the range, unclamped, at the contract's bars
    (the kernels' shift by 1/2 is exact arithmetic, not an assumption on the
    range)."""
    rng = np.random.default_rng(5)
    x = rng.uniform(lo, hi, (1, 2, 120, 150))
    y = (x + rng.normal(0.0, 0.05 * (hi - lo), x.shape)).astype(np.float32)
    x = x.astype(np.float32)
    say(f"[range] [{lo}, {hi}] {padding}")
    _flat_case(x, y, padding, f"range [{lo}, {hi}]")


def test_nullable_gradients_and_dloss_scaling():
    say("[api] grad_img1 / grad_img2 = NULL, dloss scaling")
    x, y = make_pair((2, 3, 70, 90), "uniform", 0.1, seed=11)
    _, a1, a2 = gpu_run(x, y, "valid", dloss=1.0)
    _, b1, b2 = gpu_run(x, y, "valid", dloss=-2.5)
    np.testing.assert_allclose(b1, -2.5 * a1, rtol=1e-6, atol=1e-12)
    np.testing.assert_allclose(b2, -2.5 * a2, rtol=1e-6, atol=1e-12)
    _, c1, c2 = gpu_run(x, y, "valid", grad2=False)
    assert c2 is None
    np.testing.assert_array_equal(c1, a1)
    _, d1, d2 = gpu_run(x, y, "valid", grad1=False)
    assert d1 is None
    np.testing.assert_array_equal(d2, a2)


def test_inference_forward_matches_training_forward():
    say("[api] saved_maps = NULL")
    x, y = make_pair((1, 3, 200, 300), "field", 0.05, seed=12)
    for padding in ("valid", "same"):
        lt, _, _ = gpu_run(x, y, padding)
        li, _, _ = gpu_run(x, y, padding, train=False)
        assert abs(lt - li) <= 1e-7 * abs(lt)


def test_deterministic_run_to_run():
    say("[api] determinism")
    x, y = make_pair((2, 3, 150, 260), "uniform", 0.05, seed=13)
    r = [gpu_run(x, y, "valid") for _ in range(3)]
    for k in (1, 2):
        assert r[k][0] == r[0][0]
        np.testing.assert_array_equal(r[k][1], r[0][1])
        np.testing.assert_array_equal(r[k][2], r[0][2])


@pytest.mark.parametrize("recompute", [True, False])
def test_autograd_functions(recompute):
    import torch

    import ssim_loss_amd as S

    say(f"[api] autograd recompute={recompute}")
    x, y = make_pair((2, 3, 64, 96), "uniform", 0.1, seed=14)
    dev = torch.device("cuda")
    t1 = torch.from_numpy(x).to(dev).requires_grad_(True)
    t2 = torch.from_numpy(y).to(dev)
    loss = S.ssim_loss(t1, t2, "valid", recompute=recompute)
    (0.5 * loss).backward()
    ol, o1, _ = oracle.ssim_loss(x, y, "valid", dloss=0.5)
    check_loss(float(loss.item()), ol)
    check_grad(t1.grad.cpu().numpy(), o1, "grad_img1")
    assert t2.grad is None
    # fused_ssim: mean SSIM, default padding "same"
    t1.grad = None
    s = S.fused_ssim(t1, t2)
    s.backward()
    sl, s1, _ = oracle.ssim_loss(x, y, "same", dloss=-1.0)
    assert abs(float(s.item()) - (1 - sl)) <= 1e-5 * abs(sl)
    check_grad(t1.grad.cpu().numpy(), s1, "fused_ssim grad")
    with torch.no_grad():
        v = S.fused_ssim(t1, t2, train=False)
    assert abs(float(v.item()) - (1 - sl)) <= 1e-5 * abs(sl)


def test_grad_scale_is_the_fp32_product():
    """ssim_grad_scale: out = *dloss * grad, element for element the fp32
    product, for ragged lengths, 4-byte (not 16-byte) aligned arrays and in
    place; n = 0 launches nothing."""
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    rng = np.random.default_rng(31)
    for n, off_g, off_o in [(1, 0, 0), (3, 0, 0), (4, 0, 0), (1023, 0, 0), (4097, 1, 3),
                            (6220800, 0, 0), (6220803, 2, 0), (0, 0, 0)]:
        say(f"[scale] n={n} offsets {off_g} {off_o}")
        g = rng.standard_normal(n + 4).astype(np.float32)
        s = np.float32(rng.uniform(-3, 3))
        tg = torch.from_numpy(g).to(dev)
        out = torch.full((n + 4,), 7.0, device=dev)
        dl = torch.tensor(float(s), dtype=torch.float32, device=dev)
        S.ssim_grad_scale(dl, tg[off_g:off_g + n], out[off_o:off_o + n])
        res = out.cpu().numpy()
        want = s * g[off_g:off_g + n]
        assert np.array_equal(res[off_o:off_o + n], want)
        assert (res[:off_o] == 7.0).all() and (res[off_o + n:] == 7.0).all()
        S.ssim_grad_scale(dl, tg[:n], tg[:n])  # in place
        assert np.array_equal(tg[:n].cpu().numpy(), s * g[:n])
    with pytest.raises(S.SsimError):
        a = torch.zeros(64, device=dev)
        S.ssim_grad_scale(torch.ones((), device=dev), a[:32], a[16:48])


@pytest.mark.parametrize("which", ["both", "img1", "img2"])
def test_autograd_fp32_matches_the_one_launch_step_bit_for_bit(which):
    """fp32 autograd (the forward forms the gradients with an upstream
    gradient of 1, the backward scales them): the gradients equal
    ssim_loss_and_grad's with the same upstream gradient bit for bit, for
    either image or both, and a second backward through a retained graph
    gives them again."""
    import torch

    import ssim_loss_amd as S

    say(f"[api] autograd fp32 early gradients, {which}")
    x, y = make_pair((2, 3, 70, 300), "uniform", 0.1, seed=15)
    dev = torch.device("cuda")
    t1 = torch.from_numpy(x).to(dev).requires_grad_(which in ("both", "img1"))
    t2 = torch.from_numpy(y).to(dev).requires_grad_(which in ("both", "img2"))
    loss = S.ssim_loss(t1, t2, "valid")
    w = torch.tensor(-0.37, device=dev)
    (w * loss).backward(retain_graph=True)
    l_ref, g1_ref, g2_ref = S.loss_and_grad(t1.detach(), t2.detach(), "valid", weight=w)
    torch.cuda.synchronize()
    ol, o1, o2 = oracle.ssim_loss(x, y, "valid", dloss=-0.37)
    check_loss(float(loss.item()), ol)
    assert float(loss.item()) == float(l_ref.item())
    for t, ref, o in ((t1, g1_ref, o1), (t2, g2_ref, o2)):
        if t.requires_grad:
            assert torch.equal(t.grad, ref)
            check_grad(t.grad.cpu().numpy(), o)
        else:
            assert t.grad is None
    first = [t.grad.clone() if t.grad is not None else None for t in (t1, t2)]
    for t in (t1, t2):
        t.grad = None
    (w * loss).backward()
    for t, f in zip((t1, t2), first):
        assert (t.grad is None) == (f is None)
        if f is not None:
            assert torch.equal(t.grad, f)
    # without grad mode the forward forms the loss alone
    with torch.no_grad():
        v = S.ssim_loss(t1, t2, "valid")
    check_loss(float(v.item()), ol)


def test_workspace_reuse_across_shapes():
    """The completion counter is reset by every forward, so one workspace
    serves calls of any size in sequence."""
    say("[api] workspace reuse")
    for k, shape in enumerate([(1, 1, 300, 300), (1, 1, 20, 20), (3, 2, 120, 80), (1, 1, 20, 20)]):
        x, y = make_pair(shape, "uniform", 0.1, seed=20 + k)
        gl, _, _ = gpu_run(x, y, "same", train=False)
        ol, _, _ = oracle.ssim_loss(x, y, "same", grads=False)
        check_loss(gl, ol)


def test_two_streams_get_their_own_workspaces():
    """Loss-forming calls on two streams may overlap: the binding keeps one
    workspace per (device, stream), and each stream's losses stay exact."""
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    pairs = [make_pair((2, 3, 150, 400), "uniform", 0.1, seed=70 + k) for k in range(2)]
    refs = [oracle.ssim_loss(x, y, "same", grads=False)[0] for x, y in pairs]
    streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    data = []
    for (x, y), st in zip(pairs, streams):
        with torch.cuda.stream(st):
            t1 = torch.from_numpy(x).to(dev)
            t2 = torch.from_numpy(y).to(dev)
            data.append((t1, t2, torch.empty((), dtype=torch.float32, device=dev),
                         torch.empty_like(t1), torch.empty_like(t2), S.workspace_for(dev)))
    assert data[0][5].data_ptr() != data[1][5].data_ptr()
    torch.cuda.synchronize()
    dl = torch.tensor(1.0, device=dev)
    losses = [[], []]
    for _ in range(5):
        for k, st in enumerate(streams):
            t1, t2, loss, g1, g2, _ = data[k]
            with torch.cuda.stream(st):
                S.ssim_loss_and_grad(t1, t2, "same", dl, loss, S.workspace_for(dev), g1, g2)
                losses[k].append(loss.clone())
    torch.cuda.synchronize()
    for k in range(2):
        for v in losses[k]:
            check_loss(float(v.item()), refs[k], f"stream {k}")


def test_graph_capture_replays_match_eager():
    """A training step captured in a HIP graph (the one-launch kernel, and the
    saved-maps forward + backward pair) replays with new image contents each
    time, with eager work and synchronisations between replays, and every
    replay equals the eager launches bit for bit.  The kernels record no
    memset: the loss accumulator resets itself."""
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    shape = (2, 3, 120, 333)
    t1 = torch.empty(shape, dtype=torch.float32, device=dev)
    t2 = torch.empty_like(t1)
    g1, g2, e1, e2 = (torch.empty_like(t1) for _ in range(4))
    loss = torch.empty((), dtype=torch.float32, device=dev)
    loss_e = torch.empty_like(loss)
    dl = torch.tensor(0.7, device=dev)
    ws = torch.zeros(S.ssim_workspace_bytes(), dtype=torch.uint8, device=dev)
    ws_e = torch.zeros_like(ws)
    maps = S.alloc_saved_maps(t1, "valid")
    steps = {
        "one launch": lambda w, l, a, b: S.ssim_loss_and_grad(t1, t2, "valid", dl, l, w, a, b),
        "saved maps": lambda w, l, a, b: (S.ssim_forward(t1, t2, "valid", l, maps, w),
                                          S.ssim_backward(dl, t1, t2, "valid", maps, a, b)),
    }
    for name, step in steps.items():
        x, y = make_pair(shape, "uniform", 0.1, seed=80)
        t1.copy_(torch.from_numpy(x))
        t2.copy_(torch.from_numpy(y))
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step(ws, loss, g1, g2)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(ws, loss, g1, g2)
        for k in range(4):
            say(f"  {name}: replay {k}")
            x, y = make_pair(shape, "uniform", 0.05 + 0.05 * k, seed=81 + k)
            t1.copy_(torch.from_numpy(x))
            t2.copy_(torch.from_numpy(y))
            graph.replay()
            torch.cuda.synchronize()
            step(ws_e, loss_e, e1, e2)
            torch.cuda.synchronize()
            assert float(loss.item()) == float(loss_e.item()), (name, k)
            assert torch.equal(g1, e1) and torch.equal(g2, e2), (name, k)
            if k == 0:
                ol, _, _ = oracle.ssim_loss(x, y, "valid", grads=False)
                check_loss(float(loss.item()), ol, name)


def test_non_finite_input_gives_nan_loss_and_leaves_the_workspace_ready():
    """A NaN or infinite pixel makes the loss NaN (as the plain definition
    does) in every loss-forming kernel: the strip forward (training and
    inference), the one-launch step, the cached-reference step and the volume
    forward.  The reduction's accumulator is reset either way, so the next
    call on the same workspace is exact again."""
    import math

    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    ws = S.workspace_for(dev)
    x, y = make_pair((2, 3, 70, 300), "uniform", 0.1, seed=91)
    ol, _, _ = oracle.ssim_loss(x, y, "valid", grads=False)
    t2 = torch.from_numpy(y).to(dev)
    ref = S.reference_stats(t2, "valid")
    loss = torch.empty((), dtype=torch.float32, device=dev)
    dl = torch.tensor(1.0, device=dev)
    g1 = torch.empty_like(t2)
    g2 = torch.empty_like(t2)
    maps = S.alloc_saved_maps(t2, "valid")
    runs = {
        "forward": lambda a: S.ssim_forward(a, t2, "valid", loss, maps, ws),
        "forward(inference)": lambda a: S.ssim_forward(a, t2, "valid", loss, None, ws),
        "loss_and_grad": lambda a: S.ssim_loss_and_grad(a, t2, "valid", dl, loss, ws, g1, g2),
        "loss_and_grad_ref": lambda a: S.ssim_loss_and_grad_ref(a, t2, ref, "valid", dl, loss,
                                                                ws, g1),
    }
    for bad in (float("nan"), float("inf")):
        xb = x.copy()
        xb[1, 2, 33, 150] = bad
        tb = torch.from_numpy(xb).to(dev)
        tx = torch.from_numpy(x).to(dev)
        for name, run in runs.items():
            say(f"  {name} with {bad}")
            run(tb)
            torch.cuda.synchronize()
            assert math.isnan(float(loss.item())), name
            run(tx)
            torch.cuda.synchronize()
            check_loss(float(loss.item()), ol, name)
    xv, yv = make_pair((1, 2, 20, 19, 18), "uniform", 0.1, seed=92)
    ov, _, _ = oracle.ssim3_loss(xv, yv, "same", grads=False)
    tv2 = torch.from_numpy(yv).to(dev)
    xvb = xv.copy()
    xvb[0, 1, 7, 8, 9] = float("nan")
    S.ssim3d_forward(torch.from_numpy(xvb).to(dev), tv2, "same", loss, None, ws)
    torch.cuda.synchronize()
    assert math.isnan(float(loss.item())), "ssim3d_forward"
    S.ssim3d_forward(torch.from_numpy(xv).to(dev), tv2, "same", loss, None, ws)
    torch.cuda.synchronize()
    check_loss(float(loss.item()), ov, "ssim3d_forward")


def test_rejects_bad_inputs_on_gpu():
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    a = torch.rand(1, 1, 32, 32, device=dev)
    with pytest.raises(ValueError):
        S.ssim_loss(a, torch.rand(1, 1, 32, 31, device=dev))
    with pytest.raises(ValueError):
        S.ssim_loss(a.transpose(2, 3), a)
    with pytest.raises(S.SsimError):
        S.ssim_loss(torch.rand(1, 1, 8, 32, device=dev), torch.rand(1, 1, 8, 32, device=dev), "valid")


def test_rejects_bad_buffers_before_any_launch():
    """Output and state buffers that the kernels would write or read out of
    bounds (on the host, too small, strided, of the wrong type, or a second
    image of another shape) are refused by the binding; nothing is launched,
    so the good buffers keep the values they were filled with."""
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    a = torch.rand(1, 2, 24, 40, device=dev)
    b = torch.rand(1, 2, 24, 40, device=dev)
    ws = S.workspace_for(dev)
    loss = torch.full((), 7.0, device=dev)
    dl = torch.ones((), device=dev)
    g1 = torch.full_like(a, 3.0)
    g2 = torch.full_like(a, 3.0)
    maps = S.alloc_saved_maps(a, "valid")
    small_maps = maps[: maps.numel() - 4]
    ref = S.reference_stats(b, "valid")
    cases = {
        "grad on the host": lambda: S.ssim_loss_and_grad(a, b, "valid", dl, loss, ws,
                                                         torch.empty(a.shape), g2),
        "strided grad": lambda: S.ssim_backward_recompute(
            dl, a, b, "valid", torch.empty(1, 2, 24, 80, device=dev)[..., ::2], g2),
        "grad of another dtype": lambda: S.ssim_backward_recompute(
            dl, a, b, "valid", g1.double(), g2),
        "loss on the host": lambda: S.ssim_forward(a, b, "valid", torch.empty(()), None, ws),
        "fp64 loss": lambda: S.ssim_loss_and_grad(a, b, "valid", dl, loss.double(), ws, g1, g2),
        "empty dloss": lambda: S.ssim_backward_recompute(torch.empty(0, device=dev), a, b,
                                                         "valid", g1, g2),
        "small workspace": lambda: S.ssim_forward(a, b, "valid", loss, None, ws[:4]),
        "short saved maps (forward)": lambda: S.ssim_forward(a, b, "valid", loss, small_maps, ws),
        "short saved maps (backward)": lambda: S.ssim_backward(dl, a, b, "valid", small_maps, g1,
                                                               g2),
        "maps of another padding": lambda: S.ssim_forward(a, b, "same", loss, maps, ws),
        "second image of another shape": lambda: S.ssim_backward(
            dl, a, b[:, :1], "valid", maps, g1, g2),
        "short reference": lambda: S.ssim_loss_and_grad_ref(a, b, ref[:-1], "valid", dl, loss,
                                                             ws, g1),
        "volume maps short": lambda: S.ssim3d_forward(
            a.reshape(1, 1, 2, 24, 40), b.reshape(1, 1, 2, 24, 40), "same", loss,
            torch.empty(4, device=dev), ws),
    }
    torch.cuda.synchronize()
    for name, call in cases.items():
        say(f"[edge] bad buffer: {name}")
        with pytest.raises((TypeError, ValueError)):
            call()
    torch.cuda.synchronize()
    assert float(loss.item()) == 7.0
    assert bool((g1 == 3.0).all()) and bool((g2 == 3.0).all())


def test_maximum_plane_size():
    """Two planes of 2^27 elements (8192 x 16384, the documented limit; 1 GiB
    per tensor): the one-launch step (whose strips span both planes behind one
    descriptor, offsets near 1 GiB) and the saved-maps pair, each against the
    oracle's whole loss and its gradients at sampled pixels (corners, plane
    edges, strip boundaries, random points)."""
    import torch

    import ssim_loss_amd as S

    shape = (2, 1, 8192, 16384)
    N, C, H, W = shape
    say(f"[edge] maximum plane {shape}")
    x, y = make_pair(shape, "uniform", 0.05, seed=2027)
    M = float(N * C * (H - 10) * (W - 10))
    dloss = 0.9
    dev = torch.device("cuda")
    t1 = torch.from_numpy(x).to(dev)
    t2 = torch.from_numpy(y).to(dev)
    rng = np.random.default_rng(5)
    pts = [(n, 0, u, v) for n in range(N) for u in (0, 1, H - 2, H - 1)
           for v in (0, 9, 235, 236, W - 12, W - 1)]
    pts += [(int(rng.integers(N)), 0, int(rng.integers(H)), int(rng.integers(W))) for _ in range(120)]
    say("  oracle samples")
    o1 = np.zeros(len(pts))
    o2 = np.zeros(len(pts))
    for k, (n, c, u, v) in enumerate(pts):
        o1[k], o2[k] = oracle.sample_grad(x[n, c], y[n, c], "valid", M, dloss, u, v)
    say("  oracle loss")
    ol, _, _ = oracle.ssim_loss(x, y, "valid", grads=False)
    idx = torch.tensor(pts, dtype=torch.long, device=dev)

    def samples(g):
        return g[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].cpu().numpy().astype(np.float64)

    say("  one launch")
    loss, g1, g2 = S.loss_and_grad(t1, t2, "valid", weight=dloss)
    torch.cuda.synchronize()
    check_loss(float(loss.item()), ol, "one launch")
    check_grad(samples(g1), o1, "one launch grad_img1")
    check_grad(samples(g2), o2, "one launch grad_img2")
    del g1, g2
    say("  saved maps")
    ws = S.workspace_for(dev)
    maps = S.alloc_saved_maps(t1, "valid")
    dl = torch.tensor(dloss, device=dev)
    g1 = torch.empty_like(t1)
    g2 = torch.empty_like(t2)
    S.ssim_forward(t1, t2, "valid", loss, maps, ws)
    S.ssim_backward(dl, t1, t2, "valid", maps, g1, g2)
    torch.cuda.synchronize()
    check_loss(float(loss.item()), ol, "saved maps")
    check_grad(samples(g1), o1, "saved maps grad_img1")
    check_grad(samples(g2), o2, "saved maps grad_img2")
