"""The allocation-free entry point (ssim_loss_and_grad_noalloc) against the
entry point it varies (ssim_loss_and_grad, with a caller's workspace), both
through the C ABI: the same kernel, so the same bits, and both within the
contract's tolerance of the oracle.  Two calls in a row, the second on a
smaller input, so that the second starts from the accumulator the first
left behind."""
import numpy as np
import pytest

from gpu_util import check_grad, check_loss, say

pytestmark = pytest.mark.gpu


def _pair(shape, seed):
    from ssim_loss_amd.inputs import make_pair

    return make_pair(shape, "uniform", 0.05, seed)


def test_noalloc_matches_loss_and_grad_on_two_calls():
    import torch

    import oracle
    import ssim_loss_amd as S

    dev = torch.device("cuda")
    ws = S.workspace_for(dev)
    for shape, padding, seed in (((2, 3, 300, 520), "valid", 11), ((1, 2, 70, 90), "same", 12)):
        say("noalloc", shape, padding, seed)
        x, y = _pair(shape, seed)
        t1 = torch.from_numpy(x).to(dev)
        t2 = torch.from_numpy(y).to(dev)
        dl = torch.tensor(0.75, dtype=torch.float32, device=dev)
        l_ref, l_na = (torch.empty((), dtype=torch.float32, device=dev) for _ in range(2))
        g_ref = (torch.empty_like(t1), torch.empty_like(t2))
        g_na = (torch.full_like(t1, float("nan")), torch.full_like(t2, float("nan")))
        S.ssim_loss_and_grad(t1, t2, padding, dl, l_ref, ws, *g_ref)
        S.ssim_loss_and_grad_noalloc(t1, t2, padding, dl, l_na, *g_na)
        torch.cuda.synchronize()
        assert l_na.item() == l_ref.item(), (l_na.item(), l_ref.item())
        for a, b in zip(g_na, g_ref):
            assert torch.equal(a, b)
        ol, ogx, ogy = oracle.ssim_loss(x, y, padding, dloss=0.75)
        check_loss(float(l_na.item()), ol, f"noalloc {shape} {padding}")
        check_grad(g_na[0].cpu().numpy(), ogx, "noalloc grad_img1")
        check_grad(g_na[1].cpu().numpy(), ogy, "noalloc grad_img2")


def test_noalloc_repeated_calls_leave_the_accumulator_clear():
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    x, y = _pair((1, 1, 64, 64), 0)
    t1 = torch.from_numpy(x).to(dev)
    t2 = torch.from_numpy(y).to(dev)
    dl = torch.ones((), dtype=torch.float32, device=dev)
    losses = []
    for _ in range(5):
        loss = torch.empty((), dtype=torch.float32, device=dev)
        S.ssim_loss_and_grad_noalloc(t1, t2, "valid", dl, loss, None, None)
        losses.append(loss)
    torch.cuda.synchronize()
    vals = {float(l.item()) for l in losses}
    assert len(vals) == 1, vals


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
def test_noalloc_half_images_match_loss_and_grad(dtype):
    """Half-precision images and gradients: the same bits as
    ssim_loss_and_grad, on two calls in a row (the second smaller)."""
    import torch

    import ssim_loss_amd as S

    dev = torch.device("cuda")
    ws = S.workspace_for(dev)
    td = getattr(torch, dtype)
    for shape, padding, seed in (((1, 3, 260, 400), "same", 21), ((1, 1, 40, 60), "valid", 22)):
        say("noalloc", dtype, shape, padding, seed)
        x, y = _pair(shape, seed)
        t1 = torch.from_numpy(x).to(dev).to(td)
        t2 = torch.from_numpy(y).to(dev).to(td)
        dl = torch.tensor(64.0, dtype=torch.float32, device=dev)
        l_ref, l_na = (torch.empty((), dtype=torch.float32, device=dev) for _ in range(2))
        g_ref = (torch.empty_like(t1), torch.empty_like(t2))
        g_na = (torch.full_like(t1, float("nan")), torch.full_like(t2, float("nan")))
        S.ssim_loss_and_grad(t1, t2, padding, dl, l_ref, ws, *g_ref)
        S.ssim_loss_and_grad_noalloc(t1, t2, padding, dl, l_na, *g_na)
        torch.cuda.synchronize()
        assert l_na.item() == l_ref.item(), (l_na.item(), l_ref.item())
        for a, b in zip(g_na, g_ref):
            assert torch.equal(a, b)
