"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, and rejects bad arguments with the
documented codes before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import ssim_loss_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssim_loss_amd.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssim(?:3d)?_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ["ssim_forward", "ssim_backward", "ssim_forward_typed", "ssim_backward_typed",
              "ssim_backward_recompute", "ssim_loss_and_grad", "ssim_reference_bytes",
              "ssim_reference_stats", "ssim_loss_and_grad_ref", "ssim3d_forward",
              "ssim3d_backward", "ssim3d_saved_maps_bytes", "ssim3d_map_shape",
              "ssim_saved_maps_bytes", "ssim_workspace_bytes", "ssim_strerror",
              "ssim_abi_version", "ssim_taps", "ssim_map_shape"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(S.build.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(lib, n), n


def test_abi_version_and_strerror():
    # the header, the built library and the bindings agree on the version
    hdr = open(HEADER).read()
    v = int(re.search(r"#define SSIM_ABI_VERSION (\d+)", hdr).group(1))
    assert S.ssim_abi_version() == v == S.ABI_VERSION
    for code in range(0, -10, -1):
        assert S.ssim_strerror(code)
    assert "unknown" in S.ssim_strerror(-99)


def test_kernel_taps_are_the_oracle_taps_rounded_once():
    g = np.array(S.ssim_taps(), np.float32)
    np.testing.assert_array_equal(g, oracle.taps().astype(np.float32))
    np.testing.assert_array_equal(g, g[::-1])


@pytest.mark.parametrize("H,W,padding", [(11, 11, "valid"), (64, 37, "valid"), (1, 1, "same"),
                                         (1080, 1920, "same"), (2160, 3840, "valid")])
def test_map_shape_matches_oracle(H, W, padding):
    assert S.ssim_map_shape(H, W, padding) == oracle.out_shape(H, W, padding)


def test_saved_maps_bytes():
    # four fp32 map planes per image plane, row pitch = Wo rounded up to 4
    assert S.ssim_saved_maps_bytes(1, 3, 1080, 1920, "valid") == 16 * 3 * 1070 * 1912
    assert S.ssim_saved_maps_bytes(1, 3, 1080, 1920, "same") == 16 * 3 * 1080 * 1920
    assert S.ssim_saved_maps_bytes(8, 3, 2160, 3840, "valid") == 16 * 24 * 2150 * 3832
    assert S.ssim_saved_maps_bytes(1, 1, 10, 30, "valid") == 0
    assert S.ssim_saved_maps_bytes(1, 1, 30, 30, 7) == 0
    assert S.ssim_workspace_bytes() >= 8 and S.ssim_workspace_bytes() % 8 == 0


def _fwd(lib, img1=0x1000, img2=0x100000, N=1, C=1, H=64, W=64, padding=0, loss=0x200000,
         maps=0x300000, ws=0x900000):
    return lib.ssim_forward(img1, img2, N, C, H, W, padding, loss, maps, ws, None)


def _bwd(lib, dloss=0x1000, img1=0x10000, img2=0x100000, N=1, C=1, H=64, W=64, padding=0,
         maps=0x300000, g1=0x900000, g2=0xA00000):
    return lib.ssim_backward(dloss, img1, img2, N, C, H, W, padding, maps, g1, g2, None)


def test_forward_argument_errors_return_before_any_hip_call():
    lib = S.lib()
    assert _fwd(lib, img1=None) == -1
    assert _fwd(lib, loss=None) == -1
    assert _fwd(lib, ws=None) == -1
    assert _fwd(lib, padding=2) == -3
    assert _fwd(lib, N=0) == -2
    assert _fwd(lib, C=-1) == -2
    assert _fwd(lib, H=10) == -2          # valid needs H >= 11
    assert _fwd(lib, W=10) == -2
    assert _fwd(lib, H=(1 << 14) + 1, W=1 << 13) == -4   # a plane over 2^27 elements
    assert _fwd(lib, H=11, W=(1 << 20) + 1) == -4  # a row longer than 2^20
    assert _fwd(lib, maps=0x300004) == -2          # saved maps must be 16-byte aligned
    assert _fwd(lib, loss=0x1000 + 64) == -5       # loss inside img1
    assert _fwd(lib, maps=0x100000 + 4096) == -5   # maps overlap img2
    assert _fwd(lib, ws=0x300000 + 1024) == -5     # workspace overlaps maps


def test_backward_argument_errors_return_before_any_hip_call():
    lib = S.lib()
    assert _bwd(lib, dloss=None) == -1
    assert _bwd(lib, maps=None) == -1
    assert _bwd(lib, img2=None) == -1
    assert _bwd(lib, padding=-1) == -3
    assert _bwd(lib, H=5, padding=0) == -2
    assert _bwd(lib, g1=0x10000 + 128) == -5          # grad overlaps img1
    assert _bwd(lib, g2=0x900000 + 8) == -5           # grads overlap each other
    assert _bwd(lib, g1=0x300000 + 16) == -5          # grad overlaps the maps
    assert _bwd(lib, g1=None, g2=None) == 0           # nothing to do: no launch


def test_typed_entry_points_validate_dtype_and_alignment():
    lib = S.lib()
    fwd = lambda dt, **kw: lib.ssim_forward_typed(
        kw.get("img1", 0x1000), 0x100000, dt, 1, 1, 64, kw.get("W", 64), 0, 0x200000,
        kw.get("maps", 0x300000), 0x900000, None)
    bwd = lambda dt: lib.ssim_backward_typed(0x1000, 0x10000, 0x100000, dt, 1, 1, 64, 64, 0,
                                             0x300000, 0x900000, 0xA00000, None)
    for dt in (3, -1, 99):
        assert fwd(dt) == -8
        assert bwd(dt) == -8
    assert fwd(1, img1=None) == -1
    assert fwd(2, W=10) == -2
    assert fwd(1, maps=0x300008) == -2
    assert fwd(1, img1=0x1001) == -2          # a half image must be 2-byte aligned
    assert _fwd(lib, img1=0x1002) == -2       # an fp32 image 4-byte aligned
    assert _bwd(lib, g1=0x900002) == -2
    # a half-precision plane of 2^27 elements is still the limit
    assert lib.ssim_forward_typed(0x1000, 0x100000, 1, 1, 1, (1 << 14) + 1, 1 << 13, 0,
                                  0x200000, None, 0x900000, None) == -4


def test_typed_overlap_uses_element_size():
    lib = S.lib()
    # a 64x64 fp16 image at 0x10000 spans 8 KiB; a loss 4 KiB in overlaps it
    assert lib.ssim_forward_typed(0x10000, 0x100000, 1, 1, 1, 64, 64, 0, 0x10000 + 4096,
                                  None, 0x900000, None) == -5
    assert S.ssim_strerror(-8)


def _rec(lib, dloss=0x1000, img1=0x10000, img2=0x100000, dt=0, N=1, C=1, H=64, W=64, padding=0,
         g1=0x900000, g2=0xA00000):
    return lib.ssim_backward_recompute(dloss, img1, img2, dt, N, C, H, W, padding, g1, g2, None)


def _lag(lib, img1=0x10000, img2=0x100000, dt=0, N=1, C=1, H=64, W=64, padding=0, dloss=0x1000,
         loss=0x2000, ws=0x300000, g1=0x900000, g2=0xA00000):
    return lib.ssim_loss_and_grad(img1, img2, dt, N, C, H, W, padding, dloss, loss, ws, g1, g2,
                                  None)


def test_recompute_argument_errors_return_before_any_hip_call():
    lib = S.lib()
    assert _rec(lib, dloss=None) == -1
    assert _rec(lib, img1=None) == -1
    assert _rec(lib, dt=5) == -8
    assert _rec(lib, padding=3) == -3
    assert _rec(lib, H=10) == -2
    assert _rec(lib, img2=0x100002) == -2           # fp32 image not 4-byte aligned
    assert _rec(lib, dt=1, g1=0x900001) == -2       # fp16 gradient not 2-byte aligned
    assert _rec(lib, g1=0x10000 + 64) == -5         # gradient inside img1
    assert _rec(lib, g2=0x900000 + 4) == -5         # gradients overlap
    assert _rec(lib, g1=0x1000 - 8) == -5           # gradient covers dloss
    assert _rec(lib, H=1 << 14, W=(1 << 13) + 4) == -4
    assert _rec(lib, g1=None, g2=None) == 0         # nothing to do: no launch


def test_loss_and_grad_argument_errors_return_before_any_hip_call():
    lib = S.lib()
    assert _lag(lib, loss=None) == -1
    assert _lag(lib, ws=None) == -1
    assert _lag(lib, dloss=None) == -1
    assert _lag(lib, dt=-1) == -8
    assert _lag(lib, padding=9) == -3
    assert _lag(lib, W=0) == -2
    assert _lag(lib, loss=0x100000 + 16) == -5      # loss inside img2
    assert _lag(lib, ws=0x900000 + 4096) == -5      # workspace overlaps a gradient
    assert _lag(lib, loss=0x300000 + 8) == -5       # loss inside the workspace


def test_noalloc_argument_errors_return_before_any_hip_call():
    lib = S.lib()
    f = lambda **kw: lib.ssim_loss_and_grad_noalloc(
        kw.get("img1", 0x10000), 0x100000, kw.get("dt", 0), 1, 1, kw.get("H", 64), 64,
        kw.get("pad", 0), kw.get("dloss", 0x1000), kw.get("loss", 0x2000), kw.get("g1", 0x900000),
        kw.get("g2", 0xA00000), None)
    assert S.ssim_noalloc_scratch_bytes() >= S.ssim_workspace_bytes()
    assert f(loss=None) == -1
    assert f(dloss=None) == -1
    assert f(img1=None) == -1
    assert f(dt=3) == -8
    assert f(pad=2) == -3
    assert f(H=10) == -2
    assert f(img1=0x10002) == -2
    assert f(loss=0x100000 + 16) == -5      # loss inside img2
    assert f(g1=0xA00000 + 8) == -5         # gradients overlap
    assert f(g2=0x10000 + 4096) == -5       # gradient inside img1
    assert "scratch" in S.ssim_strerror(-9)


def test_grad_scale_argument_errors_return_before_any_hip_call():
    lib = S.lib()
    f = lambda dl, g, o, n: lib.ssim_grad_scale(dl, g, o, n, None)
    assert f(None, None, None, 0) == 0                   # nothing to do: no launch
    assert f(0x1000, 0x10000, 0x20000, -1) == -2
    assert f(None, 0x10000, 0x20000, 8) == -1
    assert f(0x1000, None, 0x20000, 8) == -1
    assert f(0x1000, 0x10000, None, 8) == -1
    assert f(0x1000, 0x10002, 0x20000, 8) == -2          # not 4-byte aligned
    assert f(0x1000, 0x10000, 0x10000 + 16, 8) == -5     # partial overlap
    assert f(0x1000, 0x10000, 0x10000 - 16, 8) == -5
    assert f(0x1000, 0x10000, 0x20000, 1 << 62) == -4
    assert f(0x20000 + 16, 0x10000, 0x20000, 8) == -5     # dloss inside out
    assert f(0x20000 + 28, 0x10000, 0x20000, 8) == -5     # its last element
    assert f(0x10000 + 8, 0x10000, 0x10000, 8) == -5     # in place, dloss inside


def test_reference_argument_errors_return_before_any_hip_call():
    lib = S.lib()
    assert S.ssim_reference_bytes(1, 3, 1080, 1920, "valid") == 4 * 3 * 1070 * 1912
    assert S.ssim_reference_bytes(1, 1, 5, 30, "valid") == 0
    st = lambda **kw: lib.ssim_reference_stats(kw.get("img", 0x10000), kw.get("dt", 0), 1, 1, 64,
                                               64, kw.get("pad", 0), kw.get("ref", 0x300000), None)
    assert st(img=None) == -1
    assert st(ref=None) == -1
    assert st(dt=4) == -8
    assert st(pad=2) == -3
    assert st(ref=0x300004) == -2
    assert st(ref=0x10000 + 256) == -5
    lg = lambda **kw: lib.ssim_loss_and_grad_ref(
        0x10000, 0x100000, kw.get("ref", 0x300000), 0, 1, 1, 64, 64, 0, 0x1000,
        kw.get("loss", 0x2000), 0x500000, kw.get("g1", 0x900000), None)
    assert lg(ref=None) == -1
    assert lg(loss=None) == -1
    assert lg(ref=0x300008) == -2
    assert lg(g1=0x300000 + 64) == -5     # gradient overlaps the cached statistics


def test_volume_shapes_and_argument_errors():
    lib = S.lib()
    assert S.ssim3d_map_shape(96, 96, 96, "same") == (96, 96, 96)
    assert S.ssim3d_map_shape(12, 20, 11, "valid") == (2, 10, 1)
    assert S.ssim3d_saved_maps_bytes(2, 3, 96, 96, 96, "same") == 16 * 6 * 96 ** 3
    assert S.ssim3d_saved_maps_bytes(1, 1, 10, 20, 20, "valid") == 0
    fwd = lambda **kw: lib.ssim3d_forward(
        kw.get("x", 0x10000), kw.get("y", 0x200000), kw.get("dt", 0), 1, 1, kw.get("D", 16), 16,
        16, kw.get("pad", 1), kw.get("loss", 0x400000), kw.get("maps", None), kw.get("ws", 0x500000),
        None)
    assert fwd(x=None) == -1
    assert fwd(loss=None) == -1
    assert fwd(pad=4) == -3
    assert fwd(dt=7) == -8
    assert fwd(D=0) == -2
    assert fwd(D=5, pad=0) == -2
    assert fwd(x=0x10002) == -2
    assert fwd(maps=0x600008) == -2
    assert fwd(loss=0x10000 + 64) == -5
    assert fwd(D=1 << 20) == -4       # a volume of more than 2^27 voxels
    bwd = lambda **kw: lib.ssim3d_backward(
        0x1000, 0x10000, 0x200000, 0, 1, 1, 16, 16, 16, 1, kw.get("maps", 0x600000),
        kw.get("g1", 0x800000), kw.get("g2", 0x900000), None)
    assert bwd(maps=None) == -1
    assert bwd(g1=0x600000 + 16) == -5
    assert bwd(g1=0x900000 + 4) == -5
    assert bwd(g1=None, g2=None) == 0


def test_python_binding_rejects_cpu_tensors():
    import torch

    x = torch.zeros(1, 1, 16, 16)
    with pytest.raises(TypeError):
        S.ssim_loss(x, x)
    with pytest.raises(TypeError):
        S.ssim_loss(x.double(), x.double())
    with pytest.raises(TypeError):
        S.ssim_loss(x.half(), x.half())


def test_python_binding_buffer_checks():
    """The binding's checks of output and state buffers (run on host tensors,
    with the host as the images' device)."""
    import torch

    cpu = torch.device("cpu")
    S._check_buffer(None, "maps", cpu, 64, torch.float32)  # NULL: the C function decides
    S._check_buffer(torch.empty(16), "maps", cpu, 64, torch.float32)
    S._check_scalars(cpu, loss=torch.empty(()), dloss=torch.empty(1))
    with pytest.raises(ValueError):
        S._check_buffer(torch.empty(15), "maps", cpu, 64, torch.float32)
    with pytest.raises(ValueError):
        S._check_buffer(torch.empty(32)[::2], "maps", cpu, 64, torch.float32)
    with pytest.raises(TypeError):
        S._check_buffer(torch.empty(16, dtype=torch.float64), "maps", cpu, 64, torch.float32)
    with pytest.raises(TypeError):
        S._check_buffer(torch.empty(16), "maps", torch.device("cuda", 0), 64)
    with pytest.raises(TypeError):
        S._check_buffer(np.empty(16, np.float32), "maps", cpu, 64)
    with pytest.raises(ValueError):
        S._check_scalars(cpu, loss=torch.empty(0))
    with pytest.raises(TypeError):
        S._check_scalars(cpu, dloss=torch.empty((), dtype=torch.float16))
    with pytest.raises(ValueError):
        S._check_workspace(torch.empty(S.ssim_workspace_bytes() - 1, dtype=torch.uint8), cpu)
    x = torch.empty(1, 1, 4, 4)
    S._check_grads(x, (None, torch.empty(1, 1, 4, 4)))
    with pytest.raises(TypeError):
        S._check_grads(x, (torch.empty(1, 1, 4, 5),))


def test_build_entry_point_compiles_and_checks_the_abi():
    """__graft_entry__.build() compiles the library and the oracle in-tree
    (the atomic rename leaves the copy this process loaded intact) and checks
    the built library's ABI version against the bindings."""
    import importlib

    entry = importlib.import_module("__graft_entry__")
    entry.build()
