"""Fused SSIM loss (forward + backward) on AMD MI355X: thin Python binding.

The C ABI (``include/ssim_loss_amd.h``) is the product; this module only
marshals torch tensors into its pointers and sizes and calls it on torch's
current HIP stream.  Every step of the computation runs in the HIP kernels of
``libssim_loss_amd.so``; there is no fallback path.  If the library is
missing, importing the functions below raises.

Functions with the C names (images and gradients may be float32, float16 or
bfloat16 tensors; the C functions ssim_forward_typed / ssim_backward_typed
are called for the half types):
  ssim_forward(img1, img2, padding, loss, saved_maps, workspace)
  ssim_backward(dloss, img1, img2, padding, saved_maps, grad_img1, grad_img2)
  ssim_backward_recompute(dloss, img1, img2, padding, grad_img1, grad_img2)
  ssim_loss_and_grad(img1, img2, padding, dloss, loss, workspace, grad_img1, grad_img2)
  ssim_loss_and_grad_noalloc(img1, img2, padding, dloss, loss, grad_img1, grad_img2)
  ssim_grad_scale(dloss, grad, out)
  ssim_saved_maps_bytes, ssim_workspace_bytes, ssim_map_shape, ssim_taps,
  ssim_strerror, ssim_abi_version
Autograd conveniences ("TriSSIM" / "Fully Fused Differentiable SSIM", Usage):
  ssim_loss(img1, img2, padding="valid", train=True, recompute=True)
      -> 1 - mean SSIM; by default no maps are kept between forward and
         backward: for fp32 images the forward forms the loss and the
         gradients in one launch and the backward scales them by the upstream
         gradient; for half types the backward forms the statistics again
         from the images.  recompute=False saves the statistics
  fused_ssim(img1, img2, padding="same", train=True)  -> mean SSIM
One-pass step, for an upstream gradient known in advance:
  loss_and_grad(img1, img2, padding="valid", weight=1.0)
      -> (weight-free loss, weight * dloss/dimg1, weight * dloss/dimg2)
Cached reference statistics (a fixed second image, only the first one
differentiable):
  ref = reference_stats(img2, padding="valid")
  loss_and_grad_ref(img1, img2, ref, padding="valid", weight=1.0)
      -> (loss, weight * dloss/dimg1)
Volumes (NCDHW, "Fully Fused Differentiable SSIM", 3D data):
  ssim3d_forward, ssim3d_backward, ssim3d_saved_maps_bytes, ssim3d_map_shape
  ssim3d_loss(vol1, vol2, padding="same", train=True) -> 1 - mean SSIM
  fused_ssim3d(vol1, vol2, padding="same", train=True) -> mean SSIM
"""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

# SSIM_ABI_VERSION of include/ssim_loss_amd.h that these bindings follow; a
# library built from another version is refused at load time
ABI_VERSION = 8

PAD = {"valid": 0, "same": 1}
SSIM_OK = 0
SSIM_DTYPE = {"float32": 0, "float16": 1, "bfloat16": 2}

_lib = None
_lock = threading.Lock()


class SsimError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {ssim_strerror(code)} (code {code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        # SSIM_LOSS_AMD_LIB names another build of the same sources (e.g. one
        # with host-side sanitizers); there is never a fallback implementation
        path = os.environ.get("SSIM_LOSS_AMD_LIB", LIB_PATH)
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it first (python -m ssim_loss_amd.build "
                "or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(path)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.ssim_abi_version.restype = i32
        L.ssim_abi_version.argtypes = []
        if L.ssim_abi_version() != ABI_VERSION:
            raise ImportError(
                f"{path} implements ABI version {L.ssim_abi_version()}, these bindings "
                f"version {ABI_VERSION}: rebuild it")
        L.ssim_strerror.restype = ctypes.c_char_p
        L.ssim_strerror.argtypes = [i32]
        L.ssim_taps.restype = None
        L.ssim_taps.argtypes = [vp]
        L.ssim_map_shape.restype = i32
        L.ssim_map_shape.argtypes = [i64, i64, i32, vp, vp]
        L.ssim_saved_maps_bytes.restype = sz
        L.ssim_saved_maps_bytes.argtypes = [i64, i64, i64, i64, i32]
        L.ssim_workspace_bytes.restype = sz
        L.ssim_workspace_bytes.argtypes = []
        L.ssim_forward.restype = i32
        L.ssim_forward.argtypes = [vp, vp, i64, i64, i64, i64, i32, vp, vp, vp, vp]
        L.ssim_backward.restype = i32
        L.ssim_backward.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, vp, vp, vp, vp]
        L.ssim_forward_typed.restype = i32
        L.ssim_forward_typed.argtypes = [vp, vp, i32, i64, i64, i64, i64, i32, vp, vp, vp, vp]
        L.ssim_backward_typed.restype = i32
        L.ssim_backward_typed.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i32, vp, vp, vp,
                                          vp]
        L.ssim_backward_recompute.restype = i32
        L.ssim_backward_recompute.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i32, vp, vp,
                                              vp]
        L.ssim3d_map_shape.restype = i32
        L.ssim3d_map_shape.argtypes = [i64, i64, i64, i32, vp, vp, vp]
        L.ssim3d_saved_maps_bytes.restype = sz
        L.ssim3d_saved_maps_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
        L.ssim3d_forward.restype = i32
        L.ssim3d_forward.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i32, vp, vp, vp, vp]
        L.ssim3d_backward.restype = i32
        L.ssim3d_backward.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, vp, vp, vp,
                                      vp]
        L.ssim_reference_bytes.restype = sz
        L.ssim_reference_bytes.argtypes = [i64, i64, i64, i64, i32]
        L.ssim_reference_stats.restype = i32
        L.ssim_reference_stats.argtypes = [vp, i32, i64, i64, i64, i64, i32, vp, vp]
        L.ssim_loss_and_grad_ref.restype = i32
        L.ssim_loss_and_grad_ref.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i32, vp, vp,
                                             vp, vp, vp]
        L.ssim_grad_scale.restype = i32
        L.ssim_grad_scale.argtypes = [vp, vp, vp, i64, vp]
        L.ssim_loss_and_grad.restype = i32
        L.ssim_loss_and_grad.argtypes = [vp, vp, i32, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp,
                                         vp]
        L.ssim_loss_and_grad_noalloc.restype = i32
        L.ssim_loss_and_grad_noalloc.argtypes = [vp, vp, i32, i64, i64, i64, i64, i32, vp, vp, vp,
                                                 vp, vp]
        L.ssim_noalloc_scratch_bytes.restype = sz
        L.ssim_noalloc_scratch_bytes.argtypes = []
        _lib = L
    return _lib


def _pad(padding) -> int:
    if isinstance(padding, str):
        if padding not in PAD:
            raise ValueError(f"padding must be 'valid' or 'same', got {padding!r}")
        return PAD[padding]
    return int(padding)


# --------------------------------------------------------------------------- host-only calls
def ssim_abi_version() -> int:
    return int(lib().ssim_abi_version())


def ssim_strerror(code: int) -> str:
    return lib().ssim_strerror(int(code)).decode()


def ssim_taps() -> list[float]:
    buf = (ctypes.c_float * 11)()
    lib().ssim_taps(buf)
    return list(buf)


def ssim_map_shape(H: int, W: int, padding) -> tuple[int, int]:
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().ssim_map_shape(int(H), int(W), _pad(padding), ctypes.byref(ho), ctypes.byref(wo))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim_map_shape")
    return int(ho.value), int(wo.value)


def ssim_saved_maps_bytes(N: int, C: int, H: int, W: int, padding) -> int:
    return int(lib().ssim_saved_maps_bytes(int(N), int(C), int(H), int(W), _pad(padding)))


def ssim_workspace_bytes() -> int:
    return int(lib().ssim_workspace_bytes())


# --------------------------------------------------------------------------- device calls
_raw_stream = None


def _current_stream(index: int) -> int:
    """The raw HIP stream torch's current stream on device `index` wraps (the
    accessor without a Python stream object: a few hundredths of the cost)."""
    global _raw_stream
    if _raw_stream is None:
        import torch

        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None) or (
            lambda i: torch.cuda.current_stream(i).cuda_stream)
    return _raw_stream(index)


def _stream_ptr(t) -> int:
    return _current_stream(t.device.index)


def _dptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    return SSIM_DTYPE[str(t.dtype).replace("torch.", "")]


def _check_image(t, name, ndim=4):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise TypeError(f"{name} must be float32, float16 or bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor, got device {t.device}")
    layout = "NCHW" if ndim == 4 else "NCDHW"
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {layout} ({ndim}-D), got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous {layout}")


def _check_buffer(t, name, dev, nbytes=0, dtype=None):
    """A caller's output or state buffer: a contiguous tensor on the images'
    device `dev` holding at least `nbytes` bytes (of `dtype`, when given).
    None is passed on as NULL: the C function decides whether it may be."""
    if t is None:
        return
    if not isinstance(t, _torch().Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != dev:
        raise TypeError(f"{name} must be a tensor on {dev}, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.nbytes < nbytes:
        raise ValueError(f"{name} holds {t.nbytes} bytes, needs {nbytes}")


def _check_scalars(dev, **bufs):
    """loss / dloss: one fp32 value each on the images' device."""
    for name, t in bufs.items():
        _check_buffer(t, name, dev, 4, _torch().float32)


def _check_workspace(ws, dev):
    global _ws_bytes
    if _ws_bytes is None:
        _ws_bytes = ssim_workspace_bytes()
    _check_buffer(ws, "workspace", dev, _ws_bytes)


_ws_bytes = None


def ssim_forward(img1, img2, padding, loss, saved_maps, workspace) -> None:
    """Calls the C ``ssim_forward`` on torch's current stream.  All arguments
    are preallocated device tensors (saved_maps may be None)."""
    _check_image(img1, "img1")
    _check_image(img2, "img2")
    if img1.shape != img2.shape:
        raise ValueError("img1 and img2 must have the same shape")
    if img1.dtype != img2.dtype:
        raise TypeError("img1 and img2 must have the same dtype")
    N, C, H, W = img1.shape
    _check_scalars(img1.device, loss=loss)
    _check_buffer(saved_maps, "saved_maps", img1.device,
                  ssim_saved_maps_bytes(N, C, H, W, padding), _f32())
    _check_workspace(workspace, img1.device)
    code = _dtype_code(img1)
    if code == 0:
        rc = lib().ssim_forward(_dptr(img1), _dptr(img2), N, C, H, W, _pad(padding), _dptr(loss),
                                _dptr(saved_maps), _dptr(workspace), _stream_ptr(img1))
    else:
        rc = lib().ssim_forward_typed(_dptr(img1), _dptr(img2), code, N, C, H, W, _pad(padding),
                                      _dptr(loss), _dptr(saved_maps), _dptr(workspace),
                                      _stream_ptr(img1))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim_forward")


def ssim_backward(dloss, img1, img2, padding, saved_maps, grad_img1, grad_img2) -> None:
    """Calls the C ``ssim_backward`` on torch's current stream."""
    _check_image(img1, "img1")
    _check_image(img2, "img2")
    if img1.dtype != img2.dtype:
        raise TypeError("img1 and img2 must have the same dtype")
    if img1.shape != img2.shape:
        raise ValueError("img1 and img2 must have the same shape")
    _check_grads(img1, (grad_img1, grad_img2))
    N, C, H, W = img1.shape
    _check_scalars(img1.device, dloss=dloss)
    _check_buffer(saved_maps, "saved_maps", img1.device,
                  ssim_saved_maps_bytes(N, C, H, W, padding), _f32())
    code = _dtype_code(img1)
    if code == 0:
        rc = lib().ssim_backward(_dptr(dloss), _dptr(img1), _dptr(img2), N, C, H, W,
                                 _pad(padding), _dptr(saved_maps), _dptr(grad_img1),
                                 _dptr(grad_img2), _stream_ptr(img1))
    else:
        rc = lib().ssim_backward_typed(_dptr(dloss), _dptr(img1), _dptr(img2), code, N, C, H, W,
                                       _pad(padding), _dptr(saved_maps), _dptr(grad_img1),
                                       _dptr(grad_img2), _stream_ptr(img1))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim_backward")


def _torch():
    import torch

    return torch


def _f32():
    return _torch().float32


def _check_grads(img1, grads):
    for g in grads:
        if g is not None:
            if g.dtype != img1.dtype or g.shape != img1.shape:
                raise TypeError("gradients must have the images' dtype and shape")
            _check_buffer(g, "gradient", img1.device)


def _check_pair_and_grads(img1, img2, grads, ndim=4):
    _check_image(img1, "img1", ndim)
    _check_image(img2, "img2", ndim)
    if img1.shape != img2.shape:
        raise ValueError("img1 and img2 must have the same shape")
    if img1.dtype != img2.dtype:
        raise TypeError("img1 and img2 must have the same dtype")
    _check_grads(img1, grads)


def ssim_backward_recompute(dloss, img1, img2, padding, grad_img1, grad_img2) -> None:
    """Calls the C ``ssim_backward_recompute`` (no saved maps) on torch's
    current stream."""
    _check_pair_and_grads(img1, img2, (grad_img1, grad_img2))
    _check_scalars(img1.device, dloss=dloss)
    N, C, H, W = img1.shape
    rc = lib().ssim_backward_recompute(_dptr(dloss), _dptr(img1), _dptr(img2), _dtype_code(img1),
                                       N, C, H, W, _pad(padding), _dptr(grad_img1),
                                       _dptr(grad_img2), _stream_ptr(img1))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim_backward_recompute")


def ssim_loss_and_grad(img1, img2, padding, dloss, loss, workspace, grad_img1, grad_img2) -> None:
    """Calls the C ``ssim_loss_and_grad`` (loss and gradients in one launch)
    on torch's current stream."""
    _check_pair_and_grads(img1, img2, (grad_img1, grad_img2))
    _check_scalars(img1.device, dloss=dloss, loss=loss)
    _check_workspace(workspace, img1.device)
    N, C, H, W = img1.shape
    rc = lib().ssim_loss_and_grad(_dptr(img1), _dptr(img2), _dtype_code(img1), N, C, H, W,
                                  _pad(padding), _dptr(dloss), _dptr(loss), _dptr(workspace),
                                  _dptr(grad_img1), _dptr(grad_img2), _stream_ptr(img1))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim_loss_and_grad")


def ssim_loss_and_grad_noalloc(img1, img2, padding, dloss, loss, grad_img1, grad_img2) -> None:
    """Calls the C ``ssim_loss_and_grad_noalloc`` (the one-launch step with
    the loss accumulator in the library's own device array: no workspace) on
    torch's current stream.  Calls that may overlap on one GPU race on that
    array."""
    _check_pair_and_grads(img1, img2, (grad_img1, grad_img2))
    _check_scalars(img1.device, dloss=dloss, loss=loss)
    N, C, H, W = img1.shape
    rc = lib().ssim_loss_and_grad_noalloc(_dptr(img1), _dptr(img2), _dtype_code(img1), N, C, H,
                                          W, _pad(padding), _dptr(dloss), _dptr(loss),
                                          _dptr(grad_img1), _dptr(grad_img2), _stream_ptr(img1))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim_loss_and_grad_noalloc")


def ssim_noalloc_scratch_bytes() -> int:
    return int(lib().ssim_noalloc_scratch_bytes())


def ssim_grad_scale(dloss, grad, out) -> None:
    """Calls the C ``ssim_grad_scale`` (out = *dloss * grad, fp32) on torch's
    current stream; out may be grad itself."""
    import torch

    if not isinstance(grad, torch.Tensor) or grad.device.type != "cuda":
        raise TypeError("grad must be a GPU tensor")
    if grad.dtype != torch.float32 or not grad.is_contiguous():
        raise TypeError("grad must be a contiguous float32 tensor")
    _check_buffer(out, "out", grad.device, grad.nbytes, torch.float32)
    if out is None or out.numel() != grad.numel():
        raise ValueError("out must have grad's number of elements")
    _check_scalars(grad.device, dloss=dloss)
    rc = lib().ssim_grad_scale(_dptr(dloss), _dptr(grad), _dptr(out), grad.numel(),
                               _stream_ptr(grad))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim_grad_scale")


# --------------------------------------------------------------------------- buffers
_workspaces: dict = {}


def workspace_for(device) -> "torch.Tensor":
    """A zero-initialised workspace per (device, current stream), created once
    (zeroed on that stream, so before its first use there).  Calls on one
    stream run in order, so they may share it; calls on different streams get
    different workspaces and may overlap."""
    import torch

    dev = torch.device(device)
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (index, _current_stream(index))
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.zeros(ssim_workspace_bytes(), dtype=torch.uint8,
                         device=torch.device("cuda", index))
        _workspaces[key] = ws
    return ws


def alloc_saved_maps(img1, padding) -> "torch.Tensor":
    import torch

    N, C, H, W = img1.shape
    nbytes = ssim_saved_maps_bytes(N, C, H, W, padding)
    if nbytes == 0:
        raise SsimError(-2, "ssim_saved_maps_bytes")
    return torch.empty(nbytes // 4, dtype=torch.float32, device=img1.device)


# --------------------------------------------------------------------------- autograd
def _make_function():
    import torch

    class _SsimLoss(torch.autograd.Function):
        @staticmethod
        def forward(ctx, img1, img2, padding, train, recompute, grads):
            img1 = img1.detach()
            img2 = img2.detach()
            dev = img1.device
            loss = torch.empty((), dtype=torch.float32, device=dev)
            ctx.padding = padding
            ctx.train = train
            ctx.recompute = recompute
            ctx.dev = dev
            # fp32 images whose gradient is wanted, while the step stays in the
            # last-level cache: the gradients with an upstream gradient of 1,
            # in the launch that forms the loss; the backward scales them in
            # place (bit for bit the one-launch result).  Both gradients share
            # one buffer, so one scale launch serves both.
            ctx.early = bool(train and recompute and grads and img1.dtype == torch.float32
                             and 4 * img1.nbytes <= EARLY_GRADIENT_BYTES)
            if ctx.early:
                want1, want2 = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
                gbuf = torch.empty((int(want1) + int(want2),) + tuple(img1.shape),
                                   dtype=torch.float32, device=dev)
                g1 = gbuf[0] if want1 else None
                g2 = gbuf[-1] if want2 else None
                # ssim_loss checked the images; the other buffers are made here
                N, C, H, W = img1.shape
                rc = lib().ssim_loss_and_grad(
                    img1.data_ptr(), img2.data_ptr(), SSIM_DTYPE["float32"], N, C, H, W,
                    _pad(padding), _one(dev).data_ptr(), loss.data_ptr(),
                    workspace_for(dev).data_ptr(), _dptr(g1), _dptr(g2), _current_stream(dev.index))
                if rc != SSIM_OK:
                    raise SsimError(rc, "ssim_loss_and_grad")
                # (an intermediate, kept on ctx: the backward scales it in place)
                ctx.gbuf = gbuf
                ctx.scaled = False
                ctx.save_for_backward(img1, img2)
                return loss
            maps = alloc_saved_maps(img1, padding) if train and not recompute else None
            N, C, H, W = img1.shape
            rc = lib().ssim_forward_typed(
                img1.data_ptr(), img2.data_ptr(), _dtype_code(img1), N, C, H, W, _pad(padding),
                loss.data_ptr(), _dptr(maps), workspace_for(dev).data_ptr(),
                _current_stream(dev.index))
            if rc != SSIM_OK:
                raise SsimError(rc, "ssim_forward")
            if train:
                if recompute:
                    ctx.save_for_backward(img1, img2)
                else:
                    ctx.save_for_backward(img1, img2, maps)
            return loss

        @staticmethod
        def backward(ctx, dloss):
            if not ctx.train:
                raise RuntimeError("ssim_loss was called with train=False; no gradient saved")
            want1, want2 = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
            dl = dloss.detach().to(device=ctx.dev, dtype=torch.float32).reshape(()).contiguous()
            if ctx.early and not ctx.scaled:
                # the first backward scales the gradients in place, in one
                # launch over both
                gbuf = ctx.gbuf
                ctx.gbuf = None
                ctx.scaled = True
                rc = lib().ssim_grad_scale(dl.data_ptr(), gbuf.data_ptr(), gbuf.data_ptr(),
                                           gbuf.numel(), _current_stream(gbuf.device.index))
                if rc != SSIM_OK:
                    raise SsimError(rc, "ssim_grad_scale")
                g1 = gbuf[0] if want1 else None
                g2 = gbuf[-1] if want2 else None
                return g1, g2, None, None, None, None
            # (a second backward through an early step, retain_graph=True, forms
            # the gradients again from the images)
            if ctx.recompute:
                img1, img2 = ctx.saved_tensors
            else:
                img1, img2, maps = ctx.saved_tensors
            g1 = torch.empty_like(img1) if want1 else None
            g2 = torch.empty_like(img2) if want2 else None
            N, C, H, W = img1.shape
            stream = _current_stream(ctx.dev.index)
            if ctx.recompute:
                rc = lib().ssim_backward_recompute(
                    dl.data_ptr(), img1.data_ptr(), img2.data_ptr(), _dtype_code(img1), N, C, H, W,
                    _pad(ctx.padding), _dptr(g1), _dptr(g2), stream)
                where = "ssim_backward_recompute"
            else:
                rc = lib().ssim_backward_typed(
                    dl.data_ptr(), img1.data_ptr(), img2.data_ptr(), _dtype_code(img1), N, C, H, W,
                    _pad(ctx.padding), maps.data_ptr(), _dptr(g1), _dptr(g2), stream)
                where = "ssim_backward"
            if rc != SSIM_OK:
                raise SsimError(rc, where)
            return g1, g2, None, None, None, None

    return _SsimLoss


_fn = None

# Above this many bytes of images and gradients (4 image-size buffers) a step
# cannot stay in the 256 MB last-level cache between its forward and backward:
# there the inference forward and the recomputing backward cost less GPU time
# than the one-launch forward plus the scale pass, and hold no gradient
# buffers between the two.
EARLY_GRADIENT_BYTES = 256 << 20


def ssim_loss(img1, img2, padding: str = "valid", train: bool = True, recompute: bool = True):
    """loss = 1 - mean SSIM (a 0-d fp32 tensor on the images' device), with
    gradients for whichever of img1 / img2 requires them.  With recompute
    (the default) no blurred statistics are kept between forward and
    backward.  For fp32 images whose gradient is wanted, up to
    EARLY_GRADIENT_BYTES of images and gradients, the forward forms the loss
    and the gradients (for an upstream gradient of 1) in one launch and the
    backward multiplies them by the upstream gradient in place, giving
    ssim_loss_and_grad's result bit for bit (the gradients are formed under
    grad mode even if no backward follows); otherwise the forward forms the
    loss alone and the backward forms the statistics again from the images.
    recompute=False saves the four blurred statistics (16 bytes per map
    entry) for the backward to read, as the pages' training mode does.  All
    three give the same gradient to the contract's tolerance."""
    global _fn
    if _fn is None:
        _fn = _make_function()
    _check_image(img1, "img1")
    _check_image(img2, "img2")
    if img1.shape != img2.shape:
        raise ValueError("img1 and img2 must have the same shape")
    if img1.dtype != img2.dtype:
        raise TypeError("img1 and img2 must have the same dtype")
    _pad(padding)
    import torch

    grads = torch.is_grad_enabled() and (img1.requires_grad or img2.requires_grad)
    return _fn.apply(img1, img2, padding, bool(train), bool(recompute), grads)


def fused_ssim(img1, img2, padding: str = "same", train: bool = True):
    """Mean SSIM ("Fully Fused Differentiable SSIM", Usage: default padding
    "same")."""
    return 1.0 - ssim_loss(img1, img2, padding, train)


_ones: dict = {}


def _one(dev):
    """A 0-d fp32 1.0 on `dev`, made once per device (read only).  It is
    copied from the host, which waits for the copy, so that calls on any
    stream may read it afterwards."""
    import torch

    one = _ones.get(dev)
    if one is None:
        one = torch.ones((), dtype=torch.float32).to(dev)
        _ones[dev] = one
    return one


def _dloss_tensor(weight, dev):
    """The upstream gradient as a 0-d fp32 device tensor.  A number is filled
    in on the stream (a copy from the host would wait for it)."""
    import torch

    if isinstance(weight, torch.Tensor):
        return weight.detach().to(device=dev, dtype=torch.float32).reshape(()).contiguous()
    return torch.full((), float(weight), dtype=torch.float32, device=dev)


def loss_and_grad(img1, img2, padding: str = "valid", weight=1.0, grad1: bool = True,
                  grad2: bool = True):
    """One launch for a training step whose upstream gradient is known before
    the forward: returns (loss, grad_img1, grad_img2) with loss = 1 - mean
    SSIM and grad = weight * d loss / d img (None where not asked for).
    `weight` is a number or a 0-d device tensor (e.g. the SSIM term's weight
    in a training loss)."""
    import torch

    _check_pair_and_grads(img1, img2, ())
    dev = img1.device
    dl = _dloss_tensor(weight, dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    g1 = torch.empty_like(img1) if grad1 else None
    g2 = torch.empty_like(img2) if grad2 else None
    ssim_loss_and_grad(img1.detach(), img2.detach(), padding, dl, loss, workspace_for(dev), g1, g2)
    return loss, g1, g2


# --------------------------------------------------------------------------- cached reference


def ssim_reference_bytes(N: int, C: int, H: int, W: int, padding) -> int:
    return int(lib().ssim_reference_bytes(int(N), int(C), int(H), int(W), _pad(padding)))


def ssim_reference_stats(img2, padding, ref) -> None:
    """Calls the C ``ssim_reference_stats`` on torch's current stream."""
    _check_image(img2, "img2")
    N, C, H, W = img2.shape
    _check_buffer(ref, "ref", img2.device, ssim_reference_bytes(N, C, H, W, padding), _f32())
    rc = lib().ssim_reference_stats(_dptr(img2), _dtype_code(img2), N, C, H, W, _pad(padding),
                                    _dptr(ref), _stream_ptr(img2))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim_reference_stats")


def ssim_loss_and_grad_ref(img1, img2, ref, padding, dloss, loss, workspace, grad_img1) -> None:
    """Calls the C ``ssim_loss_and_grad_ref`` on torch's current stream."""
    _check_pair_and_grads(img1, img2, (grad_img1,))
    N, C, H, W = img1.shape
    _check_scalars(img1.device, dloss=dloss, loss=loss)
    _check_buffer(ref, "ref", img1.device, ssim_reference_bytes(N, C, H, W, padding), _f32())
    _check_workspace(workspace, img1.device)
    rc = lib().ssim_loss_and_grad_ref(_dptr(img1), _dptr(img2), _dptr(ref), _dtype_code(img1), N,
                                      C, H, W, _pad(padding), _dptr(dloss), _dptr(loss),
                                      _dptr(workspace), _dptr(grad_img1), _stream_ptr(img1))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim_loss_and_grad_ref")


def reference_stats(img2, padding: str = "valid") -> "torch.Tensor":
    """The cached statistics of a fixed reference image (a device fp32 tensor
    of ssim_reference_bytes bytes), for loss_and_grad_ref."""
    import torch

    N, C, H, W = img2.shape
    nbytes = ssim_reference_bytes(N, C, H, W, padding)
    if nbytes == 0:
        raise SsimError(-2, "ssim_reference_bytes")
    ref = torch.empty(nbytes // 4, dtype=torch.float32, device=img2.device)
    ssim_reference_stats(img2.detach(), padding, ref)
    return ref


def loss_and_grad_ref(img1, img2, ref, padding: str = "valid", weight=1.0, grad1: bool = True):
    """(loss, weight * d loss / d img1) in one launch, with the reference's
    statistics read from `ref` (reference_stats of this img2)."""
    import torch

    _check_pair_and_grads(img1, img2, ())
    dev = img1.device
    dl = _dloss_tensor(weight, dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    g1 = torch.empty_like(img1) if grad1 else None
    ssim_loss_and_grad_ref(img1.detach(), img2.detach(), ref, padding, dl, loss,
                           workspace_for(dev), g1)
    return loss, g1


# --------------------------------------------------------------------------- volumes


def ssim3d_map_shape(D: int, H: int, W: int, padding) -> tuple[int, int, int]:
    do, ho, wo = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = lib().ssim3d_map_shape(int(D), int(H), int(W), _pad(padding), ctypes.byref(do),
                                ctypes.byref(ho), ctypes.byref(wo))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim3d_map_shape")
    return int(do.value), int(ho.value), int(wo.value)


def ssim3d_saved_maps_bytes(N: int, C: int, D: int, H: int, W: int, padding) -> int:
    return int(lib().ssim3d_saved_maps_bytes(int(N), int(C), int(D), int(H), int(W),
                                             _pad(padding)))


def ssim3d_forward(vol1, vol2, padding, loss, saved_maps, workspace) -> None:
    """Calls the C ``ssim3d_forward`` on torch's current stream (saved_maps
    may be None: inference)."""
    _check_pair_and_grads(vol1, vol2, (), ndim=5)
    N, C, D, H, W = vol1.shape
    _check_scalars(vol1.device, loss=loss)
    _check_buffer(saved_maps, "saved_maps", vol1.device,
                  ssim3d_saved_maps_bytes(N, C, D, H, W, padding), _f32())
    _check_workspace(workspace, vol1.device)
    rc = lib().ssim3d_forward(_dptr(vol1), _dptr(vol2), _dtype_code(vol1), N, C, D, H, W,
                              _pad(padding), _dptr(loss), _dptr(saved_maps), _dptr(workspace),
                              _stream_ptr(vol1))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim3d_forward")


def ssim3d_backward(dloss, vol1, vol2, padding, saved_maps, grad_vol1, grad_vol2) -> None:
    """Calls the C ``ssim3d_backward`` on torch's current stream."""
    _check_pair_and_grads(vol1, vol2, (grad_vol1, grad_vol2), ndim=5)
    N, C, D, H, W = vol1.shape
    _check_scalars(vol1.device, dloss=dloss)
    _check_buffer(saved_maps, "saved_maps", vol1.device,
                  ssim3d_saved_maps_bytes(N, C, D, H, W, padding), _f32())
    rc = lib().ssim3d_backward(_dptr(dloss), _dptr(vol1), _dptr(vol2), _dtype_code(vol1), N, C,
                               D, H, W, _pad(padding), _dptr(saved_maps), _dptr(grad_vol1),
                               _dptr(grad_vol2), _stream_ptr(vol1))
    if rc != SSIM_OK:
        raise SsimError(rc, "ssim3d_backward")


def alloc_saved_maps3d(vol1, padding) -> "torch.Tensor":
    import torch

    N, C, D, H, W = vol1.shape
    nbytes = ssim3d_saved_maps_bytes(N, C, D, H, W, padding)
    if nbytes == 0:
        raise SsimError(-2, "ssim3d_saved_maps_bytes")
    return torch.empty(nbytes // 4, dtype=torch.float32, device=vol1.device)


def _make_function3d():
    import torch

    class _Ssim3dLoss(torch.autograd.Function):
        @staticmethod
        def forward(ctx, vol1, vol2, padding, train):
            vol1 = vol1.detach()
            vol2 = vol2.detach()
            loss = torch.empty((), dtype=torch.float32, device=vol1.device)
            maps = alloc_saved_maps3d(vol1, padding) if train else None
            ssim3d_forward(vol1, vol2, padding, loss, maps, workspace_for(vol1.device))
            ctx.padding = padding
            ctx.train = train
            if train:
                ctx.save_for_backward(vol1, vol2, maps)
            return loss

        @staticmethod
        def backward(ctx, dloss):
            if not ctx.train:
                raise RuntimeError("ssim3d_loss was called with train=False; no gradient saved")
            vol1, vol2, maps = ctx.saved_tensors
            want1, want2 = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
            g1 = torch.empty_like(vol1) if want1 else None
            g2 = torch.empty_like(vol2) if want2 else None
            dl = dloss.detach().to(dtype=torch.float32).contiguous()
            ssim3d_backward(dl, vol1, vol2, ctx.padding, maps, g1, g2)
            return g1, g2, None, None

    return _Ssim3dLoss


_fn3d = None


def ssim3d_loss(vol1, vol2, padding: str = "same", train: bool = True):
    """loss = 1 - mean SSIM of two NCDHW volumes (the 11x11x11 window), with
    gradients for whichever of vol1 / vol2 requires them."""
    global _fn3d
    if _fn3d is None:
        _fn3d = _make_function3d()
    _check_pair_and_grads(vol1, vol2, (), ndim=5)
    _pad(padding)
    return _fn3d.apply(vol1, vol2, padding, bool(train))


def fused_ssim3d(vol1, vol2, padding: str = "same", train: bool = True):
    """Mean SSIM of two volumes ("Fully Fused Differentiable SSIM", 3D data:
    fused_ssim3d on [BS, CH, D, H, W])."""
    return 1.0 - ssim3d_loss(vol1, vol2, padding, train)
