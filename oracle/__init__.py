"""fp64 CPU oracle for the SSIM loss (ctypes wrapper over ``ssim_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``ssim_loss_amd``) and never imports it.

What each function follows is stated in ``ssim_oracle.c``; in short:
  - window: 11x11 Gaussian, sigma 1.5, normalised ("Fully Fused Differentiable
    SSIM", opening section);
  - padding "valid" / "same" with zero fill ("Fully Fused Differentiable SSIM",
    Usage);
  - loss = 1 - mean SSIM; gradients by the chain rule through the adjoint of
    the blur ("TriSSIM", How it works / Usage);
  - volumes (NCDHW): the same on the 11x11x11 window ("Fully Fused
    Differentiable SSIM", 3D data).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build

PAD = {"valid": 0, "same": 1}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("SSIM_ORACLE_LIB")  # another build, e.g. a sanitised one
    if path is None:
        path = LIB_PATH
        if not os.path.exists(path):
            build()
    lib = ctypes.CDLL(path)
    i64, dbl, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    vp = ctypes.c_void_p
    lib.oracle_taps.argtypes = [vp]
    lib.oracle_c1.restype = dbl
    lib.oracle_c2.restype = dbl
    lib.oracle_out_shape.argtypes = [i64, i64, i32, vp, vp]
    lib.oracle_out_shape.restype = i32
    lib.oracle_blur.argtypes = [vp, i64, i64, i32, vp]
    lib.oracle_blur_adjoint.argtypes = [vp, i64, i64, i32, vp]
    lib.oracle_ssim_map_plane.argtypes = [vp, vp, i64, i64, i32, vp]
    lib.oracle_ssim_plane.argtypes = [vp, vp, i64, i64, i32, dbl, dbl, vp, vp]
    lib.oracle_ssim_plane.restype = dbl
    for f in (lib.oracle_ssim_f64, lib.oracle_ssim_f32):
        f.argtypes = [vp, vp, i64, i64, i64, i64, i32, dbl, vp, vp, vp]
        f.restype = i32
    lib.oracle_sample_ssim_f32.argtypes = [vp, vp, i64, i64, i32, i64, i64]
    lib.oracle_sample_ssim_f32.restype = dbl
    lib.oracle_sample_grad_f32.argtypes = [vp, vp, i64, i64, i32, dbl, dbl, i64, i64, vp, vp]
    lib.oracle_out_shape3.argtypes = [i64, i64, i64, i32, vp, vp, vp]
    lib.oracle_out_shape3.restype = i32
    lib.oracle_blur3.argtypes = [vp, i64, i64, i64, i32, vp]
    lib.oracle_ssim3_volume.argtypes = [vp, vp, i64, i64, i64, i32, dbl, dbl, vp, vp]
    lib.oracle_ssim3_volume.restype = dbl
    lib.oracle_ssim3_f32.argtypes = [vp, vp, i64, i64, i64, i64, i64, i32, dbl, vp, vp, vp]
    lib.oracle_ssim3_f32.restype = i32
    lib.oracle_sample_grad3_f32.argtypes = [vp, vp, i64, i64, i64, i32, dbl, dbl, i64, i64, i64,
                                            vp, vp]
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_max_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _pad(padding) -> int:
    if isinstance(padding, str):
        return PAD[padding]
    return int(padding)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def taps() -> np.ndarray:
    g = np.zeros(11, np.float64)
    _load().oracle_taps(_ptr(g))
    return g


def constants() -> tuple[float, float]:
    lib = _load()
    return float(lib.oracle_c1()), float(lib.oracle_c2())


def out_shape(H: int, W: int, padding) -> tuple[int, int]:
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    _load().oracle_out_shape(H, W, _pad(padding), ctypes.byref(ho), ctypes.byref(wo))
    return int(ho.value), int(wo.value)


def blur(img: np.ndarray, padding) -> np.ndarray:
    """B applied to one H x W fp64 plane."""
    img = np.ascontiguousarray(img, np.float64)
    H, W = img.shape
    Ho, Wo = out_shape(H, W, padding)
    out = np.zeros((max(Ho, 0), max(Wo, 0)), np.float64)
    _load().oracle_blur(_ptr(img), H, W, _pad(padding), _ptr(out))
    return out


def blur_adjoint(m: np.ndarray, H: int, W: int, padding) -> np.ndarray:
    """B^T applied to one Ho x Wo fp64 map, giving an H x W plane."""
    m = np.ascontiguousarray(m, np.float64)
    assert m.shape == out_shape(H, W, padding)
    out = np.zeros((H, W), np.float64)
    _load().oracle_blur_adjoint(_ptr(m), H, W, _pad(padding), _ptr(out))
    return out


def ssim_map(x: np.ndarray, y: np.ndarray, padding) -> np.ndarray:
    """SSIM map of one fp64 H x W plane pair."""
    x = np.ascontiguousarray(x, np.float64)
    y = np.ascontiguousarray(y, np.float64)
    H, W = x.shape
    Ho, Wo = out_shape(H, W, padding)
    out = np.zeros((Ho, Wo), np.float64)
    _load().oracle_ssim_map_plane(_ptr(x), _ptr(y), H, W, _pad(padding), _ptr(out))
    return out


def ssim_loss(x: np.ndarray, y: np.ndarray, padding="valid", dloss: float = 1.0,
              grads: bool = True):
    """loss = 1 - mean SSIM over an NCHW batch, and dloss * d loss / d(x, y).

    fp32 inputs are consumed as they are (the exact buffers a GPU run uses);
    fp64 inputs are used as given.  Returns (loss, grad_x, grad_y) with fp64
    gradients, or (loss, None, None) when grads is False.
    """
    assert x.shape == y.shape and x.ndim == 4
    N, C, H, W = x.shape
    lib = _load()
    if x.dtype == np.float32 and y.dtype == np.float32:
        x = np.ascontiguousarray(x)
        y = np.ascontiguousarray(y)
        fn = lib.oracle_ssim_f32
    else:
        x = np.ascontiguousarray(x, np.float64)
        y = np.ascontiguousarray(y, np.float64)
        fn = lib.oracle_ssim_f64
    loss = ctypes.c_double()
    gx = np.zeros(x.shape, np.float64) if grads else None
    gy = np.zeros(x.shape, np.float64) if grads else None
    rc = fn(_ptr(x), _ptr(y), N, C, H, W, _pad(padding), float(dloss), ctypes.byref(loss),
            _ptr(gx) if grads else None, _ptr(gy) if grads else None)
    if rc != 0:
        raise ValueError(f"oracle rejected the input (code {rc})")
    return float(loss.value), gx, gy


def sample_ssim(x_plane: np.ndarray, y_plane: np.ndarray, padding, i: int, j: int) -> float:
    """SSIM map value at output (i, j) of one fp32 plane pair."""
    assert x_plane.dtype == np.float32 and x_plane.flags.c_contiguous
    H, W = x_plane.shape
    return float(_load().oracle_sample_ssim_f32(_ptr(x_plane), _ptr(y_plane), H, W,
                                                _pad(padding), i, j))


def sample_grad(x_plane: np.ndarray, y_plane: np.ndarray, padding, M: float, dloss: float,
                u: int, v: int) -> tuple[float, float]:
    """(grad_x, grad_y) at input (u, v) of one fp32 plane pair, for a loss whose
    mean covers M map entries in total, times dloss."""
    assert x_plane.dtype == np.float32 and x_plane.flags.c_contiguous
    H, W = x_plane.shape
    gx, gy = ctypes.c_double(), ctypes.c_double()
    _load().oracle_sample_grad_f32(_ptr(x_plane), _ptr(y_plane), H, W, _pad(padding),
                                   float(M), float(dloss), u, v, ctypes.byref(gx),
                                   ctypes.byref(gy))
    return float(gx.value), float(gy.value)


# --------------------------------------------------------------------------- volumes


def out_shape3(D: int, H: int, W: int, padding) -> tuple[int, int, int]:
    do, ho, wo = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _load().oracle_out_shape3(D, H, W, _pad(padding), ctypes.byref(do), ctypes.byref(ho),
                              ctypes.byref(wo))
    return int(do.value), int(ho.value), int(wo.value)


def blur3(vol: np.ndarray, padding) -> np.ndarray:
    """B3 (the 11x11x11 window) applied to one D x H x W fp64 volume."""
    vol = np.ascontiguousarray(vol, np.float64)
    D, H, W = vol.shape
    shape = out_shape3(D, H, W, padding)
    out = np.zeros(tuple(max(n, 0) for n in shape), np.float64)
    _load().oracle_blur3(_ptr(vol), D, H, W, _pad(padding), _ptr(out))
    return out


def ssim3_loss(x: np.ndarray, y: np.ndarray, padding="same", dloss: float = 1.0,
               grads: bool = True):
    """loss = 1 - mean SSIM over an NCDHW batch of volumes, and
    dloss * d loss / d(x, y).  fp32 inputs are consumed as they are; fp64
    inputs are used as given.  Returns (loss, grad_x, grad_y) (fp64 gradients,
    or None when grads is False)."""
    import math

    assert x.shape == y.shape and x.ndim == 5
    N, C, D, H, W = x.shape
    lib = _load()
    gx = np.zeros(x.shape, np.float64) if grads else None
    gy = np.zeros(x.shape, np.float64) if grads else None
    if x.dtype == np.float32 and y.dtype == np.float32:
        x = np.ascontiguousarray(x)
        y = np.ascontiguousarray(y)
        loss = ctypes.c_double()
        rc = lib.oracle_ssim3_f32(_ptr(x), _ptr(y), N, C, D, H, W, _pad(padding), float(dloss),
                                  ctypes.byref(loss), _ptr(gx) if grads else None,
                                  _ptr(gy) if grads else None)
        if rc != 0:
            raise ValueError(f"oracle rejected the input (code {rc})")
        return float(loss.value), gx, gy
    x = np.ascontiguousarray(x, np.float64)
    y = np.ascontiguousarray(y, np.float64)
    Do, Ho, Wo = out_shape3(D, H, W, padding)
    if min(Do, Ho, Wo) <= 0:
        raise ValueError("empty SSIM map")
    M = float(N * C * Do * Ho * Wo)
    sums = []
    for n in range(N):
        for c in range(C):
            sums.append(lib.oracle_ssim3_volume(
                _ptr(x[n, c]), _ptr(y[n, c]), D, H, W, _pad(padding), M, float(dloss),
                _ptr(gx[n, c]) if grads else None, _ptr(gy[n, c]) if grads else None))
    return 1.0 - math.fsum(sums) / M, gx, gy


def sample_grad3(x_vol: np.ndarray, y_vol: np.ndarray, padding, M: float, dloss: float,
                 t: int, u: int, v: int) -> tuple[float, float]:
    """(grad_x, grad_y) at voxel (t, u, v) of one fp32 volume pair, for a loss
    whose mean covers M map entries in total, times dloss."""
    assert x_vol.dtype == np.float32 and x_vol.flags.c_contiguous
    D, H, W = x_vol.shape
    gx, gy = ctypes.c_double(), ctypes.c_double()
    _load().oracle_sample_grad3_f32(_ptr(x_vol), _ptr(y_vol), D, H, W, _pad(padding), float(M),
                                    float(dloss), t, u, v, ctypes.byref(gx), ctypes.byref(gy))
    return float(gx.value), float(gy.value)
