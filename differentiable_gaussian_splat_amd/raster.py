"""Python binding of ``libgsplat_hip.so`` (C ABI in ``include/gsplat.h``).

The functions named ``gs_*`` marshal torch device tensors into the C calls of
the same names and raise :class:`GsError` on a non-zero status; all arithmetic
happens in the HIP kernels. PyTorch provides device memory and the current
stream. :class:`Rasterizer` adds buffer management (workspaces, growing the
pair buffers) and :func:`rasterize` an autograd wrapper.

The library must be built (``__graft_entry__.build()``); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import threading
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgsplat_hip.so")

GS_OK, GS_ERR_INVALID_ARG, GS_ERR_CAPACITY, GS_ERR_HIP, GS_ERR_UNSUPPORTED = 0, -1, -2, -3, -4


class GsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gsplat status {status}: {msg}")
        self.status = status


class GsCapacityError(GsError):
    def __init__(self, status, msg, needed):
        super().__init__(status, msg)
        self.needed = needed


class GsCamera(C.Structure):
    _fields_ = [("width", C.c_int32), ("height", C.c_int32), ("fx", C.c_float), ("fy", C.c_float),
                ("cx", C.c_float), ("cy", C.c_float), ("R", C.c_float * 9), ("t", C.c_float * 3)]


class GsOptions(C.Structure):
    _fields_ = [("sh_degree", C.c_int32), ("sh_rows", C.c_int32), ("tile_size", C.c_int32),
                ("lowpass", C.c_float), ("near_plane", C.c_float), ("bg", C.c_float * 3),
                ("overwrite_grads", C.c_int32)]


class GsDensifyStats(C.Structure):
    _fields_ = [("grad_accum", C.c_void_p), ("count", C.c_void_p), ("max_radius", C.c_void_p)]


def make_densify_stats(grad_accum, count, max_radius) -> GsDensifyStats:
    """Densification statistics arrays (float32 [n], int32 [n], int32 [n]),
    accumulated by the backward when passed as ``stats``."""
    return GsDensifyStats(grad_accum.data_ptr(), count.data_ptr(), max_radius.data_ptr())


def _stats(st):
    return None if st is None else C.byref(st)


class GsAdamOptions(C.Structure):
    _fields_ = [("lr_means", C.c_float), ("lr_scales", C.c_float), ("lr_quats", C.c_float),
                ("lr_opacity", C.c_float), ("lr_sh_dc", C.c_float), ("lr_sh_rest", C.c_float),
                ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float), ("step", C.c_int32)]


EXPORTS = ["gs_default_options", "gs_version", "gs_last_error", "gs_release_thread_state", "gs_preprocess",
           "gs_bin_sort_workspace_size",
           "gs_bin_sort", "gs_render_fwd", "gs_render_ckpt_bytes", "gs_render_bwd_workspace_size", "gs_render_bwd",
           "gs_render_bwd_raster",
           "gs_preprocess_bwd", "gs_preprocess_views", "gs_bin_sort_views_workspace_size", "gs_bin_sort_views",
           "gs_render_fwd_views", "gs_render_bwd_raster_views", "gs_preprocess_bwd_views", "gs_adam_step",
           "gs_mb_render_bwd_naive", "gs_mb_render_bwd_adaptive", "gs_mb_hbm_read", "gs_mb_hbm_copy", "gs_mb_atomic", "gs_render_bwd_noalloc",
           "gs_mb_render_counts", "gs_surfel_preprocess", "gs_surfel_render_fwd", "gs_surfel_render_bwd_raster",
           "gs_surfel_preprocess_bwd", "gs_surfel_render_bwd_workspace_size", "gs_surfel_render_bwd"]
SURFEL_GRAD_STRIDE = 16
NOALLOC_MAX_N = 1 << 20  # GS_NOALLOC_MAX_N
MAX_VIEWS = 32
GRAD2D_STRIDE = 12

_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Open the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(python differentiable_gaussian_splat_amd/build.py)")
        L = C.CDLL(path)
        P, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
        cam, opt = C.POINTER(GsCamera), C.POINTER(GsOptions)
        L.gs_default_options.restype = GsOptions
        L.gs_version.restype = C.c_char_p
        L.gs_last_error.restype = C.c_char_p
        L.gs_release_thread_state.argtypes = []
        L.gs_release_thread_state.restype = i32
        L.gs_preprocess.argtypes = [cam, opt, i64] + [P] * 5 + [P] * 7 + [P]
        L.gs_preprocess.restype = i32
        L.gs_bin_sort_workspace_size.argtypes = [i64, i64, i32, i32]
        L.gs_bin_sort_workspace_size.restype = sz
        L.gs_bin_sort.argtypes = [cam, opt, i64, P, P, P, P, P, sz, i64, P, P, P, C.POINTER(C.c_int64), P]
        L.gs_bin_sort.restype = i32
        L.gs_render_fwd.argtypes = [cam, opt, i64, P, P, i64, P, P, P, P, P, P, P, sz, P]
        L.gs_render_fwd.restype = i32
        L.gs_render_ckpt_bytes.argtypes = [i32, i32]
        L.gs_render_ckpt_bytes.restype = sz
        L.gs_render_bwd_workspace_size.argtypes = [i64]
        L.gs_render_bwd_workspace_size.restype = sz
        dst = C.POINTER(GsDensifyStats)
        L.gs_render_bwd.argtypes = ([cam, opt, i64] + [P] * 5 + [P] * 5 + [P, P, i64] + [P] * 3 + [P] * 6 +
                                    [P, sz, P, sz, dst, P])
        L.gs_render_bwd.restype = i32
        L.gs_render_bwd_noalloc.argtypes = ([cam, opt, i64] + [P] * 5 + [P] * 5 + [P, P, i64] + [P] * 3 + [P] * 6 +
                                            [P, sz, dst, P])
        L.gs_render_bwd_noalloc.restype = i32
        L.gs_render_bwd_raster.argtypes = [cam, opt, i64, P, P, i64] + [P] * 7 + [P, sz, P]
        L.gs_render_bwd_raster.restype = i32
        L.gs_preprocess_bwd.argtypes = [cam, opt, i64] + [P] * 8 + [P] * 6 + [dst, P]
        L.gs_preprocess_bwd.restype = i32
        PP = C.POINTER(C.c_void_p)  # five device pointers
        L.gs_preprocess_views.argtypes = [cam, i32, opt, i64] + [P] * 5 + [P] * 8 + [P]
        L.gs_preprocess_views.restype = i32
        L.gs_bin_sort_views_workspace_size.argtypes = [i32, i64, i64, i32, i32]
        L.gs_bin_sort_views_workspace_size.restype = sz
        L.gs_bin_sort_views.argtypes = [cam, i32, opt, i64, P, P, P, P, P, sz, i64, P, P, P, C.POINTER(C.c_int64), P]
        L.gs_bin_sort_views.restype = i32
        L.gs_render_fwd_views.argtypes = [cam, i32, opt, i64, P, P, i64, P, P, P, P, P, P, P]
        L.gs_render_fwd_views.restype = i32
        L.gs_render_bwd_raster_views.argtypes = [cam, i32, opt, i64, P, P, i64] + [P] * 7 + [P]
        L.gs_render_bwd_raster_views.restype = i32
        L.gs_preprocess_bwd_views.argtypes = [cam, i32, opt, i64] + [P] * 8 + [P] * 6 + [dst, P]
        L.gs_preprocess_bwd_views.restype = i32
        L.gs_adam_step.argtypes = [C.POINTER(GsAdamOptions), i64, i32, PP, PP, PP, PP, P, P, P, P]
        L.gs_adam_step.restype = i32
        L.gs_mb_render_bwd_naive.argtypes = [cam, opt, i64, P, P, i64] + [P] * 7 + [P, P]
        L.gs_mb_render_bwd_naive.restype = i32
        L.gs_mb_render_bwd_adaptive.argtypes = [cam, opt, i64, P, P, i64] + [P] * 7 + [P, sz, i32, P]
        L.gs_mb_render_bwd_adaptive.restype = i32
        L.gs_mb_render_counts.argtypes = [cam, opt, P, P, i64, P, P, P, P, P]
        L.gs_mb_render_counts.restype = i32
        L.gs_surfel_preprocess.argtypes = [cam, opt, i64] + [P] * 5 + [P] * 7 + [P]
        L.gs_surfel_preprocess.restype = i32
        L.gs_surfel_render_fwd.argtypes = [cam, opt, i64, P, P, i64, P, P, P, P, P, P, sz, P]
        L.gs_surfel_render_fwd.restype = i32
        L.gs_surfel_render_bwd_raster.argtypes = [cam, opt, i64, P, P, i64] + [P] * 6 + [P, sz, P]
        L.gs_surfel_render_bwd_raster.restype = i32
        L.gs_surfel_preprocess_bwd.argtypes = [cam, opt, i64] + [P] * 8 + [P] * 5 + [P]
        L.gs_surfel_preprocess_bwd.restype = i32
        L.gs_surfel_render_bwd_workspace_size.argtypes = [i64]
        L.gs_surfel_render_bwd_workspace_size.restype = sz
        L.gs_surfel_render_bwd.argtypes = ([cam, opt, i64] + [P] * 8 + [P, P, i64] + [P] * 3 + [P] * 5 +
                                           [P, sz, P, sz, P])
        L.gs_surfel_render_bwd.restype = i32
        L.gs_mb_hbm_read.argtypes = [P, sz, P, P]
        L.gs_mb_hbm_read.restype = i32
        L.gs_mb_hbm_copy.argtypes = [P, P, sz, P]
        L.gs_mb_hbm_copy.restype = i32
        L.gs_mb_atomic.argtypes = [P, i64, i64, i32, P]
        L.gs_mb_atomic.restype = i32
        _lib = L
        return L


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _check(status: int, name: str):
    if status != GS_OK:
        raise GsError(status, f"{name}: {load_library().gs_last_error().decode()}")


def make_camera(cam) -> GsCamera:
    """GsCamera from an object with width, height, fx, fy, cx, cy, R (3x3), t (3)."""
    c = GsCamera()
    c.width, c.height = int(cam.width), int(cam.height)
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    R = [float(x) for row in (cam.R.tolist() if hasattr(cam.R, "tolist") else cam.R) for x in row]
    t = [float(x) for x in (cam.t.tolist() if hasattr(cam.t, "tolist") else cam.t)]
    c.R = (C.c_float * 9)(*R)
    c.t = (C.c_float * 3)(*t)
    return c


def make_options(sh_degree=3, sh_rows=0, lowpass=0.3, near_plane=0.2, bg=(0.0, 0.0, 0.0), tile_size=16,
                 overwrite_grads=False) -> GsOptions:
    o = GsOptions()
    o.sh_degree, o.sh_rows, o.tile_size = int(sh_degree), int(sh_rows), int(tile_size)
    o.lowpass, o.near_plane = float(lowpass), float(near_plane)
    o.bg = (C.c_float * 3)(*[float(x) for x in bg])
    o.overwrite_grads = 1 if overwrite_grads else 0
    return o


# ------------------------------------------------------------------ thin C-ABI wrappers

def gs_version() -> str:
    return load_library().gs_version().decode()


def gs_release_thread_state():
    """Frees the calling thread's pair-count readback buffers (gs_bin_sort makes them again)."""
    _check(load_library().gs_release_thread_state(), "gs_release_thread_state")


def gs_preprocess(cam: GsCamera, opt: GsOptions, means, scales, quats, opacities, sh, means2d, depths,
                  conic_opacity, rgb, radii, tiles_touched, clamped, stream=None):
    n = means.shape[0]
    st = load_library().gs_preprocess(C.byref(cam), C.byref(opt), n, _p(means), _p(scales), _p(quats),
                                      _p(opacities), _p(sh), _p(means2d), _p(depths), _p(conic_opacity), _p(rgb),
                                      _p(radii), _p(tiles_touched), _p(clamped), _stream(stream))
    _check(st, "gs_preprocess")


def gs_bin_sort_workspace_size(n, pair_capacity, width, height) -> int:
    return int(load_library().gs_bin_sort_workspace_size(n, pair_capacity, width, height))


def gs_bin_sort(cam: GsCamera, opt: GsOptions, means2d, depths, radii, tiles_touched, workspace, pair_capacity,
                keys, values, ranges, stream=None) -> int:
    """Returns the pair count P; raises GsCapacityError (with .needed) if P > pair_capacity."""
    n = means2d.shape[0]
    npairs = C.c_int64(0)
    st = load_library().gs_bin_sort(C.byref(cam), C.byref(opt), n, _p(means2d), _p(depths), _p(radii),
                                    _p(tiles_touched), _p(workspace),
                                    workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                    pair_capacity, _p(keys), _p(values), _p(ranges), C.byref(npairs),
                                    _stream(stream))
    if st == GS_ERR_CAPACITY:
        raise GsCapacityError(st, load_library().gs_last_error().decode(), npairs.value)
    _check(st, "gs_bin_sort")
    return int(npairs.value)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def gs_render_ckpt_bytes(width, height) -> int:
    """Bytes of render checkpoints for one view of this size (0: not used)."""
    return int(load_library().gs_render_ckpt_bytes(width, height))


def gs_render_fwd(cam: GsCamera, opt: GsOptions, n, ranges, values, n_pairs, means2d, conic_opacity, rgb, image,
                  final_T, n_contrib, ckpt=None, stream=None):
    st = load_library().gs_render_fwd(C.byref(cam), C.byref(opt), n, _p(ranges), _p(values), n_pairs, _p(means2d),
                                      _p(conic_opacity), _p(rgb), _p(image), _p(final_T), _p(n_contrib), _p(ckpt),
                                      _nbytes(ckpt), _stream(stream))
    _check(st, "gs_render_fwd")


def gs_render_bwd_workspace_size(n) -> int:
    return int(load_library().gs_render_bwd_workspace_size(n))


def gs_render_bwd(cam: GsCamera, opt: GsOptions, means, scales, quats, opacities, sh, means2d, conic_opacity, rgb,
                  radii, clamped, ranges, values, n_pairs, final_T, n_contrib, dL_dimage, dL_dmeans, dL_dscales,
                  dL_dquats, dL_dopacities, dL_dsh, dL_dmeans2d, workspace, stats=None, ckpt=None, stream=None):
    n = means.shape[0]
    st = load_library().gs_render_bwd(
        C.byref(cam), C.byref(opt), n, _p(means), _p(scales), _p(quats), _p(opacities), _p(sh), _p(means2d),
        _p(conic_opacity), _p(rgb), _p(radii), _p(clamped), _p(ranges), _p(values), n_pairs, _p(final_T),
        _p(n_contrib), _p(dL_dimage), _p(dL_dmeans), _p(dL_dscales), _p(dL_dquats), _p(dL_dopacities), _p(dL_dsh),
        _p(dL_dmeans2d), _p(workspace), workspace.numel() * workspace.element_size(), _p(ckpt), _nbytes(ckpt),
        _stats(stats), _stream(stream))
    _check(st, "gs_render_bwd")


def gs_render_bwd_noalloc(cam: GsCamera, opt: GsOptions, means, scales, quats, opacities, sh, means2d, conic_opacity,
                          rgb, radii, clamped, ranges, values, n_pairs, final_T, n_contrib, dL_dimage, dL_dmeans,
                          dL_dscales, dL_dquats, dL_dopacities, dL_dsh, dL_dmeans2d, stats=None, ckpt=None,
                          stream=None):
    """gs_render_bwd with the library's own fixed scratch instead of a workspace
    (at most NOALLOC_MAX_N Gaussians; calls on one GPU must not overlap)."""
    n = means.shape[0]
    st = load_library().gs_render_bwd_noalloc(
        C.byref(cam), C.byref(opt), n, _p(means), _p(scales), _p(quats), _p(opacities), _p(sh), _p(means2d),
        _p(conic_opacity), _p(rgb), _p(radii), _p(clamped), _p(ranges), _p(values), n_pairs, _p(final_T),
        _p(n_contrib), _p(dL_dimage), _p(dL_dmeans), _p(dL_dscales), _p(dL_dquats), _p(dL_dopacities), _p(dL_dsh),
        _p(dL_dmeans2d), _p(ckpt), _nbytes(ckpt), _stats(stats), _stream(stream))
    _check(st, "gs_render_bwd_noalloc")


def gs_render_bwd_raster(cam: GsCamera, opt: GsOptions, n, ranges, values, n_pairs, means2d, conic_opacity, rgb,
                         final_T, n_contrib, dL_dimage, grad2d, ckpt=None, stream=None):
    st = load_library().gs_render_bwd_raster(C.byref(cam), C.byref(opt), n, _p(ranges), _p(values), n_pairs,
                                             _p(means2d), _p(conic_opacity), _p(rgb), _p(final_T), _p(n_contrib),
                                             _p(dL_dimage), _p(grad2d), _p(ckpt), _nbytes(ckpt), _stream(stream))
    _check(st, "gs_render_bwd_raster")


def gs_preprocess_bwd(cam: GsCamera, opt: GsOptions, means, scales, quats, sh, conic_opacity, radii, clamped, grad2d,
                      dL_dmeans, dL_dscales, dL_dquats, dL_dopacities, dL_dsh, dL_dmeans2d=None, stats=None,
                      stream=None):
    n = means.shape[0]
    st = load_library().gs_preprocess_bwd(C.byref(cam), C.byref(opt), n, _p(means), _p(scales), _p(quats), _p(sh),
                                          _p(conic_opacity), _p(radii), _p(clamped), _p(grad2d), _p(dL_dmeans),
                                          _p(dL_dscales), _p(dL_dquats), _p(dL_dopacities), _p(dL_dsh),
                                          _p(dL_dmeans2d), _stats(stats), _stream(stream))
    _check(st, "gs_preprocess_bwd")


# ------------------------------------------------------------------ several views per launch

def make_cameras(cameras):
    """ctypes array of GsCamera (one image size) for the *_views calls."""
    cams = [c if isinstance(c, GsCamera) else make_camera(c) for c in cameras]
    return (GsCamera * len(cams))(*cams)


def gs_preprocess_views(cams, opt: GsOptions, means, scales, quats, opacities, sh, means2d, depths, conic_opacity,
                        rgb, radii, tiles_touched, clamped, vis_mask=None, stream=None):
    n = means.shape[0]
    st = load_library().gs_preprocess_views(cams, len(cams), C.byref(opt), n, _p(means), _p(scales), _p(quats),
                                            _p(opacities), _p(sh), _p(means2d), _p(depths), _p(conic_opacity),
                                            _p(rgb), _p(radii), _p(tiles_touched), _p(clamped), _p(vis_mask),
                                            _stream(stream))
    _check(st, "gs_preprocess_views")


def gs_bin_sort_views_workspace_size(n_views, n, pair_capacity, width, height) -> int:
    return int(load_library().gs_bin_sort_views_workspace_size(n_views, n, pair_capacity, width, height))


def gs_bin_sort_views(cams, opt: GsOptions, n, means2d, depths, radii, tiles_touched, workspace, pair_capacity, keys,
                      values, ranges, stream=None) -> int:
    """Returns the pair count P over all views; raises GsCapacityError (with
    .needed) if P > pair_capacity."""
    npairs = C.c_int64(0)
    st = load_library().gs_bin_sort_views(cams, len(cams), C.byref(opt), n, _p(means2d), _p(depths), _p(radii),
                                          _p(tiles_touched), _p(workspace),
                                          workspace.numel() * workspace.element_size() if workspace is not None
                                          else 0, pair_capacity, _p(keys), _p(values), _p(ranges),
                                          C.byref(npairs), _stream(stream))
    if st == GS_ERR_CAPACITY:
        raise GsCapacityError(st, load_library().gs_last_error().decode(), npairs.value)
    _check(st, "gs_bin_sort_views")
    return int(npairs.value)


def gs_render_fwd_views(cams, opt: GsOptions, n, ranges, values, n_pairs, means2d, conic_opacity, rgb, image, final_T,
                        n_contrib, stream=None):
    st = load_library().gs_render_fwd_views(cams, len(cams), C.byref(opt), n, _p(ranges), _p(values), n_pairs,
                                            _p(means2d), _p(conic_opacity), _p(rgb), _p(image), _p(final_T),
                                            _p(n_contrib), _stream(stream))
    _check(st, "gs_render_fwd_views")


def gs_render_bwd_raster_views(cams, opt: GsOptions, n, ranges, values, n_pairs, means2d, conic_opacity, rgb,
                               final_T, n_contrib, dL_dimage, grad2d, stream=None):
    st = load_library().gs_render_bwd_raster_views(cams, len(cams), C.byref(opt), n, _p(ranges), _p(values),
                                                   n_pairs, _p(means2d), _p(conic_opacity), _p(rgb), _p(final_T),
                                                   _p(n_contrib), _p(dL_dimage), _p(grad2d), _stream(stream))
    _check(st, "gs_render_bwd_raster_views")


def gs_preprocess_bwd_views(cams, opt: GsOptions, means, scales, quats, sh, conic_opacity, radii, clamped, grad2d,
                            dL_dmeans, dL_dscales, dL_dquats, dL_dopacities, dL_dsh, dL_dmeans2d=None, stats=None,
                            stream=None):
    n = means.shape[0]
    st = load_library().gs_preprocess_bwd_views(cams, len(cams), C.byref(opt), n, _p(means), _p(scales), _p(quats),
                                                _p(sh), _p(conic_opacity), _p(radii), _p(clamped), _p(grad2d),
                                                _p(dL_dmeans), _p(dL_dscales), _p(dL_dquats), _p(dL_dopacities),
                                                _p(dL_dsh), _p(dL_dmeans2d), _stats(stats), _stream(stream))
    _check(st, "gs_preprocess_bwd_views")


PARAM_GROUPS = ("means", "log_scales", "quats", "opacity_logits", "sh")


def make_adam_options(step, lr_means=1.6e-4, lr_scales=5e-3, lr_quats=1e-3, lr_opacity=5e-2, lr_sh_dc=2.5e-3,
                      lr_sh_rest=2.5e-3 / 20, beta1=0.9, beta2=0.999, eps=1e-15) -> GsAdamOptions:
    o = GsAdamOptions()
    o.lr_means, o.lr_scales, o.lr_quats, o.lr_opacity = lr_means, lr_scales, lr_quats, lr_opacity
    o.lr_sh_dc, o.lr_sh_rest = lr_sh_dc, lr_sh_rest
    o.beta1, o.beta2, o.eps, o.step = beta1, beta2, eps, int(step)
    return o


def gs_adam_step(opt: GsAdamOptions, params: dict, grads: dict, exp_avg: dict, exp_avg_sq: dict, scales,
                 opacities, grad_norm=None, stream=None):
    """One fused Adam update. params / exp_avg / exp_avg_sq: dicts over
    PARAM_GROUPS (raw parameters and their moments, updated in place); grads:
    the rasterizer's gradients keyed means, scales, quats, opacities, sh (with
    respect to the activated scales and opacities)."""
    n = params["means"].shape[0]
    sh_rows = params["sh"].shape[1]
    arr = lambda ts: (C.c_void_p * 5)(*[t.data_ptr() for t in ts])
    gkeys = ("means", "scales", "quats", "opacities", "sh")
    st = load_library().gs_adam_step(C.byref(opt), n, sh_rows, arr([params[k] for k in PARAM_GROUPS]),
                                     arr([grads[k] for k in gkeys]), arr([exp_avg[k] for k in PARAM_GROUPS]),
                                     arr([exp_avg_sq[k] for k in PARAM_GROUPS]), _p(scales), _p(opacities),
                                     _p(grad_norm), _stream(stream))
    _check(st, "gs_adam_step")


def gs_mb_render_bwd_naive(cam: GsCamera, opt: GsOptions, n, ranges, values, n_pairs, means2d, conic_opacity, rgb,
                           final_T, n_contrib, dL_dimage, grad2d, lane_hist=None, stream=None):
    st = load_library().gs_mb_render_bwd_naive(C.byref(cam), C.byref(opt), n, _p(ranges), _p(values), n_pairs,
                                               _p(means2d), _p(conic_opacity), _p(rgb), _p(final_T), _p(n_contrib),
                                               _p(dL_dimage), _p(grad2d), _p(lane_hist), _stream(stream))
    _check(st, "gs_mb_render_bwd_naive")


def gs_mb_render_bwd_adaptive(cam: GsCamera, opt: GsOptions, n, ranges, values, n_pairs, means2d, conic_opacity,
                              rgb, final_T, n_contrib, dL_dimage, grad2d, ckpt, direct_max, stream=None):
    st = load_library().gs_mb_render_bwd_adaptive(C.byref(cam), C.byref(opt), n, _p(ranges), _p(values), n_pairs,
                                                  _p(means2d), _p(conic_opacity), _p(rgb), _p(final_T),
                                                  _p(n_contrib), _p(dL_dimage), _p(grad2d), _p(ckpt), _nbytes(ckpt),
                                                  int(direct_max), _stream(stream))
    _check(st, "gs_mb_render_bwd_adaptive")


def gs_mb_render_counts(cam: GsCamera, opt: GsOptions, ranges, values, n_pairs, means2d, conic_opacity, rgb, counts,
                        stream=None):
    """Adds the blending work counts of one view to counts (int64 [7]): E_f, E_f
    evaluated by the forward, E_blend, E_b, P_c, executed backward band-steps,
    the backward's walked tile-entries."""
    st = load_library().gs_mb_render_counts(C.byref(cam), C.byref(opt), _p(ranges), _p(values), n_pairs,
                                            _p(means2d), _p(conic_opacity), _p(rgb), _p(counts), _stream(stream))
    _check(st, "gs_mb_render_counts")


# ---------------------------------------------------------------- 2D Gaussian surfels

def gs_surfel_preprocess(cam: GsCamera, opt: GsOptions, means, scales, quats, opacities, sh, means2d, depths,
                         transforms, rgb, radii, tiles_touched, clamped, stream=None):
    n = means.shape[0]
    st = load_library().gs_surfel_preprocess(C.byref(cam), C.byref(opt), n, _p(means), _p(scales), _p(quats),
                                             _p(opacities), _p(sh), _p(means2d), _p(depths), _p(transforms), _p(rgb),
                                             _p(radii), _p(tiles_touched), _p(clamped), _stream(stream))
    _check(st, "gs_surfel_preprocess")


def gs_surfel_render_fwd(cam: GsCamera, opt: GsOptions, n, ranges, values, n_pairs, transforms, rgb, image, final_T,
                         n_contrib, ckpt=None, stream=None):
    st = load_library().gs_surfel_render_fwd(C.byref(cam), C.byref(opt), n, _p(ranges), _p(values), n_pairs,
                                             _p(transforms), _p(rgb), _p(image), _p(final_T), _p(n_contrib),
                                             _p(ckpt), _nbytes(ckpt), _stream(stream))
    _check(st, "gs_surfel_render_fwd")


def gs_surfel_render_bwd_raster(cam: GsCamera, opt: GsOptions, n, ranges, values, n_pairs, transforms, rgb, final_T,
                                n_contrib, dL_dimage, grad, ckpt=None, stream=None):
    st = load_library().gs_surfel_render_bwd_raster(C.byref(cam), C.byref(opt), n, _p(ranges), _p(values), n_pairs,
                                                    _p(transforms), _p(rgb), _p(final_T), _p(n_contrib),
                                                    _p(dL_dimage), _p(grad), _p(ckpt), _nbytes(ckpt),
                                                    _stream(stream))
    _check(st, "gs_surfel_render_bwd_raster")


def gs_surfel_preprocess_bwd(cam: GsCamera, opt: GsOptions, means, scales, quats, sh, transforms, radii, clamped,
                             grad, dL_dmeans, dL_dscales, dL_dquats, dL_dopacities, dL_dsh, stream=None):
    n = means.shape[0]
    st = load_library().gs_surfel_preprocess_bwd(C.byref(cam), C.byref(opt), n, _p(means), _p(scales), _p(quats),
                                                 _p(sh), _p(transforms), _p(radii), _p(clamped), _p(grad),
                                                 _p(dL_dmeans), _p(dL_dscales), _p(dL_dquats), _p(dL_dopacities),
                                                 _p(dL_dsh), _stream(stream))
    _check(st, "gs_surfel_preprocess_bwd")


def gs_surfel_render_bwd_workspace_size(n) -> int:
    return int(load_library().gs_surfel_render_bwd_workspace_size(n))


def gs_surfel_render_bwd(cam: GsCamera, opt: GsOptions, means, scales, quats, sh, transforms, rgb, radii, clamped,
                         ranges, values, n_pairs, final_T, n_contrib, dL_dimage, dL_dmeans, dL_dscales, dL_dquats,
                         dL_dopacities, dL_dsh, workspace, ckpt=None, stream=None):
    n = means.shape[0]
    st = load_library().gs_surfel_render_bwd(
        C.byref(cam), C.byref(opt), n, _p(means), _p(scales), _p(quats), _p(sh), _p(transforms), _p(rgb), _p(radii),
        _p(clamped), _p(ranges), _p(values), n_pairs, _p(final_T), _p(n_contrib), _p(dL_dimage), _p(dL_dmeans),
        _p(dL_dscales), _p(dL_dquats), _p(dL_dopacities), _p(dL_dsh), _p(workspace),
        workspace.numel() * workspace.element_size(), _p(ckpt), _nbytes(ckpt), _stream(stream))
    _check(st, "gs_surfel_render_bwd")


def gs_mb_hbm_read(src, sink, stream=None):
    _check(load_library().gs_mb_hbm_read(_p(src), src.numel() * src.element_size(), _p(sink), _stream(stream)),
           "gs_mb_hbm_read")


def gs_mb_hbm_copy(dst, src, stream=None):
    _check(load_library().gs_mb_hbm_copy(_p(dst), _p(src), src.numel() * src.element_size(), _stream(stream)),
           "gs_mb_hbm_copy")


def gs_mb_atomic(records, n_records, n_ops, lanes_per_record, stream=None):
    _check(load_library().gs_mb_atomic(_p(records), n_records, n_ops, lanes_per_record, _stream(stream)),
           "gs_mb_atomic")


# ------------------------------------------------------------------ buffer management

@dataclass
class Frame:
    """Device state of one rendered view, kept for its backward."""
    cam: GsCamera
    opt: GsOptions
    width: int
    height: int
    means2d: torch.Tensor
    depths: torch.Tensor
    conic_opacity: torch.Tensor
    rgb: torch.Tensor
    radii: torch.Tensor
    tiles_touched: torch.Tensor
    clamped: torch.Tensor
    n_pairs: int
    keys: torch.Tensor | None
    values: torch.Tensor
    ranges: torch.Tensor
    image: torch.Tensor
    final_T: torch.Tensor
    n_contrib: torch.Tensor
    ckpt: torch.Tensor | None = None  # the forward's render checkpoints, read by this frame's backward


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


class Rasterizer:
    """Owns the workspaces and pair buffers across calls (sized on first use,
    grown when a frame needs more pairs)."""

    def __init__(self, device="cuda", pair_capacity: int = 0, want_keys: bool = False):
        self.device = torch.device(device)
        self.pair_capacity = int(pair_capacity)
        self.want_keys = want_keys
        self._values = None
        self._keys = None
        self._bin_ws = None
        self._bwd_ws = None
        self._ws_key = None

    def _ensure_pairs(self, cap: int):
        if self._values is None or self._values.numel() < max(cap, 1):
            self.pair_capacity = max(cap, 1)
            self._values = _empty(self.pair_capacity, torch.int32, self.device)
            self._keys = _empty(self.pair_capacity, torch.int64, self.device) if self.want_keys else None

    def _ensure_bin_ws(self, n, W, H):
        need = gs_bin_sort_workspace_size(n, self.pair_capacity, W, H)
        if self._bin_ws is None or self._bin_ws.numel() < need:
            self._bin_ws = _empty(need, torch.uint8, self.device)

    def preprocess(self, cam, opt, means, scales, quats, opacities, sh):
        n = means.shape[0]
        dev = means.device
        out = dict(means2d=_empty((n, 2), torch.float32, dev), depths=_empty(n, torch.float32, dev),
                   conic_opacity=_empty((n, 4), torch.float32, dev), rgb=_empty((n, 3), torch.float32, dev),
                   radii=_empty(n, torch.int32, dev), tiles_touched=_empty(n, torch.int32, dev),
                   clamped=_empty(n, torch.uint8, dev))
        gs_preprocess(cam, opt, means, scales, quats, opacities, sh, out["means2d"], out["depths"],
                      out["conic_opacity"], out["rgb"], out["radii"], out["tiles_touched"], out["clamped"])
        return out

    def bin_sort(self, cam, opt, pre, ranges=None):
        n = pre["means2d"].shape[0]
        W, H = cam.width, cam.height
        ntiles = ((W + 15) // 16) * ((H + 15) // 16)
        if ranges is None:
            ranges = _empty((ntiles, 2), torch.int32, self.device)
        self._ensure_pairs(self.pair_capacity)
        while True:
            self._ensure_bin_ws(n, W, H)
            try:
                P = gs_bin_sort(cam, opt, pre["means2d"], pre["depths"], pre["radii"], pre["tiles_touched"],
                                self._bin_ws, self.pair_capacity, self._keys, self._values, ranges)
                return P, ranges
            except GsCapacityError as e:
                self._values = None
                self._ensure_pairs(int(e.needed * 1.15) + 1024)

    def forward(self, camera, means, scales, quats, opacities, sh, sh_degree, lowpass=0.3, near_plane=0.2,
                bg=(0.0, 0.0, 0.0)) -> Frame:
        cam = camera if isinstance(camera, GsCamera) else make_camera(camera)
        rows = sh.shape[1]
        opt = make_options(sh_degree, rows, lowpass, near_plane, bg)
        pre = self.preprocess(cam, opt, means, scales, quats, opacities, sh)
        P, ranges = self.bin_sort(cam, opt, pre)
        W, H = cam.width, cam.height
        image = _empty((3, H, W), torch.float32, self.device)
        final_T = _empty((H, W), torch.float32, self.device)
        n_contrib = _empty((H, W), torch.int32, self.device)
        # checkpoints belong to this frame (its backward reads them), so each frame gets its own
        nck = gs_render_ckpt_bytes(W, H)
        ckpt = _empty(nck, torch.uint8, self.device) if nck else None
        gs_render_fwd(cam, opt, means.shape[0], ranges, self._values, P, pre["means2d"], pre["conic_opacity"],
                      pre["rgb"], image, final_T, n_contrib, ckpt)
        return Frame(cam, opt, W, H, pre["means2d"], pre["depths"], pre["conic_opacity"], pre["rgb"], pre["radii"],
                     pre["tiles_touched"], pre["clamped"], P, self._keys, self._values, ranges, image, final_T,
                     n_contrib, ckpt)

    def backward(self, frame: Frame, means, scales, quats, opacities, sh, dL_dimage, grads: dict,
                 want_means2d: bool = False, overwrite: bool = False, stats: GsDensifyStats | None = None):
        """Accumulates parameter gradients into ``grads`` (keys means, scales,
        quats, opacities, sh and optionally means2d), or with ``overwrite``
        writes them (every row), so that ``grads`` need not be zeroed."""
        n = means.shape[0]
        need = gs_render_bwd_workspace_size(n)
        if self._bwd_ws is None or self._bwd_ws.numel() < need:
            self._bwd_ws = _empty(need, torch.uint8, self.device)
        if want_means2d and "means2d" not in grads:
            grads["means2d"] = (_empty((n, 2), torch.float32, means.device) if overwrite else
                                torch.zeros((n, 2), dtype=torch.float32, device=means.device))
        opt = frame.opt
        if overwrite:
            opt = GsOptions.from_buffer_copy(frame.opt)
            opt.overwrite_grads = 1
        gs_render_bwd(frame.cam, opt, means, scales, quats, opacities, sh, frame.means2d, frame.conic_opacity,
                      frame.rgb, frame.radii, frame.clamped, frame.ranges, frame.values, frame.n_pairs,
                      frame.final_T, frame.n_contrib, dL_dimage, grads["means"], grads["scales"], grads["quats"],
                      grads["opacities"], grads["sh"], grads.get("means2d") if want_means2d else None,
                      self._bwd_ws, stats, frame.ckpt)
        return grads

    def surfel_forward(self, camera, means, scales, quats, opacities, sh, sh_degree, near_plane=0.2,
                       bg=(0.0, 0.0, 0.0)) -> "Frame":
        """2D Gaussian surfels (scales [n, 2]): projection, the same binning, compositing.
        The frame's conic_opacity field holds the surfels' transforms [n, 12]."""
        cam = camera if isinstance(camera, GsCamera) else make_camera(camera)
        opt = make_options(sh_degree, sh.shape[1], 0.3, near_plane, bg)
        n, dev = means.shape[0], means.device
        pre = dict(means2d=_empty((n, 2), torch.float32, dev), depths=_empty(n, torch.float32, dev),
                   conic_opacity=_empty((n, 12), torch.float32, dev), rgb=_empty((n, 3), torch.float32, dev),
                   radii=_empty(n, torch.int32, dev), tiles_touched=_empty(n, torch.int32, dev),
                   clamped=_empty(n, torch.uint8, dev))
        gs_surfel_preprocess(cam, opt, means, scales, quats, opacities, sh, pre["means2d"], pre["depths"],
                             pre["conic_opacity"], pre["rgb"], pre["radii"], pre["tiles_touched"], pre["clamped"])
        P, ranges = self.bin_sort(cam, opt, pre)
        W, H = cam.width, cam.height
        image = _empty((3, H, W), torch.float32, self.device)
        final_T = _empty((H, W), torch.float32, self.device)
        n_contrib = _empty((H, W), torch.int32, self.device)
        nck = gs_render_ckpt_bytes(W, H)
        ckpt = _empty(nck, torch.uint8, self.device) if nck else None
        gs_surfel_render_fwd(cam, opt, n, ranges, self._values, P, pre["conic_opacity"], pre["rgb"], image, final_T,
                             n_contrib, ckpt)
        return Frame(cam, opt, W, H, pre["means2d"], pre["depths"], pre["conic_opacity"], pre["rgb"], pre["radii"],
                     pre["tiles_touched"], pre["clamped"], P, self._keys, self._values, ranges, image, final_T,
                     n_contrib, ckpt)

    def surfel_backward(self, frame: "Frame", means, scales, quats, sh, dL_dimage, grads: dict,
                        overwrite: bool = False):
        """Accumulates (or with ``overwrite`` writes) surfel parameter gradients
        into ``grads`` (means [n,3], scales [n,2], quats, opacities, sh)."""
        n = means.shape[0]
        need = gs_surfel_render_bwd_workspace_size(n)
        if self._bwd_ws is None or self._bwd_ws.numel() < need:
            self._bwd_ws = _empty(need, torch.uint8, self.device)
        opt = frame.opt
        if overwrite:
            opt = GsOptions.from_buffer_copy(frame.opt)
            opt.overwrite_grads = 1
        gs_surfel_render_bwd(frame.cam, opt, means, scales, quats, sh, frame.conic_opacity, frame.rgb, frame.radii,
                             frame.clamped, frame.ranges, frame.values, frame.n_pairs, frame.final_T,
                             frame.n_contrib, dL_dimage, grads["means"], grads["scales"], grads["quats"],
                             grads["opacities"], grads["sh"], self._bwd_ws, frame.ckpt)
        return grads


@dataclass
class ViewsFrame:
    """Device state of V views rendered in one batch: per-view arrays carry a
    leading view axis (entry v n + g), the pair list covers all views."""
    cams: object
    opt: GsOptions
    width: int
    height: int
    means2d: torch.Tensor
    depths: torch.Tensor
    conic_opacity: torch.Tensor
    rgb: torch.Tensor
    radii: torch.Tensor
    tiles_touched: torch.Tensor
    clamped: torch.Tensor
    vis_mask: torch.Tensor
    n_pairs: int
    keys: torch.Tensor | None
    values: torch.Tensor
    ranges: torch.Tensor
    image: torch.Tensor
    final_T: torch.Tensor
    n_contrib: torch.Tensor


class ViewsRasterizer(Rasterizer):
    """Rasterizer of V views of one image size per launch."""

    def forward_views(self, cameras, means, scales, quats, opacities, sh, sh_degree, lowpass=0.3, near_plane=0.2,
                      bg=(0.0, 0.0, 0.0)) -> ViewsFrame:
        cams = cameras if isinstance(cameras, C.Array) else make_cameras(cameras)
        V, n, dev = len(cams), means.shape[0], means.device
        opt = make_options(sh_degree, sh.shape[1], lowpass, near_plane, bg)
        pre = dict(means2d=_empty((V, n, 2), torch.float32, dev), depths=_empty((V, n), torch.float32, dev),
                   conic_opacity=_empty((V, n, 4), torch.float32, dev), rgb=_empty((V, n, 3), torch.float32, dev),
                   radii=_empty((V, n), torch.int32, dev), tiles_touched=_empty((V, n), torch.int32, dev),
                   clamped=_empty((V, n), torch.uint8, dev), vis_mask=_empty(n, torch.int32, dev))
        gs_preprocess_views(cams, opt, means, scales, quats, opacities, sh, pre["means2d"], pre["depths"],
                            pre["conic_opacity"], pre["rgb"], pre["radii"], pre["tiles_touched"], pre["clamped"],
                            pre["vis_mask"])
        W, H = cams[0].width, cams[0].height
        ntiles = ((W + 15) // 16) * ((H + 15) // 16)
        ranges = _empty((V * ntiles, 2), torch.int32, self.device)
        self._ensure_pairs(self.pair_capacity)
        while True:
            need = gs_bin_sort_views_workspace_size(V, n, self.pair_capacity, W, H)
            if self._bin_ws is None or self._bin_ws.numel() < need:
                self._bin_ws = _empty(need, torch.uint8, self.device)
            try:
                P = gs_bin_sort_views(cams, opt, n, pre["means2d"], pre["depths"], pre["radii"],
                                      pre["tiles_touched"], self._bin_ws, self.pair_capacity, self._keys,
                                      self._values, ranges)
                break
            except GsCapacityError as e:
                self._values = None
                self._ensure_pairs(int(e.needed * 1.15) + 1024)
        image = _empty((V, 3, H, W), torch.float32, self.device)
        final_T = _empty((V, H, W), torch.float32, self.device)
        n_contrib = _empty((V, H, W), torch.int32, self.device)
        gs_render_fwd_views(cams, opt, n, ranges, self._values, P, pre["means2d"], pre["conic_opacity"], pre["rgb"],
                            image, final_T, n_contrib)
        return ViewsFrame(cams, opt, W, H, pre["means2d"], pre["depths"], pre["conic_opacity"], pre["rgb"],
                          pre["radii"], pre["tiles_touched"], pre["clamped"], pre["vis_mask"], P, self._keys,
                          self._values, ranges, image, final_T, n_contrib)

    def backward_views(self, frame: ViewsFrame, means, scales, quats, opacities, sh, dL_dimage, grads: dict,
                       want_means2d: bool = False, overwrite: bool = False, stats: GsDensifyStats | None = None):
        """Sum over the frame's views of the gradients (added into ``grads``,
        or written with ``overwrite``); grads["means2d"] gets [V, n, 2]."""
        V, n = len(frame.cams), means.shape[0]
        grad2d = torch.zeros((V, n, GRAD2D_STRIDE), dtype=torch.float32, device=means.device)
        if want_means2d and "means2d" not in grads:
            grads["means2d"] = (_empty((V, n, 2), torch.float32, means.device) if overwrite else
                                torch.zeros((V, n, 2), dtype=torch.float32, device=means.device))
        opt = frame.opt
        if overwrite:
            opt = GsOptions.from_buffer_copy(frame.opt)
            opt.overwrite_grads = 1
        gs_render_bwd_raster_views(frame.cams, opt, n, frame.ranges, frame.values, frame.n_pairs, frame.means2d,
                                   frame.conic_opacity, frame.rgb, frame.final_T, frame.n_contrib, dL_dimage, grad2d)
        gs_preprocess_bwd_views(frame.cams, opt, means, scales, quats, sh, frame.conic_opacity, frame.radii,
                                frame.clamped, grad2d, grads["means"], grads["scales"], grads["quats"],
                                grads["opacities"], grads["sh"], grads.get("means2d") if want_means2d else None,
                                stats)
        return grads


def zero_grads(means, sh):
    n = means.shape[0]
    dev = means.device
    return dict(means=torch.zeros((n, 3), device=dev), scales=torch.zeros((n, 3), device=dev),
                quats=torch.zeros((n, 4), device=dev), opacities=torch.zeros(n, device=dev),
                sh=torch.zeros_like(sh))


def empty_grads(means, sh):
    """Gradient buffers for a backward with overwrite=True (contents undefined)."""
    n = means.shape[0]
    dev = means.device
    return dict(means=_empty((n, 3), torch.float32, dev), scales=_empty((n, 3), torch.float32, dev),
                quats=_empty((n, 4), torch.float32, dev), opacities=_empty(n, torch.float32, dev),
                sh=torch.empty_like(sh))


class _RasterizeFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, means, scales, quats, opacities, sh, rasterizer, camera, sh_degree, lowpass, near_plane, bg):
        frame = rasterizer.forward(camera, means, scales, quats, opacities, sh, sh_degree, lowpass, near_plane, bg)
        ctx.rasterizer = rasterizer
        ctx.frame = frame
        ctx.save_for_backward(means, scales, quats, opacities, sh)
        # the pair buffer is shared across frames of one Rasterizer: keep this frame's values
        ctx.values = frame.values[: max(frame.n_pairs, 1)].clone()
        return frame.image

    @staticmethod
    def backward(ctx, dL_dimage):
        means, scales, quats, opacities, sh = ctx.saved_tensors
        frame = ctx.frame
        frame.values = ctx.values
        grads = empty_grads(means, sh)
        ctx.rasterizer.backward(frame, means.contiguous(), scales.contiguous(), quats.contiguous(),
                                opacities.contiguous(), sh.contiguous(), dL_dimage.contiguous(), grads, overwrite=True)
        return grads["means"], grads["scales"], grads["quats"], grads["opacities"], grads["sh"], None, None, None, \
            None, None, None


def rasterize(means, scales, quats, opacities, sh, camera, sh_degree=3, rasterizer: Rasterizer | None = None,
              lowpass=0.3, near_plane=0.2, bg=(0.0, 0.0, 0.0)):
    """Differentiable image [3, H, W] of the Gaussians seen by ``camera``
    (activated scales and opacities; quaternions (w, x, y, z))."""
    r = rasterizer if rasterizer is not None else Rasterizer(means.device)
    return _RasterizeFn.apply(means.contiguous(), scales.contiguous(), quats.contiguous(), opacities.contiguous(),
                              sh.contiguous(), r, camera, sh_degree, lowpass, near_plane, tuple(bg))
