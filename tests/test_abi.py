"""C ABI checks that need no GPU: the library loads, exports every function
``include/gsplat.h`` declares, and rejects bad arguments before launching."""
import ctypes as C
import os
import re

import pytest

from differentiable_gaussian_splat_amd import raster
from differentiable_gaussian_splat_amd.scenes import Camera, make_scene

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "gsplat.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gs_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_four_phases():
    fns = header_functions()
    for f in ("gs_preprocess", "gs_bin_sort", "gs_render_fwd", "gs_render_bwd"):
        assert f in fns


def test_library_exports_every_declared_function():
    L = raster.load_library()
    missing = [f for f in header_functions() if not hasattr(L, f)]
    assert not missing, missing
    assert sorted(raster.EXPORTS) == header_functions()


def test_struct_layouts_match_header():
    # gs_camera: 2 int32 + 4 float + 9 float + 3 float; gs_options: 3 int32 + 2 float + 3 float + 1 int32
    assert C.sizeof(raster.GsCamera) == 4 * (2 + 4 + 9 + 3)
    assert C.sizeof(raster.GsOptions) == 4 * (3 + 2 + 3 + 1)
    d = raster.load_library().gs_default_options()
    assert (d.sh_degree, d.sh_rows, d.tile_size, d.overwrite_grads) == (3, 0, 16, 0)
    assert abs(d.lowpass - 0.3) < 1e-7 and abs(d.near_plane - 0.2) < 1e-7


def test_version_and_last_error():
    assert "gfx950" in raster.gs_version()
    assert isinstance(raster.load_library().gs_last_error(), bytes)


def _cam():
    return raster.make_camera(make_scene(1, 0, n=4).cameras[0])


@pytest.mark.parametrize("mutate,code", [
    (lambda c, o: setattr(o, "sh_degree", 4), raster.GS_ERR_INVALID_ARG),
    (lambda c, o: setattr(o, "tile_size", 8), raster.GS_ERR_UNSUPPORTED),
    (lambda c, o: setattr(c, "fx", 0.0), raster.GS_ERR_INVALID_ARG),
    (lambda c, o: setattr(c, "width", 0), raster.GS_ERR_INVALID_ARG),
    (lambda c, o: setattr(o, "near_plane", -1.0), raster.GS_ERR_INVALID_ARG),
    (lambda c, o: setattr(o, "sh_rows", 3), raster.GS_ERR_INVALID_ARG),
    (lambda c, o: setattr(o, "lowpass", float("nan")), raster.GS_ERR_INVALID_ARG),
    (lambda c, o: setattr(o, "overwrite_grads", 2), raster.GS_ERR_INVALID_ARG),
])
def test_invalid_arguments_rejected_before_launch(mutate, code):
    """Validation runs on the host and returns before any HIP call."""
    L = raster.load_library()
    cam, opt = _cam(), raster.make_options(3)
    mutate(cam, opt)
    P = C.c_void_p
    dummy = P(4096)  # never dereferenced: validation fails first
    st = L.gs_preprocess(C.byref(cam), C.byref(opt), 10, *([dummy] * 12), None)
    assert st == code
    assert len(L.gs_last_error()) > 0


def test_null_pointers_and_sizes_rejected():
    L = raster.load_library()
    cam, opt = _cam(), raster.make_options(0)
    P = C.c_void_p
    d = P(4096)
    assert L.gs_preprocess(None, C.byref(opt), 1, *([d] * 12), None) == raster.GS_ERR_INVALID_ARG
    assert L.gs_preprocess(C.byref(cam), C.byref(opt), -1, *([d] * 12), None) == raster.GS_ERR_INVALID_ARG
    args = [d] * 12
    args[5] = None  # means2d
    assert L.gs_preprocess(C.byref(cam), C.byref(opt), 5, *args, None) == raster.GS_ERR_INVALID_ARG
    assert b"means2d" in L.gs_last_error()
    misaligned = [d] * 12
    misaligned[2] = P(4100)  # quats not 16-byte aligned
    assert L.gs_preprocess(C.byref(cam), C.byref(opt), 5, *misaligned, None) == raster.GS_ERR_INVALID_ARG
    # bin_sort: workspace too small, capacity out of range
    n_pairs = C.c_int64(0)
    st = L.gs_bin_sort(C.byref(cam), C.byref(opt), 100, d, d, d, d, P(4096 * 256), 16, 1000, None, d, d,
                       C.byref(n_pairs), None)
    assert st == raster.GS_ERR_INVALID_ARG and b"workspace" in L.gs_last_error()
    st = L.gs_bin_sort(C.byref(cam), C.byref(opt), 100, d, d, d, d, P(4096 * 256), 1 << 40, -5, None, d, d,
                       C.byref(n_pairs), None)
    assert st == raster.GS_ERR_INVALID_ARG
    # render_bwd: workspace too small
    st = L.gs_render_bwd(C.byref(cam), C.byref(opt), 100, *([d] * 12), 10, d, d, d, *([d] * 6), P(4096 * 256), 64,
                         None, 0, None, None)
    assert st == raster.GS_ERR_INVALID_ARG and b"workspace" in L.gs_last_error()
    # render checkpoints: too small, or misaligned (on a 1920x1080 camera: 8160 tiles)
    import numpy as np
    cam = raster.make_camera(Camera(1920, 1080, 1400.0, 1400.0, 960.0, 540.0, np.eye(3, dtype=np.float32),
                                    np.zeros(3, np.float32)))
    need = raster.gs_render_ckpt_bytes(cam.width, cam.height)
    assert need == 8160 * (5 * 256 + 1) * 16
    img = [d] * 6
    st = L.gs_render_fwd(C.byref(cam), C.byref(opt), 100, d, d, 10, d, d, d, *img[:3], P(4096 * 256), need - 16, None)
    assert st == raster.GS_ERR_INVALID_ARG and b"ckpt" in L.gs_last_error()
    st = L.gs_render_bwd_raster(C.byref(cam), C.byref(opt), 100, d, d, 10, *([d] * 7), P(4096 * 256 + 8), need, None)
    assert st == raster.GS_ERR_INVALID_ARG and b"ckpt" in L.gs_last_error()


def test_render_ckpt_bytes_by_grid_size():
    # checkpoints only for one-view grids of 4096..32767 tiles
    assert raster.gs_render_ckpt_bytes(128, 128) == 0
    assert raster.gs_render_ckpt_bytes(800, 800) == 0
    assert raster.gs_render_ckpt_bytes(1024, 1024) == 4096 * (5 * 256 + 1) * 16
    assert raster.gs_render_ckpt_bytes(1920, 1080) == 8160 * (5 * 256 + 1) * 16
    assert raster.gs_render_ckpt_bytes(4096, 2048) == 0  # 32768 tiles
    assert raster.gs_render_ckpt_bytes(0, 100) == 0 and raster.gs_render_ckpt_bytes(40000, 100) == 0


def test_workspace_sizes_monotone():
    # super-tile entries (at most one per pair) are sized by the pair capacity
    a = raster.gs_bin_sort_workspace_size(1000, 10_000, 128, 128)
    b = raster.gs_bin_sort_workspace_size(1000, 20_000, 128, 128)
    assert 0 < a < b and a % 256 == 0 and b - a >= 4 * 4 * 10_000
    assert raster.gs_bin_sort_workspace_size(2000, 10_000, 128, 128) > a
    c = raster.gs_bin_sort_workspace_size(1000, 10_000, 2560, 2200)
    assert c > a and c % 256 == 0
    assert raster.gs_render_bwd_workspace_size(1000) >= 1000 * 12 * 4


def test_adam_arguments_rejected_before_launch():
    """Validation runs on the host and returns before any HIP call."""
    L = raster.load_library()
    P5 = C.c_void_p * 5
    d = C.c_void_p(256)
    five = P5(*([d] * 5))
    for step, b1, eps in ((0, 0.9, 1e-15), (1, 1.0, 1e-15), (1, 0.9, -1.0)):
        o = raster.make_adam_options(step, beta1=b1, eps=eps)
        st = L.gs_adam_step(C.byref(o), 4, 16, five, five, five, five, d, d, None, None)
        assert st == raster.GS_ERR_INVALID_ARG, (step, b1, eps)
    o = raster.make_adam_options(1)
    assert L.gs_adam_step(C.byref(o), 4, 0, five, five, five, five, d, d, None, None) == raster.GS_ERR_INVALID_ARG
    assert L.gs_adam_step(C.byref(o), 0, 16, None, None, None, None, None, None, None, None) == raster.GS_OK



def test_views_arguments_rejected_before_launch():
    """The batched calls check the view count, the total size and that every
    camera is valid and of one image size, before any HIP call."""
    L = raster.load_library()
    sc = make_scene(5, 0, n=4)
    opt = raster.make_options(3)
    d = C.c_void_p(4096)
    cams = raster.make_cameras(sc.cameras[:3])

    def pre(cs, V, n=10):
        return L.gs_preprocess_views(cs, V, C.byref(opt), n, *([d] * 12), None, None)

    assert pre(cams, 0) == raster.GS_ERR_INVALID_ARG and b"n_views" in L.gs_last_error()
    big = raster.make_cameras(sc.cameras * 3)  # 48 cameras
    assert pre(big, raster.MAX_VIEWS + 1) == raster.GS_ERR_INVALID_ARG
    assert pre(cams, 3, n=1 << 30) == raster.GS_ERR_INVALID_ARG
    odd = raster.make_cameras(sc.cameras[:3])
    odd[2].width = 1280
    assert pre(odd, 3) == raster.GS_ERR_INVALID_ARG and b"camera 2" in L.gs_last_error()
    bad = raster.make_cameras(sc.cameras[:3])
    bad[1].fy = float("nan")
    assert pre(bad, 3) == raster.GS_ERR_INVALID_ARG and b"camera 1" in L.gs_last_error()
    n_pairs = C.c_int64(0)
    st = L.gs_bin_sort_views(cams, 3, C.byref(opt), 100, d, d, d, d, C.c_void_p(4096 * 256), 16, 1000, None, d, d,
                             C.byref(n_pairs), None)
    assert st == raster.GS_ERR_INVALID_ARG and b"workspace" in L.gs_last_error()
    assert L.gs_preprocess_views(cams, 3, C.byref(opt), 0, *([None] * 12), None, None) == raster.GS_OK


def test_views_workspace_grows_with_views():
    one = raster.gs_bin_sort_views_workspace_size(1, 1000, 10_000, 128, 128)
    assert one == raster.gs_bin_sort_workspace_size(1000, 10_000, 128, 128)
    four = raster.gs_bin_sort_views_workspace_size(4, 1000, 10_000, 128, 128)
    assert four > one and four % 256 == 0
    assert raster.gs_bin_sort_views_workspace_size(0, 1000, 10_000, 128, 128) == 0
    assert raster.gs_bin_sort_views_workspace_size(raster.MAX_VIEWS + 1, 1000, 10_000, 128, 128) == 0


def test_noalloc_backward_rejects_more_than_its_scratch():
    """gs_render_bwd_noalloc refuses n above its fixed scratch before it touches
    any pointer or launches anything."""
    L = raster.load_library()
    cam, opt = _cam(), L.gs_default_options()
    args = [None] * 5 + [None] * 5 + [None, None, 0] + [None] * 3 + [None] * 6 + [None, 0, None, None]
    st = L.gs_render_bwd_noalloc(C.byref(cam), C.byref(opt), raster.NOALLOC_MAX_N + 1, *args)
    assert st == raster.GS_ERR_CAPACITY
    assert b"scratch" in L.gs_last_error()
    assert L.gs_render_bwd_noalloc(C.byref(cam), C.byref(opt), 0, *args) == raster.GS_OK
