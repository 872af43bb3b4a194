"""ctypes front end of the fp64 CPU oracle (``gs_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. The product path (the HIP library and its binding)
never imports it. It is built with gcc, independently of the HIP library.

Every function takes NumPy arrays; float inputs are widened to float64
exactly before the call, so the oracle sees the same numbers as the GPU.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgs_oracle.so")
_lock = threading.Lock()
_lib = None

TILE = 16


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP for independent pixels/Gaussians)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wno-unused-function",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            L = C.CDLL(_LIB_PATH)
            P = C.c_void_p
            i64, i32, f64 = C.c_int64, C.c_int, C.c_double
            L.orc_preprocess.argtypes = [i64, P, i32, i32, f64, f64] + [P] * 5 + [P] * 10
            L.orc_preprocess.restype = None
            L.orc_bin_sort.argtypes = [i64, i32, i32, P, P, P, i64, P, P, P]
            L.orc_bin_sort.restype = i64
            L.orc_render_fwd.argtypes = [i32, i32] + [P] * 10
            L.orc_render_fwd.restype = None
            L.orc_render_fwd_pixels.argtypes = [i32, i32] + [P] * 7 + [i64, P, P, P, P]
            L.orc_render_fwd_pixels.restype = None
            L.orc_match_fwd.argtypes = [i32, i32] + [P] * 10 + [f64, i32, f64, P]
            L.orc_match_fwd.restype = i64
            L.orc_match_fwd_pixels.argtypes = [i32, i32] + [P] * 7 + [i64, P, P, P] + [f64, i32, f64, P]
            L.orc_match_fwd_pixels.restype = i64
            L.orc_render_bwd.argtypes = [i32, i32, i64] + [P] * 9
            L.orc_render_bwd.restype = None
            L.orc_render_bwd_pixels.argtypes = [i32, i32, i64] + [P] * 8 + [i64, P, P]
            L.orc_render_bwd_pixels.restype = None
            L.orc_preprocess_bwd.argtypes = [i64, P, i32, i32, f64, f64] + [P] * 6 + [P] * 6
            L.orc_preprocess_bwd.restype = None
            L.orc_sh_basis.argtypes = [i32, f64, f64, f64, P]
            L.orc_sh_basis_grad.argtypes = [i32, f64, f64, f64, P]
            L.orc_decision_hash.argtypes = [i32, i32] + [P] * 5
            L.orc_decision_hash.restype = C.c_uint64
            L.orc_surfel_preprocess.argtypes = [i64, P, i32, i32, f64] + [P] * 5 + [P] * 9
            L.orc_surfel_preprocess.restype = None
            L.orc_surfel_render_fwd.argtypes = [i32, i32] + [P] * 10
            L.orc_surfel_render_fwd.restype = None
            L.orc_surfel_match_fwd.argtypes = [i32, i32] + [P] * 10 + [f64, i32, f64, P]
            L.orc_surfel_match_fwd.restype = i64
            L.orc_surfel_render_bwd.argtypes = [i32, i32] + [P] * 9
            L.orc_surfel_render_bwd.restype = None
            L.orc_surfel_decision_hash.argtypes = [i32, i32] + [P] * 5
            L.orc_surfel_decision_hash.restype = C.c_uint64
            L.orc_surfel_preprocess_bwd.argtypes = [i64, P, i32, i32, f64] + [P] * 6 + [P] * 5
            L.orc_surfel_preprocess_bwd.restype = None
            L.orc_set_threads.argtypes = [i32]
            L.orc_max_threads.restype = i32
            _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _d(a, shape=None):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a if shape is None else a.reshape(shape)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def sh_basis(deg, d):
    K = (deg + 1) ** 2
    out = np.zeros(K)
    lib().orc_sh_basis(deg, float(d[0]), float(d[1]), float(d[2]), _p(out))
    return out


def sh_basis_grad(deg, d):
    K = (deg + 1) ** 2
    out = np.zeros((K, 3))
    lib().orc_sh_basis_grad(deg, float(d[0]), float(d[1]), float(d[2]), _p(out))
    return out


def cam_array(cam) -> np.ndarray:
    return cam.as_array() if hasattr(cam, "as_array") else _d(cam)


def preprocess(means, scales, quats, opac, sh, cam, deg, lowpass=0.3, near=0.2):
    """Steps O1-O10 for every Gaussian; returns a dict of float64/int arrays."""
    means, scales, quats, opac = _d(means), _d(scales), _d(quats), _d(opac)
    sh = _d(sh)
    N = means.shape[0]
    rows = sh.shape[1] if sh.ndim == 3 else 1
    out = dict(
        means2d=np.zeros((N, 2)), depth=np.zeros(N), cov2d=np.zeros((N, 3)), conic=np.zeros((N, 3)),
        rgb=np.zeros((N, 3)), radii=np.zeros(N, np.int32), rect=np.zeros((N, 4), np.int64),
        tiles=np.zeros(N, np.int64), clamp=np.zeros((N, 3), np.uint8), margin=np.zeros(N),
    )
    cv = cam_array(cam)
    lib().orc_preprocess(N, _p(cv), deg, rows, float(np.float32(lowpass)), float(np.float32(near)),
                         _p(means), _p(scales), _p(quats), _p(opac), _p(sh),
                         _p(out["means2d"]), _p(out["depth"]), _p(out["cov2d"]), _p(out["conic"]),
                         _p(out["rgb"]), _p(out["radii"]), _p(out["rect"]), _p(out["tiles"]),
                         _p(out["clamp"]), _p(out["margin"]))
    return out


def bin_sort(means2d, radii, depth32, W, H):
    """Step O11: returns (keys u64[P], values u32[P], ranges u32[TX*TY, 2])."""
    means2d = _d(means2d)
    radii = np.ascontiguousarray(radii, dtype=np.int32)
    depth32 = np.ascontiguousarray(depth32, dtype=np.float32)
    N = means2d.shape[0]
    L = lib()
    P = L.orc_bin_sort(N, W, H, _p(means2d), _p(radii), _p(depth32), 0, None, None, None)
    TX, TY = (W + TILE - 1) // TILE, (H + TILE - 1) // TILE
    keys = np.zeros(max(P, 1), np.uint64)
    values = np.zeros(max(P, 1), np.uint32)
    ranges = np.zeros((TX * TY, 2), np.uint32)
    P2 = L.orc_bin_sort(N, W, H, _p(means2d), _p(radii), _p(depth32), P, _p(keys), _p(values), _p(ranges))
    assert P2 == P
    return keys[:P], values[:P], ranges


def render_fwd(W, H, ranges, values, means2d, conic, opac, rgb, bg=(0.0, 0.0, 0.0)):
    """Step O12 over the image: (image[3,H,W], final_T[H,W], n_contrib[H,W])."""
    ranges = np.ascontiguousarray(ranges, np.uint32)
    values = np.ascontiguousarray(values, np.uint32) if len(values) else np.zeros(1, np.uint32)
    image = np.zeros((3, H, W))
    T = np.zeros((H, W))
    nc = np.zeros((H, W), np.uint32)
    lib().orc_render_fwd(W, H, _p(ranges), _p(values), _p(_d(means2d)), _p(_d(conic)), _p(_d(opac)),
                         _p(_d(rgb)), _p(_d(bg)), _p(image), _p(T), _p(nc))
    return image, T, nc


def render_fwd_pixels(W, H, ranges, values, means2d, conic, opac, rgb, pix, bg=(0.0, 0.0, 0.0)):
    """Step O12 at the sampled pixels ``pix`` (flat indices py*W+px)."""
    pix = np.ascontiguousarray(pix, np.int64)
    n = pix.shape[0]
    img = np.zeros((n, 3))
    T = np.zeros(n)
    nc = np.zeros(n, np.uint32)
    values = np.ascontiguousarray(values, np.uint32) if len(values) else np.zeros(1, np.uint32)
    lib().orc_render_fwd_pixels(W, H, _p(np.ascontiguousarray(ranges, np.uint32)), _p(values),
                                _p(_d(means2d)), _p(_d(conic)), _p(_d(opac)), _p(_d(rgb)), _p(_d(bg)),
                                n, _p(pix), _p(img), _p(T), _p(nc))
    return img, T, nc


def match_fwd(W, H, ranges, values, means2d, conic, opac, rgb, gpu_image, gpu_T, gpu_nc,
              bg=(0.0, 0.0, 0.0), d_alpha=4e-6, max_amb=4, tol=1e-5):
    """Decision-aware comparison of an fp32 forward with step O12.

    Returns the per-pixel status (0 natural match, 1 match on another branch of
    a decision within rounding of its threshold, 2 masked, 3 mismatch)."""
    status = np.zeros((H, W), np.int8)
    values = np.ascontiguousarray(values, np.uint32) if len(values) else np.zeros(1, np.uint32)
    lib().orc_match_fwd(W, H, _p(np.ascontiguousarray(ranges, np.uint32)), _p(values), _p(_d(means2d)),
                        _p(_d(conic)), _p(_d(opac)), _p(_d(rgb)), _p(_d(bg)),
                        _p(np.ascontiguousarray(gpu_image, np.float32)),
                        _p(np.ascontiguousarray(gpu_T, np.float32)),
                        _p(np.ascontiguousarray(gpu_nc, np.uint32)), float(d_alpha), int(max_amb),
                        float(tol), _p(status))
    return status


def match_fwd_pixels(W, H, ranges, values, means2d, conic, opac, rgb, pix, gpu_image, gpu_T, gpu_nc,
                     bg=(0.0, 0.0, 0.0), d_alpha=4e-6, max_amb=4, tol=1e-5):
    """:func:`match_fwd` at the sampled pixels ``pix`` (flat py*W+px); the GPU
    image/final_T/n_contrib are the full-frame arrays."""
    pix = np.ascontiguousarray(pix, np.int64)
    n = pix.shape[0]
    HW = W * H
    img = np.asarray(gpu_image, np.float32).reshape(3, HW)
    rgbT = np.ascontiguousarray(np.stack([img[0, pix], img[1, pix], img[2, pix],
                                          np.asarray(gpu_T, np.float32).reshape(HW)[pix]], axis=1), np.float32)
    nc = np.ascontiguousarray(np.asarray(gpu_nc).reshape(HW)[pix], np.uint32)
    status = np.zeros(n, np.int8)
    values = np.ascontiguousarray(values, np.uint32) if len(values) else np.zeros(1, np.uint32)
    lib().orc_match_fwd_pixels(W, H, _p(np.ascontiguousarray(ranges, np.uint32)), _p(values), _p(_d(means2d)),
                               _p(_d(conic)), _p(_d(opac)), _p(_d(rgb)), _p(_d(bg)), n, _p(pix), _p(rgbT), _p(nc),
                               float(d_alpha), int(max_amb), float(tol), _p(status))
    return status


def render_bwd(W, H, N, ranges, values, means2d, conic, opac, rgb, dL_dimage, bg=(0.0, 0.0, 0.0)):
    """Step O13: per-Gaussian sums grad2d[N, 9] = (drgb, dopacity, da, db, dc, du, dv)."""
    grad2d = np.zeros((N, 9))
    values = np.ascontiguousarray(values, np.uint32) if len(values) else np.zeros(1, np.uint32)
    lib().orc_render_bwd(W, H, N, _p(np.ascontiguousarray(ranges, np.uint32)), _p(values), _p(_d(means2d)),
                         _p(_d(conic)), _p(_d(opac)), _p(_d(rgb)), _p(_d(bg)), _p(_d(dL_dimage)),
                         _p(grad2d))
    return grad2d


def render_bwd_pixels(W, H, N, ranges, values, means2d, conic, opac, rgb, dL_dimage, pix, bg=(0.0, 0.0, 0.0)):
    """Step O13 restricted to the sampled pixels ``pix`` (flat indices py*W+px)."""
    grad2d = np.zeros((N, 9))
    pix = np.ascontiguousarray(pix, np.int64)
    values = np.ascontiguousarray(values, np.uint32) if len(values) else np.zeros(1, np.uint32)
    lib().orc_render_bwd_pixels(W, H, N, _p(np.ascontiguousarray(ranges, np.uint32)), _p(values), _p(_d(means2d)),
                                _p(_d(conic)), _p(_d(opac)), _p(_d(rgb)), _p(_d(bg)), _p(_d(dL_dimage)),
                                pix.shape[0], _p(pix), _p(grad2d))
    return grad2d


def preprocess_bwd(means, scales, quats, opac, sh, cam, deg, grad2d, lowpass=0.3, near=0.2):
    """Step O14: parameter gradients from grad2d (fresh zero buffers)."""
    means, scales, quats, opac, sh = _d(means), _d(scales), _d(quats), _d(opac), _d(sh)
    N = means.shape[0]
    rows = sh.shape[1] if sh.ndim == 3 else 1
    g = dict(means=np.zeros((N, 3)), scales=np.zeros((N, 3)), quats=np.zeros((N, 4)),
             opacities=np.zeros(N), sh=np.zeros_like(sh), means2d=np.zeros((N, 2)))
    lib().orc_preprocess_bwd(N, _p(cam_array(cam)), deg, rows, float(np.float32(lowpass)),
                             float(np.float32(near)), _p(means), _p(scales), _p(quats), _p(opac), _p(sh),
                             _p(_d(grad2d)), _p(g["means"]), _p(g["scales"]), _p(g["quats"]),
                             _p(g["opacities"]), _p(g["sh"]), _p(g["means2d"]))
    return g


def decision_hash(W, H, ranges, values, means2d, conic, opac):
    """Hash of every pixel's O12 decisions (blended entries, alpha clamps, stop)."""
    values = np.ascontiguousarray(values, np.uint32) if len(values) else np.zeros(1, np.uint32)
    return int(lib().orc_decision_hash(W, H, _p(np.ascontiguousarray(ranges, np.uint32)), _p(values),
                                       _p(_d(means2d)), _p(_d(conic)), _p(_d(opac))))


def ldl_to_conic(q):
    """Standard conic (a, b, c) of a quadratic form given as q = (a, beta, gamma)
    with Q(d) = a (dx + beta dy)^2 + gamma dy^2, i.e. b = a beta, c = gamma + a beta^2."""
    q = _d(q)
    a, be, ga = q[:, 0], q[:, 1], q[:, 2]
    return np.stack([a, a * be, ga + a * be * be], axis=1)


def forward(params, cam, deg, lowpass=0.3, near=0.2, bg=(0.0, 0.0, 0.0)):
    """O1-O12 end to end from raw parameters. ``params`` has means, scales,
    quats, opacities, sh (NumPy). Returns every intermediate."""
    pre = preprocess(params["means"], params["scales"], params["quats"], params["opacities"], params["sh"],
                     cam, deg, lowpass, near)
    W, H = int(cam.width), int(cam.height)
    depth32 = pre["depth"].astype(np.float32)
    keys, values, ranges = bin_sort(pre["means2d"], pre["radii"], depth32, W, H)
    image, T, nc = render_fwd(W, H, ranges, values, pre["means2d"], pre["conic"], params["opacities"],
                              pre["rgb"], bg)
    return dict(pre=pre, keys=keys, values=values, ranges=ranges, image=image, final_T=T, n_contrib=nc)


def backward(params, cam, deg, fwd, dL_dimage, lowpass=0.3, near=0.2, bg=(0.0, 0.0, 0.0)):
    """O13-O14 end to end, using the intermediates of :func:`forward`."""
    pre = fwd["pre"]
    W, H = int(cam.width), int(cam.height)
    N = pre["means2d"].shape[0]
    grad2d = render_bwd(W, H, N, fwd["ranges"], fwd["values"], pre["means2d"], pre["conic"],
                        params["opacities"], pre["rgb"], dL_dimage, bg)
    g = preprocess_bwd(params["means"], params["scales"], params["quats"], params["opacities"], params["sh"],
                       cam, deg, grad2d, lowpass, near)
    g["grad2d"] = grad2d
    return g


# ---------------------------------------------------------------- phase U: the optimizer update

ADAM_GROUPS = ("means", "log_scales", "quats", "opacity_logits", "sh")


def adam_step(params, grads, exp_avg, exp_avg_sq, step, lr, beta1=0.9, beta2=0.999, eps=1e-15):
    """Step O15 (phase U, the optimizer update the Odin page's Fig. 7 caption
    names, with the Adam optimizer of its referee report, major comment 1), in
    float64, plain NumPy, from the published definition of Adam.

    params, exp_avg, exp_avg_sq: dicts over ADAM_GROUPS of raw parameters and
    moments (means, log-scales, quaternions, opacity logits, SH [N, rows, 3]);
    grads: the rasterizer's gradients keyed means, scales, quats, opacities,
    sh, with respect to the ACTIVATED scales = exp(log_scales) and opacities =
    sigmoid(logits); lr: dict with keys means, scales, quats, opacity, sh_dc,
    sh_rest. Returns (params, exp_avg, exp_avg_sq, scales, opacities,
    grad_norm), all new arrays.

    Steps: chain the activated gradients to the raw ones at the parameters'
    values before the update; per scalar m <- b1 m + (1 - b1) g,
    v <- b2 v + (1 - b2) g^2, p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps);
    grad_norm = L2 norm of each Gaussian's raw gradient."""
    d = {k: np.asarray(params[k], np.float64) for k in ADAM_GROUPS}
    scales_before = np.exp(d["log_scales"])
    sig_before = 1.0 / (1.0 + np.exp(-d["opacity_logits"]))
    raw = {
        "means": np.asarray(grads["means"], np.float64),
        "log_scales": np.asarray(grads["scales"], np.float64) * scales_before,
        "quats": np.asarray(grads["quats"], np.float64),
        "opacity_logits": np.asarray(grads["opacities"], np.float64) * sig_before * (1.0 - sig_before),
        "sh": np.asarray(grads["sh"], np.float64),
    }
    rows = d["sh"].shape[1]
    lr_sh = np.full((1, rows, 1), lr["sh_rest"], np.float64)
    lr_sh[0, 0, 0] = lr["sh_dc"]
    lrs = {"means": lr["means"], "log_scales": lr["scales"], "quats": lr["quats"], "opacity_logits": lr["opacity"],
           "sh": lr_sh}
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    out_p, out_m, out_v = {}, {}, {}
    for k in ADAM_GROUPS:
        g = raw[k]
        m = beta1 * np.asarray(exp_avg[k], np.float64) + (1.0 - beta1) * g
        v = beta2 * np.asarray(exp_avg_sq[k], np.float64) + (1.0 - beta2) * g * g
        out_p[k] = d[k] - lrs[k] * (m / bc1) / (np.sqrt(v / bc2) + eps)
        out_m[k], out_v[k] = m, v
    n = d["means"].shape[0]
    norm2 = np.zeros(n)
    for k in ADAM_GROUPS:
        norm2 += (raw[k].reshape(n, -1) ** 2).sum(axis=1)
    return (out_p, out_m, out_v, np.exp(out_p["log_scales"]), 1.0 / (1.0 + np.exp(-out_p["opacity_logits"])),
            np.sqrt(norm2))


def densify_stats(grad2d, radii, grad_accum, count, max_radius):
    """Densification statistics of one view (the inputs of the densify and
    prune steps whose structural changes the Odin page synchronises): for
    every Gaussian drawn in the view (radius > 0), add the norm of its
    screen-mean gradient (dL/du, dL/dv) -- the last two of the nine pixel
    sums of :func:`render_bwd` -- count the view, and keep the largest radius.
    Returns new arrays."""
    g = np.asarray(grad2d, np.float64)
    drawn = np.asarray(radii) > 0
    acc = np.asarray(grad_accum, np.float64).copy()
    cnt = np.asarray(count, np.int64).copy()
    mr = np.asarray(max_radius, np.int64).copy()
    acc[drawn] += np.sqrt(g[drawn, 7] ** 2 + g[drawn, 8] ** 2)
    cnt[drawn] += 1
    mr[drawn] = np.maximum(mr[drawn], np.asarray(radii)[drawn])
    return acc, cnt, mr


# ---------------------------------------------------------------- 2D Gaussian surfels (S1-S10)

SURFEL_GRAD_N = 15  # drgb[3], dopacity, dM[9] (row-major), dc[2]


def surfel_preprocess(means, scales, quats, opac, sh, cam, deg, near=0.2):
    """Steps S1-S7 for every surfel (scales [N, 2]); returns a dict with means2d
    (the projected centre c), depth, tf (the homography M [N, 9]), rgb, radii,
    rect, tiles, clamp and margin."""
    means, scales, quats, opac, sh = _d(means), _d(scales), _d(quats), _d(opac), _d(sh)
    N = means.shape[0]
    rows = sh.shape[1] if sh.ndim == 3 else 1
    out = dict(means2d=np.zeros((N, 2)), depth=np.zeros(N), tf=np.zeros((N, 9)), rgb=np.zeros((N, 3)),
               radii=np.zeros(N, np.int32), rect=np.zeros((N, 4), np.int64), tiles=np.zeros(N, np.int64),
               clamp=np.zeros((N, 3), np.uint8), margin=np.zeros(N))
    lib().orc_surfel_preprocess(N, _p(cam_array(cam)), deg, rows, float(np.float32(near)), _p(means), _p(scales),
                                _p(quats), _p(opac), _p(sh), _p(out["means2d"]), _p(out["depth"]), _p(out["tf"]),
                                _p(out["rgb"]), _p(out["radii"]), _p(out["rect"]), _p(out["tiles"]),
                                _p(out["clamp"]), _p(out["margin"]))
    return out


def _vals(values):
    return np.ascontiguousarray(values, np.uint32) if len(values) else np.zeros(1, np.uint32)


def surfel_render_fwd(W, H, ranges, values, means2d, tf, opac, rgb, bg=(0.0, 0.0, 0.0)):
    """S8 with O12 over the image: (image[3,H,W], final_T[H,W], n_contrib[H,W])."""
    image, T, nc = np.zeros((3, H, W)), np.zeros((H, W)), np.zeros((H, W), np.uint32)
    lib().orc_surfel_render_fwd(W, H, _p(np.ascontiguousarray(ranges, np.uint32)), _p(_vals(values)),
                                _p(_d(means2d)), _p(_d(tf)), _p(_d(opac)), _p(_d(rgb)), _p(_d(bg)), _p(image),
                                _p(T), _p(nc))
    return image, T, nc


def surfel_match_fwd(W, H, ranges, values, means2d, tf, opac, rgb, gpu_image, gpu_T, gpu_nc,
                     bg=(0.0, 0.0, 0.0), d_alpha=4e-6, max_amb=4, tol=1e-5):
    """:func:`match_fwd` for surfels."""
    status = np.zeros((H, W), np.int8)
    lib().orc_surfel_match_fwd(W, H, _p(np.ascontiguousarray(ranges, np.uint32)), _p(_vals(values)),
                               _p(_d(means2d)), _p(_d(tf)), _p(_d(opac)), _p(_d(rgb)), _p(_d(bg)),
                               _p(np.ascontiguousarray(gpu_image, np.float32)),
                               _p(np.ascontiguousarray(gpu_T, np.float32)),
                               _p(np.ascontiguousarray(gpu_nc, np.uint32)), float(d_alpha), int(max_amb),
                               float(tol), _p(status))
    return status


def surfel_render_bwd(W, H, N, ranges, values, means2d, tf, opac, rgb, dL_dimage, bg=(0.0, 0.0, 0.0)):
    """S9: per-surfel sums [N, 15] = (drgb, dopacity, dM row-major, dc)."""
    grad = np.zeros((N, SURFEL_GRAD_N))
    lib().orc_surfel_render_bwd(W, H, _p(np.ascontiguousarray(ranges, np.uint32)), _p(_vals(values)),
                                _p(_d(means2d)), _p(_d(tf)), _p(_d(opac)), _p(_d(rgb)), _p(_d(bg)),
                                _p(_d(dL_dimage)), _p(grad))
    return grad


def surfel_decision_hash(W, H, ranges, values, means2d, tf, opac):
    return int(lib().orc_surfel_decision_hash(W, H, _p(np.ascontiguousarray(ranges, np.uint32)), _p(_vals(values)),
                                              _p(_d(means2d)), _p(_d(tf)), _p(_d(opac))))


def surfel_preprocess_bwd(means, scales, quats, opac, sh, cam, deg, grad, near=0.2):
    """S10: parameter gradients (scales [N, 2]) from the S9 sums."""
    means, scales, quats, opac, sh = _d(means), _d(scales), _d(quats), _d(opac), _d(sh)
    N = means.shape[0]
    rows = sh.shape[1] if sh.ndim == 3 else 1
    g = dict(means=np.zeros((N, 3)), scales=np.zeros((N, 2)), quats=np.zeros((N, 4)), opacities=np.zeros(N),
             sh=np.zeros_like(sh))
    lib().orc_surfel_preprocess_bwd(N, _p(cam_array(cam)), deg, rows, float(np.float32(near)), _p(means),
                                    _p(scales), _p(quats), _p(opac), _p(sh), _p(_d(grad)), _p(g["means"]),
                                    _p(g["scales"]), _p(g["quats"]), _p(g["opacities"]), _p(g["sh"]))
    return g


def surfel_forward(params, cam, deg, near=0.2, bg=(0.0, 0.0, 0.0)):
    """S1-S8 end to end (binning by O11 on (c, r))."""
    pre = surfel_preprocess(params["means"], params["scales"], params["quats"], params["opacities"], params["sh"],
                            cam, deg, near)
    W, H = int(cam.width), int(cam.height)
    keys, values, ranges = bin_sort(pre["means2d"], pre["radii"], pre["depth"].astype(np.float32), W, H)
    image, T, nc = surfel_render_fwd(W, H, ranges, values, pre["means2d"], pre["tf"], params["opacities"],
                                     pre["rgb"], bg)
    return dict(pre=pre, keys=keys, values=values, ranges=ranges, image=image, final_T=T, n_contrib=nc)


def surfel_backward(params, cam, deg, fwd, dL_dimage, near=0.2, bg=(0.0, 0.0, 0.0)):
    """S9-S10 end to end from :func:`surfel_forward`'s intermediates."""
    pre = fwd["pre"]
    W, H = int(cam.width), int(cam.height)
    N = pre["means2d"].shape[0]
    grad = surfel_render_bwd(W, H, N, fwd["ranges"], fwd["values"], pre["means2d"], pre["tf"],
                             params["opacities"], pre["rgb"], dL_dimage, bg)
    g = surfel_preprocess_bwd(params["means"], params["scales"], params["quats"], params["opacities"],
                              params["sh"], cam, deg, grad, near)
    g["grad"] = grad
    return g
