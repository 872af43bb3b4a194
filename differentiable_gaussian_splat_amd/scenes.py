"""Seeded synthetic scenes for the Gaussian-splatting rasterizer.

This module only draws inputs. It holds none of the rasterizer's arithmetic
(no projection of covariances, no compositing, no sorting), so both the HIP
path and the fp64 oracle can take their inputs from it without sharing any
part of the method.

The five workloads stand in for the datasets the source pages evaluate on
(Mip-NeRF 360, Tanks and Temples, Deep Blending, MatrixCity), which are not
available here: every array is drawn from NumPy's PCG64 with
``seed = 1000 * config + s`` in a fixed order (means, log-scales, quaternion
normals, opacity logits, SH coefficients, upstream image gradient).

Parameters come out both raw (log-scales, opacity logits) and activated
(``scales = exp(log_scales)``, ``opacities = sigmoid(logits)``), both fp32.
The rasterizer consumes the activated values.

Camera convention: world-to-camera ``x_c = R x_w + t`` with ``R`` row-major,
x right, y down, z forward; pixel ``(px, py)`` has its centre at
``(px + 0.5, py + 0.5)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SH_C0 = 0.28209479177387814  # Y_0^0 = 1 / (2 sqrt(pi)); used to encode an RGB as a DC coefficient


@dataclass
class Camera:
    width: int
    height: int
    fx: float
    fy: float
    cx: float
    cy: float
    R: np.ndarray  # (3, 3) float32, world -> camera rotation
    t: np.ndarray  # (3,) float32

    def as_array(self) -> np.ndarray:
        """18 doubles: W, H, fx, fy, cx, cy, R (row-major), t, the last 13 as the
        fp32 values the rasterizer's camera holds (exactly)."""
        v = [self.width, self.height] + [float(np.float32(x)) for x in (self.fx, self.fy, self.cx, self.cy)]
        v += [float(x) for x in np.asarray(self.R, np.float32).reshape(9)]
        v += [float(x) for x in np.asarray(self.t, np.float32).reshape(3)]
        return np.array(v, dtype=np.float64)


@dataclass
class Scene:
    config: int
    seed: int
    means: np.ndarray        # (N, 3) f32
    log_scales: np.ndarray   # (N, 3) f32
    scales: np.ndarray       # (N, 3) f32 = exp(log_scales)
    quats: np.ndarray        # (N, 4) f32, (w, x, y, z), unit length up to rounding
    opacity_logits: np.ndarray  # (N,) f32
    opacities: np.ndarray    # (N,) f32 = sigmoid(logits)
    sh: np.ndarray           # (N, K, 3) f32
    sh_degree: int
    cameras: list = field(default_factory=list)
    dL_dimage: np.ndarray | None = None  # (V, 3, H, W) f32
    name: str = ""

    @property
    def n(self) -> int:
        return int(self.means.shape[0])


CONFIG_NAMES = {
    1: "tiny: 1k Gaussians, SH0, 128x128",
    2: "medium: 100k Gaussians, SH3, 800x800",
    3: "contention: 1M Gaussians, SH3, 1920x1080, 64 clusters + 2% large",
    4: "worst-atomics: 20k large Gaussians, SH3, 1920x1080",
    5: "large-share: 6M Gaussians, SH3, 16 views of 1920x1080",
}


def _identity_camera(w, h, fx, fy, cx, cy) -> Camera:
    return Camera(w, h, float(fx), float(fy), float(cx), float(cy),
                  np.eye(3, dtype=np.float32), np.zeros(3, np.float32))


def ring_cameras(n_views=16, radius=8.0, w=1920, h=1080, f=1400.0) -> list:
    """Cameras on a circle of the given radius in the plane y = 0, each looking
    at the origin. View k: theta = 2 pi k / n, centre radius*(sin, 0, -cos),
    rotation rows (cos, 0, sin), (0, 1, 0), (-sin, 0, cos), t = (0, 0, radius)."""
    cams = []
    for k in range(n_views):
        th = 2.0 * math.pi * k / n_views
        c, s = math.cos(th), math.sin(th)
        R = np.array([[c, 0.0, s], [0.0, 1.0, 0.0], [-s, 0.0, c]], np.float32)
        t = np.array([0.0, 0.0, radius], np.float32)
        cams.append(Camera(w, h, f, f, w / 2.0, h / 2.0, R, t))
    return cams


def _random_quats(rng, n):
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    return q.astype(np.float32)


def _sigmoid32(x):
    x = x.astype(np.float32)
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def _backproject(u, v, z, cam: Camera):
    """Camera-frame point at pixel (u, v) and depth z (identity-pose cameras)."""
    x = (u - cam.cx) * z / cam.fx
    y = (v - cam.cy) * z / cam.fy
    return np.stack([x, y, z], axis=1)


def _sh_coeffs(rng, n, k, dc_uniform=True):
    sh = np.empty((n, k, 3), np.float32)
    sh[:, 0, :] = rng.uniform(0.0, 1.0, (n, 3)) if dc_uniform else 0.0
    if k > 1:
        sh[:, 1:, :] = rng.normal(0.0, 0.2, (n, k - 1, 3))
    return sh


def make_scene(config: int, seed: int = 0, n: int | None = None, with_grad: bool = True) -> Scene:
    """Build config ``config`` (1..5) with sub-seed ``seed``; ``n`` overrides the
    Gaussian count (same distributions) for reduced test sizes."""
    rng = np.random.Generator(np.random.PCG64(1000 * config + seed))
    if config == 1:
        N = 1000 if n is None else n
        cam = _identity_camera(128, 128, 150.0, 150.0, 64.0, 64.0)
        cams = [cam]
        means = np.stack([rng.uniform(-1, 1, N), rng.uniform(-1, 1, N), rng.uniform(2, 6, N)], 1)
        log_s = rng.normal(-3.0, 0.5, (N, 3))
        quats = _random_quats(rng, N)
        logit = rng.normal(0.0, 1.0, N)
        rgb = rng.uniform(0.0, 1.0, (N, 3))
        sh = ((rgb - 0.5) / SH_C0).astype(np.float32).reshape(N, 1, 3)
        deg = 0
    elif config == 2:
        N = 100_000 if n is None else n
        cam = _identity_camera(800, 800, 1100.0, 1100.0, 400.0, 400.0)
        cams = [cam]
        # volume-uniform in the frustum: z^3 uniform on [2^3, 10^3], pixel uniform
        z = np.cbrt(8.0 + rng.uniform(0, 1, N) * 992.0)
        u = rng.uniform(0, cam.width, N)
        v = rng.uniform(0, cam.height, N)
        means = _backproject(u, v, z, cam)
        log_s = rng.normal(-4.0, 0.7, (N, 3))
        quats = _random_quats(rng, N)
        logit = rng.normal(0.0, 1.5, N)
        deg = 3
        sh = _sh_coeffs(rng, N, 16)
    elif config == 3:
        N = 1_000_000 if n is None else n
        cam = _identity_camera(1920, 1080, 1400.0, 1400.0, 960.0, 540.0)
        cams = [cam]
        nc = 64
        cu = rng.uniform(0, cam.width, nc)
        cv = rng.uniform(0, cam.height, nc)
        cz = rng.uniform(2.0, 12.0, nc)
        centres = _backproject(cu, cv, cz, cam)
        assign = rng.integers(0, nc, N)
        means = centres[assign] + rng.normal(0.0, 0.1, (N, 3))
        log_s = rng.normal(-4.5, 0.8, (N, 3))
        big = rng.permutation(N)[: int(round(0.02 * N))]
        log_s[big, :] = -1.0
        quats = _random_quats(rng, N)
        logit = rng.normal(0.0, 1.5, N)
        deg = 3
        sh = _sh_coeffs(rng, N, 16)
    elif config == 4:
        N = 20_000 if n is None else n
        cam = _identity_camera(1920, 1080, 1400.0, 1400.0, 960.0, 540.0)
        cams = [cam]
        z = rng.uniform(3.0, 5.0, N)
        u = rng.uniform(0, cam.width, N)
        v = rng.uniform(0, cam.height, N)
        means = _backproject(u, v, z, cam)
        log_s = rng.normal(-0.5, 0.3, (N, 3))
        quats = _random_quats(rng, N)
        logit = rng.normal(-2.0, 0.5, N)
        deg = 3
        sh = _sh_coeffs(rng, N, 16)
    elif config == 5:
        N = 6_000_000 if n is None else n
        cams = ring_cameras()
        nc = 512
        centres = rng.uniform(-10.0, 10.0, (nc, 3))
        assign = rng.integers(0, nc, N)
        means = centres[assign] + rng.normal(0.0, 0.1, (N, 3))
        log_s = rng.normal(-4.5, 0.8, (N, 3))
        quats = _random_quats(rng, N)
        logit = rng.normal(0.0, 1.5, N)
        deg = 3
        sh = _sh_coeffs(rng, N, 16)
    else:
        raise ValueError(f"unknown config {config}")

    means = means.astype(np.float32)
    log_s = log_s.astype(np.float32)
    logit = logit.astype(np.float32)
    sc = Scene(
        config=config, seed=seed, means=means, log_scales=log_s,
        scales=np.exp(log_s).astype(np.float32), quats=quats,
        opacity_logits=logit, opacities=_sigmoid32(logit),
        sh=np.ascontiguousarray(sh.astype(np.float32)), sh_degree=deg, cameras=cams,
        name=CONFIG_NAMES[config],
    )
    if with_grad:
        c0 = cams[0]
        sc.dL_dimage = rng.standard_normal((len(cams), 3, c0.height, c0.width), dtype=np.float32)
    return sc


def subset(scene: Scene, idx) -> Scene:
    """The same scene restricted to Gaussians ``idx`` (cameras and upstream gradient kept)."""
    idx = np.asarray(idx)
    return Scene(scene.config, scene.seed, scene.means[idx].copy(), scene.log_scales[idx].copy(),
                 scene.scales[idx].copy(), scene.quats[idx].copy(), scene.opacity_logits[idx].copy(),
                 scene.opacities[idx].copy(), scene.sh[idx].copy(), scene.sh_degree,
                 list(scene.cameras), scene.dL_dimage, scene.name)


def surfel_scales(scene: Scene) -> np.ndarray:
    """The 2D Gaussian surfel variant of a workload: the same draws, with a
    surfel's two scales (s_u, s_v) taken from the first two of the Gaussian's
    three (fp32, [N, 2])."""
    return np.ascontiguousarray(scene.scales[:, :2])
