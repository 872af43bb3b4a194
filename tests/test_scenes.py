"""Checks of the seeded scene generator (CPU only).

Every parity case and the benchmark draw their inputs from
``differentiable_gaussian_splat_amd.scenes``; these tests tie its output to the
workload statements it follows: the same seed gives the same bytes, the
distributions have the stated parameters (N(a, b) read with b the standard
deviation), the frustum-shaped workloads project inside their images, and the
ring of cameras of the 16-view workload looks at the origin from radius 8.
"""
import hashlib
import math

import numpy as np
import pytest
from scipy import stats

from differentiable_gaussian_splat_amd.scenes import SH_C0, make_scene, ring_cameras

FIELDS = ("means", "log_scales", "scales", "quats", "opacity_logits", "opacities", "sh", "dL_dimage")


def _digest(sc):
    h = hashlib.sha256()
    for f in FIELDS:
        a = getattr(sc, f)
        h.update(f.encode())
        h.update(str(a.dtype).encode() + str(a.shape).encode())
        h.update(np.ascontiguousarray(a).tobytes())
    for c in sc.cameras:
        h.update(c.as_array().tobytes())
    return h.hexdigest()


@pytest.fixture(scope="module")
def scene5():
    return make_scene(5, 0)


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_same_seed_same_bytes(config):
    a, b = make_scene(config, 0), make_scene(config, 0)
    assert _digest(a) == _digest(b)
    c = make_scene(config, 1)
    assert not np.array_equal(a.means, c.means)


def test_same_seed_same_bytes_large_share(scene5):
    assert _digest(make_scene(5, 0)) == _digest(scene5)


def _project(cam, x):
    xc = x.astype(np.float64) @ cam.R.astype(np.float64).T + cam.t.astype(np.float64)
    z = xc[:, 2]
    return cam.fx * xc[:, 0] / z + cam.cx, cam.fy * xc[:, 1] / z + cam.cy, z


def test_ring_cameras_look_at_the_origin():
    """Reading of the 16-view rig: each camera is a proper rotation, sits on the
    circle of radius 8 in the plane y = 0, and maps the origin to the principal
    point at depth 8."""
    cams = ring_cameras()
    assert len(cams) == 16
    centres = []
    for k, cam in enumerate(cams):
        R = cam.R.astype(np.float64)
        np.testing.assert_allclose(R @ R.T, np.eye(3), atol=1e-6)
        assert np.linalg.det(R) == pytest.approx(1.0, abs=1e-6)
        u, v, z = _project(cam, np.zeros((1, 3)))
        assert (u[0], v[0], z[0]) == (pytest.approx(cam.cx, abs=1e-4), pytest.approx(cam.cy, abs=1e-4),
                                      pytest.approx(8.0, abs=1e-5))
        c = np.linalg.solve(R, -cam.t.astype(np.float64))  # camera centre: R c + t = 0
        assert np.linalg.norm(c) == pytest.approx(8.0, abs=1e-5) and abs(c[1]) < 1e-6
        centres.append(c)
        assert (cam.width, cam.height, cam.fx, cam.fy) == (1920, 1080, 1400.0, 1400.0)
    ang = np.unwrap([math.atan2(c[0], -c[2]) for c in centres])
    np.testing.assert_allclose(np.diff(ang), 2 * math.pi / 16, atol=1e-6)


def test_large_share_visible_fraction(scene5):
    """About a fifth of the 6M Gaussians lie in front of each camera and inside
    its image (the workload says about 20%)."""
    fr = []
    for cam in scene5.cameras:
        u, v, z = _project(cam, scene5.means)
        fr.append(np.mean((z > 0.2) & (u >= 0) & (u < cam.width) & (v >= 0) & (v < cam.height)))
    fr = np.array(fr)
    assert 0.12 < fr.min() and fr.max() < 0.35 and 0.17 < fr.mean() < 0.27, fr


def test_tiny_scene_distributions():
    sc = make_scene(1, 0)
    assert sc.n == 1000 and sc.sh.shape == (1000, 1, 3) and sc.sh_degree == 0
    x, y, z = sc.means.T
    assert x.min() >= -1 and x.max() <= 1 and y.min() >= -1 and y.max() <= 1 and z.min() >= 2 and z.max() <= 6
    for a, lo, hi in ((x, -1, 1), (y, -1, 1), (z, 2, 6)):
        assert stats.kstest(a, "uniform", args=(lo, hi - lo)).pvalue > 1e-3
    ls = sc.log_scales.ravel()
    assert abs(ls.mean() + 3.0) < 0.05 and abs(ls.std() - 0.5) < 0.03
    rgb = sc.sh[:, 0, :].astype(np.float64) * SH_C0 + 0.5
    assert rgb.min() >= -1e-6 and rgb.max() <= 1 + 1e-6
    assert stats.kstest(rgb.ravel(), "uniform").pvalue > 1e-3
    assert abs(sc.opacity_logits.mean()) < 0.1 and abs(sc.opacity_logits.std() - 1.0) < 0.06


def _common_sh3(sc, logit_mean, logit_std):
    assert sc.sh.shape[1:] == (16, 3) and sc.sh_degree == 3
    dc = sc.sh[:, 0, :]
    assert dc.min() >= 0 and dc.max() <= 1
    rest = sc.sh[:, 1:, :].astype(np.float64)
    assert abs(rest.mean()) < 0.01 and abs(rest.std() - 0.2) < 0.005
    lg = sc.opacity_logits.astype(np.float64)
    assert abs(lg.mean() - logit_mean) < 0.05 * logit_std + 0.01
    assert abs(lg.std() - logit_std) < 0.03 * logit_std
    np.testing.assert_allclose(sc.opacities, 1.0 / (1.0 + np.exp(-lg)), rtol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(sc.quats.astype(np.float64), axis=1), 1.0, atol=1e-6)
    np.testing.assert_allclose(sc.scales, np.exp(sc.log_scales.astype(np.float64)), rtol=1e-6)
    g = sc.dL_dimage.astype(np.float64).ravel()[:2_000_000]
    assert abs(g.mean()) < 0.005 and abs(g.std() - 1.0) < 0.005


def test_medium_scene_frustum():
    """Reading: volume-uniform in the frustum with z in [2, 10], so z^3 is
    uniform on [8, 1000] and every mean projects inside the 800x800 image."""
    sc = make_scene(2, 0)
    cam = sc.cameras[0]
    u, v, z = _project(cam, sc.means)
    assert z.min() >= 2 - 1e-5 and z.max() <= 10 + 1e-5
    assert u.min() >= -1e-3 and u.max() <= 800 + 1e-3 and v.min() >= -1e-3 and v.max() <= 800 + 1e-3
    assert stats.kstest(z ** 3, "uniform", args=(8.0, 992.0)).pvalue > 1e-3
    assert stats.kstest(u, "uniform", args=(0.0, 800.0)).pvalue > 1e-3
    ls = sc.log_scales.astype(np.float64).ravel()
    assert abs(ls.mean() + 4.0) < 0.01 and abs(ls.std() - 0.7) < 0.01
    _common_sh3(sc, 0.0, 1.5)


def test_contention_scene_clusters_and_large_share():
    """64 isotropic clusters of standard deviation 0.1 with centres at depth
    2..12, and exactly 2% of the Gaussians at log-scale -1 on every axis."""
    sc = make_scene(3, 0)
    ls = sc.log_scales.astype(np.float64)
    big = np.all(ls == -1.0, axis=1)
    assert big.sum() == 20_000
    rest = ls[~big].ravel()
    assert abs(rest.mean() + 4.5) < 0.01 and abs(rest.std() - 0.8) < 0.01
    # cluster structure: the nearest of the 64 densest cells explains each point within a few sigma
    m = sc.means.astype(np.float64)
    from scipy.cluster.vq import kmeans2
    cent, lab = kmeans2(m[::50], 64, seed=1, minit="++", iter=30)
    d = np.linalg.norm(m[::50] - cent[lab], axis=1)
    assert np.median(d) < 0.25  # chi with 3 dof, sigma 0.1: median 0.154
    cam = sc.cameras[0]
    u, v, z = _project(cam, cent)
    assert z.min() > 1.5 and z.max() < 12.5
    _common_sh3(sc, 0.0, 1.5)


def test_worst_atomics_scene():
    sc = make_scene(4, 0)
    cam = sc.cameras[0]
    u, v, z = _project(cam, sc.means)
    assert z.min() >= 3 - 1e-5 and z.max() <= 5 + 1e-5
    assert stats.kstest(z, "uniform", args=(3.0, 2.0)).pvalue > 1e-3
    assert u.min() >= -1e-2 and u.max() <= 1920 + 1e-2 and v.min() >= -1e-2 and v.max() <= 1080 + 1e-2
    ls = sc.log_scales.astype(np.float64).ravel()
    assert abs(ls.mean() + 0.5) < 0.01 and abs(ls.std() - 0.3) < 0.01
    _common_sh3(sc, -2.0, 0.5)


def test_large_share_box_and_clusters(scene5):
    m = scene5.means
    assert m.min() > -10.8 and m.max() < 10.8
    ls = scene5.log_scales.astype(np.float64).ravel()[:3_000_000]
    assert abs(ls.mean() + 4.5) < 0.005 and abs(ls.std() - 0.8) < 0.005
    assert scene5.n == 6_000_000 and len(scene5.cameras) == 16
