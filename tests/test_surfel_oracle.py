"""Pins of the fp64 surfel oracle (2D Gaussian surfels, steps S1-S10) to facts
outside itself (CPU only): closed forms of a surfel facing the camera, the
ray-plane intersection computed independently (ray parameter from the plane
equation, then coordinates along the surfel's axes), the image of the 3-sigma
disc sampled densely, symmetries of the surfel, and central differences of the
oracle's own forward for the backward."""
import math

import numpy as np
import pytest
from scipy.spatial.transform import Rotation

from differentiable_gaussian_splat_amd.scenes import SH_C0, Camera
from oracle import oracle as O
from tests.test_oracle import cam_of, world_of

A_MAX = float(np.float32(0.99))
A_MIN = float(np.float32(1.0) / np.float32(255.0))


def surfel_params(means, scales, quats, opac, rgb=None, sh=None):
    means = np.atleast_2d(np.asarray(means, np.float64))
    n = means.shape[0]
    if sh is None:
        rgb = np.broadcast_to(np.asarray(rgb, np.float64), (n, 3))
        sh = ((rgb - 0.5) / SH_C0).reshape(n, 1, 3)
    return dict(means=means, scales=np.broadcast_to(np.asarray(scales, np.float64), (n, 2)).copy(),
                quats=np.broadcast_to(np.asarray(quats, np.float64), (n, 4)).copy(),
                opacities=np.broadcast_to(np.asarray(opac, np.float64), (n,)).copy(), sh=np.asarray(sh, np.float64))


def quat_wxyz(R):
    x, y, z, w = Rotation.from_matrix(R).as_quat()
    return np.array([w, x, y, z])


def facing_quat(cam):
    """Quaternion whose axes t_u, t_v, t_w map to the camera's x, y, z: R Rq = I."""
    return quat_wxyz(cam.R.astype(np.float64).T)


@pytest.mark.parametrize("o", [0.05, 0.5, 0.99])
@pytest.mark.parametrize("rotated", [False, True])
def test_facing_surfel_at_pixel_centre(o, rotated):
    """A surfel facing the camera whose centre projects onto a pixel centre
    gives alpha = min(0.99, o) there."""
    rng = np.random.default_rng(3)
    R = Rotation.random(random_state=rng).as_matrix() if rotated else None
    cam = cam_of(64, 48, 90.0, 31.3, 22.7, R, [0.3, -0.2, 0.5] if rotated else None)
    px, py, z = 20, 31, 3.0
    xc = [(px + 0.5 - cam.cx) * z / cam.fx, (py + 0.5 - cam.cy) * z / cam.fy, z]
    rgb = np.array([0.2, 0.7, 0.4])
    p = surfel_params(world_of(cam, xc), [0.05, 0.02], facing_quat(cam), o, rgb)
    f = O.surfel_forward(p, cam, 0)
    a = min(A_MAX, o)
    # (an fp32 camera rotation is orthonormal to ~1e-7: the centre lands within that of the pixel centre)
    np.testing.assert_allclose(f["image"][:, py, px], rgb * a, atol=1e-9)
    assert f["final_T"][py, px] == pytest.approx(1 - a, abs=1e-9)
    assert f["n_contrib"][py, px] == 1


@pytest.mark.parametrize("su,sv", [(0.1, 0.02), (0.004, 0.003)])
def test_facing_surfel_falloff_along_its_axes(su, sv):
    """Identity camera and quaternion: t_u is the camera's x axis, t_v its y
    axis. A pixel dx pixels right of the centre meets the surfel at
    u = dx z / (fx s_u); dy below it at v = dy z / (fy s_v). alpha =
    o exp(-min(u^2 + v^2, 2 (dx^2 + dy^2)) / 2): the surfel's own falloff or the
    screen filter of variance 1/2, whichever is wider."""
    cam = cam_of(96, 96, 120.0, 48.0, 48.0)
    z, o = 2.5, 0.8
    p = surfel_params([[0.5 * z / 120.0, 0.5 * z / 120.0, z]], [su, sv], [1.0, 0, 0, 0], o, [1.0, 1.0, 1.0])
    f = O.surfel_forward(p, cam, 0)
    c = 48 + 0.5  # the centre projects onto pixel (48, 48)'s centre
    for dx, dy in [(1, 0), (3, 0), (0, 1), (0, 2), (2, 1), (-2, -1), (0, 4)]:
        x, y = c + dx, c + dy
        u, v = dx * z / (120.0 * su), dy * z / (120.0 * sv)
        a = min(A_MAX, o * math.exp(-0.5 * min(u * u + v * v, 2.0 * (dx * dx + dy * dy))))
        a = a if a >= A_MIN else 0.0
        got = f["image"][0, int(y), int(x)]
        assert got == pytest.approx(a, abs=1e-12), (dx, dy, got, a)


def _independent_alpha(p, cam, g, x, y):
    """alpha of surfel g at pixel centre (x, y) by intersecting the pixel's ray
    with the surfel's plane directly: lambda from n . (lambda d - X) = 0, then
    the hit point's coordinates along the axes a and b."""
    R, t = cam.R.astype(np.float64), cam.t.astype(np.float64)
    Rq = Rotation.from_quat(np.roll(p["quats"][g] / np.linalg.norm(p["quats"][g]), -1)).as_matrix()
    X = R @ p["means"][g] + t
    a = p["scales"][g, 0] * (R @ Rq[:, 0])
    b = p["scales"][g, 1] * (R @ Rq[:, 1])
    n = np.cross(a, b)
    d = np.array([(x - cam.cx) / cam.fx, (y - cam.cy) / cam.fy, 1.0])
    lam = n @ X / (n @ d)
    hit = lam * d - X  # in the plane spanned by a and b: hit = u a + v b (Gram system; fp32 R is not exactly orthonormal)
    u, v = np.linalg.solve(np.array([[a @ a, a @ b], [a @ b, b @ b]]), np.array([hit @ a, hit @ b]))
    c = np.array([cam.fx * X[0] / X[2] + cam.cx, cam.fy * X[1] / X[2] + cam.cy])
    rho2 = 2.0 * ((x - c[0]) ** 2 + (y - c[1]) ** 2)
    return min(A_MAX, p["opacities"][g] * math.exp(-0.5 * min(u * u + v * v, rho2)))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tilted_surfel_against_direct_ray_plane_intersection(seed):
    """S8's intersection through the two planes h_x, h_y against a direct
    ray-plane intersection, for a tilted surfel under a posed camera."""
    rng = np.random.default_rng(seed)
    R = Rotation.random(random_state=rng).as_matrix()
    cam = cam_of(80, 64, 100.0, 40.3, 31.8, R, rng.normal(0, 0.3, 3))
    z = 2.0
    xc = [(rng.uniform(30, 50) - cam.cx) * z / cam.fx, (rng.uniform(25, 40) - cam.cy) * z / cam.fy, z]
    q = Rotation.random(random_state=rng).as_quat()
    p = surfel_params(world_of(cam, xc), [0.08, 0.03], np.roll(q, 1), 0.9, [1.0, 1.0, 1.0])
    f = O.surfel_forward(p, cam, 0)
    assert f["pre"]["radii"][0] > 0
    checked = 0
    for py in range(cam.height):
        for px in range(cam.width):
            got = f["image"][0, py, px]
            a = _independent_alpha(p, cam, 0, px + 0.5, py + 0.5)
            if got > 0:
                assert got == pytest.approx(a, rel=1e-9, abs=1e-12), (px, py)
                checked += 1
            else:  # outside the tile rectangle, or skipped
                assert a < A_MIN or not _in_rect(f, px, py)
    assert checked > 30


def _in_rect(f, px, py):
    X0, X1, Y0, Y1 = f["pre"]["rect"][0]
    return X0 <= px // 16 <= X1 and Y0 <= py // 16 <= Y1


@pytest.mark.parametrize("seed", range(6))
def test_radius_bounds_the_projected_disc(seed):
    """S5: every point of the 3-sigma disc, projected through the camera
    directly, lies within r of the centre's projection in x and in y, and r is
    tight (within a pixel) unless the screen filter's 3 sigma sets it."""
    rng = np.random.default_rng(100 + seed)
    R = Rotation.random(random_state=rng).as_matrix()
    cam = cam_of(128, 96, 110.0, 64.0, 48.0, R, rng.normal(0, 0.2, 3))
    z = rng.uniform(1.5, 3.0)
    xc = [rng.uniform(-0.3, 0.3) * z, rng.uniform(-0.3, 0.3) * z, z]
    q = Rotation.random(random_state=rng).as_quat()
    s = np.exp(rng.normal(-2.5, 0.6, 2))
    p = surfel_params(world_of(cam, xc), s, np.roll(q, 1), 0.5, [0.5, 0.5, 0.5])
    pre = O.surfel_preprocess(p["means"], p["scales"], p["quats"], p["opacities"], p["sh"], cam, 0)
    r, c = pre["radii"][0], pre["means2d"][0]
    assert r > 0
    Rq = Rotation.from_quat(q).as_matrix()
    th = np.linspace(0, 2 * math.pi, 4000, endpoint=False)
    pts = p["means"][0] + 3 * (np.outer(np.cos(th), s[0] * Rq[:, 0]) + np.outer(np.sin(th), s[1] * Rq[:, 1]))
    X = pts @ cam.R.astype(np.float64).T + cam.t.astype(np.float64)
    sx = cam.fx * X[:, 0] / X[:, 2] + cam.cx
    sy = cam.fy * X[:, 1] / X[:, 2] + cam.cy
    ext = max(np.abs(sx - c[0]).max(), np.abs(sy - c[1]).max())
    assert ext <= r + 1e-9
    assert r == math.ceil(max(ext, 3 * math.sqrt(0.5))) or abs(ext - round(ext)) < 1e-3


def test_swapping_axes_by_a_quarter_turn_leaves_the_image():
    """Turning a surfel a quarter turn about its normal and swapping its two
    scales describes the same surfel: t_u' = t_v, t_v' = -t_u."""
    rng = np.random.default_rng(7)
    R = Rotation.random(random_state=rng).as_matrix()
    cam = cam_of(64, 64, 80.0, 32.0, 32.0, R, [0.1, 0.2, -0.1])
    n = 6
    z = rng.uniform(2, 3, n)
    xc = np.stack([rng.uniform(-0.3, 0.3, n) * z, rng.uniform(-0.3, 0.3, n) * z, z], 1)
    means = np.stack([world_of(cam, x) for x in xc])
    qs = Rotation.random(n, random_state=rng)
    s = np.exp(rng.normal(-2.5, 0.4, (n, 2)))
    sh = rng.normal(0, 0.3, (n, 16, 3))
    p0 = surfel_params(means, s, np.roll(qs.as_quat(), 1, axis=1), rng.uniform(0.3, 0.9, n), sh=sh)
    q1 = qs * Rotation.from_euler("z", 90, degrees=True)
    p1 = dict(p0, quats=np.roll(q1.as_quat(), 1, axis=1), scales=s[:, ::-1].copy())
    f0, f1 = O.surfel_forward(p0, cam, 3), O.surfel_forward(p1, cam, 3)
    np.testing.assert_allclose(f1["image"], f0["image"], atol=1e-12)
    np.testing.assert_array_equal(f1["pre"]["radii"], f0["pre"]["radii"])
    # and swapping the scales without the turn does change it
    p2 = dict(p0, scales=s[:, ::-1].copy())
    assert np.abs(O.surfel_forward(p2, cam, 3)["image"] - f0["image"]).max() > 1e-3


def test_surfel_partition_of_unity_and_invariants():
    rng = np.random.default_rng(5)
    cam = cam_of(48, 40, 60.0, 24.0, 20.0)
    n = 40
    z = rng.uniform(2, 4, n)
    means = np.stack([(rng.uniform(0, 48, n) - 24) * z / 60, (rng.uniform(0, 40, n) - 20) * z / 60, z], 1)
    b = np.array([0.3, 0.6, 0.9])
    p = surfel_params(means, np.exp(rng.normal(-2.3, 0.4, (n, 2))), rng.standard_normal((n, 4)),
                      rng.uniform(0.1, 0.99, n), b)
    f = O.surfel_forward(p, cam, 0, bg=tuple(b))
    np.testing.assert_allclose(f["image"], np.broadcast_to(b[:, None, None], f["image"].shape), atol=1e-12)
    p1 = dict(p, sh=((np.ones((n, 3)) - 0.5) / SH_C0).reshape(n, 1, 3))
    f1 = O.surfel_forward(p1, cam, 0)
    np.testing.assert_allclose(f1["image"][0], 1 - f1["final_T"], atol=1e-12)
    assert f1["final_T"].min() >= float(np.float32(1e-4))
    # quaternion scale does not matter
    f2 = O.surfel_forward(dict(p, quats=p["quats"] * -2.5), cam, 0, bg=tuple(b))
    np.testing.assert_allclose(f2["image"], f["image"], atol=1e-12)


def test_surfel_translation_invariance_degree3():
    rng = np.random.default_rng(9)
    R = Rotation.random(random_state=rng).as_matrix()
    cam = cam_of(48, 40, 60.0, 24.3, 19.8, R, rng.normal(0, 0.3, 3))
    n = 12
    z = rng.uniform(2, 4, n)
    xc = np.stack([(rng.uniform(0, 48, n) - cam.cx) * z / 60, (rng.uniform(0, 40, n) - cam.cy) * z / 60, z], 1)
    p = surfel_params(np.stack([world_of(cam, x) for x in xc]), np.exp(rng.normal(-2.2, 0.4, (n, 2))),
                      rng.standard_normal((n, 4)), rng.uniform(0.2, 0.9, n), sh=rng.normal(0, 0.4, (n, 16, 3)))
    f0 = O.surfel_forward(p, cam, 3)
    t2 = (cam.t.astype(np.float64) + np.array([0.5, -0.25, 0.75])).astype(np.float32)
    delta = np.linalg.solve(cam.R.astype(np.float64), cam.t.astype(np.float64) - t2.astype(np.float64))
    cam2 = Camera(cam.width, cam.height, cam.fx, cam.fy, cam.cx, cam.cy, cam.R, t2)
    f1 = O.surfel_forward(dict(p, means=p["means"] + delta), cam2, 3)
    np.testing.assert_array_equal(f1["values"], f0["values"])
    np.testing.assert_allclose(f1["image"], f0["image"], atol=1e-6)


def test_surfel_culling():
    cam = cam_of(32, 32, 40.0, 16.0, 16.0)
    # centre behind the near plane; 3-sigma disc reaching behind it; non-finite; a small facing surfel
    # (3 sigma = 2.4 px, so the screen filter's 3 sigma of 2.12 px does not set r = 3)
    p = surfel_params([[0, 0, 0.19], [0, 0, 0.5], [0, 0, 2.0], [0, 0, 2.0]], [[0.01, 0.01], [0.2, 0.2],
                                                                              [0.01, np.inf], [0.04, 0.04]],
                      [[1, 0, 0, 0], Rotation.from_euler("x", 60, degrees=True).as_quat()[[3, 0, 1, 2]],
                       [1, 0, 0, 0], [1, 0, 0, 0]], 0.5, [0.5, 0.5, 0.5])
    pre = O.surfel_preprocess(p["means"], p["scales"], p["quats"], p["opacities"], p["sh"], cam, 0)
    np.testing.assert_array_equal(pre["radii"], [0, 0, 0, 3])


# ---------------------------------------------------------------- finite differences

def surfel_fd_scene(seed, n=8, W=40, H=32, deg=3):
    rng = np.random.default_rng(seed)
    R = Rotation.random(random_state=rng).as_matrix()
    cam = cam_of(W, H, 50.0, W / 2 + 0.3, H / 2 - 0.2, R, rng.normal(0, 0.3, 3))
    z = rng.uniform(2.0, 3.5, n)
    xc = np.stack([(rng.uniform(0, W, n) - cam.cx) * z / cam.fx, (rng.uniform(0, H, n) - cam.cy) * z / cam.fy, z], 1)
    means = np.stack([world_of(cam, x) for x in xc])
    K = (deg + 1) ** 2
    sh = rng.normal(0, 0.4, (n, K, 3))
    sh[:, 0, :] = rng.normal(0.2, 1.2, (n, 3))
    p = dict(means=means, scales=np.exp(rng.normal(-1.6, 0.4, (n, 2))), quats=rng.standard_normal((n, 4)),
             opacities=rng.uniform(0.2, 0.95, n), sh=sh)
    p["opacities"][:2] = 0.995
    dL = rng.standard_normal((3, H, W))
    return p, cam, dL


def _surfel_sig(f, p):
    pre = f["pre"]
    W, H = f["image"].shape[2], f["image"].shape[1]
    return (pre["radii"].tobytes(), pre["clamp"].tobytes(), f["values"].tobytes(), f["ranges"].tobytes(),
            O.surfel_decision_hash(W, H, f["ranges"], f["values"], pre["means2d"], pre["tf"], p["opacities"]))


@pytest.mark.parametrize("seed,deg", [(1, 3), (2, 1), (4, 0)])
def test_surfel_backward_matches_central_differences(seed, deg):
    """Every parameter gradient of L = sum(dL * image) against central
    differences of the surfel forward, where x +- h keep every decision."""
    p, cam, dL = surfel_fd_scene(seed, deg=deg)
    K = (deg + 1) ** 2
    p["sh"] = p["sh"][:, :K]
    f = O.surfel_forward(p, cam, deg)
    assert (f["pre"]["radii"] > 0).sum() >= 5
    g = O.surfel_backward(p, cam, deg, f, dL)
    sig0 = _surfel_sig(f, p)
    rng = np.random.default_rng(seed)
    checked = 0
    for key in ("means", "scales", "quats", "opacities", "sh"):
        flat = p[key].reshape(-1)
        for idx in rng.choice(flat.size, min(flat.size, 14), replace=False):
            x0 = flat[idx]
            h = 1e-6 * max(1.0, abs(x0))
            vals = []
            for sgn in (1, -1):
                q = {k: v.copy() for k, v in p.items()}
                q[key].reshape(-1)[idx] = x0 + sgn * h
                fq = O.surfel_forward(q, cam, deg)
                if _surfel_sig(fq, q) != sig0:
                    break
                vals.append(float((dL * fq["image"]).sum()))
            if len(vals) < 2:
                continue
            fd = (vals[0] - vals[1]) / (2 * h)
            an = g[key].reshape(-1)[idx]
            assert an == pytest.approx(fd, rel=2e-5, abs=2e-7 * max(1.0, abs(fd))), (key, idx, an, fd)
            checked += 1
    assert checked >= 40


def test_surfel_render_backward_matches_central_differences():
    """S9 alone: the sums dL/dM (row-major), dL/dc and dL/do against central
    differences of S8 + O12 in M, c and o, on a scene whose screen filter is
    the larger falloff at some pixels and the surfel's own at others."""
    p, cam, dL = surfel_fd_scene(11, n=8, deg=0)
    p["sh"] = p["sh"][:, :1]
    p["scales"][:3] *= 0.05  # small on screen: the filter decides around their centres
    f = O.surfel_forward(p, cam, 0)
    pre = f["pre"]
    W, H = cam.width, cam.height
    N = p["means"].shape[0]
    grad = O.surfel_render_bwd(W, H, N, f["ranges"], f["values"], pre["means2d"], pre["tf"], p["opacities"],
                               pre["rgb"], dL)

    def loss(tf, c, o):
        img, _, _ = O.surfel_render_fwd(W, H, f["ranges"], f["values"], c, tf, o, pre["rgb"])
        return float((dL * img).sum())

    def sig(tf, c, o):
        return O.surfel_decision_hash(W, H, f["ranges"], f["values"], c, tf, o)

    s0 = sig(pre["tf"], pre["means2d"], p["opacities"])
    checked = 0
    for g in range(N):
        if pre["radii"][g] == 0:
            continue
        for which, n_el, off in (("tf", 9, 4), ("c", 2, 13), ("o", 1, 3)):
            for e in range(n_el):
                base = {"tf": pre["tf"].copy(), "c": pre["means2d"].copy(), "o": p["opacities"].copy()}
                arr = base[which].reshape(N, -1)
                x0 = arr[g, e]
                h = 1e-6 * max(1.0, abs(x0))
                vals = []
                for sgn in (1, -1):
                    b2 = {k: v.copy() for k, v in base.items()}
                    b2[which].reshape(N, -1)[g, e] = x0 + sgn * h
                    if sig(b2["tf"], b2["c"], b2["o"]) != s0:
                        break
                    vals.append(loss(b2["tf"], b2["c"], b2["o"]))
                if len(vals) < 2:
                    continue
                fd = (vals[0] - vals[1]) / (2 * h)
                an = grad[g, off + e]
                assert an == pytest.approx(fd, rel=2e-5, abs=1e-8 * max(1.0, abs(fd))), (which, g, e, an, fd)
                checked += 1
    assert checked >= 60
    assert np.abs(grad[:, 13:15]).max() > 0 and np.abs(grad[:, 4:13]).max() > 0
