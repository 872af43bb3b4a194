"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (from the arithmetic; see the oracle's step list):
- tile lists, sorted keys and ranges: bit-exact (integer work on the same inputs);
- image: every pixel within 1e-5 absolute of the oracle run on the GPU's own
  projection and lists, along the oracle's decisions or along the other branch
  of a skip/stop decision that lies within fp32 rounding of its threshold;
- gradients: relative L2 error <= 1e-3 per tensor (summation order differs);
- projection: relative 1e-5 on the screen mean, depth and colour; integer
  outputs exact except where the oracle flags its value within 1e-5 of a cut.
"""
import numpy as np
import pytest
import torch

from differentiable_gaussian_splat_amd import raster
from differentiable_gaussian_splat_amd.scenes import Camera, make_scene, subset
from oracle import oracle as O
from tests.gpu_helpers import (check_preprocess, frame_np, gpu_backward, gpu_frame, params_dev, params_np,
                               rel_l2, to_dev)

pytestmark = pytest.mark.gpu

# (config, seed, n): reduced counts the oracle finishes in seconds, several tiles and ragged tails
CASES = [(1, 0, None), (1, 1, None), (2, 0, 20_000), (3, 0, 40_000), (4, 0, 600), (5, 0, 150_000)]
IDS = [f"c{c}s{s}n{n or 'full'}" for c, s, n in CASES]


def scene(c, s, n):
    sc = make_scene(c, s, n=n)
    return sc


def _view(sc):
    return 3 if sc.config == 5 else 0


@pytest.mark.parametrize("c,s,n", CASES, ids=IDS)
def test_preprocess_parity(c, s, n):
    sc = scene(c, s, n)
    v = _view(sc)
    r, pd, fr = gpu_frame(sc, v)
    check_preprocess(sc, v, frame_np(fr))


@pytest.mark.parametrize("c,s,n", CASES, ids=IDS)
def test_bin_sort_bit_exact(c, s, n):
    sc = scene(c, s, n)
    v = _view(sc)
    r, pd, fr = gpu_frame(sc, v)
    g = frame_np(fr)
    cam = sc.cameras[v]
    keys, values, ranges = O.bin_sort(g["means2d"], g["radii"], g["depth32"], cam.width, cam.height)
    assert g["P"] == len(values)
    np.testing.assert_array_equal(g["values"], values)
    np.testing.assert_array_equal(g["keys"], keys)
    np.testing.assert_array_equal(g["ranges"], ranges)


def test_release_thread_state_then_bin_sort_again():
    """gs_release_thread_state frees the calling thread's pair-count readback buffer and event;
    the next gs_bin_sort on that thread makes them again. Checked on the main thread (twice in a
    row: the second call has nothing to free) and on a second thread that bins, releases and
    bins again: every run gives the same lists."""
    import threading
    sc = scene(2, 0, 20_000)
    ref = frame_np(gpu_frame(sc, 0)[2])
    raster.gs_release_thread_state()
    raster.gs_release_thread_state()
    out = {}

    def worker():
        try:
            out["a"] = frame_np(gpu_frame(sc, 0)[2])
            raster.gs_release_thread_state()
            out["b"] = frame_np(gpu_frame(sc, 0)[2])
            raster.gs_release_thread_state()
        except Exception as e:  # reported below
            out["err"] = e

    t = threading.Thread(target=worker)
    t.start()
    t.join()
    assert "err" not in out, out.get("err")
    again = frame_np(gpu_frame(sc, 0)[2])
    for g in (out["a"], out["b"], again):
        assert g["P"] == ref["P"]
        np.testing.assert_array_equal(g["values"], ref["values"])
        np.testing.assert_array_equal(g["ranges"], ref["ranges"])


@pytest.mark.parametrize("c,s,n", CASES, ids=IDS)
def test_forward_parity(c, s, n):
    sc = scene(c, s, n)
    v = _view(sc)
    r, pd, fr = gpu_frame(sc, v)
    g = frame_np(fr)
    cam = sc.cameras[v]
    st = O.match_fwd(cam.width, cam.height, g["ranges"], g["values"], g["means2d"], g["conic"], g["opac"],
                     g["rgb"], g["image"], g["final_T"], g["n_contrib"])
    n3 = int((st == 3).sum())
    n_other = int((st >= 1).sum())
    assert n3 == 0, f"{n3} pixels match no oracle branch"
    assert n_other <= max(4, 1e-3 * st.size), n_other
    assert g["final_T"].min() >= np.float32(1e-4)


@pytest.mark.parametrize("c,s,n", CASES, ids=IDS)
def test_backward_parity_stagewise(c, s, n):
    """Oracle backward on the GPU's projection and lists vs the GPU backward."""
    sc = scene(c, s, n)
    v = _view(sc)
    r, pd, fr = gpu_frame(sc, v)
    g = frame_np(fr)
    cam = sc.cameras[v]
    dL = sc.dL_dimage[v]
    gg = gpu_backward(r, fr, pd, dL)
    grad2d = O.render_bwd(cam.width, cam.height, sc.n, g["ranges"], g["values"], g["means2d"], g["conic"],
                          g["opac"], g["rgb"], dL)
    og = O.preprocess_bwd(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh, cam, sc.sh_degree, grad2d)
    for k in ("means", "scales", "quats", "opacities", "sh", "means2d"):
        e = rel_l2(gg[k], og[k])
        assert e <= 1e-3, (k, e)


@pytest.mark.parametrize("c,s,n", [(1, 0, None), (1, 2, None), (2, 1, 5000), (4, 1, 300)])
def test_backward_parity_end_to_end(c, s, n):
    sc = scene(c, s, n)
    r, pd, fr = gpu_frame(sc, 0)
    dL = sc.dL_dimage[0]
    gg = gpu_backward(r, fr, pd, dL)
    p = params_np(sc)
    f = O.forward(p, sc.cameras[0], sc.sh_degree)
    og = O.backward(p, sc.cameras[0], sc.sh_degree, f, dL)
    for k in ("means", "scales", "quats", "opacities", "sh", "means2d"):
        e = rel_l2(gg[k], og[k])
        assert e <= 1e-3, (k, e)
    # end-to-end image (oracle from raw inputs): reported bound, not the gated stage-wise check
    img = frame_np(fr)["image"]
    assert np.abs(img - f["image"]).max() < 1e-2


# ---------------------------------------------------------------- edge cases

def _tiny_cam(W, H, rng=None):
    """Intrinsics as fp32 values (the rasterizer's camera holds fp32; the oracle gets the same values)."""
    if rng is None:
        return Camera(W, H, 90.0, 90.0, W / 2, H / 2, np.eye(3, dtype=np.float32), np.zeros(3, np.float32))
    from scipy.spatial.transform import Rotation
    R = Rotation.random(random_state=rng).as_matrix().astype(np.float32)
    f32 = lambda x: float(np.float32(x))
    return Camera(W, H, 90.0, 85.0, f32(W / 2 + 0.3), f32(H / 2 - 0.7), R, rng.normal(0, 0.3, 3).astype(np.float32))


def _scene_for(cam, n, rng, deg=1, big=0):
    z = rng.uniform(1.5, 5, n)
    xc = np.stack([(rng.uniform(-10, cam.width + 10, n) - cam.cx) * z / cam.fx,
                   (rng.uniform(-10, cam.height + 10, n) - cam.cy) * z / cam.fy, z], 1)
    R, t = cam.R.astype(np.float64), cam.t.astype(np.float64)
    means = ((xc - t) @ R).astype(np.float32)
    K = (deg + 1) ** 2
    sc = make_scene(1, 0, n=max(n, 1))
    sc = subset(sc, np.zeros(n, int)) if n else subset(sc, np.zeros(0, int))
    sc.means = means
    sc.scales = np.exp(rng.normal(-3.0, 0.5, (n, 3))).astype(np.float32)
    sc.scales[:big] = 2.0
    sc.quats = rng.standard_normal((n, 4)).astype(np.float32)
    sc.opacities = rng.uniform(0.05, 0.99, n).astype(np.float32)
    sc.sh = rng.normal(0, 0.3, (n, K, 3)).astype(np.float32)
    sc.sh_degree = deg
    sc.cameras = [cam]
    sc.dL_dimage = rng.standard_normal((1, 3, cam.height, cam.width)).astype(np.float32)
    return sc


def _full_check(sc, bg=(0.0, 0.0, 0.0)):
    r, pd, fr = gpu_frame(sc, 0, bg=bg)
    g = frame_np(fr)
    cam = sc.cameras[0]
    keys, values, ranges = O.bin_sort(g["means2d"], g["radii"], g["depth32"], cam.width, cam.height)
    np.testing.assert_array_equal(g["values"], values)
    np.testing.assert_array_equal(g["ranges"], ranges)
    st = O.match_fwd(cam.width, cam.height, g["ranges"], g["values"], g["means2d"], g["conic"], g["opac"], g["rgb"],
                     g["image"], g["final_T"], g["n_contrib"], bg=bg)
    assert int((st == 3).sum()) == 0
    dL = sc.dL_dimage[0]
    gg = gpu_backward(r, fr, pd, dL)
    grad2d = O.render_bwd(cam.width, cam.height, sc.n, g["ranges"], g["values"], g["means2d"], g["conic"], g["opac"],
                          g["rgb"], dL, bg=bg)
    og = O.preprocess_bwd(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh, cam, sc.sh_degree, grad2d)
    for k in ("means", "scales", "quats", "opacities", "sh"):
        assert rel_l2(gg[k], og[k]) <= 1e-3, k
    return g, gg


def test_ragged_image_rotated_camera_and_background():
    rng = np.random.default_rng(3)
    cam = _tiny_cam(100, 70, rng)
    sc = _scene_for(cam, 300, rng, deg=2)
    _full_check(sc, bg=(0.2, 0.5, 0.9))


def test_large_gaussians_cover_every_tile():
    rng = np.random.default_rng(4)
    cam = _tiny_cam(96, 64)
    sc = _scene_for(cam, 200, rng, deg=3, big=3)
    g, _ = _full_check(sc)
    assert g["tiles"][:3].max() == ((96 + 15) // 16) * ((64 + 15) // 16)


def test_empty_and_fully_culled_scenes():
    rng = np.random.default_rng(5)
    cam = _tiny_cam(64, 48)
    for n in (0, 50):
        sc = _scene_for(cam, n, rng)
        if n:
            sc.means[:, 2] = -5.0  # behind the camera
        r, pd, fr = gpu_frame(sc, 0, bg=(0.1, 0.2, 0.3))
        assert fr.n_pairs == 0
        img = fr.image.cpu().numpy()
        for ch, b in enumerate((0.1, 0.2, 0.3)):
            assert np.all(img[ch] == np.float32(b))
        assert np.all(fr.final_T.cpu().numpy() == 1.0)
        assert np.all(fr.n_contrib.cpu().numpy() == 0)
        gg = gpu_backward(r, fr, pd, sc.dL_dimage[0], want_means2d=False)
        for k, v in gg.items():
            assert np.all(v == 0.0), k


def test_non_finite_inputs_are_culled():
    rng = np.random.default_rng(6)
    cam = _tiny_cam(64, 64)
    sc = _scene_for(cam, 100, rng)
    sc.means[0, 0] = np.nan
    sc.scales[1, 2] = np.inf
    sc.quats[2] = 0.0
    sc.opacities[3] = np.nan
    sc.sh[4, 1, 2] = np.inf
    r, pd, fr = gpu_frame(sc, 0)
    radii = fr.radii.cpu().numpy()
    assert np.all(radii[:5] == 0)
    o = O.preprocess(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh, cam, sc.sh_degree)
    assert np.all(o["radii"][:5] == 0)
    _full_check(sc)


def test_capacity_round_trip():
    sc = make_scene(1, 0)
    pd = params_dev(sc)
    cam = raster.make_camera(sc.cameras[0])
    opt = raster.make_options(sc.sh_degree)
    r = raster.Rasterizer(to_dev(np.zeros(1)).device, pair_capacity=10, want_keys=True)
    pre = r.preprocess(cam, opt, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"])
    r._ensure_pairs(10)
    r._ensure_bin_ws(sc.n, cam.width, cam.height)
    ranges = torch.full((64, 2), -7, dtype=torch.int32, device=pd["means"].device)
    with pytest.raises(raster.GsCapacityError) as ei:
        raster.gs_bin_sort(cam, opt, pre["means2d"], pre["depths"], pre["radii"], pre["tiles_touched"], r._bin_ws,
                           10, r._keys, r._values, ranges)
    need = ei.value.needed
    assert need == int(pre["tiles_touched"].sum().item())
    assert torch.all(ranges == -7)  # nothing written on a capacity error
    P, ranges2 = r.bin_sort(cam, opt, pre)
    assert P == need


def test_forward_deterministic_and_backward_spread():
    sc = make_scene(2, 3, n=20_000)
    r, pd, fr1 = gpu_frame(sc, 0)
    a = frame_np(fr1)
    _, _, fr2 = gpu_frame(sc, 0, rasterizer=r, pd=pd)
    b = frame_np(fr2)
    for k in ("image", "final_T", "n_contrib", "values", "ranges"):
        np.testing.assert_array_equal(a[k], b[k])
    g1 = gpu_backward(r, fr2, pd, sc.dL_dimage[0])
    g2 = gpu_backward(r, fr2, pd, sc.dL_dimage[0])
    for k in g1:
        assert rel_l2(g1[k], g2[k]) < 1e-5, k


def test_multi_view_accumulation():
    sc = make_scene(5, 1, n=60_000)
    pd = params_dev(sc)
    r = raster.Rasterizer(pd["means"].device)
    total = raster.zero_grads(pd["means"], pd["sh"])
    singles = []
    for v in (0, 5, 10):
        fr = r.forward(sc.cameras[v], pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], 3)
        dL = to_dev(sc.dL_dimage[v])
        r.backward(fr, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], dL, total)
        one = raster.zero_grads(pd["means"], pd["sh"])
        r.backward(fr, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], dL, one)
        singles.append({k: x.cpu().numpy().astype(np.float64) for k, x in one.items()})
    torch.cuda.synchronize()
    for k in total:
        s = sum(d[k] for d in singles)
        # Equal up to the order of the per-tile float atomics. That order moves
        # the summed pixel moments by ~1e-7 relative, but the chain rule through
        # the conic amplifies it for scales and rotations (up to ~1e-4 here), so
        # the bound is the gradient parity bar; exact accumulation is checked on
        # the deterministic chain-rule step below.
        assert rel_l2(total[k].cpu().numpy(), s) < 1e-3, k


@pytest.mark.parametrize("deg", [3, 1])
def test_chain_rule_accumulates_exactly(deg):
    """Both backward halves add into their outputs. The parameter step run
    twice on the same pixel sums gives exactly twice the first result (no
    atomics in this step).
    Degree 3 with 16 stored rows stages whole SH records; degree 1 stages a
    prefix of each record; 59_993 Gaussians leave a ragged last block."""
    sc = make_scene(5, 1, n=59_993)
    r, pd, fr = gpu_frame(sc, 0, sh_degree=deg)
    n = sc.n
    grad2d = torch.zeros(n * raster.GRAD2D_STRIDE, dtype=torch.float32, device=pd["means"].device)
    raster.gs_render_bwd_raster(fr.cam, fr.opt, n, fr.ranges, fr.values, fr.n_pairs, fr.means2d, fr.conic_opacity,
                                fr.rgb, fr.final_T, fr.n_contrib, to_dev(sc.dL_dimage[0]), grad2d)
    # the raster half adds into grad2d too: two calls give twice one (to atomic-order rounding)
    twice = torch.zeros_like(grad2d)
    for _ in range(2):
        raster.gs_render_bwd_raster(fr.cam, fr.opt, n, fr.ranges, fr.values, fr.n_pairs, fr.means2d,
                                    fr.conic_opacity, fr.rgb, fr.final_T, fr.n_contrib, to_dev(sc.dL_dimage[0]),
                                    twice)
    torch.cuda.synchronize()
    assert rel_l2(twice.cpu().numpy().astype(np.float64), 2.0 * grad2d.cpu().numpy().astype(np.float64)) < 1e-5
    g = raster.zero_grads(pd["means"], pd["sh"])
    g["means2d"] = torch.zeros((n, 2), dtype=torch.float32, device=pd["means"].device)
    outs = [g["means"], g["scales"], g["quats"], g["opacities"], g["sh"], g["means2d"]]
    snap = None
    for _ in range(2):
        raster.gs_preprocess_bwd(fr.cam, fr.opt, pd["means"], pd["scales"], pd["quats"], pd["sh"], fr.conic_opacity,
                                 fr.radii, fr.clamped, grad2d, *outs)
        torch.cuda.synchronize()
        if snap is None:
            snap = {k: v.clone() for k, v in g.items()}
    for k in g:
        assert torch.any(snap[k] != 0), k
        assert torch.equal(g[k], 2 * snap[k]), k
    if deg == 1:
        assert torch.all(g["sh"][:, 4:, :] == 0)
    # overwrite_grads = 1 writes every row: from NaN-filled buffers it gives exactly the
    # one-call result into zeroed buffers (zeros for culled Gaussians and for the
    # stored SH rows beyond the active degree). Degree-3 rows are written by a kernel of
    # their own (rows in registers) that shares the chain rule's source with the adding
    # kernel; the file compiles without contraction, so both round alike.
    ow = raster.GsOptions.from_buffer_copy(fr.opt)
    ow.overwrite_grads = 1
    w = {k: torch.full_like(v, float("nan")) for k, v in g.items()}
    culled = fr.radii <= 0
    first = None
    for _ in range(2):
        raster.gs_preprocess_bwd(fr.cam, ow, pd["means"], pd["scales"], pd["quats"], pd["sh"], fr.conic_opacity,
                                 fr.radii, fr.clamped, grad2d, w["means"], w["scales"], w["quats"], w["opacities"],
                                 w["sh"], w["means2d"])
        torch.cuda.synchronize()
        for k in g:
            assert torch.all(torch.isfinite(w[k])), k
            assert torch.all(w[k][culled] == 0), k
            assert torch.equal(w[k], snap[k]), (k, rel_l2(w[k].cpu().numpy().astype(np.float64),
                                                          snap[k].cpu().numpy().astype(np.float64)))
        if first is None:
            first = {k: v.clone() for k, v in w.items()}
        else:
            for k in g:
                assert torch.equal(w[k], first[k]), k
    if deg == 1:
        assert torch.all(w["sh"][:, 4:, :] == 0)
    assert torch.any(culled)


def test_backward_overwrite_matches_accumulate_into_zeros():
    """The whole backward with overwrite: gradient buffers full of NaN come out
    equal (to atomic-order rounding in the pixel sums) to a backward into
    zeroed buffers, culled Gaussians at exactly zero."""
    sc = make_scene(5, 2, n=40_000)
    r, pd, fr = gpu_frame(sc, 3)
    dL = to_dev(sc.dL_dimage[3])
    acc = raster.zero_grads(pd["means"], pd["sh"])
    r.backward(fr, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], dL, acc, want_means2d=True)
    ow = {k: torch.full_like(v, float("nan")) for k, v in acc.items()}
    r.backward(fr, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], dL, ow, want_means2d=True,
               overwrite=True)
    torch.cuda.synchronize()
    culled = (fr.radii <= 0).cpu().numpy()
    assert culled.any() and (~culled).any()
    for k in acc:
        a, o = acc[k].cpu().numpy().astype(np.float64), ow[k].cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(o)), k
        assert np.all(o[culled] == 0.0), k
        assert rel_l2(o, a) < 1e-5, k


def test_lower_active_sh_degree_than_stored():
    sc = make_scene(2, 2, n=3000)  # 16 rows stored
    sc_deg1 = subset(sc, np.arange(sc.n))
    r, pd, fr = gpu_frame(sc, 0, sh_degree=1)
    g = frame_np(fr)
    o = O.preprocess(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh[:, :4], sc.cameras[0], 1)
    same = (g["radii"] > 0) & (o["radii"] > 0)
    np.testing.assert_array_less(np.abs(g["rgb"] - o["rgb"])[same], 1e-5 * (1 + np.abs(o["rgb"][same])))
    gg = gpu_backward(r, fr, pd, sc.dL_dimage[0])
    assert np.all(gg["sh"][:, 4:, :] == 0.0)
    del sc_deg1


def test_large_tile_grid_two_pass_super_sort():
    """2560x2200 = 22080 tiles in 20x18 = 360 super-tiles: grouping the
    super-tile entries takes two radix passes (9 key bits) instead of one."""
    rng = np.random.default_rng(8)
    cam = Camera(2560, 2200, 1500.0, 1500.0, 1280.0, 1100.0, np.eye(3, dtype=np.float32), np.zeros(3, np.float32))
    sc = _scene_for(cam, 3000, rng, deg=1, big=20)
    sc.scales[:20] = 0.3
    _full_check(sc)


@pytest.mark.parametrize("bg", [(0.0, 0.0, 0.0), (0.2, 0.5, 0.9)])
def test_backward_split_of_deep_tiles(bg):
    """On grids of 4096 tiles or more the backward cuts a deep tile's walk into
    pieces of 256 entries from the forward's checkpoints (a walk past the fifth
    piece ends in a tail shared by two waves by row bands); without
    checkpoints a tile walking 512 entries or more is shared by two waves by
    row bands. 1500 faint Gaussians heaped on the middle of a 1024x1024 frame
    walk about 1400 entries there; a few hundred more are spread thinly
    elsewhere. With a background, each piece's colour behind its start takes
    the T_final bg term."""
    rng = np.random.default_rng(11)
    cam = Camera(1024, 1024, 1000.0, 1000.0, 512.0, 512.0, np.eye(3, dtype=np.float32), np.zeros(3, np.float32))
    n_heap, n_rest = 1500, 400
    sc = _scene_for(cam, n_heap + n_rest, rng, deg=1)
    z = rng.uniform(3.0, 5.0, n_heap)
    uv = rng.normal(512.0, 12.0, (n_heap, 2))
    sc.means[:n_heap] = np.stack([(uv[:, 0] - 512.0) * z / 1000.0, (uv[:, 1] - 512.0) * z / 1000.0, z],
                                 1).astype(np.float32)
    sc.scales[:n_heap] = np.exp(rng.normal(-3.5, 0.2, (n_heap, 3))).astype(np.float32)
    sc.opacities[:n_heap] = rng.uniform(0.01, 0.03, n_heap).astype(np.float32)
    g, _ = _full_check(sc, bg=bg)
    nc = g["n_contrib"].astype(np.int64)
    walks = nc.reshape(64, 16, 64, 16).max(axis=(1, 3))
    # pieces of 256 entries from four checkpoint slots reach entry 1280: tiles walking further
    # take the tail piece that two waves share by row bands (4 tiles here, the deepest at 1471)
    assert (walks > 1280).sum() >= 1 and ((walks > 0) & (walks < 512)).sum() > 100, \
        (walks.max(), (walks > 1280).sum())
    # the deep tiles' walks cut into pieces from the forward's checkpoints, and split by row bands
    # without them (ckpt = NULL): the same pixel sums up to summation order
    r, pd, fr = gpu_frame(sc, 0, bg=bg)
    assert fr.ckpt is not None
    dL = to_dev(sc.dL_dimage[0])
    sums = []
    for ck in (fr.ckpt, None):
        g2 = torch.zeros((sc.n, raster.GRAD2D_STRIDE), dtype=torch.float32, device=dL.device)
        raster.gs_render_bwd_raster(fr.cam, fr.opt, sc.n, fr.ranges, fr.values, fr.n_pairs, fr.means2d,
                                    fr.conic_opacity, fr.rgb, fr.final_T, fr.n_contrib, dL, g2, ck)
        torch.cuda.synchronize()
        sums.append(g2.cpu().numpy().astype(np.float64))
    for c in range(9):
        assert rel_l2(sums[0][:, c], sums[1][:, c]) < 1e-5, (c, rel_l2(sums[0][:, c], sums[1][:, c]))


@pytest.mark.parametrize("direct_max", [0, 8, 64])
def test_adaptive_backward_matches_reduced(direct_max):
    """The measurement kernel that switches per (wave, entry) between the wave
    reduction and direct atomics by the number of blending lanes computes the
    same pixel sums as the reduced backward raster (up to summation order), at
    0 (always reduce), 8 and 64 (always direct) lanes. A 1080p grid, so that the
    forward's checkpoints and the pieces kernel are in play."""
    sc = make_scene(3, 0, n=40_000)
    r, pd, fr = gpu_frame(sc, 0)
    assert fr.ckpt is not None
    n = sc.n
    dL = to_dev(sc.dL_dimage[0])
    red = torch.zeros((n, raster.GRAD2D_STRIDE), dtype=torch.float32, device=pd["means"].device)
    ada = torch.zeros_like(red)
    args = (fr.cam, fr.opt, n, fr.ranges, fr.values, fr.n_pairs, fr.means2d, fr.conic_opacity, fr.rgb, fr.final_T,
            fr.n_contrib, dL)
    raster.gs_render_bwd_raster(*args, red, fr.ckpt)
    raster.gs_mb_render_bwd_adaptive(*args, ada, fr.ckpt, direct_max)
    torch.cuda.synchronize()
    a, b = red.cpu().numpy().astype(np.float64), ada.cpu().numpy().astype(np.float64)
    assert np.count_nonzero(a[:, :9]) > 0
    for c in range(9):
        assert rel_l2(b[:, c], a[:, c]) < 1e-5, (c, rel_l2(b[:, c], a[:, c]))
    assert not b[:, 9:].any()


def test_naive_atomic_backward_matches_reduced():
    """The measurement kernel with per-pixel atomics computes the same pixel
    sums as the wave-reduced backward raster (up to summation order)."""
    sc = make_scene(2, 1, n=20_000)
    r, pd, fr = gpu_frame(sc, 0)
    n = sc.n
    dL = to_dev(sc.dL_dimage[0])
    red = torch.zeros((n, raster.GRAD2D_STRIDE), dtype=torch.float32, device=pd["means"].device)
    naive = torch.zeros_like(red)
    args = (fr.cam, fr.opt, n, fr.ranges, fr.values, fr.n_pairs, fr.means2d, fr.conic_opacity, fr.rgb, fr.final_T,
            fr.n_contrib, dL)
    raster.gs_render_bwd_raster(*args, red)
    hist = torch.zeros(65, dtype=torch.int32, device=red.device)
    raster.gs_mb_render_bwd_naive(*args, naive, hist)
    torch.cuda.synchronize()
    # lanes per (wave, entry) update: at least one, and never more updates than blended pixel-entries
    h = hist.cpu().numpy().astype(np.int64)
    assert h[0] == 0 and h.sum() > 0
    assert (h * np.arange(65)).sum() <= int(fr.n_contrib.sum())
    a, b = red.cpu().numpy().astype(np.float64), naive.cpu().numpy().astype(np.float64)
    assert np.count_nonzero(a[:, :9]) > 0
    for c in range(9):
        assert rel_l2(b[:, c], a[:, c]) < 1e-5, (c, rel_l2(b[:, c], a[:, c]))
    assert not b[:, 9:].any()
