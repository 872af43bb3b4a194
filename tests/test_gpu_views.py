"""Several views per launch (the *_views calls) against the single-view calls
and the oracle, on a reduced share of the 16-view 1080p ring scene.

The batched projection, binning and forward run the single-view arithmetic per
view, so each view's slice must equal the single-view result bit for bit (pair
values offset by v n, ranges by the pairs of earlier views, tile ids in the
keys by v times the tiles per view); the oracle checks the batched slices
directly as well. The backward sums each Gaussian's views in registers: its
parameter gradients equal the sum of the single-view gradients up to the
order of summation, and the oracle's summed per-view gradients within the
gradient bar (1e-3 relative L2)."""
import numpy as np
import pytest
import torch

from differentiable_gaussian_splat_amd import raster
from differentiable_gaussian_splat_amd.scenes import make_scene
from oracle import oracle as O
from tests.gpu_helpers import dev, frame_np, gpu_frame, params_dev, rel_l2, to_dev

pytestmark = pytest.mark.gpu

VIEWS = (1, 4, 9, 14)
PRE_FIELDS = ("means2d", "depths", "conic_opacity", "rgb", "radii", "tiles_touched", "clamped")
GRAD_KEYS = ("means", "scales", "quats", "opacities", "sh")


def _views_frame(sc, views, pd, sh_degree=None):
    r = raster.ViewsRasterizer(dev(), want_keys=True)
    deg = sc.sh_degree if sh_degree is None else sh_degree
    fr = r.forward_views([sc.cameras[v] for v in views], pd["means"], pd["scales"], pd["quats"], pd["opacities"],
                         pd["sh"], deg)
    torch.cuda.synchronize()
    return r, fr


def _view_slice(fb, i, n, ntiles, start, P_i):
    """View i of a batched frame in single-view form (values and ranges
    shifted back), as the oracle takes it."""
    co = fb.conic_opacity[i].cpu().numpy()
    rg = fb.ranges.view(-1, ntiles, 2)[i].cpu().numpy().view(np.uint32).astype(np.int64)
    empty = rg[:, 1] == rg[:, 0]
    rg = np.where(empty[:, None], 0, rg - start).astype(np.uint32)
    vals = fb.values[start:start + P_i].cpu().numpy().view(np.uint32).astype(np.int64) - i * n
    return dict(means2d=fb.means2d[i].cpu().numpy().astype(np.float64), conic=O.ldl_to_conic(co[:, :3]),
                opac=co[:, 3].astype(np.float64), rgb=fb.rgb[i].cpu().numpy().astype(np.float64),
                radii=fb.radii[i].cpu().numpy(), depth32=fb.depths[i].cpu().numpy(), ranges=rg,
                values=vals.astype(np.uint32))


def test_views_forward_equals_single_views_and_oracle():
    sc = make_scene(5, 2, n=50_000)
    n, V = sc.n, len(VIEWS)
    pd = params_dev(sc)
    _, fb = _views_frame(sc, VIEWS, pd)
    W, H = fb.width, fb.height
    ntiles = ((W + 15) // 16) * ((H + 15) // 16)
    mask = fb.vis_mask.cpu().numpy().view(np.uint32)
    keys_b = fb.keys[:fb.n_pairs].cpu().numpy().view(np.uint64)
    vals_b = fb.values[:fb.n_pairs].cpu().numpy().view(np.uint32).astype(np.int64)
    rg_b = fb.ranges.view(V, ntiles, 2).cpu().numpy().view(np.uint32).astype(np.int64)
    start = 0
    for i, v in enumerate(VIEWS):
        _, _, fs = gpu_frame(sc, v, pd=pd)
        s = frame_np(fs)
        for name in PRE_FIELDS:
            assert torch.equal(getattr(fb, name)[i], getattr(fs, name)), (v, name)
        np.testing.assert_array_equal((mask >> i) & 1, (s["radii"] > 0).astype(np.uint32))
        P_i = s["P"]
        assert P_i > 0
        rs = s["ranges"].astype(np.int64)
        empty = rs[:, 1] == rs[:, 0]
        np.testing.assert_array_equal(rg_b[i][empty], 0)
        np.testing.assert_array_equal(rg_b[i][~empty], rs[~empty] + start)
        np.testing.assert_array_equal(vals_b[start:start + P_i], s["values"].astype(np.int64) + i * n)
        np.testing.assert_array_equal(keys_b[start:start + P_i], s["keys"] + np.uint64((i * ntiles) << 32))
        assert torch.equal(fb.image[i], fs.image) and torch.equal(fb.final_T[i], fs.final_T)
        assert torch.equal(fb.n_contrib[i], fs.n_contrib)
        if i in (0, V - 1):
            # the oracle on the batched slice itself: binning bit-exact, blending decision-aware to 1e-5
            g = _view_slice(fb, i, n, ntiles, start, P_i)
            keys_o, values_o, ranges_o = O.bin_sort(g["means2d"], g["radii"], g["depth32"], W, H)
            np.testing.assert_array_equal(g["values"], values_o)
            np.testing.assert_array_equal(g["ranges"], ranges_o)
            st = O.match_fwd(W, H, g["ranges"], g["values"], g["means2d"], g["conic"], g["opac"], g["rgb"],
                             fb.image[i].cpu().numpy(), fb.final_T[i].cpu().numpy(),
                             fb.n_contrib[i].cpu().numpy().view(np.uint32))
            assert int((st == 3).sum()) == 0
            assert int((st >= 1).sum()) <= max(4, 1e-3 * st.size)
        start += P_i
    assert fb.n_pairs == start
    # a Gaussian outside every view has an empty scope
    assert (mask == 0).any() and (mask != 0).any()


def _dL(sc, views):
    return to_dev(np.ascontiguousarray(np.stack([sc.dL_dimage[v] for v in views])))


def test_views_backward_against_oracle_and_single_views():
    sc = make_scene(5, 2, n=50_000)
    n, V = sc.n, len(VIEWS)
    pd = params_dev(sc)
    r, fb = _views_frame(sc, VIEWS, pd)
    W, H = fb.width, fb.height
    ntiles = ((W + 15) // 16) * ((H + 15) // 16)
    gb = raster.zero_grads(pd["means"], pd["sh"])
    r.backward_views(fb, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], _dL(sc, VIEWS), gb,
                     want_means2d=True)
    torch.cuda.synchronize()
    gb = {k: x.cpu().numpy().astype(np.float64) for k, x in gb.items()}
    # the oracle, view by view on the batched forward's slices, summed
    osum = {k: 0.0 for k in GRAD_KEYS}
    start = 0
    single = {k: 0.0 for k in GRAD_KEYS}
    for i, v in enumerate(VIEWS):
        rs, _, fs = gpu_frame(sc, v, pd=pd)
        P_i = fs.n_pairs
        g = _view_slice(fb, i, n, ntiles, start, P_i)
        start += P_i
        grad2d = O.render_bwd(W, H, n, g["ranges"], g["values"], g["means2d"], g["conic"], g["opac"], g["rgb"],
                              sc.dL_dimage[v])
        og = O.preprocess_bwd(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh, sc.cameras[v], sc.sh_degree,
                              grad2d)
        for k in GRAD_KEYS:
            osum[k] = osum[k] + og[k]
        assert rel_l2(gb["means2d"][i], og["means2d"]) <= 1e-3, (v, "means2d")
        one = raster.zero_grads(pd["means"], pd["sh"])
        rs.backward(fs, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], to_dev(sc.dL_dimage[v]),
                    one)
        torch.cuda.synchronize()
        for k in GRAD_KEYS:
            single[k] = single[k] + one[k].cpu().numpy().astype(np.float64)
    for k in GRAD_KEYS:
        assert rel_l2(gb[k], osum[k]) <= 1e-3, (k, rel_l2(gb[k], osum[k]))
        # the single-view path on the same views: equal up to atomic and summation order
        assert rel_l2(gb[k], single[k]) <= 1e-3, (k, rel_l2(gb[k], single[k]))


@pytest.mark.parametrize("deg", [3, 1])
def test_views_chain_rule_against_single_view_calls(deg):
    """The parameter step alone, fed the same pixel sums: the batched sum over
    views against V single-view calls accumulating into one buffer (equal up
    to summation order), per-view d(u, v) and the densification statistics
    (counts and radii exact), and overwrite against accumulate into zeros
    (exact). 49_999 Gaussians leave a ragged last block."""
    sc = make_scene(5, 4, n=49_999)
    n, V = sc.n, len(VIEWS)
    pd = params_dev(sc)
    r, fb = _views_frame(sc, VIEWS, pd, sh_degree=deg)
    grad2d = torch.zeros((V, n, raster.GRAD2D_STRIDE), dtype=torch.float32, device=dev())
    opt = fb.opt
    raster.gs_render_bwd_raster_views(fb.cams, opt, n, fb.ranges, fb.values, fb.n_pairs, fb.means2d,
                                      fb.conic_opacity, fb.rgb, fb.final_T, fb.n_contrib, _dL(sc, VIEWS), grad2d)

    def stats():
        t = (torch.zeros(n, dtype=torch.float32, device=dev()), torch.zeros(n, dtype=torch.int32, device=dev()),
             torch.zeros(n, dtype=torch.int32, device=dev()))
        return t, raster.make_densify_stats(*t)

    args = (pd["means"], pd["scales"], pd["quats"], pd["sh"])
    gb = raster.zero_grads(pd["means"], pd["sh"])
    m2b = torch.zeros((V, n, 2), dtype=torch.float32, device=dev())
    tb, sb = stats()
    raster.gs_preprocess_bwd_views(fb.cams, opt, *args, fb.conic_opacity, fb.radii, fb.clamped, grad2d, gb["means"],
                                   gb["scales"], gb["quats"], gb["opacities"], gb["sh"], m2b, sb)
    gs = raster.zero_grads(pd["means"], pd["sh"])
    m2s = torch.zeros((V, n, 2), dtype=torch.float32, device=dev())
    ts, ss = stats()
    for i in range(V):
        raster.gs_preprocess_bwd(fb.cams[i], opt, *args, fb.conic_opacity[i], fb.radii[i], fb.clamped[i], grad2d[i],
                                 gs["means"], gs["scales"], gs["quats"], gs["opacities"], gs["sh"], m2s[i], ss)
    # overwrite into garbage: the same bits as accumulating into zeros
    ow = {k: torch.full_like(x, float("nan")) for k, x in gb.items()}
    m2o = torch.full_like(m2b, float("nan"))
    opt_w = raster.GsOptions.from_buffer_copy(opt)
    opt_w.overwrite_grads = 1
    raster.gs_preprocess_bwd_views(fb.cams, opt_w, *args, fb.conic_opacity, fb.radii, fb.clamped, grad2d,
                                   ow["means"], ow["scales"], ow["quats"], ow["opacities"], ow["sh"], m2o)
    torch.cuda.synchronize()
    for k in GRAD_KEYS:
        a, b = gb[k].cpu().numpy().astype(np.float64), gs[k].cpu().numpy().astype(np.float64)
        assert rel_l2(a, b) <= 1e-6, (k, rel_l2(a, b))
        assert torch.equal(ow[k], gb[k]), k
    assert torch.equal(m2b, m2s)
    assert torch.equal(m2o, m2b)
    assert torch.equal(tb[1], ts[1]) and torch.equal(tb[2], ts[2])
    assert int(tb[1].max()) >= 2
    np.testing.assert_allclose(tb[0].cpu().numpy(), ts[0].cpu().numpy(), rtol=1e-6, atol=0)
    # rows beyond the active degree are written as zeros by the overwrite
    if deg < 3:
        K = (deg + 1) ** 2
        assert torch.count_nonzero(ow["sh"][:, K:]) == 0


def test_views_single_view_batch_and_empty_views():
    """V = 1 through the batched calls equals the single-view call; a camera
    that sees nothing adds an empty view; n = 0 is a no-op."""
    sc = make_scene(5, 5, n=20_000)
    pd = params_dev(sc)
    _, f1 = _views_frame(sc, (7,), pd)
    _, _, fs = gpu_frame(sc, 7, pd=pd)
    for name in PRE_FIELDS:
        assert torch.equal(getattr(f1, name)[0], getattr(fs, name)), name
    assert f1.n_pairs == fs.n_pairs
    assert torch.equal(f1.values[:f1.n_pairs], fs.values[:fs.n_pairs])
    assert torch.equal(f1.image[0], fs.image)
    # a camera looking away from the scene, between two real ones
    away = sc.cameras[3].__class__(**{**sc.cameras[3].__dict__})
    away.t = (np.asarray(away.t, np.float32) + np.array([0, 0, -1e4], np.float32)).astype(np.float32)
    r = raster.ViewsRasterizer(dev(), want_keys=True)
    cams = [sc.cameras[3], away, sc.cameras[11]]
    fv = r.forward_views(cams, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], sc.sh_degree)
    torch.cuda.synchronize()
    assert int(fv.radii[1].max()) == 0
    assert torch.equal(fv.image[1], torch.zeros_like(fv.image[1]))
    assert torch.equal(fv.final_T[1], torch.ones_like(fv.final_T[1]))
    mask = fv.vis_mask.cpu().numpy().view(np.uint32)
    assert not ((mask >> 1) & 1).any()
    _, _, f3 = gpu_frame(sc, 3, pd=pd)
    assert torch.equal(fv.image[0], f3.image)
    g = raster.zero_grads(pd["means"], pd["sh"])
    dL = to_dev(np.ascontiguousarray(np.stack([sc.dL_dimage[3], sc.dL_dimage[0], sc.dL_dimage[11]])))
    r.backward_views(fv, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], dL, g,
                     want_means2d=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["means2d"][1]) == 0
    assert all(torch.isfinite(x).all() for x in g.values())
    # no Gaussians at all
    e = {k: x[:0] for k, x in pd.items()}
    fe = r.forward_views(cams, e["means"], e["scales"], e["quats"], e["opacities"], e["sh"], sc.sh_degree)
    torch.cuda.synchronize()
    assert fe.n_pairs == 0 and torch.equal(fe.image, torch.zeros_like(fe.image))


def test_views_max_batch():
    """GS_MAX_VIEWS views of a small ring (each camera of the 16-view ring
    twice, the second time shifted) in one batch: every view equals its
    single-view render."""
    sc = make_scene(5, 6, n=8_000)
    pd = params_dev(sc)
    cams = []
    for v in range(raster.MAX_VIEWS):
        c = sc.cameras[v % 16].__class__(**{**sc.cameras[v % 16].__dict__})
        c.width, c.height, c.fx, c.fy, c.cx, c.cy = 240, 136, c.fx / 8, c.fy / 8, 120.0 + (v // 16), 68.0
        cams.append(c)
    r = raster.ViewsRasterizer(dev(), want_keys=True)
    fv = r.forward_views(cams, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], sc.sh_degree)
    torch.cuda.synchronize()
    mask = fv.vis_mask.cpu().numpy().view(np.uint32)
    assert ((mask >> 31) & 1).any()
    for v in (0, 17, 31):
        rs = raster.Rasterizer(dev())
        fs = rs.forward(cams[v], pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], sc.sh_degree)
        torch.cuda.synchronize()
        assert torch.equal(fv.image[v], fs.image), v
        assert torch.equal(fv.n_contrib[v], fs.n_contrib), v


def test_views_split_of_deep_tiles():
    """Two 1024x1024 views in one launch (8192 tiles: the backward's layout
    that shares a deep tile between two waves) of 1500 faint Gaussians heaped
    on the middle, whose walks there pass 1000 entries: each view's image
    equals the single-view call's bit for bit, and the summed gradients equal
    the single-view sums and the oracle's within the gradient bar."""
    from differentiable_gaussian_splat_amd.scenes import Camera
    from tests.test_gpu_parity import _scene_for
    rng = np.random.default_rng(12)
    cam0 = Camera(1024, 1024, 1000.0, 1000.0, 512.0, 512.0, np.eye(3, dtype=np.float32), np.zeros(3, np.float32))
    cam1 = Camera(1024, 1024, 1000.0, 1000.0, 500.0, 530.0, np.eye(3, dtype=np.float32),
                  np.array([0.05, -0.03, 0.2], np.float32))
    n_heap, n_rest = 1500, 400
    sc = _scene_for(cam0, n_heap + n_rest, rng, deg=1)
    z = rng.uniform(3.0, 5.0, n_heap)
    uv = rng.normal(512.0, 12.0, (n_heap, 2))
    sc.means[:n_heap] = np.stack([(uv[:, 0] - 512.0) * z / 1000.0, (uv[:, 1] - 512.0) * z / 1000.0, z],
                                 1).astype(np.float32)
    sc.scales[:n_heap] = np.exp(rng.normal(-3.5, 0.2, (n_heap, 3))).astype(np.float32)
    sc.opacities[:n_heap] = rng.uniform(0.01, 0.03, n_heap).astype(np.float32)
    sc.cameras = [cam0, cam1]
    sc.dL_dimage = rng.standard_normal((2, 3, 1024, 1024)).astype(np.float32)
    pd = params_dev(sc)
    r, fb = _views_frame(sc, (0, 1), pd)
    walks = fb.n_contrib.cpu().numpy().view(np.uint32).astype(np.int64).reshape(2, 64, 16, 64, 16).max(axis=(2, 4))
    assert walks.max(axis=(1, 2)).min() >= 768 and ((walks > 0) & (walks < 512)).sum() > 100
    gb = raster.zero_grads(pd["means"], pd["sh"])
    r.backward_views(fb, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], _dL(sc, (0, 1)), gb)
    torch.cuda.synchronize()
    gb = {k: x.cpu().numpy().astype(np.float64) for k, x in gb.items()}
    single = {k: 0.0 for k in GRAD_KEYS}
    osum = {k: 0.0 for k in GRAD_KEYS}
    for v in (0, 1):
        rs, _, fs = gpu_frame(sc, v, pd=pd)
        assert torch.equal(fb.image[v], fs.image)
        one = raster.zero_grads(pd["means"], pd["sh"])
        rs.backward(fs, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], to_dev(sc.dL_dimage[v]),
                    one)
        torch.cuda.synchronize()
        g = frame_np(fs)
        grad2d = O.render_bwd(1024, 1024, sc.n, g["ranges"], g["values"], g["means2d"], g["conic"], g["opac"],
                              g["rgb"], sc.dL_dimage[v])
        og = O.preprocess_bwd(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh, sc.cameras[v], sc.sh_degree,
                              grad2d)
        for k in GRAD_KEYS:
            single[k] = single[k] + one[k].cpu().numpy().astype(np.float64)
            osum[k] = osum[k] + og[k]
    for k in GRAD_KEYS:
        assert rel_l2(gb[k], single[k]) <= 1e-3, (k, rel_l2(gb[k], single[k]))
        assert rel_l2(gb[k], osum[k]) <= 1e-3, (k, rel_l2(gb[k], osum[k]))
