"""Densification statistics from the backward against the oracle's, over
three views of a 6M-Gaussian-share scene at reduced size: the oracle runs
each view's backward on the GPU's own forward outputs and accumulates the
screen-mean gradient norms. Counts and radii are exact; the norms come from
pixel sums added by atomics, so they agree to rounding (1e-4 relative L2,
1e-3 per Gaussian above 1% of the largest)."""
import numpy as np
import pytest
import torch

from differentiable_gaussian_splat_amd import raster
from differentiable_gaussian_splat_amd.scenes import make_scene
from oracle import oracle as O
from tests.gpu_helpers import frame_np, params_dev, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("overwrite", [False, True])
def test_densify_stats_over_views(overwrite):
    sc = make_scene(5, 3, n=40_000)
    n = sc.n
    pd = params_dev(sc)
    r = raster.Rasterizer(pd["means"].device)
    acc = torch.zeros(n, dtype=torch.float32, device="cuda")
    cnt = torch.zeros(n, dtype=torch.int32, device="cuda")
    mr = torch.zeros(n, dtype=torch.int32, device="cuda")
    stats = raster.make_densify_stats(acc, cnt, mr)
    o_acc, o_cnt, o_mr = np.zeros(n), np.zeros(n, np.int64), np.zeros(n, np.int64)
    grads = raster.zero_grads(pd["means"], pd["sh"])
    for i, v in enumerate((2, 6, 11)):
        cam = sc.cameras[v]
        fr = r.forward(cam, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], sc.sh_degree)
        r.backward(fr, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], to_dev(sc.dL_dimage[v]),
                   grads, overwrite=overwrite and i == 0, stats=stats)
        torch.cuda.synchronize()
        g = frame_np(fr)
        grad2d = O.render_bwd(cam.width, cam.height, n, g["ranges"], g["values"], g["means2d"], g["conic"],
                              g["opac"], g["rgb"], sc.dL_dimage[v])
        o_acc, o_cnt, o_mr = O.densify_stats(grad2d, g["radii"], o_acc, o_cnt, o_mr)
    np.testing.assert_array_equal(cnt.cpu().numpy(), o_cnt)
    np.testing.assert_array_equal(mr.cpu().numpy(), o_mr)
    assert o_cnt.max() >= 2 and (o_cnt == 0).any()
    a = acc.cpu().numpy().astype(np.float64)
    assert rel_l2(a, o_acc) < 1e-4
    big = o_acc > 1e-2 * o_acc.max()
    np.testing.assert_allclose(a[big], o_acc[big], rtol=1e-3)
    assert np.all(a[o_cnt == 0] == 0.0)
