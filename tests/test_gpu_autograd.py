"""The autograd wrapper (raster.rasterize) against the oracle: gradients of a
loss reach the raw parameters through torch's own exp / sigmoid, and two
views rendered through one Rasterizer (which shares its pair buffer across
frames) before one backward get their own lists back."""
import numpy as np
import pytest
import torch

from differentiable_gaussian_splat_amd import raster
from differentiable_gaussian_splat_amd.scenes import make_scene
from oracle import oracle as O
from tests.gpu_helpers import dev, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def _raw(sc):
    leaf = lambda a: to_dev(a).requires_grad_()
    return dict(means=leaf(sc.means), log_scales=leaf(sc.log_scales), quats=leaf(sc.quats),
                logits=leaf(sc.opacity_logits), sh=leaf(sc.sh))


def _oracle_raw_grads(sc, views):
    """Oracle gradients summed over views, chained to log-scales and logits
    (d/dlog s = s d/ds, d/dlogit = o (1 - o) d/do) in fp64."""
    p = dict(means=sc.means, scales=sc.scales, quats=sc.quats, opacities=sc.opacities, sh=sc.sh)
    tot = None
    for v in views:
        f = O.forward(p, sc.cameras[v], sc.sh_degree)
        g = O.backward(p, sc.cameras[v], sc.sh_degree, f, sc.dL_dimage[v])
        tot = g if tot is None else {k: tot[k] + g[k] for k in g}
    s = sc.scales.astype(np.float64)
    o = sc.opacities.astype(np.float64)
    return dict(means=tot["means"], log_scales=tot["scales"] * s, quats=tot["quats"],
                logits=tot["opacities"] * o * (1.0 - o), sh=tot["sh"])


def _render(raw, cam, deg, r=None):
    return raster.rasterize(raw["means"], torch.exp(raw["log_scales"]), raw["quats"], torch.sigmoid(raw["logits"]),
                            raw["sh"], cam, sh_degree=deg, rasterizer=r)


def test_rasterize_backward_reaches_raw_parameters():
    sc = make_scene(2, 3, n=6_000)
    raw = _raw(sc)
    img = _render(raw, sc.cameras[0], sc.sh_degree)
    assert img.shape == (3, sc.cameras[0].height, sc.cameras[0].width)
    (img * to_dev(sc.dL_dimage[0])).sum().backward()
    torch.cuda.synchronize()
    og = _oracle_raw_grads(sc, [0])
    for k, t in raw.items():
        e = rel_l2(t.grad.cpu().numpy().astype(np.float64), og[k])
        assert e <= 1e-3, (k, e)


def test_rasterize_two_views_one_loss():
    sc = make_scene(5, 7, n=30_000)
    raw = _raw(sc)
    r = raster.Rasterizer(dev())
    views = (2, 9)
    imgs = [_render(raw, sc.cameras[v], sc.sh_degree, r) for v in views]
    loss = sum((im * to_dev(sc.dL_dimage[v])).sum() for im, v in zip(imgs, views))
    loss.backward()
    torch.cuda.synchronize()
    og = _oracle_raw_grads(sc, views)
    for k, t in raw.items():
        e = rel_l2(t.grad.cpu().numpy().astype(np.float64), og[k])
        assert e <= 1e-3, (k, e)
