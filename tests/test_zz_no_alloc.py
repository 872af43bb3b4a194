"""The backward that allocates nothing (gs_render_bwd_noalloc) against
gs_render_bwd on the same inputs, through the C ABI: two calls in a row, the
second with fewer Gaussians than the first, so that a record the first call
left in the library's scratch would show in the second's gradients."""
import numpy as np
import pytest
import torch

from differentiable_gaussian_splat_amd import raster
from differentiable_gaussian_splat_amd.scenes import make_scene
from tests.gpu_helpers import gpu_frame, rel_l2, to_dev

pytestmark = pytest.mark.gpu

KEYS = ("means", "scales", "quats", "opacities", "sh", "means2d")


def _zeros(pd):
    g = raster.zero_grads(pd["means"], pd["sh"])
    g["means2d"] = torch.zeros((pd["means"].shape[0], 2), dtype=torch.float32, device=pd["means"].device)
    return g


def _both(sc):
    r, pd, fr = gpu_frame(sc, 0, want_keys=False)
    dL = to_dev(sc.dL_dimage[0])
    ref = _zeros(pd)
    r.backward(fr, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], dL, ref, want_means2d=True)
    out = _zeros(pd)
    raster.gs_render_bwd_noalloc(fr.cam, fr.opt, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"],
                                 fr.means2d, fr.conic_opacity, fr.rgb, fr.radii, fr.clamped, fr.ranges, fr.values,
                                 fr.n_pairs, fr.final_T, fr.n_contrib, dL, out["means"], out["scales"], out["quats"],
                                 out["opacities"], out["sh"], out["means2d"], ckpt=fr.ckpt)
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy().astype(np.float64) for k, v in ref.items()},
            {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()})


def test_noalloc_backward_matches_workspace_backward_twice():
    # first call: a large frame (2500 tiles of 800x800, 60k Gaussians); second: 1000 Gaussians at 128x128
    for sc in (make_scene(2, 0, n=60_000), make_scene(1, 0)):
        print(f"noalloc: config {sc.config}, n={sc.n}", flush=True)
        ref, out = _both(sc)
        for k in KEYS:
            e = rel_l2(out[k], ref[k])
            assert np.isfinite(out[k]).all() and e <= 1e-5, (sc.config, k, e)
