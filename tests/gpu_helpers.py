"""Shared plumbing for the GPU parity tests: run the HIP path through the C
ABI and hand its stage outputs to the oracle as float64 / uint32 arrays."""
from __future__ import annotations

import numpy as np
import torch

from differentiable_gaussian_splat_amd import raster
from oracle import oracle as O


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def params_np(sc):
    return dict(means=sc.means, scales=sc.scales, quats=sc.quats, opacities=sc.opacities, sh=sc.sh)


def params_dev(sc):
    return {k: to_dev(v) for k, v in params_np(sc).items()}


def gpu_frame(sc, view=0, rasterizer=None, bg=(0.0, 0.0, 0.0), sh_degree=None, want_keys=True, pd=None):
    r = rasterizer or raster.Rasterizer(dev(), want_keys=want_keys)
    pd = pd or params_dev(sc)
    deg = sc.sh_degree if sh_degree is None else sh_degree
    fr = r.forward(sc.cameras[view], pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], deg, bg=bg)
    torch.cuda.synchronize()
    return r, pd, fr


def frame_np(fr):
    """GPU stage outputs as the oracle takes them."""
    co = fr.conic_opacity.cpu().numpy()
    P = fr.n_pairs
    out = dict(
        means2d=fr.means2d.cpu().numpy().astype(np.float64),
        depth32=fr.depths.cpu().numpy(),
        ldl=co[:, :3],
        conic=O.ldl_to_conic(co[:, :3]),
        opac=co[:, 3].astype(np.float64),
        rgb=fr.rgb.cpu().numpy().astype(np.float64),
        radii=fr.radii.cpu().numpy(),
        tiles=fr.tiles_touched.cpu().numpy().view(np.uint32),
        clamped=fr.clamped.cpu().numpy(),
        values=fr.values[:P].cpu().numpy().view(np.uint32).copy(),
        ranges=fr.ranges.cpu().numpy().view(np.uint32).copy(),
        image=fr.image.cpu().numpy(),
        final_T=fr.final_T.cpu().numpy(),
        n_contrib=fr.n_contrib.cpu().numpy().view(np.uint32),
        P=P,
    )
    if fr.keys is not None:
        out["keys"] = fr.keys[:P].cpu().numpy().view(np.uint64).copy()
    return out


def gpu_backward(r, fr, pd, dL, want_means2d=True):
    grads = raster.zero_grads(pd["means"], pd["sh"])
    r.backward(fr, pd["means"], pd["scales"], pd["quats"], pd["opacities"], pd["sh"], to_dev(dL), grads,
               want_means2d=want_means2d)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)
