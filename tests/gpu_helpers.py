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


# Bound on the factored conic's relative error: each of a, beta, gamma is one
# fp32 rounding (2^-24 relative) of a double value that agrees with the fp64
# oracle's to about 1e-16 times the condition number (at most about 5e5 in
# the seeded workloads), so 4 ulps leaves room for both.
CONIC_TOL = 4 * 2.0 ** -24


def check_preprocess(sc, v, g, idx=None):
    """Projection of view v: GPU stage outputs ``g`` (frame_np) against the
    oracle, for all Gaussians or the subset ``idx``: continuous outputs within
    1e-5 relative, integer outputs exact except where the oracle flags its
    value within 1e-5 of a cut (and rare)."""
    cam = sc.cameras[v]
    if idx is None:
        idx = np.arange(sc.n)
    o = O.preprocess(sc.means[idx], sc.scales[idx], sc.quats[idx], sc.opacities[idx], sc.sh[idx], cam,
                     sc.sh_degree)
    g = {k: (val[idx] if isinstance(val, np.ndarray) and val.shape[:1] == (sc.n,) else val) for k, val in g.items()}
    amb = o["margin"] < 1e-5
    vis_g, vis_o = g["radii"] > 0, o["radii"] > 0
    assert np.all((vis_g == vis_o) | amb)
    assert vis_o.sum() > 0
    same = vis_g & vis_o
    assert np.all((g["radii"] == o["radii"])[same & ~amb])
    assert np.all((g["tiles"] == o["tiles"])[same & ~amb])
    # integer disagreements only ever at flagged Gaussians, and rare
    n_int = (((g["radii"] != o["radii"]) | (g["tiles"] != o["tiles"])) & (vis_g | vis_o)).sum()
    assert n_int <= max(2, 1e-3 * vis_o.sum()), n_int
    sc_uv = np.abs(g["means2d"] - np.array([cam.cx, cam.cy])) + np.array([cam.cx, cam.cy]) + 1.0
    np.testing.assert_array_less(np.abs(g["means2d"] - o["means2d"])[same], 1e-5 * sc_uv[same])
    np.testing.assert_array_less(np.abs(g["depth32"] - o["depth"])[same], 1e-5 * o["depth"][same])
    np.testing.assert_array_less(np.abs(g["rgb"] - o["rgb"])[same], 1e-5 * (1 + np.abs(o["rgb"][same])))
    # conic in factored form against the oracle's 2D covariance (a = C/det, beta = -B/C, gamma = 1/C).
    # The HIP projection forms Sigma' and its inverse in double and rounds each output once, so
    # the bound is flat: a few fp32 roundings, whatever the conditioning. The condition numbers
    # are printed for the record: kappa = A C / det (of the inverse) and kappa_C, that of C
    # itself, which sums the squares of the second projected row V1 Rq diag(s) and cancels
    # when that row is nearly orthogonal to the Gaussian's long axes.
    A, B, Cc = o["cov2d"][same].T
    det = A * Cc - B * B
    a_o, be_o, ga_o = Cc / det, -B / Cc, 1.0 / Cc
    kappa = A * Cc / det
    R = np.asarray(cam.R, np.float64)
    xc = sc.means[idx].astype(np.float64) @ R.T + np.asarray(cam.t, np.float64)
    zc, yc = xc[:, 2], xc[:, 1]
    v1sq = (cam.fy / zc) ** 2 * (1.0 + (yc / zc) ** 2)
    ssq = (sc.scales[idx].astype(np.float64) ** 2).sum(1)
    kC = (v1sq * ssq)[same] / Cc
    ldl = g["ldl"][same].astype(np.float64)
    err_a = np.abs(ldl[:, 0] - a_o) / a_o
    err_g = np.abs(ldl[:, 2] - ga_o) / ga_o
    err_b = np.abs(ldl[:, 1] - be_o) / np.sqrt(A / Cc)
    print(f"conic: {same.sum()} Gaussians, max kappa {kappa.max():.3g}, max kappa_C {kC.max():.3g}, "
          f"max rel err a {err_a.max():.2e} beta {err_b.max():.2e} gamma {err_g.max():.2e}")
    tol = CONIC_TOL
    assert err_a.max() <= tol and err_g.max() <= tol and err_b.max() <= tol, \
        (err_a.max(), err_g.max(), err_b.max(), kappa.max(), kC.max())
    np.testing.assert_array_equal(g["clamped"][same], (o["clamp"][same] * [1, 2, 4]).sum(1))
