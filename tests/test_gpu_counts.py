"""The blending work counter (gs_mb_render_counts, a measurement entry point)
against the forward's own outputs and against a recount from the oracle's
per-pixel walk (fp64 falloff on the GPU's projection and lists)."""
import numpy as np
import pytest
import torch

from differentiable_gaussian_splat_amd import raster
from differentiable_gaussian_splat_amd.scenes import make_scene
from tests.gpu_helpers import frame_np, gpu_frame

pytestmark = pytest.mark.gpu

A_MAX = float(np.float32(0.99))
A_MIN = float(np.float32(1.0) / np.float32(255.0))
T_MIN = float(np.float32(1e-4))


def recount(W, H, ranges, values, means2d, conic, opac):
    """E_f, E_blend, P_c and the (4x16 column strip, entry) pairs with a blended pixel,
    walking each tile's list front to back in fp64 (the compositing rule as the
    oracle states it)."""
    TX, TY = (W + 15) // 16, (H + 15) // 16
    ys, xs = np.mgrid[0:16, 0:16]
    ef = eb = pc = bx = 0
    for t in range(TX * TY):
        lo, hi = (int(x) for x in ranges[t])
        if lo == hi:
            continue
        g = values[lo:hi].astype(np.int64)
        ty, tx = divmod(t, TX)
        px, py = tx * 16 + xs.ravel(), ty * 16 + ys.ravel()
        active = (px < W) & (py < H)
        dx = (px + 0.5)[:, None] - means2d[g, 0][None, :]
        dy = (py + 0.5)[:, None] - means2d[g, 1][None, :]
        a, b, c = conic[g, 0], conic[g, 1], conic[g, 2]
        Q = a * dx * dx + 2 * b * dx * dy + c * dy * dy
        al = np.minimum(A_MAX, opac[g] * np.exp(-0.5 * Q))
        T = np.ones(256)
        band = xs.ravel() // 4  # the backward's column strips
        for j in range(len(g)):
            if not active.any():
                break
            ef += int(active.sum())
            cand = active & (al[:, j] >= A_MIN)
            Tn = T * (1 - al[:, j])
            stop = cand & (Tn < T_MIN)
            bl = cand & ~stop
            active &= ~stop
            T = np.where(bl, Tn, T)
            eb += int(bl.sum())
            pc += int(bl.any())
            bx += len(np.unique(band[bl]))
    return ef, eb, pc, bx


@pytest.mark.parametrize("config,seed,n", [(1, 0, None), (1, 1, None), (2, 0, 3000)])
def test_counts_against_forward_and_recount(config, seed, n):
    sc = make_scene(config, seed, n=n)
    if config == 2:  # a 256x256 corner of the 800x800 camera keeps the recount quick
        cam = sc.cameras[0]
        cam.width = cam.height = 256
    r, pd, fr = gpu_frame(sc, 0, want_keys=False)
    g = frame_np(fr)
    cam = sc.cameras[0]
    W, H = cam.width, cam.height
    cnt = torch.zeros(8, dtype=torch.int64, device=pd["means"].device)
    raster.gs_mb_render_counts(fr.cam, fr.opt, fr.ranges, fr.values, fr.n_pairs, fr.means2d, fr.conic_opacity,
                               fr.rgb, cnt)
    torch.cuda.synchronize()
    E_f, E_f_eval, E_blend, E_b, P_c, band_exec, walked = (int(x) for x in cnt.cpu().tolist()[:7])
    # the forward's own outputs: same decisions, so exact
    nc = g["n_contrib"].astype(np.int64)
    assert E_b == int(nc.sum())
    TX, TY = (W + 15) // 16, (H + 15) // 16
    ncp = np.zeros((TY * 16, TX * 16), np.int64)
    ncp[:H, :W] = nc
    assert walked == int(ncp.reshape(TY, 16, TX, 16).max(axis=(1, 3)).sum())
    assert E_blend <= E_f_eval <= E_f and E_blend <= E_b and P_c <= g["P"] and band_exec <= 4 * P_c
    assert P_c <= band_exec and E_blend <= 64 * band_exec
    # against the fp64 recount: decisions within rounding of a cut may differ, nothing else
    ef, eb, pc, bx = recount(W, H, g["ranges"], g["values"], g["means2d"], g["conic"], g["opac"])
    print(f"config {config}: E_f {E_f}/{ef} E_blend {E_blend}/{eb} P_c {P_c}/{pc} bands {band_exec}/{bx}")
    for got, ref in ((E_f, ef), (E_blend, eb), (P_c, pc), (band_exec, bx)):
        assert abs(got - ref) <= max(2, 1e-4 * ref), (got, ref)
