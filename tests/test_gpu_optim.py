"""The fused optimizer update (gs_adam_step) against the oracle's float64
Adam with the activation chain, step by step from the GPU's own state.

Tolerances come from the float32 arithmetic: a parameter carries its own
rounding (6e-8 relative) and the update lr * m_hat / (sqrt(v_hat) + eps),
whose ratio is computed to ~1e-6 relative; the second moment to ~1e-6
relative; the first moment to ~1e-6 of the largest one (its two terms can
cancel).
Gradients are drawn away from zero so that no moment underflows in float32.
"""
import numpy as np
import pytest
import torch

from differentiable_gaussian_splat_amd import raster
from oracle import oracle as O

pytestmark = pytest.mark.gpu

LR = dict(means=1.6e-4, scales=5e-3, quats=1e-3, opacity=5e-2, sh_dc=2.5e-3, sh_rest=1.25e-4)
# the oracle takes the float32 values the GPU receives, widened exactly
F32 = lambda x: float(np.float32(x))
LR32 = {k: F32(v) for k, v in LR.items()}
B1, B2, EPS = F32(0.9), F32(0.999), F32(1e-15)
LR_OF = dict(means="means", log_scales="scales", quats="quats", opacity_logits="opacity")


def _state(n, rows, seed):
    rng = np.random.default_rng(seed)
    p = dict(means=rng.normal(0, 3, (n, 3)), log_scales=rng.normal(-4.5, 0.8, (n, 3)),
             quats=rng.normal(0, 1, (n, 4)), opacity_logits=rng.normal(0, 1.5, n),
             sh=rng.normal(0, 0.2, (n, rows, 3)))
    return {k: v.astype(np.float32) for k, v in p.items()}, rng


def _grads(rng, n, rows):
    def away(shape, scale):
        x = rng.normal(0, 1, shape)
        return (np.sign(x) * (0.1 + np.abs(x)) * scale).astype(np.float32)
    return dict(means=away((n, 3), 1.0), scales=away((n, 3), 100.0), quats=away((n, 4), 1.0),
                opacities=away(n, 1.0), sh=away((n, rows, 3), 0.3))


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("n,rows", [(50_003, 16), (3_001, 1), (64, 4), (65, 9)])
def test_adam_step_matches_oracle(n, rows):
    p, rng = _state(n, rows, 40 + rows)
    dp = {k: _dev(v) for k, v in p.items()}
    dm = {k: torch.zeros_like(v) for k, v in dp.items()}
    dv = {k: torch.zeros_like(v) for k, v in dp.items()}
    scales = torch.empty((n, 3), dtype=torch.float32, device="cuda")
    opac = torch.empty(n, dtype=torch.float32, device="cuda")
    norm = torch.empty(n, dtype=torch.float32, device="cuda")
    for step in (1, 2, 3):
        g = _grads(rng, n, rows)
        before = {k: v.cpu().numpy() for k, v in dp.items()}
        m0 = {k: v.cpu().numpy() for k, v in dm.items()}
        v0 = {k: v.cpu().numpy() for k, v in dv.items()}
        opt = raster.make_adam_options(step, **{f"lr_{k}": v for k, v in LR.items()}, eps=1e-15)
        raster.gs_adam_step(opt, dp, {k: _dev(v) for k, v in g.items()}, dm, dv, scales, opac, norm)
        torch.cuda.synchronize()
        op, om, ov, osc, oop, onorm = O.adam_step(before, g, m0, v0, step, LR32, beta1=B1, beta2=B2, eps=EPS)
        for k in O.ADAM_GROUPS:
            lr = LR[LR_OF[k]] if k in LR_OF else LR["sh_dc"]
            got = dp[k].cpu().numpy().astype(np.float64)
            np.testing.assert_allclose(got, op[k], rtol=3e-7, atol=1e-5 * lr, err_msg=f"{k} step {step}")
            # b1 m + (1 - b1) g can cancel: its rounding is relative to the terms, not the result
            np.testing.assert_allclose(dm[k].cpu().numpy(), om[k], rtol=2e-6, atol=2e-7 * np.abs(om[k]).max(),
                                       err_msg=f"m {k}")
            np.testing.assert_allclose(dv[k].cpu().numpy(), ov[k], rtol=2e-6, atol=1e-12, err_msg=f"v {k}")
        np.testing.assert_allclose(scales.cpu().numpy(), osc, rtol=1e-6)
        np.testing.assert_allclose(opac.cpu().numpy(), oop, rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(norm.cpu().numpy(), onorm, rtol=1e-5)


def test_adam_step_without_norm_and_empty():
    n, rows = 1000, 16
    p, rng = _state(n, rows, 7)
    dp = {k: _dev(v) for k, v in p.items()}
    dm = {k: torch.zeros_like(v) for k, v in dp.items()}
    dv = {k: torch.zeros_like(v) for k, v in dp.items()}
    scales = torch.empty((n, 3), dtype=torch.float32, device="cuda")
    opac = torch.empty(n, dtype=torch.float32, device="cuda")
    g = _grads(rng, n, rows)
    raster.gs_adam_step(raster.make_adam_options(1), dp, {k: _dev(v) for k, v in g.items()}, dm, dv, scales, opac)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(dp["sh"]))
    e = {k: v[:0] for k, v in dp.items()}
    raster.gs_adam_step(raster.make_adam_options(1), e, {k: v[:0] for k, v in dp.items()} | {"scales": e["log_scales"],
                        "opacities": e["opacity_logits"]}, e, e, scales[:0], opac[:0])


@pytest.mark.parametrize("n,rows", [(20_011, 16), (3_001, 9)])
def test_adam_norm_is_the_same_bit_for_bit(n, rows):
    """The per-Gaussian gradient norm sums the SH gradients in a fixed order
    (segmented wave sums, no float atomics): the same step from the same state
    gives the same norm, bit for bit (float4 records at 16 rows, element-wise
    records at 9)."""
    p, rng = _state(n, rows, 11)
    g = {k: _dev(v) for k, v in _grads(rng, n, rows).items()}
    norms = []
    for _ in range(2):
        dp = {k: _dev(v) for k, v in p.items()}
        dm = {k: torch.zeros_like(v) for k, v in dp.items()}
        dv = {k: torch.zeros_like(v) for k, v in dp.items()}
        scales = torch.empty((n, 3), dtype=torch.float32, device="cuda")
        opac = torch.empty(n, dtype=torch.float32, device="cuda")
        norm = torch.empty(n, dtype=torch.float32, device="cuda")
        raster.gs_adam_step(raster.make_adam_options(1), dp, g, dm, dv, scales, opac, norm)
        torch.cuda.synchronize()
        norms.append(norm.clone())
    assert torch.equal(norms[0], norms[1])
    # and it is the norm: the square root of the sum of the chained squared gradients
    assert torch.all(norms[0] > 0)
