#!/usr/bin/env python3
"""Benchmark: forward + backward splat rasterization, ms per frame, on one MI355X.

A step is one pass of the whole hot path on one synthetic frame whose inputs
are already resident in HBM: gs_preprocess -> gs_bin_sort -> gs_render_fwd ->
(zero the per-view pixel sums) -> gs_render_bwd (its two halves,
gs_render_bwd_raster and gs_preprocess_bwd, called in turn so that the
raster kernel can be timed on its own; the step's first view writes the
parameter gradients, later views add into them). Default workload: the
contention-heavy scene (1,000,000 Gaussians, SH degree 3, 1920x1080, 64
clusters plus 2% large Gaussians). The step time comes from the host clock
between two device synchronisations; inside the timed steps HIP events are
recorded on the launch stream only around the backward raster kernel (an
event record costs the stream a few microseconds). The per-stage breakdown
comes from extra steps, outside the timed region, with events around every
call.

The fp64 CPU oracle is timed on a bounded sample of the same frame on the
host cores (cpu_baseline): a reported baseline, not a target.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd splat-raster ms/frame, 1M Gaussians @1080p; % HBM/atomic roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
# Published fp32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz x 2 (dual-issue
# packed fp32) x 2 (an FMA is two flops) = 157.3 TFLOP/s. This build compiles packed
# fp32 off, so an all-FMA stream reaches at most half of it.
FP32_PEAK_TFLOPS = 256 * 4 * 16 * 2.4e9 * 2 * 2 / 1e12
# Flops of the blending arithmetic, an FMA counted as two, exp2 and reciprocal as
# one each, comparisons and selects not at all (the kernels' own formulation):
# - evaluating alpha at a (pixel, entry): w and dy from the record's values at the
#   tile's first pixel (4), the exponent a2 w^2 + g2 dy^2 + log2 o (6), exp2 (1);
ALPHA_FLOPS = 11
# - forward, per blended entry: alpha T (1), three colour FMAs (6), T update (2);
FWD_BLEND_FLOPS = 9
# - backward, per blended entry: T in front of it (1 - alpha, rcp, mul: 3), alpha T (1),
#   colour gradient (6), rgb . dL/dC (5), its difference with S (1), S update (2),
#   h (1), h w and h dy (2), the six moment sums (9).
BWD_GRAD_FLOPS = 30
ATOMICS_PER_TILE_ENTRY = 9      # one add per gradient value per (tile, Gaussian)
PROFILES = os.path.join(ROOT, "profiles")
STAGES = ["preprocess", "bin_sort", "render_fwd", "zero_pixel_sums", "render_bwd_raster", "preprocess_bwd"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload (1..5); 3 is the headline frame")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-baseline", type=int, default=1, help="1: time the oracle on a sample")
    ap.add_argument("--cpu-tile-frac", type=float, default=0.005, help="fraction of tiles the oracle renders")
    ap.add_argument("--cpu-sort-frac", type=float, default=0.1, help="fraction of Gaussians the oracle bins")
    return ap.parse_args()


def stage_rooflines(n, rows, pairs, ntiles, pixels, walked, bwd_bytes, stage_ms, views):
    """Each stage's algorithmic HBM bytes per frame (the least any design
    moves), its floor at the published 8 TB/s and its fraction of that floor;
    the whole frame's floor is their sum. The two blending stages are VALU
    bound (their fraction here is of the HBM floor only); both count a 40-byte
    record per walked (tile, entry), the walk of each tile's deepest pixel."""
    par = 4 * (11 + 3 * rows)  # one Gaussian's parameters (or their gradients)
    P = float(np.mean(pairs))
    by = {
        "preprocess": n * (par + 49),                        # parameters in, projection out
        "bin_sort": n * 20 + P * 4 + ntiles * 8,             # projection in, values and ranges out
        "render_fwd": walked * 40 + pixels * 20,             # walked records in, image / T / n_contrib out
        "zero_pixel_sums": n * 48,
        "render_bwd_raster": bwd_bytes,                      # walked records, per-pixel inputs, sums out
        # parameters, projection and sums in; gradients written (first view of a step) or read and written
        "preprocess_bwd": n * (par + 16 + 4 + 1 + 48) + n * par * (1 + (views - 1) / views),
    }
    out, floor_total = {}, 0.0
    for k, t in zip(STAGES, stage_ms):
        floor = by[k] / (HBM_PEAK_GBPS * 1e9) * 1e3
        floor_total += floor
        out[k] = {"bound": "hbm", "bytes": int(by[k]), "floor_ms": round(floor, 4), "frac": round(floor / t, 4)}
    out["frame"] = {"floor_ms": round(floor_total, 4), "frac": round(floor_total / float(sum(stage_ms)), 4),
                    "note": "sum of the stage floors over the sum of the stage times; blending is VALU bound"}
    return out


def backward_bytes(n_contrib, ranges, W, H, n_touched):
    """Algorithmic HBM bytes of one gs_render_bwd_raster launch: per walked list
    entry the record read (value 4 + mean 8 + conic/opacity 16 + colour 12 =
    40 B), per pixel its final T, n_contrib and upstream gradient (20 B), per
    touched Gaussian its 36-byte result written once (the per-tile partial sums
    meet in L2)."""
    TX = (W + 15) // 16
    TY = (H + 15) // 16
    nc = np.zeros((TY * 16, TX * 16), np.int64)
    nc[:H, :W] = n_contrib
    walked = nc.reshape(TY, 16, TX, 16).max(axis=(1, 3)).reshape(-1)  # per tile: its deepest pixel
    lens = (ranges[:, 1].astype(np.int64) - ranges[:, 0].astype(np.int64))
    walked = np.minimum(walked, lens)
    return int(40 * walked.sum() + 20 * W * H + 36 * n_touched), int(walked.sum())


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this rasterizer runs on one GPU only; --gpus must be 1 "
                          "(the multi-GPU design is described, not built)"}))
        sys.exit(2)

    import torch

    from differentiable_gaussian_splat_amd import raster, scenes

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    t0 = time.time()
    sc = scenes.make_scene(args.config, args.seed)
    log(f"[bench] scene config {args.config}: N={sc.n}, views={len(sc.cameras)}, built in {time.time() - t0:.1f}s")
    views = list(range(len(sc.cameras)))
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    means, scales, quats, opac, sh = to(sc.means), to(sc.scales), to(sc.quats), to(sc.opacities), to(sc.sh)
    dLs = [to(sc.dL_dimage[v]) for v in views]
    n = sc.n
    cams = [raster.make_camera(sc.cameras[v]) for v in views]
    opt = raster.make_options(sc.sh_degree, sc.sh.shape[1])
    # the step's first view writes the parameter gradients, the others add into them
    opt_first = raster.make_options(sc.sh_degree, sc.sh.shape[1], overwrite_grads=True)
    W, H = cams[0].width, cams[0].height
    ntiles = ((W + 15) // 16) * ((H + 15) // 16)

    # persistent buffers, sized once (a first untimed frame per view measures P)
    # values and ranges only: the renderer reads no 64-bit keys (gs_bin_sort takes keys = NULL)
    r = raster.Rasterizer(dev, want_keys=False)
    P_max = 0
    for v in views:
        pre = r.preprocess(cams[v], opt, means, scales, quats, opac, sh)
        P, _ = r.bin_sort(cams[v], opt, pre)
        P_max = max(P_max, P)
    cap = int(P_max * 1.02) + 4096
    r._values = None
    r._ensure_pairs(cap)
    r._ensure_bin_ws(n, W, H)
    E = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
    means2d, depths, conic, rgb = E((n, 2), torch.float32), E(n, torch.float32), E((n, 4), torch.float32), \
        E((n, 3), torch.float32)
    radii, tiles, clamped = E(n, torch.int32), E(n, torch.int32), E(n, torch.uint8)
    ranges = E((ntiles, 2), torch.int32)
    image, final_T, n_contrib = E((3, H, W), torch.float32), E((H, W), torch.float32), E((H, W), torch.int32)
    grad2d = E((n, raster.GRAD2D_STRIDE), torch.float32)
    # the forward's render checkpoints, read by the backward raster of the same view (none on small grids)
    nck = raster.gs_render_ckpt_bytes(W, H)
    ckpt = E(nck, torch.uint8) if nck else None
    grads = raster.empty_grads(means, sh)
    stream = torch.cuda.current_stream()
    mk = lambda: [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in views]
    ev_steps = [mk() for _ in range(args.steps)]
    ev_warm = mk()
    stage_ms = np.zeros(len(STAGES))
    last_P = [0] * len(views)

    BWD0, BWD1 = STAGES.index("render_bwd_raster"), STAGES.index("render_bwd_raster") + 1

    def step(ev, all_stages, keys=None):
        for vi, v in enumerate(views):
            e = ev[vi]
            mark = (lambda k: e[k].record(stream)) if all_stages else (lambda k: None)
            cam = cams[v]
            mark(0)
            raster.gs_preprocess(cam, opt, means, scales, quats, opac, sh, means2d, depths, conic, rgb, radii, tiles,
                                 clamped)
            mark(1)
            P = raster.gs_bin_sort(cam, opt, means2d, depths, radii, tiles, r._bin_ws, r.pair_capacity, keys,
                                   r._values, ranges)
            last_P[vi] = P
            mark(2)
            raster.gs_render_fwd(cam, opt, n, ranges, r._values, P, means2d, conic, rgb, image, final_T, n_contrib,
                                 ckpt)
            mark(3)
            grad2d.zero_()  # the pixel sums belong to one view
            e[BWD0].record(stream)
            raster.gs_render_bwd_raster(cam, opt, n, ranges, r._values, P, means2d, conic, rgb, final_T, n_contrib,
                                        dLs[vi], grad2d, ckpt)
            e[BWD1].record(stream)
            raster.gs_preprocess_bwd(cam, opt_first if vi == 0 else opt, means, scales, quats, sh, conic, radii,
                                     clamped, grad2d, grads["means"], grads["scales"], grads["quats"],
                                     grads["opacities"], grads["sh"])
            mark(6)

    for _ in range(args.warmup):
        step(ev_warm, True)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps), P per view max {max(last_P)}")
    # timed region: K steps between two synchronisations (events only around the backward raster kernel)
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(ev_steps[i], False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = 1000.0 * elapsed / args.steps
    frames = args.steps * len(views)
    ms_per_frame = 1000.0 * elapsed / frames
    bwd_launch_ms = sum(e[BWD0].elapsed_time(e[BWD1]) for ev in ev_steps for e in ev) / frames
    # per-stage breakdown: extra steps with events around every call (not timed)
    n_stage_steps = min(args.steps, 5)
    ev_stage = [mk() for _ in range(n_stage_steps)]
    for i in range(n_stage_steps):
        step(ev_stage[i], True)
    torch.cuda.synchronize()
    for ev in ev_stage:
        for e in ev:
            for k in range(len(STAGES)):
                stage_ms[k] += e[k].elapsed_time(e[k + 1])
    stage_ms /= n_stage_steps * len(views)
    log(f"[bench] {args.steps} steps in {elapsed:.3f}s: {ms_per_frame:.3f} ms/frame; "
        + ", ".join(f"{s} {t:.3f}" for s, t in zip(STAGES, stage_ms)))
    # the same steps with the sorted 64-bit keys written too (the renderer does not read them)
    keys_buf = E(r.pair_capacity, torch.int64)
    step(ev_warm, False, keys_buf)
    torch.cuda.synchronize()
    t_k = time.perf_counter()
    for i in range(args.steps):
        step(ev_steps[i], False, keys_buf)
    torch.cuda.synchronize()
    ms_keys = 1000.0 * (time.perf_counter() - t_k) / frames
    ev_k = [mk() for _ in range(n_stage_steps)]
    for i in range(n_stage_steps):
        step(ev_k[i], True, keys_buf)
    torch.cuda.synchronize()
    bin_keys_ms = sum(e[1].elapsed_time(e[2]) for ev in ev_k for e in ev) / (n_stage_steps * len(views))
    del keys_buf

    # algorithmic work of the last frame (outside the timed region)
    nc_np = n_contrib.cpu().numpy().astype(np.int64)
    rg_np = ranges.cpu().numpy().view(np.uint32)
    touched = int((radii > 0).sum().item())
    bwd_bytes, walked = backward_bytes(nc_np, rg_np, W, H, touched)
    E_b = int(nc_np.sum())
    t_bwd = bwd_launch_ms * 1e-3  # the backward raster kernel's mean launch time in the timed steps
    # blending work of the last view, counted with the forward's own decisions (gs_mb_render_counts)
    cnt = torch.zeros(8, dtype=torch.int64, device=dev)
    raster.gs_mb_render_counts(cams[views[-1]], opt, ranges, r._values, last_P[-1], means2d, conic, rgb, cnt)
    cnt = [int(x) for x in cnt.cpu().tolist()]
    E_f, E_f_eval, E_blend, E_b_cnt, P_c, band_exec, walked_cnt = cnt[:7]
    # the backward: gradient math on blended entries, alpha on the walked ones that did not blend
    bwd_flops = (ALPHA_FLOPS + BWD_GRAD_FLOPS) * E_blend + ALPHA_FLOPS * (E_b_cnt - E_blend)
    fwd_flops = (ALPHA_FLOPS + FWD_BLEND_FLOPS) * E_blend + ALPHA_FLOPS * (E_f_eval - E_blend)
    bwd_tflops = bwd_flops / t_bwd / 1e12

    batched = time_batched_views(args, raster, dev, sc, cams, opt, means, scales, quats, opac, sh, dLs, last_P,
                                 1000.0 * elapsed / args.steps) if len(views) > 1 else None
    surfel = time_surfels(args, raster, scenes, dev, sc, cams, opt, opt_first, means, quats, opac, sh, dLs)

    # measured denominators: HBM streaming read, and no-return fp32 atomic adds
    # in the backward's flush pattern (9 lanes on one record, records hashed
    # over the visible Gaussians)
    def timed(fn, reps):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    hbm_read = buf.numel() / timed(lambda: raster.gs_mb_hbm_read(buf, sink), 5) / 1e9
    # known-size copy: the reference for scaling rocprof's FETCH_SIZE / WRITE_SIZE
    half = buf.numel() // 4
    raster.gs_mb_hbm_copy(buf[half:2 * half], buf[:half])
    del buf
    # the optimizer update (phase U), timed on its own: not part of the frame's value
    rows = sh.shape[1]
    raw = {"means": means.clone(), "log_scales": torch.log(scales), "quats": quats.clone(),
           "opacity_logits": torch.logit(opac.double()).float(), "sh": sh.clone()}
    m_state = {k: torch.zeros_like(v) for k, v in raw.items()}
    v_state = {k: torch.zeros_like(v) for k, v in raw.items()}
    act_scales, act_opac = torch.empty_like(scales), torch.empty_like(opac)
    gnorm = torch.empty(n, dtype=torch.float32, device=dev)
    adam_step = [0]

    def adam():
        adam_step[0] += 1
        raster.gs_adam_step(raster.make_adam_options(adam_step[0]), raw, grads, m_state, v_state, act_scales,
                            act_opac, gnorm)
    t_adam = timed(adam, 10)
    # densification statistics: the chain-rule step of the last view with and without them
    d_acc = torch.zeros(n, dtype=torch.float32, device=dev)
    d_cnt = torch.zeros(n, dtype=torch.int32, device=dev)
    d_mr = torch.zeros(n, dtype=torch.int32, device=dev)
    dstats = raster.make_densify_stats(d_acc, d_cnt, d_mr)
    cam_last = cams[views[-1]]

    def chain(st):
        raster.gs_preprocess_bwd(cam_last, opt, means, scales, quats, sh, conic, radii, clamped, grad2d,
                                 grads["means"], grads["scales"], grads["quats"], grads["opacities"], grads["sh"],
                                 stats=st)
    t_chain = timed(lambda: chain(None), 5)
    t_chain_stats = timed(lambda: chain(dstats), 5)
    adam_bytes = n * (4 * 4 * (11 + 3 * rows) + 3 * 4 * (11 + 3 * rows) + 4 * 5)
    del raw, m_state, v_state
    n_atomics = ATOMICS_PER_TILE_ENTRY * walked
    recs = torch.zeros((max(touched, 1), raster.GRAD2D_STRIDE), dtype=torch.float32, device=dev)
    t_at = timed(lambda: raster.gs_mb_atomic(recs, recs.shape[0], n_atomics, ATOMICS_PER_TILE_ENTRY), 3)
    # the same backward raster with per-pixel atomics (no wave reduction): the pattern the pages measure
    g2n = torch.zeros_like(grad2d)
    cam_last, dl_last = cams[views[-1]], dLs[-1]
    t_naive = timed(lambda: raster.gs_mb_render_bwd_naive(cam_last, opt, n, ranges, r._values, last_P[-1], means2d,
                                                          conic, rgb, final_T, n_contrib, dl_last, g2n), 2)
    lane_hist = torch.zeros(65, dtype=torch.int32, device=dev)
    raster.gs_mb_render_bwd_naive(cam_last, opt, n, ranges, r._values, last_P[-1], means2d, conic, rgb, final_T,
                                  n_contrib, dl_last, g2n, lane_hist)
    lh = lane_hist.cpu().numpy().astype(np.float64)
    # the adaptive switch (direct atomics when few lanes blend an entry, else the wave reduction) on the
    # pieces kernel, at several lane counts; 0 is the reduced kernel itself
    adaptive = None
    if ckpt is not None:
        adaptive = {}
        for dm in (0, 4, 8, 16, 64):
            adaptive[str(dm)] = round(1e3 * timed(lambda: raster.gs_mb_render_bwd_adaptive(
                cam_last, opt, n, ranges, r._values, last_P[-1], means2d, conic, rgb, final_T, n_contrib, dl_last,
                g2n, ckpt, dm), 5), 4)
    del g2n
    atomic_rate = n_atomics / t_at
    del recs
    t_hbm_floor = bwd_bytes / (hbm_read * 1e9)
    stage_roof = stage_rooflines(n, sh.shape[1], last_P, ntiles, W * H, walked, bwd_bytes, stage_ms, len(views))
    t_atomic_floor = n_atomics / atomic_rate

    # the backward raster's kernel for one view's grid (see bwd_layout in render.hip)
    bwd_kernel = "k_render_bwd_pieces" if 4096 <= ntiles < 32768 else "k_render_bwd"
    result = {
        "metric": METRIC,
        "value": round(ms_per_frame, 4),
        "unit": "ms/frame",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": scenes.CONFIG_NAMES[args.config],
            "config": args.config, "seed": args.seed, "gaussians": n, "views_per_step": len(views),
            "image": [W, H], "sh_degree": sc.sh_degree, "pairs": int(max(last_P)),
            "visible": touched, "E_b": E_b, "bwd_tile_entries_walked": walked, "keys": False,
        },
        "keys_on": {"ms_per_frame": round(ms_keys, 4), "bin_sort_ms": round(bin_keys_ms, 4),
                    "note": "the same steps with gs_bin_sort also writing the sorted 64-bit (tile, depth) keys; "
                            "the timed steps pass keys = NULL (the renderer reads values and ranges only)"},
        "stages_ms": {s: round(float(t), 4) for s, t in zip(STAGES, stage_ms)},
        "roofline": {
            "kernel": bwd_kernel,
            "bound": "alu",
            "achieved": round(bwd_tflops, 2),
            "peak": round(FP32_PEAK_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(bwd_tflops / FP32_PEAK_TFLOPS, 4),
            "traffic": pmc_traffic(bwd_kernel, args.config),
            "work": (f"{ALPHA_FLOPS + BWD_GRAD_FLOPS} flops (FMA = 2) per blended pixel-entry x E_blend + "
                     f"{ALPHA_FLOPS} per walked, unblended pixel-entry x (E_b - E_blend) = {bwd_flops}"),
            "launch_ms": round(t_bwd * 1e3, 4),
            "note": "packed fp32 is compiled off, so 0.5 is the ceiling of an all-FMA stream",
        },
        "forward_roofline": {
            "kernel": "k_render_fwd", "bound": "alu",
            "achieved": round(fwd_flops / (stage_ms[STAGES.index("render_fwd")] * 1e-3) / 1e12, 2),
            "peak": round(FP32_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
            "frac": round(fwd_flops / (stage_ms[STAGES.index("render_fwd")] * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4),
            "work": (f"{ALPHA_FLOPS + FWD_BLEND_FLOPS} flops per blended pixel-entry x E_blend + {ALPHA_FLOPS} per "
                     f"evaluated, unblended pixel-entry x (E_f_eval - E_blend) = {fwd_flops}"),
            "stage_ms": round(float(stage_ms[STAGES.index("render_fwd")]), 4),
        },
        "blend_counts": {
            "E_f": E_f, "E_f_eval": E_f_eval, "E_blend": E_blend, "E_b": E_b_cnt, "P": int(last_P[-1]), "P_c": P_c,
            "bwd_strip_steps": band_exec, "bwd_lane_use": round(E_blend / max(64 * band_exec, 1), 4),
            "bwd_tile_entries_walked": walked_cnt,
            "note": "one view, the forward's own decisions: E_f entries evaluated per pixel up to its stop (E_f_eval "
                    "those passing the 16x4 band's bound), E_blend blended, E_b walked by the reverse pass, P_c "
                    "(tile, entry) pairs with a blended pixel, bwd_strip_steps (4x16 column strip, entry) pairs the backward "
                    "executes, bwd_lane_use = E_blend / (64 bwd_strip_steps)",
        },
        "stage_rooflines": stage_roof,
        "naive_atomic_bwd": {
            "ms": round(t_naive * 1e3, 3), "atomics": 9 * E_b, "reduced_ms": round(t_bwd * 1e3, 4),
            "atomics_reduced": n_atomics, "slowdown": round(t_naive / t_bwd, 1),
            "lanes_per_update": {"steps": int(lh.sum()), "mean": round(float((lh * np.arange(65)).sum() / lh.sum()), 2),
                                 "all_64": round(float(lh[64] / lh.sum()), 4),
                                 "at_most_8": round(float(lh[1:9].sum() / lh.sum()), 4),
                                 "quartiles": [int(np.searchsorted(np.cumsum(lh) / lh.sum(), q)) for q in
                                               (0.25, 0.5, 0.75)]},
            "note": "gs_mb_render_bwd_naive: each lane adds its own pixel's nine terms with its own atomics (about "
                    "9 per blended pixel-entry), against the wave-reduced backward raster (9 per tile-entry)",
        },
        "adaptive_bwd": None if adaptive is None else {
            "ms_by_direct_max": adaptive,
            "note": "gs_mb_render_bwd_adaptive: per (wave, entry), at most direct_max blending lanes add their "
                    "terms with their own atomics, more reduce over the wave (0: the reduced kernel; 64: direct "
                    "atomics always); the last view, after the timed steps",
        },
        "bwd_hbm_atomic_roofline": {
            "hbm_bytes": bwd_bytes,
            "hbm_floor_ms": round(t_hbm_floor * 1e3, 4),
            "atomics": n_atomics,
            "atomic_rate_per_s": round(atomic_rate, 1),
            "atomic_floor_ms": round(t_atomic_floor * 1e3, 4),
            "frac": round(max(t_hbm_floor, t_atomic_floor) / t_bwd, 4),
        },
        "measured_hbm_read_GBps": round(hbm_read, 1),
        "optimizer_step": {
            "kernel": "k_adam_step", "ms": round(t_adam * 1e3, 4), "bytes": adam_bytes,
            "achieved_GBps": round(adam_bytes / t_adam / 1e9, 1),
            "frac_hbm_peak": round(adam_bytes / t_adam / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "fused Adam update of the raw parameters with the exp / sigmoid chain and per-Gaussian "
                    "gradient norm (4 arrays read, 3 written per parameter); timed apart, not in value",
        },
        "densify_stats": {
            "chain_rule_ms": round(t_chain * 1e3, 4), "chain_rule_with_stats_ms": round(t_chain_stats * 1e3, 4),
            "note": "gs_preprocess_bwd of the last view without and with the densification statistics (12 B "
                    "read-modify-written per drawn Gaussian); timed apart, not in value",
        },
    }

    if batched is not None:
        result["batched_views"] = batched
    result["surfels"] = surfel
    if args.cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sc, args, fr_state=dict(
            means2d=means2d.cpu().numpy(), conic=conic.cpu().numpy(), rgb=rgb.cpu().numpy(),
            radii=radii.cpu().numpy(), depths=depths.cpu().numpy(), values=r._values[:last_P[-1]].cpu().numpy(),
            ranges=rg_np, P=last_P[-1]), view=views[-1])
    print(json.dumps(result), flush=True)


BATCH_STAGES = ["preprocess_views", "bin_sort_views", "render_fwd_views", "zero_pixel_sums",
                "render_bwd_raster_views", "preprocess_bwd_views"]


def time_batched_views(args, raster, dev, sc, cams, opt, means, scales, quats, opac, sh, dLs, last_P, serial_ms):
    """The same step with all views in one launch per phase (the *_views
    calls), timed the same way; per-view figures beside the serial loop's."""
    import torch
    V, n = len(cams), sc.n
    W, H = cams[0].width, cams[0].height
    ntiles = ((W + 15) // 16) * ((H + 15) // 16)
    ca = raster.make_cameras(cams)
    opt_w = raster.GsOptions.from_buffer_copy(opt)
    opt_w.overwrite_grads = 1
    E = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
    means2d, depths, conic, rgb = E((V, n, 2), torch.float32), E((V, n), torch.float32), E((V, n, 4), torch.float32), \
        E((V, n, 3), torch.float32)
    radii, tiles, clamped, mask = E((V, n), torch.int32), E((V, n), torch.int32), E((V, n), torch.uint8), \
        E(n, torch.int32)
    ranges = E((V * ntiles, 2), torch.int32)
    cap = int(sum(last_P) * 1.02) + 4096
    values = E(cap, torch.int32)
    ws = E(raster.gs_bin_sort_views_workspace_size(V, n, cap, W, H), torch.uint8)
    image, final_T, n_contrib = E((V, 3, H, W), torch.float32), E((V, H, W), torch.float32), E((V, H, W), torch.int32)
    dL = torch.stack(dLs)
    grad2d = E((V, n, raster.GRAD2D_STRIDE), torch.float32)
    grads = raster.empty_grads(means, sh)
    stream = torch.cuda.current_stream()
    P_box = [0]

    def step(ev):
        mark = (lambda k: ev[k].record(stream)) if ev else (lambda k: None)
        mark(0)
        raster.gs_preprocess_views(ca, opt, means, scales, quats, opac, sh, means2d, depths, conic, rgb, radii, tiles,
                                   clamped, mask)
        mark(1)
        P = raster.gs_bin_sort_views(ca, opt, n, means2d, depths, radii, tiles, ws, cap, None, values, ranges)
        P_box[0] = P
        mark(2)
        raster.gs_render_fwd_views(ca, opt, n, ranges, values, P, means2d, conic, rgb, image, final_T, n_contrib)
        mark(3)
        grad2d.zero_()
        mark(4)
        raster.gs_render_bwd_raster_views(ca, opt, n, ranges, values, P, means2d, conic, rgb, final_T, n_contrib, dL,
                                          grad2d)
        mark(5)
        raster.gs_preprocess_bwd_views(ca, opt_w, means, scales, quats, sh, conic, radii, clamped, grad2d,
                                       grads["means"], grads["scales"], grads["quats"], grads["opacities"],
                                       grads["sh"])
        mark(6)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(None)
    torch.cuda.synchronize()
    ms = 1000.0 * (time.perf_counter() - t0) / args.steps
    reps = min(args.steps, 5)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(BATCH_STAGES) + 1)] for _ in range(reps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    st = [sum(e[k].elapsed_time(e[k + 1]) for e in evs) / reps / V for k in range(len(BATCH_STAGES))]
    log(f"[bench] batched {V} views: {ms:.3f} ms/step, {ms / V:.3f} ms/view (serial {serial_ms / V:.3f}); "
        + ", ".join(f"{s} {t:.3f}" for s, t in zip(BATCH_STAGES, st)))
    del ws, grad2d, dL, image
    return {"views": V, "ms_per_step": round(ms, 4), "ms_per_view": round(ms / V, 4),
            "serial_ms_per_view": round(serial_ms / V, 4), "speedup_vs_serial": round(serial_ms / ms, 3),
            "pairs": P_box[0], "stages_ms_per_view": {s: round(float(t), 4) for s, t in zip(BATCH_STAGES, st)},
            "note": "all views in one launch per phase (gs_*_views): parameters read once, one binning pass over "
                    "the stacked tile grids, gradients summed per Gaussian before one write"}


SURFEL_STAGES = ["surfel_preprocess", "bin_sort", "surfel_render_fwd", "zero_pixel_sums", "surfel_render_bwd_raster",
                 "surfel_preprocess_bwd"]


def time_surfels(args, raster, scenes, dev, sc, cams, opt, opt_first, means, quats, opac, sh, dLs):
    """The same frame with 2D Gaussian surfels (each Gaussian's first two scales
    as the surfel's), timed the same way: the gs_surfel_* calls with the same
    binning; not part of value."""
    import torch
    n = sc.n
    scales2 = torch.from_numpy(scenes.surfel_scales(sc)).to(dev)
    W, H = cams[0].width, cams[0].height
    ntiles = ((W + 15) // 16) * ((H + 15) // 16)
    E = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
    means2d, depths, tf, rgb = E((n, 2), torch.float32), E(n, torch.float32), E((n, 12), torch.float32), \
        E((n, 3), torch.float32)
    radii, tiles, clamped = E(n, torch.int32), E(n, torch.int32), E(n, torch.uint8)
    ranges = E((ntiles, 2), torch.int32)
    image, final_T, n_contrib = E((3, H, W), torch.float32), E((H, W), torch.float32), E((H, W), torch.int32)
    grad = E((n, raster.SURFEL_GRAD_STRIDE), torch.float32)
    grads = dict(means=E((n, 3), torch.float32), scales=E((n, 2), torch.float32), quats=E((n, 4), torch.float32),
                 opacities=E(n, torch.float32), sh=E(tuple(sh.shape), torch.float32))
    stream = torch.cuda.current_stream()
    P_box = [0]
    cap = 0
    for cam in cams:  # pair buffers of their own, sized for the surfels' footprints
        raster.gs_surfel_preprocess(cam, opt, means, scales2, quats, opac, sh, means2d, depths, tf, rgb, radii, tiles,
                                    clamped)
        cap = max(cap, int(tiles.to(torch.int64).sum().item() * 1.02) + 4096)
    values = E(cap, torch.int32)
    bin_ws = E(raster.gs_bin_sort_workspace_size(n, cap, W, H), torch.uint8)
    nck = raster.gs_render_ckpt_bytes(W, H)
    ckpt = E(nck, torch.uint8) if nck else None  # render checkpoints, as in the frame above

    def step(evs):
        for vi, cam in enumerate(cams):
            ev = evs[vi] if evs else None
            mark = (lambda k: ev[k].record(stream)) if ev else (lambda k: None)
            mark(0)
            raster.gs_surfel_preprocess(cam, opt, means, scales2, quats, opac, sh, means2d, depths, tf, rgb, radii,
                                        tiles, clamped)
            mark(1)
            P = raster.gs_bin_sort(cam, opt, means2d, depths, radii, tiles, bin_ws, cap, None, values, ranges)
            P_box[0] = P
            mark(2)
            raster.gs_surfel_render_fwd(cam, opt, n, ranges, values, P, tf, rgb, image, final_T, n_contrib, ckpt)
            mark(3)
            grad.zero_()
            mark(4)
            raster.gs_surfel_render_bwd_raster(cam, opt, n, ranges, values, P, tf, rgb, final_T, n_contrib, dLs[vi],
                                               grad, ckpt)
            mark(5)
            raster.gs_surfel_preprocess_bwd(cam, opt_first if vi == 0 else opt, means, scales2, quats, sh, tf, radii,
                                            clamped, grad, grads["means"], grads["scales"], grads["quats"],
                                            grads["opacities"], grads["sh"])
            mark(6)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(None)
    torch.cuda.synchronize()
    ms = 1000.0 * (time.perf_counter() - t0) / (args.steps * len(cams))
    reps = min(args.steps, 5)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(SURFEL_STAGES) + 1)] for _ in cams]
           for _ in range(reps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    st = [sum(ev[k].elapsed_time(ev[k + 1]) for e in evs for ev in e) / (reps * len(cams))
          for k in range(len(SURFEL_STAGES))]
    log(f"[bench] surfels: {ms:.3f} ms/frame; " + ", ".join(f"{a} {b:.3f}" for a, b in zip(SURFEL_STAGES, st)))
    del values, bin_ws, ckpt
    return {"ms_per_frame": round(ms, 4), "pairs": int(P_box[0]), "visible": int((radii > 0).sum().item()),
            "stages_ms": {a: round(float(b), 4) for a, b in zip(SURFEL_STAGES, st)},
            "note": "2D Gaussian surfels on the same draws (a surfel's two scales are the Gaussian's first two): "
                    "gs_surfel_preprocess, gs_bin_sort, gs_surfel_render_fwd and gs_surfel_render_bwd_raster "
                    "(with render checkpoints, as the frame), gs_surfel_preprocess_bwd; timed like the frame, "
                    "not part of value"}


def pmc_traffic(kernel, config):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by the copy kernel's own
    reading), or None if there is none for this workload or the kernel's
    sources changed since it was taken."""
    import hashlib
    path = os.path.join(PROFILES, f"{kernel}_c{config}_pmc.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
    srcs = fields.get("sources", "").split()
    h = hashlib.sha256()
    for rel in srcs:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    if not srcs or h.hexdigest() != fields.get("sources_sha256"):
        return None
    return int(float(fields["hbm_bytes_per_launch"]))


def cpu_baseline(sc, args, fr_state, view):
    """The fp64 oracle on a bounded sample of the frame, scaled to ms per frame:
    all Gaussians for the per-Gaussian steps, a random fraction of Gaussians for
    the pair sort (scaled by the pair count), and a random fraction of tiles for
    the per-pixel forward and backward (scaled by the tile count)."""
    from oracle import oracle as O

    full = _cpu_sample(O, sc, args, fr_state, view)
    threads = O.max_threads()
    O.set_threads(1)
    try:
        one = _cpu_sample(O, sc, args, fr_state, view)
    finally:
        O.set_threads(threads)
    total_ms = 1000.0 * sum(full["t"].values())
    total_1 = 1000.0 * sum(one["t"].values())
    return {
        "value": round(total_ms, 1),
        "unit": "ms/frame",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 oracle, {threads} OpenMP threads: preprocess and its backward on all {sc.n} Gaussians; "
                   f"pair sort on a random {args.cpu_sort_frac:.0%} of Gaussians scaled by pair count; per-pixel "
                   f"forward and backward on {full['k']} random tiles of {full['ntiles']} scaled by tile count"),
        "stages_s": {s: round(v, 3) for s, v in full["t"].items()},
        "one_thread": {"value": round(total_1, 1), "unit": "ms/frame", "cores": 1,
                       "stages_s": {s: round(v, 3) for s, v in one["t"].items()}},
    }


def _cpu_sample(O, sc, args, fr_state, view):
    """One timing of the oracle's stages on the sample, scaled to the frame."""
    cam = sc.cameras[view]
    W, H = cam.width, cam.height
    rng = np.random.default_rng(1234)
    t = {}
    t0 = time.perf_counter()
    pre = O.preprocess(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh, cam, sc.sh_degree)
    t["preprocess"] = time.perf_counter() - t0
    # pair sort on a Gaussian subset, scaled by pairs
    sub = rng.random(sc.n) < args.cpu_sort_frac
    t0 = time.perf_counter()
    keys, values, ranges = O.bin_sort(pre["means2d"][sub], pre["radii"][sub], pre["depth"][sub].astype(np.float32), W, H)
    ts = time.perf_counter() - t0
    P_full = int(pre["tiles"].sum())
    t["bin_sort"] = ts * P_full / max(len(values), 1)
    # per-pixel stages on sampled tiles, on the GPU's lists (the same frame)
    TX, TY = (W + 15) // 16, (H + 15) // 16
    ntiles = TX * TY
    k = max(1, int(round(args.cpu_tile_frac * ntiles)))
    tiles = rng.choice(ntiles, k, replace=False)
    pix = []
    for tt in tiles:
        ty, tx = divmod(int(tt), TX)
        ys, xs = np.meshgrid(np.arange(ty * 16, min(ty * 16 + 16, H)), np.arange(tx * 16, min(tx * 16 + 16, W)),
                             indexing="ij")
        pix.append((ys * W + xs).reshape(-1))
    pix = np.concatenate(pix)
    co = fr_state["conic"]
    conic_std = O.ldl_to_conic(co[:, :3])
    vals = fr_state["values"].view(np.uint32)
    t0 = time.perf_counter()
    O.render_fwd_pixels(W, H, fr_state["ranges"], vals, fr_state["means2d"], conic_std, co[:, 3], fr_state["rgb"], pix)
    t["render_fwd"] = (time.perf_counter() - t0) * ntiles / k
    t0 = time.perf_counter()
    g2 = O.render_bwd_pixels(W, H, sc.n, fr_state["ranges"], vals, fr_state["means2d"], conic_std, co[:, 3],
                             fr_state["rgb"], sc.dL_dimage[view], pix)
    t["render_bwd"] = (time.perf_counter() - t0) * ntiles / k
    t0 = time.perf_counter()
    O.preprocess_bwd(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh, cam, sc.sh_degree, g2)
    t["preprocess_bwd"] = time.perf_counter() - t0
    return {"t": t, "k": k, "ntiles": ntiles}


if __name__ == "__main__":
    main()
