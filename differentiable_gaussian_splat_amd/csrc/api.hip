// C ABI of the rasterizer: argument validation, workspace carving, launches.
// Every entry point validates before launching anything, maps HIP failures to
// GS_ERR_HIP with the HIP message, and lets no exception escape.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/gsplat.h"
#include "common.hpp"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

gs_status fail(gs_status code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

gs_status hip_check(hipError_t e, const char* where) {
    if (e == hipSuccess) return GS_OK;
    return fail(GS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The densification statistics' arrays, or all null when none are asked for.
gs::DensifyStats densify_arrays(const gs_densify_stats* st) {
    gs::DensifyStats d{nullptr, nullptr, nullptr};
    if (st) d = gs::DensifyStats{st->grad_accum, st->count, st->max_radius};
    return d;
}

#define REQUIRE(cond, ...)                                        \
    do {                                                          \
        if (!(cond)) return fail(GS_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p) REQUIRE((p) != nullptr, "%s must not be NULL", #p)

struct Checked {
    gs::DevCam cam;
    int K, sh_rows, ntiles;
};

gs_status check_common(const gs_camera* cam, const gs_options* opt, int64_t n, Checked& out) {
    REQUIRE_PTR(cam);
    REQUIRE_PTR(opt);
    REQUIRE(n >= 0 && n < ((int64_t)1 << 31), "n must be in [0, 2^31), got %lld", (long long)n);
    REQUIRE(cam->width > 0 && cam->height > 0 && cam->width <= 32768 && cam->height <= 32768,
            "image size must be in 1..32768, got %d x %d", cam->width, cam->height);
    REQUIRE(isfinite(cam->fx) && isfinite(cam->fy) && cam->fx > 0.f && cam->fy > 0.f,
            "focal lengths must be finite and > 0");
    REQUIRE(isfinite(cam->cx) && isfinite(cam->cy), "principal point must be finite");
    for (int i = 0; i < 9; ++i) REQUIRE(isfinite(cam->R[i]), "camera R must be finite");
    for (int i = 0; i < 3; ++i) REQUIRE(isfinite(cam->t[i]), "camera t must be finite");
    REQUIRE(opt->sh_degree >= 0 && opt->sh_degree <= 3, "sh_degree must be in 0..3, got %d", opt->sh_degree);
    if (opt->tile_size != gs::TILE)
        return fail(GS_ERR_UNSUPPORTED, "tile_size must be %d, got %d", gs::TILE, opt->tile_size);
    int K = (opt->sh_degree + 1) * (opt->sh_degree + 1);
    int rows = opt->sh_rows == 0 ? K : opt->sh_rows;
    REQUIRE(rows >= K && rows <= 64, "sh_rows must be 0 or in [(deg+1)^2, 64], got %d", opt->sh_rows);
    REQUIRE(isfinite(opt->lowpass) && opt->lowpass >= 0.f, "lowpass must be finite and >= 0");
    REQUIRE(isfinite(opt->near_plane) && opt->near_plane > 0.f, "near_plane must be finite and > 0");
    for (int i = 0; i < 3; ++i) REQUIRE(isfinite(opt->bg[i]), "bg must be finite");
    REQUIRE(opt->overwrite_grads == 0 || opt->overwrite_grads == 1, "overwrite_grads must be 0 or 1, got %d",
            opt->overwrite_grads);
    gs::DevCam& d = out.cam;
    d.W = cam->width;
    d.H = cam->height;
    d.TX = (cam->width + gs::TILE - 1) / gs::TILE;
    d.TY = (cam->height + gs::TILE - 1) / gs::TILE;
    d.fx = cam->fx;
    d.fy = cam->fy;
    d.cx = cam->cx;
    d.cy = cam->cy;
    for (int i = 0; i < 9; ++i) d.R[i] = cam->R[i];
    for (int i = 0; i < 3; ++i) d.t[i] = cam->t[i];
    for (int j = 0; j < 3; ++j) {  // camera centre -R^T t, formed in double
        double c = 0.0;
        for (int i = 0; i < 3; ++i) c -= (double)cam->R[3 * i + j] * (double)cam->t[i];
        d.campos[j] = (float)c;
    }
    out.K = K;
    out.sh_rows = rows;
    out.ntiles = d.TX * d.TY;
    return GS_OK;
}

// The cameras of a batched call: each one checked as a single view, all of
// one image size; n is the number of Gaussians (per-view arrays hold V n).
struct CheckedViews {
    Checked first;
    gs::CamSet set;
    int V;
};

gs_status check_views(const gs_camera* cams, int32_t V, const gs_options* opt, int64_t n, CheckedViews& out) {
    REQUIRE_PTR(cams);
    REQUIRE(V >= 1 && V <= GS_MAX_VIEWS, "n_views must be in 1..%d, got %d", GS_MAX_VIEWS, V);
    REQUIRE(n >= 0 && n * V < ((int64_t)1 << 31), "n x n_views must be below 2^31, got %lld x %d", (long long)n, V);
    memset(&out.set, 0, sizeof(out.set));
    for (int v = 0; v < V; ++v) {
        Checked c;
        gs_status st = check_common(&cams[v], opt, n, c);
        if (st != GS_OK) {
            char msg[sizeof(g_err)];
            snprintf(msg, sizeof(msg), "%s", g_err);
            return fail(st, "camera %d: %s", v, msg);
        }
        REQUIRE(cams[v].width == cams[0].width && cams[v].height == cams[0].height,
                "all views must have one image size: camera %d is %d x %d, camera 0 %d x %d", v, cams[v].width,
                cams[v].height, cams[0].width, cams[0].height);
        if (v == 0) out.first = c;
        out.set.c[v] = c.cam;
    }
    // one workgroup per tile and band: keep the launch's work-items below 2^32
    REQUIRE((int64_t)V * out.first.ntiles <= ((int64_t)1 << 24), "n_views x tiles per view must be <= 2^24, got %lld",
            (long long)V * out.first.ntiles);
    out.V = V;
    return GS_OK;
}

// Host side of gs_bin_sort's pair-count readback: a small pinned, host-coherent
// buffer (written by a kernel through its device address) and an event per
// (thread, device), created on first use and kept until the thread calls
// gs_release_thread_state (or the process ends).
struct Readback {
    int device = -1;
    unsigned long long* host = nullptr;
    unsigned long long* mapped = nullptr;
    hipEvent_t ev = nullptr;
};

constexpr int READBACK_DEVICES = 16;
thread_local Readback t_readback[READBACK_DEVICES];

gs_status readback_for_current_device(Readback*& out) {
    Readback* slots = t_readback;
    int dev = 0;
    gs_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (st != GS_OK) return st;
    if (dev < 0 || dev >= READBACK_DEVICES) return fail(GS_ERR_UNSUPPORTED, "device index %d >= 16", dev);
    Readback& r = slots[dev];
    if (r.device != dev) {
        st = hip_check(hipHostMalloc((void**)&r.host, 64, hipHostMallocMapped | hipHostMallocCoherent),
                       "hipHostMalloc");
        if (st != GS_OK) return st;
        st = hip_check(hipHostGetDevicePointer((void**)&r.mapped, r.host, 0), "hipHostGetDevicePointer");
        if (st != GS_OK) return st;
        st = hip_check(hipEventCreateWithFlags(&r.ev, hipEventDisableTiming), "hipEventCreateWithFlags");
        if (st != GS_OK) return st;
        r.device = dev;
    }
    out = &r;
    return GS_OK;
}

}  // namespace

extern "C" {

gs_options gs_default_options(void) {
    gs_options o;
    o.sh_degree = 3;
    o.sh_rows = 0;
    o.tile_size = gs::TILE;
    o.lowpass = 0.3f;
    o.near_plane = 0.2f;
    o.bg[0] = o.bg[1] = o.bg[2] = 0.f;
    o.overwrite_grads = 0;
    return o;
}

const char* gs_version(void) { return "gsplat-hip 0.1.0 (gfx950)"; }

const char* gs_last_error(void) { return g_err; }

gs_status gs_release_thread_state(void) {
    gs_status st = GS_OK;
    for (int d = 0; d < READBACK_DEVICES; ++d) {
        Readback& r = t_readback[d];
        if (r.device < 0) continue;
        // a failed gs_bin_sort may have left its count kernel in flight: let it write first
        gs_status e = hip_check(hipEventSynchronize(r.ev), "gs_release_thread_state(wait)");
        if (e == GS_OK) e = hip_check(hipEventDestroy(r.ev), "gs_release_thread_state(event)");
        if (e == GS_OK) e = hip_check(hipHostFree(r.host), "gs_release_thread_state(host buffer)");
        if (e != GS_OK) {
            st = e;
            continue;  // kept: a later call may retry
        }
        r = Readback{};
    }
    return st;
}

gs_status gs_preprocess(const gs_camera* cam, const gs_options* opt, int64_t n, const float* means,
                        const float* scales, const float* quats, const float* opacities, const float* sh,
                        float* means2d, float* depths, float* conic_opacity, float* rgb, int32_t* radii,
                        uint32_t* tiles_touched, uint8_t* clamped, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE_PTR(means);
        REQUIRE_PTR(scales);
        REQUIRE_PTR(quats);
        REQUIRE_PTR(opacities);
        REQUIRE_PTR(sh);
        REQUIRE_PTR(means2d);
        REQUIRE_PTR(depths);
        REQUIRE_PTR(conic_opacity);
        REQUIRE_PTR(rgb);
        REQUIRE_PTR(radii);
        REQUIRE_PTR(tiles_touched);
        REQUIRE_PTR(clamped);
        REQUIRE(aligned(quats, 16), "quats must be 16-byte aligned");
        REQUIRE(aligned(conic_opacity, 16), "conic_opacity must be 16-byte aligned");
        REQUIRE(aligned(means2d, 8), "means2d must be 8-byte aligned");
        return hip_check(gs::launch_preprocess(c.cam, c.K, c.sh_rows, opt->lowpass, opt->near_plane, (int)n, means,
                                               scales, quats, opacities, sh, means2d, depths, conic_opacity, rgb,
                                               radii, tiles_touched, clamped, (hipStream_t)stream),
                         "gs_preprocess");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_preprocess: unexpected exception");
    }
}

size_t gs_bin_sort_workspace_size(int64_t n, int64_t pair_capacity, int32_t width, int32_t height) {
    if (n < 0 || pair_capacity < 0 || width <= 0 || height <= 0) return 0;
    return gs::bin_layout(n, pair_capacity, (width + 15) / 16, (height + 15) / 16).total;
}

size_t gs_render_ckpt_bytes(int32_t width, int32_t height) {
    if (width <= 0 || height <= 0 || width > 32768 || height > 32768) return 0;
    return gs::render_ckpt_bytes((width + 15) / 16, (height + 15) / 16);
}

gs_status gs_bin_sort(const gs_camera* cam, const gs_options* opt, int64_t n, const float* means2d,
                      const float* depths, const int32_t* radii, const uint32_t* tiles_touched, void* workspace,
                      size_t workspace_bytes, int64_t pair_capacity, uint64_t* keys, uint32_t* values,
                      uint32_t* ranges, int64_t* n_pairs, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        REQUIRE_PTR(n_pairs);
        REQUIRE_PTR(ranges);
        REQUIRE(pair_capacity >= 0 && pair_capacity < ((int64_t)1 << 31), "pair_capacity must be in [0, 2^31)");
        REQUIRE(pair_capacity == 0 || values != nullptr, "values must not be NULL");
        if (n > 0) {
            REQUIRE_PTR(means2d);
            REQUIRE_PTR(depths);
            REQUIRE_PTR(radii);
            REQUIRE_PTR(tiles_touched);
            REQUIRE_PTR(workspace);
            REQUIRE(aligned(means2d, 8), "means2d must be 8-byte aligned");
            REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
        }
        gs::BinLayout L = gs::bin_layout(n, pair_capacity, c.cam.TX, c.cam.TY);
        if (n > 0)
            REQUIRE(workspace_bytes >= L.total, "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
        hipStream_t s = (hipStream_t)stream;
        if (n == 0) {
            *n_pairs = 0;
            return hip_check(gs::launch_fill_u32(ranges, (size_t)2 * c.ntiles, 0u, s), "gs_bin_sort");
        }
        Readback* rb = nullptr;
        st = readback_for_current_device(rb);
        if (st != GS_OK) return st;
        char* ws = reinterpret_cast<char*>(workspace);
        st = hip_check(gs::launch_bin_count((int)n, 0, c.cam.TX, c.cam.TY, means2d, radii, depths, tiles_touched, ws, L,
                                            rb->mapped, rb->ev, s),
                       "gs_bin_sort(count)");
        if (st != GS_OK) return st;
        // the one wait: for the pair count only; the depth sort keeps running
        st = hip_check(hipEventSynchronize(rb->ev), "gs_bin_sort(wait)");
        if (st != GS_OK) return st;
        const unsigned long long P = rb->host[0], P1 = rb->host[1];
        *n_pairs = (int64_t)P;
        if (P >= (1ull << 31)) return fail(GS_ERR_UNSUPPORTED, "pair count %llu exceeds 2^31 - 1", P);
        if ((int64_t)P > pair_capacity)
            return fail(GS_ERR_CAPACITY, "pair count %llu exceeds capacity %lld", P, (long long)pair_capacity);
        // every super-tile entry holds at least one of the Gaussian's pairs
        if (P1 > P) return fail(GS_ERR_HIP, "super-tile entries %llu exceed pairs %llu", P1, P);
        return hip_check(gs::launch_bin_emit((int)n, (int)P, (int)P1, c.cam.TX, c.cam.TY, depths, ws, L, keys,
                                             values, ranges, s),
                         "gs_bin_sort(emit)");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_bin_sort: unexpected exception");
    }
}

// The render checkpoints: null, or 16-byte aligned and at least
// gs_render_ckpt_bytes of the camera's image size.
static gs_status check_ckpt(const void* ckpt, size_t ckpt_bytes, const Checked& c) {
    if (!ckpt) return GS_OK;
    REQUIRE(aligned(ckpt, 16), "ckpt must be 16-byte aligned");
    REQUIRE(ckpt_bytes >= gs::render_ckpt_bytes(c.cam.TX, c.cam.TY),
            "ckpt_bytes %zu < gs_render_ckpt_bytes %zu", ckpt_bytes, gs::render_ckpt_bytes(c.cam.TX, c.cam.TY));
    return GS_OK;
}

gs_status gs_render_fwd(const gs_camera* cam, const gs_options* opt, int64_t n, const uint32_t* ranges,
                        const uint32_t* values, int64_t n_pairs, const float* means2d, const float* conic_opacity,
                        const float* rgb, float* image, float* final_T, uint32_t* n_contrib, void* ckpt,
                        size_t ckpt_bytes, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        REQUIRE_PTR(ranges);
        REQUIRE_PTR(image);
        REQUIRE_PTR(final_T);
        REQUIRE_PTR(n_contrib);
        REQUIRE(n_pairs >= 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
        if (n_pairs > 0) {
            REQUIRE(n > 0, "n_pairs > 0 needs n > 0");
            REQUIRE_PTR(values);
            REQUIRE_PTR(means2d);
            REQUIRE_PTR(conic_opacity);
            REQUIRE_PTR(rgb);
            REQUIRE(aligned(means2d, 8), "means2d must be 8-byte aligned");
            REQUIRE(aligned(conic_opacity, 16), "conic_opacity must be 16-byte aligned");
        }
        REQUIRE(aligned(ranges, 8), "ranges must be 8-byte aligned");
        st = check_ckpt(ckpt, ckpt_bytes, c);
        if (st != GS_OK) return st;
        return hip_check(gs::launch_render_fwd(1, c.cam.W, c.cam.H, c.cam.TX, c.cam.TY, ranges, values, means2d,
                                               conic_opacity, rgb, opt->bg, image, final_T, n_contrib,
                                               static_cast<float*>(ckpt), (hipStream_t)stream),
                         "gs_render_fwd");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_render_fwd: unexpected exception");
    }
}

}  // extern "C"

namespace {

// gs_render_bwd with its pixel-sum records at grad2d (n records of 48 bytes,
// 256-byte aligned): arguments checked, records zeroed by a fill kernel, the
// backward raster, the chain rule.
gs_status render_bwd_into(const char* name, const gs_camera* cam, const gs_options* opt, int64_t n,
                          const float* means, const float* scales, const float* quats, const float* opacities,
                          const float* sh, const float* means2d, const float* conic_opacity, const float* rgb,
                          const int32_t* radii, const uint8_t* clamped, const uint32_t* ranges,
                          const uint32_t* values, int64_t n_pairs, const float* final_T, const uint32_t* n_contrib,
                          const float* dL_dimage, float* dL_dmeans, float* dL_dscales, float* dL_dquats,
                          float* dL_dopacities, float* dL_dsh, float* dL_dmeans2d, float* grad2d, const void* ckpt,
                          size_t ckpt_bytes, const gs_densify_stats* stats, void* stream) {
    REQUIRE_PTR(means);
    REQUIRE_PTR(scales);
    REQUIRE_PTR(quats);
    REQUIRE_PTR(opacities);
    REQUIRE_PTR(sh);
    REQUIRE_PTR(means2d);
    REQUIRE_PTR(conic_opacity);
    REQUIRE_PTR(rgb);
    REQUIRE_PTR(radii);
    REQUIRE_PTR(clamped);
    REQUIRE_PTR(ranges);
    REQUIRE_PTR(final_T);
    REQUIRE_PTR(n_contrib);
    REQUIRE_PTR(dL_dimage);
    REQUIRE_PTR(dL_dmeans);
    REQUIRE_PTR(dL_dscales);
    REQUIRE_PTR(dL_dquats);
    REQUIRE_PTR(dL_dopacities);
    REQUIRE_PTR(dL_dsh);
    REQUIRE(n_pairs >= 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
    REQUIRE(n_pairs == 0 || values != nullptr, "values must not be NULL");
    REQUIRE(aligned(quats, 16) && aligned(dL_dquats, 16), "quats and dL_dquats must be 16-byte aligned");
    REQUIRE(aligned(conic_opacity, 16), "conic_opacity must be 16-byte aligned");
    REQUIRE(aligned(means2d, 8) && aligned(ranges, 8), "means2d and ranges must be 8-byte aligned");
    REQUIRE(!stats || (stats->grad_accum && stats->count && stats->max_radius),
            "stats: grad_accum, count and max_radius must all be set");
    Checked c;
    gs_status st = check_common(cam, opt, n, c);
    if (st != GS_OK) return st;
    st = check_ckpt(ckpt, ckpt_bytes, c);
    if (st != GS_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    std::string where = std::string(name) + "(zero)";
    st = hip_check(gs::launch_fill_u32(reinterpret_cast<uint32_t*>(grad2d), (size_t)n * gs::GRAD2D_STRIDE, 0u, s),
                   where.c_str());
    if (st != GS_OK) return st;
    if (n_pairs > 0) {
        where = std::string(name) + "(raster)";
        st = hip_check(gs::launch_render_bwd(1, c.cam.W, c.cam.H, c.cam.TX, c.cam.TY, ranges, values, means2d,
                                             conic_opacity, rgb, opt->bg, final_T, n_contrib, dL_dimage, grad2d,
                                             static_cast<const float*>(ckpt), s),
                       where.c_str());
        if (st != GS_OK) return st;
    }
    where = std::string(name) + "(chain)";
    return hip_check(gs::launch_preprocess_bwd(c.cam, c.K, c.sh_rows, opt->lowpass, opt->near_plane, (int)n, means,
                                               scales, quats, sh, conic_opacity, radii, clamped, grad2d, dL_dmeans,
                                               dL_dscales, dL_dquats, dL_dopacities, dL_dsh, dL_dmeans2d,
                                               opt->overwrite_grads != 0, densify_arrays(stats), s),
                     where.c_str());
}

// Pixel-sum records of gs_render_bwd_noalloc: GS_NOALLOC_MAX_N records of
// 48 bytes (48 MiB), one copy per GPU, held from the library's load on that
// GPU until the process ends. Host code never passes this name to a kernel
// (on the host it is a stand-in, not a device address): it takes the
// device's own address from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[(size_t)GS_NOALLOC_MAX_N * gs::GRAD2D_STRIDE];

struct ScratchSlot {
    std::once_flag once;
    float* ptr = nullptr;
    hipError_t err = hipSuccess;
};

gs_status scratch_for_current_device(float*& out) {
    static ScratchSlot slots[16];
    int dev = 0;
    gs_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (st != GS_OK) return st;
    if (dev < 0 || dev >= READBACK_DEVICES) return fail(GS_ERR_UNSUPPORTED, "device index %d >= 16", dev);
    ScratchSlot& sl = slots[dev];
    // the current device is `dev` here, so the address is that device's copy
    std::call_once(sl.once, [&sl] { sl.err = hipGetSymbolAddress((void**)&sl.ptr, HIP_SYMBOL(scratch)); });
    if (sl.err != hipSuccess || sl.ptr == nullptr)
        return fail(GS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    sl.err != hipSuccess ? hipGetErrorString(sl.err) : "null address");
    out = sl.ptr;
    return GS_OK;
}

}  // namespace

extern "C" {

size_t gs_render_bwd_workspace_size(int64_t n) {
    if (n < 0) return 0;
    return ((size_t)(n > 0 ? n : 1) * gs::GRAD2D_STRIDE * sizeof(float) + 255) & ~(size_t)255;
}

gs_status gs_render_bwd(const gs_camera* cam, const gs_options* opt, int64_t n, const float* means,
                        const float* scales, const float* quats, const float* opacities, const float* sh,
                        const float* means2d, const float* conic_opacity, const float* rgb, const int32_t* radii,
                        const uint8_t* clamped, const uint32_t* ranges, const uint32_t* values, int64_t n_pairs,
                        const float* final_T, const uint32_t* n_contrib, const float* dL_dimage, float* dL_dmeans,
                        float* dL_dscales, float* dL_dquats, float* dL_dopacities, float* dL_dsh,
                        float* dL_dmeans2d, void* workspace, size_t workspace_bytes, const void* ckpt,
                        size_t ckpt_bytes, const gs_densify_stats* stats, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE_PTR(workspace);
        REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
        size_t need = gs_render_bwd_workspace_size(n);
        REQUIRE(workspace_bytes >= need, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
        return render_bwd_into("gs_render_bwd", cam, opt, n, means, scales, quats, opacities, sh, means2d,
                               conic_opacity, rgb, radii, clamped, ranges, values, n_pairs, final_T, n_contrib,
                               dL_dimage, dL_dmeans, dL_dscales, dL_dquats, dL_dopacities, dL_dsh, dL_dmeans2d,
                               reinterpret_cast<float*>(workspace), ckpt, ckpt_bytes, stats, stream);
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_render_bwd: unexpected exception");
    }
}

gs_status gs_render_bwd_noalloc(const gs_camera* cam, const gs_options* opt, int64_t n, const float* means,
                                const float* scales, const float* quats, const float* opacities, const float* sh,
                                const float* means2d, const float* conic_opacity, const float* rgb,
                                const int32_t* radii, const uint8_t* clamped, const uint32_t* ranges,
                                const uint32_t* values, int64_t n_pairs, const float* final_T,
                                const uint32_t* n_contrib, const float* dL_dimage, float* dL_dmeans,
                                float* dL_dscales, float* dL_dquats, float* dL_dopacities, float* dL_dsh,
                                float* dL_dmeans2d, const void* ckpt, size_t ckpt_bytes,
                                const gs_densify_stats* stats, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n > GS_NOALLOC_MAX_N)
            return fail(GS_ERR_CAPACITY, "gs_render_bwd_noalloc: n = %lld exceeds its fixed scratch of %d Gaussians",
                        (long long)n, GS_NOALLOC_MAX_N);
        if (n == 0) return GS_OK;
        float* grad2d = nullptr;
        st = scratch_for_current_device(grad2d);
        if (st != GS_OK) return st;
        return render_bwd_into("gs_render_bwd_noalloc", cam, opt, n, means, scales, quats, opacities, sh, means2d,
                               conic_opacity, rgb, radii, clamped, ranges, values, n_pairs, final_T, n_contrib,
                               dL_dimage, dL_dmeans, dL_dscales, dL_dquats, dL_dopacities, dL_dsh, dL_dmeans2d,
                               grad2d, ckpt, ckpt_bytes, stats, stream);
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_render_bwd_noalloc: unexpected exception");
    }
}

gs_status gs_render_bwd_raster(const gs_camera* cam, const gs_options* opt, int64_t n, const uint32_t* ranges,
                               const uint32_t* values, int64_t n_pairs, const float* means2d,
                               const float* conic_opacity, const float* rgb, const float* final_T,
                               const uint32_t* n_contrib, const float* dL_dimage, float* grad2d, const void* ckpt,
                               size_t ckpt_bytes, void* stream) {
    try {
        g_err[0] = 0;
        static_assert(GS_GRAD2D_STRIDE == gs::GRAD2D_STRIDE, "record stride");
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE_PTR(ranges);
        REQUIRE_PTR(final_T);
        REQUIRE_PTR(n_contrib);
        REQUIRE_PTR(dL_dimage);
        REQUIRE_PTR(grad2d);
        REQUIRE(n_pairs >= 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
        if (n_pairs > 0) {
            REQUIRE_PTR(values);
            REQUIRE_PTR(means2d);
            REQUIRE_PTR(conic_opacity);
            REQUIRE_PTR(rgb);
        }
        REQUIRE(aligned(grad2d, 16), "grad2d must be 16-byte aligned");
        REQUIRE(aligned(conic_opacity, 16), "conic_opacity must be 16-byte aligned");
        REQUIRE(aligned(means2d, 8) && aligned(ranges, 8), "means2d and ranges must be 8-byte aligned");
        if (n_pairs == 0) return GS_OK;
        st = check_ckpt(ckpt, ckpt_bytes, c);
        if (st != GS_OK) return st;
        return hip_check(gs::launch_render_bwd(1, c.cam.W, c.cam.H, c.cam.TX, c.cam.TY, ranges, values, means2d,
                                               conic_opacity, rgb, opt->bg, final_T, n_contrib, dL_dimage, grad2d,
                                               static_cast<const float*>(ckpt), (hipStream_t)stream),
                         "gs_render_bwd_raster");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_render_bwd_raster: unexpected exception");
    }
}

gs_status gs_preprocess_bwd(const gs_camera* cam, const gs_options* opt, int64_t n, const float* means,
                            const float* scales, const float* quats, const float* sh, const float* conic_opacity,
                            const int32_t* radii, const uint8_t* clamped, const float* grad2d, float* dL_dmeans,
                            float* dL_dscales, float* dL_dquats, float* dL_dopacities, float* dL_dsh,
                            float* dL_dmeans2d, const gs_densify_stats* stats, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE_PTR(means);
        REQUIRE_PTR(scales);
        REQUIRE_PTR(quats);
        REQUIRE_PTR(sh);
        REQUIRE_PTR(conic_opacity);
        REQUIRE_PTR(radii);
        REQUIRE_PTR(clamped);
        REQUIRE_PTR(grad2d);
        REQUIRE_PTR(dL_dmeans);
        REQUIRE_PTR(dL_dscales);
        REQUIRE_PTR(dL_dquats);
        REQUIRE_PTR(dL_dopacities);
        REQUIRE_PTR(dL_dsh);
        REQUIRE(aligned(quats, 16) && aligned(dL_dquats, 16), "quats and dL_dquats must be 16-byte aligned");
        REQUIRE(aligned(conic_opacity, 16) && aligned(grad2d, 16), "conic_opacity and grad2d must be 16-byte aligned");
        REQUIRE(!stats || (stats->grad_accum && stats->count && stats->max_radius),
                "stats: grad_accum, count and max_radius must all be set");
        return hip_check(gs::launch_preprocess_bwd(c.cam, c.K, c.sh_rows, opt->lowpass, opt->near_plane, (int)n,
                                                   means, scales, quats, sh, conic_opacity, radii, clamped, grad2d,
                                                   dL_dmeans, dL_dscales, dL_dquats, dL_dopacities, dL_dsh,
                                                   dL_dmeans2d, opt->overwrite_grads != 0, densify_arrays(stats),
                                                   (hipStream_t)stream),
                         "gs_preprocess_bwd");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_preprocess_bwd: unexpected exception");
    }
}

// ---------------------------------------------------------------- 2D Gaussian surfels

gs_status gs_surfel_preprocess(const gs_camera* cam, const gs_options* opt, int64_t n, const float* means,
                               const float* scales, const float* quats, const float* opacities, const float* sh,
                               float* means2d, float* depths, float* transforms, float* rgb, int32_t* radii,
                               uint32_t* tiles_touched, uint8_t* clamped, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE(means && scales && quats && opacities && sh && means2d && depths && transforms && rgb && radii &&
                    tiles_touched && clamped,
                "gs_surfel_preprocess: NULL array");
        REQUIRE(aligned(quats, 16) && aligned(transforms, 16) && aligned(means2d, 8),
                "quats and transforms must be 16-byte aligned, means2d 8-byte aligned");
        return hip_check(gs::launch_surfel_preprocess(c.cam, c.K, c.sh_rows, opt->near_plane, (int)n, means, scales,
                                                      quats, opacities, sh, means2d, depths, transforms, rgb, radii,
                                                      tiles_touched, clamped, (hipStream_t)stream),
                         "gs_surfel_preprocess");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_surfel_preprocess: unexpected exception");
    }
}

gs_status gs_surfel_render_fwd(const gs_camera* cam, const gs_options* opt, int64_t n, const uint32_t* ranges,
                               const uint32_t* values, int64_t n_pairs, const float* transforms, const float* rgb,
                               float* image, float* final_T, uint32_t* n_contrib, void* ckpt, size_t ckpt_bytes,
                               void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        REQUIRE(ranges && image && final_T && n_contrib, "gs_surfel_render_fwd: NULL array");
        st = check_ckpt(ckpt, ckpt_bytes, c);
        if (st != GS_OK) return st;
        REQUIRE(n_pairs >= 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
        REQUIRE(n_pairs == 0 || (values && transforms && rgb), "gs_surfel_render_fwd: NULL array");
        REQUIRE(aligned(ranges, 8) && (!transforms || aligned(transforms, 16)),
                "ranges must be 8-byte aligned, transforms 16-byte aligned");
        return hip_check(gs::launch_surfel_render_fwd(c.cam.W, c.cam.H, c.cam.TX, c.cam.TY, ranges, values,
                                                      transforms, rgb, opt->bg, image, final_T, n_contrib,
                                                      static_cast<float*>(ckpt), (hipStream_t)stream),
                         "gs_surfel_render_fwd");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_surfel_render_fwd: unexpected exception");
    }
}

gs_status gs_surfel_render_bwd_raster(const gs_camera* cam, const gs_options* opt, int64_t n, const uint32_t* ranges,
                                      const uint32_t* values, int64_t n_pairs, const float* transforms,
                                      const float* rgb, const float* final_T, const uint32_t* n_contrib,
                                      const float* dL_dimage, float* grad, const void* ckpt, size_t ckpt_bytes,
                                      void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE(ranges && final_T && n_contrib && dL_dimage && grad, "gs_surfel_render_bwd_raster: NULL array");
        st = check_ckpt(ckpt, ckpt_bytes, c);
        if (st != GS_OK) return st;
        REQUIRE(n_pairs >= 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
        if (n_pairs == 0) return GS_OK;
        REQUIRE(values && transforms && rgb, "gs_surfel_render_bwd_raster: NULL array");
        REQUIRE(aligned(ranges, 8) && aligned(transforms, 16) && aligned(grad, 16),
                "ranges must be 8-byte aligned, transforms and grad 16-byte aligned");
        return hip_check(gs::launch_surfel_render_bwd(c.cam.W, c.cam.H, c.cam.TX, c.cam.TY, ranges, values,
                                                      transforms, rgb, opt->bg, final_T, n_contrib, dL_dimage, grad,
                                                      static_cast<const float*>(ckpt), (hipStream_t)stream),
                         "gs_surfel_render_bwd_raster");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_surfel_render_bwd_raster: unexpected exception");
    }
}

gs_status gs_surfel_preprocess_bwd(const gs_camera* cam, const gs_options* opt, int64_t n, const float* means,
                                   const float* scales, const float* quats, const float* sh, const float* transforms,
                                   const int32_t* radii, const uint8_t* clamped, const float* grad, float* dL_dmeans,
                                   float* dL_dscales, float* dL_dquats, float* dL_dopacities, float* dL_dsh,
                                   void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE(means && scales && quats && sh && transforms && radii && clamped && grad && dL_dmeans && dL_dscales &&
                    dL_dquats && dL_dopacities && dL_dsh,
                "gs_surfel_preprocess_bwd: NULL array");
        REQUIRE(aligned(quats, 16) && aligned(dL_dquats, 16) && aligned(transforms, 16) && aligned(grad, 16),
                "quats, dL_dquats, transforms and grad must be 16-byte aligned");
        return hip_check(gs::launch_surfel_preprocess_bwd(c.cam, c.K, c.sh_rows, (int)n, means, scales, quats, sh,
                                                          transforms, radii, clamped, grad, dL_dmeans, dL_dscales,
                                                          dL_dquats, dL_dopacities, dL_dsh,
                                                          opt->overwrite_grads != 0, (hipStream_t)stream),
                         "gs_surfel_preprocess_bwd");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_surfel_preprocess_bwd: unexpected exception");
    }
}

size_t gs_surfel_render_bwd_workspace_size(int64_t n) {
    if (n < 0) return 0;
    return ((size_t)(n > 0 ? n : 1) * gs::SURFEL_GRAD_STRIDE * sizeof(float) + 255) & ~(size_t)255;
}

gs_status gs_surfel_render_bwd(const gs_camera* cam, const gs_options* opt, int64_t n, const float* means,
                               const float* scales, const float* quats, const float* sh, const float* transforms,
                               const float* rgb, const int32_t* radii, const uint8_t* clamped, const uint32_t* ranges,
                               const uint32_t* values, int64_t n_pairs, const float* final_T,
                               const uint32_t* n_contrib, const float* dL_dimage, float* dL_dmeans,
                               float* dL_dscales, float* dL_dquats, float* dL_dopacities, float* dL_dsh,
                               void* workspace, size_t workspace_bytes, const void* ckpt, size_t ckpt_bytes,
                               void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE(workspace && aligned(workspace, 256), "workspace must be non-NULL and 256-byte aligned");
        const size_t need = gs_surfel_render_bwd_workspace_size(n);
        REQUIRE(workspace_bytes >= need, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
        float* grad = reinterpret_cast<float*>(workspace);
        hipStream_t s = (hipStream_t)stream;
        st = hip_check(gs::launch_fill_u32(reinterpret_cast<uint32_t*>(grad), (size_t)n * gs::SURFEL_GRAD_STRIDE, 0u,
                                           s),
                       "gs_surfel_render_bwd(zero)");
        if (st != GS_OK) return st;
        st = gs_surfel_render_bwd_raster(cam, opt, n, ranges, values, n_pairs, transforms, rgb, final_T, n_contrib,
                                         dL_dimage, grad, ckpt, ckpt_bytes, stream);
        if (st != GS_OK) return st;
        return gs_surfel_preprocess_bwd(cam, opt, n, means, scales, quats, sh, transforms, radii, clamped, grad,
                                        dL_dmeans, dL_dscales, dL_dquats, dL_dopacities, dL_dsh, stream);
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_surfel_render_bwd: unexpected exception");
    }
}

// ---------------------------------------------------------------- several views per launch

gs_status gs_preprocess_views(const gs_camera* cams, int32_t n_views, const gs_options* opt, int64_t n,
                              const float* means, const float* scales, const float* quats, const float* opacities,
                              const float* sh, float* means2d, float* depths, float* conic_opacity, float* rgb,
                              int32_t* radii, uint32_t* tiles_touched, uint8_t* clamped, uint32_t* vis_mask,
                              void* stream) {
    try {
        g_err[0] = 0;
        CheckedViews c;
        gs_status st = check_views(cams, n_views, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE_PTR(means);
        REQUIRE_PTR(scales);
        REQUIRE_PTR(quats);
        REQUIRE_PTR(opacities);
        REQUIRE_PTR(sh);
        REQUIRE_PTR(means2d);
        REQUIRE_PTR(depths);
        REQUIRE_PTR(conic_opacity);
        REQUIRE_PTR(rgb);
        REQUIRE_PTR(radii);
        REQUIRE_PTR(tiles_touched);
        REQUIRE_PTR(clamped);
        REQUIRE(aligned(quats, 16), "quats must be 16-byte aligned");
        REQUIRE(aligned(conic_opacity, 16), "conic_opacity must be 16-byte aligned");
        REQUIRE(aligned(means2d, 8), "means2d must be 8-byte aligned");
        return hip_check(gs::launch_preprocess_views(c.set, c.V, c.first.K, c.first.sh_rows, opt->lowpass,
                                                     opt->near_plane, (int)n, means, scales, quats, opacities, sh,
                                                     means2d, depths, conic_opacity, rgb, radii, tiles_touched,
                                                     clamped, vis_mask, (hipStream_t)stream),
                         "gs_preprocess_views");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_preprocess_views: unexpected exception");
    }
}

size_t gs_bin_sort_views_workspace_size(int32_t n_views, int64_t n, int64_t pair_capacity, int32_t width,
                                        int32_t height) {
    if (n_views < 1 || n_views > GS_MAX_VIEWS || n < 0 || pair_capacity < 0 || width <= 0 || height <= 0) return 0;
    return gs::bin_layout(n * n_views, pair_capacity, (width + 15) / 16, n_views * ((height + 15) / 16)).total;
}

gs_status gs_bin_sort_views(const gs_camera* cams, int32_t n_views, const gs_options* opt, int64_t n,
                            const float* means2d, const float* depths, const int32_t* radii,
                            const uint32_t* tiles_touched, void* workspace, size_t workspace_bytes,
                            int64_t pair_capacity, uint64_t* keys, uint32_t* values, uint32_t* ranges,
                            int64_t* n_pairs, void* stream) {
    try {
        g_err[0] = 0;
        CheckedViews c;
        gs_status st = check_views(cams, n_views, opt, n, c);
        if (st != GS_OK) return st;
        REQUIRE_PTR(n_pairs);
        REQUIRE_PTR(ranges);
        REQUIRE(pair_capacity >= 0 && pair_capacity < ((int64_t)1 << 31), "pair_capacity must be in [0, 2^31)");
        REQUIRE(pair_capacity == 0 || values != nullptr, "values must not be NULL");
        const int64_t total = n * c.V;
        const int TX = c.first.cam.TX, TY = c.first.cam.TY;
        if (total > 0) {
            REQUIRE_PTR(means2d);
            REQUIRE_PTR(depths);
            REQUIRE_PTR(radii);
            REQUIRE_PTR(tiles_touched);
            REQUIRE_PTR(workspace);
            REQUIRE(aligned(means2d, 8), "means2d must be 8-byte aligned");
            REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
        }
        gs::BinLayout L = gs::bin_layout(total, pair_capacity, TX, c.V * TY);
        if (total > 0)
            REQUIRE(workspace_bytes >= L.total, "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
        hipStream_t s = (hipStream_t)stream;
        if (total == 0) {
            *n_pairs = 0;
            return hip_check(gs::launch_fill_u32(ranges, (size_t)2 * c.V * c.first.ntiles, 0u, s),
                             "gs_bin_sort_views");
        }
        Readback* rb = nullptr;
        st = readback_for_current_device(rb);
        if (st != GS_OK) return st;
        char* ws = reinterpret_cast<char*>(workspace);
        st = hip_check(gs::launch_bin_count((int)total, c.V > 1 ? (int)n : 0, TX, TY, means2d, radii, depths,
                                            tiles_touched, ws, L, rb->mapped, rb->ev, s),
                       "gs_bin_sort_views(count)");
        if (st != GS_OK) return st;
        st = hip_check(hipEventSynchronize(rb->ev), "gs_bin_sort_views(wait)");
        if (st != GS_OK) return st;
        const unsigned long long P = rb->host[0], P1 = rb->host[1];
        *n_pairs = (int64_t)P;
        if (P >= (1ull << 31)) return fail(GS_ERR_UNSUPPORTED, "pair count %llu exceeds 2^31 - 1", P);
        if ((int64_t)P > pair_capacity)
            return fail(GS_ERR_CAPACITY, "pair count %llu exceeds capacity %lld", P, (long long)pair_capacity);
        if (P1 > P) return fail(GS_ERR_HIP, "super-tile entries %llu exceed pairs %llu", P1, P);
        return hip_check(gs::launch_bin_emit((int)total, (int)P, (int)P1, TX, c.V * TY, depths, ws, L, keys, values,
                                             ranges, s),
                         "gs_bin_sort_views(emit)");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_bin_sort_views: unexpected exception");
    }
}

gs_status gs_render_fwd_views(const gs_camera* cams, int32_t n_views, const gs_options* opt, int64_t n,
                              const uint32_t* ranges, const uint32_t* values, int64_t n_pairs, const float* means2d,
                              const float* conic_opacity, const float* rgb, float* image, float* final_T,
                              uint32_t* n_contrib, void* stream) {
    try {
        g_err[0] = 0;
        CheckedViews c;
        gs_status st = check_views(cams, n_views, opt, n, c);
        if (st != GS_OK) return st;
        REQUIRE_PTR(ranges);
        REQUIRE_PTR(image);
        REQUIRE_PTR(final_T);
        REQUIRE_PTR(n_contrib);
        REQUIRE(n_pairs >= 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
        if (n_pairs > 0) {
            REQUIRE(n > 0, "n_pairs > 0 needs n > 0");
            REQUIRE_PTR(values);
            REQUIRE_PTR(means2d);
            REQUIRE_PTR(conic_opacity);
            REQUIRE_PTR(rgb);
            REQUIRE(aligned(means2d, 8), "means2d must be 8-byte aligned");
            REQUIRE(aligned(conic_opacity, 16), "conic_opacity must be 16-byte aligned");
        }
        REQUIRE(aligned(ranges, 8), "ranges must be 8-byte aligned");
        const gs::DevCam& d = c.first.cam;
        return hip_check(gs::launch_render_fwd(c.V, d.W, d.H, d.TX, d.TY, ranges, values, means2d, conic_opacity, rgb,
                                               opt->bg, image, final_T, n_contrib, nullptr, (hipStream_t)stream),
                         "gs_render_fwd_views");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_render_fwd_views: unexpected exception");
    }
}

gs_status gs_render_bwd_raster_views(const gs_camera* cams, int32_t n_views, const gs_options* opt, int64_t n,
                                     const uint32_t* ranges, const uint32_t* values, int64_t n_pairs,
                                     const float* means2d, const float* conic_opacity, const float* rgb,
                                     const float* final_T, const uint32_t* n_contrib, const float* dL_dimage,
                                     float* grad2d, void* stream) {
    try {
        g_err[0] = 0;
        CheckedViews c;
        gs_status st = check_views(cams, n_views, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE_PTR(ranges);
        REQUIRE_PTR(final_T);
        REQUIRE_PTR(n_contrib);
        REQUIRE_PTR(dL_dimage);
        REQUIRE_PTR(grad2d);
        REQUIRE(n_pairs >= 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
        if (n_pairs > 0) {
            REQUIRE_PTR(values);
            REQUIRE_PTR(means2d);
            REQUIRE_PTR(conic_opacity);
            REQUIRE_PTR(rgb);
        }
        REQUIRE(aligned(grad2d, 16), "grad2d must be 16-byte aligned");
        REQUIRE(aligned(conic_opacity, 16), "conic_opacity must be 16-byte aligned");
        REQUIRE(aligned(means2d, 8) && aligned(ranges, 8), "means2d and ranges must be 8-byte aligned");
        if (n_pairs == 0) return GS_OK;
        const gs::DevCam& d = c.first.cam;
        return hip_check(gs::launch_render_bwd(c.V, d.W, d.H, d.TX, d.TY, ranges, values, means2d, conic_opacity, rgb,
                                               opt->bg, final_T, n_contrib, dL_dimage, grad2d, nullptr,
                                               (hipStream_t)stream),
                         "gs_render_bwd_raster_views");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_render_bwd_raster_views: unexpected exception");
    }
}

gs_status gs_preprocess_bwd_views(const gs_camera* cams, int32_t n_views, const gs_options* opt, int64_t n,
                                  const float* means, const float* scales, const float* quats, const float* sh,
                                  const float* conic_opacity, const int32_t* radii, const uint8_t* clamped,
                                  const float* grad2d, float* dL_dmeans, float* dL_dscales, float* dL_dquats,
                                  float* dL_dopacities, float* dL_dsh, float* dL_dmeans2d,
                                  const gs_densify_stats* stats, void* stream) {
    try {
        g_err[0] = 0;
        CheckedViews c;
        gs_status st = check_views(cams, n_views, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0) return GS_OK;
        REQUIRE_PTR(means);
        REQUIRE_PTR(scales);
        REQUIRE_PTR(quats);
        REQUIRE_PTR(sh);
        REQUIRE_PTR(conic_opacity);
        REQUIRE_PTR(radii);
        REQUIRE_PTR(clamped);
        REQUIRE_PTR(grad2d);
        REQUIRE_PTR(dL_dmeans);
        REQUIRE_PTR(dL_dscales);
        REQUIRE_PTR(dL_dquats);
        REQUIRE_PTR(dL_dopacities);
        REQUIRE_PTR(dL_dsh);
        REQUIRE(aligned(quats, 16) && aligned(dL_dquats, 16), "quats and dL_dquats must be 16-byte aligned");
        REQUIRE(aligned(conic_opacity, 16) && aligned(grad2d, 16), "conic_opacity and grad2d must be 16-byte aligned");
        REQUIRE(!stats || (stats->grad_accum && stats->count && stats->max_radius),
                "stats: grad_accum, count and max_radius must all be set");
        return hip_check(gs::launch_preprocess_bwd_views(c.set, c.V, c.first.K, c.first.sh_rows, opt->lowpass,
                                                         opt->near_plane, (int)n, means, scales, quats, sh,
                                                         conic_opacity, radii, clamped, grad2d, dL_dmeans, dL_dscales,
                                                         dL_dquats, dL_dopacities, dL_dsh, dL_dmeans2d,
                                                         opt->overwrite_grads != 0, densify_arrays(stats),
                                                         (hipStream_t)stream),
                         "gs_preprocess_bwd_views");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_preprocess_bwd_views: unexpected exception");
    }
}

gs_status gs_adam_step(const gs_adam_options* opt, int64_t n, int32_t sh_rows, float* const params[5],
                       const float* const grads[5], float* const exp_avg[5], float* const exp_avg_sq[5],
                       float* scales, float* opacities, float* grad_norm, void* stream) {
    try {
        g_err[0] = 0;
        REQUIRE_PTR(opt);
        REQUIRE(n >= 0 && n < ((int64_t)1 << 31), "n must be in [0, 2^31), got %lld", (long long)n);
        REQUIRE(sh_rows >= 1 && sh_rows <= 64, "sh_rows must be in [1, 64], got %d", sh_rows);
        REQUIRE(opt->step >= 1, "step must be >= 1, got %d", opt->step);
        REQUIRE(opt->beta1 >= 0.f && opt->beta1 < 1.f && opt->beta2 >= 0.f && opt->beta2 < 1.f,
                "beta1 and beta2 must be in [0, 1)");
        REQUIRE(isfinite(opt->eps) && opt->eps >= 0.f, "eps must be finite and >= 0");
        const float lrs[6] = {opt->lr_means, opt->lr_scales, opt->lr_quats, opt->lr_opacity, opt->lr_sh_dc,
                              opt->lr_sh_rest};
        for (float l : lrs) REQUIRE(isfinite(l), "learning rates must be finite");
        if (n == 0) return GS_OK;
        REQUIRE_PTR(params);
        REQUIRE_PTR(grads);
        REQUIRE_PTR(exp_avg);
        REQUIRE_PTR(exp_avg_sq);
        REQUIRE_PTR(scales);
        REQUIRE_PTR(opacities);
        for (int i = 0; i < 5; ++i) {
            REQUIRE(params[i] && grads[i] && exp_avg[i] && exp_avg_sq[i], "array %d of params/grads/state is NULL", i);
            REQUIRE(aligned(params[i], 16) && aligned(grads[i], 16) && aligned(exp_avg[i], 16) &&
                        aligned(exp_avg_sq[i], 16),
                    "array %d of params/grads/state must be 16-byte aligned", i);
        }
        REQUIRE(aligned(scales, 16) && aligned(opacities, 16) && aligned(grad_norm, 16),
                "scales, opacities and grad_norm must be 16-byte aligned");
        gs::AdamLr lr{opt->lr_means, opt->lr_scales, opt->lr_quats, opt->lr_opacity, opt->lr_sh_dc, opt->lr_sh_rest};
        return hip_check(gs::launch_adam_step(lr, opt->beta1, opt->beta2, opt->eps, opt->step, (int)n, sh_rows,
                                              params, grads, exp_avg, exp_avg_sq, scales, opacities, grad_norm,
                                              (hipStream_t)stream),
                         "gs_adam_step");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_adam_step: unexpected exception");
    }
}

gs_status gs_mb_render_bwd_adaptive(const gs_camera* cam, const gs_options* opt, int64_t n, const uint32_t* ranges,
                                    const uint32_t* values, int64_t n_pairs, const float* means2d,
                                    const float* conic_opacity, const float* rgb, const float* final_T,
                                    const uint32_t* n_contrib, const float* dL_dimage, float* grad2d,
                                    const void* ckpt, size_t ckpt_bytes, int32_t direct_max, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        REQUIRE(direct_max >= 0 && direct_max <= 64, "direct_max must be in [0, 64], got %d", direct_max);
        if (n == 0 || n_pairs == 0) return GS_OK;
        REQUIRE(n_pairs > 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
        REQUIRE(ranges && values && means2d && conic_opacity && rgb && final_T && n_contrib && dL_dimage && grad2d,
                "gs_mb_render_bwd_adaptive: NULL array");
        REQUIRE(aligned(grad2d, 16) && aligned(conic_opacity, 16) && aligned(means2d, 8) && aligned(ranges, 8),
                "gs_mb_render_bwd_adaptive: misaligned array");
        if (!ckpt || gs::render_ckpt_bytes(c.cam.TX, c.cam.TY) == 0)
            return fail(GS_ERR_UNSUPPORTED,
                        "gs_mb_render_bwd_adaptive: needs the forward's checkpoints (grids of 4096..32767 tiles)");
        st = check_ckpt(ckpt, ckpt_bytes, c);
        if (st != GS_OK) return st;
        return hip_check(gs::launch_render_bwd_adaptive(c.cam.W, c.cam.H, c.cam.TX, c.cam.TY, ranges, values, means2d,
                                                        conic_opacity, rgb, opt->bg, final_T, n_contrib, dL_dimage,
                                                        grad2d, static_cast<const float*>(ckpt), direct_max,
                                                        (hipStream_t)stream),
                         "gs_mb_render_bwd_adaptive");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_mb_render_bwd_adaptive: unexpected exception");
    }
}

gs_status gs_mb_render_bwd_naive(const gs_camera* cam, const gs_options* opt, int64_t n, const uint32_t* ranges,
                                 const uint32_t* values, int64_t n_pairs, const float* means2d,
                                 const float* conic_opacity, const float* rgb, const float* final_T,
                                 const uint32_t* n_contrib, const float* dL_dimage, float* grad2d,
                                 uint32_t* lane_hist, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, n, c);
        if (st != GS_OK) return st;
        if (n == 0 || n_pairs == 0) return GS_OK;
        REQUIRE(n_pairs > 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
        REQUIRE(ranges && values && means2d && conic_opacity && rgb && final_T && n_contrib && dL_dimage && grad2d,
                "gs_mb_render_bwd_naive: NULL array");
        REQUIRE(aligned(grad2d, 16) && aligned(conic_opacity, 16) && aligned(means2d, 8) && aligned(ranges, 8),
                "gs_mb_render_bwd_naive: misaligned array");
        return hip_check(gs::launch_render_bwd_naive(c.cam.W, c.cam.H, c.cam.TX, c.cam.TY, ranges, values, means2d,
                                                     conic_opacity, rgb, opt->bg, final_T, n_contrib, dL_dimage,
                                                     grad2d, lane_hist, (hipStream_t)stream),
                         "gs_mb_render_bwd_naive");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_mb_render_bwd_naive: unexpected exception");
    }
}

gs_status gs_mb_render_counts(const gs_camera* cam, const gs_options* opt, const uint32_t* ranges,
                              const uint32_t* values, int64_t n_pairs, const float* means2d,
                              const float* conic_opacity, const float* rgb, uint64_t* counts, void* stream) {
    try {
        g_err[0] = 0;
        Checked c;
        gs_status st = check_common(cam, opt, 0, c);
        if (st != GS_OK) return st;
        REQUIRE(counts && ranges, "gs_mb_render_counts: NULL array");
        REQUIRE(n_pairs >= 0 && n_pairs < ((int64_t)1 << 31), "n_pairs must be in [0, 2^31)");
        if (n_pairs == 0) return GS_OK;
        REQUIRE(values && means2d && conic_opacity && rgb, "gs_mb_render_counts: NULL array");
        REQUIRE(aligned(conic_opacity, 16) && aligned(means2d, 8) && aligned(ranges, 8) && aligned(counts, 8),
                "gs_mb_render_counts: misaligned array");
        return hip_check(gs::launch_render_counts(c.cam.W, c.cam.H, c.cam.TX, c.cam.TY, ranges, values, means2d,
                                                  conic_opacity, rgb, reinterpret_cast<unsigned long long*>(counts),
                                                  (hipStream_t)stream),
                         "gs_mb_render_counts");
    } catch (...) {
        return fail(GS_ERR_HIP, "gs_mb_render_counts: unexpected exception");
    }
}

gs_status gs_mb_hbm_read(const void* src, size_t bytes, float* sink, void* stream) {
    if (!src || !sink || bytes % 16 || !aligned(src, 16)) return fail(GS_ERR_INVALID_ARG, "gs_mb_hbm_read: bad args");
    return hip_check(gs::launch_mb_read(src, bytes, sink, (hipStream_t)stream), "gs_mb_hbm_read");
}

gs_status gs_mb_hbm_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16 || !aligned(src, 16) || !aligned(dst, 16))
        return fail(GS_ERR_INVALID_ARG, "gs_mb_hbm_copy: bad args");
    return hip_check(gs::launch_mb_copy(dst, src, bytes, (hipStream_t)stream), "gs_mb_hbm_copy");
}

gs_status gs_mb_atomic(float* records, int64_t n_records, int64_t n_ops, int32_t lanes_per_record, void* stream) {
    if (!records || n_records < 1 || n_records > 0x7fffffff || n_ops < 0 || lanes_per_record < 1 ||
        lanes_per_record > gs::GRAD2D_STRIDE)
        return fail(GS_ERR_INVALID_ARG, "gs_mb_atomic: bad args");
    return hip_check(gs::launch_mb_atomic(records, n_records, n_ops, lanes_per_record, (hipStream_t)stream),
                     "gs_mb_atomic");
}

}  // extern "C"
