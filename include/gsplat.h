/*
 * gsplat.h -- C ABI of the MI355X (gfx950) tile-based 3D Gaussian splatting
 * rasterizer: forward and backward.
 *
 * The method is the rasterizer of "3D Gaussian Splatting for Real-Time
 * Radiance Field Rendering", which the DISTWAR page ("DISTWAR: Fast
 * Differentiable Rendering on Raster-based Rendering Pipelines", abstract)
 * names as the workload whose gradient computation is bound by atomic
 * updates; the Odin page splits one training iteration into preprocessing,
 * rendering and backward computation (Fig. 7 caption). The four calls below
 * are those three phases, with rendering split into binning and blending:
 *
 *   gs_preprocess  per-Gaussian EWA projection to a 2D conic, screen radius,
 *                  tile rectangle and spherical-harmonics colour   (phase P)
 *   gs_bin_sort    one (tile, depth) pair per touched tile, sorted by tile
 *                  then depth then Gaussian index; per-tile ranges  (phase R)
 *   gs_render_fwd  per pixel front-to-back alpha blending           (phase R)
 *   gs_render_bwd  reverse blend summed into per-Gaussian gradients and the
 *                  chain rule back to the parameters                (phase B)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every array argument is a DEVICE pointer to caller-owned, contiguous,
 *   row-major memory unless marked "host". The library allocates no device
 *   memory: scratch comes from a caller-supplied workspace. Two things it
 *   does keep: gs_bin_sort's pair-count readback, a 64-byte pinned, mapped
 *   host buffer and a HIP event per (calling thread, device), created on the
 *   thread's first call on that device and kept until the thread calls
 *   gs_release_thread_state() (or the process ends); and the fixed scratch
 *   array of gs_render_bwd_noalloc, one per GPU, kept until the process ends.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream). The single exception is gs_bin_sort, which blocks the calling
 *   thread once, until the pair count has reached the host.
 * - Arguments are validated before anything is launched. On an error nothing
 *   is written, and gs_last_error() returns a message (thread-local). No C++
 *   exception crosses this interface.
 * - Gaussian parameters are the ACTIVATED ones: scales s > 0 (not log-scales),
 *   opacities o in (0, 1] (not logits), quaternions (w, x, y, z) of any
 *   non-zero norm (normalised inside). Gradients are with respect to exactly
 *   these arrays; an exp / sigmoid reparameterisation is the caller's chain.
 * - Camera: x_c = R x_w + t with R row-major; x right, y down, z forward;
 *   pixel (px, py) has its centre at (px + 0.5, py + 0.5).
 * - Screen-space conic. conic_opacity[g] = (a, beta, gamma, opacity) holds the
 *   inverse 2D covariance in factored form: for d = pixel centre - (u, v),
 *       d^T Sigma'^-1 d = a (dx + beta dy)^2 + gamma dy^2 ,
 *   i.e. the standard conic entries are (a, a beta, gamma + a beta^2). Both
 *   terms are non-negative, so fp32 evaluation loses no digits to cancellation.
 * - Compositing constants: alpha = min(0.99, o exp(-Q/2)); an entry with
 *   alpha < 1/255 is skipped; a pixel stops before the entry that would take
 *   its transmittance below 1e-4 (that entry is not blended).
 * - Sizes: n < 2^31 Gaussians, pair counts < 2^31, width, height <= 32768.
 */
#ifndef GSPLAT_H
#define GSPLAT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gs_status;
#define GS_OK 0
#define GS_ERR_INVALID_ARG (-1) /* bad argument; nothing launched or written */
#define GS_ERR_CAPACITY (-2)    /* pair buffers too small; *n_pairs = needed  */
#define GS_ERR_HIP (-3)         /* a HIP call failed; message in gs_last_error */
#define GS_ERR_UNSUPPORTED (-4) /* valid but unsupported (e.g. tile_size != 16) */

/* Pinhole camera. */
typedef struct gs_camera {
    int32_t width, height; /* image size in pixels, 1..32768 */
    float fx, fy;          /* focal lengths in pixels, > 0 */
    float cx, cy;          /* principal point in pixels */
    float R[9];            /* world -> camera rotation, row-major */
    float t[3];            /* world -> camera translation */
} gs_camera;

/* Rasterization options. */
typedef struct gs_options {
    int32_t sh_degree;  /* 0..3: colour uses K = (sh_degree + 1)^2 SH rows    */
    int32_t sh_rows;    /* rows stored per Gaussian in `sh` (>= K); 0 means K */
    int32_t tile_size;  /* must be 16                                         */
    float lowpass;      /* added to both diagonal entries of the 2D covariance, px^2 (0.3) */
    float near_plane;   /* Gaussians with camera-space z <= near_plane are culled (0.2)   */
    float bg[3];        /* background colour, blended with the final transmittance       */
    int32_t overwrite_grads; /* 0: the backward ADDS into the parameter gradients; 1: it
                                WRITES them, every row (zeros for culled Gaussians and for
                                SH rows at or beyond K), as if they had been zeroed first */
} gs_options;

/* Default options: sh_degree 3, sh_rows 0, tile 16, lowpass 0.3, near 0.2, bg 0,
 * overwrite_grads 0. */
gs_options gs_default_options(void);

const char *gs_version(void);
/* Message of the last failed call on this thread ("" if none). */
const char *gs_last_error(void);

/*
 * gs_release_thread_state -- frees the calling thread's pair-count readback
 * buffers and events (see the conventions above), after waiting for any
 * count kernel still writing them. For callers that start and end many
 * threads; a later gs_bin_sort on the thread creates them again. Returns
 * GS_ERR_HIP if a HIP call fails (what could not be freed is kept).
 */
gs_status gs_release_thread_state(void);

/*
 * gs_preprocess -- per-Gaussian projection (phase P).
 *
 * For each Gaussian g < n: cull (z <= near_plane, any non-finite input or
 * derived value, a zero quaternion, a screen position or 3-sigma extent beyond
 * 2^24 px, an empty tile rectangle); otherwise the EWA 2D covariance
 * Sigma' = J W Sigma W^T J^T + lowpass I, its inverse as the factored conic,
 * the radius r = ceil(3 sqrt(lambda_max(Sigma'))), the screen mean
 * (u, v) = (fx x/z + cx, fy y/z + cy), the tile rectangle
 * X0 = max(0, floor((floor(u) - r)/16)), X1 = min(TX-1, floor((floor(u) + r)/16))
 * (same for y), and rgb = max(0, sum_k sh[g,k] Y_k(dir) + 0.5) with dir the
 * unit vector from the camera centre to the mean and Y_k the real spherical
 * harmonics of degree <= sh_degree.
 *
 * in : means[n,3], scales[n,3], quats[n,4] (w,x,y,z; 16-byte aligned),
 *      opacities[n], sh[n, sh_rows, 3]
 * out: means2d[n,2] (u, v; 8-byte aligned), depths[n] (camera z),
 *      conic_opacity[n,4] (a, beta, gamma, opacity; 16-byte aligned),
 *      rgb[n,3], radii[n] (0 = culled), tiles_touched[n] (rectangle area,
 *      0 = culled), clamped[n] (bit c set when colour channel c was clamped at 0).
 * A culled Gaussian gets radii = tiles_touched = 0 and zeros elsewhere.
 */
gs_status gs_preprocess(const gs_camera *cam, const gs_options *opt, int64_t n,
                        const float *means, const float *scales, const float *quats,
                        const float *opacities, const float *sh,
                        float *means2d, float *depths, float *conic_opacity, float *rgb,
                        int32_t *radii, uint32_t *tiles_touched, uint8_t *clamped,
                        void *stream);

/* Workspace bytes gs_bin_sort needs for n Gaussians and pair_capacity pairs. */
size_t gs_bin_sort_workspace_size(int64_t n, int64_t pair_capacity, int32_t width, int32_t height);

/*
 * gs_bin_sort -- tile binning with a (tile, depth) key sort.
 *
 * Emits one pair per (visible Gaussian, tile of its rectangle), with key
 * (tile_id << 32) | bits(fp32 depth), tile_id = ty * TX + tx, value = Gaussian
 * index, and sorts the pairs ascending by key, equal keys by ascending index
 * (the result is unique). ranges[t] = [first, last + 1) of tile t in the
 * sorted order, (0, 0) for an empty tile.
 *
 * in : means2d, depths, radii, tiles_touched as written by gs_preprocess
 * ws : workspace of workspace_bytes >= gs_bin_sort_workspace_size(...), 256-byte aligned
 * out: values[pair_capacity], ranges[TX*TY, 2], keys[pair_capacity] (may be NULL:
 *      the keys are fully determined by ranges, values and depths),
 *      *n_pairs (host) = P.
 * Blocks once, on an event recorded right after the reduction that yields P
 * (the depth sort queued behind it keeps the GPU busy meanwhile), to read P
 * on the host. If P > pair_capacity it returns
 * GS_ERR_CAPACITY with *n_pairs = P and writes nothing else; the caller grows
 * its buffers and calls again.
 */
gs_status gs_bin_sort(const gs_camera *cam, const gs_options *opt, int64_t n,
                      const float *means2d, const float *depths, const int32_t *radii,
                      const uint32_t *tiles_touched, void *workspace, size_t workspace_bytes,
                      int64_t pair_capacity, uint64_t *keys, uint32_t *values, uint32_t *ranges,
                      int64_t *n_pairs, void *stream);

/*
 * gs_render_fwd -- front-to-back blending per pixel (phase R).
 *
 * Pixel p of tile t walks values[ranges[t]] in order: alpha as above; skip
 * alpha < 1/255; stop before the entry that would take T below 1e-4;
 * C += rgb alpha T; T *= (1 - alpha).
 * out: image[3,H,W] = C + T bg (planar), final_T[H,W] = T,
 *      n_contrib[H,W] = 1-based position (within the tile's list) of the last
 *      blended entry, 0 if none.
 * ckpt (nullable): render checkpoints for the backward of the same frame, a
 *      16-byte aligned device buffer of ckpt_bytes >= gs_render_ckpt_bytes(W, H)
 *      (caller-owned, no initialisation needed: every tile's 16-byte walk
 *      summary is written, the per-pixel states only for tiles whose walk
 *      passes 256 entries). Passed again to gs_render_bwd / gs_render_bwd_raster
 *      with the same frame, it lets the backward cut a deep tile's walk into
 *      pieces of 256 entries run by separate waves, each starting from the
 *      state the forward saw there. The backward's results do not depend on it
 *      beyond rounding. A buffer from another frame gives wrong gradients (no
 *      out-of-bounds access). NULL, or a size where gs_render_ckpt_bytes is 0:
 *      none.
 * The result is deterministic (no atomics).
 */
gs_status gs_render_fwd(const gs_camera *cam, const gs_options *opt, int64_t n,
                        const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                        const float *means2d, const float *conic_opacity, const float *rgb,
                        float *image, float *final_T, uint32_t *n_contrib,
                        void *ckpt, size_t ckpt_bytes, void *stream);

/* Bytes of render checkpoints for one view of width x height pixels; 0 where
 * the backward does not use them (grids of fewer than 4096 or of 32768 or more
 * 16x16 tiles, or an invalid size). */
size_t gs_render_ckpt_bytes(int32_t width, int32_t height);

/* Workspace bytes gs_render_bwd needs for n Gaussians. */
size_t gs_render_bwd_workspace_size(int64_t n);

/*
 * gs_render_bwd -- backward of gs_render_fwd and gs_preprocess (phase B).
 *
 * Per pixel, walks its blended entries in reverse with the upstream gradient
 * dL_dimage[3,H,W], forms each entry's contribution to the gradients of its
 * colour, opacity, conic and screen mean, sums them per Gaussian (wave-level
 * reduction first, then one fp32 atomic add per value per (tile, Gaussian)),
 * then applies the chain rule of gs_preprocess per Gaussian.
 *
 * in : the inputs and outputs of gs_preprocess and gs_bin_sort, final_T and
 *      n_contrib from gs_render_fwd, dL_dimage[3,H,W]
 * out: ACCUMULATED (+=) dL_dmeans[n,3], dL_dscales[n,3], dL_dquats[n,4],
 *      dL_dopacities[n], dL_dsh[n, sh_rows, 3] (rows < K), and, if non-NULL,
 *      dL_dmeans2d[n,2] (gradient with respect to (u, v)); with
 *      opt->overwrite_grads = 1 all of them are WRITTEN instead (every row).
 * ws : workspace of workspace_bytes >= gs_render_bwd_workspace_size(n)
 * ckpt (nullable): the checkpoints gs_render_fwd wrote for this frame (same
 *      buffer and size), or NULL.
 * stats (nullable): densification statistics of this view, added (see
 *      gs_densify_stats).
 * The caller zeroes the gradient buffers once per step (or renders the step's
 * first view with overwrite_grads = 1); several views rendered in turn on one
 * stream then sum their gradients.
 * Summation order across tiles is not fixed (atomics): results agree to
 * rounding between runs, not bit for bit.
 */
/*
 * Densification statistics (optional output of the backward): the inputs to
 * the densify and prune steps whose structural changes the Odin page
 * synchronises (referee report, weakest assumptions: structural versions for
 * densification, pruning and opacity reset). For every Gaussian drawn in the
 * view (radius > 0), per call:
 *   grad_accum[g] += |(dL/du, dL/dv)|   (the view's screen-mean gradient norm)
 *   count[g]      += 1
 *   max_radius[g]  = max(max_radius[g], radius[g])
 * The three arrays have n entries each (int32 for count and max_radius) and
 * are the caller's to zero. Each Gaussian is updated by one thread per call:
 * no atomics, deterministic.
 */
typedef struct gs_densify_stats {
    float *grad_accum;
    int32_t *count;
    int32_t *max_radius;
} gs_densify_stats;

gs_status gs_render_bwd(const gs_camera *cam, const gs_options *opt, int64_t n,
                        const float *means, const float *scales, const float *quats,
                        const float *opacities, const float *sh,
                        const float *means2d, const float *conic_opacity, const float *rgb,
                        const int32_t *radii, const uint8_t *clamped,
                        const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                        const float *final_T, const uint32_t *n_contrib, const float *dL_dimage,
                        float *dL_dmeans, float *dL_dscales, float *dL_dquats,
                        float *dL_dopacities, float *dL_dsh, float *dL_dmeans2d,
                        void *workspace, size_t workspace_bytes, const void *ckpt, size_t ckpt_bytes,
                        const gs_densify_stats *stats, void *stream);

/*
 * gs_render_bwd_noalloc -- gs_render_bwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments, results and error behaviour as
 * gs_render_bwd, without workspace / workspace_bytes: the per-Gaussian pixel
 * sums go to a scratch array inside the library (GS_NOALLOC_MAX_N records of
 * 48 bytes, 48 MiB, one copy per GPU, held from the library's load on that GPU
 * until the process ends). The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.
 *   n > GS_NOALLOC_MAX_N -> GS_ERR_CAPACITY, nothing launched.
 * The scratch array keeps the last call's contents; each call clears the part
 * it uses (a fill kernel on the stream, no hipMemsetAsync). All calls on one
 * GPU share it, so calls that overlap on one GPU (concurrent streams or host
 * threads) race: the caller serialises them.
 */
#define GS_NOALLOC_MAX_N (1 << 20)
gs_status gs_render_bwd_noalloc(const gs_camera *cam, const gs_options *opt, int64_t n,
                                const float *means, const float *scales, const float *quats,
                                const float *opacities, const float *sh,
                                const float *means2d, const float *conic_opacity, const float *rgb,
                                const int32_t *radii, const uint8_t *clamped,
                                const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                                const float *final_T, const uint32_t *n_contrib, const float *dL_dimage,
                                float *dL_dmeans, float *dL_dscales, float *dL_dquats,
                                float *dL_dopacities, float *dL_dsh, float *dL_dmeans2d,
                                const void *ckpt, size_t ckpt_bytes,
                                const gs_densify_stats *stats, void *stream);

/* The two halves of gs_render_bwd, for callers that time or test them apart
 * (gs_render_bwd = gs_render_bwd_raster followed by gs_preprocess_bwd). */

/* Per-Gaussian pixel sums of the reverse blend of ONE view, ADDED to
 * grad2d[n, GS_GRAD2D_STRIDE] (16-byte aligned; the caller zeroes it before
 * each view: the sums belong to that view's projection). With, per blended
 * (pixel, Gaussian) entry, w = dx + beta dy and h = opacity G dL/dalpha
 * (h = 0 where alpha was clamped at 0.99), record g holds
 *   [0..2] dL/drgb, [3] sum h, [4] sum h w^2, [5] sum h w dy, [6] sum h dy^2,
 *   [7] sum h w, [8] sum h dy, [9..11] unused (zero).
 * The sums are linear in the pixels, so per-tile partial sums are added
 * atomically; gs_preprocess_bwd turns them into conic and mean gradients.
 * ckpt (nullable): as in gs_render_bwd. */
#define GS_GRAD2D_STRIDE 12
gs_status gs_render_bwd_raster(const gs_camera *cam, const gs_options *opt, int64_t n,
                               const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                               const float *means2d, const float *conic_opacity, const float *rgb,
                               const float *final_T, const uint32_t *n_contrib, const float *dL_dimage,
                               float *grad2d, const void *ckpt, size_t ckpt_bytes, void *stream);

/* Chain rule from grad2d (as written by gs_render_bwd_raster) to the
 * parameters; outputs ACCUMULATE (+=), or are written with
 * opt->overwrite_grads = 1, exactly as in gs_render_bwd. */
gs_status gs_preprocess_bwd(const gs_camera *cam, const gs_options *opt, int64_t n,
                            const float *means, const float *scales, const float *quats, const float *sh,
                            const float *conic_opacity, const int32_t *radii, const uint8_t *clamped,
                            const float *grad2d, float *dL_dmeans, float *dL_dscales, float *dL_dquats,
                            float *dL_dopacities, float *dL_dsh, float *dL_dmeans2d,
                            const gs_densify_stats *stats, void *stream);

/* ------------------------------------------------------------------------
 * 2D Gaussian surfels (planar Gaussians): the second pipeline the Odin review
 * page evaluates beside 3D Gaussian splatting (referee report summary: 3DGS,
 * 2DGS, TamingGS, DashGS), after "2D Gaussian Splatting for Geometrically
 * Accurate Radiance Fields" in its references. The page prints none of the
 * method's formulas; the library's reading:
 *  - a surfel has a centre mean[3], a unit quaternion whose rotation's first
 *    two columns are its tangent axes t_u, t_v, two activated scales
 *    scales[n,2] = (s_u, s_v), an opacity and SH colour (as gs_preprocess);
 *  - the surfel point (u, v) is the world point mean + u s_u t_u + v s_v t_v;
 *    with a = s_u R t_u, b = s_v R t_v, X = R mean + t (camera frame) it lands
 *    at the homogeneous screen point M (u, v, 1), M = K [a | b | X],
 *    K = [[fx, 0, cx], [0, fy, cy], [0, 0, 1]];
 *  - culled when the centre's depth or the nearest point of the 3-sigma disc
 *    u^2 + v^2 <= 9 is at or before the near plane, on non-finite inputs, or
 *    when |c| or the extent passes 2^24 px;
 *  - c = the projected centre, depth = its camera z; radius r = ceil of the
 *    largest distance from c to a side of the bounding box of the disc's
 *    image (tangents of the dual conic M diag(1, 1, -1/9) M^T), at least
 *    3 sqrt(1/2) (the screen filter's 3 sigma); the tile rectangle is that of
 *    gs_preprocess on (c, r), so gs_bin_sort bins surfels unchanged;
 *  - per pixel centre (x, y): h_x = M0 - x M2, h_y = M1 - y M2 (rows of M),
 *    k = h_x x h_y, (u, v) = (k0, k1) / k2; G = exp(-rho / 2) with
 *    rho = min(u^2 + v^2, 2 |(x, y) - c|^2) (the surfel's own falloff or a
 *    screen filter of variance 1/2, the wider one); alpha = min(0.99, o G)
 *    and the compositing rules of gs_render_fwd.
 * transforms[n,12] (16-byte aligned): three float4 per surfel,
 * (M row 0, opacity), (M row 1, c_x), (M row 2, c_y).
 * grad[n, GS_SURFEL_GRAD_STRIDE] pixel sums: [0..2] dL/drgb, [3] sum of
 * h = alpha dL/dalpha (0 where alpha sat at 0.99), [4..6] sum of dL/dk,
 * [7..9] sum of (x - c_x) dL/dk, [10..12] sum of (y - c_y) dL/dk, for the
 * expansion k = h_x x h_y = N01 + x N12 - y N02 (N01 = M0 x M1, N12 = M1 x M2,
 * N02 = M0 x M2), [13..14] sum of h ((x, y) - c) over the pixels where the
 * screen filter is the wider falloff, [15] zero.
 * Ownership, errors, streams and accumulation as the 3D Gaussian calls.
 * ------------------------------------------------------------------------ */
#define GS_SURFEL_GRAD_STRIDE 16

/* The projection of n surfels: the outputs of gs_preprocess with transforms
 * in place of conic_opacity (culled surfels: zeros). */
gs_status gs_surfel_preprocess(const gs_camera *cam, const gs_options *opt, int64_t n,
                               const float *means, const float *scales, const float *quats,
                               const float *opacities, const float *sh,
                               float *means2d, float *depths, float *transforms, float *rgb,
                               int32_t *radii, uint32_t *tiles_touched, uint8_t *clamped, void *stream);

/* Per-pixel compositing of the binned surfels (lists from gs_bin_sort on the
 * surfels' means2d, depths, radii, tiles_touched): image[3,H,W], final_T[H,W],
 * n_contrib[H,W] as gs_render_fwd. ckpt (nullable): render checkpoints for the
 * backward of the same frame, exactly as gs_render_fwd's (same size,
 * gs_render_ckpt_bytes(W, H), and the same contract). */
gs_status gs_surfel_render_fwd(const gs_camera *cam, const gs_options *opt, int64_t n,
                               const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                               const float *transforms, const float *rgb,
                               float *image, float *final_T, uint32_t *n_contrib,
                               void *ckpt, size_t ckpt_bytes, void *stream);

/* The reverse blend's per-surfel pixel sums of ONE view, ADDED to
 * grad[n, GS_SURFEL_GRAD_STRIDE] (the caller zeroes it per view). ckpt
 * (nullable): the checkpoints gs_surfel_render_fwd wrote for this frame (same
 * buffer and size), which let deep tiles' walks be cut into pieces, or NULL. */
gs_status gs_surfel_render_bwd_raster(const gs_camera *cam, const gs_options *opt, int64_t n,
                                      const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                                      const float *transforms, const float *rgb, const float *final_T,
                                      const uint32_t *n_contrib, const float *dL_dimage, float *grad,
                                      const void *ckpt, size_t ckpt_bytes, void *stream);

/* The chain rule from grad to the activated parameters: ACCUMULATED (+=)
 * dL_dmeans[n,3], dL_dscales[n,2], dL_dquats[n,4], dL_dopacities[n],
 * dL_dsh[n, sh_rows, 3] (rows < K), or WRITTEN with opt->overwrite_grads = 1. */
gs_status gs_surfel_preprocess_bwd(const gs_camera *cam, const gs_options *opt, int64_t n,
                                   const float *means, const float *scales, const float *quats,
                                   const float *sh, const float *transforms, const int32_t *radii,
                                   const uint8_t *clamped, const float *grad, float *dL_dmeans,
                                   float *dL_dscales, float *dL_dquats, float *dL_dopacities,
                                   float *dL_dsh, void *stream);

/* Workspace bytes of gs_surfel_render_bwd for n surfels. */
size_t gs_surfel_render_bwd_workspace_size(int64_t n);

/* gs_surfel_render_bwd_raster into a zeroed workspace (with ckpt, nullable, as
 * there), then gs_surfel_preprocess_bwd. */
gs_status gs_surfel_render_bwd(const gs_camera *cam, const gs_options *opt, int64_t n,
                               const float *means, const float *scales, const float *quats,
                               const float *sh, const float *transforms, const float *rgb,
                               const int32_t *radii, const uint8_t *clamped,
                               const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                               const float *final_T, const uint32_t *n_contrib, const float *dL_dimage,
                               float *dL_dmeans, float *dL_dscales, float *dL_dquats,
                               float *dL_dopacities, float *dL_dsh,
                               void *workspace, size_t workspace_bytes, const void *ckpt, size_t ckpt_bytes,
                               void *stream);

/* ---------------------------------------------------------------------------
 * Several views per launch
 *
 * On the Odin page each training view reads and updates only a sparse,
 * view-dependent subset of the primitives, held as that view's primitive
 * scope (axioms, first domain assumption), which its runtime checks before
 * overlapping views (central objects: read / update primitive scopes); the
 * Gaian page traces which points each pass reads or writes (methodology,
 * static access profiling). The calls below render V views of ONE
 * image size in one launch per phase instead of V: the parameters are read
 * once per Gaussian, the views' tile grids are stacked into one binning pass
 * (the view leads the sort key), and the chain rule sums the views' gradients
 * per Gaussian before writing them once.
 *
 * Layout: the same per-Gaussian arrays as the single-view calls, with a
 * leading view axis: means2d[V, n, 2], depths[V, n], conic_opacity[V, n, 4],
 * rgb[V, n, 3], radii[V, n], tiles_touched[V, n], clamped[V, n],
 * grad2d[V, n, GS_GRAD2D_STRIDE], dL_dmeans2d[V, n, 2]; images
 * image[V, 3, H, W], final_T[V, H, W], n_contrib[V, H, W], dL_dimage[V, 3, H, W].
 * Entry v n + g holds Gaussian g in view v; each view's values are those the
 * single-view call computes for that camera. The parameters and their
 * gradients keep their single-view shapes. Requires 1 <= V <= GS_MAX_VIEWS,
 * V n < 2^31, V times the tiles of one view <= 2^24, and every camera of one
 * width and height (GS_ERR_INVALID_ARG otherwise, naming the camera).
 * ------------------------------------------------------------------------ */
#define GS_MAX_VIEWS 32

/* gs_preprocess for V cameras (host array cams[V]). vis_mask (nullable) gets
 * one word per Gaussian: bit v set iff it is drawn in view v (radius > 0), the
 * per-view scope of the Gaussian. */
gs_status gs_preprocess_views(const gs_camera *cams, int32_t n_views, const gs_options *opt, int64_t n,
                              const float *means, const float *scales, const float *quats,
                              const float *opacities, const float *sh,
                              float *means2d, float *depths, float *conic_opacity, float *rgb,
                              int32_t *radii, uint32_t *tiles_touched, uint8_t *clamped, uint32_t *vis_mask,
                              void *stream);

/* Workspace bytes gs_bin_sort_views needs. */
size_t gs_bin_sort_views_workspace_size(int32_t n_views, int64_t n, int64_t pair_capacity, int32_t width,
                                        int32_t height);

/* gs_bin_sort over all V views at once. The views' grids of TX x TY tiles are
 * stacked: tile t of view v has the id v TX TY + t, so the key
 * (id << 32) | depth bits orders the pairs by view, then tile, then depth,
 * then entry index; the value is the entry index v n + g. ranges[V TX TY, 2].
 * View v's part of the result is the single-view result for that camera
 * with its values offset by v n and its ranges by the pairs of views < v. */
gs_status gs_bin_sort_views(const gs_camera *cams, int32_t n_views, const gs_options *opt, int64_t n,
                            const float *means2d, const float *depths, const int32_t *radii,
                            const uint32_t *tiles_touched, void *workspace, size_t workspace_bytes,
                            int64_t pair_capacity, uint64_t *keys, uint32_t *values, uint32_t *ranges,
                            int64_t *n_pairs, void *stream);

/* gs_render_fwd of all V views, one launch, on the output of gs_bin_sort_views. */
gs_status gs_render_fwd_views(const gs_camera *cams, int32_t n_views, const gs_options *opt, int64_t n,
                              const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                              const float *means2d, const float *conic_opacity, const float *rgb,
                              float *image, float *final_T, uint32_t *n_contrib, void *stream);

/* gs_render_bwd_raster of all V views: per entry v n + g, the pixel sums of
 * view v, ADDED into grad2d[V, n, GS_GRAD2D_STRIDE] (zeroed by the caller). */
gs_status gs_render_bwd_raster_views(const gs_camera *cams, int32_t n_views, const gs_options *opt, int64_t n,
                                     const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                                     const float *means2d, const float *conic_opacity, const float *rgb,
                                     const float *final_T, const uint32_t *n_contrib, const float *dL_dimage,
                                     float *grad2d, void *stream);

/* gs_preprocess_bwd of all V views: each Gaussian's gradient is the sum over
 * the views that drew it, added once into (or with overwrite_grads = 1
 * written as) the parameter gradients; dL_dmeans2d (nullable) gets each
 * view's dL/d(u, v) at entry v n + g. stats (nullable) takes every drawn view
 * as one call of gs_preprocess_bwd would (count += the number of such views).
 * Equal to V single-view calls up to the order of the summation. */
gs_status gs_preprocess_bwd_views(const gs_camera *cams, int32_t n_views, const gs_options *opt, int64_t n,
                                  const float *means, const float *scales, const float *quats, const float *sh,
                                  const float *conic_opacity, const int32_t *radii, const uint8_t *clamped,
                                  const float *grad2d, float *dL_dmeans, float *dL_dscales, float *dL_dquats,
                                  float *dL_dopacities, float *dL_dsh, float *dL_dmeans2d,
                                  const gs_densify_stats *stats, void *stream);

/* ---------------------------------------------------------------------------
 * Optimizer update (phase U)
 * ------------------------------------------------------------------------ */

/*
 * gs_adam_step -- one Adam update of every Gaussian's raw parameters, fused
 * with the activation chain and a per-Gaussian gradient magnitude.
 *
 * The Odin page names the phase (Fig. 7 caption: U, the optimizer update) and
 * the optimizer (Adam, referee report, major comment 1), and reads a
 * per-primitive gradient magnitude from a post-backward hook (same comment).
 * Raw parameters (the five arrays of `params`, in this order):
 *   means[n,3]; log_scales[n,3] (scales = exp); quats[n,4] (normalised inside
 *   the rasterizer); opacity_logits[n] (opacities = sigmoid); sh[n,sh_rows,3].
 * grads[5] are the rasterizer's gradients, in the same order and layouts, with
 * respect to the ACTIVATED scales and opacities (as gs_render_bwd writes
 * them); the call chains them to the raw ones with the parameters' values
 * before the update: g_log_scale = g_scale * exp(log_scale),
 * g_logit = g_opacity * sigmoid(logit) * (1 - sigmoid(logit)).
 * Per raw scalar p with raw gradient g, at step t = opt->step (>= 1):
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2;
 *   p -= lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps),
 * with lr by group: means, log-scales, quaternions, opacity logits, SH row 0
 * (colour DC) and SH rows >= 1. exp_avg[5] and exp_avg_sq[5] hold m and v in
 * the parameters' layouts (zeros before the first step).
 * out: params, exp_avg, exp_avg_sq updated in place; scales[n,3] =
 *      exp(new log_scales) and opacities[n] = sigmoid(new logits), the next
 *      forward's inputs; grad_norm[n] (nullable) = the L2 norm of each
 *      Gaussian's raw gradient (all its 11 + 3 sh_rows scalars).
 * Every pointer is 16-byte aligned; the arrays of different roles do not
 * overlap. Deterministic except for the summation order of grad_norm.
 */
typedef struct gs_adam_options {
    float lr_means, lr_scales, lr_quats, lr_opacity, lr_sh_dc, lr_sh_rest;
    float beta1, beta2, eps; /* beta in [0, 1), eps >= 0 */
    int32_t step;            /* t >= 1: this update's index */
} gs_adam_options;

gs_status gs_adam_step(const gs_adam_options *opt, int64_t n, int32_t sh_rows, float *const params[5],
                       const float *const grads[5], float *const exp_avg[5], float *const exp_avg_sq[5],
                       float *scales, float *opacities, float *grad_norm, void *stream);

/* ---------------------------------------------------------------------------
 * Measurement helpers (used by the benchmark to set the kernels against the
 * chip's measured limits; not part of the rasterizer).
 * ------------------------------------------------------------------------ */

/* Streaming read of `bytes` from src (summed into *sink, 1 float) -- HBM read rate. */
/* gs_render_bwd_raster of one view with the wave reduction taken out: each
 * lane adds its own pixel's nine terms with its own fp32 atomics (about 9 per
 * blended pixel-entry), the per-pixel pattern whose atomics the DISTWAR page
 * (abstract) finds to flood the L2 atomic units. Same arguments and result as
 * gs_render_bwd_raster, up to summation order; for timing the two against
 * each other only. lane_hist (nullable, 65 uint32 counters, added to) gets,
 * per (wave, list entry) step that some pixel blends, one count at the number
 * of the wave's lanes that update that Gaussian together (the page observes
 * that a warp's lanes mostly hit the same address, in varying numbers). */
gs_status gs_mb_render_bwd_naive(const gs_camera *cam, const gs_options *opt, int64_t n,
                                 const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                                 const float *means2d, const float *conic_opacity, const float *rgb,
                                 const float *final_T, const uint32_t *n_contrib, const float *dL_dimage,
                                 float *grad2d, uint32_t *lane_hist, void *stream);

/* gs_render_bwd_raster of one view with the forward's checkpoints (grids of
 * 4096..32767 tiles), switching per (wave, list entry) between the wave
 * reduction and direct atomics by the number of lanes that blend the entry:
 * at most direct_max (0..64) lanes add their own terms with their own fp32
 * atomics, more reduce over the wave first. The adaptive scheme of the ARC
 * page ("ARC: Warp-level Adaptive Atomic Reduction in GPUs to Accelerate
 * Differentiable Rendering", title and abstract); direct_max = 0 is the
 * reduced backward. Same arguments and result as gs_render_bwd_raster, up to
 * summation order; GS_ERR_UNSUPPORTED without checkpoints. For timing only. */
gs_status gs_mb_render_bwd_adaptive(const gs_camera *cam, const gs_options *opt, int64_t n,
                                    const uint32_t *ranges, const uint32_t *values, int64_t n_pairs,
                                    const float *means2d, const float *conic_opacity, const float *rgb,
                                    const float *final_T, const uint32_t *n_contrib, const float *dL_dimage,
                                    float *grad2d, const void *ckpt, size_t ckpt_bytes, int32_t direct_max,
                                    void *stream);

/* The work of one view's blending, counted with the forward's own decisions
 * (one wave per tile, 4 pixels per lane), ADDED to counts[7] (u64):
 *   [0] E_f: entries each pixel evaluates (up to and including the one that
 *       stops it, else its tile's whole list); [1] those the forward evaluates
 *       (passing its 16x4 row band's bound); [2] blended (pixel, entry) pairs;
 *   [3] E_b = sum of n_contrib; [4] P_c: (tile, entry) pairs with a blended
 *       pixel; [5] (4x16 column strip, entry) pairs with a blended pixel (the
 *       backward's executed strip-steps, 64 lanes each); [6] sum over tiles
 *       of the deepest n_contrib. Inputs as gs_render_fwd; nothing else
 *       written. */
gs_status gs_mb_render_counts(const gs_camera *cam, const gs_options *opt, const uint32_t *ranges,
                              const uint32_t *values, int64_t n_pairs, const float *means2d,
                              const float *conic_opacity, const float *rgb, uint64_t *counts, void *stream);
gs_status gs_mb_hbm_read(const void *src, size_t bytes, float *sink, void *stream);
/* Copy `bytes` from src to dst -- HBM copy rate; also the reference kernel for
 * scaling rocprof FETCH_SIZE / WRITE_SIZE counters. */
gs_status gs_mb_hbm_copy(void *dst, const void *src, size_t bytes, void *stream);
/* n_ops no-return fp32 atomic adds into records[n_records, 12] with the pattern
 * of the backward's flush: `lanes_per_record` consecutive lanes add to the
 * consecutive values of one record; records are chosen by a hash of the
 * operation index (n_records = 1 gives a single hot record). */
gs_status gs_mb_atomic(float *records, int64_t n_records, int64_t n_ops, int32_t lanes_per_record,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GSPLAT_H */
