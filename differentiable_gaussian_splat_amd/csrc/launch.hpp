// Host-side launchers of the rasterizer's kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"
#include "pieces.hpp"

namespace gs {

hipError_t launch_preprocess(const DevCam& cam, int K, int sh_rows, float lowpass, float near_plane, int n,
                             const float* means, const float* scales, const float* quats, const float* opac,
                             const float* sh, float* means2d, float* depths, float* conic_op, float* rgb,
                             int* radii, uint32_t* tiles, uint8_t* clamped, hipStream_t stream);

// Densification statistics (all null: none).
struct DensifyStats {
    float* grad_accum;
    int32_t* count;
    int32_t* max_radius;
};

hipError_t launch_preprocess_bwd(const DevCam& cam, int K, int sh_rows, float lowpass, float near_plane, int n,
                                 const float* means, const float* scales, const float* quats, const float* sh,
                                 const float* conic_op, const int* radii, const uint8_t* clamped,
                                 const float* grad2d, float* d_means, float* d_scales, float* d_quats,
                                 float* d_opac, float* d_sh, float* d_means2d, bool overwrite,
                                 const DensifyStats& stats, hipStream_t stream);

// 2D Gaussian surfels: projection (scales [n, 2]; tf [n, 12] = three float4 per
// surfel: (M row 0, opacity), (M row 1, c_x), (M row 2, c_y)), and the chain rule
// from the per-surfel pixel sums grad [n, 16].
hipError_t launch_surfel_preprocess(const DevCam& cam, int K, int sh_rows, float near_plane, int n,
                                    const float* means, const float* scales, const float* quats, const float* opac,
                                    const float* sh, float* means2d, float* depths, float* tf, float* rgb,
                                    int* radii, uint32_t* tiles, uint8_t* clamped, hipStream_t stream);
hipError_t launch_surfel_preprocess_bwd(const DevCam& cam, int K, int sh_rows, int n, const float* means,
                                        const float* scales, const float* quats, const float* sh, const float* tf,
                                        const int* radii, const uint8_t* clamped, const float* grad, float* d_means,
                                        float* d_scales, float* d_quats, float* d_opac, float* d_sh, bool overwrite,
                                        hipStream_t stream);
// ckpt (nullable, render_ckpt_bytes(TX, TY) bytes): render checkpoints, as for
// 3D Gaussians (written by the forward, read by the backward).
hipError_t launch_surfel_render_fwd(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                                    const float* tf, const float* rgb, const float* bg, float* image, float* final_T,
                                    uint32_t* n_contrib, float* ckpt, hipStream_t stream);
hipError_t launch_surfel_render_bwd(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                                    const float* tf, const float* rgb, const float* bg, const float* final_T,
                                    const uint32_t* n_contrib, const float* dL_dimage, float* grad, const float* ckpt,
                                    hipStream_t stream);
constexpr int SURFEL_GRAD_STRIDE = 16;  // floats per surfel record of pixel sums


// The same for V views of one image size (per-view arrays of V x n entries).
hipError_t launch_preprocess_views(const CamSet& cams, int V, int K, int sh_rows, float lowpass, float near_plane,
                                   int n, const float* means, const float* scales, const float* quats,
                                   const float* opac, const float* sh, float* means2d, float* depths,
                                   float* conic_op, float* rgb, int* radii, uint32_t* tiles, uint8_t* clamped,
                                   uint32_t* vis_mask, hipStream_t stream);
hipError_t launch_preprocess_bwd_views(const CamSet& cams, int V, int K, int sh_rows, float lowpass, float near_plane,
                                       int n, const float* means, const float* scales, const float* quats,
                                       const float* sh, const float* conic_op, const int* radii,
                                       const uint8_t* clamped, const float* grad2d, float* d_means, float* d_scales,
                                       float* d_quats, float* d_opac, float* d_sh, float* d_means2d, bool overwrite,
                                       const DensifyStats& stats, hipStream_t stream);

// Binning. The workspace layout is computed by bin_layout (binsort.hip).
struct BinLayout {
    size_t dkeys[2], didx[2];  // depth-sort ping-pong (n entries each)
    size_t rec;                // per depth-sorted Gaussian: uint4 record (n)
    size_t crec;               // per visible Gaussian in index order: the same record (n)
    size_t skey[2], sval[2];   // super-tile entries (super-tile id; Gaussian, clipped rectangle), ping-pong (capacity each)
    size_t sranges;            // per super-tile entry range
    size_t pfirst;             // per super-tile first piece
    size_t counts;             // per piece and tile: count, then offset within the tile's run
    size_t pinfo;              // per piece: super-tile, first entry, end entry
    size_t tile_total;         // pairs per tile
    size_t partials;           // u64 scan partials
    size_t pair_part;          // u64 per-block partial pair counts
    size_t fine;               // per row of SB depth-sorted Gaussians: the sum of their super-tile counts
    size_t hist;               // radix histograms
    size_t counters;           // u64 counters
    size_t total;
};
BinLayout bin_layout(int64_t n, int64_t capacity, int TX, int TY);

// Phase 1 (no host dependence): pair count P and super-tile entry count P1
// (written by a kernel to mapped_counts[0..1], the device address of pinned
// host-coherent memory, with `ev` recorded after that kernel),
// visible compaction, depth sort and the per-Gaussian records. n entries; for
// several views, nper entries per view and views stacked in a grid of TX x
// (views * TYv) tiles (nper = 0: one view of TX x TYv tiles).
hipError_t launch_bin_count(int n, int nper, int TX, int TYv, const float* means2d, const int* radii,
                            const float* depths, const uint32_t* tiles_touched, char* ws, const BinLayout& L,
                            unsigned long long* mapped_counts, hipEvent_t ev, hipStream_t stream);
// Phase 2 (P, P1 known on the host, P within capacity): the pairs in (tile,
// depth, index) order into `values` (and the 64-bit keys if non-NULL, their
// depth bits read from `depths`), and ranges; TY is the whole (stacked)
// grid's tile rows.
hipError_t launch_bin_emit(int n, int P, int P1, int TX, int TY, const float* depths, char* ws, const BinLayout& L,
                           uint64_t* keys, uint32_t* values, uint32_t* ranges, hipStream_t stream);

hipError_t launch_fill_u32(uint32_t* p, size_t count, uint32_t value, hipStream_t stream);

// Blending of `views` views of W x H pixels (TX x TY tiles each) whose tile
// lists are binned in one stacked grid; per-view images follow one another.
// ckpt (nullable, render_ckpt_bytes(TX, TY) bytes): the forward's per-tile
// checkpoints, which the backward of a one-view launch reads to cut deep tiles
// into pieces; both ignore it where the backward's layout does not use it.
size_t render_ckpt_bytes(int TX, int TY);
hipError_t launch_render_fwd(int views, int W, int H, int TX, int TY, const uint32_t* ranges,
                             const uint32_t* values, const float* means2d, const float* conic_op, const float* rgb,
                             const float* bg, float* image, float* final_T, uint32_t* n_contrib, float* ckpt,
                             hipStream_t stream);

hipError_t launch_render_bwd(int views, int W, int H, int TX, int TY, const uint32_t* ranges,
                             const uint32_t* values, const float* means2d, const float* conic_op, const float* rgb,
                             const float* bg, const float* final_T, const uint32_t* n_contrib,
                             const float* dL_dimage, float* grad2d, const float* ckpt, hipStream_t stream);

// The backward raster with per-pixel atomics (no wave reduction), one view: measurement only.
// lane_hist (nullable, 65 counters): per (wave, entry) step, the count of lanes updating the Gaussian.
// The pieces backward (one view with checkpoints, grids of 4096..32767 tiles),
// reducing an entry over the wave only when more than direct_max lanes blend
// it (hipErrorInvalidValue for other grids or without checkpoints).
hipError_t launch_render_bwd_adaptive(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                                      const float* means2d, const float* conic_op, const float* rgb, const float* bg,
                                      const float* final_T, const uint32_t* n_contrib, const float* dL_dimage,
                                      float* grad2d, const float* ckpt, int direct_max, hipStream_t stream);
hipError_t launch_render_bwd_naive(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                                   const float* means2d, const float* conic_op, const float* rgb, const float* bg,
                                   const float* final_T, const uint32_t* n_contrib, const float* dL_dimage,
                                   float* grad2d, uint32_t* lane_hist, hipStream_t stream);

hipError_t launch_render_counts(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                               const float* means2d, const float* conic_op, const float* rgb,
                               unsigned long long* counts, hipStream_t stream);
hipError_t launch_mb_read(const void* src, size_t bytes, float* sink, hipStream_t stream);
hipError_t launch_mb_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_mb_atomic(float* records, int64_t n_records, int64_t n_ops, int lanes, hipStream_t stream);

// Learning rates of the optimizer's parameter groups.
struct AdamLr {
    float means, scales, quats, opacity, sh_dc, sh_rest;
};

hipError_t launch_adam_step(const AdamLr& lr, float beta1, float beta2, float eps, int step, int n, int sh_rows,
                            float* const params[5], const float* const grads[5], float* const m[5],
                            float* const v[5], float* scales, float* opacities, float* grad_norm,
                            hipStream_t stream);

}  // namespace gs
