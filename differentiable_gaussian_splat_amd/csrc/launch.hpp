// Host-side launchers of the rasterizer's kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace gs {

hipError_t launch_preprocess(const DevCam& cam, int K, int sh_rows, float lowpass, float near_plane, int n,
                             const float* means, const float* scales, const float* quats, const float* opac,
                             const float* sh, float* means2d, float* depths, float* conic_op, float* rgb,
                             int* radii, uint32_t* tiles, uint8_t* clamped, hipStream_t stream);

hipError_t launch_preprocess_bwd(const DevCam& cam, int K, int sh_rows, float lowpass, float near_plane, int n,
                                 const float* means, const float* scales, const float* quats, const float* sh,
                                 const float* conic_op, const int* radii, const uint8_t* clamped,
                                 const float* grad2d, float* d_means, float* d_scales, float* d_quats,
                                 float* d_opac, float* d_sh, float* d_means2d, hipStream_t stream);

// Binning. The workspace layout is computed by bin_layout (binsort.hip).
struct BinLayout {
    size_t dkeys[2], didx[2];  // depth-sort ping-pong (n entries each)
    size_t offsets;            // per-sorted-Gaussian first pair index (n + 1)
    size_t partials;           // u64 scan partials
    size_t hist;               // radix histograms
    size_t counters;           // u64 [0] visible count, [1] and [2] pair count
    size_t chunk_counts;       // chunked placement: [chunk][tile] counts, then bases
    size_t seg;                // chunked placement: [segment][tile] sums, then bases
    size_t tile_total;         // chunked placement: pairs per tile
    size_t tkeys[2];           // radix path: pair tile-key ping-pong (capacity each)
    size_t tvals;              // radix path: pair value scratch (capacity)
    size_t total;
};
BinLayout bin_layout(int64_t n, int64_t capacity, int TX, int TY);

// Phase 1 (no host dependence): pair count P (copied to *host_P, pinned, with
// `ev` recorded after the copy), visible compaction, depth sort and
// per-Gaussian first pair index.
hipError_t launch_bin_count(int n, const float* depths, const uint32_t* tiles_touched, char* ws, const BinLayout& L,
                            unsigned long long* host_P, hipEvent_t ev, hipStream_t stream);
// Phase 2 (P known on the host and within capacity): ranges, then the tile
// sort of the generated pairs into `values` (and the 64-bit keys if non-NULL).
hipError_t launch_bin_emit(int n, int P, int TX, int TY, const float* means2d, const int* radii,
                           const float* depths, char* ws, const BinLayout& L, uint64_t* keys,
                           uint32_t* values, uint32_t* ranges, hipStream_t stream);

hipError_t launch_fill_u32(uint32_t* p, size_t count, uint32_t value, hipStream_t stream);

hipError_t launch_render_fwd(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                             const float* means2d, const float* conic_op, const float* rgb, const float* bg,
                             float* image, float* final_T, uint32_t* n_contrib, hipStream_t stream);

hipError_t launch_render_bwd(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                             const float* means2d, const float* conic_op, const float* rgb, const float* bg,
                             const float* final_T, const uint32_t* n_contrib, const float* dL_dimage,
                             float* grad2d, hipStream_t stream);

hipError_t launch_mb_read(const void* src, size_t bytes, float* sink, hipStream_t stream);
hipError_t launch_mb_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_mb_atomic(float* records, int64_t n_records, int64_t n_ops, int lanes, hipStream_t stream);

}  // namespace gs
