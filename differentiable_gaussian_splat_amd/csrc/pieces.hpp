// Render checkpoints and the work of one wave of the pieces backward, shared
// by the rasterizers of 3D Gaussians (render.hip) and of surfels (surfel.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gs {

// Render checkpoints (one view's tile grid, written by the forward): for each
// tile, the forward's per-pixel state (T, C) after list entries CKPT_EVERY k - 1,
// k = 1..CKPT_SLOTS, then the pixel's final colour: (CKPT_SLOTS + 1) x 256
// float4 per tile, pixel (row r, column c) of the tile at float4 16 r + c of a
// slot. A slot is written only when the tile's band wave walks past its entry;
// the backward reads only such slots. After all tiles' slots, one uint4 per
// tile: each row band's walk (its deepest blended entry), always written.
constexpr int PIECES_CHUNK = 1024;         // tiles per dispatch chunk of the 3D pieces backward
constexpr int SURFEL_PIECES_CHUNK = 2048;  // and of the surfel one
constexpr int CKPT_EVERY = 256;
constexpr int CKPT_SLOTS = 4;

// One wave of the pieces backward: tile `tile`, list entries [lo, hi) of the
// row bands set in `sel`, starting from checkpoint slot ck (null: from the
// final state) with ck_end the tile's final-colour slot; bw holds the tile's
// row bands' walks.
struct PieceWork {
    int tile, lo, hi;
    uint32_t sel;
    const float4* ck;
    const float4* ck_end;
    uint4 bw;
};

// Block b of a pieces launch ((CKPT_SLOTS + 2) chunk blocks per chunk of
// `chunk` tiles): false when it has no work. A tile gets one wave per
// piece of CKPT_EVERY entries, each piece starting from the checkpoint after
// its last entry; a walk past the last checkpoint ends in a tail piece from
// the final state that two waves share by row bands (0-1 and 2-3). Dispatch
// order, chunk by chunk: the chunk's later waves (most return at once), then
// its first pieces, so that a deep tile's pieces start together and the first
// pieces of the early chunks do not wait behind every tile's later waves.
__device__ __forceinline__ bool piece_work(int b, int ntiles, int chunk, const float4* __restrict__ ckpt,
                                           const uint2* __restrict__ ranges, PieceWork& pw) {
    constexpr int PIECES = CKPT_SLOTS + 1;  // slots in the checkpoint buffer per tile
    constexpr int WAVES = CKPT_SLOTS + 2;   // waves per tile
    const int cb = b / (WAVES * chunk), r = b - cb * WAVES * chunk;
    const int t0 = cb * chunk, tn = min(chunk, ntiles - t0);
    if (r >= WAVES * tn) return false;  // past the last tile
    int w, tile;
    if (r < (WAVES - 1) * tn) {
        w = 1 + r / tn;
        tile = t0 + r % tn;
    } else {
        w = 0;
        tile = t0 + r - (WAVES - 1) * tn;
    }
    // the tile's walk, from its row bands' walks the forward left after the checkpoints, at most
    // the list's length
    const uint4 bw = reinterpret_cast<const uint4*>(ckpt + (size_t)ntiles * PIECES * 256)[tile];
    const uint2 rg = ranges[tile];
    const uint32_t walk = min(max(max(bw.x, bw.y), max(bw.z, bw.w)), rg.y - rg.x);
    const int need = (int)((walk + CKPT_EVERY - 1) / CKPT_EVERY);
    const bool deep = need > PIECES;
    int piece = w;
    uint32_t sel = 0xFu;
    if (deep) {
        if (w >= CKPT_SLOTS) {  // the tail, bands 0-1 or 2-3
            piece = CKPT_SLOTS;
            sel = w == CKPT_SLOTS ? 0x3u : 0xCu;
        }
    } else if (w >= max(need, 1)) {
        return false;
    }
    const int pieces = deep ? PIECES : need;
    const bool tail = piece >= pieces - 1;  // the last piece walks to the end from the final state
    const float4* tck = ckpt + (size_t)tile * PIECES * 256;
    pw.tile = tile;
    pw.lo = piece * CKPT_EVERY;
    pw.hi = tail ? INT32_MAX : pw.lo + CKPT_EVERY;
    pw.sel = sel;
    pw.ck = tail ? nullptr : tck + (size_t)piece * 256;
    pw.ck_end = tck + CKPT_SLOTS * 256;
    pw.bw = bw;
    return true;
}

}  // namespace gs
