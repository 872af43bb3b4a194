// Per-tile alpha blending, forward and backward.
//
// Work layout (CDNA4, wave64): the 16x16 pixels of a tile are split into bands
// of 16 columns x 4 PPL rows, one 64-lane wave per band, each lane owning the
// PPL pixels (px, py0 + 4k), k < PPL, of one column of its band. A wave walks
// its tile's depth-sorted list on its own: it stages the records through LDS
// 64 at a time (each lane gathers one) and every lane reads each record by
// LDS broadcast. A band stops as soon as its own pixels are done, so a deep
// corner of a tile no longer holds the whole tile's pixels.
//
// Backward. The DISTWAR page ("DISTWAR: Fast Differentiable Rendering on
// Raster-based Rendering Pipelines", abstract) and the ARC page ("ARC:
// Warp-level Adaptive Atomic Reduction in GPUs to Accelerate Differentiable
// Rendering", abstract) find this step bound by atomic updates that flood the
// L2 atomic units, because all lanes of a warp update the same Gaussian. Here
// each lane first sums its pixels' terms in registers, each 16-lane row then
// reduces them with DPP (a reduce-scatter: 8 values land in 8 lanes), the row
// partials of a 64-record batch meet in LDS, and the batch is flushed with all
// lanes active: one fp32 atomic add per value per (band, Gaussian), 9
// consecutive lanes per Gaussian record.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace gs {

namespace {

constexpr int BATCH = 64;  // records staged per LDS batch

static_assert(CKPT_EVERY % BATCH == 0, "checkpoints fall on batch ends");

// A staged record: (w0, dy0, a2, beta), (g2, log2 o, r, g), b. One LDS
// address serves all three reads.
struct alignas(16) Staged {
    float4 a;
    float4 b;
    float4 c;  // (b, -, -, -)
};

// Tiles differ in depth by up to ~6x the mean, and the deepest band's wave
// alone takes most of the kernel's time while it shares its SIMD with light
// ones. Waves with long walks get a higher issue priority on their SIMD
// (s_setprio: arbitration among the SIMD's waves only), so they finish early
// while the light bands fill the other SIMDs.
__device__ __forceinline__ void set_walk_priority(uint32_t walk) {
    if (walk >= 512u) __builtin_amdgcn_s_setprio(3);
    else if (walk >= 256u) __builtin_amdgcn_s_setprio(2);
    else if (walk >= 128u) __builtin_amdgcn_s_setprio(1);
}

// True when no pixel centre of the band [x_lo, x_hi] x [y_lo, y_hi] can reach
// alpha >= 1/255 for this record: with the conic's smaller eigenvalue lmin,
// Q(d) >= lmin |d|^2 >= lmin dist(mean, band)^2, and alpha >= 1/255 needs
// Q <= 2 ln(255 o). The margins (0.1% and 1e-3) lie far above fp32 rounding,
// so a skipped record is one the per-pixel test would skip too: results are
// unchanged, only the per-pixel work for such records is saved.
struct MissTest {
    float lmin, qthr;
    __device__ __forceinline__ MissTest(float4 c, float lo) {
        const float a = c.x, beta = c.y, gamma = c.z;  // Q = a (dx + beta dy)^2 + gamma dy^2
        const float m11 = a * beta * beta + gamma;
        const float tr = a + m11, det = a * gamma;
        const float h = 0.5f * tr;
        const float lmax = h + sqrtf(fmaxf(h * h - det, 0.f));
        lmin = det / lmax;
        // 2 ln(255 o) = 2 ln 2 (log2 o + log2 255)
        qthr = 1.3862943611198906f * (lo + 7.9943534368588578f) + 1e-3f;
    }
    __device__ __forceinline__ bool misses(float u, float v, float x_lo, float x_hi, float y_lo, float y_hi) const {
        const float ddx = fmaxf(0.f, fmaxf(x_lo - u, u - x_hi));
        const float ddy = fmaxf(0.f, fmaxf(y_lo - v, v - y_hi));
        return lmin * (ddx * ddx + ddy * ddy) * 0.999f > qthr;
    }
};

__device__ __forceinline__ bool band_misses(float u, float v, float4 c, float lo, float x_lo, float x_hi, float y_lo,
                                            float y_hi) {
    return MissTest(c, lo).misses(u, v, x_lo, x_hi, y_lo, y_hi);
}

// The forward's staged record: a2 and the colour, then for each of the band's
// 4 rows the row's w at the tile's first column, wrow = beta ly + w0, and its
// exponent term et = g2 dy^2 + log2 o (dy = dy0 + ly), each rounded as the
// backward forms them (fp32, one fma each). A pixel then needs
// w = wrow + lx and the exponent a2 w^2 + et.
struct alignas(16) RowStaged {
    float4 k;       // (a2, r, g, b)
    float2 row[4];  // (wrow, et) per row
    uint32_t pos;   // the entry's position in the tile's list, counted from 1
};

// Forms the staged record of Gaussian g for the 4 rows ly = y0 .. y0 + 3 of a
// band (ly counted from the tile's first row); w0 and dy0, w and dy at the
// tile's first pixel centre (ox, oy), are formed in double and rounded once.
// Returns whether the record misses the band (see band_misses); clamp tells
// whether its alpha may reach the 0.99 clamp.
__device__ __forceinline__ bool form_record_rows(uint32_t g, const float2* __restrict__ means2d,
                                                 const float4* __restrict__ conic_op,
                                                 const float* __restrict__ rgb, RowStaged& rec, bool& clamp,
                                                 double ox, double oy, float y0, float x_lo, float x_hi, float y_lo,
                                                 float y_hi) {
    const float2 m = means2d[g];
    const float4 c = conic_op[g];
    const float4 k = falloff_consts(c);
    const double ddy = oy - (double)m.y;
    const float w0 = (float)((ox - (double)m.x) + (double)c.y * ddy), dy0 = (float)ddy;
    const float r = rgb[3 * (size_t)g], gg = rgb[3 * (size_t)g + 1], bb = rgb[3 * (size_t)g + 2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float ly = y0 + (float)i;
        float wrow, et;
        {
#pragma clang fp contract(off)
            wrow = __fmaf_rn(k.y, ly, w0);
            const float dy = dy0 + ly;
            const float gdy = k.z * dy;
            et = __fmaf_rn(gdy, dy, k.w);
        }
        rec.row[i] = make_float2(wrow, et);
    }
    rec.k = make_float4(k.x, r, gg, bb);
    clamp = c.w > CLAMP_FREE_OPACITY;
    return band_misses(m.x, m.y, c, k.w, x_lo, x_hi, y_lo, y_hi);
}

// The backward's staging: as stage_record, but returns a mask of the PPL row
// bands of the tile (rows [4k, 4k + 4)) the record may reach; bit k is also
// clear when the record lies at or past every blended entry of band k
// (pos >= band_last[k]).
template <int PPL>
__device__ __forceinline__ uint32_t stage_record_bands(uint32_t g, uint32_t pos, const uint32_t* band_last,
                                                       const float2* __restrict__ means2d,
                                                       const float4* __restrict__ conic_op,
                                                       const float* __restrict__ rgb, Staged* s_rec, int lane,
                                                       double ox, double oy, float x_lo,
                                                       float x_hi, float y_lo) {
    const float2 m = means2d[g];
    const float4 c = conic_op[g];
    const float4 k = falloff_consts(c);
    const double ddy = oy - (double)m.y;
    const double w0 = (ox - (double)m.x) + (double)c.y * ddy;
    s_rec[lane].a = make_float4((float)w0, (float)ddy, k.x, k.y);
    s_rec[lane].b = make_float4(k.z, k.w, rgb[3 * (size_t)g], rgb[3 * (size_t)g + 1]);
    s_rec[lane].c.x = rgb[3 * (size_t)g + 2];
    const MissTest mt(c, k.w);
    uint32_t mask = 0u;
#pragma unroll
    for (int b = 0; b < PPL; ++b) {
        const float y0 = y_lo + 4.f * b;
        if (pos < band_last[b] && !mt.misses(m.x, m.y, x_lo, x_hi, y0, y0 + 3.f)) mask |= 1u << b;
    }
    return mask;
}

// The backward's staging: as stage_record, but returns a mask of the wave's PPL
// column strips (strip s = columns [4 s, 4 s + 4) of the tile, all 16 rows;
// the wave's k-th strip is s = strip0 + k) the record may reach; bit k is also
// clear when the record lies at or past every blended entry of strip k
// (pos >= strip_last[k]). Bit 4 is set when the record's alpha may sit at the
// clamp (opacity above CLAMP_FREE_OPACITY); below, alpha = o G never reaches it.
template <int PPL>
__device__ __forceinline__ uint32_t stage_record_strips(uint32_t g, uint32_t pos, const uint32_t* strip_last,
                                                        const float2* __restrict__ means2d,
                                                        const float4* __restrict__ conic_op,
                                                        const float* __restrict__ rgb, Staged* s_rec, int lane,
                                                        double ox, double oy, float x_lo, float y_lo, float y_hi,
                                                        int strip0) {
    const float2 m = means2d[g];
    const float4 c = conic_op[g];
    const float4 k = falloff_consts(c);
    const double ddy = oy - (double)m.y;
    const double w0 = (ox - (double)m.x) + (double)c.y * ddy;
    s_rec[lane].a = make_float4((float)w0, (float)ddy, k.x, k.y);
    s_rec[lane].b = make_float4(k.z, k.w, rgb[3 * (size_t)g], rgb[3 * (size_t)g + 1]);
    s_rec[lane].c.x = rgb[3 * (size_t)g + 2];
    const MissTest mt(c, k.w);
    uint32_t mask = c.w > CLAMP_FREE_OPACITY ? 16u : 0u;
#pragma unroll
    for (int b = 0; b < PPL; ++b) {
        const float x0 = x_lo + 4.f * (float)(strip0 + b);
        if (pos < strip_last[b] && !mt.misses(m.x, m.y, x0, x0 + 3.f, y_lo, y_hi)) mask |= 1u << b;
    }
    return mask;
}

// Forward. Per pixel: alpha = min(0.99, o G); entries with alpha < 1/255 are
// skipped; an entry that would take T below 1e-4 is not blended and ends the
// pixel; otherwise C += rgb alpha T and T -= alpha T. L is 1 while the pixel
// walks and 0 once it has stopped (or lies outside the image): a stopped
// pixel's effective alpha is 0, which changes nothing, and its T (>= 1e-4)
// can never trigger the stop test again.

template <int PPL>
__global__ __launch_bounds__(64) void k_render_fwd(int W, int H, int TX, int TY, int ntiles,
                                                 const uint2* __restrict__ ranges,
                                                 const uint32_t* __restrict__ values,
                                                 const float2* __restrict__ means2d,
                                                 const float4* __restrict__ conic_op, const float* __restrict__ rgb,
                                                 float bg0, float bg1, float bg2, float* __restrict__ image,
                                                 float* __restrict__ final_T, uint32_t* __restrict__ n_contrib,
                                                 float4* __restrict__ ckpt) {
    static_assert(PPL == 1, "one band of 16x4 pixels per wave");
    __shared__ RowStaged s_rec[BATCH];
    // Workgroups go to the 8 XCDs round-robin by index (b -> XCD b % 8). Tile
    // 8q + x takes workgroups 32q + 8 band + x, so its four band waves, which
    // stage the same records, share XCD x and its L2.
    const int b = blockIdx.x;
    const int tile = ((b >> 5) << 3) + (b & 7), band = (b >> 3) & 3;
    if (tile >= ntiles) return;
    int tx, ty;
    const size_t view_px = view_of_tile(tile, TX, TY, tx, ty) * (size_t)W * H;
    image += 3 * view_px;
    final_T += view_px;
    n_contrib += view_px;
    const int lane = threadIdx.x;
    const int row = lane >> 4;  // the lane's row of the band
    const int px = tx * TILE + (lane & 15);
    const int py = ty * TILE + band * 4 + row;
    const double ox = (double)(tx * TILE) + 0.5, oy = (double)(ty * TILE) + 0.5;  // the tile's first pixel centre
    const float lx = (float)(lane & 15);                                         // this lane's offset from it
    float T = 1.f, C0 = 0.f, C1 = 0.f, C2 = 0.f;
    // an entry blends where alpha >= thr: ALPHA_MIN while the pixel walks, above any alpha (2) once it has
    // stopped (or lies outside the image), so that a stopped pixel's alpha counts as 0 and its T (>= T_MIN)
    // never triggers the stop test again
    float thr = (px < W && py < H) ? ALPHA_MIN : 2.f;
    uint32_t last = 0u;
    // pixel-centre rectangle of the band
    const float bx_lo = (float)(tx * TILE) + 0.5f, bx_hi = bx_lo + 15.f;
    const float by_lo = (float)(ty * TILE + band * 4) + 0.5f, by_hi = by_lo + 3.f;
    auto walking = [&]() { return __any(thr < 1.f); };
    const uint2 rg = ranges[tile];
    bool wrote_ckpt = false;
    for (uint32_t bs = rg.x; bs < rg.y; bs += BATCH) {
        if (!walking()) break;
        set_walk_priority(bs - rg.x);  // a wave still walking deep into its list is a heavy one
        const uint32_t idx = bs + lane;
        bool miss = true, clamp = false;
        RowStaged rec;
        if (idx < rg.y)
            miss = form_record_rows(values[idx], means2d, conic_op, rgb, rec, clamp, ox, oy, (float)(band * 4),
                                    bx_lo, bx_hi, by_lo, by_hi);
        // the records some pixel of the band may blend, packed in list order: the walk below then reads
        // consecutive slots at fixed offsets from one base per run, with each entry's list position
        // (counted from 1) beside it
        const uint64_t keep = __ballot(!miss);
        const int cnt = __popcll(keep);
        if (!miss) {
            const int slot = __builtin_amdgcn_mbcnt_hi((uint32_t)(keep >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)keep, 0u));
            rec.pos = bs - rg.x + 1 + (uint32_t)lane;
            s_rec[slot] = rec;
        }
        __syncthreads();
        // entries in runs of 8 (unrolled, one exit test each), the band's walk checked between runs; a batch
        // none of whose records can reach the alpha clamp takes a copy without the clamp's min
        auto walk_runs = [&](auto clamp_tag) {
            constexpr bool CLAMP = decltype(clamp_tag)::value;
            for (int m0 = 0; m0 < cnt; m0 += 8) {
                // the run's base offset is held in a vector register (opaque to the compiler), so that every
                // read of the run addresses from it with a constant offset instead of re-forming it per entry
                uint32_t run_off = (uint32_t)m0 * (uint32_t)sizeof(RowStaged);
                asm volatile("" : "+v"(run_off));
                const RowStaged* run =
                    reinterpret_cast<const RowStaged*>(reinterpret_cast<const char*>(s_rec) + run_off);
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    if (m0 + m >= cnt) break;
                    const float4 K = run[m].k;
                    const float2 R = run[m].row[row];
                    const uint32_t pos = run[m].pos;
                    float q;
                    {
#pragma clang fp contract(off)
                        const float w = R.x + lx;
                        const float aw = K.x * w;
                        q = __fmaf_rn(aw, w, R.y);
                    }
                    const float oG = __builtin_amdgcn_exp2f(q);
                    const float al = CLAMP ? fminf(ALPHA_MAX, oG) : oG;
                    // the entry passes the alpha test; it blends unless it would take T below T_MIN, which
                    // ends the pixel instead
                    const bool pass = al >= thr;
                    const float Tn = __fmaf_rn(-al, T, T);
                    const bool stop = pass && Tn < T_MIN;
                    const bool blend = pass && !stop;
                    thr = stop ? 2.f : thr;
                    const float wt = blend ? al * T : 0.f;
                    C0 = fmaf(K.y, wt, C0);
                    C1 = fmaf(K.z, wt, C1);
                    C2 = fmaf(K.w, wt, C2);
                    T = blend ? Tn : T;
                    last = blend ? pos : last;
                    asm volatile("" : "+v"(last) : "v"(pos));  // pos is read with the record, not under the mask
                }
                if (!walking()) break;
            }
        };
        if (__ballot(!miss && clamp)) walk_runs(std::true_type{});
        else walk_runs(std::false_type{});
        __syncthreads();
        if (ckpt) {
            // the state after a whole batch that ends a checkpoint interval, while still walking
            const uint32_t done = bs - rg.x + BATCH;
            if (bs + BATCH <= rg.y && done % CKPT_EVERY == 0 && done / CKPT_EVERY <= CKPT_SLOTS && walking()) {
                ckpt[((size_t)tile * (CKPT_SLOTS + 1) + done / CKPT_EVERY - 1) * 256 + band * 64 + lane] =
                    make_float4(T, C0, C1, C2);
                wrote_ckpt = true;
            }
        }
    }
    if (wrote_ckpt)  // the final colour, beside the checkpoints
        ckpt[((size_t)tile * (CKPT_SLOTS + 1) + CKPT_SLOTS) * 256 + band * 64 + lane] = make_float4(C0, C1, C2, T);
    if (ckpt) {  // the band's walk, for the backward's choice of pieces
        const uint32_t bw = wave_max_u32(last);
        if (lane == 0)
            reinterpret_cast<uint32_t*>(ckpt + (size_t)ntiles * (CKPT_SLOTS + 1) * 256)[4 * tile + band] = bw;
    }
    const size_t HW = (size_t)W * H;
    if (px < W && py < H) {
        const size_t p = (size_t)py * W + px;
        image[p] = fmaf(T, bg0, C0);
        image[HW + p] = fmaf(T, bg1, C1);
        image[2 * HW + p] = fmaf(T, bg2, C2);
        final_T[p] = T;
        n_contrib[p] = last;
    }
}

// Backward: the forward's blended entries in reverse, per pixel. T is
// restored entry by entry (T in front = T behind / (1 - alpha)); S = A . dL/dC
// with A the colour behind the current entry (starting as the background), so
// dL/dalpha = T (rgb . dL/dC - S).
// NAIVE (measurement only, PPL = 1): every lane adds its own pixel's terms
// with its own atomics, the per-pixel pattern the DISTWAR and ARC pages
// measure, instead of reducing over the wave first. ADAPT (measurement only):
// per entry, the wave reduces only when more than direct_max of its lanes
// blend; otherwise those lanes add their terms directly (the switch between
// reduction and direct atomics by the number of lanes that the ARC page's
// title names).
// LDS of one backward wave: a batch of staged records, their Gaussians, the
// per-row partial sums and which entries some pixel blended.
template <int NB>
struct BwdShared {
    Staged rec[NB];
    uint32_t g[NB];
    float part[NB * 4 * GRAD2D_N];  // [entry][row of 16 lanes][value]
    uint32_t has[NB];
};

// The backward of one wave: strip group `band` (of 4 / PPL) of tile `tile`.
// Lane l owns the pixels of tile row r = l / 4 at columns 4 s + l % 4 of its
// PPL column strips s = band PPL + k (strip s: columns [4 s, 4 s + 4), all 16
// rows), so a lane's pixels share one row: dy and its exponent term are
// formed once per entry, and the moments with dy factor out of the pixel loop
// (sum h w dy = dy sum h w, sum h dy^2 = dy^2 sum h, sum h dy = dy sum h).
// Only the strips set in band_sel are walked, and only list entries
// [walk_lo, walk_hi). A pixel whose row band (rows [4 b, 4 b + 4)) blends
// nothing at or past walk_hi in the forward (rb_walk, the forward's walk of
// each row band) starts from the final state (T = final_T, colour behind =
// background); the others start from the forward's checkpoint `ck` after
// entry walk_hi - 1 (T there, and the colour behind it,
// (C_final - C there + final_T bg) / T), with ck_end holding C_final; a
// checkpoint slot holds pixel (r, c) at float4 16 r + c. ck is null when
// walk_hi is past the walk.
template <int PPL, int NB, bool NAIVE, bool ADAPT = false>
__device__ __forceinline__ void bwd_walk(int tile, int band, uint32_t band_sel, int walk_lo, int walk_hi,
                                         const float4* __restrict__ ck, const float4* __restrict__ ck_end,
                                         uint4 rb_walk, int W, int H, int TX, int TY,
                                         const uint2* __restrict__ ranges, const uint32_t* __restrict__ values,
                                         const float2* __restrict__ means2d, const float4* __restrict__ conic_op,
                                         const float* __restrict__ rgb, float bg0, float bg1, float bg2,
                                         const float* __restrict__ final_T, const uint32_t* __restrict__ n_contrib,
                                         const float* __restrict__ dL_dimage, float* __restrict__ grad2d,
                                         uint32_t* __restrict__ lane_hist, BwdShared<NB>& sh, int direct_max = -1) {
    Staged* s_rec = sh.rec;
    uint32_t* s_g = sh.g;
    float* s_part = sh.part;
    uint32_t* s_has = sh.has;
    int tx, ty;
    const size_t view_px = view_of_tile(tile, TX, TY, tx, ty) * (size_t)W * H;
    final_T += view_px;
    n_contrib += view_px;
    dL_dimage += 3 * view_px;
    const int lane = threadIdx.x;
    // lane roles in the in-row reduce-scatter (see row_reduce_scatter8)
    const int rl = lane & 15, row = lane >> 4;
    const bool c1 = ((rl ^ (rl >> 2)) & 1) != 0;
    const bool c2 = (((rl >> 1) ^ (rl >> 2)) & 1) != 0;
    const bool c3 = ((rl >> 2) & 1) != 0;
    const bool writer = rl < 9;
    const int slot = rl < 8 ? (c1 ? 4 : 0) + (c2 ? 2 : 0) + (c3 ? 1 : 0) : 8;
    const int r = lane >> 2, q = lane & 3;  // this lane's row in the tile, column within a strip
    const int strip0 = band * PPL;
    const int py = ty * TILE + r;
    const double ox = (double)(tx * TILE) + 0.5, oy = (double)(ty * TILE) + 0.5;  // the tile's first pixel centre
    const float ly = (float)r;                                                   // this lane's row offset
    const size_t HW = (size_t)W * H;
    const uint32_t rbw = (r >> 2) == 0 ? rb_walk.x : (r >> 2) == 1 ? rb_walk.y : (r >> 2) == 2 ? rb_walk.z : rb_walk.w;
    float lx[PPL], T[PPL], g0[PPL], g1[PPL], g2[PPL], S[PPL];
    uint32_t last[PPL], strip_last[PPL];
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
        const int col = 4 * (strip0 + k) + q;
        const int px = tx * TILE + col;
        lx[k] = (float)col;
        const bool in = px < W && py < H;
        const size_t p = in ? (size_t)py * W + px : 0;
        T[k] = in ? final_T[p] : 1.f;
        last[k] = in ? n_contrib[p] : 0u;
        g0[k] = in ? dL_dimage[p] : 0.f;
        g1[k] = in ? dL_dimage[HW + p] : 0.f;
        g2[k] = in ? dL_dimage[2 * HW + p] : 0.f;
        S[k] = fmaf(bg0, g0[k], fmaf(bg1, g1[k], bg2 * g2[k]));
        strip_last[k] = __builtin_amdgcn_readfirstlane(wave_max_u32(last[k]));  // deepest blended entry of strip k
        if (!((band_sel >> k) & 1u)) {  // strip k belongs to another wave: none of its entries is walked here
            strip_last[k] = 0u;
            last[k] = 0u;  // and its pixels blend nothing (the strip pass evaluates every strip)
        }
        if (ck && rbw > (uint32_t)walk_hi) {  // this pixel's row band walked past walk_hi in the forward
            const int lp = 16 * r + col;      // the pixel's float4 in a checkpoint slot
            const float4 c = ck[lp], e = ck_end[lp];
            const float behind = fmaf(g0[k], e.x - c.y, fmaf(g1[k], e.y - c.z, g2[k] * (e.z - c.w)));
            S[k] = in ? fmaf(T[k], S[k], behind) / c.x : 0.f;
            T[k] = in ? c.x : 1.f;
        }
    }
    uint32_t mylast = 0;
#pragma unroll
    for (int k = 0; k < PPL; ++k) mylast = max(mylast, strip_last[k]);
    const float bx_lo = (float)(tx * TILE) + 0.5f;
    const float by_lo = (float)(ty * TILE) + 0.5f;
    const uint2 rg = ranges[tile];
    // never walk past the tile's list, whatever n_contrib holds
    const uint32_t maxlast = min(min(mylast, rg.y - rg.x), (uint32_t)walk_hi);
    set_walk_priority(maxlast - min(maxlast, (uint32_t)walk_lo));
    for (int hi = (int)maxlast; hi > walk_lo; hi -= NB) {
        const int lo = max(walk_lo, hi - NB);
        const int cnt = hi - lo;
        uint32_t strips = 0u;
        if (lane < cnt) {
            const uint32_t g = values[rg.x + lo + lane];
            strips = stage_record_strips<PPL>(g, (uint32_t)(lo + lane), strip_last, means2d, conic_op, rgb, s_rec,
                                              lane, ox, oy, bx_lo, by_lo, by_lo + 15.f, strip0);
            s_g[lane] = g;
            s_has[lane] = 0u;
        }
        uint64_t todo = __ballot((strips & 0xFu) != 0u);  // records some strip may blend
        __syncthreads();
        while (todo) {
            const int j = 63 - __builtin_clzll(todo);  // backwards through the list
            todo &= ~(1ull << j);
            const uint32_t bm = __builtin_amdgcn_readlane(strips, j);  // bit 4: opacity above the clamp
            const float4 A = s_rec[j].a;
            const float4 B = s_rec[j].b;
            const float cb = s_rec[j].c.x;
            const uint32_t pos = (uint32_t)(lo + j);
            // this lane's row: dy and the exponent's dy term, as falloff() forms them
            const float dy = A.y + ly;
            float et, wrow;
            {
#pragma clang fp contract(off)
                const float gdy = B.x * dy;
                et = __fmaf_rn(gdy, dy, B.y);
                wrow = __fmaf_rn(A.w, ly, A.x);
            }
            float acc[GRAD2D_N];
#pragma unroll
            for (int c = 0; c < GRAD2D_N; ++c) acc[c] = 0.f;
            float Hs = 0.f, HW1 = 0.f, HW2 = 0.f;  // sums over this lane's pixels of h, h w, h w^2
            bool any = false, mine = false;
            // the strips' pixel work, in two versions: a record whose opacity is at most 0.99 never
            // reaches the alpha clamp (alpha = o G <= o), so it skips the clamp's min and test. All
            // strips go through it, even those the record cannot reach (their pixels fail the
            // alpha test and add zeros, exactly): the strips' chains are independent, so all their
            // tests go first and all their gradient terms after, without a branch between them,
            // which costs less than skipping the unreachable ones
            auto strips_pass = [&](auto clamp_tag) {
                constexpr bool CLAMP = decltype(clamp_tag)::value;
                // one pixel's blend test (the forward's own arithmetic on the same values)
                auto eval = [&](int k, float& w, float& oG, float& al) {
#pragma clang fp contract(off)
                    w = wrow + lx[k];
                    const float aw = A.z * w;
                    oG = __builtin_amdgcn_exp2f(__fmaf_rn(aw, w, et));
                    al = CLAMP ? fminf(ALPHA_MAX, oG) : oG;
                };
                // one pixel's gradient terms; a pixel that did not blend this entry takes alpha = 0,
                // which leaves its T, S and every sum unchanged
                auto grad = [&](int k, float w, float oG, float al, bool blended) {
                    const float av = blended ? al : 0.f;
                    T[k] = T[k] * __builtin_amdgcn_rcpf(1.0f - av);  // T in front of this entry
                    const float wt = av * T[k];
                    acc[0] = fmaf(wt, g0[k], acc[0]);
                    acc[1] = fmaf(wt, g1[k], acc[1]);
                    acc[2] = fmaf(wt, g2[k], acc[2]);
                    const float cdl = fmaf(B.z, g0[k], fmaf(B.w, g1[k], cb * g2[k]));
                    const float d = cdl - S[k];
                    S[k] = fmaf(av, d, S[k]);
                    // h = o G dL/dalpha = -2 dL/dQ = alpha T d where alpha = o G; zero where alpha
                    // sat at its 0.99 clamp (and wherever the pixel did not blend: wt = 0). The
                    // moments stay in (w, dy), the conic's own axes: sums in (dx, dy) would
                    // cancel for elongated Gaussians.
                    const float h = (!CLAMP || oG <= ALPHA_MAX) ? wt * d : 0.f;
                    const float hw = h * w;
                    Hs += h;
                    HW2 = fmaf(hw, w, HW2);
                    HW1 += hw;
                };
                float w[PPL], oG[PPL], al[PPL];
                bool bl[PPL], anyb = false;
#pragma unroll
                for (int k = 0; k < PPL; ++k) {
                    eval(k, w[k], oG[k], al[k]);
                    bl[k] = pos < last[k] && al[k] >= ALPHA_MIN;
                    anyb = anyb || bl[k];
                }
                if (!__any(anyb)) return;
                any = true;
                mine = mine || anyb;
#pragma unroll
                for (int k = 0; k < PPL; ++k) grad(k, w[k], oG[k], al[k], bl[k]);
            };
            if (bm & 16u) strips_pass(std::true_type{});
            else strips_pass(std::false_type{});
            if (!any) continue;
            const float hy = Hs * dy;
            acc[3] = Hs;
            acc[4] = HW2;
            acc[5] = HW1 * dy;
            acc[6] = hy * dy;
            acc[7] = HW1;
            acc[8] = hy;
            if (NAIVE) {
                if (mine) {
                    float* dst = grad2d + (size_t)s_g[j] * GRAD2D_STRIDE;
#pragma unroll
                    for (int c = 0; c < GRAD2D_N; ++c) atomicAdd(&dst[c], acc[c]);
                }
                // how many lanes of the wave update this Gaussian together (the whole wave votes)
                const uint64_t who = __ballot(mine);
                if (lane_hist && lane == 0) atomicAdd(&lane_hist[__popcll(who)], 1u);
                continue;
            }
            if (ADAPT) {
                // measurement: when at most direct_max lanes blend the entry, they add their own terms
                // with their own atomics instead of reducing over the wave first
                if (__popcll(__ballot(mine)) <= (uint32_t)direct_max) {
                    if (mine) {
                        float* dst = grad2d + (size_t)s_g[j] * GRAD2D_STRIDE;
#pragma unroll
                        for (int c = 0; c < GRAD2D_N; ++c) atomicAdd(&dst[c], acc[c]);
                    }
                    continue;
                }
            }
            // per 16-lane row: values 0..7 by reduce-scatter (lane slot holds one), value 8 by a row sum
            const float u = row_reduce_scatter8(acc, c1, c2, c3);
            const float x8 = row_sum16(acc[8]);
            if (writer) s_part[(j * 4 + row) * GRAD2D_N + slot] = rl < 8 ? u : x8;
            if (lane == 0) s_has[j] = 1u;
        }
        __syncthreads();
        // one atomic add per value per (wave, Gaussian): the 4 row partials summed here
        for (int v = lane; v < cnt * GRAD2D_N; v += 64) {
            const int e = v / GRAD2D_N;
            const int c = v - e * GRAD2D_N;
            if (s_has[e]) {
                const float* p = &s_part[e * 4 * GRAD2D_N + c];
                const float val = (p[0] + p[GRAD2D_N]) + (p[2 * GRAD2D_N] + p[3 * GRAD2D_N]);
                if (val != 0.f) atomicAdd(&grad2d[(size_t)s_g[e] * GRAD2D_STRIDE + c], val);
            }
        }
        __syncthreads();
    }
}

// One wave per band group: tile blockIdx.x / (4 / PPL), bands of PPL rows.
template <int PPL, int NB, bool NAIVE = false>
__global__ __launch_bounds__(64) void k_render_bwd(int W, int H, int TX, int TY, const uint2* __restrict__ ranges,
                                                 const uint32_t* __restrict__ values,
                                                 const float2* __restrict__ means2d,
                                                 const float4* __restrict__ conic_op, const float* __restrict__ rgb,
                                                 float bg0, float bg1, float bg2, const float* __restrict__ final_T,
                                                 const uint32_t* __restrict__ n_contrib,
                                                 const float* __restrict__ dL_dimage, float* __restrict__ grad2d,
                                                 uint32_t* __restrict__ lane_hist = nullptr) {
    constexpr int BANDS = 4 / PPL;
    __shared__ BwdShared<NB> sh;
    const int tile = blockIdx.x / BANDS, band = blockIdx.x - tile * BANDS;
    bwd_walk<PPL, NB, NAIVE>(tile, band, 0xFu, 0, INT32_MAX, nullptr, nullptr, make_uint4(0u, 0u, 0u, 0u), W, H, TX,
                             TY, ranges, values,
                             means2d, conic_op, rgb, bg0, bg1, bg2, final_T, n_contrib, dL_dimage, grad2d, lane_hist,
                             sh);
}

// Two waves per tile, the tile's walk deciding their roles. A wave walks its
// list serially, entry after entry, so a tile whose walk is many times the
// mean (a dense cluster) holds its SIMD long after the light tiles are done,
// with few waves left to hide its latencies. Tiles that walk at least
// `split_walk` entries go to both waves, each taking two of the four 16x4 row
// bands (half the pixel work per entry, at the price of a second reduction);
// the others stay with the first wave, four pixels per lane, and the second
// returns at once. Both roles run the same four-band code.
template <int NB>
__global__ __launch_bounds__(64) void k_render_bwd_split(int W, int H, int TX, int TY, int ntiles,
                                                       uint32_t split_walk, const uint2* __restrict__ ranges,
                                                       const uint32_t* __restrict__ values,
                                                       const float2* __restrict__ means2d,
                                                       const float4* __restrict__ conic_op,
                                                       const float* __restrict__ rgb, float bg0, float bg1, float bg2,
                                                       const float* __restrict__ final_T,
                                                       const uint32_t* __restrict__ n_contrib,
                                                       const float* __restrict__ dL_dimage,
                                                       float* __restrict__ grad2d) {
    __shared__ BwdShared<NB> sh;
    // Workgroups [0, ntiles) are the tiles' second waves (most return at once; a
    // split tile's starts walking right away), then [ntiles, 2 ntiles) their
    // first waves: one contiguous run of real work. (Interleaving a tile's
    // waves instead put the working ones on a fixed stride of the dispatch
    // order, which the hardware's round-robin placement mapped onto a fraction
    // of the CUs.)
    const int b = blockIdx.x;
    const int sub = b < ntiles ? 1 : 0, tile = b - (1 - sub) * ntiles;
    // the tile's walk: its deepest blended entry over all 256 pixels, at most the list's length
    int tx, ty;
    const uint32_t* nc = n_contrib + view_of_tile(tile, TX, TY, tx, ty) * (size_t)W * H;
    const int lane = threadIdx.x;
    const int px = tx * TILE + (lane & 15);
    uint32_t walk = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int py = ty * TILE + (lane >> 4) + 4 * k;
        if (px < W && py < H) walk = max(walk, nc[(size_t)py * W + px]);
    }
    const uint2 rg = ranges[tile];
    walk = min((uint32_t)__builtin_amdgcn_readfirstlane(wave_max_u32(walk)), rg.y - rg.x);
    const bool split = walk >= split_walk;
    if (!split && sub != 0) return;
    bwd_walk<4, NB, false>(tile, 0, split ? 3u << (2 * sub) : 0xFu, 0, INT32_MAX, nullptr, nullptr,
                           make_uint4(0u, 0u, 0u, 0u), W, H, TX, TY,
                           ranges, values, means2d, conic_op, rgb, bg0, bg1, bg2, final_T, n_contrib, dL_dimage,
                           grad2d, nullptr, sh);
}

// With the forward's checkpoints: a tile's walk is cut into pieces of
// CKPT_EVERY entries, one wave each, every wave over all four row bands. The
// piece [lo, hi) starts from the checkpoint after entry hi - 1, so the pieces
// are independent: a deep tile's walk is spread over several waves without the
// extra per-entry reductions of a split by bands. A walk longer than
// (CKPT_SLOTS + 1) pieces ends in a tail piece [CKPT_SLOTS CKPT_EVERY, walk)
// from the final state, which two waves share by row bands.
template <int NB, bool ADAPT = false>
__global__ __launch_bounds__(64) void k_render_bwd_pieces(int W, int H, int TX, int TY, int ntiles,
                                                        const float4* __restrict__ ckpt,
                                                        const uint2* __restrict__ ranges,
                                                        const uint32_t* __restrict__ values,
                                                        const float2* __restrict__ means2d,
                                                        const float4* __restrict__ conic_op,
                                                        const float* __restrict__ rgb, float bg0, float bg1, float bg2,
                                                        const float* __restrict__ final_T,
                                                        const uint32_t* __restrict__ n_contrib,
                                                        const float* __restrict__ dL_dimage,
                                                        float* __restrict__ grad2d, int direct_max = -1) {
    __shared__ BwdShared<NB> sh;
    // the pieces and their dispatch order: piece_work (chunks of PIECES_CHUNK tiles measured against
    // one chunk for the whole grid: 0.466 -> 0.451 ms on 1M Gaussians at 1080p, 0.572 -> 0.567 ms on
    // 20k large ones)
    PieceWork pw;
    if (!piece_work(blockIdx.x, ntiles, PIECES_CHUNK, ckpt, ranges, pw)) return;
    bwd_walk<4, NB, false, ADAPT>(pw.tile, 0, pw.sel, pw.lo, pw.hi, pw.ck, pw.ck_end, pw.bw, W, H, TX, TY, ranges,
                                  values, means2d, conic_op, rgb, bg0, bg1, bg2, final_T, n_contrib, dL_dimage, grad2d,
                                  nullptr, sh, direct_max);
}

// Measurement: the work of one view's blending, counted with the forward's own
// decisions (the same staged records and falloff). One wave per tile, four
// pixels per lane (rows lane / 16 + 4 k), walking the list front to back until
// every pixel has stopped. counts[] (u64, added):
//   0 E_f        entries each pixel evaluates: list positions up to and
//                including the one that stops it, else the whole list
//   1 E_f_kernel those the forward evaluates (the entry passes its row band's
//                eigenvalue bound)
//   2 E_blend    blended (pixel, entry) pairs
//   3 E_b        sum of n_contrib: entries each pixel's reverse walk passes
//   4 P_c        (tile, entry) pairs with at least one blended pixel
//   5 band_exec  (4x16 column strip, entry) pairs with at least one blended
//                pixel: what the backward executes, 64 lanes each
//   6 walked     sum over tiles of the deepest n_contrib (the backward's walk)
__global__ __launch_bounds__(64) void k_render_counts(int W, int H, int TX, int TY, int ntiles,
                                                     const uint2* __restrict__ ranges,
                                                     const uint32_t* __restrict__ values,
                                                     const float2* __restrict__ means2d,
                                                     const float4* __restrict__ conic_op,
                                                     const float* __restrict__ rgb,
                                                     unsigned long long* __restrict__ counts) {
    __shared__ Staged s_rec[BATCH];
    const int tile = blockIdx.x;
    if (tile >= ntiles) return;
    int tx, ty;
    view_of_tile(tile, TX, TY, tx, ty);
    const int lane = threadIdx.x;
    const int px = tx * TILE + (lane & 15);
    const double ox = (double)(tx * TILE) + 0.5, oy = (double)(ty * TILE) + 0.5;
    const float lx = (float)(lane & 15);
    float ly[4], T[4], L[4];
    uint32_t last[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = (lane >> 4) + 4 * k;
        ly[k] = (float)r;
        T[k] = 1.f;
        last[k] = 0u;
        L[k] = (px < W && ty * TILE + r < H) ? 1.f : 0.f;
    }
    const float bx_lo = (float)(tx * TILE) + 0.5f, bx_hi = bx_lo + 15.f;
    const float by_lo = (float)(ty * TILE) + 0.5f;
    const uint32_t no_last[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    unsigned long long ef = 0, efk = 0, eblend = 0, pc = 0, bandx = 0;
    const uint2 rg = ranges[tile];
    for (uint32_t bs = rg.x; bs < rg.y; bs += BATCH) {
        if (!__any(L[0] + L[1] + L[2] + L[3] != 0.f)) break;
        const uint32_t idx = bs + lane;
        uint32_t bands = 0u;
        if (idx < rg.y)
            bands = stage_record_bands<4>(values[idx], 0u, no_last, means2d, conic_op, rgb, s_rec, lane, ox, oy,
                                          bx_lo, bx_hi, by_lo);
        __syncthreads();
        const int cnt = (int)min((uint32_t)BATCH, rg.y - bs);
        for (int j = 0; j < cnt; ++j) {
            const uint32_t bm = __builtin_amdgcn_readlane(bands, j);
            const float4 A = s_rec[j].a;
            const float4 B = s_rec[j].b;
            const uint32_t pos = bs - rg.x + 1 + (uint32_t)j;
            bool mine = false;  // this lane blended the entry at one of its pixels
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                ef += L[k] != 0.f ? 1u : 0u;
                if (!((bm >> k) & 1u)) continue;
                efk += L[k] != 0.f ? 1u : 0u;
                float w;
                {
#pragma clang fp contract(off)
                    w = __fmaf_rn(A.w, ly[k], A.x) + lx;  // as the forward and backward form it
                }
                const float oG = falloff(w, A.y + ly[k], A.z, B.x, B.y);
                const float al = fminf(ALPHA_MAX, oG);
                float ae = (al >= ALPHA_MIN ? al : 0.f) * L[k];
                const bool stop = __fmaf_rn(-ae, T[k], T[k]) < T_MIN;
                L[k] = stop ? 0.f : L[k];
                ae = stop ? 0.f : ae;
                T[k] = __fmaf_rn(-ae, T[k], T[k]);
                const bool blended = ae > 0.f;
                last[k] = blended ? pos : last[k];
                eblend += blended ? 1u : 0u;
                mine = mine || blended;
            }
            // the backward's column strips (columns [4 s, 4 s + 4): lanes with (lane & 15) / 4 = s)
            const uint64_t who = __ballot(mine);
            if (who) {
                ++pc;
#pragma unroll
                for (int st = 0; st < 4; ++st) bandx += (who & (0x000F000F000F000Full << (4 * st))) ? 1u : 0u;
            }
        }
        __syncthreads();
    }
    // per pixel n_contrib, the tile's deepest, and the wave's totals
    unsigned long long eb = 0;
    uint32_t deepest = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        eb += last[k];
        deepest = max(deepest, last[k]);
    }
    deepest = wave_max_u32(deepest);
    const unsigned long long per[5] = {ef, efk, eblend, eb, 0ull};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        unsigned long long v = per[c];
        for (int off = 32; off > 0; off >>= 1) v += (unsigned long long)__shfl_xor((long long)v, off);
        if (lane == 0) atomicAdd(&counts[c], v);
    }
    if (lane == 0) {
        atomicAdd(&counts[4], pc);
        atomicAdd(&counts[5], bandx);
        atomicAdd(&counts[6], (unsigned long long)deepest);
    }
}

}  // namespace

// Measured on the contention scene (1M Gaussians, 1920x1080): the forward is
// fastest with one pixel per lane (four band waves per tile: a band stops on
// its own), the backward with four (one wave per tile: each band would add its
// own atomics and its own reductions) and 32-record batches (half the LDS,
// more resident waves). On small frames one wave per tile leaves most SIMDs
// idle, and the backward's per-wave walk time decides: there it splits a tile
// over two or four band waves (measured on a 128x128 frame, 64 tiles: 87 ->
// 42 us with four; 800x800, 2500 tiles: 247 -> 228 us with two). On one
// large frame a wave per tile leaves the deep tiles (a cluster's core walks
// ten times the median) running with few waves beside them at the end. With
// the forward's checkpoints a deep tile's walk is cut into pieces of 256
// entries, one wave each, and a walk past the fifth piece ends in a tail
// piece shared by two waves by row bands (k_render_bwd_pieces). Means over 100
// launches: 1M Gaussians at 1080p 0.505 -> 0.425 ms against the band split
// alone, 20k large Gaussians 0.593 -> 0.587 ms, 6M Gaussians seen by 16
// 1080p cameras one at a time 24.7 -> 21.8 ms. Checkpoints every 128 or 192
// entries were slower; 2, 6 or 10 checkpoint slots instead of 4 trade the 6M
// scene's deep walks (up to 10k entries: 23.1, 21.2, 18.7 ms) against the cost
// of every tile's extra waves (20k large Gaussians: 0.579, 0.604, 0.630 ms).
// Without checkpoints a tile walking 512 entries
// or more splits over two waves by row bands (k_render_bwd_split; from 256 or
// 384 entries, or into four waves, it was slower: each extra wave repeats the
// per-entry reduction). A launch of many views (16 x 8160 tiles in one) keeps
// every SIMD busy to the end without either, and there the band split only
// added work (0.515 -> 0.641 ms per view): from 32768 tiles on, one wave per
// tile.
constexpr int FWD_PPL = 1;
constexpr int BWD_BATCH = 32;
constexpr int PIECES_BATCH = 64;  // the pieces backward's batch (its walks are the deep ones)
constexpr uint32_t BWD_SPLIT_WALK = 512;

// Backward layouts by launch size (tiles over all views of the launch).
enum class BwdLayout { Bands1, Bands2, Split, Tile };
BwdLayout bwd_layout(int ntiles) {
    if (ntiles < 2048) return BwdLayout::Bands1;   // four band waves per tile
    if (ntiles < 4096) return BwdLayout::Bands2;   // two
    if (ntiles < 32768) return BwdLayout::Split;   // one, two for deep tiles
    return BwdLayout::Tile;                        // one
}

size_t render_ckpt_bytes(int TX, int TY) {
    const int ntiles = TX * TY;
    if (bwd_layout(ntiles) != BwdLayout::Split) return 0;
    return (size_t)ntiles * ((CKPT_SLOTS + 1) * 256 + 1) * sizeof(float4);
}

hipError_t launch_render_fwd(int views, int W, int H, int TX, int TY, const uint32_t* ranges,
                             const uint32_t* values, const float* means2d, const float* conic_op, const float* rgb,
                             const float* bg, float* image, float* final_T, uint32_t* n_contrib, float* ckpt,
                             hipStream_t stream) {
    const int ntiles = views * TX * TY;
    if (ntiles == 0) return hipSuccess;
    // checkpoints only where the backward reads them: one view, the split layout
    float4* ck = (views == 1 && bwd_layout(ntiles) == BwdLayout::Split) ? reinterpret_cast<float4*>(ckpt) : nullptr;
    k_render_fwd<FWD_PPL><<<32 * ((ntiles + 7) / 8), 64, 0, stream>>>(
        W, H, TX, TY, ntiles, reinterpret_cast<const uint2*>(ranges), values, reinterpret_cast<const float2*>(means2d),
        reinterpret_cast<const float4*>(conic_op), rgb, bg[0], bg[1], bg[2], image, final_T, n_contrib, ck);
    return hipGetLastError();
}

hipError_t launch_render_bwd(int views, int W, int H, int TX, int TY, const uint32_t* ranges,
                             const uint32_t* values, const float* means2d, const float* conic_op, const float* rgb,
                             const float* bg, const float* final_T, const uint32_t* n_contrib,
                             const float* dL_dimage, float* grad2d, const float* ckpt, hipStream_t stream) {
    const int ntiles = views * TX * TY;
    if (ntiles == 0) return hipSuccess;
    const uint2* rg = reinterpret_cast<const uint2*>(ranges);
    const float2* m2 = reinterpret_cast<const float2*>(means2d);
    const float4* co = reinterpret_cast<const float4*>(conic_op);
    if (ckpt && views == 1 && bwd_layout(ntiles) == BwdLayout::Split) {
        k_render_bwd_pieces<PIECES_BATCH><<<(CKPT_SLOTS + 2) * PIECES_CHUNK * ((ntiles + PIECES_CHUNK - 1) / PIECES_CHUNK),
                                         64, 0, stream>>>(
            W, H, TX, TY, ntiles, reinterpret_cast<const float4*>(ckpt), rg, values, m2, co, rgb, bg[0], bg[1], bg[2],
            final_T, n_contrib, dL_dimage, grad2d);
        return hipGetLastError();
    }
    switch (bwd_layout(ntiles)) {
        case BwdLayout::Bands1:
            k_render_bwd<1, BWD_BATCH><<<ntiles * 4, 64, 0, stream>>>(W, H, TX, TY, rg, values, m2, co, rgb, bg[0], bg[1],
                                                                     bg[2], final_T, n_contrib, dL_dimage, grad2d);
            break;
        case BwdLayout::Bands2:
            k_render_bwd<2, BWD_BATCH><<<ntiles * 2, 64, 0, stream>>>(W, H, TX, TY, rg, values, m2, co, rgb, bg[0], bg[1],
                                                                     bg[2], final_T, n_contrib, dL_dimage, grad2d);
            break;
        case BwdLayout::Split:
            k_render_bwd_split<BWD_BATCH><<<2 * ntiles, 64, 0, stream>>>(W, H, TX, TY, ntiles, BWD_SPLIT_WALK, rg,
                                                                        values, m2, co, rgb, bg[0], bg[1], bg[2],
                                                                        final_T, n_contrib, dL_dimage, grad2d);
            break;
        case BwdLayout::Tile:
            k_render_bwd<4, BWD_BATCH><<<ntiles, 64, 0, stream>>>(W, H, TX, TY, rg, values, m2, co, rgb, bg[0], bg[1],
                                                                 bg[2], final_T, n_contrib, dL_dimage, grad2d);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_render_bwd_adaptive(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                                      const float* means2d, const float* conic_op, const float* rgb, const float* bg,
                                      const float* final_T, const uint32_t* n_contrib, const float* dL_dimage,
                                      float* grad2d, const float* ckpt, int direct_max, hipStream_t stream) {
    const int ntiles = TX * TY;
    if (ntiles == 0) return hipSuccess;
    if (!ckpt || bwd_layout(ntiles) != BwdLayout::Split) return hipErrorInvalidValue;
    k_render_bwd_pieces<PIECES_BATCH, true>
        <<<(CKPT_SLOTS + 2) * PIECES_CHUNK * ((ntiles + PIECES_CHUNK - 1) / PIECES_CHUNK), 64, 0, stream>>>(
            W, H, TX, TY, ntiles, reinterpret_cast<const float4*>(ckpt), reinterpret_cast<const uint2*>(ranges), values,
            reinterpret_cast<const float2*>(means2d), reinterpret_cast<const float4*>(conic_op), rgb, bg[0], bg[1],
            bg[2], final_T, n_contrib, dL_dimage, grad2d, direct_max);
    return hipGetLastError();
}

hipError_t launch_render_counts(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                               const float* means2d, const float* conic_op, const float* rgb,
                               unsigned long long* counts, hipStream_t stream) {
    const int ntiles = TX * TY;
    if (ntiles == 0) return hipSuccess;
    k_render_counts<<<ntiles, 64, 0, stream>>>(W, H, TX, TY, ntiles, reinterpret_cast<const uint2*>(ranges), values,
                                               reinterpret_cast<const float2*>(means2d),
                                               reinterpret_cast<const float4*>(conic_op), rgb, counts);
    return hipGetLastError();
}

hipError_t launch_render_bwd_naive(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                                   const float* means2d, const float* conic_op, const float* rgb, const float* bg,
                                   const float* final_T, const uint32_t* n_contrib, const float* dL_dimage,
                                   float* grad2d, uint32_t* lane_hist, hipStream_t stream) {
    const int ntiles = TX * TY;
    if (ntiles == 0) return hipSuccess;
    k_render_bwd<1, BWD_BATCH, true><<<ntiles * 4, 64, 0, stream>>>(
        W, H, TX, TY, reinterpret_cast<const uint2*>(ranges), values, reinterpret_cast<const float2*>(means2d),
        reinterpret_cast<const float4*>(conic_op), rgb, bg[0], bg[1], bg[2], final_T, n_contrib, dL_dimage, grad2d,
        lane_hist);
    return hipGetLastError();
}

}  // namespace gs
