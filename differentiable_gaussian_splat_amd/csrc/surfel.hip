// Per-tile alpha blending of 2D Gaussian surfels (planar Gaussians), forward
// and backward: the second pipeline the Odin review page evaluates beside 3D
// Gaussian splatting (referee report summary), after "2D Gaussian Splatting
// for Geometrically Accurate Radiance Fields" in its references.
//
// A surfel reaches a pixel where the pixel's ray meets its plane. With the
// surfel's screen homography M (a surfel point (u, v) lands at the
// homogeneous screen point M (u, v, 1)), the rows give the two planes through
// the ray of pixel (x, y) in the surfel's own coordinates,
// h_x = M0 - x M2 and h_y = M1 - y M2, and their cross product k gives the hit
// (u, v) = (k0, k1) / k2. The falloff is exp(-rho / 2) with
// rho = min(u^2 + v^2, 2 |pixel - c|^2): the surfel's own Gaussian or a screen
// filter of variance 1/2 around the projected centre c, whichever is wider.
// Compositing (alpha = min(0.99, o G), the 1/255 skip, the 1e-4 stop) and the
// reverse blend are those of the 3D Gaussian kernels.
//
// The kernels expand the cross product: k = N01 + x N12 - y N02 with
// N01 = M0 x M1, N12 = M1 x M2, N02 = M0 x M2, taken about the projected
// centre c: k = Kc + dx N12 - dy N02 with Kc = N01 + c_x N12 - c_y N02 (formed
// per (tile, surfel) in double from the fp32 M and rounded once; its first two
// components vanish up to c's rounding, since the ray through c meets the
// surfel at its centre) and (dx, dy) = pixel - c, which the screen filter needs
// anyway. Each component of k is then one rounding of its value at c plus two
// multiply-adds scaled by the pixel's offset from c, so u and v carry errors
// of order 1e-7 of the offset in surfel units, also for a surfel of a fraction
// of a pixel seen from a tile corner 20 pixels away. (Forming h_x, h_y and
// their cross product in fp32, or expanding about the tile's corner, left
// errors of 1e-5 in alpha on such surfels.) The backward sums dL/dk,
// dx dL/dk and dy dL/dk per surfel; the chain rule turns them into dL/dN01,
// dL/dN12 = sum x dL/dk and dL/dN02 = -sum y dL/dk, and those into dL/dM.
//
// Layout as the 3D kernels: one 64-lane wave per 16x4 row band in the forward;
// in the backward one wave per tile (a lane's four pixels in one row, one in
// each 4-column strip) or, on small grids, one per strip, with the per-entry
// sums reduced over each 16-lane row by DPP before one atomic add per value
// per (tile or strip, surfel).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace gs {

namespace {

constexpr int FWD_BATCH = 64;
static_assert(CKPT_EVERY % FWD_BATCH == 0, "checkpoints fall on batch ends");
constexpr int BWD_BATCH = 32;

// (Kc, N12.x), (N12.y, N12.z, N02.x, N02.y), (N02.z, dx0, dy0, log2 o), (rgb, -),
// (dx0, dy0) = (ox, oy) - c at the tile's first pixel centre (ox, oy)
struct alignas(16) SurfelRec {
    float4 a, b, c, d;
};

__device__ __forceinline__ void cross_d(const double p[3], const double q[3], double o[3]) {
    o[0] = fma(p[1], q[2], -p[2] * q[1]);
    o[1] = fma(p[2], q[0], -p[0] * q[2]);
    o[2] = fma(p[0], q[1], -p[1] * q[0]);
}

// Returns the surfel's opacity.
__device__ __forceinline__ float stage_surfel(uint32_t g, const float4* __restrict__ tf, const float* __restrict__ rgb,
                                              SurfelRec& s, double ox, double oy) {
    const float4 r0 = tf[3 * (size_t)g], r1 = tf[3 * (size_t)g + 1], r2 = tf[3 * (size_t)g + 2];
    const double M0[3] = {r0.x, r0.y, r0.z}, M1[3] = {r1.x, r1.y, r1.z}, M2[3] = {r2.x, r2.y, r2.z};
    double N01[3], N12[3], N02[3];
    cross_d(M0, M1, N01);
    cross_d(M1, M2, N12);
    cross_d(M0, M2, N02);
    const double cx = r1.w, cy = r2.w;
    float Kc[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) Kc[j] = (float)fma(cx, N12[j], fma(-cy, N02[j], N01[j]));
    s.a = make_float4(Kc[0], Kc[1], Kc[2], (float)N12[0]);
    s.b = make_float4((float)N12[1], (float)N12[2], (float)N02[0], (float)N02[1]);
    s.c = make_float4((float)N02[2], (float)(ox - (double)r1.w), (float)(oy - (double)r2.w),
                      __builtin_amdgcn_logf(r0.w));
    s.d = make_float4(rgb[3 * (size_t)g], rgb[3 * (size_t)g + 1], rgb[3 * (size_t)g + 2], 0.f);
    return r0.w;
}

// Whether some pixel centre of a rectangle [x_lo, x_hi] x [y_lo, y_hi] may
// reach alpha >= 1/255 for this surfel (misses: certainly not) (M rows r0..r2 with o in r0.w and the
// projected centre c in (r1.w, r2.w)). alpha >= 1/255 needs rho <= qthr =
// 2 ln(255 o), so either the screen filter's 2 |pixel - c|^2 <= qthr, or the
// ray's hit on the plane within u^2 + v^2 <= qthr: its screen image is the
// conic with dual D = M diag(1, 1, -1/qthr) M^T, whose bounding box has, per
// axis, the tangent lines t = (D_a2 +- sqrt(D_a2^2 - D_aa D_22)) / D_22 (in
// double). qthr is enlarged by 0.1% + 1e-3 and the filter's bound shrunk by
// 0.1%, far above the fp32 rounding of the per-pixel test, so a record this
// skips is one the per-pixel test would skip too. A disc whose image is not a
// bounded ellipse (D_22 >= 0: it reaches the camera plane) is never skipped.
struct SurfelReach {
    float qthr, cx, cy;
    bool none;  // o below 1/255: no pixel reaches the threshold
    bool box;   // the own branch's image is bounded by [x0, x1] x [y0, y1]
    double x0, x1, y0, y1;
    __device__ __forceinline__ SurfelReach(float4 r0, float4 r1, float4 r2) {
        qthr = 1.3862943611198906f * (__builtin_amdgcn_logf(r0.w) + 7.9943534368588578f) * 1.001f + 1e-3f;
        none = !(qthr > 0.f);
        cx = r1.w;
        cy = r2.w;
        box = false;
        x0 = x1 = y0 = y1 = 0.0;
        if (none) return;
        const double M[9] = {r0.x, r0.y, r0.z, r1.x, r1.y, r1.z, r2.x, r2.y, r2.z};
        const double iq = 1.0 / (double)qthr;
        auto dual = [&](int i, int j) {
            return fma(M[3 * i], M[3 * j], fma(M[3 * i + 1], M[3 * j + 1], -M[3 * i + 2] * M[3 * j + 2] * iq));
        };
        const double D22 = dual(2, 2);
        if (!(D22 < 0.0)) return;
        double t[4];
#pragma unroll
        for (int ax = 0; ax < 2; ++ax) {
            const double A = dual(ax, ax), B = dual(ax, 2);
            const double disc = fma(B, B, -A * D22);
            if (!(disc >= 0.0)) return;
            const double sq = sqrt(disc);
            t[2 * ax] = (B + sq) / D22;  // D22 < 0: the lower tangent
            t[2 * ax + 1] = (B - sq) / D22;
        }
        box = true;
        x0 = t[0] - 0.01;
        x1 = t[1] + 0.01;
        y0 = t[2] - 0.01;
        y1 = t[3] + 0.01;
    }
    __device__ __forceinline__ bool misses(float x_lo, float x_hi, float y_lo, float y_hi) const {
        if (none) return true;
        const float ddx = fmaxf(0.f, fmaxf(x_lo - cx, cx - x_hi)), ddy = fmaxf(0.f, fmaxf(y_lo - cy, cy - y_hi));
        if (2.f * (ddx * ddx + ddy * ddy) * 0.999f <= qthr) return false;  // the filter may reach the rectangle
        if (!box) return false;
        return x1 < (double)x_lo || x0 > (double)x_hi || y1 < (double)y_lo || y0 > (double)y_hi;
    }
};

// One (pixel, surfel) evaluation at offset (lx, ly) from the tile's first
// pixel centre, in two parts: the terms that depend only on the row
// (surfel_row_terms: dy, k_j before its column term, dy^2), formed once for
// the pixels of a row, and the rest (surfel_hit_in_row). The forward stages
// the same row terms and takes the same fp32 steps (contraction fixed), so
// the forward and the backward take the same decisions bit for bit.
struct SurfelHit {
    float inv, u, v, rho3, dx, dy, oG;
    bool own;  // the surfel's own falloff is the wider one
};

struct SurfelRowTerms {
    float dy, r0, r1, r2, dy2;
};
__device__ __forceinline__ SurfelRowTerms surfel_row_terms(const SurfelRec& s, float ly) {
#pragma clang fp contract(off)
    SurfelRowTerms t;
    t.dy = s.c.z + ly;
    t.r0 = __fmaf_rn(-t.dy, s.b.z, s.a.x);
    t.r1 = __fmaf_rn(-t.dy, s.b.w, s.a.y);
    t.r2 = __fmaf_rn(-t.dy, s.c.x, s.a.z);
    t.dy2 = t.dy * t.dy;
    return t;
}
__device__ __forceinline__ void surfel_hit_in_row(const SurfelRec& s, const SurfelRowTerms& t, float lx, SurfelHit& e) {
#pragma clang fp contract(off)
    e.dx = s.c.y + lx;
    e.dy = t.dy;
    const float k0 = __fmaf_rn(e.dx, s.a.w, t.r0);
    const float k1 = __fmaf_rn(e.dx, s.b.x, t.r1);
    const float k2 = __fmaf_rn(e.dx, s.b.y, t.r2);
    e.inv = __builtin_amdgcn_rcpf(k2);
    e.u = k0 * e.inv;
    e.v = k1 * e.inv;
    e.rho3 = __fmaf_rn(e.u, e.u, e.v * e.v);
    const float rho2 = 2.f * __fmaf_rn(e.dx, e.dx, t.dy2);
    e.own = e.rho3 <= rho2;
    const float rho = e.own ? e.rho3 : rho2;
    e.oG = __builtin_amdgcn_exp2f(__fmaf_rn(rho, NEG_HALF_LOG2E, s.c.w));
}

// The forward's staged surfel: per row of its band the terms of the hit that
// depend only on the row, (k_j at the row's first column before the column
// term, dy^2, as surfel_row_terms), then (N12, dx0), (log2 o, rgb) and the
// entry's list position. surfel_hit_row with them takes the same fp32 steps
// as surfel_hit_in_row, so the forward's decisions are the backward's bit for
// bit.
struct alignas(16) SurfelRowRec {
    float4 row[4];
    float4 n;
    float4 e;
    uint32_t pos;
};

__device__ __forceinline__ void surfel_row_rec(const SurfelRec& s, float ly0, SurfelRowRec& r) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float dy = s.c.z + (ly0 + (float)i);
        r.row[i] = make_float4(__fmaf_rn(-dy, s.b.z, s.a.x), __fmaf_rn(-dy, s.b.w, s.a.y),
                               __fmaf_rn(-dy, s.c.x, s.a.z), dy * dy);
    }
    r.n = make_float4(s.a.w, s.b.x, s.b.y, s.c.y);
    r.e = make_float4(s.c.w, s.d.x, s.d.y, s.d.z);
}

// The hit's alpha at column lx of a row (surfel_hit_in_row's): K = (k_j at
// the row, dy^2), N = (N12, dx0).
__device__ __forceinline__ float surfel_hit_row(float4 K, float4 N, float lo, float lx) {
#pragma clang fp contract(off)
    const float dx = N.w + lx;
    const float k0 = __fmaf_rn(dx, N.x, K.x);
    const float k1 = __fmaf_rn(dx, N.y, K.y);
    const float k2 = __fmaf_rn(dx, N.z, K.z);
    const float inv = __builtin_amdgcn_rcpf(k2);
    const float u = k0 * inv, v = k1 * inv;
    const float rho3 = __fmaf_rn(u, u, v * v);
    const float rho2 = 2.f * __fmaf_rn(dx, dx, K.w);
    const float rho = rho3 <= rho2 ? rho3 : rho2;
    return __builtin_amdgcn_exp2f(__fmaf_rn(rho, NEG_HALF_LOG2E, lo));
}

// Forward: four waves per tile, one per 16x4 band, one pixel per lane
// (tile 8q + x on workgroups 32q + 8 band + x: its four bands share XCD x).
// ckpt (nullable): the render checkpoints (layout beside CKPT_EVERY), for the
// backward's pieces.
__global__ __launch_bounds__(64) void k_surfel_fwd(int W, int H, int TX, int ntiles, const uint2* __restrict__ ranges,
                                                 const uint32_t* __restrict__ values, const float4* __restrict__ tf,
                                                 const float* __restrict__ rgb, float bg0, float bg1, float bg2,
                                                 float* __restrict__ image, float* __restrict__ final_T,
                                                 uint32_t* __restrict__ n_contrib, float4* __restrict__ ckpt) {
    __shared__ SurfelRowRec s_rec[FWD_BATCH];
    const int b = blockIdx.x;
    const int tile = ((b >> 5) << 3) + (b & 7), band = (b >> 3) & 3;
    if (tile >= ntiles) return;
    const int ty = tile / TX, tx = tile - ty * TX;
    const int lane = threadIdx.x;
    const int px = tx * TILE + (lane & 15), py = ty * TILE + band * 4 + (lane >> 4);
    const double ox = (double)(tx * TILE) + 0.5, oy = (double)(ty * TILE) + 0.5;
    const float lx = (float)(lane & 15);
    const int row = lane >> 4;  // the lane's row of the band
    float T = 1.f, C0 = 0.f, C1 = 0.f, C2 = 0.f;
    // an entry blends where alpha >= thr: ALPHA_MIN while the pixel walks, 2 (above any alpha) once it has
    // stopped or lies outside the image
    float thr = (px < W && py < H) ? ALPHA_MIN : 2.f;
    uint32_t last = 0u;
    // pixel-centre rectangle of the band
    const float bx_lo = (float)(tx * TILE) + 0.5f, bx_hi = bx_lo + 15.f;
    const float by_lo = (float)(ty * TILE + band * 4) + 0.5f, by_hi = by_lo + 3.f;
    const uint2 rg = ranges[tile];
    bool wrote_ckpt = false;
    for (uint32_t bs = rg.x; bs < rg.y; bs += FWD_BATCH) {
        if (!__any(thr < 1.f)) break;
        const uint32_t idx = bs + lane;
        bool miss = true, clamp = false;
        SurfelRowRec rec;
        if (idx < rg.y) {
            const uint32_t g = values[idx];
            SurfelRec full;
            clamp = stage_surfel(g, tf, rgb, full, ox, oy) > CLAMP_FREE_OPACITY;
            surfel_row_rec(full, (float)(band * 4), rec);
            miss = SurfelReach(tf[3 * (size_t)g], tf[3 * (size_t)g + 1], tf[3 * (size_t)g + 2])
                       .misses(bx_lo, bx_hi, by_lo, by_hi);
        }
        // the records some pixel of the band may blend, packed in list order, each with its list position
        // (counted from 1) in its last word: the walk reads each run of eight at constant offsets from one base
        const uint64_t keep = __ballot(!miss);
        const int cnt = __popcll(keep);
        if (!miss) {
            rec.pos = bs - rg.x + 1 + (uint32_t)lane;
            s_rec[__builtin_amdgcn_mbcnt_hi((uint32_t)(keep >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)keep, 0u))] =
                rec;
        }
        const bool clamp_batch = __ballot(!miss && clamp) != 0ull;
        __syncthreads();
        // entries in runs of 8 (unrolled, one exit test each), the walk test between runs; a batch none of
        // whose kept records has an opacity above CLAMP_FREE_OPACITY never reaches the alpha clamp (o G <= o)
        // and takes a copy without the clamp's min
        auto walk_runs = [&](auto clamp_tag) {
            constexpr bool CLAMP = decltype(clamp_tag)::value;
            for (int m0 = 0; m0 < cnt; m0 += 8) {
                uint32_t run_off = (uint32_t)m0 * (uint32_t)sizeof(SurfelRowRec);
                asm volatile("" : "+v"(run_off));  // one base register per run (opaque to the compiler)
                const SurfelRowRec* run =
                    reinterpret_cast<const SurfelRowRec*>(reinterpret_cast<const char*>(s_rec) + run_off);
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    if (m0 + m >= cnt) break;
                    const float4 D = run[m].e;  // (log2 o, rgb)
                    const float oG = surfel_hit_row(run[m].row[row], run[m].n, D.x, lx);
                    const uint32_t pos = run[m].pos;
                    const float al = CLAMP ? fminf(ALPHA_MAX, oG) : oG;
                    const bool pass = al >= thr;
                    const float Tn = __fmaf_rn(-al, T, T);
                    const bool stop = pass && Tn < T_MIN;  // the entry would end the pixel: not blended
                    const bool blend = pass && !stop;
                    thr = stop ? 2.f : thr;
                    const float wt = blend ? al * T : 0.f;
                    C0 = fmaf(D.y, wt, C0);
                    C1 = fmaf(D.z, wt, C1);
                    C2 = fmaf(D.w, wt, C2);
                    T = blend ? Tn : T;
                    last = blend ? pos : last;
                    asm volatile("" : "+v"(last) : "v"(pos));  // pos is read with the record, not under the mask
                }
                if (!__any(thr < 1.f)) break;
            }
        };
        if (clamp_batch) walk_runs(std::true_type{});
        else walk_runs(std::false_type{});
        __syncthreads();
        if (ckpt) {
            // the state after a whole batch that ends a checkpoint interval, while still walking
            const uint32_t done = bs - rg.x + FWD_BATCH;
            if (bs + FWD_BATCH <= rg.y && done % CKPT_EVERY == 0 && done / CKPT_EVERY <= CKPT_SLOTS &&
                __any(thr < 1.f)) {
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
    if (px < W && py < H) {
        const size_t HW = (size_t)W * H, p = (size_t)py * W + px;
        image[p] = fmaf(T, bg0, C0);
        image[HW + p] = fmaf(T, bg1, C1);
        image[2 * HW + p] = fmaf(T, bg2, C2);
        final_T[p] = T;
        n_contrib[p] = last;
    }
}

template <int NB>
struct SurfelBwdShared {
    SurfelRec rec[NB];
    uint32_t g[NB];
    float part[NB * 4 * SURFEL_GRAD_STRIDE];  // [entry][row of 16 lanes][value]
    uint32_t has[NB];
};

// Backward: the forward's blended entries in reverse per pixel (T restored as
// T / (1 - alpha), S = the colour behind . dL/dC). Lane l owns the pixels of
// tile row r = l / 4 at columns 4 s + l % 4 of its PPL column strips
// s = band PPL + k (strip s: columns [4 s, 4 s + 4), all 16 rows), so a
// lane's pixels share one row: the hit's row terms are formed once per entry
// (surfel_row_terms), and the sums times dy factor out of the pixel loop. Per blended entry, with h = alpha dL/dalpha
// (zero where alpha sat at 0.99): dL/drho = -h/2. On the surfel's own branch
// dL/dk = h / k2 (-u, -v, u^2 + v^2), summed as is and times dx and dy; on
// the filter's branch h (pixel - c) is summed for dL/dc. Record per surfel
// (16 floats): dL/drgb, sum h, sum dL/dk, sum dx dL/dk, sum dy dL/dk,
// sum h (pixel - c) over filter-branch pixels, 0.
// One wave's walk: strips band PPL .. band PPL + PPL - 1 of tile `tile` (pixel
// k of a lane lies in strip band PPL + k), only those set in band_sel (bit k),
// over list entries [walk_lo, walk_hi). A pixel whose row band blends nothing
// at or past walk_hi in the forward (rb_walk: each band's walk) starts from the
// final state; the others from the forward's checkpoint ck after entry
// walk_hi - 1 (T there, and the colour behind it, (C_final - C there +
// final_T bg) / T, with ck_end holding C_final). ck is null when walk_hi is
// past the walk.
template <int PPL>
__device__ __forceinline__ void surfel_bwd_walk(int tile, int band, uint32_t band_sel, int walk_lo, int walk_hi,
                                                const float4* __restrict__ ck, const float4* __restrict__ ck_end,
                                                uint4 rb_walk, int W, int H, int TX,
                                                const uint2* __restrict__ ranges, const uint32_t* __restrict__ values,
                                                const float4* __restrict__ tf, const float* __restrict__ rgb,
                                                float bg0, float bg1, float bg2, const float* __restrict__ final_T,
                                                const uint32_t* __restrict__ n_contrib,
                                                const float* __restrict__ dL_dimage, float* __restrict__ grad,
                                                SurfelBwdShared<BWD_BATCH>& sh) {
    constexpr int NB = BWD_BATCH;
    const int ty = tile / TX, tx = tile - ty * TX;
    const int lane = threadIdx.x;
    const int rl = lane & 15, row = lane >> 4;
    const bool c1 = ((rl ^ (rl >> 2)) & 1) != 0;
    const bool c2 = (((rl >> 1) ^ (rl >> 2)) & 1) != 0;
    const bool c3 = ((rl >> 2) & 1) != 0;
    const int slot = (c1 ? 4 : 0) + (c2 ? 2 : 0) + (c3 ? 1 : 0);
    const double ox = (double)(tx * TILE) + 0.5, oy = (double)(ty * TILE) + 0.5;
    const int r = lane >> 2, q4 = lane & 3;  // this lane's row in the tile, column within a strip
    const float ly = (float)r;
    const size_t HW = (size_t)W * H;
    const int py = ty * TILE + r;
    const int rb = r >> 2;
    const uint32_t rbw = rb == 0 ? rb_walk.x : rb == 1 ? rb_walk.y : rb == 2 ? rb_walk.z : rb_walk.w;
    float lx[PPL], T[PPL], g0[PPL], g1[PPL], g2[PPL], S[PPL];
    uint32_t last[PPL], band_last[PPL];
    uint32_t mylast = 0u;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
        const int col = 4 * (band * PPL + k) + q4;
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
        band_last[k] = __builtin_amdgcn_readfirstlane(wave_max_u32(last[k]));
        if (!((band_sel >> k) & 1u)) {  // the strip belongs to another wave: none of its entries is walked here
            band_last[k] = 0u;
            last[k] = 0u;
        }
        if (ck && rbw > (uint32_t)walk_hi) {  // this pixel's row band walked past walk_hi in the forward
            const int lp = 16 * r + col;      // the pixel's float4 in a checkpoint slot
            const float4 c = ck[lp], e = ck_end[lp];
            const float behind = fmaf(g0[k], e.x - c.y, fmaf(g1[k], e.y - c.z, g2[k] * (e.z - c.w)));
            S[k] = in ? fmaf(T[k], S[k], behind) / c.x : 0.f;
            T[k] = in ? c.x : 1.f;
        }
        mylast = max(mylast, band_last[k]);
    }
    const uint2 rg = ranges[tile];
    // never walk past the tile's list, whatever n_contrib holds
    const uint32_t maxlast = min(min(mylast, rg.y - rg.x), (uint32_t)walk_hi);
    // pixel-centre rectangle of the wave's first strip (strip k lies 4 k columns right)
    const float bx_lo = (float)(tx * TILE + 4 * band * PPL) + 0.5f;
    const float by_lo = (float)(ty * TILE) + 0.5f, by_hi = by_lo + 15.f;
    for (int hi = (int)maxlast; hi > walk_lo; hi -= NB) {
        const int lo = max(walk_lo, hi - NB);
        const int cnt = hi - lo;
        bool reach = false;  // some strip this wave walks past the entry may blend it
        bool clamp = false;  // its alpha may reach the 0.99 clamp
        if (lane < cnt) {
            const uint32_t gg = values[rg.x + lo + lane];
            clamp = stage_surfel(gg, tf, rgb, sh.rec[lane], ox, oy) > CLAMP_FREE_OPACITY;
            sh.g[lane] = gg;
            sh.has[lane] = 0u;
            const SurfelReach sr(tf[3 * (size_t)gg], tf[3 * (size_t)gg + 1], tf[3 * (size_t)gg + 2]);
            const uint32_t pl = (uint32_t)(lo + lane);
#pragma unroll
            for (int k = 0; k < PPL; ++k) {
                const float x0 = bx_lo + (float)(4 * k);
                reach = reach || (pl < band_last[k] && !sr.misses(x0, x0 + 3.f, by_lo, by_hi));
            }
        }
        uint64_t todo = __ballot(reach);
        const bool clamp_batch = __ballot(reach && clamp) != 0ull;
        __syncthreads();
        // a batch none of whose walked records can reach the alpha clamp (rho >= 0: o G <= o) takes a copy
        // without the clamp's min and test
        auto walk_entries = [&](auto clamp_tag) {
            constexpr bool CLAMP = decltype(clamp_tag)::value;
            while (todo) {
                const int j = 63 - __builtin_clzll(todo);  // backwards through the list
                todo &= ~(1ull << j);
                const uint32_t pos = (uint32_t)(lo + j);
                const SurfelRec& R = sh.rec[j];
                float acc[SURFEL_GRAD_STRIDE];
#pragma unroll
                for (int c = 0; c < SURFEL_GRAD_STRIDE; ++c) acc[c] = 0.f;
                // every strip's pixel through one branch-free pass: the blend tests first, one wave vote,
                // then the gradient terms (a pixel that did not blend takes alpha = 0, which leaves T, S
                // and every sum unchanged)
                const SurfelRowTerms rt = surfel_row_terms(R, ly);
                SurfelHit e[PPL];
                float al[PPL];
                bool bl[PPL], anyb = false;
#pragma unroll
                for (int k = 0; k < PPL; ++k) {
                    surfel_hit_in_row(R, rt, lx[k], e[k]);
                    al[k] = CLAMP ? fminf(ALPHA_MAX, e[k].oG) : e[k].oG;
                    bl[k] = pos < last[k] && al[k] >= ALPHA_MIN;
                    anyb = anyb || bl[k];
                }
                if (!__any(anyb)) continue;
#pragma unroll
                for (int k = 0; k < PPL; ++k) {
                    const float av = bl[k] ? al[k] : 0.f;
                    T[k] = T[k] * __builtin_amdgcn_rcpf(1.0f - av);  // T in front of this entry
                    const float wt = av * T[k];
                    acc[0] = fmaf(wt, g0[k], acc[0]);
                    acc[1] = fmaf(wt, g1[k], acc[1]);
                    acc[2] = fmaf(wt, g2[k], acc[2]);
                    const float cdl = fmaf(R.d.x, g0[k], fmaf(R.d.y, g1[k], R.d.z * g2[k]));
                    const float d = cdl - S[k];
                    S[k] = fmaf(av, d, S[k]);
                    const float h = (!CLAMP || e[k].oG <= ALPHA_MAX) ? wt * d : 0.f;  // alpha dL/dalpha
                    acc[3] += h;
                    const float h3 = e[k].own ? h : 0.f, hf = e[k].own ? 0.f : h;
                    // dL/dk = h / k2 (-u, -v, u^2 + v^2) on the surfel's own branch
                    const float q = h3 * e[k].inv;
                    const float dk0 = -e[k].u * q, dk1 = -e[k].v * q, dk2 = e[k].own ? e[k].rho3 * q : 0.f;
                    acc[4] += dk0;
                    acc[5] += dk1;
                    acc[6] += dk2;
                    acc[7] = fmaf(e[k].dx, dk0, acc[7]);
                    acc[8] = fmaf(e[k].dx, dk1, acc[8]);
                    acc[9] = fmaf(e[k].dx, dk2, acc[9]);
                    acc[13] = fmaf(hf, e[k].dx, acc[13]);
                    acc[14] += hf;  // times dy below: the lane's pixels share dy
                }
                acc[10] = rt.dy * acc[4];
                acc[11] = rt.dy * acc[5];
                acc[12] = rt.dy * acc[6];
                acc[14] *= rt.dy;
                // per 16-lane row: values 0-7 and 8-15 by two reduce-scatters (lanes 0-7 hold them)
                const float ua = row_reduce_scatter8(acc, c1, c2, c3);
                const float ub = row_reduce_scatter8(acc + 8, c1, c2, c3);
                if (rl < 8) {
                    sh.part[(j * 4 + row) * SURFEL_GRAD_STRIDE + slot] = ua;
                    sh.part[(j * 4 + row) * SURFEL_GRAD_STRIDE + 8 + slot] = ub;
                }
                if (lane == 0) sh.has[j] = 1u;
            }
        };
        if (clamp_batch) walk_entries(std::true_type{});
        else walk_entries(std::false_type{});
        __syncthreads();
        // one atomic add per value per (tile or band, surfel)
        for (int v = lane; v < cnt * 15; v += 64) {
            const int e = v / 15;
            const int c = v - e * 15;
            if (!sh.has[e]) continue;
            const float* pp = &sh.part[e * 4 * SURFEL_GRAD_STRIDE];
            auto rowsum = [&](int cc) {
                return (pp[cc] + pp[SURFEL_GRAD_STRIDE + cc]) + (pp[2 * SURFEL_GRAD_STRIDE + cc] + pp[3 * SURFEL_GRAD_STRIDE + cc]);
            };
            const float val = rowsum(c);
            if (val != 0.f) atomicAdd(&grad[(size_t)sh.g[e] * SURFEL_GRAD_STRIDE + c], val);
        }
        __syncthreads();
    }
}

template <int PPL>
__global__ __launch_bounds__(64) void k_surfel_bwd(int W, int H, int TX, const uint2* __restrict__ ranges,
                                                 const uint32_t* __restrict__ values, const float4* __restrict__ tf,
                                                 const float* __restrict__ rgb, float bg0, float bg1, float bg2,
                                                 const float* __restrict__ final_T,
                                                 const uint32_t* __restrict__ n_contrib,
                                                 const float* __restrict__ dL_dimage, float* __restrict__ grad) {
    constexpr int BANDS = 4 / PPL;
    __shared__ SurfelBwdShared<BWD_BATCH> sh;
    const int tile = blockIdx.x / BANDS, band = blockIdx.x - tile * BANDS;
    surfel_bwd_walk<PPL>(tile, band, 0xFu, 0, INT32_MAX, nullptr, nullptr, make_uint4(0u, 0u, 0u, 0u), W, H, TX, ranges,
                         values, tf, rgb, bg0, bg1, bg2, final_T, n_contrib, dL_dimage, grad, sh);
}

// The backward cut along deep tiles' walks, from the forward's checkpoints
// (piece_work: one wave per piece of CKPT_EVERY entries, each starting from
// the checkpoint after its last entry, so the pieces are independent).
__global__ __launch_bounds__(64) void k_surfel_bwd_pieces(int W, int H, int TX, int ntiles,
                                                        const float4* __restrict__ ckpt,
                                                        const uint2* __restrict__ ranges,
                                                        const uint32_t* __restrict__ values,
                                                        const float4* __restrict__ tf, const float* __restrict__ rgb,
                                                        float bg0, float bg1, float bg2,
                                                        const float* __restrict__ final_T,
                                                        const uint32_t* __restrict__ n_contrib,
                                                        const float* __restrict__ dL_dimage,
                                                        float* __restrict__ grad) {
    __shared__ SurfelBwdShared<BWD_BATCH> sh;
    PieceWork pw;
    if (!piece_work(blockIdx.x, ntiles, SURFEL_PIECES_CHUNK, ckpt, ranges, pw)) return;
    surfel_bwd_walk<4>(pw.tile, 0, pw.sel, pw.lo, pw.hi, pw.ck, pw.ck_end, pw.bw, W, H, TX, ranges, values, tf, rgb,
                       bg0, bg1, bg2, final_T, n_contrib, dL_dimage, grad, sh);
}

}  // namespace

hipError_t launch_surfel_render_fwd(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                                    const float* tf, const float* rgb, const float* bg, float* image, float* final_T,
                                    uint32_t* n_contrib, float* ckpt, hipStream_t stream) {
    const int ntiles = TX * TY;
    if (ntiles == 0) return hipSuccess;
    // checkpoints only where the backward reads them
    float4* ck = render_ckpt_bytes(TX, TY) ? reinterpret_cast<float4*>(ckpt) : nullptr;
    k_surfel_fwd<<<32 * ((ntiles + 7) / 8), 64, 0, stream>>>(W, H, TX, ntiles, reinterpret_cast<const uint2*>(ranges),
                                                             values, reinterpret_cast<const float4*>(tf), rgb, bg[0],
                                                             bg[1], bg[2], image, final_T, n_contrib, ck);
    return hipGetLastError();
}

hipError_t launch_surfel_render_bwd(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                                    const float* tf, const float* rgb, const float* bg, const float* final_T,
                                    const uint32_t* n_contrib, const float* dL_dimage, float* grad, const float* ckpt,
                                    hipStream_t stream) {
    const int ntiles = TX * TY;
    if (ntiles == 0) return hipSuccess;
    const uint2* rg = reinterpret_cast<const uint2*>(ranges);
    const float4* t4 = reinterpret_cast<const float4*>(tf);
    if (ckpt && render_ckpt_bytes(TX, TY)) {  // deep tiles cut into pieces from the forward's checkpoints
        k_surfel_bwd_pieces<<<(CKPT_SLOTS + 2) * SURFEL_PIECES_CHUNK *
                                  ((ntiles + SURFEL_PIECES_CHUNK - 1) / SURFEL_PIECES_CHUNK),
                              64, 0, stream>>>(W, H, TX, ntiles, reinterpret_cast<const float4*>(ckpt), rg, values, t4, rgb,
                                        bg[0], bg[1], bg[2], final_T, n_contrib, dL_dimage, grad);
        return hipGetLastError();
    }
    // small grids: a wave per 16x4 band keeps more SIMDs busy; large ones: a wave per tile
    if (ntiles < 2048)
        k_surfel_bwd<1><<<ntiles * 4, 64, 0, stream>>>(W, H, TX, rg, values, t4, rgb, bg[0], bg[1], bg[2], final_T,
                                                       n_contrib, dL_dimage, grad);
    else
        k_surfel_bwd<4><<<ntiles, 64, 0, stream>>>(W, H, TX, rg, values, t4, rgb, bg[0], bg[1], bg[2], final_T,
                                                   n_contrib, dL_dimage, grad);
    return hipGetLastError();
}

}  // namespace gs
