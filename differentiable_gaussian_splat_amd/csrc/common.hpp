// Device-side definitions shared by the rasterizer's kernels (gfx950, wave64).
//
// The method is the tile-based rasterizer of 3D Gaussian Splatting (named in the
// abstract of the DISTWAR page, "DISTWAR: Fast Differentiable Rendering on
// Raster-based Rendering Pipelines"). The constants below are that method's
// compositing constants; the pages themselves print none of them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gs {

constexpr int TILE = 16;             // tile edge in pixels
constexpr float ALPHA_MAX = 0.99f;   // alpha = min(0.99, o G)
// At or below this opacity, o G (formed as exp2 of an exponent at most log2 o, each step a few ulps
// off) stays far below ALPHA_MAX, so the clamp's min and test can be left out exactly.
constexpr float CLAMP_FREE_OPACITY = 0.989f;
constexpr float ALPHA_MIN = 1.0f / 255.0f;  // entries below are skipped
constexpr float T_MIN = 1e-4f;       // a pixel stops before T would drop below
constexpr float BIG = 16777216.0f;   // 2^24: beyond this fp32 no longer resolves pixels
constexpr float NEG_HALF_LOG2E = -0.72134752044448170368f;  // -log2(e)/2: exp(-Q/2) = 2^(Q * this)

// Per-Gaussian values the backward's reverse blend sums over pixels (see
// k_render_bwd): colour gradient (3), then with h = o G dL/dalpha per pixel,
// sum h, sum h w^2, sum h w dy, sum h dy^2, sum h w, sum h dy, where
// w = dx + beta dy. The chain rule turns these into conic/mean gradients.
constexpr int GRAD2D_N = 9;
constexpr int GRAD2D_STRIDE = 12;    // floats per Gaussian record (48 B, 16-B aligned)

// Camera as the kernels take it (by value): intrinsics, tile grid, world->camera
// rotation R (row-major) and translation t, and the camera centre -R^T t.
struct DevCam {
    int W, H, TX, TY;
    float fx, fy, cx, cy;
    float R[9];
    float t[3];
    float campos[3];
};

// The cameras of one batched launch (views of one image size), passed by
// value: a launch's view index is wave-uniform, so they are read with scalar
// loads from the kernel arguments.
constexpr int MAX_VIEWS = 32;
struct CamSet {
    DevCam c[MAX_VIEWS];
};

__device__ __forceinline__ bool finitef(float x) { return __builtin_isfinite(x); }

// Tile rectangle of a Gaussian with screen mean (u, v) and integer radius r:
// the tiles holding a pixel column within r of floor(u) and a pixel row
// within r of floor(v), clamped to the grid. Returns false when empty.
// |u|, |v|, r <= 2^24 keeps every intermediate inside int32; ">> 4" on a
// signed int is the floor division by 16 (arithmetic shift).
__device__ __forceinline__ bool tile_rect(float u, float v, int r, int TX, int TY,
                                          int& X0, int& X1, int& Y0, int& Y1) {
    int fu = (int)floorf(u), fv = (int)floorf(v);
    X0 = max(0, (fu - r) >> 4);
    X1 = min(TX - 1, (fu + r) >> 4);
    Y0 = max(0, (fv - r) >> 4);
    Y1 = min(TY - 1, (fv + r) >> 4);
    return X0 <= X1 && Y0 <= Y1;
}

// Tile `tile` of the grid of views stacked vertically (TX x TY tiles each):
// its view, returned, and its column and row inside that view.
__device__ __forceinline__ int view_of_tile(int tile, int TX, int TY, int& tx, int& ty) {
    const int row = tile / TX;
    const int view = row / TY;
    tx = tile - row * TX;
    ty = row - view * TY;
    return view;
}

// j -> (j / w, j % w) for 0 <= j < 2^23 and 1 <= w <= 2^11: a float
// reciprocal gives q within one of the quotient; one exact fixup each way.
__device__ __forceinline__ void divmod_small(int j, int w, int& q, int& r) {
    q = (int)(((float)j + 0.5f) * __builtin_amdgcn_rcpf((float)w));
    r = j - q * w;
    if (r < 0) { q -= 1; r += w; }
    if (r >= w) { q += 1; r -= w; }
}

// Opacity-weighted Gaussian falloff o G at a pixel, with the conic in
// factored form Q = a w^2 + gamma dy^2, w = dx + beta dy, (dx, dy) = pixel
// centre - screen mean, and the per-record constants staged as
// a2 = -a log2(e)/2, g2 = -gamma log2(e)/2 and lo = log2(o):
// o G = o exp(-Q/2) = 2^(a2 w^2 + g2 dy^2 + lo). The caller forms w and dy from
// their values at the tile's first pixel (staged per record with extra
// precision) plus the pixel's small offset in the tile: a Gaussian whose mean
// lies thousands of pixels away would otherwise lose w to cancellation
// between dx and beta dy. The forward and the backward call this same function
// on the same staged values so that both take the same skip decisions bit for
// bit; contraction is fixed by hand.
__device__ __forceinline__ float falloff(float w, float dy, float a2, float g2, float lo) {
#pragma clang fp contract(off)
    const float aw = a2 * w;
    const float gdy = g2 * dy;
    return __builtin_amdgcn_exp2f(__fmaf_rn(aw, w, __fmaf_rn(gdy, dy, lo)));
}

// The staged constants of one record (conic_opacity = (a, beta, gamma, o)).
__device__ __forceinline__ float4 falloff_consts(float4 c) {
    return make_float4(c.x * NEG_HALF_LOG2E, c.y, c.z * NEG_HALF_LOG2E, __builtin_amdgcn_logf(c.w));
}

// ---------------------------------------------------------------- wave64 helpers

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_zero_fill(float src) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(src), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes; the total is valid in lane 63. DPP steps: pairs,
// quads, then rotations by 4 and 8 inside each 16-lane row (every lane holds
// its row sum), then row broadcasts 15 and 31 fold the four rows into row 3.
__device__ __forceinline__ float wave_sum_to_lane63(float x) {
    x += dpp_zero_fill<0xB1, 0xF>(x);   // quad_perm [1,0,3,2]
    x += dpp_zero_fill<0x4E, 0xF>(x);   // quad_perm [2,3,0,1]
    x += dpp_zero_fill<0x124, 0xF>(x);  // row_ror:4
    x += dpp_zero_fill<0x128, 0xF>(x);  // row_ror:8
    x += dpp_zero_fill<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_zero_fill<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

template <int CTRL>
__device__ __forceinline__ float dpp_row(float src) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(src), CTRL, 0xF, 0xF, false));
}

// Sum over each 16-lane row; every lane of the row gets the row's sum.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_row<0xB1>(x);   // partner lane ^ 1
    x += dpp_row<0x4E>(x);   // partner lane ^ 2
    x += dpp_row<0x124>(x);  // row_ror:4
    x += dpp_row<0x128>(x);  // row_ror:8
    return x;
}

// Reduce-scatter of 8 values over each 16-lane row in 4 butterfly steps. The
// partners lane^1, lane^2 (quad_perm), lane^7 (row_half_mirror) and lane^8
// (row_ror:8) form a basis of the 4-bit lane index, so recursive halving along
// them is exact: with c1 = b0^b2, c2 = b1^b2, c3 = b2 (b = bits of lane & 15),
// each lane keeps half of its values per step and ends with the row sum of
// value 4 c1 + 2 c2 + c3. Lanes 0..7 of a row hold the 8 distinct values.
// Costs 22 VALU ops instead of 8 x 4 for eight plain row sums.
__device__ __forceinline__ float row_reduce_scatter8(const float* x, bool c1, bool c2, bool c3) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = c1 ? x[4 + i] : x[i];
        const float send = c1 ? x[i] : x[4 + i];
        y[i] = keep + dpp_row<0xB1>(send);
    }
    float z[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = c2 ? y[2 + i] : y[i];
        const float send = c2 ? y[i] : y[2 + i];
        z[i] = keep + dpp_row<0x4E>(send);
    }
    const float keep = c3 ? z[1] : z[0];
    const float send = c3 ? z[0] : z[1];
    float u = keep + dpp_row<0x141>(send);  // row_half_mirror: lane ^ 7 inside each 8
    u += dpp_row<0x128>(u);                 // row_ror:8 = lane ^ 8
    return u;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (1ull << (threadIdx.x & 63)) - 1ull;
}

// Point of exchange for lanes of one wave that talk through LDS without a
// block barrier. The hardware already runs a wave's LDS accesses in order;
// the wave-scope fences (no instructions) keep the compiler from forwarding
// a lane's own earlier store to a later load of the same address, which
// would miss what other lanes wrote there in between.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- spherical harmonics
// Real SH with the Condon-Shortley phase kept, index k = l^2 + l + m, degree <= 3,
// evaluated at a unit direction (x, y, z). Constants are the textbook
// normalisations sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!) (times sqrt 2 for m != 0).
constexpr float SH_C0 = 0.28209479177387814f;
constexpr float SH_C1 = 0.4886025119029199f;
constexpr float SH_C2a = 1.0925484305920792f;   // xy, yz, xz terms
constexpr float SH_C2b = 0.31539156525252005f;  // 2z^2 - x^2 - y^2
constexpr float SH_C2c = 0.5462742152960396f;   // x^2 - y^2
constexpr float SH_C3a = 0.5900435899266435f;   // |m| = 3
constexpr float SH_C3b = 2.890611442640554f;    // xyz
constexpr float SH_C3c = 0.4570457994644658f;   // |m| = 1
constexpr float SH_C3d = 0.3731763325901154f;   // m = 0
constexpr float SH_C3e = 1.445305721320277f;    // m = 2

__device__ __forceinline__ void sh_eval(int K, float x, float y, float z, float* Y) {
    Y[0] = SH_C0;
    if (K <= 1) return;
    Y[1] = -SH_C1 * y;
    Y[2] = SH_C1 * z;
    Y[3] = -SH_C1 * x;
    if (K <= 4) return;
    float xx = x * x, yy = y * y, zz = z * z;
    Y[4] = SH_C2a * x * y;
    Y[5] = -SH_C2a * y * z;
    Y[6] = SH_C2b * (2.f * zz - xx - yy);
    Y[7] = -SH_C2a * x * z;
    Y[8] = SH_C2c * (xx - yy);
    if (K <= 9) return;
    Y[9] = -SH_C3a * y * (3.f * xx - yy);
    Y[10] = SH_C3b * x * y * z;
    Y[11] = -SH_C3c * y * (4.f * zz - xx - yy);
    Y[12] = SH_C3d * z * (2.f * zz - 3.f * xx - 3.f * yy);
    Y[13] = -SH_C3c * x * (4.f * zz - xx - yy);
    Y[14] = SH_C3e * z * (xx - yy);
    Y[15] = -SH_C3a * x * (xx - 3.f * yy);
}

// g += sum_k c[k] * grad(Y_k) at (x, y, z), x, y, z treated as independent.
__device__ __forceinline__ void sh_grad_accum(int K, float x, float y, float z, const float* c, float3& g) {
    if (K <= 1) return;
    g.y -= SH_C1 * c[1];
    g.z += SH_C1 * c[2];
    g.x -= SH_C1 * c[3];
    if (K <= 4) return;
    float xx = x * x, yy = y * y, zz = z * z;
    g.x += SH_C2a * y * c[4];
    g.y += SH_C2a * x * c[4];
    g.y -= SH_C2a * z * c[5];
    g.z -= SH_C2a * y * c[5];
    g.x -= 2.f * SH_C2b * x * c[6];
    g.y -= 2.f * SH_C2b * y * c[6];
    g.z += 4.f * SH_C2b * z * c[6];
    g.x -= SH_C2a * z * c[7];
    g.z -= SH_C2a * x * c[7];
    g.x += 2.f * SH_C2c * x * c[8];
    g.y -= 2.f * SH_C2c * y * c[8];
    if (K <= 9) return;
    g.x -= SH_C3a * 6.f * x * y * c[9];
    g.y -= SH_C3a * (3.f * xx - 3.f * yy) * c[9];
    g.x += SH_C3b * y * z * c[10];
    g.y += SH_C3b * x * z * c[10];
    g.z += SH_C3b * x * y * c[10];
    g.x += SH_C3c * 2.f * x * y * c[11];
    g.y -= SH_C3c * (4.f * zz - xx - 3.f * yy) * c[11];
    g.z -= SH_C3c * 8.f * y * z * c[11];
    g.x -= SH_C3d * 6.f * x * z * c[12];
    g.y -= SH_C3d * 6.f * y * z * c[12];
    g.z += SH_C3d * (6.f * zz - 3.f * xx - 3.f * yy) * c[12];
    g.x -= SH_C3c * (4.f * zz - 3.f * xx - yy) * c[13];
    g.y += SH_C3c * 2.f * x * y * c[13];
    g.z -= SH_C3c * 8.f * x * z * c[13];
    g.x += SH_C3e * 2.f * x * z * c[14];
    g.y -= SH_C3e * 2.f * y * z * c[14];
    g.z += SH_C3e * (xx - yy) * c[14];
    g.x -= SH_C3a * (3.f * xx - 3.f * yy) * c[15];
    g.y += SH_C3a * 6.f * x * y * c[15];
}

}  // namespace gs
