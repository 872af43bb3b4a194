// Per-tile alpha blending, forward and backward.
//
// Work layout (CDNA4, wave64): one 64-lane wave per 16x16 tile, each lane
// owning the 4 pixels (px, py0 + 4k), k = 0..3, of one column of the tile.
// The tile's depth-sorted Gaussian list is staged through LDS 64 records at a
// time (each lane gathers one record); every lane then reads each record by
// LDS broadcast. One wave per tile needs no barrier between waves, and 4
// pixels per lane give four independent blends per LDS read.
//
// Backward. The DISTWAR page ("DISTWAR: Fast Differentiable Rendering on
// Raster-based Rendering Pipelines", abstract) and the ARC page ("ARC:
// Warp-level Adaptive Atomic Reduction in GPUs to Accelerate Differentiable
// Rendering", abstract) find this step bound by atomic updates that flood the
// L2 atomic units, because all lanes of a warp update the same Gaussian. Here
// each lane first sums its 4 pixels' terms in registers, the wave then sums
// its 64 lanes with DPP (6 cross-lane adds per value, result in lane 63) --
// only for entries where some lane contributed -- and the per-tile totals of a
// 64-record batch are flushed with all lanes active: one fp32 atomic add per
// value per (tile, Gaussian), 9 consecutive lanes per Gaussian record.
#include "common.hpp"
#include "launch.hpp"

namespace gs {

namespace {

constexpr int PPL = 4;     // pixels per lane
constexpr int BATCH = 64;  // records staged per LDS batch

__global__ __launch_bounds__(64) void k_render_fwd(int W, int H, int TX, const uint2* __restrict__ ranges,
                                                 const uint32_t* __restrict__ values,
                                                 const float2* __restrict__ means2d,
                                                 const float4* __restrict__ conic_op, const float* __restrict__ rgb,
                                                 float bg0, float bg1, float bg2, float* __restrict__ image,
                                                 float* __restrict__ final_T, uint32_t* __restrict__ n_contrib) {
    __shared__ float4 s_a[BATCH];  // u, v, a, beta
    __shared__ float4 s_b[BATCH];  // gamma, opacity, r, g
    __shared__ float s_c[BATCH];   // b
    const int tile = blockIdx.x;
    const int tx = tile % TX, ty = tile / TX;
    const int lane = threadIdx.x;
    const int px = tx * TILE + (lane & 15);
    const int py0 = ty * TILE + (lane >> 4);
    const float pxc = (float)px + 0.5f;
    float pyc[PPL], T[PPL], C0[PPL], C1[PPL], C2[PPL];
    uint32_t last[PPL];
    bool done[PPL];
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
        int py = py0 + 4 * k;
        pyc[k] = (float)py + 0.5f;
        T[k] = 1.f;
        C0[k] = C1[k] = C2[k] = 0.f;
        last[k] = 0u;
        done[k] = !(px < W && py < H);
    }
    const uint2 rg = ranges[tile];
    for (uint32_t bs = rg.x; bs < rg.y; bs += BATCH) {
        if (__all(done[0] && done[1] && done[2] && done[3])) break;
        uint32_t idx = bs + lane;
        if (idx < rg.y) {
            uint32_t g = values[idx];
            float2 m = means2d[g];
            float4 c = conic_op[g];
            s_a[lane] = make_float4(m.x, m.y, c.x, c.y);
            s_b[lane] = make_float4(c.z, c.w, rgb[3 * (size_t)g], rgb[3 * (size_t)g + 1]);
            s_c[lane] = rgb[3 * (size_t)g + 2];
        }
        __syncthreads();
        const int cnt = (int)min((uint32_t)BATCH, rg.y - bs);
        const uint32_t pos0 = bs - rg.x + 1;
        for (int j = 0; j < cnt; ++j) {
            if ((j & 7) == 7 && __all(done[0] && done[1] && done[2] && done[3])) break;
            const float4 A = s_a[j];
            const float4 B = s_b[j];
            const float cb = s_c[j];
            const float dx = pxc - A.x;
#pragma unroll
            for (int k = 0; k < PPL; ++k) {
                float w, G, oG;
                falloff(dx, pyc[k] - A.y, A.z, A.w, B.x, B.y, w, G, oG);
                const float alpha = fminf(ALPHA_MAX, oG);
                bool take = !done[k] && alpha >= ALPHA_MIN;
                const float Tn = T[k] * (1.0f - alpha);
                const bool stop = take && Tn < T_MIN;
                take = take && !stop;
                done[k] = done[k] || stop;
                const float wt = take ? alpha * T[k] : 0.f;
                C0[k] = fmaf(B.z, wt, C0[k]);
                C1[k] = fmaf(B.w, wt, C1[k]);
                C2[k] = fmaf(cb, wt, C2[k]);
                T[k] = take ? Tn : T[k];
                last[k] = take ? pos0 + (uint32_t)j : last[k];
            }
        }
        __syncthreads();
    }
    const size_t HW = (size_t)W * H;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
        int py = py0 + 4 * k;
        if (px < W && py < H) {
            size_t p = (size_t)py * W + px;
            image[p] = fmaf(T[k], bg0, C0[k]);
            image[HW + p] = fmaf(T[k], bg1, C1[k]);
            image[2 * HW + p] = fmaf(T[k], bg2, C2[k]);
            final_T[p] = T[k];
            n_contrib[p] = last[k];
        }
    }
}

__global__ __launch_bounds__(64) void k_render_bwd(int W, int H, int TX, const uint2* __restrict__ ranges,
                                                 const uint32_t* __restrict__ values,
                                                 const float2* __restrict__ means2d,
                                                 const float4* __restrict__ conic_op, const float* __restrict__ rgb,
                                                 float bg0, float bg1, float bg2, const float* __restrict__ final_T,
                                                 const uint32_t* __restrict__ n_contrib,
                                                 const float* __restrict__ dL_dimage, float* __restrict__ grad2d) {
    __shared__ float4 s_a[BATCH];
    __shared__ float4 s_b[BATCH];
    __shared__ float s_c[BATCH];
    __shared__ uint32_t s_g[BATCH];
    __shared__ float s_part[BATCH * 4 * GRAD2D_N];  // [entry][row of 16 lanes][value]
    __shared__ uint32_t s_has[BATCH];
    const int tile = blockIdx.x;
    const int tx = tile % TX, ty = tile / TX;
    const int lane = threadIdx.x;
    // lane roles in the in-row reduce-scatter (see row_reduce_scatter8)
    const int rl = lane & 15, row = lane >> 4;
    const bool c1 = ((rl ^ (rl >> 2)) & 1) != 0;
    const bool c2 = (((rl >> 1) ^ (rl >> 2)) & 1) != 0;
    const bool c3 = ((rl >> 2) & 1) != 0;
    const bool writer = rl < 9;
    const int slot = rl < 8 ? (c1 ? 4 : 0) + (c2 ? 2 : 0) + (c3 ? 1 : 0) : 8;
    const int px = tx * TILE + (lane & 15);
    const int py0 = ty * TILE + (lane >> 4);
    const float pxc = (float)px + 0.5f;
    const size_t HW = (size_t)W * H;
    float pyc[PPL], T[PPL], g0[PPL], g1[PPL], g2[PPL], S[PPL];
    uint32_t last[PPL];
    uint32_t mylast = 0;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
        int py = py0 + 4 * k;
        pyc[k] = (float)py + 0.5f;
        bool in = px < W && py < H;
        size_t p = in ? (size_t)py * W + px : 0;
        T[k] = in ? final_T[p] : 1.f;
        last[k] = in ? n_contrib[p] : 0u;
        g0[k] = in ? dL_dimage[p] : 0.f;
        g1[k] = in ? dL_dimage[HW + p] : 0.f;
        g2[k] = in ? dL_dimage[2 * HW + p] : 0.f;
        // S = A . dL/dC with A the normalised colour behind the current entry (starts as bg)
        S[k] = fmaf(bg0, g0[k], fmaf(bg1, g1[k], bg2 * g2[k]));
        mylast = max(mylast, last[k]);
    }
    const uint2 rg = ranges[tile];
    // never walk past the tile's list, whatever n_contrib holds
    const uint32_t maxlast = min(wave_max_u32(mylast), rg.y - rg.x);
    for (int hi = (int)maxlast; hi > 0; hi -= BATCH) {
        const int lo = max(0, hi - BATCH);
        const int cnt = hi - lo;
        if (lane < cnt) {
            uint32_t g = values[rg.x + lo + lane];
            float2 m = means2d[g];
            float4 c = conic_op[g];
            s_a[lane] = make_float4(m.x, m.y, c.x, c.y);
            s_b[lane] = make_float4(c.z, c.w, rgb[3 * (size_t)g], rgb[3 * (size_t)g + 1]);
            s_c[lane] = rgb[3 * (size_t)g + 2];
            s_g[lane] = g;
        }
        __syncthreads();
        for (int j = cnt - 1; j >= 0; --j) {
            const float4 A = s_a[j];
            const float4 B = s_b[j];
            const float cb = s_c[j];
            const uint32_t pos = (uint32_t)(lo + j);
            const float dx = pxc - A.x;
            // which of this lane's pixels blended this entry (same test as the forward)
            float w[PPL], dy[PPL], oG[PPL], al[PPL];
            bool blended[PPL];
            bool any = false;
#pragma unroll
            for (int k = 0; k < PPL; ++k) {
                float G;
                dy[k] = pyc[k] - A.y;
                falloff(dx, dy[k], A.z, A.w, B.x, B.y, w[k], G, oG[k]);
                al[k] = fminf(ALPHA_MAX, oG[k]);
                blended[k] = pos < last[k] && al[k] >= ALPHA_MIN;
                any = any || blended[k];
            }
            if (!__any(any)) {
                if (lane == 0) s_has[j] = 0u;
                continue;
            }
            // branch-free: a pixel that did not blend this entry takes alpha = 0,
            // which leaves its T, S and every sum unchanged
            float acc[GRAD2D_N];
#pragma unroll
            for (int c = 0; c < GRAD2D_N; ++c) acc[c] = 0.f;
#pragma unroll
            for (int k = 0; k < PPL; ++k) {
                const float av = blended[k] ? al[k] : 0.f;
                T[k] = T[k] * __builtin_amdgcn_rcpf(1.0f - av);  // T in front of this entry
                const float wt = av * T[k];
                acc[0] = fmaf(wt, g0[k], acc[0]);
                acc[1] = fmaf(wt, g1[k], acc[1]);
                acc[2] = fmaf(wt, g2[k], acc[2]);
                const float cdl = fmaf(B.z, g0[k], fmaf(B.w, g1[k], cb * g2[k]));
                const float d = cdl - S[k];
                S[k] = fmaf(av, d, S[k]);
                // h = o G dL/dalpha = -2 dL/dQ; zero where alpha sat at its 0.99 clamp
                const float h = (blended[k] && oG[k] <= ALPHA_MAX) ? oG[k] * (T[k] * d) : 0.f;
                const float hw = h * w[k], hy = h * dy[k];
                acc[3] += h;
                acc[4] = fmaf(hw, w[k], acc[4]);
                acc[5] = fmaf(hw, dy[k], acc[5]);
                acc[6] = fmaf(hy, dy[k], acc[6]);
                acc[7] += hw;
                acc[8] += hy;
            }
            // per 16-lane row: values 0..7 by reduce-scatter (lane slot holds one), value 8 by a row sum
            const float u = row_reduce_scatter8(acc, c1, c2, c3);
            const float x8 = row_sum16(acc[8]);
            if (writer) s_part[(j * 4 + row) * GRAD2D_N + slot] = rl < 8 ? u : x8;
            if (lane == 0) s_has[j] = 1u;
        }
        __syncthreads();
        // one atomic add per value per (tile, Gaussian): the 4 row partials summed here
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

}  // namespace

hipError_t launch_render_fwd(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                             const float* means2d, const float* conic_op, const float* rgb, const float* bg,
                             float* image, float* final_T, uint32_t* n_contrib, hipStream_t stream) {
    int ntiles = TX * TY;
    if (ntiles == 0) return hipSuccess;
    k_render_fwd<<<ntiles, 64, 0, stream>>>(W, H, TX, reinterpret_cast<const uint2*>(ranges), values,
                                            reinterpret_cast<const float2*>(means2d),
                                            reinterpret_cast<const float4*>(conic_op), rgb, bg[0], bg[1], bg[2],
                                            image, final_T, n_contrib);
    return hipGetLastError();
}

hipError_t launch_render_bwd(int W, int H, int TX, int TY, const uint32_t* ranges, const uint32_t* values,
                             const float* means2d, const float* conic_op, const float* rgb, const float* bg,
                             const float* final_T, const uint32_t* n_contrib, const float* dL_dimage,
                             float* grad2d, hipStream_t stream) {
    int ntiles = TX * TY;
    if (ntiles == 0) return hipSuccess;
    k_render_bwd<<<ntiles, 64, 0, stream>>>(W, H, TX, reinterpret_cast<const uint2*>(ranges), values,
                                            reinterpret_cast<const float2*>(means2d),
                                            reinterpret_cast<const float4*>(conic_op), rgb, bg[0], bg[1], bg[2],
                                            final_T, n_contrib, dL_dimage, grad2d);
    return hipGetLastError();
}

}  // namespace gs
