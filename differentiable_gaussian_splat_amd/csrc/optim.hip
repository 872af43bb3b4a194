// Phase U: one Adam update of the raw Gaussian parameters, fused with the
// activation chain (scales = exp(log_scales), opacities = sigmoid(logits))
// and a per-Gaussian gradient magnitude. The Odin page names the phase
// ("Odin: Primitive-Level Synchronization for Distributed Point-Based Neural
// Rendering", Fig. 7 caption) and the optimizer (referee report, major
// comment 1); Adam itself is the published method of Kingma and Ba.
//
// Work layout: each 64-lane wave owns 64 consecutive Gaussians. The small
// parameter groups go lane = Gaussian. The SH block of the 64 Gaussians is
// one contiguous run in every array and is walked as flat float4s with
// consecutive lanes on consecutive addresses (the update is element-wise).
// The squared SH gradients of one step's lanes that belong to one Gaussian
// (consecutive lanes) are summed by a segmented tree over the wave, and the
// segment's first lane adds the sum to the Gaussian's LDS slot, which the
// Gaussian's own lane reads at the end: a fixed order, so the norm is the
// same bit for bit from run to run.
#include <cmath>

#include "common.hpp"
#include "launch.hpp"

namespace gs {

namespace {

constexpr int OB = 256;  // threads per block: four waves of 64 Gaussians

struct AdamK {
    float b1, omb1, b2, omb2, eps, ibc1, ibc2s;
};

__device__ __forceinline__ void adam1(float& p, float& m, float& v, float g, float lr, const AdamK& k) {
    m = fmaf(k.b1, m, k.omb1 * g);
    v = fmaf(k.b2, v, k.omb2 * (g * g));
    const float den = fmaf(sqrtf(v), k.ibc2s, k.eps);
    p = fmaf(-(lr * k.ibc1), m / den, p);
}

// sigmoid(x) and its derivative sigmoid(x) (1 - sigmoid(x)), from e = exp(-|x|) <= 1:
// sigmoid(|x|) = 1 / (1 + e), sigmoid(-|x|) = e sigmoid(|x|), and the derivative
// (even in x) = e sigmoid(|x|)^2, with no 1 - s cancellation for large |x|.
__device__ __forceinline__ float sigmoidf(float x, float* deriv = nullptr) {
    const float e = expf(-fabsf(x));
    const float sp = 1.0f / (1.0f + e);
    if (deriv) *deriv = e * sp * sp;
    return x >= 0.f ? sp : e * sp;
}

// Adds x into s[j] for every valid lane, where the lanes sharing a j are
// consecutive: a segmented tree sum (lane i takes lane i + off's partial when
// both lie in one segment), then the segment's first lane adds, with a plain
// LDS update (one writer per j per call; the wave's calls run in order).
__device__ __forceinline__ void seg_add(float* s, int j, float x, bool valid) {
    const int lane = threadIdx.x & 63;
    const int key = valid ? j : -1 - lane;  // invalid lanes form segments of their own
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_down(x, off);
        const int ky = __shfl_down(key, off);
        if (lane + off < 64 && ky == key) x += y;
    }
    const int kprev = __shfl_up(key, 1);
    if (valid && (lane == 0 || kprev != key)) s[j] += x;
}

__global__ __launch_bounds__(OB) void k_adam_step(AdamLr lr, AdamK k, int n, int rec, float* __restrict__ means,
                                                 float* __restrict__ lsc, float4* __restrict__ quats,
                                                 float* __restrict__ logit, float* __restrict__ sh,
                                                 const float* __restrict__ g_means, const float* __restrict__ g_sc,
                                                 const float4* __restrict__ g_quats, const float* __restrict__ g_op,
                                                 const float* __restrict__ g_sh, float* __restrict__ m_means,
                                                 float* __restrict__ m_lsc, float4* __restrict__ m_quats,
                                                 float* __restrict__ m_logit, float* __restrict__ m_sh,
                                                 float* __restrict__ v_means, float* __restrict__ v_lsc,
                                                 float4* __restrict__ v_quats, float* __restrict__ v_logit,
                                                 float* __restrict__ v_sh, float* __restrict__ scales_out,
                                                 float* __restrict__ opac_out, float* __restrict__ grad_norm) {
    __shared__ float s_norm[OB / 64][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int base = (blockIdx.x * (OB / 64) + w) * 64;
    if (base >= n) return;  // whole waves only: nothing below needs the block
    const int cnt = min(64, n - base);
    s_norm[w][lane] = 0.f;
    wave_lds_sync();
    // SH: the wave's run of cnt * rec floats, element-wise
    const size_t r0 = (size_t)base * rec;
    const int total = cnt * rec;
    // every lane runs every step (the segmented sums need the whole wave); lanes past the run idle
    if ((rec & 3) == 0) {
        for (int f0 = 0; 4 * f0 < total; f0 += 64) {
            const int f = f0 + lane;
            const bool valid = 4 * f < total;
            int j = 0, e = 0;
            float sq = 0.f;
            if (valid) {
                const size_t o = r0 + 4 * (size_t)f;
                float4 p = *reinterpret_cast<const float4*>(sh + o);
                const float4 g = *reinterpret_cast<const float4*>(g_sh + o);
                float4 m = *reinterpret_cast<const float4*>(m_sh + o);
                float4 v = *reinterpret_cast<const float4*>(v_sh + o);
                divmod_small(4 * f, rec, j, e);  // Gaussian j of the wave, its element e (a float4 stays in one record)
                const float l0 = e < 3 ? lr.sh_dc : lr.sh_rest, l1 = e + 1 < 3 ? lr.sh_dc : lr.sh_rest;
                const float l2 = e + 2 < 3 ? lr.sh_dc : lr.sh_rest;
                adam1(p.x, m.x, v.x, g.x, l0, k);
                adam1(p.y, m.y, v.y, g.y, l1, k);
                adam1(p.z, m.z, v.z, g.z, l2, k);
                adam1(p.w, m.w, v.w, g.w, lr.sh_rest, k);  // element e + 3 >= 3
                *reinterpret_cast<float4*>(sh + o) = p;
                *reinterpret_cast<float4*>(m_sh + o) = m;
                *reinterpret_cast<float4*>(v_sh + o) = v;
                sq = fmaf(g.x, g.x, fmaf(g.y, g.y, fmaf(g.z, g.z, g.w * g.w)));
            }
            seg_add(s_norm[w], j, sq, valid);
        }
    } else {
        for (int f0 = 0; f0 < total; f0 += 64) {
            const int f = f0 + lane;
            const bool valid = f < total;
            int j = 0, e = 0;
            float sq = 0.f;
            if (valid) {
                const size_t o = r0 + (size_t)f;
                float p = sh[o], m = m_sh[o], v = v_sh[o];
                const float g = g_sh[o];
                divmod_small(f, rec, j, e);
                adam1(p, m, v, g, e < 3 ? lr.sh_dc : lr.sh_rest, k);
                sh[o] = p;
                m_sh[o] = m;
                v_sh[o] = v;
                sq = g * g;
            }
            seg_add(s_norm[w], j, sq, valid);
        }
    }
    wave_lds_sync();
    if (lane >= cnt) return;
    const size_t gi = (size_t)base + lane;
    float n2 = s_norm[w][lane];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const size_t o = 3 * gi + c;
        // means
        {
            float p = means[o], m = m_means[o], v = v_means[o];
            const float g = g_means[o];
            adam1(p, m, v, g, lr.means, k);
            means[o] = p;
            m_means[o] = m;
            v_means[o] = v;
            n2 = fmaf(g, g, n2);
        }
        // log-scales: chain from the activated scale at the value before the update
        {
            float p = lsc[o], m = m_lsc[o], v = v_lsc[o];
            const float g = g_sc[o] * expf(p);
            adam1(p, m, v, g, lr.scales, k);
            lsc[o] = p;
            m_lsc[o] = m;
            v_lsc[o] = v;
            scales_out[o] = expf(p);
            n2 = fmaf(g, g, n2);
        }
    }
    {
        float4 p = quats[gi], m = m_quats[gi], v = v_quats[gi];
        const float4 g = g_quats[gi];
        adam1(p.x, m.x, v.x, g.x, lr.quats, k);
        adam1(p.y, m.y, v.y, g.y, lr.quats, k);
        adam1(p.z, m.z, v.z, g.z, lr.quats, k);
        adam1(p.w, m.w, v.w, g.w, lr.quats, k);
        quats[gi] = p;
        m_quats[gi] = m;
        v_quats[gi] = v;
        n2 = fmaf(g.x, g.x, fmaf(g.y, g.y, fmaf(g.z, g.z, fmaf(g.w, g.w, n2))));
    }
    {
        float p = logit[gi], m = m_logit[gi], v = v_logit[gi];
        float ds;
        sigmoidf(p, &ds);
        const float g = g_op[gi] * ds;
        adam1(p, m, v, g, lr.opacity, k);
        logit[gi] = p;
        m_logit[gi] = m;
        v_logit[gi] = v;
        opac_out[gi] = sigmoidf(p);
        n2 = fmaf(g, g, n2);
    }
    if (grad_norm) grad_norm[gi] = sqrtf(n2);
}

}  // namespace

hipError_t launch_adam_step(const AdamLr& lr, float beta1, float beta2, float eps, int step, int n, int sh_rows,
                            float* const params[5], const float* const grads[5], float* const m[5],
                            float* const v[5], float* scales, float* opacities, float* grad_norm,
                            hipStream_t stream) {
    if (n == 0) return hipSuccess;
    AdamK k;
    k.b1 = beta1;
    k.omb1 = 1.0f - beta1;
    k.b2 = beta2;
    k.omb2 = 1.0f - beta2;
    k.eps = eps;
    // bias corrections in double, rounded once
    k.ibc1 = (float)(1.0 / (1.0 - std::pow((double)beta1, (double)step)));
    k.ibc2s = (float)(1.0 / std::sqrt(1.0 - std::pow((double)beta2, (double)step)));
    const int waves = (n + 63) / 64;
    const int blocks = (waves + OB / 64 - 1) / (OB / 64);
    k_adam_step<<<blocks, OB, 0, stream>>>(
        lr, k, n, 3 * sh_rows, params[0], params[1], reinterpret_cast<float4*>(params[2]), params[3], params[4],
        grads[0], grads[1], reinterpret_cast<const float4*>(grads[2]), grads[3], grads[4], m[0], m[1],
        reinterpret_cast<float4*>(m[2]), m[3], m[4], v[0], v[1], reinterpret_cast<float4*>(v[2]), v[3], v[4], scales,
        opacities, grad_norm);
    return hipGetLastError();
}

}  // namespace gs
