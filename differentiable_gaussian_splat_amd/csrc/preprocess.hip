// Per-Gaussian projection (forward) and its chain rule (backward), one lane per
// Gaussian. This is the "preprocessing" phase of a 3D Gaussian Splatting
// training iteration (Odin page, Fig. 7 caption: phases P/R/B/U/C).
//
// Numerics. The 2D covariance is Sigma' = T T^T + lowpass I with
// T = (J R) Rq diag(s) (2x3), and its inverse is stored factored as
// Q = a (dx + beta dy)^2 + gamma dy^2 (a = C/det, beta = -B/C, gamma = 1/C).
// The projection forms it in double (see project). The chain rule works in
// fp32; where it needs T0 x T1 it uses the closed form
// T0 x T1 = (fx fy / z^3) s1 s2 s3 diag(1/s) Rq^T (mu - campos) (Lagrange's
// identity gives det(T T^T) = |T0 x T1|^2), which has no cancellation.
//
// No floating-point contraction in this file: a product feeds an add only
// where an fma is written out. The same functions are inlined into several
// kernels (one view or many, SH rows in LDS or in registers, adding or
// writing the gradients); without contraction each kernel rounds every
// operation exactly as written, so their results agree bit for bit. (Set
// before the includes, so that it covers the shared helpers too.)
#pragma clang fp contract(off)

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace gs {

namespace {

struct Geo {
    float x, y, z;      // camera-frame mean
    float qn[4];        // unit quaternion (w, x, y, z)
    float qnorm;
    float Rq[9];        // rotation of the Gaussian, row-major
    float V[6];         // J R (2x3)
    float P[6];         // V Rq (2x3)
    float T[6];         // P diag(s)
    float A0, B0, C0;   // T T^T
};

// Steps shared by the forward and the backward: camera transform, quaternion
// rotation, and the 2x3 factor T of the projected covariance.
__device__ __forceinline__ bool geometry(const DevCam& cam, float near_plane, float mx, float my, float mz,
                                         float s0, float s1, float s2, float4 q, Geo& g) {
    g.x = fmaf(cam.R[0], mx, fmaf(cam.R[1], my, fmaf(cam.R[2], mz, cam.t[0])));
    g.y = fmaf(cam.R[3], mx, fmaf(cam.R[4], my, fmaf(cam.R[5], mz, cam.t[1])));
    g.z = fmaf(cam.R[6], mx, fmaf(cam.R[7], my, fmaf(cam.R[8], mz, cam.t[2])));
    // the near-plane test on the depth formed in double, as the projection takes it
    const double zd = fma((double)cam.R[6], (double)mx,
                          fma((double)cam.R[7], (double)my, fma((double)cam.R[8], (double)mz, (double)cam.t[2])));
    if (!(zd > (double)near_plane)) return false;
    float qq = q.x * q.x + q.y * q.y + q.z * q.z + q.w * q.w;
    if (!(qq > 0.f) || !finitef(qq)) return false;
    g.qnorm = sqrtf(qq);
    float inv = 1.0f / g.qnorm;
    float w = q.x * inv, x = q.y * inv, y = q.z * inv, z = q.w * inv;
    g.qn[0] = w; g.qn[1] = x; g.qn[2] = y; g.qn[3] = z;
    g.Rq[0] = 1.f - 2.f * (y * y + z * z);
    g.Rq[1] = 2.f * (x * y - w * z);
    g.Rq[2] = 2.f * (x * z + w * y);
    g.Rq[3] = 2.f * (x * y + w * z);
    g.Rq[4] = 1.f - 2.f * (x * x + z * z);
    g.Rq[5] = 2.f * (y * z - w * x);
    g.Rq[6] = 2.f * (x * z - w * y);
    g.Rq[7] = 2.f * (y * z + w * x);
    g.Rq[8] = 1.f - 2.f * (x * x + y * y);
    // J = [[fx/z, 0, -fx x/z^2], [0, fy/z, -fy y/z^2]]; V = J R
    float iz = 1.0f / g.z;
    float xz = g.x * iz, yz = g.y * iz;
    float fxz = cam.fx * iz, fyz = cam.fy * iz;
    for (int j = 0; j < 3; ++j) {
        g.V[j] = fxz * fmaf(-xz, cam.R[6 + j], cam.R[j]);
        g.V[3 + j] = fyz * fmaf(-yz, cam.R[6 + j], cam.R[3 + j]);
    }
    float s[3] = {s0, s1, s2};
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 3; ++j) {
            float p = fmaf(g.V[3 * i], g.Rq[j], fmaf(g.V[3 * i + 1], g.Rq[3 + j], g.V[3 * i + 2] * g.Rq[6 + j]));
            g.P[3 * i + j] = p;
            g.T[3 * i + j] = p * s[j];
        }
    g.A0 = fmaf(g.T[0], g.T[0], fmaf(g.T[1], g.T[1], g.T[2] * g.T[2]));
    g.C0 = fmaf(g.T[3], g.T[3], fmaf(g.T[4], g.T[4], g.T[5] * g.T[5]));
    g.B0 = fmaf(g.T[0], g.T[3], fmaf(g.T[1], g.T[4], g.T[2] * g.T[5]));
    return true;
}

// Copies the first `used` floats of each of the 64 records of this block
// (records of `rec` floats from record `base`) into LDS rows of `stride`
// floats, and back. When the records are fully used and 16-byte aligned the
// wave's region is one contiguous run moved with float4 accesses, all issued
// before any is waited on; otherwise 8 records at a time.
constexpr int STAGE_V4 = 12;  // float4s per lane for 64 records of up to 48 floats

__device__ __forceinline__ void stage_in(const float* __restrict__ src, float* dst, int base, int n, int rec,
                                         int used, int stride) {
    const int lane = threadIdx.x;
    const int cnt = min(64, n - base);
    const float* r0 = src + (size_t)base * rec;
    if (used == rec && rec <= 48 && ((uintptr_t)r0 & 15u) == 0) {
        const int total = cnt * rec;
        float4 v[STAGE_V4];
#pragma unroll
        for (int m = 0; m < STAGE_V4; ++m) {
            const int f = (m * 64 + lane) * 4;
            if (f + 3 < total) v[m] = *reinterpret_cast<const float4*>(r0 + f);
        }
#pragma unroll
        for (int m = 0; m < STAGE_V4; ++m) {
            const int f = (m * 64 + lane) * 4;
            const float e4[4] = {v[m].x, v[m].y, v[m].z, v[m].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int idx = f + c;
                if (idx < total) {
                    int j, e;
                    divmod_small(idx, rec, j, e);
                    dst[j * stride + e] = f + 3 < total ? e4[c] : r0[idx];
                }
            }
        }
        return;
    }
    for (int j0 = 0; j0 < cnt; j0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (j0 + u < cnt && lane < used) ? src[(size_t)(base + j0 + u) * rec + lane] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u < cnt && lane < used) dst[(j0 + u) * stride + lane] = v[u];
        for (int e = lane + 64; e < used; e += 64)
            for (int u = 0; u < 8 && j0 + u < cnt; ++u) dst[(j0 + u) * stride + e] = src[(size_t)(base + j0 + u) * rec + e];
    }
}

__device__ __forceinline__ void stage_out(const float* src, float* __restrict__ dst, int base, int n, int rec,
                                          int used, int stride) {
    const int lane = threadIdx.x;
    const int cnt = min(64, n - base);
    float* r0 = dst + (size_t)base * rec;
    if (used == rec && rec <= 48 && ((uintptr_t)r0 & 15u) == 0) {
        const int total = cnt * rec;
#pragma unroll
        for (int m = 0; m < STAGE_V4; ++m) {
            const int f = (m * 64 + lane) * 4;
            float e4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int idx = f + c;
                e4[c] = 0.f;
                if (idx < total) {
                    int j, e;
                    divmod_small(idx, rec, j, e);
                    e4[c] = src[j * stride + e];
                }
            }
            if (f + 3 < total) {
                *reinterpret_cast<float4*>(r0 + f) = make_float4(e4[0], e4[1], e4[2], e4[3]);
            } else {
                for (int c = 0; c < 4; ++c)
                    if (f + c < total) r0[f + c] = e4[c];
            }
        }
        return;
    }
    for (int j = 0; j < cnt; ++j)
        for (int e = lane; e < used; e += 64) dst[(size_t)(base + j) * rec + e] = src[j * stride + e];
}

// As stage_out, adding the LDS rows into the destination records.
__device__ __forceinline__ void stage_out_add(const float* src, float* __restrict__ dst, int base, int n, int rec,
                                              int used, int stride) {
    const int lane = threadIdx.x;
    const int cnt = min(64, n - base);
    float* r0 = dst + (size_t)base * rec;
    if (used == rec && rec <= 48 && ((uintptr_t)r0 & 15u) == 0) {
        const int total = cnt * rec;
        float4 v[STAGE_V4];
#pragma unroll
        for (int m = 0; m < STAGE_V4; ++m) {
            const int f = (m * 64 + lane) * 4;
            if (f + 3 < total) v[m] = *reinterpret_cast<const float4*>(r0 + f);
        }
#pragma unroll
        for (int m = 0; m < STAGE_V4; ++m) {
            const int f = (m * 64 + lane) * 4;
            float e4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int idx = f + c;
                e4[c] = 0.f;
                if (idx < total) {
                    int j, e;
                    divmod_small(idx, rec, j, e);
                    e4[c] = src[j * stride + e];
                }
            }
            if (f + 3 < total) {
                *reinterpret_cast<float4*>(r0 + f) =
                    make_float4(v[m].x + e4[0], v[m].y + e4[1], v[m].z + e4[2], v[m].w + e4[3]);
            } else {
                for (int c = 0; c < 4; ++c)
                    if (f + c < total) r0[f + c] += e4[c];
            }
        }
        return;
    }
    for (int j = 0; j < cnt; ++j)
        for (int e = lane; e < used; e += 64) dst[(size_t)(base + j) * rec + e] += src[j * stride + e];
}

// Blocks with few visible Gaussians (a camera that sees a fifth of the scene)
// move only the visible lanes' rows, each lane its own; dense blocks stage all
// 64 rows with coalesced accesses.
constexpr int SH_DENSE = 16;
// Adding degree-3 gradients, blocks with at most this many drawn Gaussians take the register kernel.
constexpr int BWD_REGS_MAX_VISIBLE = 32;

__device__ __forceinline__ void copy_own_row(const float* __restrict__ src, float* row, size_t g, int rec, int used) {
    const float* r = src + g * (size_t)rec;
    if ((used & 3) == 0 && ((uintptr_t)r & 15u) == 0) {
        for (int e = 0; e < used; e += 4) {
            const float4 v = *reinterpret_cast<const float4*>(r + e);
            row[e] = v.x;
            row[e + 1] = v.y;
            row[e + 2] = v.z;
            row[e + 3] = v.w;
        }
    } else {
        for (int e = 0; e < used; ++e) row[e] = r[e];
    }
}

__device__ __forceinline__ void add_own_row(const float* row, float* __restrict__ dst, size_t g, int rec, int used) {
    float* r = dst + g * (size_t)rec;
    if ((used & 3) == 0 && ((uintptr_t)r & 15u) == 0) {
        for (int e = 0; e < used; e += 4) {
            float4 v = *reinterpret_cast<const float4*>(r + e);
            v.x += row[e];
            v.y += row[e + 1];
            v.z += row[e + 2];
            v.w += row[e + 3];
            *reinterpret_cast<float4*>(r + e) = v;
        }
    } else {
        for (int e = 0; e < used; ++e) r[e] += row[e];
    }
}

// SH rows move through LDS in chunks of CHUNK_K coefficients (3 CHUNK_K floats
// per Gaussian; 8 rows: a 64-Gaussian block needs 6.4 KB of LDS, not 12.5 KB):
// LDS, not registers, is what limits the resident waves of these kernels.
constexpr int CHUNK_K = 8;
constexpr int CHUNK_F = 3 * CHUNK_K;
constexpr int CHUNK_Q = CHUNK_F / 4;                        // float4s per record and chunk
constexpr int CHUNKS = (16 + CHUNK_K - 1) / CHUNK_K;        // chunks of the 16 rows of degree 3
constexpr int CHUNK_STRIDE = CHUNK_F + 1;  // odd: lanes reading their own row hit distinct banks
static_assert(CHUNK_K % 4 == 0, "a chunk is whole float4s");

// Floats [c0, c0 + used) (used <= CHUNK_F) of each of the block's records
// (records of `rec` floats from record `base`) to LDS rows of CHUNK_STRIDE
// floats. With 16-byte aligned pieces the wave moves them as float4s, all
// loads issued before any is waited on; otherwise 8 records at a time.
__device__ __forceinline__ void chunk_in(const float* __restrict__ src, float* dst, int base, int n, int rec, int c0,
                                         int used) {
    const int lane = threadIdx.x;
    const int cnt = min(64, n - base);
    const float* r0 = src + (size_t)base * rec + c0;
    if (((rec | c0 | used) & 3) == 0 && ((uintptr_t)src & 15u) == 0) {
        const int q = used >> 2;  // float4s per record, <= CHUNK_Q
        const int total = cnt * q;
        float4 v[CHUNK_Q];
#pragma unroll
        for (int m = 0; m < CHUNK_Q; ++m) {
            const int f = m * 64 + lane;
            if (f < total) {
                int j, c;
                divmod_small(f, q, j, c);
                v[m] = *reinterpret_cast<const float4*>(r0 + (size_t)j * rec + 4 * c);
            }
        }
#pragma unroll
        for (int m = 0; m < CHUNK_Q; ++m) {
            const int f = m * 64 + lane;
            if (f < total) {
                int j, c;
                divmod_small(f, q, j, c);
                float* d = dst + j * CHUNK_STRIDE + 4 * c;
                d[0] = v[m].x;
                d[1] = v[m].y;
                d[2] = v[m].z;
                d[3] = v[m].w;
            }
        }
        return;
    }
    for (int j0 = 0; j0 < cnt; j0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (j0 + u < cnt && lane < used) ? r0[(size_t)(j0 + u) * rec + lane] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u < cnt && lane < used) dst[(j0 + u) * CHUNK_STRIDE + lane] = v[u];
    }
}

// One lane's own record: floats [c0, c0 + used) to its LDS row.
__device__ __forceinline__ void chunk_in_own(const float* __restrict__ src, float* row, size_t g, int rec, int c0,
                                             int used) {
    const float* r = src + g * (size_t)rec + c0;
    if (((used & 3) == 0) && ((uintptr_t)r & 15u) == 0) {
        for (int e = 0; e < used; e += 4) {
            const float4 v = *reinterpret_cast<const float4*>(r + e);
            row[e] = v.x;
            row[e + 1] = v.y;
            row[e + 2] = v.z;
            row[e + 3] = v.w;
        }
    } else {
        for (int e = 0; e < used; ++e) row[e] = r[e];
    }
}

// Outputs of a culled Gaussian: zero radius, no tiles, zeros elsewhere.
__device__ __forceinline__ void write_culled(size_t g, float2* __restrict__ means2d, float* __restrict__ depths,
                                             float4* __restrict__ conic_op, float* __restrict__ rgb_out,
                                             int* __restrict__ radii, uint32_t* __restrict__ tiles,
                                             uint8_t* __restrict__ clamped) {
    means2d[g] = make_float2(0.f, 0.f);
    depths[g] = 0.f;
    conic_op[g] = make_float4(0.f, 0.f, 0.f, 0.f);
    rgb_out[3 * g] = 0.f;
    rgb_out[3 * g + 1] = 0.f;
    rgb_out[3 * g + 2] = 0.f;
    radii[g] = 0;
    tiles[g] = 0;
    clamped[g] = 0;
}

// Screen-space footprint of one Gaussian in one camera.
struct Proj {
    float u, v, depth, a, beta, gamma;
    int r, X0, X1, Y0, Y1;
};

// The projection of one Gaussian (finite inputs) into one camera: EWA conic
// in factored form, 3-sigma radius, tile rectangle. False when it is culled.
//
// Evaluated in double from the fp32 inputs and rounded once per output. The
// entries of T = (J R) Rq diag(s) are dot products that cancel when a
// Gaussian's long axes lie nearly along the viewing ray, and the conic is the
// inverse of T T^T + lowpass I: in fp32 both lose digits in proportion to
// those condition numbers (thin footprints seen edge-on reach 10^5). In double
// the outputs carry only their own fp32 rounding, for about a hundred extra
// double operations per Gaussian in a kernel bound by its memory traffic.
__device__ __forceinline__ bool project(const DevCam& cam, float lowpass, float near_plane, float mx, float my,
                                       float mz, float s0, float s1, float s2, float4 q, Proj& p) {
    const double X = mx, Y = my, Z = mz;
    double R[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) R[i] = (double)cam.R[i];
    const double x = fma(R[0], X, fma(R[1], Y, fma(R[2], Z, (double)cam.t[0])));
    const double y = fma(R[3], X, fma(R[4], Y, fma(R[5], Z, (double)cam.t[1])));
    const double z = fma(R[6], X, fma(R[7], Y, fma(R[8], Z, (double)cam.t[2])));
    if (!(z > (double)near_plane)) return false;
    const double qw = q.x, qx = q.y, qy = q.z, qz = q.w;
    const double qq = fma(qw, qw, fma(qx, qx, fma(qy, qy, qz * qz)));
    if (!(qq > 0.0)) return false;
    const double inv = 1.0 / sqrt(qq);
    const double w = qw * inv, a = qx * inv, b = qy * inv, c = qz * inv;
    const double Rq[9] = {1.0 - 2.0 * (b * b + c * c), 2.0 * (a * b - w * c),       2.0 * (a * c + w * b),
                          2.0 * (a * b + w * c),       1.0 - 2.0 * (a * a + c * c), 2.0 * (b * c - w * a),
                          2.0 * (a * c - w * b),       2.0 * (b * c + w * a),       1.0 - 2.0 * (a * a + b * b)};
    // J = [[fx/z, 0, -fx x/z^2], [0, fy/z, -fy y/z^2]]; V = J R; T = V Rq diag(s)
    const double iz = 1.0 / z;
    const double xz = x * iz, yz = y * iz;
    const double fxz = (double)cam.fx * iz, fyz = (double)cam.fy * iz;
    double V[6];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        V[j] = fxz * fma(-xz, R[6 + j], R[j]);
        V[3 + j] = fyz * fma(-yz, R[6 + j], R[3 + j]);
    }
    const double s[3] = {s0, s1, s2};
    double T[6];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            T[3 * i + j] = fma(V[3 * i], Rq[j], fma(V[3 * i + 1], Rq[3 + j], V[3 * i + 2] * Rq[6 + j])) * s[j];
    const double lp = lowpass;
    const double A = fma(T[0], T[0], fma(T[1], T[1], fma(T[2], T[2], lp)));
    const double C = fma(T[3], T[3], fma(T[4], T[4], fma(T[5], T[5], lp)));
    const double B = fma(T[0], T[3], fma(T[1], T[4], T[2] * T[5]));
    const double det = fma(A, C, -B * B);
    if (!(det > 0.0 && C > 0.0)) return false;
    p.a = (float)(C / det);
    p.beta = (float)(-B / C);
    p.gamma = (float)(1.0 / C);
    if (!(finitef(p.a) && p.a > 0.f && finitef(p.beta) && p.gamma > 0.f)) return false;
    const double half = 0.5 * (A - C);
    const double lam = 0.5 * (A + C) + sqrt(fma(half, half, B * B));
    const double extent = 3.0 * sqrt(lam);
    const double u = fma((double)cam.fx, xz, (double)cam.cx);
    const double v = fma((double)cam.fy, yz, (double)cam.cy);
    if (!(fabs(u) <= (double)BIG && fabs(v) <= (double)BIG && extent <= (double)BIG)) return false;  // also on NaN
    p.u = (float)u;
    p.v = (float)v;
    p.depth = (float)z;
    p.r = (int)ceil(extent);
    // the rectangle from the stored (rounded) screen mean: binning reads the same values
    return tile_rect(p.u, p.v, p.r, cam.TX, cam.TY, p.X0, p.X1, p.Y0, p.Y1);
}

// The projection of one 2D Gaussian surfel (finite inputs): tangent axes
// t_u, t_v (the first two columns of its rotation) scaled by (s_u, s_v) and
// turned into the camera frame, a = s_u R t_u and b = s_v R t_v; the surfel
// point (u, v) is the camera point X + u a + v b, so the homogeneous screen
// point is M (u, v, 1) with M = K [a | b | X]. Its 3-sigma disc must lie beyond
// the near plane; the bounding box of the disc's image (an ellipse) follows
// from the dual conic M diag(1, 1, -1/9) M^T, whose vertical and horizontal
// tangents solve a quadratic each. r is the largest distance from the
// projected centre c to a side of that box, at least 3 sigma of the screen
// filter (variance 1/2). In double, rounded once per output, as project().
struct SurfelProj {
    float M[9];
    float u, v, depth;
    int r, X0, X1, Y0, Y1;
};

constexpr double SURFEL_FILTER_VAR = 0.5;  // screen filter variance, pixels^2

__device__ __forceinline__ bool project_surfel(const DevCam& cam, float near_plane, float mx, float my, float mz,
                                              float su, float sv, float4 q, SurfelProj& p) {
    const double X = mx, Y = my, Z = mz;
    double R[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) R[i] = (double)cam.R[i];
    const double x = fma(R[0], X, fma(R[1], Y, fma(R[2], Z, (double)cam.t[0])));
    const double y = fma(R[3], X, fma(R[4], Y, fma(R[5], Z, (double)cam.t[1])));
    const double z = fma(R[6], X, fma(R[7], Y, fma(R[8], Z, (double)cam.t[2])));
    if (!(z > (double)near_plane)) return false;
    const double qw = q.x, qx = q.y, qy = q.z, qz = q.w;
    const double qq = fma(qw, qw, fma(qx, qx, fma(qy, qy, qz * qz)));
    if (!(qq > 0.0)) return false;
    const double inv = 1.0 / sqrt(qq);
    const double w = qw * inv, a1 = qx * inv, b1 = qy * inv, c1 = qz * inv;
    // columns 0 and 1 of the unit quaternion's rotation
    const double tu[3] = {1.0 - 2.0 * (b1 * b1 + c1 * c1), 2.0 * (a1 * b1 + w * c1), 2.0 * (a1 * c1 - w * b1)};
    const double tv[3] = {2.0 * (a1 * b1 - w * c1), 1.0 - 2.0 * (a1 * a1 + c1 * c1), 2.0 * (b1 * c1 + w * a1)};
    double a[3], b[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        a[i] = (double)su * fma(R[3 * i], tu[0], fma(R[3 * i + 1], tu[1], R[3 * i + 2] * tu[2]));
        b[i] = (double)sv * fma(R[3 * i], tv[0], fma(R[3 * i + 1], tv[1], R[3 * i + 2] * tv[2]));
    }
    if (!(z - 3.0 * sqrt(fma(a[2], a[2], b[2] * b[2])) > (double)near_plane)) return false;
    const double fx = cam.fx, fy = cam.fy, cx = cam.cx, cy = cam.cy;
    const double M[9] = {fma(fx, a[0], cx * a[2]), fma(fx, b[0], cx * b[2]), fma(fx, x, cx * z),
                         fma(fy, a[1], cy * a[2]), fma(fy, b[1], cy * b[2]), fma(fy, y, cy * z),
                         a[2],                     b[2],                     z};
    const double u = fma(fx, x / z, cx), v = fma(fy, y / z, cy);
    // dual conic entries D_ij = M_i0 M_j0 + M_i1 M_j1 - M_i2 M_j2 / 9
    auto dual = [&](int i, int j) { return fma(M[3 * i], M[3 * j], fma(M[3 * i + 1], M[3 * j + 1], -M[3 * i + 2] * M[3 * j + 2] / 9.0)); };
    const double D22 = dual(2, 2);
    double ext = 3.0 * sqrt(SURFEL_FILTER_VAR);
    const double cen[2] = {u, v};
#pragma unroll
    for (int ax = 0; ax < 2; ++ax) {
        const double A = dual(ax, ax), B = dual(ax, 2);
        const double disc = fma(B, B, -A * D22);
        if (!(disc >= 0.0) || D22 == 0.0) return false;
        const double sq = sqrt(disc);
        ext = fmax(ext, fmax(fabs((B + sq) / D22 - cen[ax]), fabs((B - sq) / D22 - cen[ax])));
    }
    if (!(fabs(u) <= (double)BIG && fabs(v) <= (double)BIG && ext <= (double)BIG)) return false;  // also on NaN
#pragma unroll
    for (int i = 0; i < 9; ++i) p.M[i] = (float)M[i];
    p.u = (float)u;
    p.v = (float)v;
    p.depth = (float)z;
    p.r = (int)ceil(ext);
    return tile_rect(p.u, p.v, p.r, cam.TX, cam.TY, p.X0, p.X1, p.Y0, p.Y1);
}

template <bool SURFEL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(6))) void k_preprocess(
    DevCam cam, int K, int sh_rows, float lowpass, float near_plane, int n,
    const float* __restrict__ means, const float* __restrict__ scales, const float4* __restrict__ quats,
    const float* __restrict__ opac, const float* __restrict__ sh,
    float2* __restrict__ means2d, float* __restrict__ depths, float4* __restrict__ conic_op,
    float* __restrict__ rgb_out, int* __restrict__ radii, uint32_t* __restrict__ tiles,
    uint8_t* __restrict__ clamped) {
    // SURFEL: scales hold (s_u, s_v) and conic_op three float4 per surfel, (M row 0, o),
    // (M row 1, c_x), (M row 2, c_y); otherwise three scales and one float4 (a, beta, gamma, o).
    extern __shared__ float s_sh[];
    const int base = blockIdx.x * 64;
    const int gi = base + threadIdx.x;
    const bool live = gi < n;
    const size_t g = live ? (size_t)gi : (size_t)base;
    float mx = means[3 * g], my = means[3 * g + 1], mz = means[3 * g + 2];
    constexpr int NS = SURFEL ? 2 : 3;
    float s0 = scales[NS * g], s1 = scales[NS * g + 1], s2 = SURFEL ? 1.f : scales[NS * g + 2];
    float4 q = quats[g];
    float o = opac[g];

    bool ok = live && finitef(mx) && finitef(my) && finitef(mz) && finitef(s0) && finitef(s1) && finitef(s2) &&
              finitef(q.x) && finitef(q.y) && finitef(q.z) && finitef(q.w) && finitef(o);
    // the projection's outputs first: the SH rows staged below need the registers
    if constexpr (SURFEL) {
        SurfelProj pr;
        ok = ok && project_surfel(cam, near_plane, mx, my, mz, s0, s1, q, pr);
        if (live) {
            if (ok) {
                means2d[g] = make_float2(pr.u, pr.v);
                depths[g] = pr.depth;
                conic_op[3 * g] = make_float4(pr.M[0], pr.M[1], pr.M[2], o);
                conic_op[3 * g + 1] = make_float4(pr.M[3], pr.M[4], pr.M[5], pr.u);
                conic_op[3 * g + 2] = make_float4(pr.M[6], pr.M[7], pr.M[8], pr.v);
                radii[g] = pr.r;
                tiles[g] = (uint32_t)((pr.X1 - pr.X0 + 1) * (pr.Y1 - pr.Y0 + 1));
            } else {
                write_culled(g, means2d, depths, conic_op + 2 * g, rgb_out, radii, tiles, clamped);  // [3 g]
                conic_op[3 * g + 1] = conic_op[3 * g + 2] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    } else {
        Proj pr;
        ok = ok && project(cam, lowpass, near_plane, mx, my, mz, s0, s1, s2, q, pr);
        if (live) {
            if (ok) {
                means2d[g] = make_float2(pr.u, pr.v);
                depths[g] = pr.depth;
                conic_op[g] = make_float4(pr.a, pr.beta, pr.gamma, o);
                radii[g] = pr.r;
                tiles[g] = (uint32_t)((pr.X1 - pr.X0 + 1) * (pr.Y1 - pr.Y0 + 1));
            } else {
                write_culled(g, means2d, depths, conic_op, rgb_out, radii, tiles, clamped);
            }
        }
    }
    // colour from the SH rows of the visible Gaussians, chunk by chunk through LDS
    float dx = mx - cam.campos[0], dy = my - cam.campos[1], dz = mz - cam.campos[2];
    float dist = sqrtf(fmaf(dx, dx, fmaf(dy, dy, dz * dz)));
    float id = 1.0f / dist;
    float Y[16];
    sh_eval(K, dx * id, dy * id, dz * id, Y);
    float raw[3] = {0.5f, 0.5f, 0.5f};
    float* shg = s_sh + threadIdx.x * CHUNK_STRIDE;
    const bool dense = __popcll(__ballot(ok)) > SH_DENSE;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const int k0 = c * CHUNK_K;
        if (k0 >= K) break;
        const int kc = min(CHUNK_K, K - k0);
        if (c > 0) __syncthreads();  // the previous chunk has been read
        if (dense) chunk_in(sh, s_sh, base, n, 3 * sh_rows, 3 * k0, 3 * kc);
        else if (ok) chunk_in_own(sh, shg, g, 3 * sh_rows, 3 * k0, 3 * kc);
        __syncthreads();
        if (ok) {
#pragma unroll
            for (int k = 0; k < CHUNK_K; ++k) {
                if (k >= kc) break;
                raw[0] = fmaf(shg[3 * k], Y[k0 + k], raw[0]);
                raw[1] = fmaf(shg[3 * k + 1], Y[k0 + k], raw[1]);
                raw[2] = fmaf(shg[3 * k + 2], Y[k0 + k], raw[2]);
            }
        }
    }
    if (!ok) return;
    if (!(dist > 0.f && finitef(raw[0]) && finitef(raw[1]) && finitef(raw[2]))) {  // culled after all
        if constexpr (SURFEL) {
            write_culled(g, means2d, depths, conic_op + 2 * g, rgb_out, radii, tiles, clamped);  // [3 g]
            conic_op[3 * g + 1] = conic_op[3 * g + 2] = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            write_culled(g, means2d, depths, conic_op, rgb_out, radii, tiles, clamped);
        }
        return;
    }
    uint8_t cl = 0;
    for (int c = 0; c < 3; ++c) {
        const bool neg = raw[c] < 0.f;
        cl |= (uint8_t)(neg ? (1u << c) : 0u);
        rgb_out[3 * g + c] = neg ? 0.f : raw[c];
    }
    clamped[g] = cl;
}

// Gradient contributions of one view to one Gaussian's activated parameters
// and to its screen mean (u, v).
struct ViewGrad {
    float dmu[3], ds[3], dq[4], d_o, du, dv;
};

// The chain rule of one view for one drawn Gaussian, from its summed pixel
// terms g2 (a grad2d record) and its conic / opacity `con`. `sh` gives the SH
// coefficients (sh.coef(k, c)) and takes the gradient of row k (sh.grad(k, d0,
// d1, d2)), row by row in order. False when the Gaussian does not project (its
// contribution is zero; sh.grad is not called).
template <class Sh>
__device__ __forceinline__ bool view_grad(const DevCam& cam, int K, float lowpass, float near_plane, float mx, float my,
                                          float mz, const float* s, float4 q, float4 con, const float4* g2, uint8_t cl,
                                          Sh& sh, ViewGrad& out) {
    float4 ga = g2[0], gb = g2[1], gc = g2[2];
    float dr[3] = {ga.x, ga.y, ga.z};
    float Sh_ = ga.w, Sww = gb.x, Swy = gb.y, Syy = gb.z, Sw = gb.w, Sy = gc.x;
    float a = con.x, beta = con.y, gamma = con.z, o = con.w;

    // pixel sums -> gradients of (u, v, opacity); dL/dQ = -h/2 and dQ/du = -2 a w
    out.d_o = o != 0.f ? Sh_ / o : 0.f;
    float du = a * Sw;
    float dv = fmaf(a * beta, Sw, gamma * Sy);
    out.du = du;
    out.dv = dv;

    Geo geo;
    if (!geometry(cam, near_plane, mx, my, mz, s[0], s[1], s[2], q, geo)) return false;
    float ddx = mx - cam.campos[0], ddy = my - cam.campos[1], ddz = mz - cam.campos[2];

    // dL/dSigma' = (1/2) sum_p h (Sigma'^-1 d)(Sigma'^-1 d)^T with Sigma'^-1 d = a w e + gamma dy f,
    // e = (1, beta), f = (0, 1). Since Sigma' = T T^T + lowpass I, dT = 2 dL/dSigma' T
    //   = e k^T + f m^T,  k = a^2 Sww U + a gamma Swy T1,  m = a gamma Swy U + gamma^2 Syy T1,
    // with U = e^T T = T0 + beta T1. For a thin footprint T0 and T1 are nearly parallel and
    // T0 + beta T1 cancels; U = gamma (T1 x (T0 x T1) + lowpass T0) is the same vector without
    // the cancellation, T0 x T1 taken in the closed form the projection uses.
    float e0 = fmaf(geo.Rq[0], ddx, fmaf(geo.Rq[3], ddy, geo.Rq[6] * ddz));
    float e1 = fmaf(geo.Rq[1], ddx, fmaf(geo.Rq[4], ddy, geo.Rq[7] * ddz));
    float e2 = fmaf(geo.Rq[2], ddx, fmaf(geo.Rq[5], ddy, geo.Rq[8] * ddz));
    float izc = 1.0f / geo.z;
    float kk = cam.fx * cam.fy * izc * izc * izc;
    float c0 = kk * e0 * s[1] * s[2], c1 = kk * e1 * s[0] * s[2], c2 = kk * e2 * s[0] * s[1];
    const float* T0 = geo.T;
    const float* T1 = geo.T + 3;
    float U[3] = {gamma * fmaf(lowpass, T0[0], fmaf(T1[1], c2, -T1[2] * c1)),
                  gamma * fmaf(lowpass, T0[1], fmaf(T1[2], c0, -T1[0] * c2)),
                  gamma * fmaf(lowpass, T0[2], fmaf(T1[0], c1, -T1[1] * c0))};
    float kU = a * a * Sww, kT = a * gamma * Swy, mT = gamma * gamma * Syy;
    float dT[6];
    for (int j = 0; j < 3; ++j) {
        float kj = fmaf(kU, U[j], kT * T1[j]);
        float mj = fmaf(kT, U[j], mT * T1[j]);
        dT[j] = kj;
        dT[3 + j] = fmaf(beta, kj, mj);
    }
    // T = P diag(s): dP = dT diag(s), ds_j = sum_i dT_ij P_ij
    float dP[6];
    for (int j = 0; j < 3; ++j) {
        out.ds[j] = fmaf(dT[j], geo.P[j], dT[3 + j] * geo.P[3 + j]);
        dP[j] = dT[j] * s[j];
        dP[3 + j] = dT[3 + j] * s[j];
    }
    // P = V Rq: dV = dP Rq^T, dRq = V^T dP
    float dV[6], dRq[9];
    for (int i = 0; i < 2; ++i)
        for (int k = 0; k < 3; ++k)
            dV[3 * i + k] = fmaf(dP[3 * i], geo.Rq[3 * k], fmaf(dP[3 * i + 1], geo.Rq[3 * k + 1], dP[3 * i + 2] * geo.Rq[3 * k + 2]));
    for (int k = 0; k < 3; ++k)
        for (int j = 0; j < 3; ++j) dRq[3 * k + j] = fmaf(geo.V[k], dP[j], geo.V[3 + k] * dP[3 + j]);
    // V = J R: dJ = dV R^T (only the non-constant entries of J are needed)
    float dJ00 = fmaf(dV[0], cam.R[0], fmaf(dV[1], cam.R[1], dV[2] * cam.R[2]));
    float dJ02 = fmaf(dV[0], cam.R[6], fmaf(dV[1], cam.R[7], dV[2] * cam.R[8]));
    float dJ11 = fmaf(dV[3], cam.R[3], fmaf(dV[4], cam.R[4], dV[5] * cam.R[5]));
    float dJ12 = fmaf(dV[3], cam.R[6], fmaf(dV[4], cam.R[7], dV[5] * cam.R[8]));
    // camera-space mean, through J and through (u, v)
    float iz = 1.0f / geo.z, iz2 = iz * iz, iz3 = iz2 * iz;
    float fx = cam.fx, fy = cam.fy;
    float xb = fmaf(-fx * iz2, dJ02, fx * iz * du);
    float yb = fmaf(-fy * iz2, dJ12, fy * iz * dv);
    float zb = -fx * iz2 * dJ00 - fy * iz2 * dJ11 + 2.f * fx * geo.x * iz3 * dJ02 + 2.f * fy * geo.y * iz3 * dJ12 -
               fx * geo.x * iz2 * du - fy * geo.y * iz2 * dv;
    float dmu[3];
    for (int j = 0; j < 3; ++j) dmu[j] = fmaf(cam.R[j], xb, fmaf(cam.R[3 + j], yb, cam.R[6 + j] * zb));

    // quaternion: dL/dqn_k = sum_ij dRq_ij dRq_ij/dqn_k, then the normalisation's tangent projection
    float w = geo.qn[0], x = geo.qn[1], y = geo.qn[2], z = geo.qn[3];
    float gw = 2.f * (-z * dRq[1] + y * dRq[2] + z * dRq[3] - x * dRq[5] - y * dRq[6] + x * dRq[7]);
    float gx = 2.f * (y * dRq[1] + z * dRq[2] + y * dRq[3] - 2.f * x * dRq[4] - w * dRq[5] + z * dRq[6] +
                      w * dRq[7] - 2.f * x * dRq[8]);
    float gy = 2.f * (-2.f * y * dRq[0] + x * dRq[1] + w * dRq[2] + x * dRq[3] + z * dRq[5] - w * dRq[6] +
                      z * dRq[7] - 2.f * y * dRq[8]);
    float gz = 2.f * (-2.f * z * dRq[0] - w * dRq[1] + x * dRq[2] + w * dRq[3] - 2.f * z * dRq[4] + y * dRq[5] +
                      x * dRq[6] + y * dRq[7]);
    float qdot = w * gw + x * gx + y * gy + z * gz;
    float iq = 1.0f / geo.qnorm;
    out.dq[0] = (gw - qdot * w) * iq;
    out.dq[1] = (gx - qdot * x) * iq;
    out.dq[2] = (gy - qdot * y) * iq;
    out.dq[3] = (gz - qdot * z) * iq;

    // colour: rgb = max(0, sum_k sh_k Y_k(dir) + 0.5), dir = (mu - campos) / |mu - campos|
    float dcol[3];
    for (int c = 0; c < 3; ++c) dcol[c] = (cl >> c) & 1 ? 0.f : dr[c];
    float dist = sqrtf(fmaf(ddx, ddx, fmaf(ddy, ddy, ddz * ddz)));
    float id = 1.0f / dist;
    float dxn = ddx * id, dyn = ddy * id, dzn = ddz * id;
    float Y[16], wk[16];
    sh_eval(K, dxn, dyn, dzn, Y);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (k < K) {
            wk[k] = fmaf(sh.coef(k, 0), dcol[0], fmaf(sh.coef(k, 1), dcol[1], sh.coef(k, 2) * dcol[2]));
            sh.grad(k, Y[k] * dcol[0], Y[k] * dcol[1], Y[k] * dcol[2]);
        }
    }
    float3 gdir = make_float3(0.f, 0.f, 0.f);
    sh_grad_accum(K, dxn, dyn, dzn, wk, gdir);
    float dd = dxn * gdir.x + dyn * gdir.y + dzn * gdir.z;
    out.dmu[0] = dmu[0] + (gdir.x - dxn * dd) * id;
    out.dmu[1] = dmu[1] + (gdir.y - dyn * dd) * id;
    out.dmu[2] = dmu[2] + (gdir.z - dzn * dd) * id;
    return true;
}

// An SH row in LDS whose coefficients are replaced, row by row, by their
// gradient contributions.
struct ShInPlace {
    float* row;
    __device__ float coef(int k, int c) const { return row[3 * k + c]; }
    __device__ void grad(int k, float d0, float d1, float d2) {
        row[3 * k] = d0;
        row[3 * k + 1] = d1;
        row[3 * k + 2] = d2;
    }
    __device__ void zero(int K) {
        for (int k = 0; k < 3 * K; ++k) row[k] = 0.f;
    }
};

// A row of 16 SH coefficients held in registers (every index a constant
// once the loops over k are unrolled), replaced in place by its gradient.
struct ShRegs16 {
    float c[48];
    __device__ float coef(int k, int ch) const { return c[3 * k + ch]; }
    __device__ void grad(int k, float d0, float d1, float d2) {
        c[3 * k] = d0;
        c[3 * k + 1] = d1;
        c[3 * k + 2] = d2;
    }
    __device__ void zero(int) {
#pragma unroll
        for (int e = 0; e < 48; ++e) c[e] = 0.f;
    }
};

// The chain rule for Gaussian gi. shg is its SH row in LDS: the coefficients
// on entry, replaced by their gradient contributions (zero for a culled
// Gaussian), which the caller adds to (or, with OVERWRITE, writes as) dL/dsh.
// The other outputs are added to, or with OVERWRITE written (zeros for a
// culled Gaussian); without OVERWRITE those of culled Gaussians are left
// untouched.
template <bool OVERWRITE, class ShAcc>
__device__ __forceinline__ void chain_rule(
    const DevCam& cam, int K, float lowpass, float near_plane, int gi,
    const float* __restrict__ means, const float* __restrict__ scales, const float4* __restrict__ quats,
    ShAcc& sh, const float4* __restrict__ conic_op, const int* __restrict__ radii,
    const uint8_t* __restrict__ clamped, const float* __restrict__ grad2d,
    float* __restrict__ d_means, float* __restrict__ d_scales, float* __restrict__ d_quats,
    float* __restrict__ d_opac, float* __restrict__ d_means2d, const DensifyStats& stats) {
    size_t g = (size_t)gi;
    auto culled = [&]() {
        sh.zero(K);
        if (OVERWRITE) {
            d_means[3 * g] = d_means[3 * g + 1] = d_means[3 * g + 2] = 0.f;
            d_scales[3 * g] = d_scales[3 * g + 1] = d_scales[3 * g + 2] = 0.f;
            reinterpret_cast<float4*>(d_quats)[g] = make_float4(0.f, 0.f, 0.f, 0.f);
            d_opac[g] = 0.f;
            if (d_means2d) d_means2d[2 * g] = d_means2d[2 * g + 1] = 0.f;
        }
    };
    if (radii[g] <= 0) return culled();
    const float s[3] = {scales[3 * g], scales[3 * g + 1], scales[3 * g + 2]};
    ViewGrad vg;
    if (!view_grad(cam, K, lowpass, near_plane, means[3 * g], means[3 * g + 1], means[3 * g + 2], s, quats[g],
                   conic_op[g], reinterpret_cast<const float4*>(grad2d + g * GRAD2D_STRIDE), clamped[g], sh, vg))
        return culled();

    // prior values: zero when overwriting (the compiler drops the loads)
    auto prior = [&](const float* p) { return OVERWRITE ? 0.f : *p; };
    d_means[3 * g] = prior(&d_means[3 * g]) + vg.dmu[0];
    d_means[3 * g + 1] = prior(&d_means[3 * g + 1]) + vg.dmu[1];
    d_means[3 * g + 2] = prior(&d_means[3 * g + 2]) + vg.dmu[2];
    d_scales[3 * g] = prior(&d_scales[3 * g]) + vg.ds[0];
    d_scales[3 * g + 1] = prior(&d_scales[3 * g + 1]) + vg.ds[1];
    d_scales[3 * g + 2] = prior(&d_scales[3 * g + 2]) + vg.ds[2];
    float4* dq = reinterpret_cast<float4*>(d_quats) + g;
    float4 dq0 = OVERWRITE ? make_float4(0.f, 0.f, 0.f, 0.f) : *dq;
    dq0.x += vg.dq[0];
    dq0.y += vg.dq[1];
    dq0.z += vg.dq[2];
    dq0.w += vg.dq[3];
    *dq = dq0;
    d_opac[g] = prior(&d_opac[g]) + vg.d_o;
    if (d_means2d) {
        d_means2d[2 * g] = prior(&d_means2d[2 * g]) + vg.du;
        d_means2d[2 * g + 1] = prior(&d_means2d[2 * g + 1]) + vg.dv;
    }
    if (stats.grad_accum) {  // this view's screen-mean gradient norm, count and radius
        stats.grad_accum[g] += sqrtf(fmaf(vg.du, vg.du, vg.dv * vg.dv));
        stats.count[g] += 1;
        stats.max_radius[g] = max(stats.max_radius[g], radii[g]);
    }
}

// Chain rule, per visible Gaussian, from the summed pixel terms of the
// backward blend to the activated parameters. Outputs accumulate (+=), or with
// OVERWRITE are written for every Gaussian; the SH coefficients and their
// gradient rows go through LDS.
template <bool OVERWRITE>
__global__ __launch_bounds__(64) void k_preprocess_bwd(
    DevCam cam, int K, int sh_rows, float lowpass, float near_plane, int n,
    const float* __restrict__ means, const float* __restrict__ scales, const float4* __restrict__ quats,
    const float* __restrict__ sh, const float4* __restrict__ conic_op, const int* __restrict__ radii,
    const uint8_t* __restrict__ clamped, const float* __restrict__ grad2d,
    float* __restrict__ d_means, float* __restrict__ d_scales, float* __restrict__ d_quats,
    float* __restrict__ d_opac, float* __restrict__ d_sh, float* __restrict__ d_means2d, DensifyStats stats,
    int min_visible) {
    extern __shared__ float s_sh[];
    const int stride = (3 * K) | 1;
    const int base = blockIdx.x * 64;
    const int gi = base + threadIdx.x;
    const bool vis = gi < n && radii[gi] > 0;
    const int nvis = __popcll(__ballot(vis));
    // adding: nothing to do for a block none of whose Gaussians was drawn, and blocks with
    // fewer than min_visible drawn are left to k_preprocess_bwd_add_regs
    if (!OVERWRITE && (nvis == 0 || nvis < min_visible)) return;
    const bool dense = nvis > SH_DENSE;
    float* shg = s_sh + threadIdx.x * stride;
    if (dense) stage_in(sh, s_sh, base, n, 3 * sh_rows, 3 * K, stride);
    else if (vis) copy_own_row(sh, shg, (size_t)gi, 3 * sh_rows, 3 * K);
    __syncthreads();
    ShInPlace acc{shg};
    if (gi < n)
        chain_rule<OVERWRITE>(cam, K, lowpass, near_plane, gi, means, scales, quats, acc, conic_op, radii, clamped,
                              grad2d, d_means, d_scales, d_quats, d_opac, d_means2d, stats);
    __syncthreads();
    if (OVERWRITE) {
        // every row of the block: the gradient rows (zero for culled Gaussians), then zeros
        // for the stored rows beyond the active degree
        stage_out(s_sh, d_sh, base, n, 3 * sh_rows, 3 * K, stride);
        if (gi < n)
            for (int e = 3 * K; e < 3 * sh_rows; ++e) d_sh[(size_t)gi * 3 * sh_rows + e] = 0.f;
    } else if (dense) {
        stage_out_add(s_sh, d_sh, base, n, 3 * sh_rows, 3 * K, stride);
    } else if (vis) {
        add_own_row(shg, d_sh, (size_t)gi, 3 * sh_rows, 3 * K);
    }
}

// The chain rule for rows of 16 SH coefficients (degree 3, 16-byte aligned),
// writing the gradients (as k_preprocess_bwd<true>): each lane moves its own
// row through registers, so the kernel needs no LDS and keeps more waves
// resident than the LDS-staged one.
__global__ __launch_bounds__(64) void k_preprocess_bwd_write_regs(
    DevCam cam, float lowpass, float near_plane, int n,
    const float* __restrict__ means, const float* __restrict__ scales, const float4* __restrict__ quats,
    const float4* __restrict__ sh, const float4* __restrict__ conic_op, const int* __restrict__ radii,
    const uint8_t* __restrict__ clamped, const float* __restrict__ grad2d,
    float* __restrict__ d_means, float* __restrict__ d_scales, float* __restrict__ d_quats,
    float* __restrict__ d_opac, float4* __restrict__ d_sh, float* __restrict__ d_means2d, DensifyStats stats) {
    const int gi = blockIdx.x * 64 + threadIdx.x;
    if (gi >= n) return;
    ShRegs16 acc;
    if (radii[gi] > 0) {  // a culled Gaussian's row is zeroed by chain_rule
#pragma unroll
        for (int q = 0; q < 12; ++q) {
            const float4 v = sh[(size_t)gi * 12 + q];
            acc.c[4 * q] = v.x;
            acc.c[4 * q + 1] = v.y;
            acc.c[4 * q + 2] = v.z;
            acc.c[4 * q + 3] = v.w;
        }
    }
    chain_rule<true>(cam, 16, lowpass, near_plane, gi, means, scales, quats, acc, conic_op, radii, clamped, grad2d,
                     d_means, d_scales, d_quats, d_opac, d_means2d, stats);
#pragma unroll
    for (int q = 0; q < 12; ++q)
        d_sh[(size_t)gi * 12 + q] = make_float4(acc.c[4 * q], acc.c[4 * q + 1], acc.c[4 * q + 2], acc.c[4 * q + 3]);
}

// Adding degree-3 gradients for the blocks with at most max_visible of their
// 64 Gaussians drawn (the others return; k_preprocess_bwd takes them): each
// drawn lane moves its own rows (coefficients, then the gradient row it adds
// to) through registers, so a sparse block needs no LDS.
__global__ __launch_bounds__(64) void k_preprocess_bwd_add_regs(
    DevCam cam, float lowpass, float near_plane, int n, int max_visible,
    const float* __restrict__ means, const float* __restrict__ scales, const float4* __restrict__ quats,
    const float4* __restrict__ sh, const float4* __restrict__ conic_op, const int* __restrict__ radii,
    const uint8_t* __restrict__ clamped, const float* __restrict__ grad2d,
    float* __restrict__ d_means, float* __restrict__ d_scales, float* __restrict__ d_quats,
    float* __restrict__ d_opac, float4* __restrict__ d_sh, float* __restrict__ d_means2d, DensifyStats stats) {
    const int gi = blockIdx.x * 64 + threadIdx.x;
    const bool vis = gi < n && radii[gi] > 0;
    const int nvis = __popcll(__ballot(vis));
    if (nvis > max_visible || !vis) return;
    ShRegs16 acc;
#pragma unroll
    for (int q = 0; q < 12; ++q) {
        const float4 v = sh[(size_t)gi * 12 + q];
        acc.c[4 * q] = v.x;
        acc.c[4 * q + 1] = v.y;
        acc.c[4 * q + 2] = v.z;
        acc.c[4 * q + 3] = v.w;
    }
    chain_rule<false>(cam, 16, lowpass, near_plane, gi, means, scales, quats, acc, conic_op, radii, clamped, grad2d,
                      d_means, d_scales, d_quats, d_opac, d_means2d, stats);
#pragma unroll
    for (int q = 0; q < 12; ++q) {
        float4 v = d_sh[(size_t)gi * 12 + q];
        v.x += acc.c[4 * q];
        v.y += acc.c[4 * q + 1];
        v.z += acc.c[4 * q + 2];
        v.w += acc.c[4 * q + 3];
        d_sh[(size_t)gi * 12 + q] = v;
    }
}

// ---------------------------------------------------------------- several views per launch

// Projection of every Gaussian into V cameras of one image size. The
// parameters and SH rows are read once per Gaussian; view v's outputs go to
// entry v n + g of the per-view arrays, and bit v of vis_mask[g] (if
// non-null) is set when the Gaussian is drawn in view v. Each view's outputs
// are those of the single-view kernel, operation for operation.
__global__ __launch_bounds__(64) void k_preprocess_views(
    CamSet cams, int V, int K, int sh_rows, float lowpass, float near_plane, int n,
    const float* __restrict__ means, const float* __restrict__ scales, const float4* __restrict__ quats,
    const float* __restrict__ opac, const float* __restrict__ sh,
    float2* __restrict__ means2d, float* __restrict__ depths, float4* __restrict__ conic_op,
    float* __restrict__ rgb_out, int* __restrict__ radii, uint32_t* __restrict__ tiles,
    uint8_t* __restrict__ clamped, uint32_t* __restrict__ vis_mask) {
    extern __shared__ float s_sh[];
    const int stride = (3 * K) | 1;
    const int base = blockIdx.x * 64;
    const int gi = base + threadIdx.x;
    const bool live = gi < n;
    const size_t g = live ? (size_t)gi : (size_t)base;
    const float mx = means[3 * g], my = means[3 * g + 1], mz = means[3 * g + 2];
    const float s0 = scales[3 * g], s1 = scales[3 * g + 1], s2 = scales[3 * g + 2];
    const float4 q = quats[g];
    const float o = opac[g];
    const bool fin = live && finitef(mx) && finitef(my) && finitef(mz) && finitef(s0) && finitef(s1) &&
                     finitef(s2) && finitef(q.x) && finitef(q.y) && finitef(q.z) && finitef(q.w) && finitef(o);
    // the block's SH rows, once, through LDS with coalesced reads
    stage_in(sh, s_sh, base, n, 3 * sh_rows, 3 * K, stride);
    __syncthreads();
    const float* shg = s_sh + threadIdx.x * stride;
    uint32_t mask = 0u;
    for (int v = 0; v < V; ++v) {
        const DevCam& cam = cams.c[v];
        const size_t e = (size_t)v * n + g;
        Proj pr;
        bool ok = fin && project(cam, lowpass, near_plane, mx, my, mz, s0, s1, s2, q, pr);
        float raw[3] = {0.5f, 0.5f, 0.5f};
        if (ok) {
            const float dx = mx - cam.campos[0], dy = my - cam.campos[1], dz = mz - cam.campos[2];
            const float dist = sqrtf(fmaf(dx, dx, fmaf(dy, dy, dz * dz)));
            const float id = 1.0f / dist;
            float Y[16];
            sh_eval(K, dx * id, dy * id, dz * id, Y);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                if (k >= K) break;
                raw[0] = fmaf(shg[3 * k], Y[k], raw[0]);
                raw[1] = fmaf(shg[3 * k + 1], Y[k], raw[1]);
                raw[2] = fmaf(shg[3 * k + 2], Y[k], raw[2]);
            }
            ok = dist > 0.f && finitef(raw[0]) && finitef(raw[1]) && finitef(raw[2]);
        }
        if (!live) continue;
        if (!ok) {
            write_culled(e, means2d, depths, conic_op, rgb_out, radii, tiles, clamped);
            continue;
        }
        means2d[e] = make_float2(pr.u, pr.v);
        depths[e] = pr.depth;
        conic_op[e] = make_float4(pr.a, pr.beta, pr.gamma, o);
        radii[e] = pr.r;
        tiles[e] = (uint32_t)((pr.X1 - pr.X0 + 1) * (pr.Y1 - pr.Y0 + 1));
        uint8_t cl = 0;
        for (int c = 0; c < 3; ++c) {
            const bool neg = raw[c] < 0.f;
            cl |= (uint8_t)(neg ? (1u << c) : 0u);
            rgb_out[3 * e + c] = neg ? 0.f : raw[c];
        }
        clamped[e] = cl;
        mask |= 1u << v;
    }
    if (live && vis_mask) vis_mask[g] = mask;
}

// An SH row in LDS read for its coefficients, with the gradient rows of
// every view summed in registers.
struct ShAccum {
    const float* row;
    float acc[48];
    __device__ float coef(int k, int c) const { return row[3 * k + c]; }
    __device__ void grad(int k, float d0, float d1, float d2) {
        acc[3 * k] += d0;
        acc[3 * k + 1] += d1;
        acc[3 * k + 2] += d2;
    }
};

// Chain rule of V views per Gaussian: the per-view inputs (conic, radius,
// clamp bits and pixel sums of view v at entry v n + g) are read view by view;
// the parameter gradients are summed over the views in registers and written
// once (added, or with OVERWRITE written for every Gaussian). dL/d(u, v) of
// view v goes to d_means2d[v n + g] when asked for; the densification
// statistics take every drawn view in turn.
template <bool OVERWRITE>
__global__ __launch_bounds__(64) void k_preprocess_bwd_views(
    CamSet cams, int V, int K, int sh_rows, float lowpass, float near_plane, int n,
    const float* __restrict__ means, const float* __restrict__ scales, const float4* __restrict__ quats,
    const float* __restrict__ sh, const float4* __restrict__ conic_op, const int* __restrict__ radii,
    const uint8_t* __restrict__ clamped, const float* __restrict__ grad2d,
    float* __restrict__ d_means, float* __restrict__ d_scales, float* __restrict__ d_quats,
    float* __restrict__ d_opac, float* __restrict__ d_sh, float* __restrict__ d_means2d, DensifyStats stats) {
    extern __shared__ float s_sh[];
    const int stride = (3 * K) | 1;
    const int base = blockIdx.x * 64;
    const int gi = base + threadIdx.x;
    const bool live = gi < n;
    const size_t g = live ? (size_t)gi : (size_t)base;
    uint32_t mask = 0u;  // the views that drew this Gaussian
    if (live)
        for (int v = 0; v < V; ++v) mask |= radii[(size_t)v * n + g] > 0 ? 1u << v : 0u;
    const int nvis = __popcll(__ballot(mask != 0u));
    if (!OVERWRITE && nvis == 0) return;  // nothing of this block was drawn: no gradient
    const bool dense = nvis > SH_DENSE;
    float* shg = s_sh + threadIdx.x * stride;
    if (dense) stage_in(sh, s_sh, base, n, 3 * sh_rows, 3 * K, stride);
    else if (mask) copy_own_row(sh, shg, g, 3 * sh_rows, 3 * K);
    __syncthreads();
    const float mx = means[3 * g], my = means[3 * g + 1], mz = means[3 * g + 2];
    const float s[3] = {scales[3 * g], scales[3 * g + 1], scales[3 * g + 2]};
    const float4 q = quats[g];
    ShAccum sha;
    sha.row = shg;
#pragma unroll
    for (int k = 0; k < 48; ++k) sha.acc[k] = 0.f;
    float dmu[3] = {0.f, 0.f, 0.f}, ds[3] = {0.f, 0.f, 0.f}, dq[4] = {0.f, 0.f, 0.f, 0.f}, d_o = 0.f;
    float nsum = 0.f;
    int cnt = 0, rmax = 0;
    for (int v = 0; v < V; ++v) {
        const size_t e = (size_t)v * n + g;
        bool contrib = false;
        ViewGrad vg;
        if ((mask >> v) & 1u) {
            contrib = view_grad(cams.c[v], K, lowpass, near_plane, mx, my, mz, s, q, conic_op[e],
                                reinterpret_cast<const float4*>(grad2d + e * GRAD2D_STRIDE), clamped[e], sha, vg);
            if (contrib) {
                for (int j = 0; j < 3; ++j) dmu[j] += vg.dmu[j];
                for (int j = 0; j < 3; ++j) ds[j] += vg.ds[j];
                for (int j = 0; j < 4; ++j) dq[j] += vg.dq[j];
                d_o += vg.d_o;
                nsum += sqrtf(fmaf(vg.du, vg.du, vg.dv * vg.dv));
                cnt += 1;
                rmax = max(rmax, radii[e]);
            }
        }
        if (d_means2d && live) {
            if (OVERWRITE) {
                d_means2d[2 * e] = contrib ? vg.du : 0.f;
                d_means2d[2 * e + 1] = contrib ? vg.dv : 0.f;
            } else if (contrib) {
                d_means2d[2 * e] += vg.du;
                d_means2d[2 * e + 1] += vg.dv;
            }
        }
    }
    if (live && (OVERWRITE || mask)) {
        auto prior = [&](const float* p) { return OVERWRITE ? 0.f : *p; };
        for (int j = 0; j < 3; ++j) d_means[3 * g + j] = prior(&d_means[3 * g + j]) + dmu[j];
        for (int j = 0; j < 3; ++j) d_scales[3 * g + j] = prior(&d_scales[3 * g + j]) + ds[j];
        float4* dqp = reinterpret_cast<float4*>(d_quats) + g;
        float4 dq0 = OVERWRITE ? make_float4(0.f, 0.f, 0.f, 0.f) : *dqp;
        *dqp = make_float4(dq0.x + dq[0], dq0.y + dq[1], dq0.z + dq[2], dq0.w + dq[3]);
        d_opac[g] = prior(&d_opac[g]) + d_o;
    }
    if (stats.grad_accum && live && cnt > 0) {
        stats.grad_accum[g] += nsum;
        stats.count[g] += cnt;
        stats.max_radius[g] = max(stats.max_radius[g], rmax);
    }
    // the summed SH gradient rows replace the coefficients (each lane its own row), then leave through LDS
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (k < K) {
            shg[3 * k] = sha.acc[3 * k];
            shg[3 * k + 1] = sha.acc[3 * k + 1];
            shg[3 * k + 2] = sha.acc[3 * k + 2];
        }
    }
    __syncthreads();
    if (OVERWRITE) {
        stage_out(s_sh, d_sh, base, n, 3 * sh_rows, 3 * K, stride);
        if (live)
            for (int e = 3 * K; e < 3 * sh_rows; ++e) d_sh[g * 3 * sh_rows + e] = 0.f;
    } else if (dense) {
        stage_out_add(s_sh, d_sh, base, n, 3 * sh_rows, 3 * K, stride);
    } else if (mask) {
        add_own_row(shg, d_sh, g, 3 * sh_rows, 3 * K);
    }
}


// The chain rule of one view for 2D Gaussian surfels, one lane per surfel,
// from its summed pixel terms (16 floats: dL/drgb, sum h, the sums of dL/dk
// and of (pixel - c) times it for the expanded intersection
// k = N01 + x N12 - y N02, the filter branch's sum of h (pixel - c), zero) to
// the activated parameters. The cross
// products N01 = M0 x M1, N12 = M1 x M2, N02 = M0 x M2 give dL/dM;
// M = K [a | b | X] (a = s_u R t_u, b = s_v R t_v, X = R mu + t)
// gives dL/da, dL/db and dL/dX as K^T times the columns of dL/dM; the
// projected centre c adds through X; t_u and t_v are the first two columns of
// the quaternion's rotation. Outputs accumulate (+=), or with OVERWRITE are
// written (zeros for a culled surfel and for SH rows at or past the active
// degree). The SH row moves through registers.
// VEC: SH rows of 16 coefficients (12 float4, 16-byte aligned) move as float4,
// so that each row is read and written whole; otherwise coefficient by
// coefficient.
template <bool OVERWRITE, bool VEC>
__global__ __launch_bounds__(64) void k_surfel_preprocess_bwd(
    DevCam cam, int K, int sh_rows, int n, const float* __restrict__ means, const float* __restrict__ scales,
    const float4* __restrict__ quats, const float* __restrict__ sh, const float4* __restrict__ tf,
    const int* __restrict__ radii, const uint8_t* __restrict__ clamped, const float4* __restrict__ grad,
    float* __restrict__ d_means, float* __restrict__ d_scales, float* __restrict__ d_quats,
    float* __restrict__ d_opac, float* __restrict__ d_sh) {
    const int gi = blockIdx.x * 64 + threadIdx.x;
    if (gi >= n) return;
    const size_t g = (size_t)gi;
    const float* shg = sh + g * 3 * sh_rows;
    float* dsh = d_sh + g * 3 * sh_rows;
    const bool drawn = radii[g] > 0;
    const float mx = means[3 * g], my = means[3 * g + 1], mz = means[3 * g + 2];
    const float X[3] = {fmaf(cam.R[0], mx, fmaf(cam.R[1], my, fmaf(cam.R[2], mz, cam.t[0]))),
                        fmaf(cam.R[3], mx, fmaf(cam.R[4], my, fmaf(cam.R[5], mz, cam.t[1]))),
                        fmaf(cam.R[6], mx, fmaf(cam.R[7], my, fmaf(cam.R[8], mz, cam.t[2])))};
    const float4 q = quats[g];
    const float qq = q.x * q.x + q.y * q.y + q.z * q.z + q.w * q.w;
    const float ddx = mx - cam.campos[0], ddy = my - cam.campos[1], ddz = mz - cam.campos[2];
    const float dist = sqrtf(fmaf(ddx, ddx, fmaf(ddy, ddy, ddz * ddz)));
    if (!drawn || !(X[2] > 0.f) || !(qq > 0.f) || !(dist > 0.f)) {
        if (OVERWRITE) {
            d_means[3 * g] = d_means[3 * g + 1] = d_means[3 * g + 2] = 0.f;
            d_scales[2 * g] = d_scales[2 * g + 1] = 0.f;
            reinterpret_cast<float4*>(d_quats)[g] = make_float4(0.f, 0.f, 0.f, 0.f);
            d_opac[g] = 0.f;
            if (VEC) {
#pragma unroll
                for (int q = 0; q < 12; ++q) reinterpret_cast<float4*>(dsh)[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
                for (int e = 0; e < 3 * sh_rows; ++e) dsh[e] = 0.f;
            }
        }
        return;
    }
    // the SH row first (VEC): its loads go out with the rest of the record's
    float cf[VEC ? 48 : 1];
    if (VEC) {
#pragma unroll
        for (int q = 0; q < 12; ++q) {
            const float4 v = reinterpret_cast<const float4*>(shg)[q];
            cf[4 * q] = v.x;
            cf[4 * q + 1] = v.y;
            cf[4 * q + 2] = v.z;
            cf[4 * q + 3] = v.w;
        }
    }
    const float su = scales[2 * g], sv = scales[2 * g + 1];
    const float qn = sqrtf(qq), iq = 1.0f / qn;
    const float w = q.x * iq, x = q.y * iq, y = q.z * iq, z = q.w * iq;
    const float tu[3] = {1.f - 2.f * (y * y + z * z), 2.f * (x * y + w * z), 2.f * (x * z - w * y)};
    const float tv[3] = {2.f * (x * y - w * z), 1.f - 2.f * (x * x + z * z), 2.f * (y * z + w * x)};
    // record: g0 = (drgb, sum h), g1 = (sum dL/dk, sum dx dL/dk .x), g2 = (sum dx dL/dk .yz,
    // sum dy dL/dk .xy), g3 = (sum dy dL/dk .z, sum_f h dx, sum_f h dy, 0), with (dx, dy) = pixel - c
    // and k = N01 + x N12 - y N02, N01 = M0 x M1, N12 = M1 x M2, N02 = M0 x M2 (rows Mi of M):
    // dL/dN01 = sum dL/dk, dL/dN12 = sum x dL/dk, dL/dN02 = -sum y dL/dk
    const float4 g0 = grad[4 * g], g1 = grad[4 * g + 1], g2 = grad[4 * g + 2], g3 = grad[4 * g + 3];
    const float4 t0 = tf[3 * g], t1 = tf[3 * g + 1], t2 = tf[3 * g + 2];
    const float ccx = t1.w, ccy = t2.w;
    const float dN01[3] = {g1.x, g1.y, g1.z};
    const float dN12[3] = {fmaf(ccx, g1.x, g1.w), fmaf(ccx, g1.y, g2.x), fmaf(ccx, g1.z, g2.y)};
    const float dN02[3] = {-fmaf(ccy, g1.x, g2.z), -fmaf(ccy, g1.y, g2.w), -fmaf(ccy, g1.z, g3.x)};
    const float M0[3] = {t0.x, t0.y, t0.z}, M1[3] = {t1.x, t1.y, t1.z}, M2[3] = {t2.x, t2.y, t2.z};
    auto cross = [](const float* p, const float* q, float* o) {
        o[0] = fmaf(p[1], q[2], -p[2] * q[1]);
        o[1] = fmaf(p[2], q[0], -p[0] * q[2]);
        o[2] = fmaf(p[0], q[1], -p[1] * q[0]);
    };
    // dM0 = M1 x dN01 + M2 x dN02, dM1 = dN01 x M0 + M2 x dN12, dM2 = dN12 x M1 + dN02 x M0
    float c1[3], c2[3], dM0[3], dM1[3], dM2[3];
    cross(M1, dN01, c1);
    cross(M2, dN02, c2);
#pragma unroll
    for (int j = 0; j < 3; ++j) dM0[j] = c1[j] + c2[j];
    cross(dN01, M0, c1);
    cross(M2, dN12, c2);
#pragma unroll
    for (int j = 0; j < 3; ++j) dM1[j] = c1[j] + c2[j];
    cross(dN12, M1, c1);
    cross(dN02, M0, c2);
#pragma unroll
    for (int j = 0; j < 3; ++j) dM2[j] = c1[j] + c2[j];
    const float fx = cam.fx, fy = cam.fy, cx = cam.cx, cy = cam.cy;
    // K^T = [[fx, 0, 0], [0, fy, 0], [cx, cy, 1]] times the columns of dL/dM
    const float da[3] = {fx * dM0[0], fy * dM1[0], fmaf(cx, dM0[0], fmaf(cy, dM1[0], dM2[0]))};
    const float db[3] = {fx * dM0[1], fy * dM1[1], fmaf(cx, dM0[1], fmaf(cy, dM1[1], dM2[1]))};
    float dX[3] = {fx * dM0[2], fy * dM1[2], fmaf(cx, dM0[2], fmaf(cy, dM1[2], dM2[2]))};
    // the centre c = (fx X / Z + cx, fy Y / Z + cy): dL/dc = 2 sum_f h (pixel - c)
    const float dcx = 2.f * g3.y, dcy = 2.f * g3.z;
    const float iz = 1.0f / X[2];
    dX[0] = fmaf(fx * iz, dcx, dX[0]);
    dX[1] = fmaf(fy * iz, dcy, dX[1]);
    dX[2] -= (fx * X[0] * dcx + fy * X[1] * dcy) * iz * iz;
    float dmu[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) dmu[j] = fmaf(cam.R[j], dX[0], fmaf(cam.R[3 + j], dX[1], cam.R[6 + j] * dX[2]));
    // a = s_u R t_u, b = s_v R t_v
    float dsu = 0.f, dsv = 0.f, dtu[3], dtv[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const float rtu = fmaf(cam.R[3 * i], tu[0], fmaf(cam.R[3 * i + 1], tu[1], cam.R[3 * i + 2] * tu[2]));
        const float rtv = fmaf(cam.R[3 * i], tv[0], fmaf(cam.R[3 * i + 1], tv[1], cam.R[3 * i + 2] * tv[2]));
        dsu = fmaf(rtu, da[i], dsu);
        dsv = fmaf(rtv, db[i], dsv);
        dtu[i] = su * fmaf(cam.R[i], da[0], fmaf(cam.R[3 + i], da[1], cam.R[6 + i] * da[2]));
        dtv[i] = sv * fmaf(cam.R[i], db[0], fmaf(cam.R[3 + i], db[1], cam.R[6 + i] * db[2]));
    }
    // dL/dRq (row-major): columns 0 and 1 are dL/dt_u and dL/dt_v, column 2 is zero
    const float dR[9] = {dtu[0], dtv[0], 0.f, dtu[1], dtv[1], 0.f, dtu[2], dtv[2], 0.f};
    const float gw = 2.f * (-z * dR[1] + y * dR[2] + z * dR[3] - x * dR[5] - y * dR[6] + x * dR[7]);
    const float gx = 2.f * (y * dR[1] + z * dR[2] + y * dR[3] - 2.f * x * dR[4] - w * dR[5] + z * dR[6] +
                            w * dR[7] - 2.f * x * dR[8]);
    const float gy = 2.f * (-2.f * y * dR[0] + x * dR[1] + w * dR[2] + x * dR[3] + z * dR[5] - w * dR[6] +
                            z * dR[7] - 2.f * y * dR[8]);
    const float gz = 2.f * (-2.f * z * dR[0] - w * dR[1] + x * dR[2] + w * dR[3] - 2.f * z * dR[4] + y * dR[5] +
                            x * dR[6] + y * dR[7]);
    const float qdot = w * gw + x * gx + y * gy + z * gz;
    const float4 dq = make_float4((gw - qdot * w) * iq, (gx - qdot * x) * iq, (gy - qdot * y) * iq,
                                  (gz - qdot * z) * iq);
    // colour: rgb = max(0, sum_k sh_k Y_k(dir) + 0.5), dir = (mu - campos) / |mu - campos|
    const uint8_t cl = clamped[g];
    float dcol[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) dcol[c] = (cl >> c) & 1 ? 0.f : (c == 0 ? g0.x : c == 1 ? g0.y : g0.z);
    const float id = 1.0f / dist;
    const float dxn = ddx * id, dyn = ddy * id, dzn = ddz * id;
    float Y[16], wk[16];
    sh_eval(K, dxn, dyn, dzn, Y);
    if (VEC) {
        float out[48];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const bool act = k < K;
            wk[k] = act ? fmaf(cf[3 * k], dcol[0], fmaf(cf[3 * k + 1], dcol[1], cf[3 * k + 2] * dcol[2])) : 0.f;
#pragma unroll
            for (int c = 0; c < 3; ++c) out[3 * k + c] = act ? Y[k] * dcol[c] : 0.f;
        }
        float4* d4 = reinterpret_cast<float4*>(dsh);
        if (!OVERWRITE) {
#pragma unroll
            for (int q = 0; q < 12; ++q) {
                const float4 p = d4[q];
                out[4 * q] += p.x;
                out[4 * q + 1] += p.y;
                out[4 * q + 2] += p.z;
                out[4 * q + 3] += p.w;
            }
        }
#pragma unroll
        for (int q = 0; q < 12; ++q) d4[q] = make_float4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (k < K) {
                const float c0 = shg[3 * k], c1 = shg[3 * k + 1], c2 = shg[3 * k + 2];
                wk[k] = fmaf(c0, dcol[0], fmaf(c1, dcol[1], c2 * dcol[2]));
                const float p0 = OVERWRITE ? 0.f : dsh[3 * k], p1 = OVERWRITE ? 0.f : dsh[3 * k + 1],
                            p2 = OVERWRITE ? 0.f : dsh[3 * k + 2];
                dsh[3 * k] = fmaf(Y[k], dcol[0], p0);
                dsh[3 * k + 1] = fmaf(Y[k], dcol[1], p1);
                dsh[3 * k + 2] = fmaf(Y[k], dcol[2], p2);
            }
        }
        if (OVERWRITE)
            for (int e = 3 * K; e < 3 * sh_rows; ++e) dsh[e] = 0.f;
    }
    float3 gdir = make_float3(0.f, 0.f, 0.f);
    sh_grad_accum(K, dxn, dyn, dzn, wk, gdir);
    const float dd = dxn * gdir.x + dyn * gdir.y + dzn * gdir.z;
    dmu[0] += (gdir.x - dxn * dd) * id;
    dmu[1] += (gdir.y - dyn * dd) * id;
    dmu[2] += (gdir.z - dzn * dd) * id;
    const float o = t0.w;
    auto prior = [&](const float* p) { return OVERWRITE ? 0.f : *p; };
#pragma unroll
    for (int j = 0; j < 3; ++j) d_means[3 * g + j] = prior(&d_means[3 * g + j]) + dmu[j];
    d_scales[2 * g] = prior(&d_scales[2 * g]) + dsu;
    d_scales[2 * g + 1] = prior(&d_scales[2 * g + 1]) + dsv;
    float4* dqp = reinterpret_cast<float4*>(d_quats) + g;
    float4 dq0 = OVERWRITE ? make_float4(0.f, 0.f, 0.f, 0.f) : *dqp;
    dq0.x += dq.x;
    dq0.y += dq.y;
    dq0.z += dq.z;
    dq0.w += dq.w;
    *dqp = dq0;
    d_opac[g] = prior(&d_opac[g]) + (o != 0.f ? g0.w / o : 0.f);
}

}  // namespace

hipError_t launch_preprocess(const DevCam& cam, int K, int sh_rows, float lowpass, float near_plane, int n,
                             const float* means, const float* scales, const float* quats, const float* opac,
                             const float* sh, float* means2d, float* depths, float* conic_op, float* rgb,
                             int* radii, uint32_t* tiles, uint8_t* clamped, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    int blocks = (n + 63) / 64;
    size_t lds = sizeof(float) * 64 * CHUNK_STRIDE;
    k_preprocess<false><<<blocks, 64, lds, stream>>>(cam, K, sh_rows, lowpass, near_plane, n, means, scales,
                                             reinterpret_cast<const float4*>(quats), opac, sh,
                                             reinterpret_cast<float2*>(means2d), depths,
                                             reinterpret_cast<float4*>(conic_op), rgb, radii, tiles, clamped);
    return hipGetLastError();
}

hipError_t launch_surfel_preprocess(const DevCam& cam, int K, int sh_rows, float near_plane, int n,
                                    const float* means, const float* scales, const float* quats, const float* opac,
                                    const float* sh, float* means2d, float* depths, float* tf, float* rgb,
                                    int* radii, uint32_t* tiles, uint8_t* clamped, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int blocks = (n + 63) / 64;
    const size_t lds = sizeof(float) * 64 * CHUNK_STRIDE;
    k_preprocess<true><<<blocks, 64, lds, stream>>>(cam, K, sh_rows, 0.f, near_plane, n, means, scales,
                                                    reinterpret_cast<const float4*>(quats), opac, sh,
                                                    reinterpret_cast<float2*>(means2d), depths,
                                                    reinterpret_cast<float4*>(tf), rgb, radii, tiles, clamped);
    return hipGetLastError();
}

hipError_t launch_surfel_preprocess_bwd(const DevCam& cam, int K, int sh_rows, int n, const float* means,
                                        const float* scales, const float* quats, const float* sh, const float* tf,
                                        const int* radii, const uint8_t* clamped, const float* grad, float* d_means,
                                        float* d_scales, float* d_quats, float* d_opac, float* d_sh, bool overwrite,
                                        hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int blocks = (n + 63) / 64;
    auto* q4 = reinterpret_cast<const float4*>(quats);
    auto* t4 = reinterpret_cast<const float4*>(tf);
    auto* g4 = reinterpret_cast<const float4*>(grad);
    const bool vec = sh_rows == 16 && ((uintptr_t)sh & 15u) == 0 && ((uintptr_t)d_sh & 15u) == 0;
    auto go = [&](auto ow, auto vc) {
        k_surfel_preprocess_bwd<decltype(ow)::value, decltype(vc)::value><<<blocks, 64, 0, stream>>>(
            cam, K, sh_rows, n, means, scales, q4, sh, t4, radii, clamped, g4, d_means, d_scales, d_quats, d_opac,
            d_sh);
    };
    if (overwrite) {
        if (vec) go(std::true_type{}, std::true_type{});
        else go(std::true_type{}, std::false_type{});
    } else {
        if (vec) go(std::false_type{}, std::true_type{});
        else go(std::false_type{}, std::false_type{});
    }
    return hipGetLastError();
}

hipError_t launch_preprocess_bwd(const DevCam& cam, int K, int sh_rows, float lowpass, float near_plane, int n,
                                 const float* means, const float* scales, const float* quats, const float* sh,
                                 const float* conic_op, const int* radii, const uint8_t* clamped,
                                 const float* grad2d, float* d_means, float* d_scales, float* d_quats,
                                 float* d_opac, float* d_sh, float* d_means2d, bool overwrite,
                                 const DensifyStats& stats, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    int blocks = (n + 63) / 64;
    // Writing the gradients of degree-3 rows: each lane's row in registers, no LDS. Measured
    // against the LDS-staged kernel: 1M Gaussians at 1080p (99% drawn) 0.130 -> 0.112 ms, one
    // view of 6M (22% drawn) 0.671 -> 0.506 ms. Adding into the gradients it would read them
    // back with each lane's own 192-byte row: 0.153 -> 0.203 ms at 99% drawn (0.787 -> 0.505 at
    // 22%), so that mode keeps the coalesced LDS staging.
    if (overwrite && K == 16 && sh_rows == 16 && ((uintptr_t)sh & 15u) == 0 && ((uintptr_t)d_sh & 15u) == 0) {
        k_preprocess_bwd_write_regs<<<blocks, 64, 0, stream>>>(
            cam, lowpass, near_plane, n, means, scales, reinterpret_cast<const float4*>(quats),
            reinterpret_cast<const float4*>(sh), reinterpret_cast<const float4*>(conic_op), radii, clamped, grad2d,
            d_means, d_scales, d_quats, d_opac, reinterpret_cast<float4*>(d_sh), d_means2d, stats);
        return hipGetLastError();
    }
    // Adding degree-3 gradients: blocks with at most BWD_REGS_MAX_VISIBLE of their Gaussians
    // drawn go through registers, the denser ones through the LDS staging (one view of 6M
    // Gaussians, 22% drawn: 0.787 -> 0.52 ms; 1M at 1080p, 99% drawn: unchanged).
    int min_visible = 1;
    if (!overwrite && K == 16 && sh_rows == 16 && ((uintptr_t)sh & 15u) == 0 && ((uintptr_t)d_sh & 15u) == 0) {
        k_preprocess_bwd_add_regs<<<blocks, 64, 0, stream>>>(
            cam, lowpass, near_plane, n, BWD_REGS_MAX_VISIBLE, means, scales, reinterpret_cast<const float4*>(quats),
            reinterpret_cast<const float4*>(sh), reinterpret_cast<const float4*>(conic_op), radii, clamped, grad2d,
            d_means, d_scales, d_quats, d_opac, reinterpret_cast<float4*>(d_sh), d_means2d, stats);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        min_visible = BWD_REGS_MAX_VISIBLE + 1;
    }
    size_t lds = sizeof(float) * 64 * ((3 * K) | 1);
    auto kernel = overwrite ? k_preprocess_bwd<true> : k_preprocess_bwd<false>;
    kernel<<<blocks, 64, lds, stream>>>(cam, K, sh_rows, lowpass, near_plane, n, means, scales,
                                        reinterpret_cast<const float4*>(quats), sh,
                                        reinterpret_cast<const float4*>(conic_op), radii, clamped, grad2d, d_means,
                                        d_scales, d_quats, d_opac, d_sh, d_means2d, stats, min_visible);
    return hipGetLastError();
}

hipError_t launch_preprocess_views(const CamSet& cams, int V, int K, int sh_rows, float lowpass, float near_plane,
                                   int n, const float* means, const float* scales, const float* quats,
                                   const float* opac, const float* sh, float* means2d, float* depths,
                                   float* conic_op, float* rgb, int* radii, uint32_t* tiles, uint8_t* clamped,
                                   uint32_t* vis_mask, hipStream_t stream) {
    if (n == 0 || V == 0) return hipSuccess;
    const int blocks = (n + 63) / 64;
    const size_t lds = sizeof(float) * 64 * ((3 * K) | 1);
    k_preprocess_views<<<blocks, 64, lds, stream>>>(cams, V, K, sh_rows, lowpass, near_plane, n, means, scales,
                                                    reinterpret_cast<const float4*>(quats), opac, sh,
                                                    reinterpret_cast<float2*>(means2d), depths,
                                                    reinterpret_cast<float4*>(conic_op), rgb, radii, tiles, clamped,
                                                    vis_mask);
    return hipGetLastError();
}

hipError_t launch_preprocess_bwd_views(const CamSet& cams, int V, int K, int sh_rows, float lowpass, float near_plane,
                                       int n, const float* means, const float* scales, const float* quats,
                                       const float* sh, const float* conic_op, const int* radii,
                                       const uint8_t* clamped, const float* grad2d, float* d_means, float* d_scales,
                                       float* d_quats, float* d_opac, float* d_sh, float* d_means2d, bool overwrite,
                                       const DensifyStats& stats, hipStream_t stream) {
    if (n == 0 || V == 0) return hipSuccess;
    const int blocks = (n + 63) / 64;
    const size_t lds = sizeof(float) * 64 * ((3 * K) | 1);
    auto kernel = overwrite ? k_preprocess_bwd_views<true> : k_preprocess_bwd_views<false>;
    kernel<<<blocks, 64, lds, stream>>>(cams, V, K, sh_rows, lowpass, near_plane, n, means, scales,
                                        reinterpret_cast<const float4*>(quats), sh,
                                        reinterpret_cast<const float4*>(conic_op), radii, clamped, grad2d, d_means,
                                        d_scales, d_quats, d_opac, d_sh, d_means2d, stats);
    return hipGetLastError();
}

}  // namespace gs
