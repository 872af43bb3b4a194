/*
 * gs_oracle.c -- plain, slow fp64 CPU reference of tile-based 3D Gaussian
 * splatting rasterization, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code, header,
 * table or helper with the HIP library and must never be called by it.
 *
 * What it computes. The rasterizer is the one of "3D Gaussian Splatting for
 * Real-Time Radiance Field Rendering", the method the DISTWAR page names in its
 * abstract ("e.g. 3D Gaussian Splatting") and lists among the works it builds
 * on; the Odin page cites it in its reference list and splits a training
 * iteration into preprocessing, rendering and backward computation (Fig. 7
 * caption). The pages print none of its formulas. The steps below are the plain
 * reading of that method; every point the pages leave open is a documented
 * reading of this project, repeated at the step it affects:
 *
 *   O1  camera        x_c = R x_w + t, campos = -R^T t; x right, y down, z
 *                     forward; pixel (px, py) has its centre at (px+1/2, py+1/2)
 *   O2  cull          z <= near, any non-finite input or derived value, a zero
 *                     quaternion, |u|,|v| or 3 sqrt(lambda_max) above 2^24
 *   O3  rotation      unit quaternion (w,x,y,z) -> rotation matrix Rq
 *   O4  covariance    M = Rq diag(s), Sigma = M M^T
 *   O5  EWA           J = d(projection)/d(x_c) at the mean, V = J R,
 *                     Sigma' = V Sigma V^T + lowpass I
 *   O6  conic         det = A C - B^2 (cull if <= 0), conic = Sigma'^-1
 *   O7  radius        r = ceil(3 sqrt(lambda_max(Sigma')))
 *   O8  screen mean   u = fx x/z + cx, v = fy y/z + cy, depth = z
 *   O9  tile rect     X0 = max(0, floor((floor(u) - r)/16)), X1 = min(TX-1,
 *                     floor((floor(u) + r)/16)), same for y; cull if empty
 *   O10 colour        real spherical harmonics of the view direction,
 *                     rgb = max(0, sum_k sh_k Y_k + 1/2)
 *   O11 bin + sort    one (key = tile << 32 | bits(fp32 depth), value = g)
 *                     pair per tile of the rect, sorted by (key, g)
 *   O12 forward       per pixel, front to back: alpha = min(0.99, o G),
 *                     G = exp(-Q/2), Q = d^T Sigma'^-1 d; skip alpha < 1/255;
 *                     stop before the entry that would take T below 1e-4
 *   O13 backward      per pixel, reverse over the blended entries
 *   O14 chain rule    per Gaussian, 2D gradients -> parameter gradients
 *
 * Constants are the fp32 values 0.99f, 1/255.f and 1e-4f, widened exactly.
 * Everything here is double precision, one pixel or one Gaussian at a time,
 * in the order the steps are stated; OpenMP only spreads independent pixels
 * and Gaussians over threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TILE 16
static const double ALPHA_MAX = (double)0.99f;
static const double ALPHA_MIN = (double)(1.0f / 255.0f);
static const double T_MIN = (double)1e-4f;
static const double BIG = 16777216.0; /* 2^24 */

typedef struct {
    int W, H;
    double fx, fy, cx, cy;
    double R[9];
    double t[3];
} ocam;

static ocam cam_from(const double *c)
{
    ocam k;
    k.W = (int)c[0];
    k.H = (int)c[1];
    k.fx = c[2];
    k.fy = c[3];
    k.cx = c[4];
    k.cy = c[5];
    for (int i = 0; i < 9; ++i) k.R[i] = c[6 + i];
    for (int i = 0; i < 3; ++i) k.t[i] = c[15 + i];
    return k;
}

int orc_version(void) { return 1; }

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* O10: real spherical harmonics, degree <= 3, index k = l^2 + l + m.   */
/* Normalisations are the textbook sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!) */
/* factors (times sqrt 2 for m != 0), written out as closed forms.       */
/* ------------------------------------------------------------------ */
static double shc(int which)
{
    const double pi = 3.14159265358979323846;
    switch (which) {
    case 0: return 0.5 * sqrt(1.0 / pi);          /* l=0            */
    case 1: return sqrt(3.0 / (4.0 * pi));         /* l=1            */
    case 2: return 0.5 * sqrt(15.0 / pi);          /* l=2, |m|=1,2 xy */
    case 3: return 0.25 * sqrt(5.0 / pi);          /* l=2, m=0       */
    case 4: return 0.25 * sqrt(15.0 / pi);         /* l=2, m=2       */
    case 5: return 0.25 * sqrt(35.0 / (2.0 * pi)); /* l=3, |m|=3     */
    case 6: return 0.5 * sqrt(105.0 / pi);         /* l=3, m=-2      */
    case 7: return 0.25 * sqrt(21.0 / (2.0 * pi)); /* l=3, |m|=1     */
    case 8: return 0.25 * sqrt(7.0 / pi);          /* l=3, m=0       */
    case 9: return 0.25 * sqrt(105.0 / pi);        /* l=3, m=2       */
    }
    return 0.0;
}

/* Y[k] for k < (deg+1)^2 at unit direction (x, y, z). */
void orc_sh_basis(int deg, double x, double y, double z, double *Y)
{
    Y[0] = shc(0);
    if (deg < 1) return;
    Y[1] = -shc(1) * y;
    Y[2] = shc(1) * z;
    Y[3] = -shc(1) * x;
    if (deg < 2) return;
    Y[4] = shc(2) * x * y;
    Y[5] = -shc(2) * y * z;
    Y[6] = shc(3) * (2.0 * z * z - x * x - y * y);
    Y[7] = -shc(2) * x * z;
    Y[8] = shc(4) * (x * x - y * y);
    if (deg < 3) return;
    Y[9] = -shc(5) * y * (3.0 * x * x - y * y);
    Y[10] = shc(6) * x * y * z;
    Y[11] = -shc(7) * y * (4.0 * z * z - x * x - y * y);
    Y[12] = shc(8) * z * (2.0 * z * z - 3.0 * x * x - 3.0 * y * y);
    Y[13] = -shc(7) * x * (4.0 * z * z - x * x - y * y);
    Y[14] = shc(9) * z * (x * x - y * y);
    Y[15] = -shc(5) * x * (x * x - 3.0 * y * y);
}

/* dY[k][0..2] = gradient of the polynomial Y_k with x, y, z independent. */
void orc_sh_basis_grad(int deg, double x, double y, double z, double *dY)
{
    int K = (deg + 1) * (deg + 1);
    for (int i = 0; i < 3 * K; ++i) dY[i] = 0.0;
#define G3(k, a, b, c) do { dY[3*(k)+0] = (a); dY[3*(k)+1] = (b); dY[3*(k)+2] = (c); } while (0)
    if (deg < 1) return;
    G3(1, 0.0, -shc(1), 0.0);
    G3(2, 0.0, 0.0, shc(1));
    G3(3, -shc(1), 0.0, 0.0);
    if (deg < 2) return;
    G3(4, shc(2) * y, shc(2) * x, 0.0);
    G3(5, 0.0, -shc(2) * z, -shc(2) * y);
    G3(6, -2.0 * shc(3) * x, -2.0 * shc(3) * y, 4.0 * shc(3) * z);
    G3(7, -shc(2) * z, 0.0, -shc(2) * x);
    G3(8, 2.0 * shc(4) * x, -2.0 * shc(4) * y, 0.0);
    if (deg < 3) return;
    G3(9, -shc(5) * 6.0 * x * y, -shc(5) * (3.0 * x * x - 3.0 * y * y), 0.0);
    G3(10, shc(6) * y * z, shc(6) * x * z, shc(6) * x * y);
    G3(11, -shc(7) * (-2.0 * x * y), -shc(7) * (4.0 * z * z - x * x - 3.0 * y * y),
       -shc(7) * 8.0 * y * z);
    G3(12, shc(8) * (-6.0 * x * z), shc(8) * (-6.0 * y * z),
       shc(8) * (6.0 * z * z - 3.0 * x * x - 3.0 * y * y));
    G3(13, -shc(7) * (4.0 * z * z - 3.0 * x * x - y * y), -shc(7) * (-2.0 * x * y),
       -shc(7) * 8.0 * x * z);
    G3(14, shc(9) * 2.0 * x * z, -shc(9) * 2.0 * y * z, shc(9) * (x * x - y * y));
    G3(15, -shc(5) * (3.0 * x * x - 3.0 * y * y), -shc(5) * (-6.0 * x * y), 0.0);
#undef G3
}

/* ------------------------------------------------------------------ */
/* small dense helpers (row-major)                                      */
/* ------------------------------------------------------------------ */
static int isfin(double v) { return isfinite(v) != 0; }

static int64_t floordiv(int64_t a, int64_t b) /* b > 0 */
{
    return a >= 0 ? a / b : -((-a + b - 1) / b);
}

/* O3: rotation matrix of the unit quaternion (w, x, y, z). */
static void quat_to_rot(const double q[4], double Rq[9])
{
    double w = q[0], x = q[1], y = q[2], z = q[3];
    Rq[0] = 1.0 - 2.0 * (y * y + z * z);
    Rq[1] = 2.0 * (x * y - w * z);
    Rq[2] = 2.0 * (x * z + w * y);
    Rq[3] = 2.0 * (x * y + w * z);
    Rq[4] = 1.0 - 2.0 * (x * x + z * z);
    Rq[5] = 2.0 * (y * z - w * x);
    Rq[6] = 2.0 * (x * z - w * y);
    Rq[7] = 2.0 * (y * z + w * x);
    Rq[8] = 1.0 - 2.0 * (x * x + y * y);
}

/* Everything O1-O10 derives for one Gaussian. */
typedef struct {
    int visible;
    double xc[3];       /* camera-frame mean */
    double qn[4];       /* normalised quaternion */
    double qnorm;
    double Rq[9];
    double M[9];        /* Rq diag(s) */
    double Sig[9];      /* 3D covariance */
    double J[6];        /* 2x3 */
    double V[6];        /* J R, 2x3 */
    double A, B, C;     /* Sigma' = [[A, B], [B, C]] */
    double det;
    double con[3];      /* conic (a, b, c) = Sigma'^-1 entries */
    double lam, extent; /* lambda_max and 3 sqrt(lambda_max) */
    int64_t r;
    double u, v;
    int64_t rect[4];    /* X0, X1, Y0, Y1 */
    double dir[3], dist;
    double Y[16];
    double raw[3], rgb[3];
    unsigned char clamp[3];
    double margin;      /* relative distance of the integer decisions to their cuts */
} gauss_fwd;

static double frac_margin(double x)
{
    double d = fabs(x - nearbyint(x));
    double s = fabs(x) > 1.0 ? fabs(x) : 1.0;
    return d / s;
}

static void gauss_forward(const ocam *cam, int deg, int sh_rows, double lowpass, double near_plane,
                          const double *mean, const double *scale, const double *quat,
                          double opac, const double *sh, gauss_fwd *o)
{
    memset(o, 0, sizeof(*o));
    o->margin = INFINITY;
    int K = (deg + 1) * (deg + 1);
    int TX = (cam->W + TILE - 1) / TILE, TY = (cam->H + TILE - 1) / TILE;
    int fin = isfin(opac);
    for (int i = 0; i < 3; ++i) fin &= isfin(mean[i]) & isfin(scale[i]);
    for (int i = 0; i < 4; ++i) fin &= isfin(quat[i]);
    for (int k = 0; k < K; ++k)
        for (int c = 0; c < 3; ++c) fin &= isfin(sh[3 * k + c]);
    if (!fin) return;

    /* O1 */
    for (int i = 0; i < 3; ++i)
        o->xc[i] = cam->R[3 * i] * mean[0] + cam->R[3 * i + 1] * mean[1] + cam->R[3 * i + 2] * mean[2] + cam->t[i];
    double x = o->xc[0], y = o->xc[1], z = o->xc[2];
    o->margin = fabs(z - near_plane) / near_plane;
    /* O2 */
    if (!(z > near_plane)) return;

    /* O3 */
    double qq = quat[0] * quat[0] + quat[1] * quat[1] + quat[2] * quat[2] + quat[3] * quat[3];
    if (!(qq > 0.0)) return;
    o->qnorm = sqrt(qq);
    for (int i = 0; i < 4; ++i) o->qn[i] = quat[i] / o->qnorm;
    quat_to_rot(o->qn, o->Rq);

    /* O4 */
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) o->M[3 * i + j] = o->Rq[3 * i + j] * scale[j];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double s = 0.0;
            for (int k = 0; k < 3; ++k) s += o->M[3 * i + k] * o->M[3 * j + k];
            o->Sig[3 * i + j] = s;
        }

    /* O5: Jacobian of (fx x/z + cx, fy y/z + cy) at the mean */
    o->J[0] = cam->fx / z; o->J[1] = 0.0; o->J[2] = -cam->fx * x / (z * z);
    o->J[3] = 0.0; o->J[4] = cam->fy / z; o->J[5] = -cam->fy * y / (z * z);
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 3; ++j) {
            double s = 0.0;
            for (int k = 0; k < 3; ++k) s += o->J[3 * i + k] * cam->R[3 * k + j];
            o->V[3 * i + j] = s;
        }
    double S2[4];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) {
            double s = 0.0;
            for (int a = 0; a < 3; ++a)
                for (int b = 0; b < 3; ++b) s += o->V[3 * i + a] * o->Sig[3 * a + b] * o->V[3 * j + b];
            S2[2 * i + j] = s;
        }
    o->A = S2[0] + lowpass;
    o->B = 0.5 * (S2[1] + S2[2]);
    o->C = S2[3] + lowpass;

    /* O6 */
    o->det = o->A * o->C - o->B * o->B;
    {
        double m = fabs(o->det) / (fabs(o->A * o->C) + 1e-300);
        if (m < o->margin) o->margin = m;
    }
    if (!(o->det > 0.0) || !isfin(o->det)) return;
    o->con[0] = o->C / o->det;
    o->con[1] = -o->B / o->det;
    o->con[2] = o->A / o->det;

    /* O7 */
    double mid = 0.5 * (o->A + o->C);
    double half = 0.5 * (o->A - o->C);
    o->lam = mid + sqrt(half * half + o->B * o->B);
    o->extent = 3.0 * sqrt(o->lam);

    /* O8 */
    o->u = cam->fx * x / z + cam->cx;
    o->v = cam->fy * y / z + cam->cy;
    if (!isfin(o->u) || !isfin(o->v) || !isfin(o->extent)) return;
    if (fabs(o->u) > BIG || fabs(o->v) > BIG || o->extent > BIG) return;
    o->r = (int64_t)ceil(o->extent);
    {
        double m = frac_margin(o->extent);
        if (m < o->margin) o->margin = m;
        m = frac_margin(o->u);
        if (m < o->margin) o->margin = m;
        m = frac_margin(o->v);
        if (m < o->margin) o->margin = m;
    }

    /* O9 */
    int64_t fu = (int64_t)floor(o->u), fv = (int64_t)floor(o->v);
    int64_t X0 = floordiv(fu - o->r, TILE), X1 = floordiv(fu + o->r, TILE);
    int64_t Y0 = floordiv(fv - o->r, TILE), Y1 = floordiv(fv + o->r, TILE);
    if (X0 < 0) X0 = 0;
    if (Y0 < 0) Y0 = 0;
    if (X1 > TX - 1) X1 = TX - 1;
    if (Y1 > TY - 1) Y1 = TY - 1;
    if (X0 > X1 || Y0 > Y1) return;
    o->rect[0] = X0; o->rect[1] = X1; o->rect[2] = Y0; o->rect[3] = Y1;

    /* O10 */
    double campos[3];
    for (int j = 0; j < 3; ++j)
        campos[j] = -(cam->R[j] * cam->t[0] + cam->R[3 + j] * cam->t[1] + cam->R[6 + j] * cam->t[2]);
    double d[3] = {mean[0] - campos[0], mean[1] - campos[1], mean[2] - campos[2]};
    o->dist = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
    if (!(o->dist > 0.0)) return;
    for (int j = 0; j < 3; ++j) o->dir[j] = d[j] / o->dist;
    orc_sh_basis(deg, o->dir[0], o->dir[1], o->dir[2], o->Y);
    for (int c = 0; c < 3; ++c) {
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += sh[3 * k + c] * o->Y[k];
        o->raw[c] = s + 0.5;
        o->clamp[c] = o->raw[c] < 0.0;
        o->rgb[c] = o->clamp[c] ? 0.0 : o->raw[c];
    }
    (void)sh_rows;
    o->visible = 1;
}

/*
 * orc_preprocess: O1-O10 for N Gaussians.
 * cam: 18 doubles (W, H, fx, fy, cx, cy, R[9] row-major, t[3]).
 * Inputs (double): means[N,3], scales[N,3] (activated), quats[N,4] (w,x,y,z,
 * any norm), opac[N] (activated), sh[N, sh_rows, 3] (first (deg+1)^2 rows used).
 * Outputs (any may be NULL): means2d[N,2], depth[N], cov2d[N,3] (A,B,C),
 * conic[N,3] (a,b,c), rgb[N,3], radii[N], rect[N,4] (X0,X1,Y0,Y1),
 * tiles[N], clamp[N,3], margin[N]. Culled Gaussians get zeros.
 */
void orc_preprocess(int64_t N, const double *camv, int deg, int sh_rows, double lowpass, double near_plane,
                    const double *means, const double *scales, const double *quats, const double *opac,
                    const double *sh, double *means2d, double *depth, double *cov2d, double *conic,
                    double *rgb, int32_t *radii, int64_t *rect, int64_t *tiles, uint8_t *clamp,
                    double *margin)
{
    ocam cam = cam_from(camv);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < N; ++g) {
        gauss_fwd o;
        gauss_forward(&cam, deg, sh_rows, lowpass, near_plane, means + 3 * g, scales + 3 * g,
                      quats + 4 * g, opac[g], sh + (size_t)3 * sh_rows * g, &o);
        int vis = o.visible;
        if (means2d) { means2d[2 * g] = vis ? o.u : 0.0; means2d[2 * g + 1] = vis ? o.v : 0.0; }
        if (depth) depth[g] = vis ? o.xc[2] : 0.0;
        if (cov2d) { cov2d[3 * g] = vis ? o.A : 0; cov2d[3 * g + 1] = vis ? o.B : 0; cov2d[3 * g + 2] = vis ? o.C : 0; }
        if (conic) for (int i = 0; i < 3; ++i) conic[3 * g + i] = vis ? o.con[i] : 0.0;
        if (rgb) for (int i = 0; i < 3; ++i) rgb[3 * g + i] = vis ? o.rgb[i] : 0.0;
        if (radii) radii[g] = vis ? (int32_t)o.r : 0;
        if (rect) for (int i = 0; i < 4; ++i) rect[4 * g + i] = vis ? o.rect[i] : 0;
        if (tiles) tiles[g] = vis ? (o.rect[1] - o.rect[0] + 1) * (o.rect[3] - o.rect[2] + 1) : 0;
        if (clamp) for (int i = 0; i < 3; ++i) clamp[3 * g + i] = vis ? o.clamp[i] : 0;
        if (margin) margin[g] = o.margin;
    }
}

/* ------------------------------------------------------------------ */
/* O11: binning and sort                                                */
/* ------------------------------------------------------------------ */
typedef struct {
    uint64_t key;
    uint32_t g;
} pair_t;

static int pair_cmp(const void *pa, const void *pb)
{
    const pair_t *a = (const pair_t *)pa, *b = (const pair_t *)pb;
    if (a->key != b->key) return a->key < b->key ? -1 : 1;
    if (a->g != b->g) return a->g < b->g ? -1 : 1;
    return 0;
}

/*
 * orc_bin_sort: O9 + O11 on given screen means (u, v), radii r and fp32 depths.
 * A Gaussian with r <= 0 is culled. Returns P (the pair count). When keys is
 * non-NULL and capacity >= P, writes keys[P], values[P] and ranges[TX*TY, 2]
 * ([first, last+1) of each tile, (0, 0) when empty).
 */
int64_t orc_bin_sort(int64_t N, int W, int H, const double *means2d, const int32_t *radii,
                     const float *depth, int64_t capacity, uint64_t *keys, uint32_t *values,
                     uint32_t *ranges)
{
    int TX = (W + TILE - 1) / TILE, TY = (H + TILE - 1) / TILE;
    int64_t P = 0;
    int64_t *rect = (int64_t *)malloc(sizeof(int64_t) * 4 * (N > 0 ? N : 1));
    for (int64_t g = 0; g < N; ++g) {
        rect[4 * g] = 1; rect[4 * g + 1] = 0; rect[4 * g + 2] = 1; rect[4 * g + 3] = 0;
        if (radii[g] <= 0) continue;
        int64_t fu = (int64_t)floor(means2d[2 * g]), fv = (int64_t)floor(means2d[2 * g + 1]);
        int64_t r = radii[g];
        int64_t X0 = floordiv(fu - r, TILE), X1 = floordiv(fu + r, TILE);
        int64_t Y0 = floordiv(fv - r, TILE), Y1 = floordiv(fv + r, TILE);
        if (X0 < 0) X0 = 0;
        if (Y0 < 0) Y0 = 0;
        if (X1 > TX - 1) X1 = TX - 1;
        if (Y1 > TY - 1) Y1 = TY - 1;
        if (X0 > X1 || Y0 > Y1) continue;
        rect[4 * g] = X0; rect[4 * g + 1] = X1; rect[4 * g + 2] = Y0; rect[4 * g + 3] = Y1;
        P += (X1 - X0 + 1) * (Y1 - Y0 + 1);
    }
    if (!keys || capacity < P) {
        free(rect);
        return P;
    }
    pair_t *pairs = (pair_t *)malloc(sizeof(pair_t) * (P > 0 ? P : 1));
    int64_t n = 0;
    for (int64_t g = 0; g < N; ++g) {
        if (rect[4 * g] > rect[4 * g + 1]) continue;
        uint32_t dbits;
        memcpy(&dbits, &depth[g], 4);
        for (int64_t ty = rect[4 * g + 2]; ty <= rect[4 * g + 3]; ++ty)
            for (int64_t tx = rect[4 * g]; tx <= rect[4 * g + 1]; ++tx) {
                uint64_t tile = (uint64_t)(ty * TX + tx);
                pairs[n].key = (tile << 32) | dbits;
                pairs[n].g = (uint32_t)g;
                ++n;
            }
    }
    qsort(pairs, (size_t)P, sizeof(pair_t), pair_cmp);
    for (int64_t t = 0; t < (int64_t)TX * TY; ++t) { ranges[2 * t] = 0; ranges[2 * t + 1] = 0; }
    for (int64_t i = 0; i < P; ++i) {
        keys[i] = pairs[i].key;
        values[i] = pairs[i].g;
        uint32_t t = (uint32_t)(pairs[i].key >> 32);
        if (i == 0 || (uint32_t)(pairs[i - 1].key >> 32) != t) ranges[2 * t] = (uint32_t)i;
        if (i == P - 1 || (uint32_t)(pairs[i + 1].key >> 32) != t) ranges[2 * t + 1] = (uint32_t)(i + 1);
    }
    free(pairs);
    free(rect);
    return P;
}

/* ------------------------------------------------------------------ */
/* O12: forward per pixel                                               */
/* ------------------------------------------------------------------ */
typedef struct {
    int W, H, TX;
    const uint32_t *ranges, *values;
    const double *means2d, *conic, *opac, *rgb;
    double bg[3];
    int surfel;         /* 1: 2D Gaussian surfels (S8), records in tf; 0: 3D Gaussians (conic) */
    const double *tf;   /* surfels: the screen homography M[N,3,3] of S3, row-major */
} raster_in;

/* S8 for surfel g at pixel centre (pxc, pyc); returns alpha, fills *e. */
typedef struct {
    double hx[3], hy[3], k[3], u, v, rho3, rho2, dx, dy, G, oG;
    int branch3;        /* 1: the surfel's own falloff is the larger, 0: the screen filter's */
} surfel_eval_t;
static double surfel_eval(const raster_in *in, uint32_t g, double pxc, double pyc, surfel_eval_t *e);

static double eval_alpha(const raster_in *in, uint32_t g, double pxc, double pyc, double *G_out,
                         double *dx_out, double *dy_out, double *oG_out)
{
    if (in->surfel) {
        surfel_eval_t e;
        double alpha = surfel_eval(in, g, pxc, pyc, &e);
        if (G_out) *G_out = e.G;
        if (dx_out) *dx_out = e.dx;
        if (dy_out) *dy_out = e.dy;
        if (oG_out) *oG_out = e.oG;
        return alpha;
    }
    double dx = pxc - in->means2d[2 * g], dy = pyc - in->means2d[2 * g + 1];
    double a = in->conic[3 * g], b = in->conic[3 * g + 1], c = in->conic[3 * g + 2];
    double Q = a * dx * dx + 2.0 * b * dx * dy + c * dy * dy;
    double G = exp(-0.5 * Q);
    double oG = in->opac[g] * G;
    if (G_out) *G_out = G;
    if (dx_out) *dx_out = dx;
    if (dy_out) *dy_out = dy;
    if (oG_out) *oG_out = oG;
    return oG < ALPHA_MAX ? oG : ALPHA_MAX;
}

static void pixel_forward(const raster_in *in, int px, int py, double C[3], double *T_out, uint32_t *last_out)
{
    int t = (py / TILE) * in->TX + px / TILE;
    uint32_t s = in->ranges[2 * t], e = in->ranges[2 * t + 1];
    double pxc = px + 0.5, pyc = py + 0.5;
    double T = 1.0;
    uint32_t last = 0;
    C[0] = C[1] = C[2] = 0.0;
    for (uint32_t i = s; i < e; ++i) {
        uint32_t g = in->values[i];
        double alpha = eval_alpha(in, g, pxc, pyc, NULL, NULL, NULL, NULL);
        if (alpha < ALPHA_MIN) continue;
        double Tn = T * (1.0 - alpha);
        if (Tn < T_MIN) break;
        for (int c = 0; c < 3; ++c) C[c] += in->rgb[3 * g + c] * alpha * T;
        T = Tn;
        last = i - s + 1;
    }
    *T_out = T;
    *last_out = last;
}

/*
 * orc_render_fwd: O12 over the whole image. conic holds (a, b, c) with
 * Q(d) = a dx^2 + 2 b dx dy + c dy^2. Outputs image[3,H,W] (planar),
 * final_T[H,W], n_contrib[H,W] (1-based list position of the last blended
 * entry within the tile's list; 0 if none).
 */
static void render_fwd_in(const raster_in *in, double *image, double *final_T, uint32_t *n_contrib)
{
    const int W = in->W, H = in->H;
#pragma omp parallel for schedule(dynamic, 4)
    for (int py = 0; py < H; ++py)
        for (int px = 0; px < W; ++px) {
            double C[3], T;
            uint32_t last;
            pixel_forward(in, px, py, C, &T, &last);
            size_t p = (size_t)py * W + px;
            for (int c = 0; c < 3; ++c) image[(size_t)c * W * H + p] = C[c] + T * in->bg[c];
            final_T[p] = T;
            n_contrib[p] = last;
        }
}

void orc_render_fwd(int W, int H, const uint32_t *ranges, const uint32_t *values,
                    const double *means2d, const double *conic, const double *opac, const double *rgb,
                    const double *bg, double *image, double *final_T, uint32_t *n_contrib)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, conic, opac, rgb, {bg[0], bg[1], bg[2]}};
    render_fwd_in(&in, image, final_T, n_contrib);
}

/* Forward of a list of sampled pixels (pix[i] = py * W + px). */
void orc_render_fwd_pixels(int W, int H, const uint32_t *ranges, const uint32_t *values,
                           const double *means2d, const double *conic, const double *opac,
                           const double *rgb, const double *bg, int64_t npix, const int64_t *pix,
                           double *image3, double *final_T, uint32_t *n_contrib)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, conic, opac, rgb, {bg[0], bg[1], bg[2]}};
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < npix; ++i) {
        int px = (int)(pix[i] % W), py = (int)(pix[i] / W);
        double C[3], T;
        uint32_t last;
        pixel_forward(&in, px, py, C, &T, &last);
        for (int c = 0; c < 3; ++c) image3[3 * i + c] = C[c] + T * in.bg[c];
        final_T[i] = T;
        n_contrib[i] = last;
    }
}

/* ------------------------------------------------------------------ */
/* Decision-aware matching of an fp32 forward against O12.              */
/* The fp32 evaluation and this fp64 one can take a different skip or    */
/* stop decision when alpha lies within rounding of 1/255 or T(1-alpha)   */
/* within rounding of 1e-4; both outcomes are then results of the        */
/* method. The explorer follows both branches of every such decision     */
/* (up to max_amb per pixel) and accepts the fp32 pixel if it matches     */
/* any resulting candidate.                                              */
/* ------------------------------------------------------------------ */
typedef struct {
    const raster_in *in;
    uint32_t s, e;
    double pxc, pyc;
    double d_alpha;  /* relative error bound on the fp32 alpha */
    int max_amb;
    const float *want; /* r, g, b, T */
    uint32_t want_nc;
    double tol;
    int found;       /* 1 = natural path, 2 = other branch */
    int overflow;
} explorer;

static void explore(explorer *x, uint32_t i, double T, const double C0[3], uint32_t last, int n_amb,
                    double errT, int natural)
{
    double C[3] = {C0[0], C0[1], C0[2]};
    for (; i < x->e; ++i) {
        if (x->found == 1) return;
        uint32_t g = x->in->values[i];
        double alpha = eval_alpha(x->in, g, x->pxc, x->pyc, NULL, NULL, NULL, NULL);
        int skip = alpha < ALPHA_MIN;
        if (fabs(alpha - ALPHA_MIN) <= x->d_alpha * ALPHA_MIN) {
            if (n_amb >= x->max_amb) { x->overflow = 1; return; }
            ++n_amb;
            if (!skip) { /* other branch: skip it */
                explore(x, i + 1, T, C, last, n_amb, errT, 0);
            } else {     /* other branch: take it (a stop test follows) */
                double Tn = T * (1.0 - alpha);
                if (Tn >= T_MIN || fabs(Tn - T_MIN) <= errT * T_MIN) {
                    double C2[3];
                    for (int c = 0; c < 3; ++c) C2[c] = C[c] + x->in->rgb[3 * g + c] * alpha * T;
                    double e2 = errT + 1.2e-7 + alpha / (1.0 - alpha) * x->d_alpha;
                    explore(x, i + 1, Tn, C2, i - x->s + 1, n_amb, e2, 0);
                }
                if (Tn < T_MIN || fabs(Tn - T_MIN) <= errT * T_MIN) {
                    /* taken then stopped: the pixel ends here unblended */
                    explore(x, x->e, T, C, last, n_amb, errT, 0);
                }
            }
        }
        if (skip) continue;
        double Tn = T * (1.0 - alpha);
        double eT = errT + 1.2e-7 + alpha / (1.0 - alpha) * x->d_alpha;
        int stop = Tn < T_MIN;
        if (fabs(Tn - T_MIN) <= eT * T_MIN) {
            if (n_amb >= x->max_amb) { x->overflow = 1; return; }
            ++n_amb;
            if (!stop) {
                explore(x, x->e, T, C, last, n_amb, errT, 0); /* other branch: stop here */
            } else {
                double C2[3];
                for (int c = 0; c < 3; ++c) C2[c] = C[c] + x->in->rgb[3 * g + c] * alpha * T;
                explore(x, i + 1, Tn, C2, i - x->s + 1, n_amb, eT, 0);
            }
        }
        if (stop) break;
        for (int c = 0; c < 3; ++c) C[c] += x->in->rgb[3 * g + c] * alpha * T;
        T = Tn;
        errT = eT;
        last = i - x->s + 1;
    }
    /* candidate complete */
    int ok = last == x->want_nc && fabs(T - (double)x->want[3]) <= x->tol;
    for (int c = 0; c < 3; ++c) ok &= fabs(C[c] + T * x->in->bg[c] - (double)x->want[c]) <= x->tol;
    if (ok) x->found = natural ? 1 : (x->found ? x->found : 2);
}

/*
 * orc_match_fwd: for each pixel of gpu image/final_T/n_contrib, status[p] =
 * 0 matched along the fp64 decisions, 1 matched another branch of an
 * ambiguous decision, 2 no match but more than max_amb ambiguous decisions
 * (masked), 3 mismatch. Returns the number of status-3 pixels.
 */
static int64_t match_in(const raster_in *in, const float *gpu_image, const float *gpu_T, const uint32_t *gpu_nc,
                        double d_alpha, int max_amb, double tol, int8_t *status)
{
    const int W = in->W, H = in->H;
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(+ : bad)
    for (int py = 0; py < H; ++py)
        for (int px = 0; px < W; ++px) {
            size_t p = (size_t)py * W + px;
            int t = (py / TILE) * in->TX + px / TILE;
            float want[4] = {gpu_image[p], gpu_image[(size_t)W * H + p], gpu_image[(size_t)2 * W * H + p], gpu_T[p]};
            explorer x = {in, in->ranges[2 * t], in->ranges[2 * t + 1], px + 0.5, py + 0.5, d_alpha, max_amb,
                          want, gpu_nc[p], tol, 0, 0};
            double C[3] = {0, 0, 0};
            explore(&x, x.s, 1.0, C, 0, 0, 0.0, 1);
            int st = x.found == 1 ? 0 : x.found == 2 ? 1 : x.overflow ? 2 : 3;
            status[p] = (int8_t)st;
            if (st == 3) ++bad;
        }
    return bad;
}

int64_t orc_match_fwd(int W, int H, const uint32_t *ranges, const uint32_t *values,
                      const double *means2d, const double *conic, const double *opac, const double *rgb,
                      const double *bg, const float *gpu_image, const float *gpu_T,
                      const uint32_t *gpu_nc, double d_alpha, int max_amb, double tol, int8_t *status)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, conic, opac, rgb, {bg[0], bg[1], bg[2]}};
    return match_in(&in, gpu_image, gpu_T, gpu_nc, d_alpha, max_amb, tol, status);
}

/* orc_match_fwd restricted to the pixels pix[npix] (flat py*W+px); the
 * GPU values come per sampled pixel: gpu_rgbT[npix][4] = (r, g, b, T). */
int64_t orc_match_fwd_pixels(int W, int H, const uint32_t *ranges, const uint32_t *values,
                             const double *means2d, const double *conic, const double *opac, const double *rgb,
                             const double *bg, int64_t npix, const int64_t *pix, const float *gpu_rgbT,
                             const uint32_t *gpu_nc, double d_alpha, int max_amb, double tol, int8_t *status)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, conic, opac, rgb, {bg[0], bg[1], bg[2]}};
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : bad)
    for (int64_t k = 0; k < npix; ++k) {
        int px = (int)(pix[k] % W), py = (int)(pix[k] / W);
        int t = (py / TILE) * in.TX + px / TILE;
        explorer x = {&in, ranges[2 * t], ranges[2 * t + 1], px + 0.5, py + 0.5, d_alpha, max_amb,
                      &gpu_rgbT[4 * k], gpu_nc[k], tol, 0, 0};
        double C[3] = {0, 0, 0};
        explore(&x, x.s, 1.0, C, 0, 0, 0.0, 1);
        int st = x.found == 1 ? 0 : x.found == 2 ? 1 : x.overflow ? 2 : 3;
        status[k] = (int8_t)st;
        if (st == 3) ++bad;
    }
    return bad;
}

/* ------------------------------------------------------------------ */
/* O13: backward per pixel                                              */
/* grad2d[N,9] = (drgb[3], dopacity, da, db, dc, du, dv), accumulated.   */
/* ------------------------------------------------------------------ */
typedef struct {
    uint32_t g;
    double alpha, T, G, dx, dy, oG;
} blend_rec;

#define SURFEL_GRAD_N 15
static void surfel_pixel_grad(const raster_in *in, uint32_t g, double pxc, double pyc, double dalpha, double *d);

static void pixel_backward(const raster_in *in, int px, int py, const double dL[3], double *grad2d,
                           blend_rec *buf)
{
    int t = (py / TILE) * in->TX + px / TILE;
    uint32_t s = in->ranges[2 * t], e = in->ranges[2 * t + 1];
    double pxc = px + 0.5, pyc = py + 0.5;
    /* replay O12, recording every blended entry */
    double T = 1.0;
    int nb = 0;
    for (uint32_t i = s; i < e; ++i) {
        uint32_t g = in->values[i];
        double G, dx, dy, oG;
        double alpha = eval_alpha(in, g, pxc, pyc, &G, &dx, &dy, &oG);
        if (alpha < ALPHA_MIN) continue;
        double Tn = T * (1.0 - alpha);
        if (Tn < T_MIN) break;
        blend_rec r = {g, alpha, T, G, dx, dy, oG};
        buf[nb++] = r;
        T = Tn;
    }
    /* reverse: A is the colour of everything behind the current entry, normalised */
    double A[3] = {in->bg[0], in->bg[1], in->bg[2]};
    for (int j = nb - 1; j >= 0; --j) {
        const blend_rec *r = &buf[j];
        uint32_t g = r->g;
        const double *c = &in->rgb[3 * g];
        double dalpha = 0.0;
        for (int ch = 0; ch < 3; ++ch) dalpha += (c[ch] - A[ch]) * dL[ch];
        dalpha *= r->T;
        const int nrec = in->surfel ? SURFEL_GRAD_N : 9;
        double *gg = &grad2d[(size_t)nrec * g];
        double d[SURFEL_GRAD_N] = {0};
        for (int ch = 0; ch < 3; ++ch) d[ch] = r->alpha * r->T * dL[ch];
        for (int ch = 0; ch < 3; ++ch) A[ch] = r->alpha * c[ch] + (1.0 - r->alpha) * A[ch];
        if (in->surfel) {
            if (!(r->oG > ALPHA_MAX)) surfel_pixel_grad(in, g, pxc, pyc, dalpha, d);
        } else if (!(r->oG > ALPHA_MAX)) {
            double a = in->conic[3 * g], b = in->conic[3 * g + 1], cc = in->conic[3 * g + 2];
            double dQ = -0.5 * r->G * in->opac[g] * dalpha;
            d[3] = r->G * dalpha;
            d[4] = dQ * r->dx * r->dx;
            d[5] = dQ * 2.0 * r->dx * r->dy;
            d[6] = dQ * r->dy * r->dy;
            d[7] = dQ * -2.0 * (a * r->dx + b * r->dy);
            d[8] = dQ * -2.0 * (b * r->dx + cc * r->dy);
        }
        for (int k = 0; k < nrec; ++k) {
#pragma omp atomic
            gg[k] += d[k];
        }
    }
}

static void render_bwd_in(const raster_in *in, const double *dL_dimage, double *grad2d)
{
    const int W = in->W, H = in->H;
    int TY = (H + TILE - 1) / TILE;
    uint32_t maxlen = 0;
    for (int t = 0; t < in->TX * TY; ++t)
        if (in->ranges[2 * t + 1] - in->ranges[2 * t] > maxlen) maxlen = in->ranges[2 * t + 1] - in->ranges[2 * t];
#pragma omp parallel
    {
        blend_rec *buf = (blend_rec *)malloc(sizeof(blend_rec) * (maxlen + 1));
#pragma omp for schedule(dynamic, 2)
        for (int py = 0; py < H; ++py)
            for (int px = 0; px < W; ++px) {
                size_t p = (size_t)py * W + px;
                double dL[3] = {dL_dimage[p], dL_dimage[(size_t)W * H + p], dL_dimage[(size_t)2 * W * H + p]};
                pixel_backward(in, px, py, dL, grad2d, buf);
            }
        free(buf);
    }
}

void orc_render_bwd(int W, int H, int64_t N, const uint32_t *ranges, const uint32_t *values,
                    const double *means2d, const double *conic, const double *opac, const double *rgb,
                    const double *bg, const double *dL_dimage, double *grad2d)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, conic, opac, rgb, {bg[0], bg[1], bg[2]}};
    (void)N;
    render_bwd_in(&in, dL_dimage, grad2d);
}

/* ------------------------------------------------------------------ */
/* O14: per-Gaussian chain rule                                         */
/* ------------------------------------------------------------------ */
/* d Rq / d qn_k for qn = (w, x, y, z), each a 3x3 row-major matrix. */
static void drot_dq(const double q[4], double D[4][9])
{
    double w = q[0], x = q[1], y = q[2], z = q[3];
    /* entry (i,j) of Rq differentiated by hand from quat_to_rot */
    double Dw[9] = {0, -2 * z, 2 * y, 2 * z, 0, -2 * x, -2 * y, 2 * x, 0};
    double Dx[9] = {0, 2 * y, 2 * z, 2 * y, -4 * x, -2 * w, 2 * z, 2 * w, -4 * x};
    double Dy[9] = {-4 * y, 2 * x, 2 * w, 2 * x, 0, 2 * z, -2 * w, 2 * z, -4 * y};
    double Dz[9] = {-4 * z, -2 * w, 2 * x, 2 * w, -4 * z, 2 * y, 2 * x, 2 * y, 0};
    memcpy(D[0], Dw, sizeof Dw);
    memcpy(D[1], Dx, sizeof Dx);
    memcpy(D[2], Dy, sizeof Dy);
    memcpy(D[3], Dz, sizeof Dz);
}

/*
 * orc_preprocess_bwd: O14. grad2d[N,9] as produced by orc_render_bwd.
 * Outputs are ACCUMULATED (+=): dmeans[N,3], dscales[N,3], dquats[N,4],
 * dopac[N], dsh[N,sh_rows,3], dmeans2d[N,2] (may be NULL).
 */
void orc_preprocess_bwd(int64_t N, const double *camv, int deg, int sh_rows, double lowpass, double near_plane,
                        const double *means, const double *scales, const double *quats, const double *opac,
                        const double *sh, const double *grad2d, double *dmeans, double *dscales,
                        double *dquats, double *dopac, double *dsh, double *dmeans2d)
{
    ocam cam = cam_from(camv);
    int K = (deg + 1) * (deg + 1);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < N; ++g) {
        gauss_fwd o;
        const double *shg = sh + (size_t)3 * sh_rows * g;
        gauss_forward(&cam, deg, sh_rows, lowpass, near_plane, means + 3 * g, scales + 3 * g, quats + 4 * g,
                      opac[g], shg, &o);
        if (!o.visible) continue;
        const double *d2 = grad2d + 9 * g;
        double dmu[3] = {0, 0, 0};

        /* colour */
        double draw[3];
        for (int c = 0; c < 3; ++c) draw[c] = o.clamp[c] ? 0.0 : d2[c];
        double dY[48];
        orc_sh_basis_grad(deg, o.dir[0], o.dir[1], o.dir[2], dY);
        double ddir[3] = {0, 0, 0};
        for (int k = 0; k < K; ++k)
            for (int c = 0; c < 3; ++c) {
                dsh[(size_t)3 * sh_rows * g + 3 * k + c] += o.Y[k] * draw[c];
                for (int j = 0; j < 3; ++j) ddir[j] += shg[3 * k + c] * dY[3 * k + j] * draw[c];
            }
        double dd = o.dir[0] * ddir[0] + o.dir[1] * ddir[1] + o.dir[2] * ddir[2];
        for (int j = 0; j < 3; ++j) dmu[j] += (ddir[j] - o.dir[j] * dd) / o.dist;

        /* conic -> Sigma' -> (Sigma, V) */
        double Con[4] = {o.con[0], o.con[1], o.con[1], o.con[2]};
        double Cb[4] = {d2[4], 0.5 * d2[5], 0.5 * d2[5], d2[6]};
        double tmp[4], Sb2[4];
        for (int i = 0; i < 2; ++i)
            for (int j = 0; j < 2; ++j) {
                double s = 0;
                for (int k = 0; k < 2; ++k) s += Con[2 * i + k] * Cb[2 * k + j];
                tmp[2 * i + j] = s;
            }
        for (int i = 0; i < 2; ++i)
            for (int j = 0; j < 2; ++j) {
                double s = 0;
                for (int k = 0; k < 2; ++k) s += tmp[2 * i + k] * Con[2 * k + j];
                Sb2[2 * i + j] = -s;
            }
        double Sb3[9];
        for (int a = 0; a < 3; ++a)
            for (int b = 0; b < 3; ++b) {
                double s = 0;
                for (int i = 0; i < 2; ++i)
                    for (int j = 0; j < 2; ++j) s += o.V[3 * i + a] * Sb2[2 * i + j] * o.V[3 * j + b];
                Sb3[3 * a + b] = s;
            }
        double Vb[6];
        for (int i = 0; i < 2; ++i)
            for (int b = 0; b < 3; ++b) {
                double s = 0;
                for (int j = 0; j < 2; ++j)
                    for (int a = 0; a < 3; ++a) s += Sb2[2 * i + j] * o.V[3 * j + a] * o.Sig[3 * a + b];
                Vb[3 * i + b] = 2.0 * s;
            }
        double Jb[6];
        for (int i = 0; i < 2; ++i)
            for (int k = 0; k < 3; ++k) {
                double s = 0;
                for (int j = 0; j < 3; ++j) s += Vb[3 * i + j] * cam.R[3 * k + j];
                Jb[3 * i + k] = s;
            }

        /* camera-space mean from J and from (u, v) */
        double x = o.xc[0], y = o.xc[1], z = o.xc[2];
        double fx = cam.fx, fy = cam.fy, du = d2[7], dv = d2[8];
        double xb = -fx * Jb[2] / (z * z) + fx * du / z;
        double yb = -fy * Jb[5] / (z * z) + fy * dv / z;
        double zb = -fx * Jb[0] / (z * z) - fy * Jb[4] / (z * z) + 2.0 * fx * x * Jb[2] / (z * z * z) +
                    2.0 * fy * y * Jb[5] / (z * z * z) - fx * x * du / (z * z) - fy * y * dv / (z * z);
        for (int j = 0; j < 3; ++j) dmu[j] += cam.R[j] * xb + cam.R[3 + j] * yb + cam.R[6 + j] * zb;

        /* scale and rotation */
        double Mb[9];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j) {
                double s = 0;
                for (int k = 0; k < 3; ++k) s += Sb3[3 * i + k] * o.M[3 * k + j];
                Mb[3 * i + j] = 2.0 * s;
            }
        for (int j = 0; j < 3; ++j) {
            double s = 0;
            for (int i = 0; i < 3; ++i) s += Mb[3 * i + j] * o.Rq[3 * i + j];
            dscales[3 * g + j] += s;
        }
        double Rb[9];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j) Rb[3 * i + j] = Mb[3 * i + j] * scales[3 * g + j];
        double D[4][9], qb[4];
        drot_dq(o.qn, D);
        for (int k = 0; k < 4; ++k) {
            double s = 0;
            for (int i = 0; i < 9; ++i) s += Rb[i] * D[k][i];
            qb[k] = s;
        }
        double qdot = 0;
        for (int k = 0; k < 4; ++k) qdot += o.qn[k] * qb[k];
        for (int k = 0; k < 4; ++k) dquats[4 * g + k] += (qb[k] - qdot * o.qn[k]) / o.qnorm;

        dopac[g] += d2[3];
        for (int j = 0; j < 3; ++j) dmeans[3 * g + j] += dmu[j];
        if (dmeans2d) {
            dmeans2d[2 * g] += du;
            dmeans2d[2 * g + 1] += dv;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Decision signature of O12 over an image: a hash of every pixel's     */
/* blended entries, their alpha-clamp state and its stop position. Two   */
/* parameter sets with equal signatures (and equal pair lists) lie on    */
/* the same smooth piece of the forward, where central differences are   */
/* valid.                                                               */
/* ------------------------------------------------------------------ */
static uint64_t mix64(uint64_t h, uint64_t v)
{
    h ^= v + 0x9e3779b97f4a7c15ULL + (h << 6) + (h >> 2);
    h *= 0xff51afd7ed558ccdULL;
    return h ^ (h >> 33);
}

static uint64_t decision_hash_in(const raster_in *in)
{
    const int W = in->W, H = in->H;
    uint64_t total = 0;
    for (int py = 0; py < H; ++py)
        for (int px = 0; px < W; ++px) {
            int t = (py / TILE) * in->TX + px / TILE;
            uint32_t s = in->ranges[2 * t], e = in->ranges[2 * t + 1];
            uint64_t h = mix64(0x1234567ULL, (uint64_t)py * W + px);
            double T = 1.0;
            for (uint32_t i = s; i < e; ++i) {
                double oG;
                surfel_eval_t se;
                double alpha = eval_alpha(in, in->values[i], px + 0.5, py + 0.5, NULL, NULL, NULL, &oG);
                if (alpha < ALPHA_MIN) continue;
                double Tn = T * (1.0 - alpha);
                if (Tn < T_MIN) { h = mix64(h, 0xffffffffULL + i); break; }
                uint64_t branch = 0;
                if (in->surfel) {  /* which of the two falloffs is the larger also splits the pieces */
                    surfel_eval(in, in->values[i], px + 0.5, py + 0.5, &se);
                    branch = (uint64_t)se.branch3 << 1;
                }
                h = mix64(h, 4ULL * i + branch + (oG > ALPHA_MAX ? 1 : 0));
                T = Tn;
            }
            total += h;
        }
    return total;
}

uint64_t orc_decision_hash(int W, int H, const uint32_t *ranges, const uint32_t *values,
                           const double *means2d, const double *conic, const double *opac)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, conic, opac, NULL, {0, 0, 0}};
    return decision_hash_in(&in);
}

/* O13 at the sampled pixels pix[i] = py * W + px only (grad2d accumulated). */
void orc_render_bwd_pixels(int W, int H, int64_t N, const uint32_t *ranges, const uint32_t *values,
                           const double *means2d, const double *conic, const double *opac, const double *rgb,
                           const double *bg, const double *dL_dimage, int64_t npix, const int64_t *pix,
                           double *grad2d)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, conic, opac, rgb, {bg[0], bg[1], bg[2]}};
    int TY = (H + TILE - 1) / TILE;
    uint32_t maxlen = 0;
    for (int t = 0; t < in.TX * TY; ++t)
        if (ranges[2 * t + 1] - ranges[2 * t] > maxlen) maxlen = ranges[2 * t + 1] - ranges[2 * t];
    (void)N;
#pragma omp parallel
    {
        blend_rec *buf = (blend_rec *)malloc(sizeof(blend_rec) * (maxlen + 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < npix; ++i) {
            size_t p = (size_t)pix[i];
            double dL[3] = {dL_dimage[p], dL_dimage[(size_t)W * H + p], dL_dimage[(size_t)2 * W * H + p]};
            pixel_backward(&in, (int)(p % W), (int)(p / W), dL, grad2d, buf);
        }
        free(buf);
    }
}

/* ================================================================== */
/* 2D Gaussian surfels: S1-S10.                                         */
/*                                                                      */
/* The second pipeline is the one of "2D Gaussian Splatting for          */
/* Geometrically Accurate Radiance Fields", which the Odin review page   */
/* evaluates beside 3D Gaussian splatting (referee report summary) and   */
/* lists among its references. The pages print none of its formulas;    */
/* the steps are this project's reading of that method. A surfel is a    */
/* planar Gaussian: centre mu, two tangent axes (the first two columns   */
/* of its rotation), two scales (s_u, s_v), an opacity and SH colour.    */
/*                                                                      */
/*   S1  camera      X = R mu + t; cull z <= near, non-finite inputs     */
/*   S2  frame       unit quaternion -> Rq, t_u = Rq e1, t_v = Rq e2;    */
/*                   a = s_u R t_u, b = s_v R t_v (camera frame)         */
/*   S3  homography  the surfel point (u, v) is the camera point         */
/*                   X + u a + v b, i.e. the homogeneous screen point    */
/*                   M (u, v, 1) with M = K [a | b | X],                 */
/*                   K = [[fx, 0, cx], [0, fy, cy], [0, 0, 1]]           */
/*   S4  centre      c = (fx X/Z + cx, fy Y/Z + cy), depth Z             */
/*   S5  extent      the 3-sigma disc u^2 + v^2 <= 9 lies beyond the     */
/*                   near plane (cull otherwise); its image is an        */
/*                   ellipse, bounded by the tangents of the dual conic  */
/*                   M diag(1, 1, -1/9) M^T; r = ceil of the largest     */
/*                   distance from c to a side of that box, and at least */
/*                   3 sigma_f of the screen filter                      */
/*   S6  tile rect   O9 on (c, r)                                        */
/*   S7  colour      O10                                                 */
/*   S8  per pixel   rows M0, M1, M2 of M: h_x = M0 - x M2 and            */
/*                   h_y = M1 - y M2 are the two planes through the      */
/*                   pixel's ray, written in the surfel's (u, v, 1);     */
/*                   k = h_x x h_y, (u, v) = (k0/k2, k1/k2) is where the */
/*                   ray meets the surfel plane, rho3 = u^2 + v^2; the   */
/*                   screen filter of variance sigma_f^2 = 1/2 gives     */
/*                   rho2 = |pixel - c|^2 / sigma_f^2;                   */
/*                   G = exp(-min(rho3, rho2)/2), alpha = min(0.99, o G) */
/*                   (k2 = 0, a ray parallel to the plane: rho3 = inf);  */
/*                   compositing as O12                                  */
/*   S9  backward    O13, the 2D part through S8 (sums of dL/dM and      */
/*                   dL/dc per surfel)                                   */
/*   S10 chain rule  per surfel, back through S1-S4 and S7               */
/* ================================================================== */
static const double SURFEL_FILTER_VAR = 0.5; /* sigma_f^2, in pixels^2 */

static void cross3(const double a[3], const double b[3], double o[3])
{
    o[0] = a[1] * b[2] - a[2] * b[1];
    o[1] = a[2] * b[0] - a[0] * b[2];
    o[2] = a[0] * b[1] - a[1] * b[0];
}

static double surfel_eval(const raster_in *in, uint32_t g, double pxc, double pyc, surfel_eval_t *e)
{
    const double *M = in->tf + 9 * (size_t)g;
    for (int j = 0; j < 3; ++j) {
        e->hx[j] = M[j] - pxc * M[6 + j];
        e->hy[j] = M[3 + j] - pyc * M[6 + j];
    }
    cross3(e->hx, e->hy, e->k);
    e->dx = pxc - in->means2d[2 * g];
    e->dy = pyc - in->means2d[2 * g + 1];
    e->rho2 = (e->dx * e->dx + e->dy * e->dy) / SURFEL_FILTER_VAR;
    if (e->k[2] != 0.0) {
        e->u = e->k[0] / e->k[2];
        e->v = e->k[1] / e->k[2];
        e->rho3 = e->u * e->u + e->v * e->v;
    } else {
        e->u = e->v = 0.0;
        e->rho3 = INFINITY;
    }
    e->branch3 = e->rho3 <= e->rho2;
    e->G = exp(-0.5 * (e->branch3 ? e->rho3 : e->rho2));
    e->oG = in->opac[g] * e->G;
    return e->oG < ALPHA_MAX ? e->oG : ALPHA_MAX;
}

/* S9: the 2D part of one blended (pixel, surfel) entry with dL/dalpha =
 * dalpha (alpha below its clamp): d[3] dL/do, d[4..12] dL/dM (row-major),
 * d[13..14] dL/dc. */
static void surfel_pixel_grad(const raster_in *in, uint32_t g, double pxc, double pyc, double dalpha, double *d)
{
    surfel_eval_t e;
    surfel_eval(in, g, pxc, pyc, &e);
    d[3] = e.G * dalpha;
    double drho = -0.5 * e.G * in->opac[g] * dalpha; /* alpha = o exp(-rho/2) */
    if (e.branch3) {
        double du = 2.0 * e.u * drho, dv = 2.0 * e.v * drho;
        double dk[3] = {du / e.k[2], dv / e.k[2], -(du * e.u + dv * e.v) / e.k[2]};
        double dhx[3], dhy[3];
        cross3(e.hy, dk, dhx); /* d(dk . (hx x hy))/dhx = hy x dk */
        cross3(dk, e.hx, dhy); /* and /dhy = dk x hx */
        for (int j = 0; j < 3; ++j) {
            d[4 + j] = dhx[j];
            d[7 + j] = dhy[j];
            d[10 + j] = -pxc * dhx[j] - pyc * dhy[j];
        }
    } else {
        d[13] = drho * -2.0 * e.dx / SURFEL_FILTER_VAR;
        d[14] = drho * -2.0 * e.dy / SURFEL_FILTER_VAR;
    }
}

/* Everything S1-S7 derives for one surfel. */
typedef struct {
    int visible;
    double X[3], qn[4], qnorm, Rq[9], Rtu[3], Rtv[3], a[3], b[3], M[9];
    double c[2], ext;
    int64_t r, rect[4];
    double dir[3], dist, Y[16], raw[3], rgb[3];
    unsigned char clamp[3];
    double margin;
} surfel_fwd;

static void surfel_forward(const ocam *cam, int deg, double near_plane, const double *mean, const double *scale,
                           const double *quat, double opac, const double *sh, surfel_fwd *o)
{
    memset(o, 0, sizeof(*o));
    o->margin = INFINITY;
    int K = (deg + 1) * (deg + 1);
    int TX = (cam->W + TILE - 1) / TILE, TY = (cam->H + TILE - 1) / TILE;
    int fin = isfin(opac) & isfin(scale[0]) & isfin(scale[1]);
    for (int i = 0; i < 3; ++i) fin &= isfin(mean[i]);
    for (int i = 0; i < 4; ++i) fin &= isfin(quat[i]);
    for (int k = 0; k < K; ++k)
        for (int c = 0; c < 3; ++c) fin &= isfin(sh[3 * k + c]);
    if (!fin) return;
    /* S1 */
    for (int i = 0; i < 3; ++i)
        o->X[i] = cam->R[3 * i] * mean[0] + cam->R[3 * i + 1] * mean[1] + cam->R[3 * i + 2] * mean[2] + cam->t[i];
    double Z = o->X[2];
    o->margin = fabs(Z - near_plane) / near_plane;
    if (!(Z > near_plane)) return;
    /* S2 */
    double qq = quat[0] * quat[0] + quat[1] * quat[1] + quat[2] * quat[2] + quat[3] * quat[3];
    if (!(qq > 0.0)) return;
    o->qnorm = sqrt(qq);
    for (int i = 0; i < 4; ++i) o->qn[i] = quat[i] / o->qnorm;
    quat_to_rot(o->qn, o->Rq);
    for (int i = 0; i < 3; ++i) {
        double su = 0.0, sv = 0.0;
        for (int k = 0; k < 3; ++k) {
            su += cam->R[3 * i + k] * o->Rq[3 * k];
            sv += cam->R[3 * i + k] * o->Rq[3 * k + 1];
        }
        o->Rtu[i] = su;
        o->Rtv[i] = sv;
        o->a[i] = scale[0] * su;
        o->b[i] = scale[1] * sv;
    }
    /* S3: row i of K times the columns a, b, X */
    const double Kr[3][3] = {{cam->fx, 0.0, cam->cx}, {0.0, cam->fy, cam->cy}, {0.0, 0.0, 1.0}};
    for (int i = 0; i < 3; ++i) {
        double ra = 0.0, rb = 0.0, rx = 0.0;
        for (int k = 0; k < 3; ++k) {
            ra += Kr[i][k] * o->a[k];
            rb += Kr[i][k] * o->b[k];
            rx += Kr[i][k] * o->X[k];
        }
        o->M[3 * i] = ra;
        o->M[3 * i + 1] = rb;
        o->M[3 * i + 2] = rx;
    }
    /* S4 */
    o->c[0] = cam->fx * o->X[0] / Z + cam->cx;
    o->c[1] = cam->fy * o->X[1] / Z + cam->cy;
    /* S5: the disc in front of the near plane, then the box of its image */
    double zmin = Z - 3.0 * sqrt(o->a[2] * o->a[2] + o->b[2] * o->b[2]);
    {
        double m = fabs(zmin - near_plane) / near_plane;
        if (m < o->margin) o->margin = m;
    }
    if (!(zmin > near_plane)) return;
    double Cd[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            Cd[3 * i + j] = o->M[3 * i] * o->M[3 * j] + o->M[3 * i + 1] * o->M[3 * j + 1] -
                            o->M[3 * i + 2] * o->M[3 * j + 2] / 9.0;
    double ext = 3.0 * sqrt(SURFEL_FILTER_VAR);
    for (int ax = 0; ax < 2; ++ax) {
        /* tangent lines x = s (ax 0) or y = s (ax 1): l = e_ax - s e_3, l^T Cd l = 0 */
        double A = Cd[4 * ax], B = Cd[3 * ax + 2], C = Cd[8];
        double disc = B * B - A * C;
        if (!(disc >= 0.0) || C == 0.0) return;
        double s1 = (B + sqrt(disc)) / C, s2 = (B - sqrt(disc)) / C;
        double e1 = fabs(s1 - o->c[ax]), e2 = fabs(s2 - o->c[ax]);
        if (e1 > ext) ext = e1;
        if (e2 > ext) ext = e2;
    }
    o->ext = ext;
    if (!isfin(o->c[0]) || !isfin(o->c[1]) || !isfin(ext)) return;
    if (fabs(o->c[0]) > BIG || fabs(o->c[1]) > BIG || ext > BIG) return;
    o->r = (int64_t)ceil(ext);
    {
        double m = frac_margin(ext);
        if (m < o->margin) o->margin = m;
        m = frac_margin(o->c[0]);
        if (m < o->margin) o->margin = m;
        m = frac_margin(o->c[1]);
        if (m < o->margin) o->margin = m;
    }
    /* S6 */
    int64_t fu = (int64_t)floor(o->c[0]), fv = (int64_t)floor(o->c[1]);
    int64_t X0 = floordiv(fu - o->r, TILE), X1 = floordiv(fu + o->r, TILE);
    int64_t Y0 = floordiv(fv - o->r, TILE), Y1 = floordiv(fv + o->r, TILE);
    if (X0 < 0) X0 = 0;
    if (Y0 < 0) Y0 = 0;
    if (X1 > TX - 1) X1 = TX - 1;
    if (Y1 > TY - 1) Y1 = TY - 1;
    if (X0 > X1 || Y0 > Y1) return;
    o->rect[0] = X0; o->rect[1] = X1; o->rect[2] = Y0; o->rect[3] = Y1;
    /* S7 */
    double campos[3];
    for (int j = 0; j < 3; ++j)
        campos[j] = -(cam->R[j] * cam->t[0] + cam->R[3 + j] * cam->t[1] + cam->R[6 + j] * cam->t[2]);
    double d[3] = {mean[0] - campos[0], mean[1] - campos[1], mean[2] - campos[2]};
    o->dist = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
    if (!(o->dist > 0.0)) return;
    for (int j = 0; j < 3; ++j) o->dir[j] = d[j] / o->dist;
    orc_sh_basis(deg, o->dir[0], o->dir[1], o->dir[2], o->Y);
    for (int c = 0; c < 3; ++c) {
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += sh[3 * k + c] * o->Y[k];
        o->raw[c] = s + 0.5;
        o->clamp[c] = o->raw[c] < 0.0;
        o->rgb[c] = o->clamp[c] ? 0.0 : o->raw[c];
    }
    o->visible = 1;
}

/*
 * orc_surfel_preprocess: S1-S7 for N surfels. Inputs as orc_preprocess, with
 * scales[N,2] = (s_u, s_v). Outputs (any may be NULL): means2d[N,2] (c),
 * depth[N], tf[N,9] (M, row-major), rgb[N,3], radii[N], rect[N,4], tiles[N],
 * clamp[N,3], margin[N]. Culled surfels get zeros.
 */
void orc_surfel_preprocess(int64_t N, const double *camv, int deg, int sh_rows, double near_plane,
                           const double *means, const double *scales, const double *quats, const double *opac,
                           const double *sh, double *means2d, double *depth, double *tf, double *rgb,
                           int32_t *radii, int64_t *rect, int64_t *tiles, uint8_t *clamp, double *margin)
{
    ocam cam = cam_from(camv);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < N; ++g) {
        surfel_fwd o;
        surfel_forward(&cam, deg, near_plane, means + 3 * g, scales + 2 * g, quats + 4 * g, opac[g],
                       sh + (size_t)3 * sh_rows * g, &o);
        int vis = o.visible;
        if (means2d) { means2d[2 * g] = vis ? o.c[0] : 0.0; means2d[2 * g + 1] = vis ? o.c[1] : 0.0; }
        if (depth) depth[g] = vis ? o.X[2] : 0.0;
        if (tf) for (int i = 0; i < 9; ++i) tf[9 * g + i] = vis ? o.M[i] : 0.0;
        if (rgb) for (int i = 0; i < 3; ++i) rgb[3 * g + i] = vis ? o.rgb[i] : 0.0;
        if (radii) radii[g] = vis ? (int32_t)o.r : 0;
        if (rect) for (int i = 0; i < 4; ++i) rect[4 * g + i] = vis ? o.rect[i] : 0;
        if (tiles) tiles[g] = vis ? (o.rect[1] - o.rect[0] + 1) * (o.rect[3] - o.rect[2] + 1) : 0;
        if (clamp) for (int i = 0; i < 3; ++i) clamp[3 * g + i] = vis ? o.clamp[i] : 0;
        if (margin) margin[g] = o.margin;
    }
}

/* S8 + O12 over the image, from the tile lists of orc_bin_sort on (c, r). */
void orc_surfel_render_fwd(int W, int H, const uint32_t *ranges, const uint32_t *values, const double *means2d,
                           const double *tf, const double *opac, const double *rgb, const double *bg, double *image,
                           double *final_T, uint32_t *n_contrib)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, NULL, opac, rgb, {bg[0], bg[1], bg[2]},
                    1, tf};
    render_fwd_in(&in, image, final_T, n_contrib);
}

/* orc_match_fwd for surfels. */
int64_t orc_surfel_match_fwd(int W, int H, const uint32_t *ranges, const uint32_t *values, const double *means2d,
                             const double *tf, const double *opac, const double *rgb, const double *bg,
                             const float *gpu_image, const float *gpu_T, const uint32_t *gpu_nc, double d_alpha,
                             int max_amb, double tol, int8_t *status)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, NULL, opac, rgb, {bg[0], bg[1], bg[2]},
                    1, tf};
    return match_in(&in, gpu_image, gpu_T, gpu_nc, d_alpha, max_amb, tol, status);
}

/* S9: grad[N,15] accumulated: drgb[3], dopacity, dM[9] (row-major), dc[2]. */
void orc_surfel_render_bwd(int W, int H, const uint32_t *ranges, const uint32_t *values, const double *means2d,
                           const double *tf, const double *opac, const double *rgb, const double *bg,
                           const double *dL_dimage, double *grad)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, NULL, opac, rgb, {bg[0], bg[1], bg[2]},
                    1, tf};
    render_bwd_in(&in, dL_dimage, grad);
}

uint64_t orc_surfel_decision_hash(int W, int H, const uint32_t *ranges, const uint32_t *values,
                                  const double *means2d, const double *tf, const double *opac)
{
    raster_in in = {W, H, (W + TILE - 1) / TILE, ranges, values, means2d, NULL, opac, NULL, {0, 0, 0}, 1, tf};
    return decision_hash_in(&in);
}

/*
 * orc_surfel_preprocess_bwd: S10. grad[N,15] as orc_surfel_render_bwd gives
 * it. Outputs ACCUMULATED: dmeans[N,3], dscales[N,2], dquats[N,4], dopac[N],
 * dsh[N,sh_rows,3].
 */
void orc_surfel_preprocess_bwd(int64_t N, const double *camv, int deg, int sh_rows, double near_plane,
                               const double *means, const double *scales, const double *quats, const double *opac,
                               const double *sh, const double *grad, double *dmeans, double *dscales,
                               double *dquats, double *dopac, double *dsh)
{
    ocam cam = cam_from(camv);
    int K = (deg + 1) * (deg + 1);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < N; ++g) {
        surfel_fwd o;
        const double *shg = sh + (size_t)3 * sh_rows * g;
        surfel_forward(&cam, deg, near_plane, means + 3 * g, scales + 2 * g, quats + 4 * g, opac[g], shg, &o);
        if (!o.visible) continue;
        const double *d = grad + (size_t)SURFEL_GRAD_N * g;
        double dmu[3] = {0, 0, 0};
        /* colour, as O14 */
        double draw[3];
        for (int c = 0; c < 3; ++c) draw[c] = o.clamp[c] ? 0.0 : d[c];
        double dY[48];
        orc_sh_basis_grad(deg, o.dir[0], o.dir[1], o.dir[2], dY);
        double ddir[3] = {0, 0, 0};
        for (int k = 0; k < K; ++k)
            for (int c = 0; c < 3; ++c) {
                dsh[(size_t)3 * sh_rows * g + 3 * k + c] += o.Y[k] * draw[c];
                for (int j = 0; j < 3; ++j) ddir[j] += shg[3 * k + c] * dY[3 * k + j] * draw[c];
            }
        double dd = o.dir[0] * ddir[0] + o.dir[1] * ddir[1] + o.dir[2] * ddir[2];
        for (int j = 0; j < 3; ++j) dmu[j] += (ddir[j] - o.dir[j] * dd) / o.dist;
        /* S3: M = K [a | b | X], so the columns' gradients are K^T times dM's columns */
        const double Kr[3][3] = {{cam.fx, 0.0, cam.cx}, {0.0, cam.fy, cam.cy}, {0.0, 0.0, 1.0}};
        double da[3], db[3], dX[3];
        for (int k = 0; k < 3; ++k) {
            double sa = 0.0, sb = 0.0, sx = 0.0;
            for (int i = 0; i < 3; ++i) {
                sa += Kr[i][k] * d[4 + 3 * i];
                sb += Kr[i][k] * d[4 + 3 * i + 1];
                sx += Kr[i][k] * d[4 + 3 * i + 2];
            }
            da[k] = sa;
            db[k] = sb;
            dX[k] = sx;
        }
        /* S4 */
        double Z = o.X[2];
        dX[0] += cam.fx / Z * d[13];
        dX[1] += cam.fy / Z * d[14];
        dX[2] += -cam.fx * o.X[0] / (Z * Z) * d[13] - cam.fy * o.X[1] / (Z * Z) * d[14];
        for (int j = 0; j < 3; ++j) dmu[j] += cam.R[j] * dX[0] + cam.R[3 + j] * dX[1] + cam.R[6 + j] * dX[2];
        /* S2: a = s_u R t_u, b = s_v R t_v */
        double dsu = 0.0, dsv = 0.0;
        for (int i = 0; i < 3; ++i) {
            dsu += o.Rtu[i] * da[i];
            dsv += o.Rtv[i] * db[i];
        }
        dscales[2 * g] += dsu;
        dscales[2 * g + 1] += dsv;
        double Rb[9] = {0};  /* dL/dRq: columns 0 and 1 are dL/dt_u, dL/dt_v */
        for (int k = 0; k < 3; ++k) {
            double su = 0.0, sv = 0.0;
            for (int i = 0; i < 3; ++i) {
                su += cam.R[3 * i + k] * da[i];
                sv += cam.R[3 * i + k] * db[i];
            }
            Rb[3 * k] = scales[2 * g] * su;
            Rb[3 * k + 1] = scales[2 * g + 1] * sv;
        }
        double D[4][9], qb[4];
        drot_dq(o.qn, D);
        for (int k = 0; k < 4; ++k) {
            double s = 0;
            for (int i = 0; i < 9; ++i) s += Rb[i] * D[k][i];
            qb[k] = s;
        }
        double qdot = 0;
        for (int k = 0; k < 4; ++k) qdot += o.qn[k] * qb[k];
        for (int k = 0; k < 4; ++k) dquats[4 * g + k] += (qb[k] - qdot * o.qn[k]) / o.qnorm;
        dopac[g] += d[3];
        for (int j = 0; j < 3; ++j) dmeans[3 * g + j] += dmu[j];
    }
}
