/*
 * gs_oracle.c -- CPU oracle for one training iteration of tile-based differentiable
 * 3D Gaussian splatting.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
 * baseline load this library.  It shares no code, header, table or constant with the HIP
 * library: it is a plain, slow, double-precision definition of what the HIP path computes,
 * written so that it can be checked against the mathematics by eye.
 *
 * The pages (ByteSplat arXiv 2610.02851; Grendel arXiv 2406.18533; GS-Scale arXiv
 * 2509.15645; Splaxel arXiv 2606.18588) describe the systems built around this
 * computation, not its formulas: none of them spells out the projection, compositing or
 * backward equations.  Every formula below is therefore the plainest reading of standard
 * EWA splatting with front-to-back alpha compositing, and each open constant (near plane,
 * low-pass dilation, alpha bounds, transmittance cut-off) arrives as a parameter.
 *
 * Parity status of each function:
 *   orc_sh_basis        pinned: scipy complex spherical harmonics converted to real form;
 *                       orthonormality by quadrature.
 *   orc_project         pinned: closed forms for on-axis and off-axis isotropic Gaussians,
 *                       quaternion axis test, camera-frame equivalence, box brute force.
 *   orc_raster_forward  pinned: single-Gaussian profile, telescoping identities,
 *                       two-Gaussian closed form, brute-force all-Gaussians-per-pixel.
 *   orc_raster_backward pinned: central finite differences of the loss, two-Gaussian and
 *                       single-Gaussian closed-form derivatives.
 *   orc_sh_basis_grad   pinned: central finite differences of orc_sh_basis.
 *   orc_project_f64     the same per-Gaussian function as orc_project (double inputs).
 *   orc_project_backward pinned: central finite differences of orc_project_f64 for every
 *                       parameter component (posed cameras, fx != fy, SH degree 3);
 *                       rotation invariance of isotropic Gaussians; quaternion-norm
 *                       invariance; closed forms of the colour and opacity terms.
 *   The constants themselves (0.2, 0.3, 1/255, 0.99, 1e-4, 60 degree FOV) are readings that
 *   no page fixes: parity unpinned for their values.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC gs_oracle.c -lm
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t width, height;
    double fx, fy, cx, cy;
    double R[9];      /* world -> camera rotation, row-major */
    double t[3];      /* world -> camera translation */
    double campos[3]; /* camera centre, world coordinates */
} orc_camera;

typedef struct {
    double znear;     /* Gaussians with camera z <= znear are dropped */
    double eps2d;     /* low-pass dilation added to the 2D covariance diagonal, px^2 */
    double alpha_min; /* pairs with alpha below this are skipped */
    double alpha_max; /* alpha is clamped to this */
    double t_min;     /* a pixel stops before the blend that would take T below this */
    double bg[3];     /* background colour */
    int32_t sh_degree;
    int32_t tile;     /* tile side in pixels */
} orc_params;

/* Unit roundoff of IEEE binary32, used only by the decision-margin model. */
#define EPS32 5.9604644775390625e-08

/* ------------------------------------------------------------------------------------- */
/* Real orthonormal spherical harmonics, degree 0..3, index l*l + l + m, at unit vector d. */
/* Cartesian forms of the textbook real basis (no Condon-Shortley phase).                 */
/* ------------------------------------------------------------------------------------- */
void orc_sh_basis(int degree, const double d[3], double* Y)
{
    const double x = d[0], y = d[1], z = d[2];
    const double pi = 3.14159265358979323846;
    Y[0] = 0.5 * sqrt(1.0 / pi);
    if (degree < 1) return;
    Y[1] = sqrt(3.0 / (4.0 * pi)) * y;
    Y[2] = sqrt(3.0 / (4.0 * pi)) * z;
    Y[3] = sqrt(3.0 / (4.0 * pi)) * x;
    if (degree < 2) return;
    Y[4] = 0.5 * sqrt(15.0 / pi) * x * y;
    Y[5] = 0.5 * sqrt(15.0 / pi) * y * z;
    Y[6] = 0.25 * sqrt(5.0 / pi) * (3.0 * z * z - 1.0);
    Y[7] = 0.5 * sqrt(15.0 / pi) * x * z;
    Y[8] = 0.25 * sqrt(15.0 / pi) * (x * x - y * y);
    if (degree < 3) return;
    Y[9] = 0.25 * sqrt(35.0 / (2.0 * pi)) * y * (3.0 * x * x - y * y);
    Y[10] = 0.5 * sqrt(105.0 / pi) * x * y * z;
    Y[11] = 0.25 * sqrt(21.0 / (2.0 * pi)) * y * (5.0 * z * z - 1.0);
    Y[12] = 0.25 * sqrt(7.0 / pi) * z * (5.0 * z * z - 3.0);
    Y[13] = 0.25 * sqrt(21.0 / (2.0 * pi)) * x * (5.0 * z * z - 1.0);
    Y[14] = 0.25 * sqrt(105.0 / pi) * z * (x * x - y * y);
    Y[15] = 0.25 * sqrt(35.0 / (2.0 * pi)) * x * (x * x - 3.0 * y * y);
}

/* Cartesian gradient dY[k][0..2] = dY_k/d(x, y, z) of the basis polynomials above, at d.  The
 * polynomials are differentiated as functions on R^3; a caller on the sphere projects out the
 * radial part. */
void orc_sh_basis_grad(int degree, const double d[3], double* dY)
{
    const double x = d[0], y = d[1], z = d[2];
    const double pi = 3.14159265358979323846;
    for (int k = 0; k < 48; k++) dY[k] = 0.0;
    if (degree < 1) return;
    const double c1 = sqrt(3.0 / (4.0 * pi));
    dY[3 * 1 + 1] = c1;                                   /* c1 y */
    dY[3 * 2 + 2] = c1;                                   /* c1 z */
    dY[3 * 3 + 0] = c1;                                   /* c1 x */
    if (degree < 2) return;
    const double c2 = 0.5 * sqrt(15.0 / pi), c3 = 0.25 * sqrt(5.0 / pi), c4 = 0.25 * sqrt(15.0 / pi);
    dY[3 * 4 + 0] = c2 * y;                               /* c2 x y */
    dY[3 * 4 + 1] = c2 * x;
    dY[3 * 5 + 1] = c2 * z;                               /* c2 y z */
    dY[3 * 5 + 2] = c2 * y;
    dY[3 * 6 + 2] = 6.0 * c3 * z;                         /* c3 (3 z^2 - 1) */
    dY[3 * 7 + 0] = c2 * z;                               /* c2 x z */
    dY[3 * 7 + 2] = c2 * x;
    dY[3 * 8 + 0] = 2.0 * c4 * x;                         /* c4 (x^2 - y^2) */
    dY[3 * 8 + 1] = -2.0 * c4 * y;
    if (degree < 3) return;
    const double c5 = 0.25 * sqrt(35.0 / (2.0 * pi)), c6 = 0.5 * sqrt(105.0 / pi);
    const double c7 = 0.25 * sqrt(21.0 / (2.0 * pi)), c8 = 0.25 * sqrt(7.0 / pi);
    const double c9 = 0.25 * sqrt(105.0 / pi);
    dY[3 * 9 + 0] = 6.0 * c5 * x * y;                     /* c5 y (3 x^2 - y^2) */
    dY[3 * 9 + 1] = c5 * (3.0 * x * x - 3.0 * y * y);
    dY[3 * 10 + 0] = c6 * y * z;                          /* c6 x y z */
    dY[3 * 10 + 1] = c6 * x * z;
    dY[3 * 10 + 2] = c6 * x * y;
    dY[3 * 11 + 1] = c7 * (5.0 * z * z - 1.0);            /* c7 y (5 z^2 - 1) */
    dY[3 * 11 + 2] = 10.0 * c7 * y * z;
    dY[3 * 12 + 2] = c8 * (15.0 * z * z - 3.0);           /* c8 z (5 z^2 - 3) */
    dY[3 * 13 + 0] = c7 * (5.0 * z * z - 1.0);            /* c7 x (5 z^2 - 1) */
    dY[3 * 13 + 2] = 10.0 * c7 * x * z;
    dY[3 * 14 + 0] = 2.0 * c9 * x * z;                    /* c9 z (x^2 - y^2) */
    dY[3 * 14 + 1] = -2.0 * c9 * y * z;
    dY[3 * 14 + 2] = c9 * (x * x - y * y);
    dY[3 * 15 + 0] = c5 * (3.0 * x * x - 3.0 * y * y);    /* c5 x (x^2 - 3 y^2) */
    dY[3 * 15 + 1] = -6.0 * c5 * x * y;
}

/* Rotation matrix (row-major) of the unit quaternion (w, x, y, z). */
static void quat_to_matrix(const double q[4], double M[9])
{
    const double w = q[0], x = q[1], y = q[2], z = q[3];
    M[0] = 1.0 - 2.0 * (y * y + z * z);
    M[1] = 2.0 * (x * y - w * z);
    M[2] = 2.0 * (x * z + w * y);
    M[3] = 2.0 * (x * y + w * z);
    M[4] = 1.0 - 2.0 * (x * x + z * z);
    M[5] = 2.0 * (y * z - w * x);
    M[6] = 2.0 * (x * z - w * y);
    M[7] = 2.0 * (y * z + w * x);
    M[8] = 1.0 - 2.0 * (x * x + y * y);
}

/* Distance from v to the nearest integer. */
static double frac_dist(double v)
{
    return fabs(v - nearbyint(v));
}

/*
 * Projection of one Gaussian into one view, in double precision.
 *   mu[3], ls[3] (log-scales), q[4] (w,x,y,z, any norm), logit, shc[k*3 + ch] (k < (deg+1)^2).
 * Outputs (index i of the per-Gaussian arrays): see orc_project.  Returns visibility.
 */
static int project_one(const double mu[3], const double ls[3], const double q_in[4], double logit,
                       const double* shc, const orc_camera* cam, const orc_params* p, int64_t i,
                       double* mean2d, double* cov2d, double* conic, double* opacity, double* color,
                       double* depth, int32_t* rect, int32_t* n_tiles, int8_t* flag)
{
    const int deg = p->sh_degree;
    const int nk = (deg + 1) * (deg + 1);
    flag[i] = 0;
    n_tiles[i] = 0;
    rect[4 * i + 0] = rect[4 * i + 1] = rect[4 * i + 2] = rect[4 * i + 3] = 0;
    mean2d[2 * i] = mean2d[2 * i + 1] = 0.0;
    cov2d[3 * i] = cov2d[3 * i + 1] = cov2d[3 * i + 2] = 0.0;
    conic[3 * i] = conic[3 * i + 1] = conic[3 * i + 2] = 0.0;
    opacity[i] = 0.0;
    color[3 * i] = color[3 * i + 1] = color[3 * i + 2] = 0.0;
    depth[i] = 0.0;

    double q[4];
    int finite = isfinite(logit);
    for (int k = 0; k < 3; k++) finite = finite && isfinite(mu[k]) && isfinite(ls[k]);
    for (int k = 0; k < 4; k++) finite = finite && isfinite(q_in[k]);
    if (!finite) return 0;

    /* 1. activations */
    const double o = 1.0 / (1.0 + exp(-logit));
    double s[3];
    for (int k = 0; k < 3; k++) s[k] = exp(ls[k]);
    const double qn = sqrt(q_in[0] * q_in[0] + q_in[1] * q_in[1] + q_in[2] * q_in[2] + q_in[3] * q_in[3]);
    if (!(qn > 0.0)) return 0;
    for (int k = 0; k < 4; k++) q[k] = q_in[k] / qn;

    /* 2. world -> camera, near cull */
    double tc[3];
    for (int r = 0; r < 3; r++)
        tc[r] = cam->R[3 * r + 0] * mu[0] + cam->R[3 * r + 1] * mu[1] + cam->R[3 * r + 2] * mu[2] + cam->t[r];
    if (fabs(tc[2] - p->znear) <= 1e-5 * fmax(1.0, fabs(tc[2]))) flag[i] = 1;
    if (!(tc[2] > p->znear)) return 0;

    /* 3. world covariance Sigma = Rq diag(s^2) Rq^T */
    double Rq[9], Sig[9];
    quat_to_matrix(q, Rq);
    for (int a = 0; a < 3; a++)
        for (int b = 0; b < 3; b++) {
            double acc = 0.0;
            for (int k = 0; k < 3; k++) acc += Rq[3 * a + k] * s[k] * s[k] * Rq[3 * b + k];
            Sig[3 * a + b] = acc;
        }

    /* 4. EWA: Sigma2D = J W Sigma W^T J^T, plus the low-pass dilation */
    const double tz = tc[2];
    double J[6] = {cam->fx / tz, 0.0, -cam->fx * tc[0] / (tz * tz),
                   0.0, cam->fy / tz, -cam->fy * tc[1] / (tz * tz)};
    double T[6]; /* T = J W, 2x3 */
    for (int r = 0; r < 2; r++)
        for (int c = 0; c < 3; c++) {
            double acc = 0.0;
            for (int k = 0; k < 3; k++) acc += J[3 * r + k] * cam->R[3 * k + c];
            T[3 * r + c] = acc;
        }
    double S2[4]; /* T Sigma T^T, 2x2 */
    for (int r = 0; r < 2; r++)
        for (int c = 0; c < 2; c++) {
            double acc = 0.0;
            for (int a = 0; a < 3; a++)
                for (int b = 0; b < 3; b++) acc += T[3 * r + a] * Sig[3 * a + b] * T[3 * c + b];
            S2[2 * r + c] = acc;
        }
    const double a = S2[0] + p->eps2d;
    const double b = S2[1];
    const double c = S2[3] + p->eps2d;
    const double det = a * c - b * b;
    if (!(det > 0.0) || !isfinite(det)) return 0;
    const double A = c / det, B = -b / det, C = a / det;

    /* 5. projected centre, pixel (u, v) has its centre at (u + 1/2, v + 1/2) */
    const double mx = cam->fx * tc[0] / tz + cam->cx;
    const double my = cam->fy * tc[1] / tz + cam->cy;

    /* 7. opacity-aware box: all pixels with o * exp(-q/2) >= alpha_min */
    if (fabs(255.0 * o - 1.0) <= 1e-5) flag[i] = 1;
    if (!(o * (1.0 / p->alpha_min) > 1.0)) return 0;
    const double Q = 2.0 * log(o / p->alpha_min);
    const double ex = 1.001 * sqrt(Q * a);
    const double ey = 1.001 * sqrt(Q * c);
    const double lo_x = mx - ex - 0.5, hi_x = mx + ex - 0.5;
    const double lo_y = my - ey - 0.5, hi_y = my + ey - 0.5;
    if (!(isfinite(lo_x) && isfinite(hi_x) && isfinite(lo_y) && isfinite(hi_y))) return 0;
    const double mx_margin = 1e-3 + 4e-6 * (fabs(mx) + ex);
    const double my_margin = 1e-3 + 4e-6 * (fabs(my) + ey);
    if (frac_dist(lo_x) < mx_margin || frac_dist(hi_x) < mx_margin ||
        frac_dist(lo_y) < my_margin || frac_dist(hi_y) < my_margin)
        flag[i] = 1;
    const double u0 = fmax(0.0, ceil(lo_x));
    const double u1 = fmin((double)(cam->width - 1), floor(hi_x));
    const double v0 = fmax(0.0, ceil(lo_y));
    const double v1 = fmin((double)(cam->height - 1), floor(hi_y));
    if (!(u0 <= u1) || !(v0 <= v1)) return 0;

    /* 6. colour from spherical harmonics along the viewing direction; DC taken as the
     *    base colour, lower clamp at zero */
    double dir[3] = {mu[0] - cam->campos[0], mu[1] - cam->campos[1], mu[2] - cam->campos[2]};
    const double dn = sqrt(dir[0] * dir[0] + dir[1] * dir[1] + dir[2] * dir[2]);
    if (!(dn > 0.0)) return 0;
    for (int k = 0; k < 3; k++) dir[k] /= dn;
    double Y[16];
    orc_sh_basis(deg, dir, Y);
    double col[3];
    int col_ok = 1;
    for (int ch = 0; ch < 3; ch++) {
        double v = shc[0 * 3 + ch];
        for (int k = 1; k < nk; k++) v += shc[k * 3 + ch] * Y[k];
        if (!isfinite(v)) col_ok = 0;
        col[ch] = v > 0.0 ? v : 0.0;
    }
    if (!col_ok) return 0;

    /* 8. outputs */
    const int tile = p->tile;
    const int tx0 = (int)u0 / tile, tx1 = (int)u1 / tile;
    const int ty0 = (int)v0 / tile, ty1 = (int)v1 / tile;
    mean2d[2 * i] = mx;
    mean2d[2 * i + 1] = my;
    cov2d[3 * i] = a;
    cov2d[3 * i + 1] = b;
    cov2d[3 * i + 2] = c;
    conic[3 * i] = A;
    conic[3 * i + 1] = B;
    conic[3 * i + 2] = C;
    opacity[i] = o;
    for (int ch = 0; ch < 3; ch++) color[3 * i + ch] = col[ch];
    depth[i] = tz;
    rect[4 * i + 0] = tx0;
    rect[4 * i + 1] = ty0;
    rect[4 * i + 2] = tx1;
    rect[4 * i + 3] = ty1;
    n_tiles[i] = (tx1 - tx0 + 1) * (ty1 - ty0 + 1);
    return 1;
}

/*
 * Projection of every Gaussian into one view (no compaction; the caller compacts).
 *
 * Inputs are the float32 parameter arrays in structure-of-arrays layout:
 *   means[3][n], log_scales[3][n], quats[4][n] (w,x,y,z), opacity_logits[n],
 *   sh[3*(deg+1)^2][n] with row k*3 + channel.
 * Outputs per Gaussian i (double unless stated):
 *   visible[i] (0/1), mean2d[i][2] (pixels), cov2d[i][3] = dilated 2D covariance (xx, xy, yy),
 *   conic[i][3] = (A, B, C) with q = A dx^2 + 2 B dx dy + C dy^2, opacity[i], color[i][3],
 *   depth[i] = camera-space z, rect[i][4] = (tx0, ty0, tx1, ty1) inclusive tile rectangle
 *   (int32), n_tiles[i] (int32), flag[i] = 1 when a visibility or box decision lies so close
 *   to its threshold that float32 arithmetic may decide it the other way.
 */
void orc_project(int64_t n, const float* means, const float* log_scales, const float* quats,
                 const float* opacity_logits, const float* sh, const orc_camera* cam,
                 const orc_params* p, int8_t* visible, double* mean2d, double* cov2d,
                 double* conic, double* opacity, double* color, double* depth, int32_t* rect,
                 int32_t* n_tiles, int8_t* flag)
{
    const int nk = (p->sh_degree + 1) * (p->sh_degree + 1);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double mu[3], ls[3], q[4], shc[48];
        for (int k = 0; k < 3; k++) mu[k] = means[k * n + i];
        for (int k = 0; k < 3; k++) ls[k] = log_scales[k * n + i];
        for (int k = 0; k < 4; k++) q[k] = quats[k * n + i];
        for (int k = 0; k < 3 * nk; k++) shc[k] = sh[k * n + i];
        visible[i] = (int8_t)project_one(mu, ls, q, opacity_logits[i], shc, cam, p, i, mean2d, cov2d, conic,
                                         opacity, color, depth, rect, n_tiles, flag);
    }
}

/* The same projection with double-precision parameters (used to differentiate it numerically). */
void orc_project_f64(int64_t n, const double* means, const double* log_scales, const double* quats,
                     const double* opacity_logits, const double* sh, const orc_camera* cam,
                     const orc_params* p, int8_t* visible, double* mean2d, double* cov2d,
                     double* conic, double* opacity, double* color, double* depth, int32_t* rect,
                     int32_t* n_tiles, int8_t* flag)
{
    const int nk = (p->sh_degree + 1) * (p->sh_degree + 1);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double mu[3], ls[3], q[4], shc[48];
        for (int k = 0; k < 3; k++) mu[k] = means[k * n + i];
        for (int k = 0; k < 3; k++) ls[k] = log_scales[k * n + i];
        for (int k = 0; k < 4; k++) q[k] = quats[k * n + i];
        for (int k = 0; k < 3 * nk; k++) shc[k] = sh[k * n + i];
        visible[i] = (int8_t)project_one(mu, ls, q, opacity_logits[i], shc, cam, p, i, mean2d, cov2d, conic,
                                         opacity, color, depth, rect, n_tiles, flag);
    }
}

/*
 * Backward of the projection for one view (the chain rule of orc_project, step by step in
 * reverse).  Given dL/dmean2d (n,2), dL/dconic (n,3: A, B, C), dL/dopacity (n) and dL/dcolour
 * (n,3) of the Gaussians with visible[i] = 1 (indexed by Gaussian), it ADDS this view's share
 * of dL/dmeans[3][n], dL/dlog_scales[3][n], dL/dquats[4][n] (with respect to the raw,
 * unnormalised quaternion), dL/dopacity_logits[n] and dL/dsh[3(deg+1)^2][n]; the caller sums
 * views by calling once per view.  The conic, box and culling decisions are taken as fixed
 * (they are piecewise constant).  flag[i] is set when a colour channel's value before the
 * clamp at zero is so close to zero that float32 evaluation may take the clamp the other way.
 */
void orc_project_backward(int64_t n, const double* means, const double* log_scales, const double* quats,
                          const double* opacity_logits, const double* sh, const orc_camera* cam,
                          const orc_params* p, const int8_t* visible, const double* g_mean2d,
                          const double* g_conic, const double* g_opacity, const double* g_color,
                          double* d_means, double* d_log_scales, double* d_quats, double* d_logits,
                          double* d_sh, int8_t* flag)
{
    const int deg = p->sh_degree;
    const int nk = (deg + 1) * (deg + 1);
    const double* W = cam->R;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        if (!visible[i]) continue;
        double mu[3], s[3], qr[4], q[4];
        for (int k = 0; k < 3; k++) mu[k] = means[k * n + i];
        for (int k = 0; k < 3; k++) s[k] = exp(log_scales[k * n + i]);
        for (int k = 0; k < 4; k++) qr[k] = quats[k * n + i];
        const double o = 1.0 / (1.0 + exp(-opacity_logits[i]));
        const double qn = sqrt(qr[0] * qr[0] + qr[1] * qr[1] + qr[2] * qr[2] + qr[3] * qr[3]);
        for (int k = 0; k < 4; k++) q[k] = qr[k] / qn;

        /* forward quantities */
        double tc[3];
        for (int r = 0; r < 3; r++) tc[r] = W[3 * r] * mu[0] + W[3 * r + 1] * mu[1] + W[3 * r + 2] * mu[2] + cam->t[r];
        const double tx = tc[0], ty = tc[1], tz = tc[2];
        const double fx = cam->fx, fy = cam->fy;
        double Rq[9], Sig[9];
        quat_to_matrix(q, Rq);
        for (int a = 0; a < 3; a++)
            for (int b = 0; b < 3; b++) {
                double acc = 0.0;
                for (int k = 0; k < 3; k++) acc += Rq[3 * a + k] * s[k] * s[k] * Rq[3 * b + k];
                Sig[3 * a + b] = acc;
            }
        const double J[6] = {fx / tz, 0.0, -fx * tx / (tz * tz), 0.0, fy / tz, -fy * ty / (tz * tz)};
        double T[6];
        for (int r = 0; r < 2; r++)
            for (int c = 0; c < 3; c++) {
                double acc = 0.0;
                for (int k = 0; k < 3; k++) acc += J[3 * r + k] * W[3 * k + c];
                T[3 * r + c] = acc;
            }
        double S2[4];
        for (int r = 0; r < 2; r++)
            for (int c = 0; c < 2; c++) {
                double acc = 0.0;
                for (int a = 0; a < 3; a++)
                    for (int b = 0; b < 3; b++) acc += T[3 * r + a] * Sig[3 * a + b] * T[3 * c + b];
                S2[2 * r + c] = acc;
            }
        const double a = S2[0] + p->eps2d, b = S2[1], c = S2[3] + p->eps2d;
        const double det = a * c - b * b;
        const double A = c / det, B = -b / det, C = a / det;

        /* conic M = [[A, B], [B, C]] = S^-1 of the dilated covariance S = [[a, b], [b, c]]:
         * dL/dS = -M G M with G = [[gA, gB/2], [gB/2, gC]] (the derivative of the inverse); the
         * off-diagonal b appears twice in S, so its gradient is twice the matrix entry.  The
         * dilation is a constant, so these are also the gradients of Sigma2D's xx, xy, yy. */
        const double gA = g_conic[3 * i], gB = g_conic[3 * i + 1], gC = g_conic[3 * i + 2];
        const double ga = -(A * A * gA + A * B * gB + B * B * gC);
        const double gb = -(2.0 * A * B * gA + (A * C + B * B) * gB + 2.0 * B * C * gC);
        const double gc = -(B * B * gA + B * C * gB + C * C * gC);

        /* Sigma2D = T Sigma T^T with xx = T0 Sig T0^T, xy = T0 Sig T1^T, yy = T1 Sig T1^T (rows
         * T0, T1 of T): gradients of T and of the nine entries of Sigma */
        double gT[6], gSig[9];
        for (int k = 0; k < 3; k++) {
            double st0 = 0.0, st1 = 0.0; /* (Sig T0^T)_k, (Sig T1^T)_k */
            for (int m = 0; m < 3; m++) {
                st0 += Sig[3 * k + m] * T[m];
                st1 += Sig[3 * k + m] * T[3 + m];
            }
            gT[k] = 2.0 * ga * st0 + gb * st1;
            gT[3 + k] = gb * st0 + 2.0 * gc * st1;
        }
        for (int u = 0; u < 3; u++)
            for (int v = 0; v < 3; v++)
                gSig[3 * u + v] = ga * T[u] * T[v] + gb * T[u] * T[3 + v] + gc * T[3 + u] * T[3 + v];

        /* T = J W  ->  J;  J(t) and the projected centre  ->  camera-space t */
        double gJ[6];
        for (int r = 0; r < 2; r++)
            for (int k = 0; k < 3; k++) {
                double acc = 0.0;
                for (int col = 0; col < 3; col++) acc += gT[3 * r + col] * W[3 * k + col];
                gJ[3 * r + k] = acc;
            }
        const double gmx = g_mean2d[2 * i], gmy = g_mean2d[2 * i + 1];
        double gt[3];
        gt[0] = gmx * fx / tz + gJ[2] * (-fx / (tz * tz));
        gt[1] = gmy * fy / tz + gJ[5] * (-fy / (tz * tz));
        gt[2] = -gmx * fx * tx / (tz * tz) - gmy * fy * ty / (tz * tz) + gJ[0] * (-fx / (tz * tz)) +
                gJ[2] * (2.0 * fx * tx / (tz * tz * tz)) + gJ[4] * (-fy / (tz * tz)) +
                gJ[5] * (2.0 * fy * ty / (tz * tz * tz));

        /* t = W mu + t_cam  ->  mu */
        double gmu[3];
        for (int k = 0; k < 3; k++) gmu[k] = W[k] * gt[0] + W[3 + k] * gt[1] + W[6 + k] * gt[2];

        /* Sigma = sum_k s_k^2 Rq[:,k] Rq[:,k]^T  ->  scales (then log-scales) and Rq */
        double gRq[9];
        for (int k = 0; k < 3; k++) {
            double gs = 0.0;
            for (int u = 0; u < 3; u++)
                for (int v = 0; v < 3; v++) gs += gSig[3 * u + v] * 2.0 * s[k] * Rq[3 * u + k] * Rq[3 * v + k];
            d_log_scales[k * n + i] += gs * s[k];
        }
        for (int u = 0; u < 3; u++)
            for (int k = 0; k < 3; k++) {
                double acc = 0.0;
                for (int v = 0; v < 3; v++) acc += (gSig[3 * u + v] + gSig[3 * v + u]) * Rq[3 * v + k];
                gRq[3 * u + k] = acc * s[k] * s[k];
            }

        /* Rq(q) of the unit quaternion (w, x, y, z), entry by entry */
        const double w = q[0], x = q[1], y = q[2], z = q[3];
        double gq[4] = {0.0, 0.0, 0.0, 0.0};
        gq[2] += gRq[0] * (-4.0 * y);
        gq[3] += gRq[0] * (-4.0 * z);
        gq[0] += gRq[1] * (-2.0 * z); gq[1] += gRq[1] * (2.0 * y); gq[2] += gRq[1] * (2.0 * x); gq[3] += gRq[1] * (-2.0 * w);
        gq[0] += gRq[2] * (2.0 * y);  gq[1] += gRq[2] * (2.0 * z); gq[2] += gRq[2] * (2.0 * w); gq[3] += gRq[2] * (2.0 * x);
        gq[0] += gRq[3] * (2.0 * z);  gq[1] += gRq[3] * (2.0 * y); gq[2] += gRq[3] * (2.0 * x); gq[3] += gRq[3] * (2.0 * w);
        gq[1] += gRq[4] * (-4.0 * x);
        gq[3] += gRq[4] * (-4.0 * z);
        gq[0] += gRq[5] * (-2.0 * x); gq[1] += gRq[5] * (-2.0 * w); gq[2] += gRq[5] * (2.0 * z); gq[3] += gRq[5] * (2.0 * y);
        gq[0] += gRq[6] * (-2.0 * y); gq[1] += gRq[6] * (2.0 * z); gq[2] += gRq[6] * (-2.0 * w); gq[3] += gRq[6] * (2.0 * x);
        gq[0] += gRq[7] * (2.0 * x);  gq[1] += gRq[7] * (2.0 * w); gq[2] += gRq[7] * (2.0 * z); gq[3] += gRq[7] * (2.0 * y);
        gq[1] += gRq[8] * (-4.0 * x);
        gq[2] += gRq[8] * (-4.0 * y);
        /* normalisation q = qr / |qr|: remove the radial part, divide by |qr| */
        const double qdot = gq[0] * q[0] + gq[1] * q[1] + gq[2] * q[2] + gq[3] * q[3];
        for (int k = 0; k < 4; k++) d_quats[k * n + i] += (gq[k] - q[k] * qdot) / qn;

        /* opacity = sigmoid(logit) */
        d_logits[i] += g_opacity[i] * o * (1.0 - o);

        /* colour = max(0, k0 + sum_k sh_k Y_k(dir)), dir = unit(mu - campos) */
        double dv[3] = {mu[0] - cam->campos[0], mu[1] - cam->campos[1], mu[2] - cam->campos[2]};
        const double dn = sqrt(dv[0] * dv[0] + dv[1] * dv[1] + dv[2] * dv[2]);
        double dir[3] = {dv[0] / dn, dv[1] / dn, dv[2] / dn};
        double Y[16], dY[48];
        orc_sh_basis(deg, dir, Y);
        orc_sh_basis_grad(deg, dir, dY);
        double gdir[3] = {0.0, 0.0, 0.0};
        for (int ch = 0; ch < 3; ch++) {
            const double* shc = sh + (size_t)ch * n + i; /* row k*3 + ch at shc[k * 3 * n] */
            double v = shc[0], mag = fabs(shc[0]);
            for (int k = 1; k < nk; k++) {
                v += shc[(size_t)k * 3 * n] * Y[k];
                mag += fabs(shc[(size_t)k * 3 * n] * Y[k]);
            }
            if (fabs(v) <= 1e-5 * mag) flag[i] = 1;
            if (!(v > 0.0)) continue;
            const double g = g_color[3 * i + ch];
            d_sh[(size_t)ch * n + i] += g;
            for (int k = 1; k < nk; k++) {
                d_sh[(size_t)(k * 3 + ch) * n + i] += g * Y[k];
                for (int m = 0; m < 3; m++) gdir[m] += g * shc[(size_t)k * 3 * n] * dY[3 * k + m];
            }
        }
        const double gdot = gdir[0] * dir[0] + gdir[1] * dir[1] + gdir[2] * dir[2];
        for (int m = 0; m < 3; m++) gmu[m] += (gdir[m] - dir[m] * gdot) / dn;
        for (int k = 0; k < 3; k++) d_means[k * n + i] += gmu[k];
    }
}

/*
 * Rounding-error model of the projection backward (a tolerance model, not part of the
 * definition).  Each quantity carries a first-order bound e on the error that evaluating the
 * same formulas in float32 (one rounding per operation, exp within a few ulp, inputs exact)
 * can make: e(a +- b) = e(a) + e(b) + u|a +- b|, e(ab) = |a| e(b) + |b| e(a) + u|ab|,
 * e(a / b) = e(a)/|b| + |a| e(b)/b^2 + u|a/b|, e(sqrt a) = e(a)/(2 sqrt a) + u sqrt a, with
 * u = 2^-24 (Higham, Accuracy and Stability of Numerical Algorithms, running error analysis).
 * It follows orc_project_backward step by step and ADDS, per view, the bound of that view's
 * contribution to each output plus the rounding of adding it to the running sum.
 */
typedef struct {
    double v, e;
} ve;

static ve ve_in(double v) { ve r = {v, 0.0}; return r; }
static ve ve_add(ve a, ve b) { ve r = {a.v + b.v, 0.0}; r.e = a.e + b.e + EPS32 * fabs(r.v); return r; }
static ve ve_sub(ve a, ve b) { ve r = {a.v - b.v, 0.0}; r.e = a.e + b.e + EPS32 * fabs(r.v); return r; }
static ve ve_mul(ve a, ve b)
{
    ve r = {a.v * b.v, 0.0};
    r.e = fabs(a.v) * b.e + fabs(b.v) * a.e + EPS32 * fabs(r.v);
    return r;
}
static ve ve_div(ve a, ve b)
{
    ve r = {a.v / b.v, 0.0};
    r.e = a.e / fabs(b.v) + fabs(a.v) * b.e / (b.v * b.v) + EPS32 * fabs(r.v);
    return r;
}
static ve ve_sqrt(ve a) { ve r = {sqrt(a.v), 0.0}; r.e = a.e / (2.0 * r.v) + EPS32 * r.v; return r; }
static ve ve_exp(ve a) { ve r = {exp(a.v), 0.0}; r.e = r.v * (a.e + 4.0 * EPS32); return r; }
static ve ve_k(double k, ve a) { ve r = {k * a.v, fabs(k) * a.e}; return r; } /* k a power of two */
static ve ve_neg(ve a) { ve r = {-a.v, a.e}; return r; }
static ve ve_dot3(const ve* a, const ve* b)
{
    return ve_add(ve_add(ve_mul(a[0], b[0]), ve_mul(a[1], b[1])), ve_mul(a[2], b[2]));
}

void orc_project_backward_errbound(int64_t n, const double* means, const double* log_scales, const double* quats,
                                   const double* opacity_logits, const double* sh, const orc_camera* cam,
                                   const orc_params* p, const int8_t* visible, const double* g_mean2d,
                                   const double* g_conic, const double* g_opacity, const double* g_color,
                                   double* e_means, double* e_log_scales, double* e_quats, double* e_logits,
                                   double* e_sh)
{
    const int deg = p->sh_degree;
    const int nk = (deg + 1) * (deg + 1);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        if (!visible[i]) continue;
        ve mu[3], s[3], q[4], W[9], tvec[3];
        for (int k = 0; k < 3; k++) mu[k] = ve_in(means[k * n + i]);
        for (int k = 0; k < 3; k++) s[k] = ve_exp(ve_in(log_scales[k * n + i]));
        for (int k = 0; k < 9; k++) W[k] = ve_in(cam->R[k]);
        for (int k = 0; k < 3; k++) tvec[k] = ve_in(cam->t[k]);
        const ve one = ve_in(1.0);
        const ve o = ve_div(one, ve_add(one, ve_exp(ve_in(-opacity_logits[i]))));
        ve qr[4];
        for (int k = 0; k < 4; k++) qr[k] = ve_in(quats[k * n + i]);
        ve qq = ve_mul(qr[0], qr[0]);
        for (int k = 1; k < 4; k++) qq = ve_add(qq, ve_mul(qr[k], qr[k]));
        const ve qn = ve_sqrt(qq);
        for (int k = 0; k < 4; k++) q[k] = ve_div(qr[k], qn);

        /* forward quantities */
        ve tc[3];
        for (int r = 0; r < 3; r++) tc[r] = ve_add(ve_dot3(&W[3 * r], mu), tvec[r]);
        const ve fx = ve_in(cam->fx), fy = ve_in(cam->fy);
        const ve w = q[0], x = q[1], y = q[2], z = q[3];
        ve Rq[9];
        Rq[0] = ve_sub(one, ve_k(2.0, ve_add(ve_mul(y, y), ve_mul(z, z))));
        Rq[1] = ve_k(2.0, ve_sub(ve_mul(x, y), ve_mul(w, z)));
        Rq[2] = ve_k(2.0, ve_add(ve_mul(x, z), ve_mul(w, y)));
        Rq[3] = ve_k(2.0, ve_add(ve_mul(x, y), ve_mul(w, z)));
        Rq[4] = ve_sub(one, ve_k(2.0, ve_add(ve_mul(x, x), ve_mul(z, z))));
        Rq[5] = ve_k(2.0, ve_sub(ve_mul(y, z), ve_mul(w, x)));
        Rq[6] = ve_k(2.0, ve_sub(ve_mul(x, z), ve_mul(w, y)));
        Rq[7] = ve_k(2.0, ve_add(ve_mul(y, z), ve_mul(w, x)));
        Rq[8] = ve_sub(one, ve_k(2.0, ve_add(ve_mul(x, x), ve_mul(y, y))));
        ve M[9], Sig[9];
        for (int a = 0; a < 3; a++)
            for (int k = 0; k < 3; k++) M[3 * a + k] = ve_mul(Rq[3 * a + k], s[k]);
        for (int a = 0; a < 3; a++)
            for (int b = 0; b < 3; b++) {
                const ve ra[3] = {M[3 * a], M[3 * a + 1], M[3 * a + 2]};
                const ve rb[3] = {M[3 * b], M[3 * b + 1], M[3 * b + 2]};
                Sig[3 * a + b] = ve_dot3(ra, rb);
            }
        const ve iz = ve_div(one, tc[2]);
        const ve iz2 = ve_mul(iz, iz), iz3 = ve_mul(iz2, iz);
        ve J[6] = {ve_mul(fx, iz), ve_in(0.0), ve_neg(ve_mul(ve_mul(fx, tc[0]), iz2)),
                   ve_in(0.0), ve_mul(fy, iz), ve_neg(ve_mul(ve_mul(fy, tc[1]), iz2))};
        ve T[6];
        for (int r = 0; r < 2; r++)
            for (int c = 0; c < 3; c++) {
                const ve col[3] = {W[c], W[3 + c], W[6 + c]};
                T[3 * r + c] = ve_dot3(&J[3 * r], col);
            }
        ve U[3], Vv[3];
        for (int k = 0; k < 3; k++) {
            U[k] = ve_dot3(&Sig[3 * k], &T[0]);
            Vv[k] = ve_dot3(&Sig[3 * k], &T[3]);
        }
        const ve eps = ve_in(p->eps2d);
        const ve a = ve_add(ve_dot3(&T[0], U), eps);
        const ve b = ve_dot3(&T[3], U);
        const ve c = ve_add(ve_dot3(&T[3], Vv), eps);
        const ve det = ve_sub(ve_mul(a, c), ve_mul(b, b));
        const ve idet = ve_div(one, det);
        const ve A = ve_mul(c, idet), B = ve_neg(ve_mul(b, idet)), C = ve_mul(a, idet);

        const ve gA = ve_in(g_conic[3 * i]), gB = ve_in(g_conic[3 * i + 1]), gC = ve_in(g_conic[3 * i + 2]);
        const ve ga = ve_neg(ve_add(ve_add(ve_mul(ve_mul(A, A), gA), ve_mul(ve_mul(A, B), gB)),
                                    ve_mul(ve_mul(B, B), gC)));
        const ve gb = ve_neg(ve_add(ve_add(ve_k(2.0, ve_mul(ve_mul(A, B), gA)),
                                           ve_mul(ve_add(ve_mul(A, C), ve_mul(B, B)), gB)),
                                    ve_k(2.0, ve_mul(ve_mul(B, C), gC))));
        const ve gc = ve_neg(ve_add(ve_add(ve_mul(ve_mul(B, B), gA), ve_mul(ve_mul(B, C), gB)),
                                    ve_mul(ve_mul(C, C), gC)));

        ve gT[6], Gs[9];
        for (int k = 0; k < 3; k++) {
            gT[k] = ve_add(ve_k(2.0, ve_mul(ga, U[k])), ve_mul(gb, Vv[k]));
            gT[3 + k] = ve_add(ve_mul(gb, U[k]), ve_k(2.0, ve_mul(gc, Vv[k])));
        }
        for (int u = 0; u < 3; u++)
            for (int v = 0; v < 3; v++) {
                const ve t1 = ve_k(2.0, ve_mul(ga, ve_mul(T[u], T[v])));
                const ve t2 = ve_mul(gb, ve_add(ve_mul(T[u], T[3 + v]), ve_mul(T[3 + u], T[v])));
                const ve t3 = ve_k(2.0, ve_mul(gc, ve_mul(T[3 + u], T[3 + v])));
                Gs[3 * u + v] = ve_add(ve_add(t1, t2), t3);
            }
        ve gJ[6];
        for (int r = 0; r < 2; r++)
            for (int k = 0; k < 3; k++) gJ[3 * r + k] = ve_dot3(&gT[3 * r], &W[3 * k]);
        const ve gmx = ve_in(g_mean2d[2 * i]), gmy = ve_in(g_mean2d[2 * i + 1]);
        ve gt[3];
        gt[0] = ve_sub(ve_mul(ve_mul(gmx, fx), iz), ve_mul(ve_mul(gJ[2], fx), iz2));
        gt[1] = ve_sub(ve_mul(ve_mul(gmy, fy), iz), ve_mul(ve_mul(gJ[5], fy), iz2));
        {
            const ve t1 = ve_mul(ve_mul(ve_mul(gmx, fx), tc[0]), iz2);
            const ve t2 = ve_mul(ve_mul(ve_mul(gmy, fy), tc[1]), iz2);
            const ve t3 = ve_mul(ve_mul(gJ[0], fx), iz2);
            const ve t4 = ve_k(2.0, ve_mul(ve_mul(ve_mul(gJ[2], fx), tc[0]), iz3));
            const ve t5 = ve_mul(ve_mul(gJ[4], fy), iz2);
            const ve t6 = ve_k(2.0, ve_mul(ve_mul(ve_mul(gJ[5], fy), tc[1]), iz3));
            gt[2] = ve_add(ve_sub(ve_add(ve_sub(ve_neg(ve_add(t1, t2)), t3), t4), t5), t6);
        }
        ve gmu[3];
        for (int k = 0; k < 3; k++) {
            const ve col[3] = {W[k], W[3 + k], W[6 + k]};
            gmu[k] = ve_dot3(col, gt);
        }

        ve gR[9];
        for (int k = 0; k < 3; k++) {
            const ve r[3] = {Rq[k], Rq[3 + k], Rq[6 + k]};
            ve wv[3];
            for (int u = 0; u < 3; u++) wv[u] = ve_dot3(&Gs[3 * u], r);
            const ve sk2 = ve_mul(s[k], s[k]);
            const ve gls = ve_mul(sk2, ve_dot3(r, wv));
            e_log_scales[k * n + i] += gls.e + EPS32 * fabs(gls.v);
            for (int u = 0; u < 3; u++) gR[3 * u + k] = ve_mul(sk2, wv[u]);
        }
        /* quaternion: each component is a sum of 6-8 terms 2 q_a gR_b (factors 2 and 4 exact) */
        ve gq[4];
        gq[0] = ve_k(2.0, ve_add(ve_add(ve_add(ve_sub(ve_mul(y, gR[2]), ve_mul(z, gR[1])), ve_mul(z, gR[3])),
                                        ve_sub(ve_mul(x, gR[7]), ve_mul(x, gR[5]))), ve_neg(ve_mul(y, gR[6]))));
        gq[1] = ve_k(2.0, ve_add(ve_add(ve_add(ve_mul(y, gR[1]), ve_mul(z, gR[2])), ve_add(ve_mul(y, gR[3]), ve_mul(z, gR[6]))),
                                 ve_sub(ve_sub(ve_mul(w, gR[7]), ve_mul(w, gR[5])),
                                        ve_k(2.0, ve_add(ve_mul(x, gR[4]), ve_mul(x, gR[8]))))));
        gq[2] = ve_k(2.0, ve_add(ve_add(ve_add(ve_mul(x, gR[1]), ve_mul(w, gR[2])), ve_add(ve_mul(x, gR[3]), ve_mul(z, gR[5]))),
                                 ve_sub(ve_sub(ve_mul(z, gR[7]), ve_mul(w, gR[6])),
                                        ve_k(2.0, ve_add(ve_mul(y, gR[0]), ve_mul(y, gR[8]))))));
        gq[3] = ve_k(2.0, ve_add(ve_add(ve_add(ve_mul(x, gR[2]), ve_mul(w, gR[3])), ve_add(ve_mul(y, gR[5]), ve_mul(x, gR[6]))),
                                 ve_sub(ve_sub(ve_mul(y, gR[7]), ve_mul(w, gR[1])),
                                        ve_k(2.0, ve_add(ve_mul(z, gR[0]), ve_mul(z, gR[4]))))));
        ve qd = ve_mul(gq[0], q[0]);
        for (int k = 1; k < 4; k++) qd = ve_add(qd, ve_mul(gq[k], q[k]));
        for (int k = 0; k < 4; k++) {
            const ve d = ve_div(ve_sub(gq[k], ve_mul(q[k], qd)), qn);
            e_quats[k * n + i] += d.e + EPS32 * fabs(d.v);
        }
        const ve glog = ve_mul(ve_mul(ve_in(g_opacity[i]), o), ve_sub(one, o));
        e_logits[i] += glog.e + EPS32 * fabs(glog.v);

        /* colour */
        const ve cp[3] = {ve_in(cam->campos[0]), ve_in(cam->campos[1]), ve_in(cam->campos[2])};
        ve dv[3];
        for (int k = 0; k < 3; k++) dv[k] = ve_sub(mu[k], cp[k]);
        const ve dn = ve_sqrt(ve_dot3(dv, dv));
        const ve idn = ve_div(one, dn);
        ve dir[3];
        for (int k = 0; k < 3; k++) dir[k] = ve_mul(dv[k], idn);
        double dirv[3] = {dir[0].v, dir[1].v, dir[2].v};
        double Y[16], dY[48];
        orc_sh_basis(deg, dirv, Y);
        orc_sh_basis_grad(deg, dirv, dY);
        /* basis values: polynomials of degree <= 3 in dir; bound their error by the direction's
         * error times the basis gradient plus a few roundings of the value */
        const double edir = fmax(dir[0].e, fmax(dir[1].e, dir[2].e));
        ve gdir[3] = {ve_in(0.0), ve_in(0.0), ve_in(0.0)};
        for (int ch = 0; ch < 3; ch++) {
            const double* shc = sh + (size_t)ch * n + i;
            double v = shc[0];
            for (int k = 1; k < nk; k++) v += shc[(size_t)k * 3 * n] * Y[k];
            if (!(v > 0.0)) continue;
            const ve g = ve_in(g_color[3 * i + ch]); /* the DC row's contribution g is exact */
            for (int k = 1; k < nk; k++) {
                const double gy = fabs(dY[3 * k]) + fabs(dY[3 * k + 1]) + fabs(dY[3 * k + 2]);
                const ve Yk = {Y[k], gy * edir + 8.0 * EPS32 * (fabs(Y[k]) + gy)};
                const ve t = ve_mul(g, Yk);
                e_sh[(size_t)(k * 3 + ch) * n + i] += t.e + EPS32 * fabs(t.v);
                const ve e = ve_mul(g, ve_in(shc[(size_t)k * 3 * n]));
                for (int m = 0; m < 3; m++) {
                    const ve dYm = {dY[3 * k + m], 8.0 * EPS32 * (fabs(dY[3 * k + m]) + gy) + 6.0 * gy * edir};
                    gdir[m] = ve_add(gdir[m], ve_mul(e, dYm));
                }
            }
        }
        const ve gdot = ve_dot3(gdir, dir);
        for (int m = 0; m < 3; m++) gmu[m] = ve_add(gmu[m], ve_mul(ve_sub(gdir[m], ve_mul(dir[m], gdot)), idn));
        for (int k = 0; k < 3; k++) e_means[k * n + i] += gmu[k].e + EPS32 * fabs(gmu[k].v);
    }
}

/* ------------------------------------------------------------------------------------- */
/* Rasterization                                                                          */
/* ------------------------------------------------------------------------------------- */

/* The 2D records the rasterizer reads, indexed by visible slot (double precision). */
typedef struct {
    const double* mean2d;  /* [slots][2] */
    const double* conic;   /* [slots][3] */
    const double* opacity; /* [slots] */
    const double* color;   /* [slots][3] */
} orc_records;

/* One blended entry of a pixel's walk, kept for the backward pass. */
typedef struct {
    int32_t j;        /* position in the tile list */
    int32_t slot;
    double alpha;     /* alpha used for blending */
    double T;         /* transmittance in front of this entry */
    double G;         /* exp(-q/2) */
    double dx, dy;    /* pixel centre minus projected centre */
    int clamped;      /* 1 if o*G exceeded alpha_max */
} orc_blend;

/*
 * Front-to-back compositing of one pixel over its tile list.
 * Writes C[3], returns n_contrib; *T_out = final transmittance.  When log != NULL, the
 * blended entries are appended to log (capacity n).  *flag is set when a decision (alpha
 * against alpha_min, the transmittance cut-off, alpha against alpha_max) lies within the
 * error that float32 evaluation of the same formulas can make, so that float32 code may
 * decide it differently.  Counters: evaluated pairs; n_blend[0] blended pairs and n_blend[1]
 * blended pairs with a clamped alpha.  touch[j] (optional,
 * per list position) marks the evaluated entries whose alpha reaches alpha_min within that
 * error: the entries whose gradient at this pixel a flipped decision can change.
 */
static int composite_pixel(double px, double py, const int32_t* list, int n, const orc_records* r,
                           const orc_params* p, double C[3], double* T_out, orc_blend* log,
                           int* n_log, int* flag, int* flag_clamp, int64_t* n_eval, int64_t* n_blend,
                           double* err_C, int8_t* touch, double* err_T)
{
    double T = 1.0;
    double errT = 0.0;   /* relative error model of T in float32 */
    double eC = 0.0;     /* absolute error model of C (any channel) in float32 */
    int n_contrib = 0;
    C[0] = C[1] = C[2] = 0.0;
    if (n_log) *n_log = 0;
    for (int j = 0; j < n; j++) {
        const int s = list[j];
        const double dx = px - r->mean2d[2 * s];
        const double dy = py - r->mean2d[2 * s + 1];
        const double A = r->conic[3 * s], B = r->conic[3 * s + 1], Cc = r->conic[3 * s + 2];
        const double q = A * dx * dx + 2.0 * B * dx * dy + Cc * dy * dy;
        const double G = exp(-0.5 * q);
        const double o = r->opacity[s];
        const double v = o * G;
        const double alpha = v < p->alpha_max ? v : p->alpha_max;
        if (n_eval) (*n_eval)++;
        /* float32 error model: q carries ~8 ulp of its absolute-term sum; the exponential, and
         * a logarithm of alpha_min / o where the alpha_min test is taken in log space, add up
         * to a few ulp of the exponent (16 ulp of alpha budgeted) */
        const double qabs = fabs(A) * dx * dx + 2.0 * fabs(B * dx * dy) + fabs(Cc) * dy * dy;
        const double rel_a = 0.5 * 8.0 * EPS32 * qabs + 16.0 * EPS32;
        if (fabs(v - p->alpha_min) <= 4.0 * rel_a * p->alpha_min + 1e-12) *flag = 1;
        if (fabs(v - p->alpha_max) <= 4.0 * rel_a * p->alpha_max + 1e-12) *flag_clamp = 1;
        if (touch) touch[j] = (int8_t)(v >= p->alpha_min * (1.0 - 4.0 * rel_a) - 1e-12);
        if (alpha < p->alpha_min) continue;
        const double Tn = T * (1.0 - alpha);
        const double rel_1ma = (alpha * rel_a + EPS32) / (1.0 - alpha);
        const double errTn = errT + rel_1ma + EPS32;
        if (fabs(Tn - p->t_min) <= 4.0 * errTn * p->t_min + 1e-15) *flag = 1;
        if (Tn < p->t_min) break;
        for (int ch = 0; ch < 3; ch++) C[ch] += alpha * T * r->color[3 * s + ch];
        {
            double cmax = fmax(fabs(r->color[3 * s]), fmax(fabs(r->color[3 * s + 1]), fabs(r->color[3 * s + 2])));
            eC += alpha * T * cmax * (rel_a + errT + 3.0 * EPS32) + fabs(C[0] + C[1] + C[2]) * EPS32;
        }
        if (log) {
            orc_blend* e = &log[*n_log];
            e->j = j;
            e->slot = s;
            e->alpha = alpha;
            e->T = T;
            e->G = G;
            e->dx = dx;
            e->dy = dy;
            e->clamped = !(v <= p->alpha_max);
            (*n_log)++;
        }
        if (n_blend) {
            (*n_blend)++;
            if (!(v <= p->alpha_max)) n_blend[1]++;
        }
        T = Tn;
        errT = errTn;
        n_contrib = j + 1;
    }
    for (int ch = 0; ch < 3; ch++) C[ch] += T * p->bg[ch];
    eC += T * fmax(fabs(p->bg[0]), fmax(fabs(p->bg[1]), fabs(p->bg[2]))) * (errT + EPS32);
    if (err_C) *err_C = eC;
    if (err_T) *err_T = errT;
    *T_out = T;
    return n_contrib;
}

/*
 * Forward rasterization of one view.
 * ranges[tile][2] = [start, end) into vals; vals[] = slot of each list entry; tiles are
 * row-major with tiles_x = ceil(W / tile).  Outputs: image[3][H][W], T_final[H][W],
 * n_contrib[H][W], flag[H][W] (decision within float32 reach), err_C[H][W] (float32 error
 * model of the colour, absolute), err_T[H][W] (float32 error model of T_final, relative), counters[3] = {evaluated pairs, blended pairs, blended pairs whose
 * alpha was clamped}.
 */
void orc_raster_forward(int32_t W, int32_t H, const int32_t* ranges, const int32_t* vals,
                        const double* mean2d, const double* conic, const double* opacity,
                        const double* color, const orc_params* p, double* image, double* T_final,
                        int32_t* n_contrib, int8_t* flag, double* err_C, double* err_T, int64_t* counters)
{
    const int tile = p->tile;
    const int tx_n = (W + tile - 1) / tile, ty_n = (H + tile - 1) / tile;
    const orc_records r = {mean2d, conic, opacity, color};
    int64_t tot_eval = 0, tot_blend = 0, tot_clamp = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : tot_eval, tot_blend, tot_clamp)
    for (int t = 0; t < tx_n * ty_n; t++) {
        const int tx = t % tx_n, ty = t / tx_n;
        const int32_t start = ranges[2 * t], end = ranges[2 * t + 1];
        for (int y = ty * tile; y < (ty + 1) * tile && y < H; y++)
            for (int x = tx * tile; x < (tx + 1) * tile && x < W; x++) {
                double C[3], T, eC, eT;
                int f = 0, fc = 0;
                int64_t ne = 0, nb[2] = {0, 0};
                const int nc = composite_pixel(x + 0.5, y + 0.5, vals + start, end - start, &r, p, C, &T,
                                               NULL, NULL, &f, &fc, &ne, nb, &eC, NULL, &eT);
                const int64_t px = (int64_t)y * W + x;
                for (int ch = 0; ch < 3; ch++) image[(int64_t)ch * W * H + px] = C[ch];
                T_final[px] = T;
                n_contrib[px] = nc;
                flag[px] = (int8_t)(f ? 1 : 0);
                err_C[px] = eC;
                err_T[px] = eT;
                tot_eval += ne;
                tot_blend += nb[0];
                tot_clamp += nb[1];
            }
    }
    counters[0] = tot_eval;
    counters[1] = tot_blend;
    counters[2] = tot_clamp;
}

/*
 * Backward rasterization of one view: gradients of L with respect to the per-slot 2D
 * records, given dL/dC (dldc[3][H][W]).  The forward walk of each pixel is recomputed with
 * its blend log, then the log is traversed from the last blended entry to the first:
 *   dL/dc_j     += alpha_j T_j g
 *   dL/dalpha_j  = sum_ch g_ch (T_j (c_j,ch - Bk_ch) - T_final bg_ch / (1 - alpha_j))
 *   Bk          <- alpha_j c_j + (1 - alpha_j) Bk           (colour behind entry j)
 * and, unless alpha was clamped (o G > alpha_max),
 *   dL/do       += G dL/dalpha
 *   dL/dmean2d  += o G dL/dalpha (A dx + B dy, B dx + C dy)   with d = pixel - mean2d
 *   dL/dconic   += o G dL/dalpha (-dx^2/2, -dx dy, -dy^2/2).
 * Outputs (double, accumulated over the view's pixels): d_mean2d[slots][2],
 * d_conic[slots][3], d_opacity[slots], d_color[slots][3]; mag[slots][9] = sum of the
 * absolute values of the same contributions; slot_flag[slots] = 1 when the slot was
 * evaluated at a pixel whose decisions (including the clamp) lie within float32 reach.
 * Output arrays must be zeroed by the caller.
 */
void orc_raster_backward(int32_t W, int32_t H, const int32_t* ranges, const int32_t* vals,
                         const double* mean2d, const double* conic, const double* opacity,
                         const double* color, const orc_params* p, const double* dldc,
                         const int8_t* pixel_skip, double* d_mean2d, double* d_conic,
                         double* d_opacity, double* d_color, double* mag, int8_t* slot_flag)
{
    const int tile = p->tile;
    const int tx_n = (W + tile - 1) / tile, ty_n = (H + tile - 1) / tile;
    const orc_records r = {mean2d, conic, opacity, color};
    int max_n = 0;
    for (int t = 0; t < tx_n * ty_n; t++)
        if (ranges[2 * t + 1] - ranges[2 * t] > max_n) max_n = ranges[2 * t + 1] - ranges[2 * t];
#pragma omp parallel
    {
        orc_blend* log = (orc_blend*)malloc(sizeof(orc_blend) * (size_t)(max_n > 0 ? max_n : 1));
        int8_t* touch = (int8_t*)calloc((size_t)(max_n > 0 ? max_n : 1), 1);
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < tx_n * ty_n; t++) {
            const int tx = t % tx_n, ty = t / tx_n;
            const int32_t start = ranges[2 * t], end = ranges[2 * t + 1];
            const int32_t* list = vals + start;
            for (int y = ty * tile; y < (ty + 1) * tile && y < H; y++)
                for (int x = tx * tile; x < (tx + 1) * tile && x < W; x++) {
                    const int64_t px = (int64_t)y * W + x;
                    double C[3], T_fin;
                    int f = 0, fc = 0, nl = 0;
                    int64_t n_evaluated = 0;
                    composite_pixel(x + 0.5, y + 0.5, list, end - start, &r, p, C, &T_fin, log, &nl, &f, &fc,
                                    &n_evaluated, NULL, NULL, touch, NULL);
                    if (f || fc || (pixel_skip && pixel_skip[px])) {
                        /* the slots this pixel blends, or could blend under float32 decisions */
                        for (int j = 0; j < (int)n_evaluated; j++)
                            if (touch[j]) {
#pragma omp atomic write
                                slot_flag[list[j]] = 1;
                            }
                    }
                    double g[3];
                    for (int ch = 0; ch < 3; ch++) g[ch] = dldc[(int64_t)ch * W * H + px];
                    double Bk[3] = {0.0, 0.0, 0.0};
                    for (int e = nl - 1; e >= 0; e--) {
                        const orc_blend* b = &log[e];
                        const int s = b->slot;
                        const double* c = &color[3 * s];
                        double dL_dalpha = 0.0;
                        for (int ch = 0; ch < 3; ch++) {
                            const double dc = b->alpha * b->T * g[ch];
#pragma omp atomic
                            d_color[3 * s + ch] += dc;
#pragma omp atomic
                            mag[9 * s + 6 + ch] += fabs(dc);
                            dL_dalpha += g[ch] * (b->T * (c[ch] - Bk[ch]) - T_fin * p->bg[ch] / (1.0 - b->alpha));
                        }
                        for (int ch = 0; ch < 3; ch++) Bk[ch] = b->alpha * c[ch] + (1.0 - b->alpha) * Bk[ch];
                        if (b->clamped) continue;
                        const double o = opacity[s];
                        const double A = conic[3 * s], B = conic[3 * s + 1], Cc = conic[3 * s + 2];
                        const double gh = o * b->G * dL_dalpha; /* dL/dalpha * dalpha/dG * G */
                        const double v[6] = {
                            gh * (A * b->dx + B * b->dy),       /* d mean2d x */
                            gh * (B * b->dx + Cc * b->dy),      /* d mean2d y */
                            -0.5 * gh * b->dx * b->dx,          /* d A */
                            -gh * b->dx * b->dy,                /* d B */
                            -0.5 * gh * b->dy * b->dy,          /* d C */
                            b->G * dL_dalpha};                  /* d opacity */
#pragma omp atomic
                        d_mean2d[2 * s] += v[0];
#pragma omp atomic
                        d_mean2d[2 * s + 1] += v[1];
#pragma omp atomic
                        d_conic[3 * s] += v[2];
#pragma omp atomic
                        d_conic[3 * s + 1] += v[3];
#pragma omp atomic
                        d_conic[3 * s + 2] += v[4];
#pragma omp atomic
                        d_opacity[s] += v[5];
                        for (int k = 0; k < 6; k++) {
#pragma omp atomic
                            mag[9 * s + k] += fabs(v[k]);
                        }
                    }
                }
        }
        free(log);
        free(touch);
    }
}

/*
 * Per-pixel brute force (no tiles): composite every slot in the given global order
 * (the caller passes slots sorted by depth, then slot).  Used only to pin the tiled path.
 */
void orc_raster_bruteforce(int32_t W, int32_t H, const int32_t* order, int32_t n, const double* mean2d,
                           const double* conic, const double* opacity, const double* color,
                           const orc_params* p, double* image, double* T_final, int32_t* n_contrib)
{
    const orc_records r = {mean2d, conic, opacity, color};
#pragma omp parallel for schedule(dynamic, 4)
    for (int y = 0; y < H; y++)
        for (int x = 0; x < W; x++) {
            double C[3], T;
            int f = 0, fc = 0;
            const int nc = composite_pixel(x + 0.5, y + 0.5, order, n, &r, p, C, &T, NULL, NULL, &f, &fc, NULL,
                                           NULL, NULL, NULL, NULL);
            const int64_t px = (int64_t)y * W + x;
            for (int ch = 0; ch < 3; ch++) image[(int64_t)ch * W * H + px] = C[ch];
            T_final[px] = T;
            n_contrib[px] = nc; /* position in the global order, not in a tile list */
        }
}

/* Threads the parallel loops above use (for reporting the CPU baseline). */
int orc_num_threads(void)
{
    return omp_get_max_threads();
}
