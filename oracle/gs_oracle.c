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

/* Guard band of the frustum cull: the projected centre may lie this fraction of the image size
 * beyond each image edge. */
#define GUARD 0.15

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

    /* 5b. per-view frustum cull with a guard band: the projected centre must lie inside the
     *     image widened by 15 % of its size on every side (1.3 times its half extents) */
    {
        const double gx = GUARD * cam->width, gy = GUARD * cam->height;
        const double mgx = 1e-3 + 4e-6 * fabs(mx), mgy = 1e-3 + 4e-6 * fabs(my);
        if (fabs(mx + gx) < mgx || fabs(mx - cam->width - gx) < mgx || fabs(my + gy) < mgy ||
            fabs(my - cam->height - gy) < mgy)
            flag[i] = 1;
        if (!(mx >= -gx && mx <= cam->width + gx && my >= -gy && my <= cam->height + gy)) return 0;
    }

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
        /* finite here but past float32's range (about 3.4e38): a float32 evaluation overflows */
        else if (fabs(v) > 1e38) flag[i] = 1;
        col[ch] = v > 0.0 ? v : 0.0;
    }
    /* no finite colour: the Gaussian stays in the view, transparent (opacity 0, colour 0) */
    double o_view = o;
    if (!col_ok) {
        o_view = 0.0;
        col[0] = col[1] = col[2] = 0.0;
    }

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
    opacity[i] = o_view;
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
 *   to its threshold that float32 arithmetic may decide it the other way (or a colour channel is
 *   finite but past float32's range).  The colour never decides visibility: where it is not
 *   finite the Gaussian is visible and transparent (opacity[i] = 0, colour 0).
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
            /* clamped at zero; or not finite, where the view holds the Gaussian transparent and
             * its 2D gradients are zero */
            if (!(v > 0.0) || !isfinite(v)) continue;
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

/*
 * Float32 error model of the compositing: a tolerance model for comparisons, not part of
 * the definition.  u = 2^-24 is the rounding of one correctly rounded float32 operation; a
 * hardware exponential, logarithm or reciprocal is taken as faithful (within one ulp: 2u).
 *
 * pair_alpha_error bounds the relative error of v = o exp(-q/2), evaluated in float32 from the
 * float32 records, for either of two evaluation orders:
 *   (a) the definition's: q = A dx^2 + 2B dx dy + C dy^2 term by term, exp(-q/2), times o.
 *       Each term carries four roundings (dx twice, two products) and the two additions one
 *       rounding of at most qabs = |A| dx^2 + 2|B dx dy| + |C| dy^2 each, so |dq| <= 6u qabs
 *       and rel(v) <= 3u qabs + 2u (exp) + u (times o).
 *   (b) base 2: p = a dx^2 + b dx dy + c dy^2 + log2 o with a = -log2(e) A / 2 (and b, c)
 *       rounded from a rounded constant, the terms and log2 o added by three fused
 *       multiply-adds, then v = exp2(p).  Each term carries five roundings (the constant, the
 *       scaled coefficient, dx twice, one product), each fused add one rounding of at most
 *       log2(e) qabs / 2 + |log2 o|, log2 o one ulp; so |dp| <= 8u log2(e) qabs / 2 +
 *       5u |log2 o| and rel(v) <= ln(2) |dp| + 2u = 4u qabs + 5u |ln o| + 2u.
 * The bound u (4 qabs + 5 |ln o| + 3) covers both.  A threshold compared in base-2 logarithm
 * units carries its own logarithm's ulp: 2u |ln alpha_min| more for the alpha_min test.
 *
 * Transmittance: 1 - alpha has relative error alpha rel(v) / (1 - alpha) + u, the product one
 * rounding more; so the relative error of T grows by alpha rel / (1 - alpha) + 2u per blend.
 * Colour (per channel): alpha T c has relative error rel + err(T) + 2u, and the running sum one
 * rounding of |C|; the background adds T bg with err(T) + u and one rounding.
 *
 * A decision whose fp64 margin is within these bounds is "flagged": float32 code may take it
 * the other way.  Flagged decisions are resolved, not skipped: the comparisons evaluate the
 * pixel under every combination of its flagged decisions taken the other way (up to
 * KMAX_DEC of them; a pixel with more is "unresolved" and left out).
 */
#define KMAX_DEC 3

static double pair_alpha_error(double qabs, double o)
{
    return EPS32 * (4.0 * qabs + 5.0 * fabs(log(o)) + 3.0);
}

/* A decision of a pixel's walk that float32 evaluation could take the other way. */
enum {
    DEC_AMIN = 1,  /* alpha against alpha_min at entry j: blended or skipped */
    DEC_TMIN = 2,  /* T (1 - alpha) against t_min at entry j: blended or stopped */
    DEC_CLAMP = 3  /* o G against alpha_max at entry j: geometry gradient or none */
};
typedef struct {
    int32_t j, kind;
} orc_decision;

/* One blended entry of a pixel's walk, kept for the backward pass. */
typedef struct {
    int32_t j;     /* position in the tile list */
    int32_t slot;
    double alpha;  /* alpha used for blending */
    double T;      /* transmittance in front of this entry */
    double v;      /* o exp(-q/2), before the clamp */
    double rel;    /* float32 error bound of v, relative */
    double dx, dy; /* pixel centre minus projected centre */
    int clamped;   /* no geometry gradient: o G above alpha_max */
} orc_blend;

/* One walk of a pixel over its list: inputs (forced decisions, optional log and touch
 * buffers) and outputs. */
typedef struct {
    const orc_decision* force; /* decisions taken the other way */
    int n_force;
    orc_blend* log;            /* optional, capacity n: the blended entries */
    int8_t* touch;             /* optional, per list position: v reaches alpha_min within the bound */
    double C[3], T;
    double eC[3];              /* float32 error bound of C, absolute, per channel */
    double eT;                 /* float32 error bound of T, relative */
    int n_contrib, n_log;
    orc_decision fwd[KMAX_DEC + 1]; /* flagged alpha_min / t_min decisions (first KMAX_DEC + 1) */
    orc_decision clamp[KMAX_DEC + 1];
    int n_fwd, n_clamp_flag;   /* counts (may exceed the stored) */
    int64_t n_eval, n_blend, n_clamped;
    int64_t n_box;             /* evaluated entries whose exact alpha_min box holds the pixel */
} orc_walk;

static void walk_init(orc_walk* w, const orc_decision* force, int n_force, orc_blend* log, int8_t* touch)
{
    memset(w, 0, sizeof(*w));
    w->force = force;
    w->n_force = n_force;
    w->log = log;
    w->touch = touch;
}

static int is_forced(const orc_walk* w, int32_t j, int32_t kind)
{
    for (int k = 0; k < w->n_force; k++)
        if (w->force[k].j == j && w->force[k].kind == kind) return 1;
    return 0;
}

static void note_decision(orc_walk* w, int32_t j, int32_t kind)
{
    orc_decision d = {j, kind};
    if (kind == DEC_CLAMP) {
        if (w->n_clamp_flag <= KMAX_DEC) w->clamp[w->n_clamp_flag] = d;
        w->n_clamp_flag++;
    } else {
        if (w->n_fwd <= KMAX_DEC) w->fwd[w->n_fwd] = d;
        w->n_fwd++;
    }
}

/*
 * Front-to-back compositing of one pixel (centre (px, py)) over its tile list:
 *   alpha = min(alpha_max, o exp(-q/2)), q = A dx^2 + 2B dx dy + C dy^2, d = centre - mean2d;
 *   entries with alpha < alpha_min are skipped; the walk stops before the blend that would
 *   take T below t_min (that entry is not blended); C += alpha T c; T *= 1 - alpha;
 *   finally C += T bg.
 * Decisions listed in w->force are taken the other way.
 */
static void composite_walk(double px, double py, const int32_t* list, int n, const orc_records* r,
                           const orc_params* p, orc_walk* w)
{
    const double u = EPS32;
    const double thr = 2.0 * u * fabs(log(p->alpha_min));
    double T = 1.0, errT = 0.0;
    for (int j = 0; j < n; j++) {
        const int s = list[j];
        const double dx = px - r->mean2d[2 * s];
        const double dy = py - r->mean2d[2 * s + 1];
        const double A = r->conic[3 * s], B = r->conic[3 * s + 1], Cc = r->conic[3 * s + 2];
        const double q = A * dx * dx + 2.0 * B * dx * dy + Cc * dy * dy;
        const double qabs = fabs(A) * dx * dx + 2.0 * fabs(B * dx * dy) + fabs(Cc) * dy * dy;
        const double o = r->opacity[s];
        const double v = o * exp(-0.5 * q);
        const double rel = pair_alpha_error(qabs, o);
        w->n_eval++;
        {
            /* the exact box of {o exp(-q/2) >= alpha_min}: half extents sqrt(Q Sxx), sqrt(Q Syy)
             * with Sxx = C / (AC - B^2), Syy = A / (AC - B^2) the dilated covariance's diagonal */
            const double dc = A * Cc - B * B;
            const double Q = 2.0 * log(o / p->alpha_min);
            if (Q >= 0.0 && dc > 0.0 && dx * dx <= Q * Cc / dc && dy * dy <= Q * A / dc) w->n_box++;
        }
        int pass = v >= p->alpha_min;
        if (fabs(v - p->alpha_min) <= (rel + thr) * p->alpha_min) note_decision(w, j, DEC_AMIN);
        if (w->touch) w->touch[j] = (int8_t)(v >= p->alpha_min * (1.0 - rel - thr));
        if (is_forced(w, j, DEC_AMIN)) pass = !pass;
        if (!pass) continue;
        const double alpha = v < p->alpha_max ? v : p->alpha_max;
        int clamped = !(v <= p->alpha_max);
        if (fabs(v - p->alpha_max) <= rel * p->alpha_max) note_decision(w, j, DEC_CLAMP);
        if (is_forced(w, j, DEC_CLAMP)) clamped = !clamped;
        const double Tn = T * (1.0 - alpha);
        const double errTn = errT + alpha * rel / (1.0 - alpha) + 2.0 * u;
        int stop = Tn < p->t_min;
        if (fabs(Tn - p->t_min) <= errTn * Tn) note_decision(w, j, DEC_TMIN);
        if (is_forced(w, j, DEC_TMIN)) stop = !stop;
        if (stop) break;
        for (int ch = 0; ch < 3; ch++) {
            const double c = r->color[3 * s + ch];
            w->C[ch] += alpha * T * c;
            w->eC[ch] += alpha * T * fabs(c) * (rel + errT + 2.0 * u) + u * fabs(w->C[ch]);
        }
        if (w->log) {
            orc_blend* e = &w->log[w->n_log];
            e->j = j;
            e->slot = s;
            e->alpha = alpha;
            e->T = T;
            e->v = v;
            e->rel = rel;
            e->dx = dx;
            e->dy = dy;
            e->clamped = clamped;
            w->n_log++;
        }
        w->n_blend++;
        w->n_clamped += clamped;
        T = Tn;
        errT = errTn;
        w->n_contrib = j + 1;
    }
    for (int ch = 0; ch < 3; ch++) {
        w->C[ch] += T * p->bg[ch];
        w->eC[ch] += T * fabs(p->bg[ch]) * (errT + u) + u * fabs(w->C[ch]);
    }
    w->T = T;
    w->eT = errT;
}

/* Bit k of mask selects decision k of the pixel's flagged list d[0..k). */
static int subset(const orc_decision* d, int k, int mask, orc_decision* out)
{
    int m = 0;
    for (int i = 0; i < k; i++)
        if (mask & (1 << i)) out[m++] = d[i];
    return m;
}

/*
 * Forward rasterization of one view.
 * ranges[tile][2] = [start, end) into vals; vals[] = slot of each list entry; tiles are
 * row-major with tiles_x = ceil(W / tile).  Outputs: image[3][H][W], T_final[H][W],
 * n_contrib[H][W]; flag[H][W] = the number of flagged alpha_min / t_min decisions of the pixel
 * (-1: more than KMAX_DEC, unresolved); err_C[3][H][W] (float32 error bound of the colour,
 * absolute); err_T[H][W] (of T_final, relative); counters[4] = {evaluated pairs (every list entry
 * up to the pixel's stop: E_tile), blended pairs, blended pairs whose alpha was clamped, evaluated
 * pairs whose pixel lies in the entry's exact alpha_min box (E_box)}.  Alternatives: for every pixel with 1..KMAX_DEC
 * flagged decisions and every non-empty combination of them taken the other way, one entry
 * (alt_pix = y W + x, alt_C[3], alt_T, alt_nc); *alt_n = their number (entries past alt_cap are
 * counted, not written).
 */
void orc_raster_forward(int32_t W, int32_t H, const int32_t* ranges, const int32_t* vals, const double* mean2d,
                        const double* conic, const double* opacity, const double* color, const orc_params* p,
                        double* image, double* T_final, int32_t* n_contrib, int8_t* flag, double* err_C,
                        double* err_T, int64_t alt_cap, int64_t* alt_n, int64_t* alt_pix, double* alt_C,
                        double* alt_T, int32_t* alt_nc, int64_t* counters)
{
    const int tile = p->tile;
    const int tx_n = (W + tile - 1) / tile, ty_n = (H + tile - 1) / tile;
    const orc_records r = {mean2d, conic, opacity, color};
    const int64_t plane = (int64_t)W * H;
    int64_t tot_eval = 0, tot_blend = 0, tot_clamp = 0, tot_box = 0, n_alt = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : tot_eval, tot_blend, tot_clamp, tot_box)
    for (int t = 0; t < tx_n * ty_n; t++) {
        const int tx = t % tx_n, ty = t / tx_n;
        const int32_t start = ranges[2 * t], end = ranges[2 * t + 1];
        for (int y = ty * tile; y < (ty + 1) * tile && y < H; y++)
            for (int x = tx * tile; x < (tx + 1) * tile && x < W; x++) {
                orc_walk w;
                walk_init(&w, NULL, 0, NULL, NULL);
                composite_walk(x + 0.5, y + 0.5, vals + start, end - start, &r, p, &w);
                const int64_t px = (int64_t)y * W + x;
                for (int ch = 0; ch < 3; ch++) {
                    image[ch * plane + px] = w.C[ch];
                    err_C[ch * plane + px] = w.eC[ch];
                }
                T_final[px] = w.T;
                n_contrib[px] = w.n_contrib;
                err_T[px] = w.eT;
                flag[px] = (int8_t)(w.n_fwd > KMAX_DEC ? -1 : w.n_fwd);
                tot_eval += w.n_eval;
                tot_blend += w.n_blend;
                tot_clamp += w.n_clamped;
                tot_box += w.n_box;
                if (w.n_fwd == 0 || w.n_fwd > KMAX_DEC) continue;
                for (int mask = 1; mask < (1 << w.n_fwd); mask++) {
                    orc_decision f[KMAX_DEC];
                    const int nf = subset(w.fwd, w.n_fwd, mask, f);
                    orc_walk a;
                    walk_init(&a, f, nf, NULL, NULL);
                    composite_walk(x + 0.5, y + 0.5, vals + start, end - start, &r, p, &a);
                    int64_t k;
#pragma omp atomic capture
                    k = n_alt++;
                    if (k < alt_cap) {
                        alt_pix[k] = px;
                        for (int ch = 0; ch < 3; ch++) alt_C[3 * k + ch] = a.C[ch];
                        alt_T[k] = a.T;
                        alt_nc[k] = a.n_contrib;
                    }
                }
            }
    }
    *alt_n = n_alt;
    counters[0] = tot_eval;
    counters[1] = tot_blend;
    counters[2] = tot_clamp;
    counters[3] = tot_box;
}

/* ve helpers for the compositing backward: a faithful reciprocal (one ulp) */
static ve ve_rcp(ve a)
{
    ve r = {1.0 / a.v, 0.0};
    r.e = a.e / (a.v * a.v) + 2.0 * EPS32 * fabs(r.v);
    return r;
}

/*
 * Gradient contributions of one pixel's blended entries (the walk's log), traversed from the
 * last blended entry to the first, with dL/dC = g:
 *   dL/dc_j     = alpha_j T_j g
 *   dL/dalpha_j = T_j (sum_ch g_ch c_j,ch - GB) - T_final / (1 - alpha_j) sum_ch g_ch bg_ch
 *   GB         <- GB + alpha_j (sum_ch g_ch c_j,ch - GB)      (sum_ch g_ch x colour behind)
 * and, unless alpha was clamped, with gv = o G dL/dalpha_j:
 *   dL/do       = gv / o
 *   dL/dmean2d  = gv (A dx + B dy, B dx + C dy)
 *   dL/dconic   = gv (-dx^2 / 2, -dx dy, -dy^2 / 2).
 * Per entry e of the log and component k (mean x, y, conic A, B, C, opacity, colour r, g, b):
 * val[9 e + k] = the contribution; err[9 e + k] = a first-order running bound on its float32
 * evaluation error (Higham's running error analysis, the ve arithmetic above): T_j recovered
 * from T_final by dividing by 1 - alpha (faithful reciprocals), alpha and v = o G within
 * pair_alpha_error, dx and dy rounded once, the mean gradient formed as A (gv dx) + B (gv dy)
 * and the opacity gradient as gv / o; mag[9 e + k] = the sum of the absolute values of the
 * parts that a float32 sum adds (A gv dx and B gv dy for the means).
 */
static void pixel_backward(const orc_walk* w, const orc_records* r, const orc_params* p, const double g[3],
                           double* val, double* err, double* mag)
{
    const double u = EPS32;
    const int bg = p->bg[0] != 0.0 || p->bg[1] != 0.0 || p->bg[2] != 0.0;
    const ve one = ve_in(1.0);
    const ve TN = {w->T, w->T * w->eT};
    const ve gbg = ve_add(ve_add(ve_mul(ve_in(g[0]), ve_in(p->bg[0])), ve_mul(ve_in(g[1]), ve_in(p->bg[1]))),
                          ve_mul(ve_in(g[2]), ve_in(p->bg[2])));
    ve GB = ve_in(0.0);
    double accT = w->eT; /* relative error bound of T recovered at the current entry */
    for (int e = w->n_log - 1; e >= 0; e--) {
        const orc_blend* b = &w->log[e];
        const int s = b->slot;
        const double* c = &r->color[3 * s];
        double* vv = val + 9 * e;
        double* ee = err + 9 * e;
        double* mm = mag + 9 * e;
        const ve alpha = {b->alpha, b->rel * b->alpha};
        const ve oma = ve_sub(one, alpha);
        accT += b->alpha * b->rel / (1.0 - b->alpha) + 4.0 * u;
        const ve Tj = {b->T, b->T * accT};
        const ve wgt = ve_mul(alpha, Tj);
        for (int ch = 0; ch < 3; ch++) {
            const ve dc = ve_mul(wgt, ve_in(g[ch]));
            vv[6 + ch] = dc.v;
            ee[6 + ch] = dc.e;
            mm[6 + ch] = fabs(dc.v);
        }
        const ve sgc = ve_add(ve_add(ve_mul(ve_in(g[0]), ve_in(c[0])), ve_mul(ve_in(g[1]), ve_in(c[1]))),
                              ve_mul(ve_in(g[2]), ve_in(c[2])));
        const ve ge = ve_sub(sgc, GB);
        ve dLda = ve_mul(Tj, ge);
        if (bg) dLda = ve_sub(dLda, ve_mul(ve_mul(TN, ve_rcp(oma)), gbg));
        GB = ve_add(GB, ve_mul(alpha, ge));
        if (b->clamped) {
            for (int k = 0; k < 6; k++) vv[k] = ee[k] = mm[k] = 0.0;
            continue;
        }
        const double o = r->opacity[s];
        const double A = r->conic[3 * s], B = r->conic[3 * s + 1], Cc = r->conic[3 * s + 2];
        const ve vG = {b->v, b->rel * b->v};
        const ve gv = ve_mul(vG, dLda);
        const ve dx = {b->dx, u * fabs(b->dx)}, dy = {b->dy, u * fabs(b->dy)};
        const ve gx = ve_mul(gv, dx), gy = ve_mul(gv, dy);
        vv[0] = A * gx.v + B * gy.v;
        ee[0] = fabs(A) * gx.e + fabs(B) * gy.e;
        mm[0] = fabs(A * gx.v) + fabs(B * gy.v);
        vv[1] = B * gx.v + Cc * gy.v;
        ee[1] = fabs(B) * gx.e + fabs(Cc) * gy.e;
        mm[1] = fabs(B * gx.v) + fabs(Cc * gy.v);
        const ve xx = ve_mul(gx, dx), xy = ve_mul(gx, dy), yy = ve_mul(gy, dy);
        vv[2] = -0.5 * xx.v;
        ee[2] = 0.5 * xx.e;
        mm[2] = 0.5 * fabs(xx.v);
        vv[3] = -xy.v;
        ee[3] = xy.e;
        mm[3] = fabs(xy.v);
        vv[4] = -0.5 * yy.v;
        ee[4] = 0.5 * yy.e;
        mm[4] = 0.5 * fabs(yy.v);
        vv[5] = gv.v / o;
        ee[5] = gv.e / o;
        mm[5] = fabs(gv.v / o);
    }
}

static void atomic_add9(double* dst, const double* src)
{
    for (int k = 0; k < 9; k++) {
        if (src[k] == 0.0) continue;
#pragma omp atomic
        dst[k] += src[k];
    }
}

/* Per list position: the contributions of a walk (zero for entries it does not blend). */
static void by_position(const orc_walk* w, const double* val, double* out, int n_pos)
{
    memset(out, 0, sizeof(double) * 9 * (size_t)n_pos);
    for (int e = 0; e < w->n_log; e++) memcpy(out + 9 * (size_t)w->log[e].j, val + 9 * e, sizeof(double) * 9);
}

/*
 * Backward rasterization of one view: gradients of L with respect to the per-slot 2D records,
 * given dL/dC (dldc[3][H][W]); each pixel's walk is recomputed with its blend log and
 * pixel_backward gives the contributions.
 * Outputs (double, accumulated over the view's pixels; zeroed by the caller): d_mean2d[slots][2],
 * d_conic[slots][3], d_opacity[slots], d_color[slots][3] in the component order above;
 * mag[slots][9] = summed magnitudes of the parts; err[slots][9] = summed float32 error bounds of
 * the contributions; widen[slots][9] = for the pixels with flagged decisions, the most that
 * taking any combination of them the other way changes the slot's contribution, plus, where
 * dg[3][H][W] (optional) gives an uncertainty of dL/dC, dg_ch times the contribution of a unit
 * dL/dC_ch; slot_flag[slots] = 1 for the slots a pixel with more than KMAX_DEC flagged
 * decisions may blend (unresolved, left out of comparisons).
 * stats[3] = {pixels with flagged decisions, unresolved pixels, alternative walks}.
 */
void orc_raster_backward(int32_t W, int32_t H, const int32_t* ranges, const int32_t* vals, const double* mean2d,
                         const double* conic, const double* opacity, const double* color, const orc_params* p,
                         const double* dldc, const double* dg, double* d_mean2d, double* d_conic, double* d_opacity,
                         double* d_color, double* mag, double* err, double* widen, int8_t* slot_flag,
                         int64_t* stats)
{
    const int tile = p->tile;
    const int tx_n = (W + tile - 1) / tile, ty_n = (H + tile - 1) / tile;
    const orc_records r = {mean2d, conic, opacity, color};
    const int64_t plane = (int64_t)W * H;
    int max_n = 1;
    for (int t = 0; t < tx_n * ty_n; t++)
        if (ranges[2 * t + 1] - ranges[2 * t] > max_n) max_n = ranges[2 * t + 1] - ranges[2 * t];
    int64_t n_flagged = 0, n_unresolved = 0, n_alt = 0;
#pragma omp parallel reduction(+ : n_flagged, n_unresolved, n_alt)
    {
        const size_t n9 = 9 * (size_t)max_n;
        orc_blend* log = (orc_blend*)malloc(sizeof(orc_blend) * (size_t)max_n);
        orc_blend* alog = (orc_blend*)malloc(sizeof(orc_blend) * (size_t)max_n);
        int8_t* touch = (int8_t*)calloc((size_t)max_n, 1);
        double* bv = (double*)malloc(sizeof(double) * n9);
        double* be = (double*)malloc(sizeof(double) * n9);
        double* bm = (double*)malloc(sizeof(double) * n9);
        double* tv = (double*)malloc(sizeof(double) * n9);
        double* te = (double*)malloc(sizeof(double) * n9);
        double* tm = (double*)malloc(sizeof(double) * n9);
        double* base_j = (double*)malloc(sizeof(double) * n9);
        double* alt_j = (double*)malloc(sizeof(double) * n9);
        double* wid = (double*)malloc(sizeof(double) * n9);
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < tx_n * ty_n; t++) {
            const int tx = t % tx_n, ty = t / tx_n;
            const int32_t start = ranges[2 * t], end = ranges[2 * t + 1];
            const int32_t* list = vals + start;
            const int n = end - start;
            for (int y = ty * tile; y < (ty + 1) * tile && y < H; y++)
                for (int x = tx * tile; x < (tx + 1) * tile && x < W; x++) {
                    const int64_t px = (int64_t)y * W + x;
                    const double g[3] = {dldc[px], dldc[plane + px], dldc[2 * plane + px]};
                    orc_walk w;
                    walk_init(&w, NULL, 0, log, touch);
                    composite_walk(x + 0.5, y + 0.5, list, n, &r, p, &w);
                    pixel_backward(&w, &r, p, g, bv, be, bm);
                    for (int e = 0; e < w.n_log; e++) {
                        const int s = w.log[e].slot;
                        const double* vv = bv + 9 * e;
                        const double cv[9] = {vv[0], vv[1], vv[2], vv[3], vv[4], vv[5], vv[6], vv[7], vv[8]};
                        double* outs[9] = {&d_mean2d[2 * s], &d_mean2d[2 * s + 1], &d_conic[3 * s],
                                           &d_conic[3 * s + 1], &d_conic[3 * s + 2], &d_opacity[s],
                                           &d_color[3 * s], &d_color[3 * s + 1], &d_color[3 * s + 2]};
                        for (int k = 0; k < 9; k++) {
                            if (cv[k] == 0.0) continue;
#pragma omp atomic
                            *outs[k] += cv[k];
                        }
                        atomic_add9(mag + 9 * (size_t)s, bm + 9 * e);
                        atomic_add9(err + 9 * (size_t)s, be + 9 * e);
                    }
                    const int nd = w.n_fwd + w.n_clamp_flag;
                    const int unsure = dg && (dg[px] > 0.0 || dg[plane + px] > 0.0 || dg[2 * plane + px] > 0.0);
                    if (nd == 0 && !unsure) continue;
                    n_flagged += nd > 0;
                    if (nd > KMAX_DEC) {
                        /* unresolved: the slots it blends, or could blend under float32 decisions */
                        n_unresolved++;
                        for (int j = 0; j < (int)w.n_eval; j++)
                            if (touch[j]) {
#pragma omp atomic write
                                slot_flag[list[j]] = 1;
                            }
                        continue;
                    }
                    const int n_pos = n; /* alternatives may reach further down the list */
                    by_position(&w, bv, base_j, n_pos);
                    memset(wid, 0, sizeof(double) * 9 * (size_t)n_pos);
                    orc_decision all[2 * KMAX_DEC];
                    int na = 0;
                    for (int k = 0; k < w.n_fwd; k++) all[na++] = w.fwd[k];
                    for (int k = 0; k < w.n_clamp_flag; k++) all[na++] = w.clamp[k];
                    for (int mask = 1; mask < (1 << na); mask++) {
                        orc_decision f[2 * KMAX_DEC];
                        const int nf = subset(all, na, mask, f);
                        orc_walk a;
                        walk_init(&a, f, nf, alog, NULL);
                        composite_walk(x + 0.5, y + 0.5, list, n, &r, p, &a);
                        pixel_backward(&a, &r, p, g, tv, te, tm);
                        by_position(&a, tv, alt_j, n_pos);
                        for (size_t i = 0; i < 9 * (size_t)n_pos; i++) {
                            const double d = fabs(alt_j[i] - base_j[i]);
                            if (d > wid[i]) wid[i] = d;
                        }
                        n_alt++;
                    }
                    if (unsure) {
                        for (int ch = 0; ch < 3; ch++) {
                            const double dgc = dg[ch * plane + px];
                            if (!(dgc > 0.0)) continue;
                            const double unit[3] = {ch == 0, ch == 1, ch == 2};
                            pixel_backward(&w, &r, p, unit, tv, te, tm);
                            by_position(&w, tv, alt_j, n_pos);
                            for (size_t i = 0; i < 9 * (size_t)n_pos; i++) wid[i] += dgc * fabs(alt_j[i]);
                        }
                    }
                    for (int j = 0; j < n_pos; j++) atomic_add9(widen + 9 * (size_t)list[j], wid + 9 * (size_t)j);
                }
        }
        free(log);
        free(alog);
        free(touch);
        free(bv);
        free(be);
        free(bm);
        free(tv);
        free(te);
        free(tm);
        free(base_j);
        free(alt_j);
        free(wid);
    }
    stats[0] = n_flagged;
    stats[1] = n_unresolved;
    stats[2] = n_alt;
}

/*
 * The float32 error bound of v = o exp(-q/2) for n arbitrary (pixel, record) pairs: the same
 * function the walks use, exposed so that it can be checked against float32 evaluations.
 * Outputs v[n] and rel[n].
 */
void orc_pair_alpha(int64_t n, const double* px, const double* py, const double* mean2d, const double* conic,
                    const double* opacity, double* v, double* rel)
{
    for (int64_t i = 0; i < n; i++) {
        const double dx = px[i] - mean2d[2 * i], dy = py[i] - mean2d[2 * i + 1];
        const double A = conic[3 * i], B = conic[3 * i + 1], Cc = conic[3 * i + 2];
        const double q = A * dx * dx + 2.0 * B * dx * dy + Cc * dy * dy;
        const double qabs = fabs(A) * dx * dx + 2.0 * fabs(B * dx * dy) + fabs(Cc) * dy * dy;
        v[i] = opacity[i] * exp(-0.5 * q);
        rel[i] = pair_alpha_error(qabs, opacity[i]);
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
            orc_walk w;
            walk_init(&w, NULL, 0, NULL, NULL);
            composite_walk(x + 0.5, y + 0.5, order, n, &r, p, &w);
            const int64_t px = (int64_t)y * W + x;
            for (int ch = 0; ch < 3; ch++) image[(int64_t)ch * W * H + px] = w.C[ch];
            T_final[px] = w.T;
            n_contrib[px] = w.n_contrib; /* position in the global order, not in a tile list */
        }
}

/* Threads the parallel loops above use (for reporting the CPU baseline). */
int orc_num_threads(void)
{
    return omp_get_max_threads();
}

/* Set the threads of the parallel loops above (the CPU baseline is timed at all threads and at
 * one). */
void orc_set_num_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : 1);
}
