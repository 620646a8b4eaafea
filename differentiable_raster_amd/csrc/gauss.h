// Per-Gaussian quantities that the projection and its backward both evaluate.  Both kernels
// call these functions, so the backward sees bit-identical values (in particular the colour
// before its clamp at zero, whose sign decides whether the colour gradient flows).
#pragma once

#include "common.h"

namespace gsmi {

// Activated parameters and world covariance of one Gaussian.
struct GaussFrame {
    float s[3];    // scales exp(log_scale)
    float q[4];    // normalized quaternion (w, x, y, z)
    float qn;      // norm of the raw quaternion
    float R[9];    // rotation of q, row-major
    float S[6];    // Sigma = R diag(s^2) R^T: xx, xy, xz, yy, yz, zz
    float o;       // sigmoid(logit)
    bool ok;       // every input finite and the quaternion non-zero
};

__device__ __forceinline__ GaussFrame gauss_frame(float l0, float l1, float l2, float qw, float qx, float qy, float qz,
                                                  float logit, bool finite_mean) {
    GaussFrame f;
    f.ok = finite_mean && isfinite(l0) && isfinite(l1) && isfinite(l2) && isfinite(qw) && isfinite(qx) &&
           isfinite(qy) && isfinite(qz) && isfinite(logit);
    f.o = 1.0f / (1.0f + expf(-logit));
    f.s[0] = expf(l0);
    f.s[1] = expf(l1);
    f.s[2] = expf(l2);
    f.qn = sqrtf(qw * qw + qx * qx + qy * qy + qz * qz);
    f.ok = f.ok && f.qn > 0.0f;
    const float inv = 1.0f / f.qn;
    qw *= inv;
    qx *= inv;
    qy *= inv;
    qz *= inv;
    f.q[0] = qw;
    f.q[1] = qx;
    f.q[2] = qy;
    f.q[3] = qz;
    f.R[0] = 1.0f - 2.0f * (qy * qy + qz * qz);
    f.R[1] = 2.0f * (qx * qy - qw * qz);
    f.R[2] = 2.0f * (qx * qz + qw * qy);
    f.R[3] = 2.0f * (qx * qy + qw * qz);
    f.R[4] = 1.0f - 2.0f * (qx * qx + qz * qz);
    f.R[5] = 2.0f * (qy * qz - qw * qx);
    f.R[6] = 2.0f * (qx * qz - qw * qy);
    f.R[7] = 2.0f * (qy * qz + qw * qx);
    f.R[8] = 1.0f - 2.0f * (qx * qx + qy * qy);
    // M = R diag(s); Sigma = M M^T
    const float m00 = f.R[0] * f.s[0], m01 = f.R[1] * f.s[1], m02 = f.R[2] * f.s[2];
    const float m10 = f.R[3] * f.s[0], m11 = f.R[4] * f.s[1], m12 = f.R[5] * f.s[2];
    const float m20 = f.R[6] * f.s[0], m21 = f.R[7] * f.s[1], m22 = f.R[8] * f.s[2];
    f.S[0] = fmaf(m00, m00, fmaf(m01, m01, m02 * m02));
    f.S[1] = fmaf(m00, m10, fmaf(m01, m11, m02 * m12));
    f.S[2] = fmaf(m00, m20, fmaf(m01, m21, m02 * m22));
    f.S[3] = fmaf(m10, m10, fmaf(m11, m11, m12 * m12));
    f.S[4] = fmaf(m10, m20, fmaf(m11, m21, m12 * m22));
    f.S[5] = fmaf(m20, m20, fmaf(m21, m21, m22 * m22));
    return f;
}

// Real orthonormal spherical harmonics of degree 1..deg at unit direction (x, y, z), textbook
// Cartesian forms without the Condon-Shortley phase; Y[k - 1] is basis function k = l^2 + l + m.
// Returns the number of values written (0, 3, 8 or 15).
__device__ __forceinline__ int sh_basis(int deg, float x, float y, float z, float Y[15]) {
    if (deg < 1) return 0;
    Y[0] = 0.4886025119029199f * y;  // sqrt(3/(4 pi)) (y, z, x)
    Y[1] = 0.4886025119029199f * z;
    Y[2] = 0.4886025119029199f * x;
    if (deg < 2) return 3;
    Y[3] = 1.0925484305920792f * x * y;                   // 1/2 sqrt(15/pi) xy
    Y[4] = 1.0925484305920792f * y * z;                   // 1/2 sqrt(15/pi) yz
    Y[5] = 0.31539156525252005f * (3.0f * z * z - 1.0f);  // 1/4 sqrt(5/pi) (3z^2 - 1)
    Y[6] = 1.0925484305920792f * x * z;                   // 1/2 sqrt(15/pi) xz
    Y[7] = 0.5462742152960396f * (x * x - y * y);         // 1/4 sqrt(15/pi) (x^2 - y^2)
    if (deg < 3) return 8;
    Y[8] = 0.5900435899266435f * y * (3.0f * x * x - y * y);   // 1/4 sqrt(35/(2pi))
    Y[9] = 2.890611442640554f * x * y * z;                     // 1/2 sqrt(105/pi)
    Y[10] = 0.4570457994644658f * y * (5.0f * z * z - 1.0f);   // 1/4 sqrt(21/(2pi))
    Y[11] = 0.3731763325901154f * z * (5.0f * z * z - 3.0f);   // 1/4 sqrt(7/pi)
    Y[12] = 0.4570457994644658f * x * (5.0f * z * z - 1.0f);   // 1/4 sqrt(21/(2pi))
    Y[13] = 1.445305721320277f * z * (x * x - y * y);          // 1/4 sqrt(105/pi)
    Y[14] = 0.5900435899266435f * x * (x * x - 3.0f * y * y);  // 1/4 sqrt(35/(2pi))
    return 15;
}

// sum_k e[k - 1] * grad Y_k at (x, y, z): the Cartesian gradients of the same polynomials,
// weighted (the backward's dL/d direction for weights e = dL/dY).  e[k] for k >= the number of
// basis values of `deg` must be zero.
__device__ __forceinline__ float3 sh_dir_grad(float x, float y, float z, const float e[15]) {
    const float c1 = 0.4886025119029199f, c2 = 1.0925484305920792f, c3 = 0.31539156525252005f;
    const float c4 = 0.5462742152960396f, c5 = 0.5900435899266435f, c6 = 2.890611442640554f;
    const float c7 = 0.4570457994644658f, c8 = 0.3731763325901154f, c9 = 1.445305721320277f;
    const float x2my2 = x * x - y * y, z5 = 5.0f * z * z - 1.0f;
    float3 g;
    g.x = c1 * e[2] + c2 * y * e[3] + c2 * z * e[6] + 2.0f * c4 * x * e[7] + 6.0f * c5 * x * y * e[8] +
          c6 * y * z * e[9] + c7 * z5 * e[12] + 2.0f * c9 * x * z * e[13] + 3.0f * c5 * x2my2 * e[14];
    g.y = c1 * e[0] + c2 * x * e[3] + c2 * z * e[4] - 2.0f * c4 * y * e[7] + 3.0f * c5 * x2my2 * e[8] +
          c6 * x * z * e[9] + c7 * z5 * e[10] - 2.0f * c9 * y * z * e[13] - 6.0f * c5 * x * y * e[14];
    g.z = c1 * e[1] + c2 * y * e[4] + 6.0f * c3 * z * e[5] + c2 * x * e[6] + c6 * x * y * e[9] +
          10.0f * c7 * y * z * e[10] + c8 * (15.0f * z * z - 3.0f) * e[11] + 10.0f * c7 * x * z * e[12] +
          c9 * x2my2 * e[13];
    return g;
}

// Colour channel before the clamp, one channel of sh_eval with the same operations in the same
// order (so it rounds identically): DC + sum_k sh_k Y_k.
__device__ __forceinline__ float sh_eval_channel(const float* coef, int nY, const float Y[15]) {
    float c = coef[0];
#pragma unroll
    for (int k = 0; k < 15; k++)
        if (k < nY) c = fmaf(coef[k + 1], Y[k], c);
    return c;
}

// Colour before the clamp: DC + sum_k sh_k Y_k, accumulated in basis order with one FMA per
// term.  sh points at the coefficient of Gaussian i in row 0; rows are n apart.
__device__ __forceinline__ float3 sh_eval(const float* sh, int64_t n, int nY, const float Y[15]) {
    float3 c = make_float3(sh[0], sh[n], sh[2 * n]);
#pragma unroll
    for (int k = 0; k < 15; k++) {
        if (k < nY) {
            const int64_t row = (k + 1) * 3;
            c.x = fmaf(sh[(row + 0) * n], Y[k], c.x);
            c.y = fmaf(sh[(row + 1) * n], Y[k], c.y);
            c.z = fmaf(sh[(row + 2) * n], Y[k], c.z);
        }
    }
    return c;
}

// Unit viewing direction from the camera centre to the mean; false if they coincide.
__device__ __forceinline__ bool view_dir(float mx, float my, float mz, const float campos[3], float* dx, float* dy,
                                         float* dz, float* inv_len) {
    float x = mx - campos[0], y = my - campos[1], z = mz - campos[2];
    const float dn = sqrtf(x * x + y * y + z * z);
    if (!(dn > 0.0f)) return false;
    const float idn = 1.0f / dn;
    *dx = x * idn;
    *dy = y * idn;
    *dz = z * idn;
    *inv_len = idn;
    return true;
}

}  // namespace gsmi
