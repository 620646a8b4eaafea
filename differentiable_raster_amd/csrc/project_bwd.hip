// Backward of the projection: the chain rule from the per-slot gradients of (mean2d, conic,
// opacity, colour) of every view to the Gaussian parameters (means, log-scales, raw quaternion,
// opacity logit, SH coefficients), summed over the views that see the Gaussian.
//
// One thread per Gaussian gathers its views (no atomics; every output is written once):
//  * slot lookup: visible Gaussians of a view occupy slots in ascending index order, so the
//    visible Gaussians of a 256-Gaussian block are one run of vis_ids that starts at the first
//    slot whose id is >= the block's first index.  One wave per view finds that start with a
//    64-ary search (four rounds for a million slots); unless the slot there names a Gaussian
//    past the block (then the view sees none of the block's Gaussians), the block loads the
//    256-entry window into LDS, and each thread finds its own slot there by binary search;
//  * the per-Gaussian frame (activations, rotation, world covariance) and the colour before its
//    clamp come from the same device functions as the forward projection, so the colour clamp
//    takes the forward's decision;
//  * per view: conic -> dilated 2D covariance (the dilation is constant; the derivative of the
//    inverse, -M G M, in terms of the conic M) -> T = J W and the
//    world covariance -> J(t) and the projected centre -> camera-space t -> mean; the world
//    covariance gradient is accumulated over views as a symmetric 3x3 and turned into scale and
//    rotation gradients once; colour -> SH coefficients and, through the viewing direction,
//    the mean.
// HBM-bound: 4 B per (view, slot) of vis_ids, 36 B of 2D gradients per visible (view, slot),
// and per Gaussian its parameters read once and its gradients written once (236 + 236 B at SH
// degree 3).
#include <limits.h>

#include "common.h"
#include "gauss.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;

// First position p in [0, cnt) with ids[p] >= key (cnt if none), by one wave: each round probes
// 64 evenly spaced positions and keeps the interval between the last probe below key and the
// first at or above it.
__device__ int wave_lower_bound(const int32_t* ids, int cnt, int key) {
    const int lane = threadIdx.x & (kWave - 1);
    int lo = 0, hi = cnt;  // the answer lies in [lo, hi]
    while (lo < hi) {
        const int step = (hi - lo + kWave - 1) / kWave;
        const int p = lo + lane * step;
        const bool below = p < hi && ids[p] < key;
        const int c = __popcll(__ballot(below));
        if (c == 0) {
            hi = lo;
        } else {
            const int nlo = lo + (c - 1) * step + 1;
            hi = min(hi, lo + c * step);
            lo = nlo;
        }
    }
    return lo;
}

template <int DEG>
__global__ __launch_bounds__(kBlock) void project_bwd_kernel(ProjectBwdArgs a) {
    constexpr int NY = DEG == 0 ? 0 : (DEG == 1 ? 3 : (DEG == 2 ? 8 : 15));
    constexpr int NK = NY + 1;
    __shared__ int s_lo[GS_MAX_VIEWS];
    __shared__ int s_win[GS_MAX_VIEWS][kBlock];
    __shared__ int s_slot[GS_MAX_VIEWS][kBlock];
    __shared__ int s_has[GS_MAX_VIEWS];  // 0 when the view sees none of the block's Gaussians
    const int i0 = blockIdx.x * kBlock;
    const int i = i0 + threadIdx.x;
    const int n = a.n;
    const int w = threadIdx.x / kWave;

    // 1. start of this block's run of slots in every view, the windows, then each thread's slot
    for (int v = w; v < a.V; v += kBlock / kWave) {
        const int cnt = min(a.vis_count[v], a.capacity);
        const int32_t* ids = a.vis_ids + (size_t)v * a.capacity;
        const int lo = wave_lower_bound(ids, cnt, i0);
        if ((threadIdx.x & (kWave - 1)) == 0) {
            s_lo[v] = lo;
            // the first slot at or after the block's start names a later Gaussian: none of this
            // block's Gaussians is in the view (most blocks of a large scene)
            s_has[v] = (lo < cnt && ids[lo] < i0 + kBlock) ? 1 : 0;
        }
    }
    __syncthreads();
    for (int v = 0; v < a.V; v++) {
        if (!s_has[v]) continue;  // no slot of this view in the block (uniform)
        const int cnt = min(a.vis_count[v], a.capacity);
        const int p = s_lo[v] + threadIdx.x;
        s_win[v][threadIdx.x] = p < cnt ? a.vis_ids[(size_t)v * a.capacity + p] : INT_MAX;
    }
    __syncthreads();
    if (i >= n) return;
    for (int v = 0; v < a.V; v++) {
        if (!s_has[v]) {
            s_slot[v][threadIdx.x] = -1;
            continue;
        }
        int lo = 0, hi = kBlock;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_win[v][mid] < i) lo = mid + 1;
            else hi = mid;
        }
        s_slot[v][threadIdx.x] = (lo < kBlock && s_win[v][lo] == i) ? s_lo[v] + lo : -1;
    }
    const int64_t nn = n;
    {
        // a Gaussian that no view sees gets zero gradients, without reading its parameters (they
        // may be anything, non-finite included; in a large scene most Gaussians are such); with
        // seen flags requested, its rows are not written either
        bool seen = false;
        for (int v = 0; v < a.V; v++) seen |= s_slot[v][threadIdx.x] >= 0;
        if (a.seen_out) {
            a.seen_out[i] = seen ? 1 : 0;
            if (!seen) return;
        }
        if (!seen) {
            for (int k = 0; k < 3; k++) {
                a.g_means[k * nn + i] = 0.0f;
                a.g_log_scales[k * nn + i] = 0.0f;
            }
            for (int k = 0; k < 4; k++) a.g_quats[k * nn + i] = 0.0f;
            a.g_logits[i] = 0.0f;
#pragma unroll
            for (int k = 0; k < 3 * NK; k++) a.g_sh[k * nn + i] = 0.0f;
            return;
        }
    }

    // 2. per-Gaussian frame, as the forward projection computes it
    const float mx = a.means[i], my = a.means[nn + i], mz = a.means[2 * nn + i];
    const GaussFrame f = gauss_frame(a.log_scales[i], a.log_scales[nn + i], a.log_scales[2 * nn + i], a.quats[i],
                                     a.quats[nn + i], a.quats[2 * nn + i], a.quats[3 * nn + i], a.logits[i], true);
    const float* S = f.S;
    float gmu[3] = {0.0f, 0.0f, 0.0f};
    float Gs[6] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};  // symmetrized dL/dSigma: xx, xy, xz, yy, yz, zz
    float glogit = 0.0f;

    // 3. geometry, per view
    for (int v = 0; v < a.V; v++) {
        const int slot = s_slot[v][threadIdx.x];
        if (slot < 0) continue;
        const size_t idx = (size_t)v * a.capacity + slot;
        const CamDev& c = a.cams.c[v];
        const float2 gm = a.d_mean2d[idx];
        const float gA = a.d_conic[3 * idx], gB = a.d_conic[3 * idx + 1], gC = a.d_conic[3 * idx + 2];
        const float go = a.d_opacity[idx];

        // forward quantities of this view (the forward projection's formulas)
        const float tx = fmaf(c.R[0], mx, fmaf(c.R[1], my, fmaf(c.R[2], mz, c.t[0])));
        const float ty = fmaf(c.R[3], mx, fmaf(c.R[4], my, fmaf(c.R[5], mz, c.t[1])));
        const float tz = fmaf(c.R[6], mx, fmaf(c.R[7], my, fmaf(c.R[8], mz, c.t[2])));
        const float iz = 1.0f / tz;
        const float j00 = c.fx * iz, j02 = -c.fx * tx * iz * iz;
        const float j11 = c.fy * iz, j12 = -c.fy * ty * iz * iz;
        const float T0[3] = {fmaf(j00, c.R[0], j02 * c.R[6]), fmaf(j00, c.R[1], j02 * c.R[7]),
                             fmaf(j00, c.R[2], j02 * c.R[8])};
        const float T1[3] = {fmaf(j11, c.R[3], j12 * c.R[6]), fmaf(j11, c.R[4], j12 * c.R[7]),
                             fmaf(j11, c.R[5], j12 * c.R[8])};
        // U = Sigma T0^T, Vv = Sigma T1^T
        const float U[3] = {fmaf(S[0], T0[0], fmaf(S[1], T0[1], S[2] * T0[2])),
                            fmaf(S[1], T0[0], fmaf(S[3], T0[1], S[4] * T0[2])),
                            fmaf(S[2], T0[0], fmaf(S[4], T0[1], S[5] * T0[2]))};
        const float Vv[3] = {fmaf(S[0], T1[0], fmaf(S[1], T1[1], S[2] * T1[2])),
                             fmaf(S[1], T1[0], fmaf(S[3], T1[1], S[4] * T1[2])),
                             fmaf(S[2], T1[0], fmaf(S[4], T1[1], S[5] * T1[2]))};
        const float ca = fmaf(T0[0], U[0], fmaf(T0[1], U[1], T0[2] * U[2])) + a.p.eps2d;
        const float cb = fmaf(T1[0], U[0], fmaf(T1[1], U[1], T1[2] * U[2]));
        const float cc = fmaf(T1[0], Vv[0], fmaf(T1[1], Vv[1], T1[2] * Vv[2])) + a.p.eps2d;
        const float det = ca * cc - cb * cb;
        const float idet = 1.0f / det;
        // the conic as the forward stores it: M = [[A, B], [B, C]] = Sigma'^-1
        const float A = cc * idet, B = -cb * idet, C = ca * idet;

        // M = Sigma'^-1  ->  dL/dSigma' = -M G M with G = [[gA, gB/2], [gB/2, gC]]; the
        // off-diagonal entry appears twice in Sigma', so its gradient is twice the matrix entry.
        // (Written with the conic rather than 1/det^2, whose square can leave float32 range for
        // Gaussians just beyond the near plane and far off axis.)
        const float ga = -(A * A * gA + A * B * gB + B * B * gC);
        const float gb = -(2.0f * A * B * gA + (A * C + B * B) * gB + 2.0f * B * C * gC);
        const float gcc = -(B * B * gA + B * C * gB + C * C * gC);

        // Sigma2D = T Sigma T^T: gradients of the rows of T and (symmetrized) of Sigma
        float gT0[3], gT1[3];
#pragma unroll
        for (int k = 0; k < 3; k++) {
            gT0[k] = 2.0f * ga * U[k] + gb * Vv[k];
            gT1[k] = gb * U[k] + 2.0f * gcc * Vv[k];
        }
        Gs[0] += 2.0f * ga * T0[0] * T0[0] + 2.0f * gb * T0[0] * T1[0] + 2.0f * gcc * T1[0] * T1[0];
        Gs[1] += 2.0f * ga * T0[0] * T0[1] + gb * (T0[0] * T1[1] + T1[0] * T0[1]) + 2.0f * gcc * T1[0] * T1[1];
        Gs[2] += 2.0f * ga * T0[0] * T0[2] + gb * (T0[0] * T1[2] + T1[0] * T0[2]) + 2.0f * gcc * T1[0] * T1[2];
        Gs[3] += 2.0f * ga * T0[1] * T0[1] + 2.0f * gb * T0[1] * T1[1] + 2.0f * gcc * T1[1] * T1[1];
        Gs[4] += 2.0f * ga * T0[1] * T0[2] + gb * (T0[1] * T1[2] + T1[1] * T0[2]) + 2.0f * gcc * T1[1] * T1[2];
        Gs[5] += 2.0f * ga * T0[2] * T0[2] + 2.0f * gb * T0[2] * T1[2] + 2.0f * gcc * T1[2] * T1[2];

        // T = J W  ->  the non-constant entries of J
        const float gj00 = gT0[0] * c.R[0] + gT0[1] * c.R[1] + gT0[2] * c.R[2];
        const float gj02 = gT0[0] * c.R[6] + gT0[1] * c.R[7] + gT0[2] * c.R[8];
        const float gj11 = gT1[0] * c.R[3] + gT1[1] * c.R[4] + gT1[2] * c.R[5];
        const float gj12 = gT1[0] * c.R[6] + gT1[1] * c.R[7] + gT1[2] * c.R[8];

        // J(t) and the projected centre (fx tx / tz + cx, fy ty / tz + cy)  ->  t
        const float iz2 = iz * iz, iz3 = iz2 * iz;
        const float gtx = gm.x * c.fx * iz - gj02 * c.fx * iz2;
        const float gty = gm.y * c.fy * iz - gj12 * c.fy * iz2;
        const float gtz = -gm.x * c.fx * tx * iz2 - gm.y * c.fy * ty * iz2 - gj00 * c.fx * iz2 +
                          gj02 * 2.0f * c.fx * tx * iz3 - gj11 * c.fy * iz2 + gj12 * 2.0f * c.fy * ty * iz3;
        // t = W mu + t_cam  ->  mu
        gmu[0] += c.R[0] * gtx + c.R[3] * gty + c.R[6] * gtz;
        gmu[1] += c.R[1] * gtx + c.R[4] * gty + c.R[7] * gtz;
        gmu[2] += c.R[2] * gtx + c.R[5] * gty + c.R[8] * gtz;

        // opacity = sigmoid(logit)
        glogit += go * f.o * (1.0f - f.o);
    }

    // 4. colour = max(0, DC + sum_k sh_k Y_k(dir)), one channel at a time (keeps the live
    //    coefficients and accumulators to one channel's); the clamp as the forward decided it
    for (int ch = 0; ch < 3; ch++) {
        float coef[NK], gsh[NK];
#pragma unroll
        for (int k = 0; k < NK; k++) {
            coef[k] = a.sh[(k * 3 + ch) * nn + i];
            gsh[k] = 0.0f;
        }
        for (int v = 0; v < a.V; v++) {
            const int slot = s_slot[v][threadIdx.x];
            if (slot < 0) continue;
            const size_t idx = (size_t)v * a.capacity + slot;
            const CamDev& c = a.cams.c[v];
            float dx, dy, dz, idn;
            view_dir(mx, my, mz, c.campos, &dx, &dy, &dz, &idn);
            float Y[15];
            sh_basis(DEG, dx, dy, dz, Y);
            // clamped at zero, or not finite (the view then holds the Gaussian transparent and
            // its 2D gradients are zero; a non-finite coefficient times zero would not be)
            const float val = sh_eval_channel(coef, NY, Y);
            if (!(val > 0.0f) || !isfinite(val)) continue;
            const float g = a.d_color[3 * idx + ch];
            gsh[0] += g;
            if (NY > 0) {
                float e[15];
#pragma unroll
                for (int k = 0; k < 15; k++) {
                    if (k < NY) {
                        gsh[k + 1] += g * Y[k];
                        e[k] = g * coef[k + 1];
                    } else {
                        e[k] = 0.0f;
                    }
                }
                // dir = (mu - campos) / |mu - campos|: project out the radial part
                const float3 gd = sh_dir_grad(dx, dy, dz, e);
                const float r = gd.x * dx + gd.y * dy + gd.z * dz;
                gmu[0] += (gd.x - dx * r) * idn;
                gmu[1] += (gd.y - dy * r) * idn;
                gmu[2] += (gd.z - dz * r) * idn;
            }
        }
#pragma unroll
        for (int k = 0; k < NK; k++) a.g_sh[(k * 3 + ch) * nn + i] = gsh[k];
    }

    // 5. Sigma = sum_k s_k^2 R[:,k] R[:,k]^T  ->  log-scales and rotation; rotation -> quaternion
    const float* R = f.R;
    float gR[9];
#pragma unroll
    for (int k = 0; k < 3; k++) {
        const float r0 = R[k], r1 = R[3 + k], r2 = R[6 + k];  // column k
        const float w0 = Gs[0] * r0 + Gs[1] * r1 + Gs[2] * r2;
        const float w1 = Gs[1] * r0 + Gs[3] * r1 + Gs[4] * r2;
        const float w2 = Gs[2] * r0 + Gs[4] * r1 + Gs[5] * r2;
        const float sk = f.s[k], sk2 = sk * sk;
        // d/ds_k = s_k (r . Gs r); d/dlog s_k = s_k d/ds_k
        a.g_log_scales[k * nn + i] = sk2 * (r0 * w0 + r1 * w1 + r2 * w2);
        gR[k] = sk2 * w0;
        gR[3 + k] = sk2 * w1;
        gR[6 + k] = sk2 * w2;
    }
    const float qw = f.q[0], qx = f.q[1], qy = f.q[2], qz = f.q[3];
    // derivatives of the rotation matrix entries of the unit quaternion (w, x, y, z)
    float gq[4];
    gq[0] = 2.0f * (-qz * gR[1] + qy * gR[2] + qz * gR[3] - qx * gR[5] - qy * gR[6] + qx * gR[7]);
    gq[1] = 2.0f * (qy * gR[1] + qz * gR[2] + qy * gR[3] - 2.0f * qx * gR[4] - qw * gR[5] + qz * gR[6] +
                    qw * gR[7] - 2.0f * qx * gR[8]);
    gq[2] = 2.0f * (-2.0f * qy * gR[0] + qx * gR[1] + qw * gR[2] + qx * gR[3] + qz * gR[5] - qw * gR[6] +
                    qz * gR[7] - 2.0f * qy * gR[8]);
    gq[3] = 2.0f * (-2.0f * qz * gR[0] - qw * gR[1] + qx * gR[2] + qw * gR[3] - 2.0f * qz * gR[4] + qy * gR[5] +
                    qx * gR[6] + qy * gR[7]);
    // q = raw / |raw|: remove the radial part and divide by |raw|
    const float qd = gq[0] * qw + gq[1] * qx + gq[2] * qy + gq[3] * qz;
    const float iqn = 1.0f / f.qn;
    a.g_quats[i] = (gq[0] - qw * qd) * iqn;
    a.g_quats[nn + i] = (gq[1] - qx * qd) * iqn;
    a.g_quats[2 * nn + i] = (gq[2] - qy * qd) * iqn;
    a.g_quats[3 * nn + i] = (gq[3] - qz * qd) * iqn;
    a.g_means[i] = gmu[0];
    a.g_means[nn + i] = gmu[1];
    a.g_means[2 * nn + i] = gmu[2];
    a.g_logits[i] = glogit;
}

}  // namespace

hipError_t launch_project_bwd(const ProjectBwdArgs& a, hipStream_t s) {
    if (a.n <= 0) return hipSuccess;
    const dim3 grid((a.n + kBlock - 1) / kBlock), block(kBlock);
    switch (a.p.sh_degree) {
        case 0: hipLaunchKernelGGL(project_bwd_kernel<0>, grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL(project_bwd_kernel<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(project_bwd_kernel<2>, grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL(project_bwd_kernel<3>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace gsmi
