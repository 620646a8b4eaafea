// F4: Adam over the Gaussian parameters, dense and deferred (GS-Scale, English abstract: a
// deferred optimizer update avoids the memory accesses of Gaussians whose gradient is zero).
//
// Every parameter component takes the textbook Adam step with its own moments.  The deferred
// form leaves a Gaussian untouched while its whole gradient row is zero and, at its next update,
// first replays the skipped steps with a zero gradient through the same per-element function,
// then takes the current step.  The replay performs the same float32 operations in the same order
// as the dense form would have, so the parameters and moments after a flush are bit-identical to
// the dense ones; only the memory traffic of the skipped Gaussians is saved (their gradient row
// is read, or not even that when the caller names the Gaussians to update, by a list or by
// per-Gaussian seen flags).
//
// One thread per Gaussian: the rows of a group are read and written one after the other at the
// Gaussian's column, so a wavefront touches 64 consecutive floats of each row.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;

// 1 - beta^s in float32 (the dense and the deferred kernels share this function).
__device__ __forceinline__ float bias_correction(float beta, int32_t s) { return 1.0f - powf(beta, (float)s); }

// One Adam step of one element (the dense and the deferred kernels share this function).
__device__ __forceinline__ void adam_elem(float& p, float& m, float& v, float g, float lr, const AdamHyper& h,
                                          float bc1, float bc2) {
    m = h.beta1 * m + (1.0f - h.beta1) * g;
    v = h.beta2 * v + (1.0f - h.beta2) * (g * g);
    const float mhat = m / bc1, vhat = v / bc2;
    p = p - lr * (mhat / (sqrtf(vhat) + h.eps));
}

// Steps [s0, s1] of Gaussian i: steps before s1 with a zero gradient, step s1 with its gradient
// (with_grad) or with zero as well.  bc1 / bc2: the bias corrections of step s1.
__device__ void advance(const AdamArgs& a, int64_t n, int64_t i, int32_t s0, int32_t s1, bool with_grad, float bc1,
                        float bc2) {
    for (int gi = 0; gi < a.n_groups; gi++) {
        const AdamGroup& G = a.groups[gi];
#pragma unroll 4
        for (int r = 0; r < G.rows; r++) {
            const int64_t e = (int64_t)r * n + i;
            float p = G.param[e], m = G.m[e], v = G.v[e];
            for (int32_t s = s0; s < s1; s++)
                adam_elem(p, m, v, 0.0f, G.lr, a.h, bias_correction(a.h.beta1, s), bias_correction(a.h.beta2, s));
            const float g = with_grad ? G.grad[e] : 0.0f;
            adam_elem(p, m, v, g, G.lr, a.h, bc1, bc2);
            G.param[e] = p;
            G.m[e] = m;
            G.v[e] = v;
        }
    }
}

__device__ __forceinline__ bool grad_row_zero(const AdamArgs& a, int64_t n, int64_t i) {
    for (int gi = 0; gi < a.n_groups; gi++) {
        const AdamGroup& G = a.groups[gi];
        for (int r = 0; r < G.rows; r++)
            if (G.grad[(int64_t)r * n + i] != 0.0f) return false;
    }
    return true;
}

// mode 0: dense (every Gaussian, step t); 1: deferred over all Gaussians (zero rows skipped);
// 2: deferred over the listed Gaussians; 3: deferred over the Gaussians whose seen flag is set.
__global__ __launch_bounds__(kBlock) void adam_step_kernel(AdamArgs a, int64_t n, int32_t t, int mode,
                                                           int32_t* last_step, const int32_t* active,
                                                           const uint8_t* seen, int64_t n_items) {
    const float bc1 = bias_correction(a.h.beta1, t), bc2 = bias_correction(a.h.beta2, t);
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < n_items; k += (int64_t)gridDim.x * kBlock) {
        int64_t i = k;
        if (mode == 2) {
            i = active[k];
            if (i < 0 || i >= n) continue;  // not a Gaussian of this model
        }
        if (mode == 0) {
            advance(a, n, i, t, t, true, bc1, bc2);
            continue;
        }
        if (mode == 3 && seen[i] == 0) continue;  // gradient zero by the caller's contract, not read
        const int32_t last = last_step[i];
        if (last >= t) continue;  // already current
        if (mode == 1 && grad_row_zero(a, n, i)) continue;
        advance(a, n, i, last + 1, t, true, bc1, bc2);
        last_step[i] = t;
    }
}

// Bring every Gaussian to step t: the steps after its last update, all with a zero gradient.
__global__ __launch_bounds__(kBlock) void adam_flush_kernel(AdamArgs a, int64_t n, int32_t t, int32_t* last_step) {
    const float bc1 = bias_correction(a.h.beta1, t), bc2 = bias_correction(a.h.beta2, t);
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) {
        const int32_t last = last_step[i];
        if (last >= t) continue;
        advance(a, n, i, last + 1, t, false, bc1, bc2);
        last_step[i] = t;
    }
}

unsigned blocks_for(int64_t items) {
    int64_t b = (items + kBlock - 1) / kBlock;
    if (b > 16384) b = 16384;
    if (b < 1) b = 1;
    return (unsigned)b;
}

}  // namespace

hipError_t launch_adam_step(const AdamArgs& a, int64_t n, int32_t t, int32_t* last_step, const int32_t* active,
                            int64_t n_active, hipStream_t s) {
    const int mode = last_step == nullptr ? 0 : (active == nullptr ? 1 : 2);
    const int64_t items = mode == 2 ? n_active : n;
    if (items <= 0) return hipSuccess;
    hipLaunchKernelGGL(adam_step_kernel, dim3(blocks_for(items)), dim3(kBlock), 0, s, a, n, t, mode, last_step,
                       active, nullptr, items);
    return hipGetLastError();
}

hipError_t launch_adam_step_seen(const AdamArgs& a, int64_t n, int32_t t, int32_t* last_step, const uint8_t* seen,
                                 hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(adam_step_kernel, dim3(blocks_for(n)), dim3(kBlock), 0, s, a, n, t, 3, last_step, nullptr,
                       seen, n);
    return hipGetLastError();
}

hipError_t launch_adam_flush(const AdamArgs& a, int64_t n, int32_t t, int32_t* last_step, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(adam_flush_kernel, dim3(blocks_for(n)), dim3(kBlock), 0, s, a, n, t, last_step);
    return hipGetLastError();
}

}  // namespace gsmi
