// F3: global composition of pixel-level partial renders (Splaxel, English abstract: every GPU
// renders its local subset of the Gaussians, partial pixel values are exchanged and composed
// into the image).  A partial render of a subset is its premultiplied colour C (rendered on a
// black background) and its final transmittance T.  Partials given front to back compose with
// the over operator, C = C_1 + T_1 (C_2 + T_2 (...)), T = T_1 T_2 ..., and the background enters
// once at the end: image = C + T bg.
//
// One thread per pixel of one view (grid y = view).  The partials are walked back to front, so
// each step is one FMA per channel: acc = C_i + T_i acc.  Pure streaming: 16 B read per partial
// and pixel, 16 B written.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;

__global__ __launch_bounds__(kBlock) void compose_kernel(int32_t P, int64_t plane, ComposeArgs a, float* image,
                                                         float* t_out) {
    const int64_t v = blockIdx.y;
    for (int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x; p < plane; p += (int64_t)gridDim.x * kBlock) {
        const int64_t i = v * plane + p;
        const int64_t c0 = (3 * v) * plane + p, c1 = c0 + plane, c2 = c1 + plane;
        float r = 0.0f, g = 0.0f, b = 0.0f, t = 1.0f;
        for (int k = P - 1; k >= 0; k--) {
            const float tk = a.t[k][i];
            r = fmaf(tk, r, a.c[k][c0]);
            g = fmaf(tk, g, a.c[k][c1]);
            b = fmaf(tk, b, a.c[k][c2]);
            t *= tk;
        }
        image[c0] = fmaf(t, a.bg[0], r);
        image[c1] = fmaf(t, a.bg[1], g);
        image[c2] = fmaf(t, a.bg[2], b);
        if (t_out) t_out[i] = t;
    }
}

}  // namespace

hipError_t launch_compose(int32_t P, int32_t V, int64_t plane, const ComposeArgs& a, float* image, float* t_out,
                          hipStream_t s) {
    int64_t blocks = (plane + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(compose_kernel, dim3((unsigned)blocks, (unsigned)V), dim3(kBlock), 0, s, P, plane, a, image,
                       t_out);
    return hipGetLastError();
}

}  // namespace gsmi
