// A7-A10: forward, loss-gradient, backward and fused rasterizers.
//
// One 256-thread workgroup per (view, 16x16 tile): four wavefronts, each covering an 8x8
// quarter of the tile (lane l of wave w -> pixel ((w & 1) * 8 + (l & 7), (w >> 1) * 8 + (l >> 3))).
// The tile's list is staged through LDS in batches of 256 records (one gather per thread).
//
// The forward walks the list front to back; a workgroup stops loading batches once every
// pixel has terminated.  The backward walks each pixel's blended entries back to front from
// n_contrib, recovering T by division by (1 - alpha) and carrying the colour behind; it sums
// each entry's nine gradient components over the wavefront (butterfly shuffles) and issues one
// float atomic per component from one lane.  The fused kernel runs the forward, forms dL/dC
// in registers (L1 against a target, or a supplied gradient) and runs the backward on the same
// workgroup: per-pixel C, T and n_contrib never leave registers, and when the tile's list fits
// the LDS budget its records are read from HBM once for both passes.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = kTileThreads;
constexpr int kBatch = 256;
constexpr int kFusedEntries = 1024;  // records kept resident in LDS by the fused kernel

struct TileCtx {
    int v, g, px, py, lane, w;
    bool inside;
    float fpx, fpy;
    int32_t start, n;
    size_t vbase;
};

__device__ __forceinline__ TileCtx tile_ctx(const RasterArgs& a, const int32_t* ranges) {
    TileCtx c;
    c.g = blockIdx.x;
    const int tpv = a.tiles_x * a.tiles_y;
    c.v = c.g / tpv;
    const int t = c.g - c.v * tpv;
    const int tx = t % a.tiles_x, ty = t / a.tiles_x;
    c.lane = threadIdx.x & (kWave - 1);
    c.w = threadIdx.x / kWave;
    c.px = tx * kTile + (c.w & 1) * 8 + (c.lane & 7);
    c.py = ty * kTile + (c.w >> 1) * 8 + (c.lane >> 3);
    c.inside = c.px < a.width && c.py < a.height;
    c.fpx = (float)c.px + 0.5f;
    c.fpy = (float)c.py + 0.5f;
    c.start = ranges[2 * c.g];
    c.n = ranges[2 * c.g + 1] - c.start;
    c.vbase = (size_t)c.v * a.capacity;
    return c;
}

struct Lds {
    float2* xy;
    float4* co;
    float4* rgb;
    int32_t* slot;
};

__device__ __forceinline__ void stage(const RasterArgs& a, const TileCtx& c, Lds s, int dst, int32_t j) {
    const int32_t slot = a.vals[c.start + j];
    const size_t idx = c.vbase + slot;
    s.xy[dst] = a.mean2d[idx];
    s.co[dst] = a.conic_opacity[idx];
    s.rgb[dst] = make_float4(a.color[3 * idx], a.color[3 * idx + 1], a.color[3 * idx + 2], 0.0f);
    s.slot[dst] = slot;
}

struct Fwd {
    float T, C0, C1, C2;
    int32_t last;
    bool done;
};

// Front-to-back over records [k0, k1) of LDS, list positions j = jbase + k.
// Diagnostic only: is the pixel inside the exact bounding box of {o exp(-q/2) >= alpha_min}?
__device__ __forceinline__ bool in_alpha_box(float dx, float dy, float4 co, float amin) {
    if (!(co.w > amin)) return false;
    const float det = co.x * co.z - co.y * co.y;
    const float Q = 2.0f * logf(co.w / amin);
    const float ex = 1.001f * sqrtf(Q * co.z / det), ey = 1.001f * sqrtf(Q * co.x / det);
    return fabsf(dx) <= ex && fabsf(dy) <= ey;
}

struct Counts {
    int64_t eval, blend, box;
};

template <bool COUNT>
__device__ __forceinline__ void fwd_walk(const RasterArgs& a, const TileCtx& c, Lds s, int k0, int k1, int32_t jbase,
                                         Fwd& f, Counts& cnt) {
    if (f.done) return;
    const float amin = a.p.alpha_min, amax = a.p.alpha_max, tmin = a.p.t_min;
    for (int k = k0; k < k1; k++) {
        const float2 xy = s.xy[k];
        const float4 co = s.co[k];
        const float dx = c.fpx - xy.x, dy = c.fpy - xy.y;
        const float G = pair_gauss(pair_power(dx, dy, co.x, co.y, co.z));
        const float v = co.w * G;
        const float alpha = fminf(amax, v);
        if (COUNT) {
            cnt.eval++;
            cnt.box += in_alpha_box(dx, dy, co, amin) ? 1 : 0;
        }
        if (alpha < amin) continue;
        const float Tn = f.T * one_minus_alpha(co.w, G, v, amax);
        if (Tn < tmin) {
            f.done = true;
            break;
        }
        const float wgt = alpha * f.T;
        const float4 rgb = s.rgb[k];
        f.C0 = fmaf(wgt, rgb.x, f.C0);
        f.C1 = fmaf(wgt, rgb.y, f.C1);
        f.C2 = fmaf(wgt, rgb.z, f.C2);
        f.T = Tn;
        f.last = jbase + k + 1;
        if (COUNT) cnt.blend++;
    }
}

struct Bwd {
    float T, Tfin;
    float g0, g1, g2;
    float B0, B1, B2;
    int32_t nc;
};

__device__ __forceinline__ float wave_sum(float x) {
    for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Back-to-front over records [k0, k1) of LDS (k descending), list positions j = jbase + k.
__device__ __forceinline__ void bwd_walk(const RasterArgs& a, const TileCtx& c, Lds s, int k0, int k1, int32_t jbase,
                                         Bwd& b, Grads gr) {
    const float amin = a.p.alpha_min, amax = a.p.alpha_max;
    const float bg0 = a.p.bg[0], bg1 = a.p.bg[1], bg2 = a.p.bg[2];
    for (int k = k1 - 1; k >= k0; k--) {
        float d[9];
#pragma unroll
        for (int q = 0; q < 9; q++) d[q] = 0.0f;
        bool contrib = false;
        if (jbase + k < b.nc) {
            const float2 xy = s.xy[k];
            const float4 co = s.co[k];
            const float dx = c.fpx - xy.x, dy = c.fpy - xy.y;
            const float G = pair_gauss(pair_power(dx, dy, co.x, co.y, co.z));
            const float v = co.w * G;
            const float alpha = fminf(amax, v);
            if (alpha >= amin) {
                contrib = true;
                const float oma = one_minus_alpha(co.w, G, v, amax);
                const float Tj = b.T / oma;
                const float4 rgb = s.rgb[k];
                const float bgterm = b.Tfin / oma;
                float dLda = b.g0 * (Tj * (rgb.x - b.B0) - bgterm * bg0);
                dLda = fmaf(b.g1, Tj * (rgb.y - b.B1) - bgterm * bg1, dLda);
                dLda = fmaf(b.g2, Tj * (rgb.z - b.B2) - bgterm * bg2, dLda);
                const float wgt = alpha * Tj;
                d[6] = wgt * b.g0;
                d[7] = wgt * b.g1;
                d[8] = wgt * b.g2;
                b.B0 = fmaf(alpha, rgb.x, oma * b.B0);
                b.B1 = fmaf(alpha, rgb.y, oma * b.B1);
                b.B2 = fmaf(alpha, rgb.z, oma * b.B2);
                if (v <= amax) {
                    const float gh = co.w * G * dLda;
                    d[0] = gh * fmaf(co.x, dx, co.y * dy);
                    d[1] = gh * fmaf(co.y, dx, co.z * dy);
                    d[2] = -0.5f * gh * dx * dx;
                    d[3] = -gh * dx * dy;
                    d[4] = -0.5f * gh * dy * dy;
                    d[5] = G * dLda;
                }
                b.T = Tj;
            }
        }
        if (__ballot(contrib) != 0ull) {
#pragma unroll
            for (int q = 0; q < 9; q++) d[q] = wave_sum(d[q]);
            if (c.lane == 0) {
                const size_t idx = c.vbase + s.slot[k];
                if (d[0] != 0.0f) atomicAdd(&gr.d_mean2d[idx].x, d[0]);
                if (d[1] != 0.0f) atomicAdd(&gr.d_mean2d[idx].y, d[1]);
                if (d[2] != 0.0f) atomicAdd(&gr.d_conic[3 * idx + 0], d[2]);
                if (d[3] != 0.0f) atomicAdd(&gr.d_conic[3 * idx + 1], d[3]);
                if (d[4] != 0.0f) atomicAdd(&gr.d_conic[3 * idx + 2], d[4]);
                if (d[5] != 0.0f) atomicAdd(&gr.d_opacity[idx], d[5]);
                if (d[6] != 0.0f) atomicAdd(&gr.d_color[3 * idx + 0], d[6]);
                if (d[7] != 0.0f) atomicAdd(&gr.d_color[3 * idx + 1], d[7]);
                if (d[8] != 0.0f) atomicAdd(&gr.d_color[3 * idx + 2], d[8]);
            }
        }
    }
}

__device__ __forceinline__ int block_max(int x, int* s_red) {
    for (int o = kWave / 2; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
    if ((threadIdx.x & (kWave - 1)) == 0) s_red[threadIdx.x / kWave] = x;
    __syncthreads();
    int m = s_red[0];
    for (int k = 1; k < kBlock / kWave; k++) m = max(m, s_red[k]);
    __syncthreads();
    return m;
}

__device__ __forceinline__ void add_counters(int64_t* counters, Counts c) {
    // wave sums then one atomic per wave
    for (int o = kWave / 2; o > 0; o >>= 1) {
        c.eval += __shfl_xor(c.eval, o);
        c.blend += __shfl_xor(c.blend, o);
        c.box += __shfl_xor(c.box, o);
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
        atomicAdd((unsigned long long*)&counters[0], (unsigned long long)c.eval);
        atomicAdd((unsigned long long*)&counters[1], (unsigned long long)c.blend);
        atomicAdd((unsigned long long*)&counters[2], (unsigned long long)c.box);
    }
}

template <bool COUNT>
__global__ __launch_bounds__(kBlock) void raster_fwd_kernel(RasterArgs a, float* image, float* t_final,
                                                            int32_t* n_contrib) {
    __shared__ float2 s_xy[kBatch];
    __shared__ float4 s_co[kBatch];
    __shared__ float4 s_rgb[kBatch];
    __shared__ int32_t s_slot[kBatch];
    const Lds s{s_xy, s_co, s_rgb, s_slot};
    const TileCtx c = tile_ctx(a, a.ranges);
    Fwd f{1.0f, 0.0f, 0.0f, 0.0f, 0, !c.inside};
    Counts cnts{0, 0, 0};
    for (int32_t b0 = 0; b0 < c.n; b0 += kBatch) {
        if (__syncthreads_count(f.done) == kBlock) break;
        const int32_t j = b0 + threadIdx.x;
        if (j < c.n) stage(a, c, s, threadIdx.x, j);
        __syncthreads();
        const int cnt = min(kBatch, c.n - b0);
        fwd_walk<COUNT>(a, c, s, 0, cnt, b0, f, cnts);
    }
    if (COUNT) add_counters(a.counters, cnts);
    if (!c.inside) return;
    const size_t plane = (size_t)a.width * a.height;
    const size_t p = (size_t)c.py * a.width + c.px;
    image[(size_t)(3 * c.v + 0) * plane + p] = fmaf(f.T, a.p.bg[0], f.C0);
    image[(size_t)(3 * c.v + 1) * plane + p] = fmaf(f.T, a.p.bg[1], f.C1);
    image[(size_t)(3 * c.v + 2) * plane + p] = fmaf(f.T, a.p.bg[2], f.C2);
    t_final[(size_t)c.v * plane + p] = f.T;
    n_contrib[(size_t)c.v * plane + p] = f.last;
}

__global__ __launch_bounds__(256) void loss_l1_kernel(int64_t n, const float* image, const float* target, float scale,
                                                      float* dl, float* loss_sum) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    float l = 0.0f;
    if (i < n) {
        const float d = image[i] - target[i];
        dl[i] = d > 0.0f ? scale : (d < 0.0f ? -scale : 0.0f);
        l = scale * fabsf(d);
    }
    if (loss_sum) {
        l = wave_sum(l);
        if ((threadIdx.x & (kWave - 1)) == 0 && l != 0.0f) atomicAdd(loss_sum, l);
    }
}

__global__ __launch_bounds__(256) void zero_grads_kernel(const int32_t* vis_count, int32_t V, int32_t capacity, Grads g) {
    for (int v = 0; v < V; v++) {
        const int32_t cnt = vis_count[v];
        const size_t base = (size_t)v * capacity;
        for (int32_t s = blockIdx.x * 256 + threadIdx.x; s < cnt; s += gridDim.x * 256) {
            const size_t i = base + s;
            g.d_mean2d[i] = make_float2(0.0f, 0.0f);
            g.d_conic[3 * i] = 0.0f;
            g.d_conic[3 * i + 1] = 0.0f;
            g.d_conic[3 * i + 2] = 0.0f;
            g.d_opacity[i] = 0.0f;
            g.d_color[3 * i] = 0.0f;
            g.d_color[3 * i + 1] = 0.0f;
            g.d_color[3 * i + 2] = 0.0f;
        }
    }
}

__global__ __launch_bounds__(kBlock) void raster_bwd_kernel(RasterArgs a, const float* t_final, const int32_t* n_contrib,
                                                            const float* dl, Grads gr) {
    __shared__ float2 s_xy[kBatch];
    __shared__ float4 s_co[kBatch];
    __shared__ float4 s_rgb[kBatch];
    __shared__ int32_t s_slot[kBatch];
    __shared__ int s_red[kBlock / kWave];
    const Lds s{s_xy, s_co, s_rgb, s_slot};
    const TileCtx c = tile_ctx(a, a.ranges);
    const size_t plane = (size_t)a.width * a.height;
    const size_t p = (size_t)c.py * a.width + c.px;
    Bwd b{};
    if (c.inside) {
        b.T = t_final[(size_t)c.v * plane + p];
        b.nc = n_contrib[(size_t)c.v * plane + p];
        b.g0 = dl[(size_t)(3 * c.v + 0) * plane + p];
        b.g1 = dl[(size_t)(3 * c.v + 1) * plane + p];
        b.g2 = dl[(size_t)(3 * c.v + 2) * plane + p];
    } else {
        b.T = 1.0f;
        b.nc = 0;
        b.g0 = b.g1 = b.g2 = 0.0f;
    }
    b.Tfin = b.T;
    b.B0 = b.B1 = b.B2 = 0.0f;
    const int maxnc = block_max(b.nc, s_red);
    for (int32_t bend = maxnc; bend > 0; bend -= kBatch) {
        const int32_t b0 = bend > kBatch ? bend - kBatch : 0;
        __syncthreads();
        if (b0 + (int32_t)threadIdx.x < bend) stage(a, c, s, threadIdx.x, b0 + threadIdx.x);
        __syncthreads();
        bwd_walk(a, c, s, 0, bend - b0, b0, b, gr);
    }
}

template <bool COUNT>
__global__ __launch_bounds__(kBlock) void raster_fused_kernel(RasterArgs a, int mode, const float* tgt, float scale,
                                                              float* image, float* loss_sum, Grads gr) {
    __shared__ float2 s_xy[kFusedEntries];
    __shared__ float4 s_co[kFusedEntries];
    __shared__ float4 s_rgb[kFusedEntries];
    __shared__ int32_t s_slot[kFusedEntries];
    __shared__ int s_red[kBlock / kWave];
    const Lds s{s_xy, s_co, s_rgb, s_slot};
    const TileCtx c = tile_ctx(a, a.ranges);
    const bool resident = c.n <= kFusedEntries;
    // forward
    Fwd f{1.0f, 0.0f, 0.0f, 0.0f, 0, !c.inside};
    Counts cnts{0, 0, 0};
    int32_t loaded = 0;  // resident entries staged so far
    for (int32_t b0 = 0; b0 < c.n; b0 += kBatch) {
        if (__syncthreads_count(f.done) == kBlock) break;
        const int32_t j = b0 + threadIdx.x;
        const int base = resident ? b0 : 0;
        if (j < c.n) stage(a, c, s, base + threadIdx.x, j);
        __syncthreads();
        const int cnt = min(kBatch, c.n - b0);
        fwd_walk<COUNT>(a, c, s, base, base + cnt, b0 - base, f, cnts);
        loaded = b0 + cnt;
    }
    if (COUNT) add_counters(a.counters, cnts);
    // loss gradient in registers
    const size_t plane = (size_t)a.width * a.height;
    const size_t p = (size_t)c.py * a.width + c.px;
    Bwd b{};
    b.T = f.T;
    b.Tfin = f.T;
    b.nc = c.inside ? f.last : 0;
    b.B0 = b.B1 = b.B2 = 0.0f;
    b.g0 = b.g1 = b.g2 = 0.0f;
    float lsum = 0.0f;
    if (c.inside) {
        const float C0 = fmaf(f.T, a.p.bg[0], f.C0);
        const float C1 = fmaf(f.T, a.p.bg[1], f.C1);
        const float C2 = fmaf(f.T, a.p.bg[2], f.C2);
        if (image) {
            image[(size_t)(3 * c.v + 0) * plane + p] = C0;
            image[(size_t)(3 * c.v + 1) * plane + p] = C1;
            image[(size_t)(3 * c.v + 2) * plane + p] = C2;
        }
        const float t0 = tgt[(size_t)(3 * c.v + 0) * plane + p];
        const float t1 = tgt[(size_t)(3 * c.v + 1) * plane + p];
        const float t2 = tgt[(size_t)(3 * c.v + 2) * plane + p];
        if (mode == GS_LOSS_L1) {
            const float d0 = C0 - t0, d1 = C1 - t1, d2 = C2 - t2;
            b.g0 = d0 > 0.0f ? scale : (d0 < 0.0f ? -scale : 0.0f);
            b.g1 = d1 > 0.0f ? scale : (d1 < 0.0f ? -scale : 0.0f);
            b.g2 = d2 > 0.0f ? scale : (d2 < 0.0f ? -scale : 0.0f);
            lsum = scale * (fabsf(d0) + fabsf(d1) + fabsf(d2));
        } else {
            b.g0 = t0;
            b.g1 = t1;
            b.g2 = t2;
        }
    }
    if (loss_sum && mode == GS_LOSS_L1) {
        lsum = wave_sum(lsum);
        if (c.lane == 0 && lsum != 0.0f) atomicAdd(loss_sum, lsum);
    }
    // backward
    const int maxnc = block_max(b.nc, s_red);
    if (resident) {
        // every entry below maxnc was staged by the forward (maxnc <= loaded)
        (void)loaded;
        bwd_walk(a, c, s, 0, maxnc, 0, b, gr);
    } else {
        for (int32_t bend = maxnc; bend > 0; bend -= kBatch) {
            const int32_t b0 = bend > kBatch ? bend - kBatch : 0;
            __syncthreads();
            if (b0 + (int32_t)threadIdx.x < bend) stage(a, c, s, threadIdx.x, b0 + threadIdx.x);
            __syncthreads();
            bwd_walk(a, c, s, 0, bend - b0, b0, b, gr);
        }
    }
}

}  // namespace

int32_t fused_lds_entries() { return kFusedEntries; }

hipError_t launch_raster_fwd(const RasterArgs& a, float* image, float* t_final, int32_t* n_contrib, hipStream_t s) {
    const unsigned nblocks = (unsigned)(a.V * a.tiles_x * a.tiles_y);
    if (a.counters)
        hipLaunchKernelGGL(raster_fwd_kernel<true>, dim3(nblocks), dim3(kBlock), 0, s, a, image, t_final, n_contrib);
    else
        hipLaunchKernelGGL(raster_fwd_kernel<false>, dim3(nblocks), dim3(kBlock), 0, s, a, image, t_final, n_contrib);
    return hipGetLastError();
}

hipError_t launch_loss_l1(int64_t n, const float* image, const float* target, float scale, float* dl, float* loss_sum,
                          hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(loss_l1_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, image, target, scale, dl,
                       loss_sum);
    return hipGetLastError();
}

hipError_t launch_zero_grads(const int32_t* vis_count, int32_t V, int32_t capacity, Grads g, hipStream_t s) {
    int blocks = (capacity + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_grads_kernel, dim3(blocks), dim3(256), 0, s, vis_count, V, capacity, g);
    return hipGetLastError();
}

hipError_t launch_raster_bwd(const RasterArgs& a, const float* /*image*/, const float* t_final, const int32_t* n_contrib,
                             const float* dl, Grads g, hipStream_t s) {
    hipError_t e = launch_zero_grads(a.vis_count, a.V, a.capacity, g, s);
    if (e != hipSuccess) return e;
    const unsigned nblocks = (unsigned)(a.V * a.tiles_x * a.tiles_y);
    hipLaunchKernelGGL(raster_bwd_kernel, dim3(nblocks), dim3(kBlock), 0, s, a, t_final, n_contrib, dl, g);
    return hipGetLastError();
}

hipError_t launch_raster_fused(const RasterArgs& a, int mode, const float* target_or_dl, float scale, float* image,
                               float* loss_sum, Grads g, hipStream_t s) {
    hipError_t e = launch_zero_grads(a.vis_count, a.V, a.capacity, g, s);
    if (e != hipSuccess) return e;
    const unsigned nblocks = (unsigned)(a.V * a.tiles_x * a.tiles_y);
    if (a.counters)
        hipLaunchKernelGGL(raster_fused_kernel<true>, dim3(nblocks), dim3(kBlock), 0, s, a, mode, target_or_dl, scale,
                           image, loss_sum, g);
    else
        hipLaunchKernelGGL(raster_fused_kernel<false>, dim3(nblocks), dim3(kBlock), 0, s, a, mode, target_or_dl, scale,
                           image, loss_sum, g);
    return hipGetLastError();
}

}  // namespace gsmi
