// A1: projection of 3D Gaussians into V views, with per-view culling and slot compaction.
//
// Two passes over the Gaussians, one thread per Gaussian, all V views per thread so the
// geometry (44 B per Gaussian) is read once per pass:
//   pass 1 counts the visible Gaussians of each 256-Gaussian block and view, and adds the
//          block's tile-instance count into the view's total;
//   an exclusive scan of the block counts gives each block its first slot per view;
//   pass 2 recomputes the same decisions (same code, same rounding) for the Gaussians that
//          pass 1 found in some view and writes the records of visible Gaussians at
//          slot = block offset + rank within the block, so slots follow ascending Gaussian
//          index, together with each slot's instance base (the same scan over the blocks'
//          tile-instance counts, plus a wave scan inside the block) and the packed 64-byte
//          record the rasterizers stage with one line per list entry.
// Spherical-harmonic coefficients (192 B per Gaussian at degree 3) are read only for Gaussians
// that some view sees (in a large scene most are outside every view): the counting pass checks
// at the first such view that they are bounded (which makes every colour finite) and flags the
// Gaussian, and the writing pass keeps a flagged Gaussian's coefficients in registers for all
// views.
#include "common.h"
#include "gauss.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;

struct Geo {
    float mx, my, mz;   // world mean
    float o;            // activated opacity
    float S[6];         // world covariance xx, xy, xz, yy, yz, zz
    bool ok;
};

struct Rec {
    float2 xy;
    float4 co;
    float3 rgb;
    float depth;
    ushort4 rect;
    int32_t ntiles;
};

__device__ __forceinline__ bool finitef(float x) { return isfinite(x); }

__device__ Geo load_geo(const ProjectArgs& a, int i) {
    const int n = a.n;
    Geo g;
    g.mx = a.means[i];
    g.my = a.means[n + i];
    g.mz = a.means[2 * n + i];
    const GaussFrame f = gauss_frame(a.log_scales[i], a.log_scales[n + i], a.log_scales[2 * n + i], a.quats[i],
                                     a.quats[n + i], a.quats[2 * n + i], a.quats[3 * n + i], a.logits[i],
                                     finitef(g.mx) && finitef(g.my) && finitef(g.mz));
    g.ok = f.ok;
    g.o = f.o;
#pragma unroll
    for (int k = 0; k < 6; k++) g.S[k] = f.S[k];
    return g;
}

// True when every SH coefficient of Gaussian i is finite and at most 1e30 in magnitude.  Every
// real SH basis value of degree <= 3 on the unit sphere is below 1 in magnitude, so the colour
// sum of at most 48 such terms then stays below 5e31 at every step of its evaluation: it is
// finite, and the colour cannot cull the Gaussian in any view.
template <int NK3>
__device__ __forceinline__ bool sh_bounded(const ProjectArgs& a, int i) {
    // bitwise and, unrolled: the loads are issued together (a short-circuit chain would
    // serialize them); a NaN compares false
    bool ok = true;
#pragma unroll 16
    for (int k = 0; k < NK3; k++) ok &= fabsf(a.sh[(size_t)k * a.n + i]) <= 1e30f;
    return ok;
}

// All per-view tests except the colour's finiteness, and the record without the colour.  Also
// returns the unit viewing direction.  Returns visibility so far.
__device__ bool project_geom(const ProjectArgs& a, const Geo& g, const CamDev& c, Rec& r, float3& dir) {
    if (!g.ok) return false;
    const ParamsDev& p = a.p;
    const float tx = fmaf(c.R[0], g.mx, fmaf(c.R[1], g.my, fmaf(c.R[2], g.mz, c.t[0])));
    const float ty = fmaf(c.R[3], g.mx, fmaf(c.R[4], g.my, fmaf(c.R[5], g.mz, c.t[1])));
    const float tz = fmaf(c.R[6], g.mx, fmaf(c.R[7], g.my, fmaf(c.R[8], g.mz, c.t[2])));
    if (!(tz > p.znear)) return false;
    // EWA: T = J W with J the Jacobian of the perspective map at the centre
    const float iz = 1.0f / tz;
    const float j00 = c.fx * iz, j02 = -c.fx * tx * iz * iz;
    const float j11 = c.fy * iz, j12 = -c.fy * ty * iz * iz;
    const float t00 = fmaf(j00, c.R[0], j02 * c.R[6]);
    const float t01 = fmaf(j00, c.R[1], j02 * c.R[7]);
    const float t02 = fmaf(j00, c.R[2], j02 * c.R[8]);
    const float t10 = fmaf(j11, c.R[3], j12 * c.R[6]);
    const float t11 = fmaf(j11, c.R[4], j12 * c.R[7]);
    const float t12 = fmaf(j11, c.R[5], j12 * c.R[8]);
    // U = Sigma T0^T, V = Sigma T1^T; Sigma2D = [[T0.U, T1.U], [T1.U, T1.V]]
    const float* S = g.S;
    const float u0 = fmaf(S[0], t00, fmaf(S[1], t01, S[2] * t02));
    const float u1 = fmaf(S[1], t00, fmaf(S[3], t01, S[4] * t02));
    const float u2 = fmaf(S[2], t00, fmaf(S[4], t01, S[5] * t02));
    const float v0 = fmaf(S[0], t10, fmaf(S[1], t11, S[2] * t12));
    const float v1 = fmaf(S[1], t10, fmaf(S[3], t11, S[4] * t12));
    const float v2 = fmaf(S[2], t10, fmaf(S[4], t11, S[5] * t12));
    const float ca = fmaf(t00, u0, fmaf(t01, u1, t02 * u2)) + p.eps2d;
    const float cb = fmaf(t10, u0, fmaf(t11, u1, t12 * u2));
    const float cc = fmaf(t10, v0, fmaf(t11, v1, t12 * v2)) + p.eps2d;
    const float det = ca * cc - cb * cb;
    if (!(det > 0.0f) || !finitef(det)) return false;
    const float idet = 1.0f / det;
    const float mx = fmaf(c.fx * tx, iz, c.cx);
    const float my = fmaf(c.fy * ty, iz, c.cy);
    // per-view frustum cull with a guard band: the projected centre must lie inside the image
    // widened by 15 % of its size on every side.  Beyond it lie the near-plane splats far off
    // axis, whose 2D covariance reaches 1e12 px^2: at image pixels their quadratic form cancels
    // terms of 1e8 and more, which float32 (records or arithmetic) cannot resolve.
    const float gx = kGuard * (float)c.width, gy = kGuard * (float)c.height;
    if (!(mx >= -gx && mx <= (float)c.width + gx && my >= -gy && my <= (float)c.height + gy)) return false;
    // opacity-aware box: o exp(-q/2) >= alpha_min  <=>  q <= 2 ln(o / alpha_min)
    if (!(g.o > p.alpha_min)) return false;
    const float Q = 2.0f * logf(g.o / p.alpha_min);
    const float ex = 1.001f * sqrtf(Q * ca);
    const float ey = 1.001f * sqrtf(Q * cc);
    const float lox = mx - ex - 0.5f, hix = mx + ex - 0.5f;
    const float loy = my - ey - 0.5f, hiy = my + ey - 0.5f;
    if (!(finitef(lox) && finitef(hix) && finitef(loy) && finitef(hiy))) return false;
    const float fu0 = fmaxf(0.0f, ceilf(lox)), fu1 = fminf((float)(c.width - 1), floorf(hix));
    const float fv0 = fmaxf(0.0f, ceilf(loy)), fv1 = fminf((float)(c.height - 1), floorf(hiy));
    if (!(fu0 <= fu1) || !(fv0 <= fv1)) return false;
    // viewing direction (the colour is evaluated by the caller)
    float idn;
    if (!view_dir(g.mx, g.my, g.mz, c.campos, &dir.x, &dir.y, &dir.z, &idn)) return false;
    r.xy = make_float2(mx, my);
    r.co = make_float4(cc * idet, -cb * idet, ca * idet, g.o);
    r.depth = tz;
    const int u0i = (int)fu0, u1i = (int)fu1, v0i = (int)fv0, v1i = (int)fv1;
    r.rect = make_ushort4((unsigned short)(u0i / kTile), (unsigned short)(v0i / kTile),
                          (unsigned short)(u1i / kTile), (unsigned short)(v1i / kTile));
    r.ntiles = (r.rect.z - r.rect.x + 1) * (r.rect.w - r.rect.y + 1);
    return true;
}

// Whether the colour of Gaussian i along dir is finite (the rare case of unbounded
// coefficients; kept out of line so that it does not hold registers in the counting loop).
template <int DEG>
__device__ __noinline__ bool colour_finite(const ProjectArgs& a, int i, float3 dir) {
    constexpr int NY = DEG == 0 ? 0 : (DEG == 1 ? 3 : (DEG == 2 ? 8 : 15));
    float Y[15];
    sh_basis(DEG, dir.x, dir.y, dir.z, Y);
    const float3 col = sh_eval(a.sh + i, a.n, NY, Y);
    return finitef(col.x) && finitef(col.y) && finitef(col.z);
}

template <int DEG>
// at most 80 registers: 6 waves per SIMD to hide the latency of the coefficient reads (95 otherwise)
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(6))) void project_count_kernel(ProjectArgs a) {
    constexpr int NY = DEG == 0 ? 0 : (DEG == 1 ? 3 : (DEG == 2 ? 8 : 15));
    __shared__ int s_cnt[kBlock / kWave];
    __shared__ int s_inst[kBlock / kWave];
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    Geo g;
    g.ok = false;
    if (i < a.n) g = load_geo(a, i);
    // the coefficients are checked at the first view that sees the Gaussian: most Gaussians of a
    // large scene are outside every view and their 192 bytes are never read
    bool bounded = true, checked = false, seen = false;
    const int nb = gridDim.x;
    // visible depth range of this thread over all views, as float32 bit patterns (depths are
    // above znear > 0, so the patterns order like the values)
    uint32_t dlo = 0xFFFFFFFFu, dhi = 0u;
    for (int v = 0; v < a.V; v++) {
        Rec r;
        r.ntiles = 0;
        float3 dir;
        bool vis = (i < a.n) && project_geom(a, g, a.cams.c[v], r, dir);
        if (vis && !checked) {
            bounded = sh_bounded<3 * (NY + 1)>(a, i);
            checked = true;
        }
        // some coefficient is huge or not finite: the colour itself decides
        if (vis && !bounded) vis = colour_finite<DEG>(a, i, dir);
        seen |= vis;
        if (vis) {
            dlo = min(dlo, __float_as_uint(r.depth));
            dhi = max(dhi, __float_as_uint(r.depth));
        }
        const unsigned long long m = __ballot(vis);
        int nt = vis ? r.ntiles : 0;
        for (int o = kWave / 2; o > 0; o >>= 1) nt += __shfl_xor(nt, o);
        if (lane == 0) {
            s_cnt[w] = __popcll(m);
            s_inst[w] = nt;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int c = 0, t = 0;
            for (int k = 0; k < kBlock / kWave; k++) {
                c += s_cnt[k];
                t += s_inst[k];
            }
            a.block_counts[v * nb + blockIdx.x] = c;
            a.block_counts[(a.V + v) * nb + blockIdx.x] = t;
        }
        __syncthreads();
    }
    if (i < a.n) a.seen[i] = seen ? 1 : 0;
    if (a.block_depth) {
        uint32_t nhi = ~dhi;
        for (int o = kWave / 2; o > 0; o >>= 1) {
            dlo = min(dlo, (uint32_t)__shfl_xor((int)dlo, o));
            nhi = min(nhi, (uint32_t)__shfl_xor((int)nhi, o));
        }
        // the count buffers of the view loop are free again after its last barrier
        if (lane == 0) {
            s_cnt[w] = (int)dlo;
            s_inst[w] = (int)nhi;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int k = 1; k < kBlock / kWave; k++) {
                dlo = min(dlo, (uint32_t)s_cnt[k]);
                nhi = min(nhi, (uint32_t)s_inst[k]);
            }
            a.block_depth[blockIdx.x] = make_uint2(dlo, nhi);
        }
    }
}

template <int DEG>
__global__ __launch_bounds__(kBlock) void project_write_kernel(ProjectArgs a) {
    constexpr int NY = DEG == 0 ? 0 : (DEG == 1 ? 3 : (DEG == 2 ? 8 : 15));
    constexpr int NC = 3 * (NY + 1);
    __shared__ int s_cnt[kBlock / kWave];
    __shared__ int s_inst[kBlock / kWave];
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    if (blockIdx.x == 0 && threadIdx.x < a.V) a.vis_count[threadIdx.x] = a.row_totals[threadIdx.x];
    // a block whose Gaussians no view sees (most blocks of a large scene) writes nothing
    {
        bool any = false;
        for (int v = 0; v < a.V; v++) any |= a.block_counts[v * gridDim.x + blockIdx.x] > 0;
        if (!any) return;
    }
    Geo g;
    g.ok = false;
    // the Gaussian's SH coefficients (row k*3 + channel), read once for all views, and only for
    // Gaussians that the counting pass found in some view: those outside every view (most of a
    // large scene) cost neither coefficient reads nor projection here
    float coef[NC];
#pragma unroll
    for (int k = 0; k < NC; k++) coef[k] = 0.0f;
    if (i < a.n && a.seen[i]) {
        g = load_geo(a, i);
        if (g.ok) {
#pragma unroll
            for (int k = 0; k < NC; k++) coef[k] = a.sh[(size_t)k * a.n + i];
        }
    }
    const int nb = gridDim.x;
    int view_inst = 0;  // instances of the earlier views
    for (int v = 0; v < a.V; v++) {
        Rec r;
        r.ntiles = 0;
        float3 dir;
        bool vis = (i < a.n) && project_geom(a, g, a.cams.c[v], r, dir);
        if (vis) {
            // colour along the viewing direction: DC + sum_k sh_k Y_k, in the order of sh_eval
            float Y[15];
            sh_basis(DEG, dir.x, dir.y, dir.z, Y);
            float3 col = make_float3(coef[0], coef[1], coef[2]);
#pragma unroll
            for (int k = 0; k < NY; k++) {
                col.x = fmaf(coef[3 * (k + 1) + 0], Y[k], col.x);
                col.y = fmaf(coef[3 * (k + 1) + 1], Y[k], col.y);
                col.z = fmaf(coef[3 * (k + 1) + 2], Y[k], col.z);
            }
            vis = finitef(col.x) && finitef(col.y) && finitef(col.z);
            r.rgb = make_float3(fmaxf(0.0f, col.x), fmaxf(0.0f, col.y), fmaxf(0.0f, col.z));
        }
        const unsigned long long m = __ballot(vis);
        // inclusive scan of the tile counts over the wave
        const int nt = vis ? r.ntiles : 0;
        int inc = nt;
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        if (lane == 0) s_cnt[w] = __popcll(m);
        if (lane == kWave - 1) s_inst[w] = inc;
        __syncthreads();
        int off = a.block_offsets[v * nb + blockIdx.x];
        int ioff = view_inst + a.block_offsets[(a.V + v) * nb + blockIdx.x];
        for (int k = 0; k < w; k++) {
            off += s_cnt[k];
            ioff += s_inst[k];
        }
        __syncthreads();
        if (vis) {
            const int slot = off + __popcll(m & ((1ull << lane) - 1ull));
            const int base = ioff + inc - nt;
            const size_t idx = (size_t)v * a.capacity + slot;
            a.vis_ids[idx] = i;
            a.mean2d[idx] = r.xy;
            a.conic_opacity[idx] = r.co;
            a.color[3 * idx + 0] = r.rgb.x;
            a.color[3 * idx + 1] = r.rgb.y;
            a.color[3 * idx + 2] = r.rgb.z;
            a.depth[idx] = r.depth;
            a.tile_rect[idx] = r.rect;
            a.n_tiles[idx] = r.ntiles;
            a.inst_base[idx] = base;
            float4* rec = a.raster_rec + 4 * idx;
            rec[0] = make_float4(r.xy.x, r.xy.y, r.co.x, r.co.y);
            rec[1] = make_float4(r.co.z, r.co.w, r.rgb.x, r.rgb.y);
            rec[2] = make_float4(r.rgb.z, __int_as_float((int)r.rect.x | ((int)r.rect.y << 16)),
                                 __int_as_float((int)r.rect.z | ((int)r.rect.w << 16)), __int_as_float(base));
            rec[3] = make_float4(r.depth, __int_as_float(r.ntiles), 0.0f, 0.0f);
        }
        view_inst += a.row_totals[a.V + v];
    }
}

// inst_count[v] = the 64-bit sum of row V + v of the block counts (one block per view; 64 bits,
// so that a total past 2^31 is reported as such and refused by the binning call).
// 1024 threads, four independent loads per step: a large scene has ~10^5 blocks per row, and a
// loop of dependent loads over them would take hundreds of microseconds.
constexpr int kSumBlock = 1024;

__global__ __launch_bounds__(kSumBlock) void inst_total_kernel(const int32_t* block_counts, int32_t V, int32_t nb,
                                                               int64_t* inst_count) {
    __shared__ long long s_part[kSumBlock / kWave];
    const int v = blockIdx.x;
    const int32_t* row = block_counts + (size_t)(V + v) * nb;
    long long t = 0;
    for (int32_t b0 = 0; b0 < nb; b0 += 4 * kSumBlock) {
        int x[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int32_t b = b0 + u * kSumBlock + (int)threadIdx.x;
            x[u] = b < nb ? row[b] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; u++) t += x[u];
    }
    for (int o = kWave / 2; o > 0; o >>= 1) t += __shfl_xor(t, o);
    if ((threadIdx.x & (kWave - 1)) == 0) s_part[threadIdx.x / kWave] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        long long sum = 0;
        for (int k = 0; k < kSumBlock / kWave; k++) sum += s_part[k];
        inst_count[v] = sum;
    }
}

// The count summary (one block): visible slots per view from the block scans, instances per
// view from inst_total_kernel, and the visible depth range from the per-block ranges.
__global__ __launch_bounds__(kSumBlock) void count_summary_kernel(const int32_t* row_totals,
                                                                  const int64_t* inst_count, int32_t V,
                                                                  const uint2* block_depth, int32_t nb,
                                                                  CountSummary* out) {
    __shared__ uint32_t s_lo[kSumBlock / kWave], s_nhi[kSumBlock / kWave];
    if ((int)threadIdx.x < V) {
        out->vis[threadIdx.x] = row_totals[threadIdx.x];
        out->inst[threadIdx.x] = inst_count[threadIdx.x];
    }
    uint32_t lo = 0xFFFFFFFFu, nhi = 0xFFFFFFFFu;
    for (int32_t k0 = 0; k0 < nb; k0 += 4 * kSumBlock) {
        uint2 x[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int32_t k = k0 + u * kSumBlock + (int)threadIdx.x;
            x[u] = k < nb ? block_depth[k] : make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            lo = min(lo, x[u].x);
            nhi = min(nhi, x[u].y);
        }
    }
    for (int o = kWave / 2; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
        nhi = min(nhi, (uint32_t)__shfl_xor((int)nhi, o));
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
        s_lo[threadIdx.x / kWave] = lo;
        s_nhi[threadIdx.x / kWave] = nhi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < kSumBlock / kWave; k++) {
            lo = min(lo, s_lo[k]);
            nhi = min(nhi, s_nhi[k]);
        }
        out->bits[0] = lo;
        out->bits[1] = nhi;
    }
}

}  // namespace

static int32_t project_blocks(int32_t n) { return (n + kBlock - 1) / kBlock; }

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

size_t project_ws_bytes(int32_t n, int32_t V) {
    const int32_t nb = project_blocks(n > 0 ? n : 1);
    return 2 * align256(sizeof(int32_t) * (size_t)nb * 2 * V) + align256(sizeof(int32_t) * 2 * V) +
           align256(scan_partials_bytes(nb, 2 * V)) + align256(sizeof(uint2) * (size_t)nb) +
           align256(sizeof(CountSummary)) + align256((size_t)nb * kBlock);
}

hipError_t launch_project_count(const ProjectArgs& a0, hipStream_t s) {
    ProjectArgs a = a0;
    const int32_t nb = project_blocks(a.n > 0 ? a.n : 1);
    switch (a.p.sh_degree) {
        case 0: hipLaunchKernelGGL(project_count_kernel<0>, dim3(nb), dim3(kBlock), 0, s, a); break;
        case 1: hipLaunchKernelGGL(project_count_kernel<1>, dim3(nb), dim3(kBlock), 0, s, a); break;
        case 2: hipLaunchKernelGGL(project_count_kernel<2>, dim3(nb), dim3(kBlock), 0, s, a); break;
        default: hipLaunchKernelGGL(project_count_kernel<3>, dim3(nb), dim3(kBlock), 0, s, a); break;
    }
    hipLaunchKernelGGL(inst_total_kernel, dim3(a.V), dim3(kSumBlock), 0, s, a.block_counts, a.V, nb, a.inst_count);
    hipError_t e = launch_scan_rows(a.block_counts, a.block_offsets, a.row_totals, nb, 2 * a.V, a.scan_partials, s);
    if (e != hipSuccess) return e;
    if (a.block_depth)
        hipLaunchKernelGGL(count_summary_kernel, dim3(1), dim3(kSumBlock), 0, s, a.row_totals, a.inst_count, a.V,
                           a.block_depth, nb, a.summary);
    return hipGetLastError();
}

hipError_t launch_project_write(const ProjectArgs& a0, hipStream_t s) {
    ProjectArgs a = a0;
    const int32_t nb = project_blocks(a.n > 0 ? a.n : 1);
    switch (a.p.sh_degree) {
        case 0: hipLaunchKernelGGL(project_write_kernel<0>, dim3(nb), dim3(kBlock), 0, s, a); break;
        case 1: hipLaunchKernelGGL(project_write_kernel<1>, dim3(nb), dim3(kBlock), 0, s, a); break;
        case 2: hipLaunchKernelGGL(project_write_kernel<2>, dim3(nb), dim3(kBlock), 0, s, a); break;
        default: hipLaunchKernelGGL(project_write_kernel<3>, dim3(nb), dim3(kBlock), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace gsmi
