// A1: projection of 3D Gaussians into V views, with per-view culling and slot compaction.
//
// Two passes over the Gaussians, one thread per Gaussian, all V views per thread so the
// geometry (44 B per Gaussian) is read once per pass:
//   pass 1 counts the visible Gaussians of each wavefront (64 consecutive Gaussians) and view,
//          and the wavefront's tile instances per view: wave ballots and reductions only, no
//          workgroup barrier;
//   an exclusive scan of the wavefront counts gives each wavefront its first slot per view;
//   pass 2 recomputes the same decisions (same code, same rounding) for the Gaussians that
//          pass 1 found in some view and writes the records of visible Gaussians at
//          slot = wavefront offset + rank within the wavefront, so slots follow ascending
//          Gaussian index, together with each slot's instance base (the same scan over the
//          wavefronts' tile-instance counts, plus a wave scan) and the packed 64-byte record the
//          rasterizers stage with one line per list entry.  No barrier either.
// The mean alone decides the near plane and the frustum guard of every view, so pass 1 reads
// the other 32 B of geometry only for Gaussians some view keeps.  Visibility never depends on
// the colour (a Gaussian whose colour is not finite in a view is kept there, transparent: its
// record carries opacity 0 and colour 0), so pass 1 reads no spherical-harmonic coefficient at
// all, and pass 2 reads them (192 B per Gaussian at degree 3) only for Gaussians that some view
// sees, once for all views.
#include "common.h"
#include "gauss.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;

// Wavefronts of 64 consecutive Gaussians: the unit of the counts and of the slot offsets.
__host__ __device__ __forceinline__ int32_t project_waves(int32_t n) { return n > 0 ? (n + 63) / 64 : 1; }

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

// The rest of a Gaussian's geometry (activations, world covariance) for a mean already read.
__device__ Geo load_geo_rest(const ProjectArgs& a, int i, float mx, float my, float mz) {
    const int n = a.n;
    Geo g;
    g.mx = mx;
    g.my = my;
    g.mz = mz;
    const GaussFrame f = gauss_frame(a.log_scales[i], a.log_scales[n + i], a.log_scales[2 * n + i], a.quats[i],
                                     a.quats[n + i], a.quats[2 * n + i], a.quats[3 * n + i], a.logits[i],
                                     finitef(g.mx) && finitef(g.my) && finitef(g.mz));
    g.ok = f.ok;
    g.o = f.o;
#pragma unroll
    for (int k = 0; k < 6; k++) g.S[k] = f.S[k];
    return g;
}

// The same from the eleven raw values (mean, log-scales, quaternion w x y z, opacity logit).
__device__ __forceinline__ Geo geo_from(const float raw[11]) {
    Geo g;
    g.mx = raw[0];
    g.my = raw[1];
    g.mz = raw[2];
    const GaussFrame f = gauss_frame(raw[3], raw[4], raw[5], raw[6], raw[7], raw[8], raw[9], raw[10],
                                     finitef(g.mx) && finitef(g.my) && finitef(g.mz));
    g.ok = f.ok;
    g.o = f.o;
#pragma unroll
    for (int k = 0; k < 6; k++) g.S[k] = f.S[k];
    return g;
}

// The camera-space centre of a mean and its projection, with the decisions taken from the mean
// alone: the near plane, and the per-view frustum cull with a guard band (the projected centre
// must lie inside the image widened by 15 % of its size on every side).  Beyond the guard lie
// the near-plane splats far off axis, whose 2D covariance reaches 1e12 px^2: at image pixels
// their quadratic form cancels terms of 1e8 and more, which float32 (records or arithmetic)
// cannot resolve.  The projection and the counting pass's early test both call this, so they
// decide identically.
struct Centre {
    float tx, ty, tz, iz, mx, my;
};

// A conservative form of view_centre's tests without the division: false only when the
// centre lies behind the near plane or clearly (by 1e-3 of the compared magnitudes, far above
// the float32 rounding of either form) outside the guard band, so that view_centre would fail
// too.  With tz > 0 the guard test  -g <= fx tx / tz + cx <= W + g  reads
// (-g - cx) tz <= fx tx <= (W + g - cx) tz, and likewise in y.
__device__ __forceinline__ bool view_centre_maybe(const CamDev& c, float znear, float wx, float wy, float wz) {
    const float tx = fmaf(c.R[0], wx, fmaf(c.R[1], wy, fmaf(c.R[2], wz, c.t[0])));
    const float ty = fmaf(c.R[3], wx, fmaf(c.R[4], wy, fmaf(c.R[5], wz, c.t[1])));
    const float tz = fmaf(c.R[6], wx, fmaf(c.R[7], wy, fmaf(c.R[8], wz, c.t[2])));
    if (!(tz > znear)) return false;
    const float gx = kGuard * (float)c.width, gy = kGuard * (float)c.height;
    const float u = c.fx * tx, v = c.fy * ty;
    const float ulo = (-gx - c.cx) * tz, uhi = ((float)c.width + gx - c.cx) * tz;
    const float vlo = (-gy - c.cy) * tz, vhi = ((float)c.height + gy - c.cy) * tz;
    const float su = 1e-3f * (fabsf(u) + fabsf(ulo) + fabsf(uhi)), sv = 1e-3f * (fabsf(v) + fabsf(vlo) + fabsf(vhi));
    // a NaN anywhere leaves the comparisons false: kept, and the exact test decides
    return !(u < ulo - su || u > uhi + su || v < vlo - sv || v > vhi + sv);
}

__device__ __forceinline__ bool view_centre(const CamDev& c, float znear, float wx, float wy, float wz, Centre& ce) {
    ce.tx = fmaf(c.R[0], wx, fmaf(c.R[1], wy, fmaf(c.R[2], wz, c.t[0])));
    ce.ty = fmaf(c.R[3], wx, fmaf(c.R[4], wy, fmaf(c.R[5], wz, c.t[1])));
    ce.tz = fmaf(c.R[6], wx, fmaf(c.R[7], wy, fmaf(c.R[8], wz, c.t[2])));
    if (!(ce.tz > znear)) return false;
    ce.iz = 1.0f / ce.tz;
    ce.mx = fmaf(c.fx * ce.tx, ce.iz, c.cx);
    ce.my = fmaf(c.fy * ce.ty, ce.iz, c.cy);
    const float gx = kGuard * (float)c.width, gy = kGuard * (float)c.height;
    return ce.mx >= -gx && ce.mx <= (float)c.width + gx && ce.my >= -gy && ce.my <= (float)c.height + gy;
}

// All per-view tests except the colour's finiteness, and the record without the colour.  Also
// returns the unit viewing direction.  Returns visibility so far.
__device__ bool project_geom(const ProjectArgs& a, const Geo& g, const CamDev& c, Rec& r, float3& dir) {
    if (!g.ok) return false;
    const ParamsDev& p = a.p;
    Centre ce;
    if (!view_centre(c, p.znear, g.mx, g.my, g.mz, ce)) return false;
    const float tx = ce.tx, ty = ce.ty, tz = ce.tz, iz = ce.iz;
    // EWA: T = J W with J the Jacobian of the perspective map at the centre
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
    const float mx = ce.mx, my = ce.my;
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

__device__ __forceinline__ int wave_sum_i(int x) {
    for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ __launch_bounds__(kBlock) void project_count_kernel(ProjectArgs a) {
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t nw = project_waves(a.n);
    const int32_t gw = (int32_t)(i / kWave);  // this wavefront's index over all Gaussians
    if (gw >= nw) return;                     // whole wavefronts past the last Gaussian
    // the mean alone decides the near plane and the frustum guard of every view; the remaining
    // 32 bytes of geometry are read only for Gaussians whose centre some view keeps (in a large
    // scene most Gaussians lie outside every view)
    uint32_t vmask = 0u;
    float wx = 0.0f, wy = 0.0f, wz = 0.0f;
    if (i < a.n) {
        wx = a.means[i];
        wy = a.means[a.n + i];
        wz = a.means[2 * a.n + i];
        for (int v = 0; v < a.V; v++)
            if (view_centre_maybe(a.cams.c[v], a.p.znear, wx, wy, wz)) vmask |= 1u << v;
    }
    if (__ballot(vmask != 0u) == 0ull) {
        // no view keeps any centre of this wavefront (most of a large scene): zero counts, no
        // seen flags, an empty depth range
        if (lane < 2 * a.V) a.block_counts[(size_t)lane * nw + gw] = 0;
        if (i < a.n) a.seen[i] = 0;
        if (a.block_depth && lane == 0) a.block_depth[gw] = make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
        return;
    }
    Geo g;
    g.ok = false;
    if (vmask) g = load_geo_rest(a, i, wx, wy, wz);
    bool seen = false;
    // visible depth range of this thread over all views, as float32 bit patterns (depths are
    // above znear > 0, so the patterns order like the values)
    uint32_t dlo = 0xFFFFFFFFu, dhi = 0u;
    for (int v = 0; v < a.V; v++) {
        Rec r;
        r.ntiles = 0;
        float3 dir;
        const bool vis = ((vmask >> v) & 1u) && project_geom(a, g, a.cams.c[v], r, dir);
        seen |= vis;
        if (vis) {
            dlo = min(dlo, __float_as_uint(r.depth));
            dhi = max(dhi, __float_as_uint(r.depth));
        }
        const unsigned long long m = __ballot(vis);
        const int nt = wave_sum_i(vis ? r.ntiles : 0);
        if (lane == 0) {
            a.block_counts[(size_t)v * nw + gw] = __popcll(m);
            a.block_counts[(size_t)(a.V + v) * nw + gw] = nt;
        }
    }
    if (i < a.n) a.seen[i] = seen ? 1 : 0;
    if (a.block_depth) {
        uint32_t nhi = ~dhi;
        for (int o = kWave / 2; o > 0; o >>= 1) {
            dlo = min(dlo, (uint32_t)__shfl_xor((int)dlo, o));
            nhi = min(nhi, (uint32_t)__shfl_xor((int)nhi, o));
        }
        if (lane == 0) a.block_depth[gw] = make_uint2(dlo, nhi);
    }
}

template <int DEG>
__global__ __launch_bounds__(kBlock) void project_write_kernel(ProjectArgs a) {
    constexpr int NY = DEG == 0 ? 0 : (DEG == 1 ? 3 : (DEG == 2 ? 8 : 15));
    constexpr int NC = 3 * (NY + 1);
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t nw = project_waves(a.n);
    const int32_t gw = (int32_t)(i / kWave);
    if (blockIdx.x == 0 && threadIdx.x < a.V) a.vis_count[threadIdx.x] = a.row_totals[threadIdx.x];
    if (gw >= nw) return;
    // a wavefront whose Gaussians no view sees (most of a large scene) writes nothing: its
    // per-view counts in one load, one view per lane (V <= 16)
    const int cnt_raw = a.block_counts[(size_t)min(lane, a.V - 1) * nw + gw];
    if (__ballot(lane < a.V && cnt_raw > 0) == 0ull) return;
    Geo g;
    g.ok = false;
    // the Gaussian's SH coefficients (row k*3 + channel), read once for all views, and only for
    // Gaussians that the counting pass found in some view: those outside every view (most of a
    // large scene) cost neither coefficient reads nor projection here
    float coef[NC];
#pragma unroll
    for (int k = 0; k < NC; k++) coef[k] = 0.0f;
    if (i < a.n && a.seen[i]) {
        // A seen Gaussian's geometry is valid (the counting pass ran this same code on it), so
        // the coefficient loads need not wait for that check.  Geometry loads first, then the
        // coefficients (an empty asm with a memory clobber between them keeps that order): the
        // covariance needs only the geometry, whose loads complete first, so it is built while
        // the coefficients arrive.
        float raw[11];
#pragma unroll
        for (int k = 0; k < 3; k++) raw[k] = a.means[(size_t)k * a.n + i];
#pragma unroll
        for (int k = 0; k < 3; k++) raw[3 + k] = a.log_scales[(size_t)k * a.n + i];
#pragma unroll
        for (int k = 0; k < 4; k++) raw[6 + k] = a.quats[(size_t)k * a.n + i];
        raw[10] = a.logits[i];
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < NC; k++) coef[k] = a.sh[(size_t)k * a.n + i];
        g = geo_from(raw);
    }
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
            r.rgb = make_float3(fmaxf(0.0f, col.x), fmaxf(0.0f, col.y), fmaxf(0.0f, col.z));
            if (!(finitef(col.x) && finitef(col.y) && finitef(col.z))) {
                // no colour: kept in the view, transparent (nothing ever blends it)
                r.rgb = make_float3(0.0f, 0.0f, 0.0f);
                r.co.w = 0.0f;
            }
        }
        const unsigned long long m = __ballot(vis);
        // inclusive scan of the tile counts over the wave
        const int nt = vis ? r.ntiles : 0;
        int inc = nt;
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        if (vis) {
            const int slot = a.block_offsets[(size_t)v * nw + gw] + __popcll(m & ((1ull << lane) - 1ull));
            const int base = view_inst + a.block_offsets[(size_t)(a.V + v) * nw + gw] + inc - nt;
            const size_t idx = (size_t)v * a.capacity + slot;
            a.vis_ids[idx] = i;
            // optional copies of values the packed record also holds (kernel arguments: the
            // tests are uniform)
            if (a.mean2d) a.mean2d[idx] = r.xy;
            if (a.conic_opacity) a.conic_opacity[idx] = r.co;
            if (a.color) {
                a.color[3 * idx + 0] = r.rgb.x;
                a.color[3 * idx + 1] = r.rgb.y;
                a.color[3 * idx + 2] = r.rgb.z;
            }
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

// The per-view instance totals in 64 bits (so that a total past 2^31 is reported as such and
// refused by the binning call) and the visible depth range, in two steps: kParts workgroups per
// row each reduce a strided share of the wavefront counts (rows V..2V-1) or, in row V, of the
// wavefront depth ranges, then one workgroup adds the partials up.  Every workgroup keeps many
// independent loads in flight: a large scene has ~10^6 wavefronts per row.
constexpr int kParts = 128;
constexpr int kSumBlock = 256;

__global__ __launch_bounds__(kSumBlock) void count_partials_kernel(const int32_t* block_counts, int32_t V, int32_t nw,
                                                                   const uint2* block_depth, int64_t* inst_partials,
                                                                   uint2* depth_partials) {
    __shared__ long long s_sum[kSumBlock / kWave];
    __shared__ uint32_t s_lo[kSumBlock / kWave], s_nhi[kSumBlock / kWave];
    const int v = blockIdx.y;
    const int32_t stride = kParts * kSumBlock;
    const int32_t first = blockIdx.x * kSumBlock + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    if (v < V) {
        const int32_t* row = block_counts + (size_t)(V + v) * nw;
        long long t = 0;
        for (int32_t k = first; k < nw; k += 4 * stride) {
            int x[4];
#pragma unroll
            for (int u = 0; u < 4; u++) x[u] = k + u * stride < nw ? row[k + u * stride] : 0;
#pragma unroll
            for (int u = 0; u < 4; u++) t += x[u];
        }
        for (int o = kWave / 2; o > 0; o >>= 1) t += __shfl_xor(t, o);
        if (lane == 0) s_sum[w] = t;
        __syncthreads();
        if (threadIdx.x == 0) {
            long long sum = 0;
            for (int k = 0; k < kSumBlock / kWave; k++) sum += s_sum[k];
            inst_partials[(size_t)v * kParts + blockIdx.x] = sum;
        }
    } else if (block_depth) {
        uint32_t lo = 0xFFFFFFFFu, nhi = 0xFFFFFFFFu;
        for (int32_t k = first; k < nw; k += 4 * stride) {
            uint2 x[4];
#pragma unroll
            for (int u = 0; u < 4; u++)
                x[u] = k + u * stride < nw ? block_depth[k + u * stride] : make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
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
        if (lane == 0) {
            s_lo[w] = lo;
            s_nhi[w] = nhi;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int k = 1; k < kSumBlock / kWave; k++) {
                lo = min(lo, s_lo[k]);
                nhi = min(nhi, s_nhi[k]);
            }
            depth_partials[blockIdx.x] = make_uint2(lo, nhi);
        }
    }
}

// One workgroup: inst_count[v] from the partials; with `out`, the count summary (visible slots
// per view from the scans, instances per view, the visible depth range).
__global__ __launch_bounds__(kSumBlock) void count_summary_kernel(const int32_t* row_totals, const int64_t* inst_partials,
                                                                  const uint2* depth_partials, int32_t V,
                                                                  int64_t* inst_count, CountSummary* out) {
    if ((int)threadIdx.x < V) {
        const int v = threadIdx.x;
        long long sum = 0;
        for (int k = 0; k < kParts; k++) sum += inst_partials[(size_t)v * kParts + k];
        inst_count[v] = sum;
        if (out) {
            out->vis[v] = row_totals[v];
            out->inst[v] = sum;
        }
    }
    if (out && threadIdx.x == kSumBlock - 1) {
        uint32_t lo = 0xFFFFFFFFu, nhi = 0xFFFFFFFFu;
        for (int k = 0; k < kParts; k++) {
            lo = min(lo, depth_partials[k].x);
            nhi = min(nhi, depth_partials[k].y);
        }
        out->bits[0] = lo;
        out->bits[1] = nhi;
    }
}

}  // namespace

static int32_t project_blocks(int32_t n) { return (n + kBlock - 1) / kBlock; }

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// The carving order of the projection's workspace (256-byte aligned pieces): wavefront counts,
// their scans, row totals, scan partials, wavefront depth ranges, the count summary, the seen
// flags, the instance partials, the depth partials.
size_t project_ws_bytes(int32_t n, int32_t V) {
    const int32_t nw = project_waves(n);
    return 2 * align256(sizeof(int32_t) * (size_t)nw * 2 * V) + align256(sizeof(int32_t) * 2 * V) +
           align256(scan_partials_bytes(nw, 2 * V)) + align256(sizeof(uint2) * (size_t)nw) +
           align256(sizeof(CountSummary)) + align256((size_t)nw * kWave) +
           align256(sizeof(int64_t) * (size_t)V * kParts) + align256(sizeof(uint2) * kParts);
}

int32_t project_count_waves(int32_t n) { return project_waves(n); }
int32_t project_partials() { return kParts; }

hipError_t launch_project_count(const ProjectArgs& a0, hipStream_t s) {
    ProjectArgs a = a0;
    const int32_t nb = project_blocks(a.n > 0 ? a.n : 1);
    const int32_t nw = project_waves(a.n);
    hipLaunchKernelGGL(project_count_kernel, dim3(nb), dim3(kBlock), 0, s, a);
    hipLaunchKernelGGL(count_partials_kernel, dim3(kParts, a.V + 1), dim3(kSumBlock), 0, s, a.block_counts, a.V, nw,
                       a.block_depth, a.inst_partials, a.depth_partials);
    hipError_t e = launch_scan_rows(a.block_counts, a.block_offsets, a.row_totals, nw, 2 * a.V, a.scan_partials, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(count_summary_kernel, dim3(1), dim3(kSumBlock), 0, s, a.row_totals, a.inst_partials,
                       a.depth_partials, a.V, a.inst_count, a.block_depth ? a.summary : nullptr);
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
