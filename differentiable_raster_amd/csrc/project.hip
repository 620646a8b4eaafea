// A1: projection of 3D Gaussians into V views, with per-view culling and slot compaction.
//
// Two passes over the Gaussians, one thread per Gaussian, all V views per thread so the
// geometry (44 B per Gaussian) is read once per pass:
//   pass 1 counts the visible Gaussians of each 256-Gaussian block and view, and adds the
//          block's tile-instance count into the view's total;
//   an exclusive scan of the block counts gives each block its first slot per view;
//   pass 2 recomputes the same decisions (same code, same rounding) and writes the records of
//          visible Gaussians at slot = block offset + rank within the block, so slots follow
//          ascending Gaussian index.
// Spherical-harmonic coefficients (192 B per Gaussian at degree 3) are read only for
// Gaussians that pass every geometric test in a view; later views hit the cache.
#include "common.h"

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
    const float l0 = a.log_scales[i], l1 = a.log_scales[n + i], l2 = a.log_scales[2 * n + i];
    float qw = a.quats[i], qx = a.quats[n + i], qy = a.quats[2 * n + i], qz = a.quats[3 * n + i];
    const float logit = a.logits[i];
    g.ok = finitef(g.mx) && finitef(g.my) && finitef(g.mz) && finitef(l0) && finitef(l1) && finitef(l2) &&
           finitef(qw) && finitef(qx) && finitef(qy) && finitef(qz) && finitef(logit);
    // activations: sigmoid opacity, exponential scales, normalized quaternion
    g.o = 1.0f / (1.0f + expf(-logit));
    const float s0 = expf(l0), s1 = expf(l1), s2 = expf(l2);
    const float qn = sqrtf(qw * qw + qx * qx + qy * qy + qz * qz);
    g.ok = g.ok && qn > 0.0f;
    const float inv = 1.0f / qn;
    qw *= inv;
    qx *= inv;
    qy *= inv;
    qz *= inv;
    // rotation matrix of (w, x, y, z), columns scaled by s: M = R diag(s); Sigma = M M^T
    const float r00 = 1.0f - 2.0f * (qy * qy + qz * qz), r01 = 2.0f * (qx * qy - qw * qz), r02 = 2.0f * (qx * qz + qw * qy);
    const float r10 = 2.0f * (qx * qy + qw * qz), r11 = 1.0f - 2.0f * (qx * qx + qz * qz), r12 = 2.0f * (qy * qz - qw * qx);
    const float r20 = 2.0f * (qx * qz - qw * qy), r21 = 2.0f * (qy * qz + qw * qx), r22 = 1.0f - 2.0f * (qx * qx + qy * qy);
    const float m00 = r00 * s0, m01 = r01 * s1, m02 = r02 * s2;
    const float m10 = r10 * s0, m11 = r11 * s1, m12 = r12 * s2;
    const float m20 = r20 * s0, m21 = r21 * s1, m22 = r22 * s2;
    g.S[0] = fmaf(m00, m00, fmaf(m01, m01, m02 * m02));
    g.S[1] = fmaf(m00, m10, fmaf(m01, m11, m02 * m12));
    g.S[2] = fmaf(m00, m20, fmaf(m01, m21, m02 * m22));
    g.S[3] = fmaf(m10, m10, fmaf(m11, m11, m12 * m12));
    g.S[4] = fmaf(m10, m20, fmaf(m11, m21, m12 * m22));
    g.S[5] = fmaf(m20, m20, fmaf(m21, m21, m22 * m22));
    return g;
}

// Real orthonormal spherical harmonics (textbook Cartesian forms, no Condon-Shortley phase),
// summed with the coefficients of Gaussian i; the DC rows are the base colour.
__device__ float3 sh_colour(const ProjectArgs& a, int i, float x, float y, float z) {
    const int n = a.n;
    const float* sh = a.sh;
    float3 c;
    c.x = sh[0 * n + i];
    c.y = sh[1 * n + i];
    c.z = sh[2 * n + i];
    const int deg = a.p.sh_degree;
    if (deg < 1) return c;
    float Y[15];
    Y[0] = 0.4886025119029199f * y;  // sqrt(3/(4 pi)) (y, z, x)
    Y[1] = 0.4886025119029199f * z;
    Y[2] = 0.4886025119029199f * x;
    int nk = 3;
    if (deg >= 2) {
        Y[3] = 1.0925484305920792f * x * y;                // 1/2 sqrt(15/pi) xy
        Y[4] = 1.0925484305920792f * y * z;                // 1/2 sqrt(15/pi) yz
        Y[5] = 0.31539156525252005f * (3.0f * z * z - 1.0f);  // 1/4 sqrt(5/pi) (3z^2 - 1)
        Y[6] = 1.0925484305920792f * x * z;                // 1/2 sqrt(15/pi) xz
        Y[7] = 0.5462742152960396f * (x * x - y * y);      // 1/4 sqrt(15/pi) (x^2 - y^2)
        nk = 8;
    }
    if (deg >= 3) {
        Y[8] = 0.5900435899266435f * y * (3.0f * x * x - y * y);   // 1/4 sqrt(35/(2pi))
        Y[9] = 2.890611442640554f * x * y * z;                     // 1/2 sqrt(105/pi)
        Y[10] = 0.4570457994644658f * y * (5.0f * z * z - 1.0f);   // 1/4 sqrt(21/(2pi))
        Y[11] = 0.3731763325901154f * z * (5.0f * z * z - 3.0f);   // 1/4 sqrt(7/pi)
        Y[12] = 0.4570457994644658f * x * (5.0f * z * z - 1.0f);   // 1/4 sqrt(21/(2pi))
        Y[13] = 1.445305721320277f * z * (x * x - y * y);          // 1/4 sqrt(105/pi)
        Y[14] = 0.5900435899266435f * x * (x * x - 3.0f * y * y);  // 1/4 sqrt(35/(2pi))
        nk = 15;
    }
#pragma unroll
    for (int k = 0; k < 15; k++) {
        if (k < nk) {
            const int row = (k + 1) * 3;
            c.x = fmaf(sh[(row + 0) * n + i], Y[k], c.x);
            c.y = fmaf(sh[(row + 1) * n + i], Y[k], c.y);
            c.z = fmaf(sh[(row + 2) * n + i], Y[k], c.z);
        }
    }
    return c;
}

// All per-view tests and, when visible, the record.  Returns visibility.
__device__ bool project_view(const ProjectArgs& a, const Geo& g, const CamDev& c, int i, Rec& r) {
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
    // colour along the viewing direction
    float dx = g.mx - c.campos[0], dy = g.my - c.campos[1], dz = g.mz - c.campos[2];
    const float dn = sqrtf(dx * dx + dy * dy + dz * dz);
    if (!(dn > 0.0f)) return false;
    const float idn = 1.0f / dn;
    dx *= idn;
    dy *= idn;
    dz *= idn;
    const float3 col = sh_colour(a, i, dx, dy, dz);
    if (!(finitef(col.x) && finitef(col.y) && finitef(col.z))) return false;
    r.xy = make_float2(mx, my);
    r.co = make_float4(cc * idet, -cb * idet, ca * idet, g.o);
    r.rgb = make_float3(fmaxf(0.0f, col.x), fmaxf(0.0f, col.y), fmaxf(0.0f, col.z));
    r.depth = tz;
    const int u0i = (int)fu0, u1i = (int)fu1, v0i = (int)fv0, v1i = (int)fv1;
    r.rect = make_ushort4((unsigned short)(u0i / kTile), (unsigned short)(v0i / kTile),
                          (unsigned short)(u1i / kTile), (unsigned short)(v1i / kTile));
    r.ntiles = (r.rect.z - r.rect.x + 1) * (r.rect.w - r.rect.y + 1);
    return true;
}

__global__ __launch_bounds__(kBlock) void project_count_kernel(ProjectArgs a) {
    __shared__ int s_cnt[kBlock / kWave];
    __shared__ unsigned long long s_inst[kBlock / kWave];
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    Geo g;
    g.ok = false;
    if (i < a.n) g = load_geo(a, i);
    const int nb = gridDim.x;
    for (int v = 0; v < a.V; v++) {
        Rec r;
        r.ntiles = 0;
        const bool vis = (i < a.n) && project_view(a, g, a.cams.c[v], i, r);
        const unsigned long long m = __ballot(vis);
        unsigned long long nt = vis ? (unsigned long long)r.ntiles : 0ull;
        for (int o = kWave / 2; o > 0; o >>= 1) nt += __shfl_xor(nt, o);
        if (lane == 0) {
            s_cnt[w] = __popcll(m);
            s_inst[w] = nt;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int c = 0;
            unsigned long long t = 0;
            for (int k = 0; k < kBlock / kWave; k++) {
                c += s_cnt[k];
                t += s_inst[k];
            }
            a.block_counts[v * nb + blockIdx.x] = c;
            if (t) atomicAdd((unsigned long long*)&a.inst_count[v], t);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kBlock) void project_write_kernel(ProjectArgs a) {
    __shared__ int s_cnt[kBlock / kWave];
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    Geo g;
    g.ok = false;
    if (i < a.n) g = load_geo(a, i);
    const int nb = gridDim.x;
    for (int v = 0; v < a.V; v++) {
        Rec r;
        const bool vis = (i < a.n) && project_view(a, g, a.cams.c[v], i, r);
        const unsigned long long m = __ballot(vis);
        if (lane == 0) s_cnt[w] = __popcll(m);
        __syncthreads();
        int off = a.block_offsets[v * nb + blockIdx.x];
        for (int k = 0; k < w; k++) off += s_cnt[k];
        __syncthreads();
        if (vis) {
            const int slot = off + __popcll(m & ((1ull << lane) - 1ull));
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
        }
    }
}

__global__ void zero_i64_kernel(int64_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace

static int32_t project_blocks(int32_t n) { return (n + kBlock - 1) / kBlock; }

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

size_t project_ws_bytes(int32_t n, int32_t V) {
    const int32_t nb = project_blocks(n > 0 ? n : 1);
    return 2 * align256(sizeof(int32_t) * (size_t)nb * V) + align256(scan_partials_bytes(nb, V));
}

hipError_t launch_project(const ProjectArgs& a0, hipStream_t s) {
    ProjectArgs a = a0;
    const int32_t nb = project_blocks(a.n > 0 ? a.n : 1);
    hipLaunchKernelGGL(zero_i64_kernel, dim3(1), dim3(64), 0, s, a.inst_count, a.V);
    hipLaunchKernelGGL(project_count_kernel, dim3(nb), dim3(kBlock), 0, s, a);
    hipError_t e = launch_scan_rows(a.block_counts, a.block_offsets, a.vis_count, nb, a.V, a.scan_partials, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(project_write_kernel, dim3(nb), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace gsmi
