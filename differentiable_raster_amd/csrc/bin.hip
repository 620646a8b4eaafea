// A2-A6: tile binning of the visible slots of all views.
//
// The (view, tile, depth, slot) order is produced by an LSD radix sort whose depth digits run
// first, over one entry per visible slot (key = float32 bits of camera-space z, value =
// view << 28 | slot, input in (view, slot) order); each slot then emits its tile instances in
// that depth order at offsets from a prefix sum of n_tiles, and a stable radix sort on the
// global tile id (view * tiles_per_view + tile) finishes the sort.  Emission copies a slot's
// depth to each of its instances, so this equals sorting every instance by (tile, depth) with
// ties in slot order, while the depth passes move one entry per slot instead of one per
// instance.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;
constexpr uint32_t kSlotBits = 28;
constexpr uint32_t kSlotMask = (1u << kSlotBits) - 1u;

struct ViewFirst {
    int32_t first[GS_MAX_VIEWS + 1];
};

// Depth keys relative to the smallest one: the float32 bits of positive depths order like the
// depths, and subtracting the minimum keeps that order while shortening the keys (fewer passes).
__global__ __launch_bounds__(kBlock) void depth_keys_kernel(const float* depth, ViewFirst vf, int32_t V,
                                                            int32_t capacity, int32_t total, uint32_t key_min,
                                                            uint32_t* keys, uint32_t* vals) {
    const int32_t e = blockIdx.x * kBlock + threadIdx.x;
    if (e >= total) return;
    int v = 0;
    while (v + 1 < V && e >= vf.first[v + 1]) v++;
    const int32_t slot = e - vf.first[v];
    keys[e] = __float_as_uint(depth[(size_t)v * capacity + slot]) - key_min;
    vals[e] = ((uint32_t)v << kSlotBits) | (uint32_t)slot;
}

// The values the host reads back before sizing the binning launches, packed for one copy: the
// per-view counts and the range of the visible depths' float32 bits (bits[0] = the smallest
// pattern, bits[1] = the complement of the largest).  Two steps without atomics (many blocks
// adding into one word serialize across the chip): each block reduces a strided share of the
// visible depths into partial[block], then one block reduces the partials.
__global__ __launch_bounds__(kBlock) void depth_range_kernel(const int32_t* vis_count, int32_t V, const float* depth,
                                                             int32_t capacity, uint2* partial) {
    __shared__ uint32_t s_lo[kBlock / 64], s_hi[kBlock / 64];
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int v = 0; v < V; v++) {
        const int32_t cnt = min(vis_count[v], capacity);
        const float* d = depth + (size_t)v * capacity;
        for (int32_t i = blockIdx.x * kBlock + threadIdx.x; i < cnt; i += gridDim.x * kBlock) {
            const uint32_t b = __float_as_uint(d[i]);
            lo = min(lo, b);
            hi = max(hi, b);
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
    }
    if ((threadIdx.x & 63) == 0) {
        s_lo[threadIdx.x / 64] = lo;
        s_hi[threadIdx.x / 64] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < kBlock / 64; k++) {
            lo = min(lo, s_lo[k]);
            hi = max(hi, s_hi[k]);
        }
        partial[blockIdx.x] = make_uint2(lo, ~hi);
    }
}

__global__ __launch_bounds__(kBlock) void bin_counts_kernel(const int32_t* vis_count, const int64_t* inst_count,
                                                            int32_t V, const uint2* partial, int32_t nparts,
                                                            BinReadback* out) {
    __shared__ uint32_t s_lo[kBlock / 64], s_nhi[kBlock / 64];
    if (threadIdx.x < V) {
        out->vis[threadIdx.x] = vis_count[threadIdx.x];
        out->inst[threadIdx.x] = inst_count[threadIdx.x];
    }
    uint32_t lo = 0xFFFFFFFFu, nhi = 0xFFFFFFFFu;
    for (int k = threadIdx.x; k < nparts; k += kBlock) {
        lo = min(lo, partial[k].x);
        nhi = min(nhi, partial[k].y);
    }
    for (int o = 32; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
        nhi = min(nhi, (uint32_t)__shfl_xor((int)nhi, o));
    }
    if ((threadIdx.x & 63) == 0) {
        s_lo[threadIdx.x / 64] = lo;
        s_nhi[threadIdx.x / 64] = nhi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < kBlock / 64; k++) {
            lo = min(lo, s_lo[k]);
            nhi = min(nhi, s_nhi[k]);
        }
        out->bits[0] = lo;
        out->bits[1] = nhi;
    }
}

__global__ __launch_bounds__(kBlock) void gather_ntiles_kernel(const uint32_t* packed, const int32_t* n_tiles,
                                                               int32_t capacity, int32_t total, int32_t* out) {
    const int32_t r = blockIdx.x * kBlock + threadIdx.x;
    if (r >= total) return;
    const uint32_t p = packed[r];
    out[r] = n_tiles[(size_t)(p >> kSlotBits) * capacity + (p & kSlotMask)];
}

// One thread per slot in depth order writes the slot's instances (its tiles row-major) from its
// offset on.  Rectangles of more than kSmallRect tiles are written by the whole wavefront, 64
// instances per step, so that a few large splats do not serialize on one lane.
constexpr int kSmallRect = 8;

__global__ __launch_bounds__(kBlock) void emit_kernel(const uint32_t* packed, const int32_t* offsets, const ushort4* rect,
                                                      int32_t capacity, int32_t total, int32_t tiles_x,
                                                      int32_t tiles_per_view, int32_t M, uint32_t* tile_keys,
                                                      int32_t* vals) {
    const int32_t r = blockIdx.x * kBlock + threadIdx.x;
    const int lane = threadIdx.x & 63;
    const bool live = r < total;
    uint32_t slot = 0, vbase = 0;
    ushort4 rc = make_ushort4(0, 0, 0, 0);
    int32_t o = 0;
    int nt = 0;
    if (live) {
        const uint32_t p = packed[r];
        const uint32_t v = p >> kSlotBits;
        slot = p & kSlotMask;
        rc = rect[(size_t)v * capacity + slot];
        o = offsets[r];
        vbase = v * (uint32_t)tiles_per_view;
        nt = (rc.z - rc.x + 1) * (rc.w - rc.y + 1);
    }
    const bool big = nt > kSmallRect;
    if (live && !big) {
        for (int ty = rc.y; ty <= rc.w; ty++)
            for (int tx = rc.x; tx <= rc.z; tx++) {
                if (o >= M) return;  // never past the instance count sized on the host
                tile_keys[o] = vbase + (uint32_t)(ty * tiles_x + tx);
                vals[o] = (int32_t)slot;
                o++;
            }
    }
    unsigned long long bm = __ballot(big);
    while (bm != 0ull) {
        const int src = __ffsll((long long)bm) - 1;
        bm &= bm - 1ull;
        const int32_t o0 = __shfl(o, src);
        const int n0 = __shfl(nt, src);
        const int x0 = __shfl((int)rc.x, src), y0 = __shfl((int)rc.y, src);
        const int w0 = __shfl((int)rc.z, src) - x0 + 1;
        const uint32_t vb = (uint32_t)__shfl((int)vbase, src);
        const int32_t sl = __shfl((int)slot, src);
        for (int k = lane; k < n0; k += 64) {
            const int dy = k / w0, dx = k - dy * w0;
            if (o0 + k < M) {
                tile_keys[o0 + k] = vb + (uint32_t)((y0 + dy) * tiles_x + x0 + dx);
                vals[o0 + k] = sl;
            }
        }
    }
}

__global__ __launch_bounds__(kBlock) void fill_i32_kernel(int32_t* p, int32_t value, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) p[i] = value;
}

// ranges[t] = [first, last + 1) of tile t in the sorted keys (untouched tiles keep (0, 0)).
__global__ __launch_bounds__(kBlock) void ranges_kernel(const uint32_t* keys, int32_t M, int32_t* ranges) {
    const int32_t j = blockIdx.x * kBlock + threadIdx.x;
    if (j >= M) return;
    const uint32_t k = keys[j];
    if (j == 0 || keys[j - 1] != k) ranges[2 * (size_t)k] = j;
    if (j == M - 1 || keys[j + 1] != k) ranges[2 * (size_t)k + 1] = j + 1;
}

// Heavy-first schedule: key = clz(n + 1) = 31 - floor(log2(n + 1)) in [0, 31] for a tile with n
// entries; a stable sort on this 5-bit key (ties in tile order) puts the longest lists first.
__global__ __launch_bounds__(kBlock) void tile_order_keys_kernel(const int32_t* ranges, int32_t n_tiles_total,
                                                                 uint32_t* keys, uint32_t* vals) {
    const int32_t t = blockIdx.x * kBlock + threadIdx.x;
    if (t >= n_tiles_total) return;
    keys[t] = (uint32_t)__clz(ranges[2 * t + 1] - ranges[2 * t] + 1);
    vals[t] = (uint32_t)t;
}

__global__ __launch_bounds__(kBlock) void cap_count_kernel(const int32_t* ranges, int32_t n_tiles_total, int32_t K,
                                                           int32_t* kept) {
    const int32_t t = blockIdx.x * kBlock + threadIdx.x;
    if (t >= n_tiles_total) return;
    const int32_t n = ranges[2 * t + 1] - ranges[2 * t];
    kept[t] = n < K ? n : K;
}

// Cap score o / sqrt(A C - B^2), one IEEE rounding per operation, compared as its bit pattern.
// sqrtf (not __fsqrt_rn, which lowers to the 1-ulp v_sqrt_f32 alone) gets the correctly rounded
// lowering: v_sqrt_f32 followed by an FMA-residual correction of +-1 ulp.
__device__ __forceinline__ uint32_t cap_score_bits(float4 co) {
    const float det = __fsub_rn(__fmul_rn(co.x, co.z), __fmul_rn(co.y, co.y));
    return __float_as_uint(__fdiv_rn(co.w, sqrtf(det)));
}

__device__ __forceinline__ int block_excl_scan(int x, int* s_wave, int* total) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int inc = x;
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    int off = 0, tot = 0;
    for (int k = 0; k < kBlock / kWave; k++) {
        if (k < w) off += s_wave[k];
        tot += s_wave[k];
    }
    __syncthreads();
    *total = tot;
    return off + inc - x;
}

// One block per global tile.  Tiles with at most K entries copy their list; longer lists keep
// the K best by (score desc, depth asc, slot asc).  The list is in (depth, slot) order, so the
// tie-break is list order: a radix select over the score bits (most significant digit first)
// finds the K-th best bit pattern `thr`; entries above it are kept, and of those equal to it the
// first `need` in list order.
__global__ __launch_bounds__(kBlock) void cap_select_kernel(const int32_t* ranges, const int32_t* vals,
                                                            const float4* conic_opacity, int32_t capacity,
                                                            int32_t tiles_per_view, int32_t K,
                                                            const int32_t* cap_offsets, int32_t* vals_capped,
                                                            int32_t* ranges_capped, uint32_t* scratch_bits) {
    __shared__ int s_hist[256];
    __shared__ int s_wave[kBlock / kWave];
    __shared__ uint32_t s_sel[2];
    const int32_t g = blockIdx.x;
    const int32_t start = ranges[2 * g], end = ranges[2 * g + 1];
    const int32_t n = end - start;
    const int32_t out0 = cap_offsets[g];
    const int32_t kept = n < K ? n : K;
    if (threadIdx.x == 0) {
        ranges_capped[2 * g] = kept > 0 ? out0 : 0;
        ranges_capped[2 * g + 1] = kept > 0 ? out0 + kept : 0;
    }
    if (n <= K) {
        for (int32_t j = threadIdx.x; j < n; j += kBlock) vals_capped[out0 + j] = vals[start + j];
        return;
    }
    const size_t vbase = (size_t)(g / tiles_per_view) * capacity;
    for (int32_t j = threadIdx.x; j < n; j += kBlock)
        scratch_bits[start + j] = cap_score_bits(conic_opacity[vbase + vals[start + j]]);
    __syncthreads();
    uint32_t prefix = 0, pmask = 0;
    int remaining = K;
    for (int shift = 24; shift >= 0; shift -= 8) {
        s_hist[threadIdx.x] = 0;
        __syncthreads();
        for (int32_t j = threadIdx.x; j < n; j += kBlock) {
            const uint32_t b = scratch_bits[start + j];
            if ((b & pmask) == prefix) atomicAdd(&s_hist[(b >> shift) & 255u], 1);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int cum = 0;
            int d = 255;
            for (; d > 0; d--) {
                if (cum + s_hist[d] >= remaining) break;
                cum += s_hist[d];
            }
            s_sel[0] = (uint32_t)d;
            s_sel[1] = (uint32_t)(remaining - cum);
        }
        __syncthreads();
        prefix |= s_sel[0] << shift;
        pmask |= 255u << shift;
        remaining = (int)s_sel[1];
        __syncthreads();
    }
    const uint32_t thr = prefix;
    const int need = remaining;  // entries equal to thr to keep, in list order
    int eq_seen = 0, out_seen = 0;
    for (int32_t j0 = 0; j0 < n; j0 += kBlock) {
        const int32_t j = j0 + threadIdx.x;
        const uint32_t b = j < n ? scratch_bits[start + j] : 0u;
        const int is_eq = (j < n && b == thr) ? 1 : 0;
        int eq_tot;
        const int eq_rank = eq_seen + block_excl_scan(is_eq, s_wave, &eq_tot);
        const int keep = (j < n) && (b > thr || (is_eq && eq_rank < need)) ? 1 : 0;
        int keep_tot;
        const int pos = out_seen + block_excl_scan(keep, s_wave, &keep_tot);
        if (keep) vals_capped[out0 + pos] = vals[start + j];
        eq_seen += eq_tot;
        out_seen += keep_tot;
    }
}

}  // namespace

static unsigned blocks_for(int64_t n) { return (unsigned)((n + kBlock - 1) / kBlock); }

hipError_t launch_depth_keys(const float* depth, const int64_t* view_first, int32_t V, int32_t capacity,
                             int32_t total, uint32_t key_min, uint32_t* keys, uint32_t* vals, hipStream_t s) {
    if (total <= 0) return hipSuccess;
    ViewFirst vf;
    for (int v = 0; v <= GS_MAX_VIEWS; v++) vf.first[v] = v <= V ? (int32_t)view_first[v] : total;
    hipLaunchKernelGGL(depth_keys_kernel, dim3(blocks_for(total)), dim3(kBlock), 0, s, depth, vf, V, capacity, total,
                       key_min, keys, vals);
    return hipGetLastError();
}

hipError_t launch_bin_counts(const int32_t* vis_count, const int64_t* inst_count, int32_t V, const float* depth,
                             int32_t capacity, BinReadback* out, hipStream_t s) {
    hipLaunchKernelGGL(depth_range_kernel, dim3(kDepthRangeBlocks), dim3(kBlock), 0, s, vis_count, V, depth, capacity,
                       out->partial);
    hipLaunchKernelGGL(bin_counts_kernel, dim3(1), dim3(kBlock), 0, s, vis_count, inst_count, V, out->partial,
                       kDepthRangeBlocks, out);
    return hipGetLastError();
}

hipError_t launch_gather_ntiles(const uint32_t* packed, const int32_t* n_tiles, int32_t capacity, int32_t total,
                                int32_t* out, hipStream_t s) {
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(gather_ntiles_kernel, dim3(blocks_for(total)), dim3(kBlock), 0, s, packed, n_tiles, capacity,
                       total, out);
    return hipGetLastError();
}

hipError_t launch_emit(const uint32_t* packed, const int32_t* offsets, const ushort4* rect, int32_t capacity,
                       int32_t total, int32_t tiles_x, int32_t tiles_per_view, int32_t M, uint32_t* tile_keys,
                       int32_t* vals, hipStream_t s) {
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(emit_kernel, dim3(blocks_for(total)), dim3(kBlock), 0, s, packed, offsets, rect, capacity,
                       total, tiles_x, tiles_per_view, M, tile_keys, vals);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks_for(n)), dim3(kBlock), 0, s, p, value, n);
    return hipGetLastError();
}

hipError_t launch_ranges(const uint32_t* tile_keys, int32_t M, int32_t* ranges, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(ranges_kernel, dim3(blocks_for(M)), dim3(kBlock), 0, s, tile_keys, M, ranges);
    return hipGetLastError();
}

hipError_t launch_tile_order(const int32_t* ranges, int32_t n_tiles_total, uint32_t* keys, uint32_t* vals,
                             uint32_t* keys_alt, int32_t* order, int32_t* hist, int32_t* partials, hipStream_t s) {
    if (n_tiles_total <= 0) return hipSuccess;
    hipLaunchKernelGGL(tile_order_keys_kernel, dim3(blocks_for(n_tiles_total)), dim3(kBlock), 0, s, ranges,
                       n_tiles_total, keys, vals);
    // one 5-bit pass: the result lands in the alternate buffers (keys_alt, order)
    return launch_radix_sort(keys, vals, keys_alt, reinterpret_cast<uint32_t*>(order), n_tiles_total, 5, hist,
                             partials, s);
}

hipError_t launch_cap_count(const int32_t* ranges, int32_t n_tiles_total, int32_t K, int32_t* kept, hipStream_t s) {
    hipLaunchKernelGGL(cap_count_kernel, dim3(blocks_for(n_tiles_total)), dim3(kBlock), 0, s, ranges, n_tiles_total,
                       K, kept);
    return hipGetLastError();
}

hipError_t launch_cap_select(const int32_t* ranges, const int32_t* vals, const float4* conic_opacity, int32_t capacity,
                             int32_t tiles_per_view, int32_t n_tiles_total, int32_t K, const int32_t* cap_offsets,
                             int32_t* vals_capped, int32_t* ranges_capped, uint32_t* scratch_bits, hipStream_t s) {
    hipLaunchKernelGGL(cap_select_kernel, dim3(n_tiles_total), dim3(kBlock), 0, s, ranges, vals, conic_opacity, capacity,
                       tiles_per_view, K, cap_offsets, vals_capped, ranges_capped, scratch_bits);
    return hipGetLastError();
}

}  // namespace gsmi
