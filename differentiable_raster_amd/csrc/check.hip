// GS_CHECK: validation of the binning output on the device (a debug aid; nothing on the hot path
// calls it).  Every rule is a property that the (view, tile, depth, slot) order of the tile lists
// fixes, so a correct gs_bin_tiles never trips one:
//   * the non-empty tile ranges, taken in global tile order, partition [0, count) without gaps,
//     and empty tiles hold (0, 0);
//   * every entry of tile t names a visible slot of t's view whose tile rectangle contains t, and
//     (for the full lists) its sorted tile key is t;
//   * within a list, (depth, slot) strictly increases (depths as float32 bit patterns: positive
//     depths order like their patterns);
//   * each view's list lengths add up to the n_tiles of its slots, whose instance bases follow
//     the slot order; a capped list is no longer than the cap.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ void flag(unsigned long long* viol, int kind) {
    atomicAdd(&viol[kind], 1ull);
}

// Per visible slot: the rectangle lies on the tile grid and spans n_tiles tiles, and the next
// slot's instance base follows; the n_tiles of each view are summed into sums[v].
__global__ __launch_bounds__(kBlock) void check_slots_kernel(CheckArgs a) {
    const int v = blockIdx.y;
    const int32_t s = blockIdx.x * kBlock + threadIdx.x;
    const int32_t nv = a.vis_count[v];
    long long nt = 0;
    if (s < nv && s < a.capacity) {
        const size_t idx = (size_t)v * a.capacity + s;
        const ushort4 r = a.rect[idx];
        nt = a.n_tiles[idx];
        const long long area = ((long long)r.z - r.x + 1) * ((long long)r.w - r.y + 1);
        if (r.z < r.x || r.w < r.y || r.z >= a.tiles_x || (int)r.w >= a.tpv / a.tiles_x || area != nt)
            flag(a.viol, GS_CHECK_SLOT_RECORD);
        if (s + 1 < nv && (long long)a.inst_base[idx + 1] - a.inst_base[idx] != nt) flag(a.viol, GS_CHECK_SLOT_RECORD);
    }
    for (int o = kWave / 2; o > 0; o >>= 1) nt += __shfl_xor(nt, o);
    if ((threadIdx.x & (kWave - 1)) == 0 && nt) atomicAdd((unsigned long long*)&a.sums[v], (unsigned long long)nt);
}

// One workgroup over all tiles in global order: every range against the running partition, the
// lengths summed per view into sums[V + v], the total against the count.
__global__ __launch_bounds__(kBlock) void check_tiles_kernel(CheckArgs a) {
    __shared__ long long s_wave[kBlock / kWave];
    __shared__ long long s_view[GS_MAX_VIEWS];
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    if (threadIdx.x < GS_MAX_VIEWS) s_view[threadIdx.x] = 0;
    const int32_t total_tiles = a.tpv * a.V;
    long long run = 0;  // instances of the earlier tiles
    for (int32_t t0 = 0; t0 < total_tiles; t0 += kBlock) {
        const int32_t t = t0 + threadIdx.x;
        long long len = 0;
        int32_t s = 0, e = 0;
        if (t < total_tiles) {
            s = a.ranges[2 * t];
            e = a.ranges[2 * t + 1];
            len = (long long)e - s;
            if (len < 0 || s < 0 || (long long)e > a.count) {
                flag(a.viol, GS_CHECK_RANGE);
                len = 0;
            } else if (len == 0 && (s != 0 || e != 0)) {
                flag(a.viol, GS_CHECK_RANGE);
            }
            if (a.cap > 0 && len > a.cap) flag(a.viol, GS_CHECK_CAP);
        }
        // exclusive scan of the lengths over the workgroup
        long long inc = len;
        for (int o = 1; o < kWave; o <<= 1) {
            const long long y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        if (lane == kWave - 1) s_wave[w] = inc;
        __syncthreads();
        long long before = run + inc - len, chunk = 0;
        for (int q = 0; q < kBlock / kWave; q++) {
            if (q < w) before += s_wave[q];
            chunk += s_wave[q];
        }
        if (t < total_tiles && len > 0) {
            if ((long long)s != before) flag(a.viol, GS_CHECK_RANGE);
            atomicAdd((unsigned long long*)&s_view[t / a.tpv], (unsigned long long)len);
        }
        run += chunk;
        __syncthreads();
    }
    if (threadIdx.x < a.V) a.sums[a.V + threadIdx.x] = s_view[threadIdx.x];
    if (threadIdx.x == 0 && run != a.count) flag(a.viol, GS_CHECK_COUNT);
}

// One wavefront per tile: the entries of its list.
__global__ __launch_bounds__(kWave) void check_lists_kernel(CheckArgs a) {
    const int32_t t = blockIdx.x;
    const int32_t s = a.ranges[2 * t], e = a.ranges[2 * t + 1];
    if (!(0 <= s && s <= e && (long long)e <= a.count)) return;  // reported by check_tiles_kernel
    const int v = t / a.tpv;
    const int32_t tl = t - v * a.tpv;
    const int tx = tl % a.tiles_x, ty = tl / a.tiles_x;
    const int32_t nv = a.vis_count[v];
    const size_t base = (size_t)v * a.capacity;
    for (int32_t k = s + (int32_t)threadIdx.x; k < e; k += kWave) {
        if (a.tile_keys && a.tile_keys[k] != (uint32_t)t) flag(a.viol, GS_CHECK_KEY);
        const int32_t slot = a.vals[k];
        if (slot < 0 || slot >= nv || slot >= a.capacity) {
            flag(a.viol, GS_CHECK_SLOT);
            continue;
        }
        const ushort4 r = a.rect[base + slot];
        if (tx < r.x || tx > r.z || ty < r.y || ty > r.w) flag(a.viol, GS_CHECK_RECT);
        if (k + 1 < e) {
            const int32_t nx = a.vals[k + 1];
            if (nx >= 0 && nx < nv && nx < a.capacity) {
                const uint32_t d0 = __float_as_uint(a.depth[base + slot]), d1 = __float_as_uint(a.depth[base + nx]);
                if (!(d0 < d1 || (d0 == d1 && slot < nx))) flag(a.viol, GS_CHECK_ORDER);
            }
        }
    }
}

}  // namespace

hipError_t launch_check_bins(const CheckArgs& a, bool slots, hipStream_t s) {
    if (slots) {
        const unsigned gx = (unsigned)((a.capacity + kBlock - 1) / kBlock);
        hipLaunchKernelGGL(check_slots_kernel, dim3(gx > 0 ? gx : 1, a.V), dim3(kBlock), 0, s, a);
    }
    hipLaunchKernelGGL(check_tiles_kernel, dim3(1), dim3(kBlock), 0, s, a);
    hipLaunchKernelGGL(check_lists_kernel, dim3((unsigned)(a.tpv * a.V)), dim3(kWave), 0, s, a);
    return hipGetLastError();
}

}  // namespace gsmi
