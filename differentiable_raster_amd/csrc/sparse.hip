// F2: sparse encoding of the per-view 2D gradient records and their aggregation into owner
// arrays (ByteSplat, English abstract: zero partial gradients are left out of the exchange, an
// encoder compacts the remaining records and a decoder adds the received records directly into
// the arrays of the Gaussians' owner).
//
// Encoder: a record is the nine gradient components of one (view, visible slot); it is kept when
// any component is non-zero.  Stream compaction in three launches: per-block counts of kept
// records (one 256-slot block per (block, view)), the row scan over each view's block counts,
// and a write pass that places every kept record at (records of earlier views) + (earlier
// blocks of its view) + (its rank in its block), so the output is in (view, slot) order.
// Decoder: one thread per record adds the record into its (view, Gaussian) owner entry.  Within
// one encoded stream every (view, Gaussian) is unique, so no two threads touch the same entry.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

__device__ __forceinline__ void load_record(const GradsIn& g, size_t i, float r[9]) {
    const float2 m = reinterpret_cast<const float2*>(g.d_mean2d)[i];
    r[0] = m.x;
    r[1] = m.y;
    r[2] = g.d_conic[3 * i];
    r[3] = g.d_conic[3 * i + 1];
    r[4] = g.d_conic[3 * i + 2];
    r[5] = g.d_opacity[i];
    r[6] = g.d_color[3 * i];
    r[7] = g.d_color[3 * i + 1];
    r[8] = g.d_color[3 * i + 2];
}

// Kept: some component is not zero (a NaN is kept; -0 counts as zero).
__device__ __forceinline__ bool nonzero(const float r[9]) {
    bool nz = false;
#pragma unroll
    for (int t = 0; t < 9; t++) nz |= !(r[t] == 0.0f);
    return nz;
}

__global__ __launch_bounds__(kBlock) void encode_count_kernel(int32_t capacity, const int32_t* vis_count, GradsIn g,
                                                              int32_t nb, int32_t* block_counts) {
    const int v = blockIdx.y;
    const int32_t s = blockIdx.x * kBlock + threadIdx.x;
    bool keep = false;
    if (s < vis_count[v]) {
        float r[9];
        load_record(g, (size_t)v * capacity + s, r);
        keep = nonzero(r);
    }
    const int c = __syncthreads_count(keep);
    if (threadIdx.x == 0) block_counts[(size_t)v * nb + blockIdx.x] = c;
}

__global__ __launch_bounds__(kBlock) void encode_write_kernel(int32_t V, int32_t capacity, const int32_t* vis_count,
                                                              const int32_t* vis_ids, GradsIn g, int32_t nb,
                                                              const int32_t* block_offsets, const int32_t* row_totals,
                                                              int32_t* keys, float* records, int32_t* view_offset) {
    __shared__ int s_wave[kWaves];
    const int v = blockIdx.y;
    const int32_t s = blockIdx.x * kBlock + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    float r[9];
    bool keep = false;
    const size_t i = (size_t)v * capacity + s;
    if (s < vis_count[v]) {
        load_record(g, i, r);
        keep = nonzero(r);
    }
    // rank of the record among the kept records of its block
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(keep);
    if (lane == 0) s_wave[w] = __popcll(bal);
    __syncthreads();
    int before = __popcll(bal & ((1ull << lane) - 1ull));
    for (int q = 0; q < w; q++) before += s_wave[q];
    // records of the earlier views
    int64_t base = 0;
    for (int u = 0; u < v; u++) base += row_totals[u];
    if (keep) {
        const int64_t k = base + block_offsets[(size_t)v * nb + blockIdx.x] + before;
        keys[k] = vis_ids[i];
        float* out = records + (size_t)k * 9;
#pragma unroll
        for (int t = 0; t < 9; t++) out[t] = r[t];
    }
    if (blockIdx.x == 0 && v == 0 && (int)threadIdx.x <= V) {
        int32_t off = 0;
        for (int u = 0; u < (int)threadIdx.x; u++) off += row_totals[u];
        view_offset[threadIdx.x] = off;
    }
}

__global__ __launch_bounds__(kBlock) void decode_kernel(int32_t V, int32_t n_owner, const int32_t* view_offset,
                                                        const int32_t* keys, const float* records, GradsOut o) {
    const int32_t total = view_offset[V];
    for (int32_t k = blockIdx.x * kBlock + threadIdx.x; k < total; k += gridDim.x * kBlock) {
        int v = 0;
        while (v + 1 < V && view_offset[v + 1] <= k) v++;
        const int32_t gid = keys[k];
        if (gid < 0 || gid >= n_owner) continue;  // not an owner entry
        const size_t i = (size_t)v * n_owner + gid;
        const float* r = records + (size_t)k * 9;
        o.d_mean2d[2 * i] += r[0];
        o.d_mean2d[2 * i + 1] += r[1];
        o.d_conic[3 * i] += r[2];
        o.d_conic[3 * i + 1] += r[3];
        o.d_conic[3 * i + 2] += r[4];
        o.d_opacity[i] += r[5];
        o.d_color[3 * i] += r[6];
        o.d_color[3 * i + 1] += r[7];
        o.d_color[3 * i + 2] += r[8];
    }
}

int32_t encode_blocks(int32_t capacity) { return (capacity + kBlock - 1) / kBlock > 0 ? (capacity + kBlock - 1) / kBlock : 1; }

}  // namespace

size_t encode_workspace_bytes(int32_t capacity, int32_t V) {
    const int32_t nb = encode_blocks(capacity);
    auto al = [](size_t b) { return (b + 255) & ~size_t(255); };
    return 2 * al(sizeof(int32_t) * (size_t)nb * V) + al(sizeof(int32_t) * V) + al(scan_partials_bytes(nb, V));
}

hipError_t launch_grad_encode(int32_t V, int32_t capacity, const int32_t* vis_count, const int32_t* vis_ids,
                              GradsIn g, int32_t* keys, float* records, int32_t* view_offset, void* ws,
                              hipStream_t s) {
    const int32_t nb = encode_blocks(capacity);
    auto al = [](size_t b) { return (b + 255) & ~size_t(255); };
    char* p = static_cast<char*>(ws);
    int32_t* counts = reinterpret_cast<int32_t*>(p);
    p += al(sizeof(int32_t) * (size_t)nb * V);
    int32_t* offsets = reinterpret_cast<int32_t*>(p);
    p += al(sizeof(int32_t) * (size_t)nb * V);
    int32_t* totals = reinterpret_cast<int32_t*>(p);
    p += al(sizeof(int32_t) * V);
    int32_t* partials = reinterpret_cast<int32_t*>(p);
    hipLaunchKernelGGL(encode_count_kernel, dim3(nb, V), dim3(kBlock), 0, s, capacity, vis_count, g, nb, counts);
    hipError_t e = launch_scan_rows(counts, offsets, totals, nb, V, partials, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(encode_write_kernel, dim3(nb, V), dim3(kBlock), 0, s, V, capacity, vis_count, vis_ids, g, nb,
                       offsets, totals, keys, records, view_offset);
    return hipGetLastError();
}

hipError_t launch_grad_decode(int32_t V, int32_t n_owner, int64_t max_records, const int32_t* view_offset,
                              const int32_t* keys, const float* records, GradsOut o, hipStream_t s) {
    int64_t blocks = (max_records + kBlock - 1) / kBlock;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, V, n_owner, view_offset, keys,
                       records, o);
    return hipGetLastError();
}

}  // namespace gsmi
