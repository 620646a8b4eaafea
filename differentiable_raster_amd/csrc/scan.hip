// Device-wide exclusive prefix sums of int32 rows (reduce, scan the block sums, apply; rows of at
// most 16384 values are scanned by one workgroup each in a single launch).
// Each block owns kChunk = 2048 consecutive elements, and each thread scans kItems consecutive
// ones of them.  Global memory is read and written in the coalesced order (consecutive threads,
// consecutive elements) and turned into the thread-contiguous order through LDS, whose rows are
// padded by one word so that neither order puts two lanes of an access on one bank.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;
constexpr int kItems = 8;
constexpr int kChunk = kBlock * kItems;

// Exclusive scan of one value per thread across a block of BLOCK threads; returns the prefix,
// *total the sum.
template <int BLOCK = kBlock>
__device__ __forceinline__ int block_exclusive_scan(int x, int* s_wave, int* total) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int inc = x;
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    int off = 0, tot = 0;
    for (int k = 0; k < BLOCK / kWave; k++) {
        if (k < w) off += s_wave[k];
        tot += s_wave[k];
    }
    __syncthreads();
    *total = tot;
    return off + inc - x;
}

// Values [b0, b0 + BLOCK * ITEMS) of a row (zero past n) into LDS, thread t's ITEMS consecutive
// ones at s[t * (ITEMS + 1) + k].  Ends with a barrier.
template <int BLOCK, int ITEMS>
__device__ __forceinline__ void stage_in(const int32_t* r, int64_t b0, int64_t n, int* s) {
#pragma unroll
    for (int k = 0; k < ITEMS; k++) {
        const int e = k * BLOCK + (int)threadIdx.x;
        s[(e / ITEMS) * (ITEMS + 1) + e % ITEMS] = b0 + e < n ? r[b0 + e] : 0;
    }
    __syncthreads();
}

// The reverse of stage_in: s (thread-contiguous, padded) to o[b0, min(n, b0 + BLOCK * ITEMS)).
// Starts with a barrier.
template <int BLOCK, int ITEMS>
__device__ __forceinline__ void stage_out(const int* s, int64_t b0, int64_t n, int32_t* o) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; k++) {
        const int e = k * BLOCK + (int)threadIdx.x;
        if (b0 + e < n) o[b0 + e] = s[(e / ITEMS) * (ITEMS + 1) + e % ITEMS];
    }
}

__global__ __launch_bounds__(kBlock) void scan_reduce_kernel(const int32_t* in, int32_t n, int32_t nblocks,
                                                             int32_t* partials) {
    __shared__ int s_wave[kBlock / kWave];
    const int row = blockIdx.y;
    const int32_t* r = in + (size_t)row * n;
    const int64_t b0 = (int64_t)blockIdx.x * kChunk;
    int sum = 0;  // the block's sum: any order, so the coalesced one
#pragma unroll
    for (int k = 0; k < kItems; k++) {
        const int64_t e = b0 + k * kBlock + threadIdx.x;
        if (e < n) sum += r[e];
    }
    int tot;
    block_exclusive_scan(sum, s_wave, &tot);
    if (threadIdx.x == 0) partials[(size_t)row * nblocks + blockIdx.x] = tot;
}

// One block per row scans that row's block sums in place (exclusive) and writes the total.
__global__ __launch_bounds__(kBlock) void scan_partials_kernel(int32_t* partials, int32_t nblocks, int32_t* totals) {
    __shared__ int s_wave[kBlock / kWave];
    int32_t* r = partials + (size_t)blockIdx.x * nblocks;
    int carry = 0;
    for (int32_t b0 = 0; b0 < nblocks; b0 += kBlock) {
        const int32_t j = b0 + threadIdx.x;
        const int x = j < nblocks ? r[j] : 0;
        int tot;
        const int ex = block_exclusive_scan(x, s_wave, &tot);
        if (j < nblocks) r[j] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0 && totals) totals[blockIdx.x] = carry;
}

__global__ __launch_bounds__(kBlock) void scan_apply_kernel(const int32_t* in, int32_t* out, int32_t n, int32_t nblocks,
                                                            const int32_t* partials) {
    __shared__ int s_wave[kBlock / kWave];
    __shared__ int s_v[kBlock * (kItems + 1)];
    const int row = blockIdx.y;
    const int32_t* r = in + (size_t)row * n;
    int32_t* o = out + (size_t)row * n;
    const int64_t b0 = (int64_t)blockIdx.x * kChunk;
    stage_in<kBlock, kItems>(r, b0, n, s_v);
    int* mine = s_v + threadIdx.x * (kItems + 1);
    int v[kItems];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kItems; k++) {
        v[k] = mine[k];
        sum += v[k];
    }
    int tot;
    int run = block_exclusive_scan(sum, s_wave, &tot) + partials[(size_t)row * nblocks + blockIdx.x];
#pragma unroll
    for (int k = 0; k < kItems; k++) {
        mine[k] = run;
        run += v[k];
    }
    stage_out<kBlock, kItems>(s_v, b0, n, o);
}

// One workgroup scans a[0, n) in place (exclusive): each thread takes kSmallItems consecutive
// values per step, so up to kBlock * kSmallItems values take one step and two barriers.
constexpr int kSmallItems = 16;

__global__ __launch_bounds__(kBlock) void scan_small_kernel(int32_t* a, int32_t n) {
    __shared__ int s_wave[kBlock / kWave];
    int carry = 0;
    for (int32_t b0 = 0; b0 < n; b0 += kBlock * kSmallItems) {
        const int32_t first = b0 + threadIdx.x * kSmallItems;
        int v[kSmallItems];
        int sum = 0;
#pragma unroll
        for (int k = 0; k < kSmallItems; k++) {
            v[k] = first + k < n ? a[first + k] : 0;
            sum += v[k];
        }
        int tot;
        int run = carry + block_exclusive_scan(sum, s_wave, &tot);
#pragma unroll
        for (int k = 0; k < kSmallItems; k++) {
            if (first + k < n) a[first + k] = run;
            run += v[k];
        }
        carry += tot;
    }
}

// Short rows: one workgroup of 1024 threads per row scans it in one step of kShortRow values
// (one launch instead of three, the row's loads all in flight together) and writes the row
// total.
constexpr int kShortBlock = 1024;
constexpr int32_t kShortRow = kShortBlock * kSmallItems;

__global__ __launch_bounds__(kShortBlock) void scan_rows_short_kernel(const int32_t* in, int32_t* out,
                                                                      int32_t* totals, int32_t n) {
    __shared__ int s_wave[kShortBlock / kWave];
    __shared__ int s_v[kShortBlock * (kSmallItems + 1)];
    const int32_t* r = in + (size_t)blockIdx.x * n;
    int32_t* o = out + (size_t)blockIdx.x * n;
    int carry = 0;
    int* mine = s_v + threadIdx.x * (kSmallItems + 1);
    for (int32_t b0 = 0; b0 < n; b0 += kShortBlock * kSmallItems) {
        if (b0 > 0) __syncthreads();  // the previous step's stores have read s_v
        stage_in<kShortBlock, kSmallItems>(r, b0, n, s_v);
        int v[kSmallItems];
        int sum = 0;
#pragma unroll
        for (int k = 0; k < kSmallItems; k++) {
            v[k] = mine[k];
            sum += v[k];
        }
        int tot;
        int run = carry + block_exclusive_scan<kShortBlock>(sum, s_wave, &tot);
#pragma unroll
        for (int k = 0; k < kSmallItems; k++) {
            mine[k] = run;
            run += v[k];
        }
        stage_out<kShortBlock, kSmallItems>(s_v, b0, n, o);
        carry += tot;
    }
    if (threadIdx.x == 0 && totals) totals[blockIdx.x] = carry;
}

}  // namespace

static int32_t scan_blocks(int32_t n) { return (n + kChunk - 1) / kChunk; }

size_t scan_partials_bytes(int32_t n, int32_t rows) {
    return sizeof(int32_t) * (size_t)(scan_blocks(n > 0 ? n : 1)) * (size_t)rows;
}

hipError_t launch_scan_rows(const int32_t* in, int32_t* out, int32_t* totals, int32_t n, int32_t rows,
                            int32_t* partials, hipStream_t s) {
    if (n <= kShortRow) {
        hipLaunchKernelGGL(scan_rows_short_kernel, dim3(rows), dim3(kShortBlock), 0, s, in, out, totals, n);
        return hipGetLastError();
    }
    const int32_t nb = scan_blocks(n > 0 ? n : 1);
    hipLaunchKernelGGL(scan_reduce_kernel, dim3(nb, rows), dim3(kBlock), 0, s, in, n, nb, partials);
    hipLaunchKernelGGL(scan_partials_kernel, dim3(rows), dim3(kBlock), 0, s, partials, nb, totals);
    hipLaunchKernelGGL(scan_apply_kernel, dim3(nb, rows), dim3(kBlock), 0, s, in, out, n, nb, partials);
    return hipGetLastError();
}

hipError_t launch_scan_small(int32_t* a, int32_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(scan_small_kernel, dim3(1), dim3(kBlock), 0, s, a, n);
    return hipGetLastError();
}

}  // namespace gsmi
