// Stable LSD radix sort of (uint32 key, uint32 value) pairs, up to 8 bits per pass.
//
// Per pass:
//   upsweep   - each block histograms the digit of its 2048-element tile in LDS and writes the
//               counts digit-major, hist[d * nblocks + b];
//   scan      - one exclusive scan over that array gives every (digit, block) its first output
//               position (all of digit 0 first, blocks in order within a digit);
//   downsweep - each block ranks its elements stably within the tile (wavefront match by
//               ballots on the digit bits, per-wave counts combined in LDS) and scatters them.
// Elements of a tile are visited in the order e = round * 256 + thread, so the rank within a
// tile follows the input order and the sort is stable.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;
constexpr int kItems = 8;
constexpr int kChunk = kBlock * kItems;
constexpr int kRadix = 256;
constexpr int kWaves = kBlock / kWave;

__global__ __launch_bounds__(kBlock) void radix_upsweep_kernel(const uint32_t* keys, int32_t n, int shift, uint32_t mask,
                                                               int32_t nblocks, int32_t* hist) {
    __shared__ int s_hist[kRadix];
    s_hist[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kChunk;
#pragma unroll
    for (int r = 0; r < kItems; r++) {
        const int64_t e = base + r * kBlock + threadIdx.x;
        if (e < n) atomicAdd(&s_hist[(keys[e] >> shift) & mask], 1);
    }
    __syncthreads();
    hist[(size_t)threadIdx.x * nblocks + blockIdx.x] = s_hist[threadIdx.x];
}

__global__ __launch_bounds__(kBlock) void radix_downsweep_kernel(const uint32_t* keys, const uint32_t* vals, uint32_t* okeys,
                                                                 uint32_t* ovals, int32_t n, int shift, int bits,
                                                                 int32_t nblocks, const int32_t* offsets) {
    __shared__ int s_base[kRadix];           // first output position of each digit for this block
    __shared__ int s_wcnt[kWaves][kRadix];   // per-wave digit counts of the current round
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const uint32_t mask = (1u << bits) - 1u;
    s_base[threadIdx.x] = offsets[(size_t)threadIdx.x * nblocks + blockIdx.x];
    for (int k = 0; k < kWaves; k++) s_wcnt[k][threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int r = 0; r < kItems; r++) {
        const int64_t e = base + r * kBlock + threadIdx.x;
        const bool valid = e < n;
        uint32_t key = 0, val = 0;
        if (valid) {
            key = keys[e];
            val = vals[e];
        }
        const uint32_t d = (key >> shift) & mask;
        // lanes of this wavefront holding the same digit
        unsigned long long same = __ballot(valid);
        for (int b = 0; b < bits; b++) {
            const unsigned long long m = __ballot((d >> b) & 1u);
            same &= ((d >> b) & 1u) ? m : ~m;
        }
        const int before = __popcll(same & lt);
        const bool leader = valid && before == 0;
        if (leader) s_wcnt[w][d] = __popcll(same);
        __syncthreads();
        if (valid) {
            int pos = s_base[d] + before;
            for (int k = 0; k < w; k++) pos += s_wcnt[k][d];
            okeys[pos] = key;
            ovals[pos] = val;
        }
        __syncthreads();
        {
            int add = 0;
            for (int k = 0; k < kWaves; k++) {
                add += s_wcnt[k][threadIdx.x];
                s_wcnt[k][threadIdx.x] = 0;
            }
            s_base[threadIdx.x] += add;
        }
        __syncthreads();
    }
}

}  // namespace

static int32_t radix_blocks(int32_t n) { return (n + kChunk - 1) / kChunk; }

int radix_passes(int bits) { return bits <= 0 ? 0 : (bits + 7) / 8; }

size_t radix_hist_bytes(int32_t n) { return sizeof(int32_t) * (size_t)kRadix * radix_blocks(n > 0 ? n : 1); }

size_t radix_partials_bytes(int32_t n) {
    return scan_partials_bytes(kRadix * radix_blocks(n > 0 ? n : 1), 1);
}

hipError_t launch_radix_sort(uint32_t* keys, uint32_t* vals, uint32_t* keys_alt, uint32_t* vals_alt, int32_t n,
                             int bits, int32_t* hist, int32_t* partials, hipStream_t s) {
    const int passes = radix_passes(bits);
    if (n <= 0 || passes == 0) return hipSuccess;
    const int32_t nb = radix_blocks(n);
    const int dbits = (bits + passes - 1) / passes;  // balanced digit width, <= 8
    uint32_t *ki = keys, *vi = vals, *ko = keys_alt, *vo = vals_alt;
    for (int p = 0; p < passes; p++) {
        const int shift = p * dbits;
        const int b = (bits - shift) < dbits ? (bits - shift) : dbits;
        const uint32_t mask = (1u << b) - 1u;
        hipLaunchKernelGGL(radix_upsweep_kernel, dim3(nb), dim3(kBlock), 0, s, ki, n, shift, mask, nb, hist);
        hipError_t e = launch_scan_rows(hist, hist, nullptr, kRadix * nb, 1, partials, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(radix_downsweep_kernel, dim3(nb), dim3(kBlock), 0, s, ki, vi, ko, vo, n, shift, b, nb, hist);
        uint32_t* t = ki;
        ki = ko;
        ko = t;
        t = vi;
        vi = vo;
        vo = t;
    }
    return hipGetLastError();
}

}  // namespace gsmi
