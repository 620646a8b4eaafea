// Stable LSD radix sort of (uint32 key, uint32 value) pairs, up to 9 bits per pass.
//
// Per pass, over tiles of 4096 elements (16 per thread):
//   upsweep   - each block histograms the digit of its tile in LDS and writes the counts
//               digit-major, hist[d * nblocks + b];
//   scan      - one exclusive scan over that array gives every (digit, block) its first output
//               position (all of digit 0 first, blocks in order within a digit);
//   downsweep - each block ranks its elements stably within the tile (wavefront match by
//               ballots on the digit bits, per-wave counts combined in LDS), sorts the tile by
//               digit in LDS, and writes it out in that order: the elements of one digit leave
//               as one contiguous run, so the scatter is coalesced instead of one 4-byte store
//               per random address.
// Elements of a tile are ranked in the order e = round * 256 + thread, so the rank within a
// tile follows the input order and the sort is stable.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;
constexpr int kItems = 16;
constexpr int kChunk = kBlock * kItems;
constexpr int kMaxBits = 9;
constexpr int kRadix = 1 << kMaxBits;
constexpr int kWaves = kBlock / kWave;
constexpr int kPer = kRadix / kBlock;  // digits per thread

__global__ __launch_bounds__(kBlock) void radix_upsweep_kernel(const uint32_t* keys, int32_t n, int shift, uint32_t mask,
                                                               int32_t nblocks, int32_t* hist) {
    __shared__ int s_hist[kRadix];
    const int radix = (int)mask + 1;
#pragma unroll
    for (int k = 0; k < kPer; k++) s_hist[k * kBlock + threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kChunk;
#pragma unroll
    for (int r = 0; r < kItems; r++) {
        const int64_t e = base + r * kBlock + threadIdx.x;
        if (e < n) atomicAdd(&s_hist[(keys[e] >> shift) & mask], 1);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int d = k * kBlock + threadIdx.x;
        if (d < radix) hist[(size_t)d * nblocks + blockIdx.x] = s_hist[d];
    }
}

// Exclusive scan of the kRadix per-digit counts of the block (kPer consecutive digits per
// thread); returns each digit's first position within the tile in s_out.
__device__ __forceinline__ void scan_digits(const int* s_in, int* s_out, int* s_wave) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int v[kPer];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        v[k] = s_in[threadIdx.x * kPer + k];
        sum += v[k];
    }
    int inc = sum;
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    int off = 0;
    for (int k = 0; k < w; k++) off += s_wave[k];
    int run = off + inc - sum;
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        s_out[threadIdx.x * kPer + k] = run;
        run += v[k];
    }
}

__global__ __launch_bounds__(kBlock) void radix_downsweep_kernel(const uint32_t* keys, const uint32_t* vals, uint32_t* okeys,
                                                                 uint32_t* ovals, int32_t n, int shift, int bits,
                                                                 int32_t nblocks, const int32_t* offsets) {
    __shared__ int s_base[kRadix];          // first output position of each digit for this block
    __shared__ int s_cnt[kRadix];           // running per-digit count, in tile order
    __shared__ int s_local[kRadix];         // first position of each digit in the sorted tile
    __shared__ int s_wcnt[kWaves][kRadix];  // per-wave digit counts of the current round
    __shared__ int s_wave[kWaves];
    __shared__ uint32_t s_keys[kChunk];
    __shared__ uint32_t s_vals[kChunk];
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const uint32_t mask = (1u << bits) - 1u;
    const int radix = 1 << bits;
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int d = k * kBlock + threadIdx.x;
        s_base[d] = d < radix ? offsets[(size_t)d * nblocks + blockIdx.x] : 0;
        s_cnt[d] = 0;
        for (int q = 0; q < kWaves; q++) s_wcnt[q][d] = 0;
    }
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    const unsigned long long lt = (1ull << lane) - 1ull;
    uint32_t key[kItems], val[kItems];
    int rank[kItems];
#pragma unroll
    for (int r = 0; r < kItems; r++) {
        const int64_t e = base + r * kBlock + threadIdx.x;
        const bool valid = e < n;
        key[r] = valid ? keys[e] : 0u;
        val[r] = valid ? vals[e] : 0u;
        const uint32_t d = (key[r] >> shift) & mask;
        // lanes of this wavefront holding the same digit
        unsigned long long same = __ballot(valid);
        for (int b = 0; b < bits; b++) {
            const unsigned long long m = __ballot((d >> b) & 1u);
            same &= ((d >> b) & 1u) ? m : ~m;
        }
        const int before = __popcll(same & lt);
        if (valid && before == 0) s_wcnt[w][d] = __popcll(same);
        __syncthreads();
        int rk = s_cnt[d] + before;
        for (int q = 0; q < w; q++) rk += s_wcnt[q][d];
        rank[r] = rk;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const int dd = k * kBlock + threadIdx.x;
            int add = 0;
            for (int q = 0; q < kWaves; q++) {
                add += s_wcnt[q][dd];
                s_wcnt[q][dd] = 0;
            }
            s_cnt[dd] += add;
        }
        __syncthreads();
    }
    // sort the tile by digit in LDS
    scan_digits(s_cnt, s_local, s_wave);
    __syncthreads();
    const int valid_n = (int)min((int64_t)kChunk, (int64_t)n - base);
#pragma unroll
    for (int r = 0; r < kItems; r++) {
        if (r * kBlock + (int)threadIdx.x < valid_n) {
            const int p = s_local[(key[r] >> shift) & mask] + rank[r];
            s_keys[p] = key[r];
            s_vals[p] = val[r];
        }
    }
    __syncthreads();
    // write out in digit order: consecutive threads of one digit write consecutive positions
    for (int t = threadIdx.x; t < valid_n; t += kBlock) {
        const uint32_t k = s_keys[t];
        const uint32_t d = (k >> shift) & mask;
        const int pos = s_base[d] + (t - s_local[d]);
        okeys[pos] = k;
        ovals[pos] = s_vals[t];
    }
}

}  // namespace

static int32_t radix_blocks(int32_t n) { return (n + kChunk - 1) / kChunk; }

int radix_passes(int bits) { return bits <= 0 ? 0 : (bits + kMaxBits - 1) / kMaxBits; }

size_t radix_hist_bytes(int32_t n) { return sizeof(int32_t) * (size_t)kRadix * radix_blocks(n > 0 ? n : 1); }

size_t radix_partials_bytes(int32_t n) {
    return scan_partials_bytes(kRadix * radix_blocks(n > 0 ? n : 1), 1);
}

hipError_t launch_radix_sort(uint32_t* keys, uint32_t* vals, uint32_t* keys_alt, uint32_t* vals_alt, int32_t n,
                             int bits, int32_t* hist, int32_t* partials, hipStream_t s) {
    const int passes = radix_passes(bits);
    if (n <= 0 || passes == 0) return hipSuccess;
    const int32_t nb = radix_blocks(n);
    const int dbits = (bits + passes - 1) / passes;  // balanced digit width, <= kMaxBits
    uint32_t *ki = keys, *vi = vals, *ko = keys_alt, *vo = vals_alt;
    for (int p = 0; p < passes; p++) {
        const int shift = p * dbits;
        const int b = (bits - shift) < dbits ? (bits - shift) : dbits;
        const uint32_t mask = (1u << b) - 1u;
        hipLaunchKernelGGL(radix_upsweep_kernel, dim3(nb), dim3(kBlock), 0, s, ki, n, shift, mask, nb, hist);
        hipError_t e = launch_scan_rows(hist, hist, nullptr, (1 << b) * nb, 1, partials, s);
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
