// Stable LSD radix sort of (uint32 key, uint32 value) pairs, up to 9 bits per pass.
//
// Per pass, over tiles of 256 x ITEMS elements, ITEMS = 12 (3072 elements; each of the four
// wavefronts owns 768 consecutive ones; a tile's 36.5 KB of LDS lets four workgroups share a CU),
// or 6 for sorts of at most kSmallSortN elements (twice as many tiles, so that a small sort
// spreads over more CUs; 100 K Gaussians at 720p: bin stage 188 -> 164 us):
//   upsweep   - each block histograms the digit of its tile in LDS and writes the counts
//               digit-major, hist[d * nblocks + b];
//   row scan  - one block per digit scans that digit's row over the blocks (the digit's first
//               position within the digit, per block) and writes the digit's total;
//   downsweep - each block turns the digit totals into digit starts (a scan over at most 512
//               values), ranks its elements stably (per wavefront: ballots on the digit bits
//               give each element's rank among equal digits of its 64-element round, and a
//               per-wavefront digit histogram in LDS carries the count across rounds, with no
//               workgroup barrier between rounds), sorts the tile by digit in LDS and writes it
//               out in that order: each digit's elements leave as one contiguous run.
// The rank of an element follows (wavefront, round, lane), which is the input order, so the
// sort is stable.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = 256;
constexpr int kItemsLarge = 12;
constexpr int kItemsSmall = 6;
constexpr int32_t kSmallSortN = 1024 * kBlock * kItemsSmall;  // 1.57 M elements
constexpr int kMaxBits = 9;
constexpr int kRadix = 1 << kMaxBits;
constexpr int kWaves = kBlock / kWave;
constexpr int kPer = kRadix / kBlock;  // digits per thread
constexpr int kXcds = 8;                // MI355X: workgroups are dealt round-robin to 8 XCDs

// Tile of workgroup `bid`: the workgroups that land on one XCD take a contiguous run of tiles, so
// the neighbouring parts of each digit's output run are written through the same L2.  A
// bijection of [0, nb) for any nb; upsweep and downsweep use the same one.
__device__ __forceinline__ int32_t tile_of(int32_t bid, int32_t nb) {
    const int32_t q = nb / kXcds, r = nb % kXcds, x = bid % kXcds, i = bid / kXcds;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <int ITEMS>
__global__ __launch_bounds__(kBlock) void radix_upsweep_kernel(const uint32_t* keys, int32_t n, int shift, uint32_t mask,
                                                               int32_t nblocks, int32_t* hist) {
    constexpr int kChunk = kBlock * ITEMS;
    __shared__ int s_hist[kRadix];
    const int radix = (int)mask + 1;
#pragma unroll
    for (int k = 0; k < kPer; k++) s_hist[k * kBlock + threadIdx.x] = 0;
    __syncthreads();
    const int32_t tile = tile_of(blockIdx.x, nblocks);
    const int64_t base = (int64_t)tile * kChunk;
#pragma unroll
    for (int r = 0; r < ITEMS; r++) {
        const int64_t e = base + r * kBlock + threadIdx.x;
        if (e < n) atomicAdd(&s_hist[(keys[e] >> shift) & mask], 1);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int d = k * kBlock + threadIdx.x;
        if (d < radix) hist[(size_t)d * nblocks + tile] = s_hist[d];
    }
}

// Exclusive scan over the block of one value per thread; returns the prefix, *total the sum.
__device__ __forceinline__ int block_scan(int x, int* s_wave, int* total) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int inc = x;
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    int off = 0, tot = 0;
    for (int k = 0; k < kWaves; k++) {
        if (k < w) off += s_wave[k];
        tot += s_wave[k];
    }
    __syncthreads();
    *total = tot;
    return off + inc - x;
}

// One block per digit: hist[d][b] -> the exclusive prefix over b (in place) and totals[d].
__global__ __launch_bounds__(kBlock) void radix_rowscan_kernel(int32_t* hist, int32_t nblocks, int32_t* totals) {
    __shared__ int s_wave[kWaves];
    int32_t* row = hist + (size_t)blockIdx.x * nblocks;
    int carry = 0;
    for (int32_t b0 = 0; b0 < nblocks; b0 += kBlock) {
        const int32_t b = b0 + threadIdx.x;
        const int x = b < nblocks ? row[b] : 0;
        int tot;
        const int ex = block_scan(x, s_wave, &tot);
        if (b < nblocks) row[b] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

template <int ITEMS>
__global__ __launch_bounds__(kBlock) void radix_downsweep_kernel(const uint32_t* keys, const uint32_t* vals, uint32_t* okeys,
                                                                 uint32_t* ovals, int32_t n, int shift, int bits,
                                                                 int32_t nblocks, const int32_t* rowpref,
                                                                 const int32_t* totals) {
    constexpr int kChunk = kBlock * ITEMS;
    constexpr int kWaveChunk = kWave * ITEMS;  // elements owned by one wavefront
    __shared__ int s_base[kRadix];          // first output position of each digit for this block
    __shared__ int s_local[kRadix];         // first position of each digit in the sorted tile
    __shared__ int s_whist[kWaves][kRadix]; // per-wavefront digit counts, then their prefixes
    __shared__ int s_wave[kWaves];
    __shared__ uint32_t s_keys[kChunk];
    __shared__ uint32_t s_vals[kChunk];
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const uint32_t mask = (1u << bits) - 1u;
    const int radix = 1 << bits;
    const int32_t tile = tile_of(blockIdx.x, nblocks);
    // digit starts: exclusive scan of the totals (kPer consecutive digits per thread)
    {
        int v[kPer];
        int sum = 0;
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const int d = threadIdx.x * kPer + k;
            v[k] = d < radix ? totals[d] : 0;
            sum += v[k];
        }
        int tot;
        int run = block_scan(sum, s_wave, &tot);
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const int d = threadIdx.x * kPer + k;
            s_base[d] = run + (d < radix ? rowpref[(size_t)d * nblocks + tile] : 0);
            run += v[k];
        }
    }
#pragma unroll
    for (int k = 0; k < kPer; k++)
        for (int q = 0; q < kWaves; q++) s_whist[q][k * kBlock + threadIdx.x] = 0;
    __syncthreads();
    // rank within the wavefront's elements: rounds of 64 in input order
    const int64_t wbase = (int64_t)tile * kChunk + w * kWaveChunk;
    const unsigned long long lt = (1ull << lane) - 1ull;
    int* whist = s_whist[w];
    uint32_t key[ITEMS], val[ITEMS];
    int rank[ITEMS];
#pragma unroll
    for (int r = 0; r < ITEMS; r++) {
        const int64_t e = wbase + r * kWave + lane;
        const bool valid = e < n;
        key[r] = valid ? keys[e] : 0u;
        val[r] = valid ? vals[e] : 0u;
    }
#pragma unroll
    for (int r = 0; r < ITEMS; r++) {
        const int64_t e = wbase + r * kWave + lane;
        const bool valid = e < n;
        const uint32_t d = (key[r] >> shift) & mask;
        // lanes of this round holding the same digit
        unsigned long long same = __ballot(valid);
        for (int b = 0; b < bits; b++) {
            const unsigned long long m = __ballot((d >> b) & 1u);
            same &= ((d >> b) & 1u) ? m : ~m;
        }
        const int before = __popcll(same & lt);
        // the wavefront's LDS operations are performed in order: every lane reads the count
        // before the leader of its digit adds this round's
        const int seen = whist[d];
        rank[r] = seen + before;
        if (valid && before == 0) whist[d] = seen + __popcll(same);
    }
    __syncthreads();
    // digit starts within the tile and each wavefront's start within its digit
    {
        int v[kPer];
        int sum = 0;
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const int d = threadIdx.x * kPer + k;
            int run = 0;
            for (int q = 0; q < kWaves; q++) {
                const int c = s_whist[q][d];
                s_whist[q][d] = run;
                run += c;
            }
            v[k] = run;
            sum += run;
        }
        int tot;
        int run = block_scan(sum, s_wave, &tot);
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            s_local[threadIdx.x * kPer + k] = run;
            run += v[k];
        }
    }
    __syncthreads();
    const int valid_n = (int)min((int64_t)kChunk, (int64_t)n - (int64_t)tile * kChunk);
#pragma unroll
    for (int r = 0; r < ITEMS; r++) {
        if (wbase + r * kWave + lane < n) {
            const uint32_t d = (key[r] >> shift) & mask;
            const int p = s_local[d] + whist[d] + rank[r];
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

static bool radix_small(int32_t n) { return n <= kSmallSortN; }

static int32_t radix_blocks(int32_t n) {
    const int32_t chunk = kBlock * (radix_small(n) ? kItemsSmall : kItemsLarge);
    return (n + chunk - 1) / chunk;
}

int radix_passes(int bits) { return bits <= 0 ? 0 : (bits + kMaxBits - 1) / kMaxBits; }

// digit-major histograms, then the per-digit totals, for any sort of at most n elements (the
// small tiles give sorts up to kSmallSortN more tiles than a slightly larger sort has)
size_t radix_hist_bytes(int32_t n) {
    n = n > 0 ? n : 1;
    int32_t nb = radix_blocks(n);
    const int32_t nb_small = radix_blocks(n < kSmallSortN ? n : kSmallSortN);
    if (nb_small > nb) nb = nb_small;
    return sizeof(int32_t) * ((size_t)kRadix * nb + kRadix);
}

size_t radix_partials_bytes(int32_t /*n*/) { return 0; }

hipError_t launch_radix_sort(uint32_t* keys, uint32_t* vals, uint32_t* keys_alt, uint32_t* vals_alt, int32_t n,
                             int bits, int32_t* hist, int32_t* /*partials*/, hipStream_t s) {
    const int passes = radix_passes(bits);
    if (n <= 0 || passes == 0) return hipSuccess;
    const int32_t nb = radix_blocks(n);
    int32_t* totals = hist + (size_t)kRadix * nb;
    const int dbits = (bits + passes - 1) / passes;  // balanced digit width, <= kMaxBits
    uint32_t *ki = keys, *vi = vals, *ko = keys_alt, *vo = vals_alt;
    for (int p = 0; p < passes; p++) {
        const int shift = p * dbits;
        const int b = (bits - shift) < dbits ? (bits - shift) : dbits;
        const uint32_t mask = (1u << b) - 1u;
        if (radix_small(n))
            hipLaunchKernelGGL(radix_upsweep_kernel<kItemsSmall>, dim3(nb), dim3(kBlock), 0, s, ki, n, shift, mask, nb,
                               hist);
        else
            hipLaunchKernelGGL(radix_upsweep_kernel<kItemsLarge>, dim3(nb), dim3(kBlock), 0, s, ki, n, shift, mask, nb,
                               hist);
        hipLaunchKernelGGL(radix_rowscan_kernel, dim3(1 << b), dim3(kBlock), 0, s, hist, nb, totals);
        if (radix_small(n))
            hipLaunchKernelGGL(radix_downsweep_kernel<kItemsSmall>, dim3(nb), dim3(kBlock), 0, s, ki, vi, ko, vo, n,
                               shift, b, nb, hist, totals);
        else
            hipLaunchKernelGGL(radix_downsweep_kernel<kItemsLarge>, dim3(nb), dim3(kBlock), 0, s, ki, vi, ko, vo, n,
                               shift, b, nb, hist, totals);
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
