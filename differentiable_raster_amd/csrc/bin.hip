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
// Also clears zero[0, n_zero) (the tile ranges), which saves a launch.
__global__ __launch_bounds__(kBlock) void depth_keys_kernel(const float* depth, ViewFirst vf, int32_t V,
                                                            int32_t capacity, int32_t total, uint32_t key_min,
                                                            uint32_t* keys, uint32_t* vals, int32_t* zero,
                                                            int32_t n_zero) {
    const int32_t e = blockIdx.x * kBlock + threadIdx.x;
    if (e < n_zero) zero[e] = 0;
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

// Emission.  The slots in depth order are cut into chunks of kEmitChunk; within a chunk each
// wavefront owns kEmitRounds x 64 consecutive slots, one per lane and round.  emit_count_kernel
// gathers each slot's tile rectangle (the only random access of the emission), stores it in
// depth order (two words per slot, coalesced) and sums each chunk's tile counts (the rectangles'
// areas); after an exclusive scan of those sums (one workgroup), emit_kernel reads the
// rectangles back in order, adds the earlier wavefronts' totals and an in-wave scan per round to
// the chunk's offset, and writes each slot's instances (its tiles row-major) from there.
constexpr int kEmitRounds = 4;
constexpr int kEmitWaveSlots = kWave * kEmitRounds;
constexpr int kEmitChunk = kBlock * kEmitRounds;
constexpr int kEmitWaves = kBlock / kWave;

struct EmitSlot {
    uint32_t slot, vbase;
    ushort4 rc;
    int nt;
};

// GUARD: the chunk may reach past the last slot; such slots count no instance.  Chunks that lie
// wholly inside take the unguarded form, whose loads the compiler can issue for all rounds at once.
// The rectangle comes from the depth-ordered copy that emit_count_kernel wrote.
template <bool GUARD>
__device__ __forceinline__ EmitSlot load_emit_slot(const uint32_t* packed, const uint32_t* rect_lo,
                                                   const uint32_t* rect_hi, int32_t total, int32_t tiles_per_view,
                                                   int64_t e) {
    EmitSlot q;
    q.slot = 0;
    q.vbase = 0;
    q.rc = make_ushort4(0, 0, 0, 0);
    q.nt = 0;
    if (!GUARD || e < total) {
        const uint32_t p = packed[e];
        const uint32_t lo = rect_lo[e], hi = rect_hi[e];
        q.slot = p & kSlotMask;
        q.rc = make_ushort4((unsigned short)(lo & 0xFFFFu), (unsigned short)(lo >> 16), (unsigned short)(hi & 0xFFFFu),
                            (unsigned short)(hi >> 16));
        q.vbase = (p >> kSlotBits) * (uint32_t)tiles_per_view;
        q.nt = (q.rc.z - q.rc.x + 1) * (q.rc.w - q.rc.y + 1);
    }
    return q;
}

// The slots of this lane in the wavefront's rounds.
__device__ __forceinline__ void load_emit_rounds(const uint32_t* packed, const uint32_t* rect_lo,
                                                 const uint32_t* rect_hi, int32_t total, int32_t tiles_per_view,
                                                 int64_t wbase, int lane, EmitSlot q[kEmitRounds]) {
    if ((int64_t)(blockIdx.x + 1) * kEmitChunk <= total) {
#pragma unroll
        for (int r = 0; r < kEmitRounds; r++)
            q[r] = load_emit_slot<false>(packed, rect_lo, rect_hi, total, tiles_per_view, wbase + r * kWave + lane);
    } else {
#pragma unroll
        for (int r = 0; r < kEmitRounds; r++)
            q[r] = load_emit_slot<true>(packed, rect_lo, rect_hi, total, tiles_per_view, wbase + r * kWave + lane);
    }
}

__device__ __forceinline__ int wave_total(int x) {
    for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Instance count of the slot at depth-order position e (0 past the last slot when GUARD), after
// storing its tile rectangle at e of the depth-ordered copy.
template <bool GUARD>
__device__ __forceinline__ int slot_tiles(const uint32_t* packed, const ushort4* rect, int32_t capacity, int32_t total,
                                          int64_t e, uint32_t* rect_lo, uint32_t* rect_hi) {
    if (GUARD && e >= total) return 0;
    const uint32_t p = packed[e];
    const ushort4 rc = rect[(size_t)(p >> kSlotBits) * capacity + (p & kSlotMask)];
    rect_lo[e] = (uint32_t)rc.x | ((uint32_t)rc.y << 16);
    rect_hi[e] = (uint32_t)rc.z | ((uint32_t)rc.w << 16);
    return (rc.z - rc.x + 1) * (rc.w - rc.y + 1);
}

__global__ __launch_bounds__(kBlock) void emit_count_kernel(const uint32_t* packed, const ushort4* rect,
                                                            int32_t capacity, int32_t total, int32_t* chunk_counts,
                                                            int32_t* huge_count, uint32_t* rect_lo,
                                                            uint32_t* rect_hi) {
    __shared__ int s_wave[kEmitWaves];
    if (blockIdx.x == 0 && threadIdx.x == 0) *huge_count = 0;  // the emission appends after this kernel
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int64_t wbase = (int64_t)blockIdx.x * kEmitChunk + w * kEmitWaveSlots;
    int sum = 0;
    if ((int64_t)(blockIdx.x + 1) * kEmitChunk <= total) {
#pragma unroll
        for (int r = 0; r < kEmitRounds; r++)
            sum += slot_tiles<false>(packed, rect, capacity, total, wbase + r * kWave + lane, rect_lo, rect_hi);
    } else {
#pragma unroll
        for (int r = 0; r < kEmitRounds; r++)
            sum += slot_tiles<true>(packed, rect, capacity, total, wbase + r * kWave + lane, rect_lo, rect_hi);
    }
    sum = wave_total(sum);
    if (lane == 0) s_wave[w] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int q = 0; q < kEmitWaves; q++) t += s_wave[q];
        chunk_counts[blockIdx.x] = t;
    }
}

// Rectangles of more than kSmallRect tiles are written by the whole wavefront, 64 instances per
// step, so that a few large splats do not serialize on one lane.  Rectangles of more than
// kHugeRect tiles go to a list instead and emit_huge_kernel writes each with a workgroup: near
// the camera such splats are many, and the depth order puts them all in the first chunks, where
// one wavefront would write them one after another.  Every instance's position is fixed by the
// scan, so the list order changes nothing.
constexpr int kSmallRect = 8;

__global__ __launch_bounds__(kBlock) void emit_kernel(const uint32_t* packed, const int32_t* chunk_offsets,
                                                      const uint32_t* rect_lo, const uint32_t* rect_hi, int32_t total,
                                                      int32_t tiles_x, int32_t tiles_per_view, int32_t M,
                                                      int4* huge_list, int32_t* huge_count, int32_t huge_cap,
                                                      uint32_t* tile_keys, int32_t* vals) {
    __shared__ int s_wave[kEmitWaves];
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int64_t wbase = (int64_t)blockIdx.x * kEmitChunk + w * kEmitWaveSlots;
    EmitSlot q[kEmitRounds];
    load_emit_rounds(packed, rect_lo, rect_hi, total, tiles_per_view, wbase, lane, q);
    int sum = 0;
#pragma unroll
    for (int r = 0; r < kEmitRounds; r++) sum += q[r].nt;
    sum = wave_total(sum);
    if (lane == 0) s_wave[w] = sum;
    __syncthreads();
    int32_t off = chunk_offsets[blockIdx.x];
    for (int k = 0; k < w; k++) off += s_wave[k];
#pragma unroll
    for (int r = 0; r < kEmitRounds; r++) {
        // inclusive scan of the round's counts over the wavefront
        int inc = q[r].nt;
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(inc, d);
            if (lane >= d) inc += y;
        }
        const int32_t o = off + inc - q[r].nt;
        off += __shfl(inc, kWave - 1);
        const EmitSlot& e = q[r];
        const bool big = e.nt > kSmallRect;
        if (!big) {
            int32_t oo = o;
            for (int ty = e.rc.y; ty <= e.rc.w && e.nt > 0; ty++)
                for (int tx = e.rc.x; tx <= e.rc.z; tx++) {
                    if (oo < M) {  // never past the instance count sized on the host
                        tile_keys[oo] = e.vbase + (uint32_t)(ty * tiles_x + tx);
                        vals[oo] = (int32_t)e.slot;
                    }
                    oo++;
                }
        }
        unsigned long long bm = __ballot(big);
        while (bm != 0ull) {
            const int src = __ffsll((long long)bm) - 1;
            bm &= bm - 1ull;
            const int32_t o0 = __shfl(o, src);
            const int n0 = __shfl(e.nt, src);
            const int x0 = __shfl((int)e.rc.x, src), y0 = __shfl((int)e.rc.y, src);
            const int w0 = __shfl((int)e.rc.z, src) - x0 + 1;
            const uint32_t vb = (uint32_t)__shfl((int)e.vbase, src);
            const int32_t sl = __shfl((int)e.slot, src);
            if (n0 > kHugeRect) {
                int h = 0;
                if (lane == 0) h = atomicAdd(huge_count, 1);
                h = __shfl(h, 0);
                if (h < huge_cap) {
                    if (lane == 0) {
                        huge_list[2 * h] = make_int4(o0, n0, x0 | (y0 << 16), w0);
                        huge_list[2 * h + 1] = make_int4((int)vb, sl, 0, 0);
                    }
                    continue;
                }
                // a full list (never, with the list sized for M instances): written here
            }
            for (int k = lane; k < n0; k += kWave) {
                const int dy = k / w0, dx = k - dy * w0;
                if (o0 + k < M) {
                    tile_keys[o0 + k] = vb + (uint32_t)((y0 + dy) * tiles_x + x0 + dx);
                    vals[o0 + k] = sl;
                }
            }
        }
    }
}

// One workgroup per listed rectangle (grid-stride over the list).
__global__ __launch_bounds__(kBlock) void emit_huge_kernel(const int4* huge_list, const int32_t* huge_count,
                                                           int32_t huge_cap, int32_t tiles_x, int32_t M,
                                                           uint32_t* tile_keys, int32_t* vals) {
    const int32_t cnt = min(*huge_count, huge_cap);
    for (int32_t h = blockIdx.x; h < cnt; h += gridDim.x) {
        const int4 a = huge_list[2 * h], b = huge_list[2 * h + 1];
        const int32_t o0 = a.x, n0 = a.y, x0 = a.z & 0xFFFF, y0 = a.z >> 16, w0 = a.w;
        const uint32_t vb = (uint32_t)b.x;
        for (int k = threadIdx.x; k < n0; k += kBlock) {
            const int dy = k / w0, dx = k - dy * w0;
            if (o0 + k < M) {
                tile_keys[o0 + k] = vb + (uint32_t)((y0 + dy) * tiles_x + x0 + dx);
                vals[o0 + k] = b.y;
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

// Heavy-first schedule: a stable counting sort of the tiles on the bucket key clz(n + 1) =
// 31 - floor(log2(n + 1)) in [0, 31] of a tile with n entries (ties in tile order), so the
// longest lists come first.  The tiles are cut into chunks of kOrderChunk; within a chunk each
// wavefront owns kOrderRounds x 64 consecutive tiles.  order_hist_kernel writes each chunk's
// bucket counts (bucket-major); order_scatter_kernel turns all chunks' counts into the first
// position of each bucket for its chunk, ranks its tiles stably and writes them there.
constexpr int kOrderBuckets = 32;
constexpr int kOrderBits = 5;
constexpr int kOrderRounds = 8;
constexpr int kOrderWaveTiles = kWave * kOrderRounds;
constexpr int kOrderChunk = kBlock * kOrderRounds;
constexpr int kOrderWaves = kBlock / kWave;

__device__ __forceinline__ uint32_t order_key(const int32_t* ranges, int64_t t) {
    return (uint32_t)__clz(ranges[2 * t + 1] - ranges[2 * t] + 1);
}

// Per round: the lanes of the wavefront whose valid tile has the same bucket as this lane's.
__device__ __forceinline__ unsigned long long same_bucket(bool valid, uint32_t d) {
    unsigned long long same = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
    for (int b = 0; b < kOrderBits; b++) {
        const bool bit = (d >> b) & 1u;
        const unsigned long long m = __builtin_amdgcn_ballot_w64(bit);
        same &= bit ? m : ~m;
    }
    return same;
}

__global__ __launch_bounds__(kBlock) void order_hist_kernel(const int32_t* ranges, int32_t n_tiles_total,
                                                            int32_t nchunks, int32_t* hist) {
    __shared__ int s_hist[kOrderBuckets];
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    if (threadIdx.x < kOrderBuckets) s_hist[threadIdx.x] = 0;
    __syncthreads();
    const int64_t wbase = (int64_t)blockIdx.x * kOrderChunk + w * kOrderWaveTiles;
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int r = 0; r < kOrderRounds; r++) {
        const int64_t t = wbase + r * kWave + lane;
        const bool valid = t < n_tiles_total;
        const uint32_t d = valid ? order_key(ranges, t) : 0u;
        const unsigned long long same = same_bucket(valid, d);
        // one LDS add per bucket present in the round
        if (valid && (same & lt) == 0ull) atomicAdd(&s_hist[d], __popcll(same));
    }
    __syncthreads();
    if (threadIdx.x < kOrderBuckets) hist[(size_t)threadIdx.x * nchunks + blockIdx.x] = s_hist[threadIdx.x];
}

__global__ __launch_bounds__(kBlock) void order_scatter_kernel(const int32_t* ranges, int32_t n_tiles_total,
                                                               int32_t nchunks, const int32_t* hist, int32_t* order) {
    constexpr int kParts = kBlock / kOrderBuckets;
    __shared__ int s_tot[kParts][kOrderBuckets], s_pre[kParts][kOrderBuckets];
    __shared__ int s_base[kOrderBuckets];
    __shared__ int s_whist[kOrderWaves][kOrderBuckets];
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    // every bucket's total over all chunks and its count in the chunks before this one
    {
        const int d = threadIdx.x % kOrderBuckets, part = threadIdx.x / kOrderBuckets;
        int tot = 0, pre = 0;
        for (int32_t c = part; c < nchunks; c += kParts) {
            const int x = hist[(size_t)d * nchunks + c];
            tot += x;
            pre += c < (int32_t)blockIdx.x ? x : 0;
        }
        s_tot[part][d] = tot;
        s_pre[part][d] = pre;
        for (int i = threadIdx.x; i < kOrderWaves * kOrderBuckets; i += kBlock)
            s_whist[i / kOrderBuckets][i % kOrderBuckets] = 0;
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        // exclusive scan of the bucket totals (32 lanes of the first wavefront)
        const int d = lane;
        int tot = 0, pre = 0;
        if (d < kOrderBuckets)
            for (int q = 0; q < kParts; q++) {
                tot += s_tot[q][d];
                pre += s_pre[q][d];
            }
        int inc = tot;
        for (int o = 1; o < kOrderBuckets; o <<= 1) {
            const int y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        if (d < kOrderBuckets) s_base[d] = inc - tot + pre;
    }
    __syncthreads();
    // stable rank within the wavefront's tiles: rounds of 64 in tile order; the wavefront's LDS
    // operations are performed in order, so every lane reads the count before the leader of its
    // bucket adds this round's
    const int64_t wbase = (int64_t)blockIdx.x * kOrderChunk + w * kOrderWaveTiles;
    const unsigned long long lt = (1ull << lane) - 1ull;
    int* whist = s_whist[w];
    uint32_t key[kOrderRounds];
    int rank[kOrderRounds];
#pragma unroll
    for (int r = 0; r < kOrderRounds; r++) {
        const int64_t t = wbase + r * kWave + lane;
        const bool valid = t < n_tiles_total;
        const uint32_t d = valid ? order_key(ranges, t) : 0u;
        const unsigned long long same = same_bucket(valid, d);
        const int before = __popcll(same & lt);
        const int seen = whist[d];
        key[r] = d;
        rank[r] = seen + before;
        if (valid && before == 0) whist[d] = seen + __popcll(same);
    }
    __syncthreads();
    // each wavefront's first position within its bucket in this chunk
    if (threadIdx.x < kOrderBuckets) {
        int run = 0;
        for (int q = 0; q < kOrderWaves; q++) {
            const int c = s_whist[q][threadIdx.x];
            s_whist[q][threadIdx.x] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kOrderRounds; r++) {
        const int64_t t = wbase + r * kWave + lane;
        if (t < n_tiles_total) order[s_base[key[r]] + whist[key[r]] + rank[r]] = (int32_t)t;
    }
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

// Scores of a full tile's list held in LDS up to this many entries (24 KB); longer lists keep
// them in the global scratch.
constexpr int kCapLds = 6144;

// The K best of one full tile's n > K entries by (score desc, depth asc, slot asc).  The list is
// in (depth, slot) order, so the tie-break is list order: a radix select over the score bits
// (most significant digit first) finds the K-th best bit pattern `thr`; entries above it are
// kept, and of those equal to it the first `need` in list order.  Each wavefront counts digits
// into its own histogram (scores of one tile share their leading bits, so one shared histogram
// would put every lane's increment on the same few words).
// IN_PLACE (bits in LDS): the compaction first turns each entry's bits into its output position
// (or ~0u), and the list entries are copied afterwards in one pass, so that no global load or
// store waits at the compaction's barriers.
template <bool IN_PLACE>
__device__ __forceinline__ void cap_select_full(uint32_t* bits, int32_t n, int K, const int32_t* vals_in,
                                                int32_t* vals_out, int (*s_hist)[256], int* s_wave,
                                                uint32_t* s_sel) {
    const int w = threadIdx.x / kWave;
    uint32_t prefix = 0, pmask = 0;
    int remaining = K;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int q = 0; q < kBlock / kWave; q++) s_hist[q][threadIdx.x] = 0;
        __syncthreads();
        for (int32_t j = threadIdx.x; j < n; j += kBlock) {
            const uint32_t b = bits[j];
            if ((b & pmask) == prefix) atomicAdd(&s_hist[w][(b >> shift) & 255u], 1);
        }
        __syncthreads();
        // the digit d holding the remaining-th best entry: above(d) < remaining <= above(d) +
        // hist[d], with above(d) the entries of larger digits (d = 0 when no larger digit holds
        // it); thread t takes digit 255 - t, so an exclusive prefix over the threads is above(d)
        {
            static_assert(kBlock == 256, "one digit per thread");
            const int d = 255 - (int)threadIdx.x;
            int h = 0;
#pragma unroll
            for (int q = 0; q < kBlock / kWave; q++) h += s_hist[q][d];
            int all;
            const int above = block_excl_scan(h, s_wave, &all);
            const bool sel = d > 0 ? (above < remaining && above + h >= remaining) : above < remaining;
            if (sel) {
                s_sel[0] = (uint32_t)d;
                s_sel[1] = (uint32_t)(remaining - above);
            }
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
        const uint32_t b = j < n ? bits[j] : 0u;
        const int is_eq = (j < n && b == thr) ? 1 : 0;
        int eq_tot;
        const int eq_rank = eq_seen + block_excl_scan(is_eq, s_wave, &eq_tot);
        const int keep = (j < n) && (b > thr || (is_eq && eq_rank < need)) ? 1 : 0;
        int keep_tot;
        const int pos = out_seen + block_excl_scan(keep, s_wave, &keep_tot);
        if (IN_PLACE) {
            if (j < n) bits[j] = keep ? (uint32_t)pos : ~0u;  // this thread's own entry
        } else if (keep) {
            vals_out[pos] = vals_in[j];
        }
        eq_seen += eq_tot;
        out_seen += keep_tot;
    }
    if (IN_PLACE) {
        __syncthreads();
        for (int32_t j = threadIdx.x; j < n; j += kBlock) {
            const uint32_t pos = bits[j];
            if (pos != ~0u) vals_out[pos] = vals_in[j];
        }
    }
}

// The score bits of every visible slot (slot_bits[v * capacity + s]), in one coalesced pass: the
// select then gathers 4 bytes per list entry instead of the slot's 16-byte conic and opacity.
__global__ __launch_bounds__(kBlock) void cap_slot_scores_kernel(const float4* conic_opacity, const float4* rec,
                                                                 const int32_t* vis_count, int32_t capacity,
                                                                 uint32_t* slot_bits) {
    const int v = blockIdx.y;
    const int32_t s = blockIdx.x * kBlock + threadIdx.x;
    if (s < vis_count[v] && s < capacity) {
        const size_t i = (size_t)v * capacity + s;
        float4 co;
        if (conic_opacity) {
            co = conic_opacity[i];
        } else {
            // the packed record holds the same values: (x, y, A, B), (C, o, r, g), ...
            const float4 r0 = rec[4 * i], r1 = rec[4 * i + 1];
            co = make_float4(r0.z, r0.w, r1.x, r1.y);
        }
        slot_bits[i] = cap_score_bits(co);
    }
}

// The score bits of a list's n entries into bits[0, n), gathered by slot from slot_bits; each
// thread loads four list entries, then their four scores, with all four loads of a kind in
// flight at once.
__device__ __forceinline__ void cap_scores(const int32_t* list, int32_t n, const uint32_t* slot_bits, uint32_t* bits) {
    constexpr int kU = 4;
    for (int32_t j0 = 0; j0 < n; j0 += kU * kBlock) {
        int32_t slot[kU];
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int32_t j = j0 + u * kBlock + (int32_t)threadIdx.x;
            slot[u] = j < n ? list[j] : -1;
        }
        uint32_t r[kU];
#pragma unroll
        for (int u = 0; u < kU; u++) r[u] = slot[u] >= 0 ? slot_bits[slot[u]] : 0u;
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int32_t j = j0 + u * kBlock + (int32_t)threadIdx.x;
            if (j < n) bits[j] = r[u];
        }
    }
}

// One block per global tile, heaviest first when the tile order is given.  Tiles with at most K
// entries copy their list; longer lists keep the K best (cap_select_full).
__global__ __launch_bounds__(kBlock) void cap_select_kernel(const int32_t* ranges, const int32_t* vals,
                                                            const uint32_t* slot_bits, int32_t capacity,
                                                            int32_t tiles_per_view, int32_t K,
                                                            const int32_t* cap_offsets, const int32_t* tile_order,
                                                            int32_t* vals_capped, int32_t* ranges_capped,
                                                            uint32_t* scratch_bits) {
    __shared__ uint32_t s_bits[kCapLds];
    __shared__ int s_hist[kBlock / kWave][256];
    __shared__ int s_wave[kBlock / kWave];
    __shared__ uint32_t s_sel[2];
    const int32_t g = tile_order ? tile_order[blockIdx.x] : (int32_t)blockIdx.x;
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
    if (n <= kCapLds) {
        cap_scores(vals + start, n, slot_bits + vbase, s_bits);
        __syncthreads();
        cap_select_full<true>(s_bits, n, K, vals + start, vals_capped + out0, s_hist, s_wave, s_sel);
    } else {
        uint32_t* bits = scratch_bits + start;
        cap_scores(vals + start, n, slot_bits + vbase, bits);
        __syncthreads();
        cap_select_full<false>(bits, n, K, vals + start, vals_capped + out0, s_hist, s_wave, s_sel);
    }
}

}  // namespace

static unsigned blocks_for(int64_t n) { return (unsigned)((n + kBlock - 1) / kBlock); }

hipError_t launch_depth_keys(const float* depth, const int64_t* view_first, int32_t V, int32_t capacity,
                             int32_t total, uint32_t key_min, uint32_t* keys, uint32_t* vals, int32_t* zero,
                             int32_t n_zero, hipStream_t s) {
    if (total <= 0 && n_zero <= 0) return hipSuccess;
    ViewFirst vf;
    for (int v = 0; v <= GS_MAX_VIEWS; v++) vf.first[v] = v <= V ? (int32_t)view_first[v] : total;
    hipLaunchKernelGGL(depth_keys_kernel, dim3(blocks_for(total > n_zero ? total : n_zero)), dim3(kBlock), 0, s, depth,
                       vf, V, capacity, total, key_min, keys, vals, zero, n_zero);
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

int32_t emit_chunks(int32_t total) { return total > 0 ? (total + kEmitChunk - 1) / kEmitChunk : 0; }

hipError_t launch_emit(const uint32_t* packed, const ushort4* rect, int32_t capacity, int32_t total, int32_t tiles_x,
                       int32_t tiles_per_view, int32_t M, int32_t* chunk_offsets, uint32_t* rect_lo, uint32_t* rect_hi,
                       int4* huge_list, int32_t* huge_count, int32_t huge_cap, uint32_t* tile_keys, int32_t* vals,
                       hipStream_t s) {
    const int32_t nc = emit_chunks(total);
    if (nc == 0) return hipSuccess;
    hipLaunchKernelGGL(emit_count_kernel, dim3(nc), dim3(kBlock), 0, s, packed, rect, capacity, total, chunk_offsets,
                       huge_count, rect_lo, rect_hi);
    const hipError_t e = launch_scan_small(chunk_offsets, nc, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(emit_kernel, dim3(nc), dim3(kBlock), 0, s, packed, chunk_offsets, rect_lo, rect_hi, total,
                       tiles_x, tiles_per_view, M, huge_list, huge_count, huge_cap, tile_keys, vals);
    // at most one listed rectangle per kHugeRect instances
    const int32_t grid = huge_cap < 1024 ? huge_cap : 1024;
    hipLaunchKernelGGL(emit_huge_kernel, dim3(grid), dim3(kBlock), 0, s, huge_list, huge_count, huge_cap, tiles_x, M,
                       tile_keys, vals);
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

int32_t tile_order_chunks(int32_t n_tiles_total) {
    return n_tiles_total > 0 ? (n_tiles_total + kOrderChunk - 1) / kOrderChunk : 0;
}

size_t tile_order_hist_ints(int32_t n_tiles_total) { return (size_t)kOrderBuckets * tile_order_chunks(n_tiles_total); }

hipError_t launch_tile_order(const int32_t* ranges, int32_t n_tiles_total, int32_t* hist, int32_t* order,
                             hipStream_t s) {
    const int32_t nc = tile_order_chunks(n_tiles_total);
    if (nc == 0) return hipSuccess;
    hipLaunchKernelGGL(order_hist_kernel, dim3(nc), dim3(kBlock), 0, s, ranges, n_tiles_total, nc, hist);
    hipLaunchKernelGGL(order_scatter_kernel, dim3(nc), dim3(kBlock), 0, s, ranges, n_tiles_total, nc, hist, order);
    return hipGetLastError();
}

hipError_t launch_cap_count(const int32_t* ranges, int32_t n_tiles_total, int32_t K, int32_t* kept, hipStream_t s) {
    hipLaunchKernelGGL(cap_count_kernel, dim3(blocks_for(n_tiles_total)), dim3(kBlock), 0, s, ranges, n_tiles_total,
                       K, kept);
    return hipGetLastError();
}

hipError_t launch_cap_select(const int32_t* ranges, const int32_t* vals, const float4* conic_opacity,
                             const float4* rec, const int32_t* vis_count, int32_t V, int32_t capacity, int32_t tiles_per_view,
                             int32_t n_tiles_total, int32_t K, const int32_t* cap_offsets, const int32_t* tile_order,
                             int32_t* vals_capped, int32_t* ranges_capped, uint32_t* slot_bits,
                             uint32_t* scratch_bits, hipStream_t s) {
    if (capacity > 0)
        hipLaunchKernelGGL(cap_slot_scores_kernel, dim3((unsigned)((capacity + kBlock - 1) / kBlock), (unsigned)V),
                           dim3(kBlock), 0, s, conic_opacity, rec, vis_count, capacity, slot_bits);
    hipLaunchKernelGGL(cap_select_kernel, dim3(n_tiles_total), dim3(kBlock), 0, s, ranges, vals, slot_bits, capacity,
                       tiles_per_view, K, cap_offsets, tile_order, vals_capped, ranges_capped, scratch_bits);
    return hipGetLastError();
}

}  // namespace gsmi
