// A7-A10: forward, loss-gradient, backward and fused rasterizers.
//
// One 256-thread workgroup per (view, 16x16 tile).  Each wavefront owns an 8x8 quarter of the
// tile and each of its four 16-lane DPP rows owns a 4x4 block of that quarter: lane l of wave w
// shades pixel ((w & 1) * 8 + (r & 1) * 4 + (l & 3), (w >> 1) * 8 + (r >> 1) * 4 + ((l & 15) >> 2))
// with r = l >> 4.  Splats in these scenes cover a few pixels, so giving every 4x4 block its own
// list keeps the lanes of an instruction on pixels the splat can reach.
//
// The tile's list is staged through LDS in batches of 256 entries, one gather per thread.  While
// staging, each entry gets a conservative 16-bit mask of the 4x4 blocks its alpha_min box
// touches, and every block gets its own compacted list of the batch entries that touch it
// (ballot + popcount), so a row never evaluates a pair its pixels cannot blend.  The box is
// widened beyond float32 reach and the mask is all ones for ill-conditioned conics: the culled
// pairs are pairs with alpha < alpha_min, and forward and backward cull the same pairs (they run
// this same code on the same records).
//
// Pair evaluation works in base-2 logarithm units: the staged conic is pre-scaled and the
// entry's log2(o) staged beside it, so that p2 = log2(o) - q/2 * log2(e) comes out of three FMAs
// and exp2(p2) is o * exp(-q/2) itself.  The alpha_min test is p2 >= log2(alpha_min), one
// compare with a constant, and 1 - alpha is one subtraction after the clamp.
//
// The forward walks each block's list front to back; a workgroup stops staging once every pixel
// has stopped.  The backward walks it back to front from n_contrib, recovering T by division by
// (1 - alpha) and carrying the colour behind.  It takes a staged batch in sub-batches of at most
// 128 entries whose (entry, block) pairs fit a 256-slot log in LDS: every pair gets its own slot
// (the pairs of earlier entries of the sub-batch plus the rank of the block among the entry's
// mask bits).  A row sums
// each entry's nine gradient components over its 16 lanes with DPP adds and stores the sums in
// the pair's slot with plain LDS stores; after the walk, two threads per entry add up the
// entry's slots in a fixed order and store the sums as that (Gaussian, tile) instance's partial
// record (instances numbered slot by slot, so a Gaussian's records are contiguous), and a
// per-Gaussian pass adds up each Gaussian's records.  The gradients need no atomics at all (LDS
// float atomic adds execute one lane at a time), every record is written once, and the sums are
// the same from run to run.  The fused
// kernel runs both passes on one workgroup: per-pixel C, T and n_contrib stay in registers, dL/dC
// is formed in registers, and the last staged forward batch (which holds the last blended entry
// of every pixel of the tile) is reused as the first backward batch.
#include "common.h"

namespace gsmi {
namespace {

constexpr int kBlock = kTileThreads;
constexpr int kBatch = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kRowsPerWave = 4;
constexpr int kBlocks4 = kWaves * kRowsPerWave;  // 4x4-pixel blocks per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct TileCtx {
    int v, g, px, py, lane, w, row, x0, y0, tx, ty;
    int list_id;   // this lane's 4x4 block, as a list index: w * 4 + row
    bool inside;
    float fpx, fpy;
    int32_t start, n;
    size_t vbase;
};

// Bit of the 16-bit block mask for block (i, j) of the tile (i, j in 0..3, 4-pixel units).
__device__ __forceinline__ int block_bit(int w, int r) {
    const int i = (w & 1) * 2 + (r & 1), j = (w >> 1) * 2 + (r >> 1);
    return j * 4 + i;
}

__device__ __forceinline__ TileCtx tile_ctx(const RasterArgs& a) {
    TileCtx c;
    c.g = a.tile_order ? a.tile_order[blockIdx.x] : (int)blockIdx.x;
    const int tpv = a.tiles_x * a.tiles_y;
    c.v = c.g / tpv;
    const int t = c.g - c.v * tpv;
    const int tx = t % a.tiles_x, ty = t / a.tiles_x;
    c.tx = tx;
    c.ty = ty;
    c.lane = threadIdx.x & (kWave - 1);
    c.w = threadIdx.x / kWave;
    c.row = c.lane >> 4;
    c.list_id = c.w * kRowsPerWave + c.row;
    c.x0 = tx * kTile;
    c.y0 = ty * kTile;
    const int l16 = c.lane & 15;
    c.px = c.x0 + (c.w & 1) * 8 + (c.row & 1) * 4 + (l16 & 3);
    c.py = c.y0 + (c.w >> 1) * 8 + (c.row >> 1) * 4 + (l16 >> 2);
    c.inside = c.px < a.width && c.py < a.height;
    c.fpx = (float)c.px + 0.5f;
    c.fpy = (float)c.py + 0.5f;
    c.start = a.ranges[2 * c.g];
    c.n = a.ranges[2 * c.g + 1] - c.start;
    c.vbase = (size_t)c.v * a.capacity;
    return c;
}

// One staged batch: records in evaluation-ready form, each 4x4 block's compacted list, and the
// per-entry gradient accumulators of the backward.
struct Batch {
    float2 xy[kBatch];      // projected centre
    float4 q[kBatch];       // (a, b, c, l): p2 = a dx^2 + b dx dy + c dy^2 + l = log2(o exp(-q/2))
    float4 oc[kBatch];      // (r, g, b, o): the walks read the colour as the first 12 bytes
    int32_t inst[kBatch];   // index of the (slot, tile) instance (backward only)
    // [0]: the 4x4 blocks the entry's alpha_min ellipse reaches; [1] (backward): the number of
    // (entry, block) pairs of the batch's earlier entries, its slot position in the log
    uint16_t meta[kBatch][2];
    union {
        uint8_t list[kBlocks4][kBatch];  // forward: batch indices
        uint16_t list16[kBlocks4][kBatch / 2];  // backward sub-batch: batch index | log slot << 8
    };
};

// The backward's log: one slot of nine gradient sums per (entry, block) pair of a sub-batch.
constexpr int kSlots = 256;
constexpr int kSub = 2 * kWave;  // entries per sub-batch at most
struct Log {
    // row stride kSlots + 1: the nine components of a slot fall in different LDS banks
    float v[9][kSlots + 1];
};

// Stage list position j of the tile into batch index k (one thread per entry): three 16-byte
// loads from the slot's packed 64-byte record.  INST: also the instance's index, inst_base +
// (row-major index of this tile in the slot's rectangle), where the backward stores the
// instance's gradient record.
template <bool INST>
__device__ __forceinline__ void stage(const RasterArgs& a, const TileCtx& c, Batch& b, int k, int32_t j) {
    const int32_t slot = a.vals[c.start + j];
    const float4* r = a.rec + 4 * (c.vbase + slot);
    const float4 r0 = r[0], r1 = r[1], r2 = r[2];  // (x, y, A, B), (C, o, r, g), (b, rect, rect, base)
    const float2 xy = make_float2(r0.x, r0.y);
    const float4 co = make_float4(r0.z, r0.w, r1.x, r1.y);
    const float amin = a.p.alpha_min;
    b.xy[k] = xy;
    b.q[k] = make_float4(-0.5f * kLog2e * co.x, -kLog2e * co.y, -0.5f * kLog2e * co.z, __log2f(co.w));
    b.oc[k] = make_float4(r1.z, r1.w, r2.x, co.w);
    if (INST) {
        const int lo = __float_as_int(r2.y), hi = __float_as_int(r2.z);
        const int tx0 = lo & 0xFFFF, ty0 = lo >> 16, tx1 = hi & 0xFFFF;
        b.inst[k] = __float_as_int(r2.w) + (c.ty - ty0) * (tx1 - tx0 + 1) + (c.tx - tx0);
    }
    // conservative block mask: the 4x4 blocks that the ellipse {q <= Q}, Q = 2 ln(o / alpha_min),
    // reaches.  Per block column the ellipse's vertical extent over the column's x-range is
    // found from its lower (convex) and upper (concave) arcs: at the range ends, or at the
    // ellipse's lowest / highest point when that lies inside.  The ellipse is taken 2 % larger in
    // Q (1 % in every radius) and every range 0.05 px wider, far beyond float32 rounding; an
    // ill-conditioned conic marks every block.
    uint32_t m = 0xFFFFu;
    const float A = co.x, B = co.y, C = co.z;
    const float det = A * C - B * B;
    if (co.w <= amin) {
        m = 0u;  // never reaches alpha_min (the projection culls these already)
    } else if (det > 0.0f && A * C <= 1e4f * det && isfinite(det)) {
        // hardware reciprocals and square roots (about 1 ulp): far inside the margins
        const float Q = 2.04f * __logf(co.w * __builtin_amdgcn_rcpf(amin));
        const float rdet = __builtin_amdgcn_rcpf(det);
        const float ex = __builtin_amdgcn_sqrtf(Q * C * rdet), ey = __builtin_amdgcn_sqrtf(Q * A * rdet);
        // dx of the lowest point (dy = -ey); the highest is at -xs
        const float xs = B * ey * __builtin_amdgcn_rcpf(A);
        const float QC = Q * C, invC = __builtin_amdgcn_rcpf(C);
        if (isfinite(ex) && isfinite(ey) && isfinite(xs)) {
            m = 0u;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float u0 = fmaxf((float)(c.x0 + 4 * i) + 0.45f - xy.x, -ex);
                const float u1 = fminf((float)(c.x0 + 4 * i) + 3.55f - xy.x, ex);
                if (!(u0 <= u1)) continue;
                const float r0 = __builtin_amdgcn_sqrtf(fmaxf(0.0f, fmaf(-det * u0, u0, QC)));
                const float r1 = __builtin_amdgcn_sqrtf(fmaxf(0.0f, fmaf(-det * u1, u1, QC)));
                float ylo = fminf(-fmaf(B, u0, r0), -fmaf(B, u1, r1)) * invC;
                float yhi = fmaxf(fmaf(-B, u0, r0), fmaf(-B, u1, r1)) * invC;
                if (u0 <= xs && xs <= u1) ylo = -ey;
                if (u0 <= -xs && -xs <= u1) yhi = ey;
                ylo += xy.y - 0.05f;
                yhi += xy.y + 0.05f;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float cy0 = (float)(c.y0 + 4 * j) + 0.5f, cy1 = cy0 + 3.0f;
                    m |= (ylo <= cy1 && yhi >= cy0) ? (1u << (4 * j + i)) : 0u;
                }
            }
        }
    }
    b.meta[k][0] = (uint16_t)m;
}

struct Lists {
    int len;      // this lane's block list length
    int max_len;  // longest of the wavefront's four block lists (the loop bound)
};

// Each wavefront compacts batch entries [0, cnt) into the lists of its four 4x4 blocks, in list
// order.  The lengths are wave-uniform (from the ballots).  Ends with a workgroup barrier so that
// every lane reads the list entries its neighbours wrote.
__device__ __forceinline__ Lists build_lists(const TileCtx& c, Batch& b, int cnt) {
    int len[kRowsPerWave] = {0, 0, 0, 0};
    const unsigned long long lt = (1ull << c.lane) - 1ull;
    for (int base = 0; base < cnt; base += kWave) {
        const int k = base + c.lane;
        const uint32_t m = k < cnt ? (uint32_t)b.meta[k][0] : 0u;
#pragma unroll
        for (int r = 0; r < kRowsPerWave; r++) {
            const bool hit = (m >> block_bit(c.w, r)) & 1u;
            const unsigned long long bal = __builtin_amdgcn_ballot_w64(hit);
            if (hit) b.list[c.w * kRowsPerWave + r][len[r] + __popcll(bal & lt)] = (uint8_t)k;
            len[r] += __popcll(bal);
        }
    }
    __syncthreads();
    Lists l;
    l.len = c.row == 0 ? len[0] : c.row == 1 ? len[1] : c.row == 2 ? len[2] : len[3];
    // wave-uniform; readfirstlane lets the compiler keep the walks' loop counters in SGPRs
    l.max_len = __builtin_amdgcn_readfirstlane(max(max(len[0], len[1]), max(len[2], len[3])));
    return l;
}

struct Fwd {
    float T, C0, C1, C2;
    int32_t last;
    float done;  // 1 once the pixel has stopped (a float, so that its test is one compare)
};

struct Counts {
    int64_t eval, blend, hit, staged;
};

// Front-to-back over this block's list of the staged batch (positions j = jbase + k).  Every
// lane evaluates the step without branches and keeps the result where it blends.
template <bool COUNT>
__device__ __forceinline__ void fwd_walk(const RasterArgs& a, const TileCtx& c, const Batch& b, Lists l, int32_t jbase,
                                         Fwd& f, Counts& cnt) {
    const float amax = a.p.alpha_max, tmin = a.p.t_min;
    const float l2amin = __log2f(a.p.alpha_min);
    const uint8_t* lst = b.list[c.list_id];
    // two list entries per iteration: both are evaluated (their alpha does not depend on T)
    // before the two compositing updates, in list order; entries are read one pair ahead
    int k0 = lst[0], k1 = lst[1];
    for (int i = 0; i < l.max_len; i += 2) {
        // ballots of single compares cost no vector instruction
        if ((__builtin_amdgcn_ballot_w64(f.done == 0.0f) & __builtin_amdgcn_ballot_w64(i < l.len)) == 0ull) break;
        const int ka = k0, kb = k1;  // past this lane's list: earlier staged entries, unused
        k0 = lst[min(i + 2, kBatch - 1)];
        k1 = lst[min(i + 3, kBatch - 1)];
        const float2 xya = b.xy[ka], xyb = b.xy[kb];
        const float4 qa = b.q[ka], qb = b.q[kb];
        const float4 oca = b.oc[ka], ocb = b.oc[kb];
        const float dxa = c.fpx - xya.x, dya = c.fpy - xya.y;
        const float dxb = c.fpx - xyb.x, dyb = c.fpy - xyb.y;
        const float p2a = fmaf(qa.x * dxa, dxa, fmaf(qa.y * dxa, dya, fmaf(qa.z * dya, dya, qa.w)));
        const float p2b = fmaf(qb.x * dxb, dxb, fmaf(qb.y * dxb, dyb, fmaf(qb.z * dyb, dyb, qb.w)));
        // exp2(p2) = o exp(-q/2) >= 0; alpha = min(alpha_max, o exp(-q/2))
        const float alphaa = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(p2a), 0.0f, amax);
        const float alphab = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(p2b), 0.0f, amax);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const float p2 = h ? p2b : p2a, alpha = h ? alphab : alphaa;
            const float4 oc = h ? ocb : oca;
            const int k = h ? kb : ka;
            const bool work = (f.done == 0.0f) & (i + h < l.len);
            const bool hit = work & (p2 >= l2amin);
            const float oma = 1.0f - alpha;
            const float Tn = f.T * oma;
            const bool below = Tn < tmin;
            const bool stop = hit & below;
            const bool blend = hit & !below;
            // zero where the pair does not blend: every lane's staged colour is finite (the lists
            // start zeroed, so even an index past a list names a staged entry), and 0 * c adds 0
            const float wgt = blend ? alpha * f.T : 0.0f;
            if (COUNT) {
                cnt.eval += work ? 1 : 0;
                cnt.hit += hit ? 1 : 0;
                cnt.blend += blend ? 1 : 0;
            }
            f.done = stop ? 1.0f : f.done;
            f.C0 = fmaf(wgt, oc.x, f.C0);
            f.C1 = fmaf(wgt, oc.y, f.C1);
            f.C2 = fmaf(wgt, oc.z, f.C2);
            f.T = blend ? Tn : f.T;
            f.last = blend ? jbase + k + 1 : f.last;
        }
    }
}

struct Bwd {
    float T, Tfin;
    float g0, g1, g2;
    float gbg;  // sum over channels of dL/dC * background
    // sum over channels of dL/dC times the colour behind the current entry: the backward needs
    // the colour behind only in that combination, and it obeys the same update
    // (B <- B + alpha (c - B) per channel gives GB <- GB + alpha (sum_ch g_ch c_ch - GB))
    float GB;
    int32_t nc;
};

// Sum over each 16-lane row with DPP adds; every lane of a row receives the row's total.
template <int CTRL>
__device__ __forceinline__ float dpp_src(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_total(float v) {
    v += dpp_src<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_src<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_src<0x141>(v);  // row_half_mirror
    v += dpp_src<0x140>(v);  // row_mirror
    return v;
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Reduce-scatter of nine per-lane values over each 16-lane row.  Afterwards every lane of bank
// (4-lane group) q of a row holds full row sums: w0 = component {0, 1, 5, 6}[q], w1 =
// component {2, 3, 7, 8}[q], w2 = component 4.  Each level halves the values a lane carries: a
// DPP add whose bank mask writes only part of the row lets the two halves (then the two quads of
// a half) keep different components.  One asm block, so that every DPP source was written at
// least two instructions earlier (the VALU-write to DPP-read hazard); the leading s_nop covers
// the inputs.
__device__ __forceinline__ void row_reduce_scatter(const float d[9], float& w0, float& w1, float& w2) {
    float r0, r1, r2, r3, r4, t0, t1, t2;
    asm volatile(
        "s_nop 1\n"
        // halves: row_ror:8 pairs lane i with lane i + 8 (mod 16); lanes 0-7 keep 0-3, lanes 8-15 keep 5-8
        "v_add_f32_dpp %0, %11, %11 row_ror:8 row_mask:0xf bank_mask:0x3\n"
        "v_add_f32_dpp %1, %12, %12 row_ror:8 row_mask:0xf bank_mask:0x3\n"
        "v_add_f32_dpp %2, %13, %13 row_ror:8 row_mask:0xf bank_mask:0x3\n"
        "v_add_f32_dpp %3, %14, %14 row_ror:8 row_mask:0xf bank_mask:0x3\n"
        "v_add_f32_dpp %0, %16, %16 row_ror:8 row_mask:0xf bank_mask:0xc\n"
        "v_add_f32_dpp %1, %17, %17 row_ror:8 row_mask:0xf bank_mask:0xc\n"
        "v_add_f32_dpp %2, %18, %18 row_ror:8 row_mask:0xf bank_mask:0xc\n"
        "v_add_f32_dpp %3, %19, %19 row_ror:8 row_mask:0xf bank_mask:0xc\n"
        "v_add_f32_dpp %4, %15, %15 row_ror:8 row_mask:0xf bank_mask:0xf\n"
        // quads of a half: row_half_mirror pairs lane i with lane 7 - i of its half
        "v_add_f32_dpp %5, %0, %0 row_half_mirror row_mask:0xf bank_mask:0x5\n"
        "v_add_f32_dpp %5, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xa\n"
        "v_add_f32_dpp %6, %2, %2 row_half_mirror row_mask:0xf bank_mask:0x5\n"
        "v_add_f32_dpp %6, %3, %3 row_half_mirror row_mask:0xf bank_mask:0xa\n"
        "v_add_f32_dpp %7, %4, %4 row_half_mirror row_mask:0xf bank_mask:0xf\n"
        // within the quad
        "v_add_f32_dpp %8, %5, %5 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
        "v_add_f32_dpp %9, %6, %6 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
        "v_add_f32_dpp %10, %7, %7 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
        "s_nop 0\n"
        "v_add_f32_dpp %8, %8, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
        "v_add_f32_dpp %9, %9, %9 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
        "v_add_f32_dpp %10, %10, %10 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(w0),
          "=&v"(w1), "=&v"(w2)
        : "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]), "v"(d[4]), "v"(d[5]), "v"(d[6]), "v"(d[7]), "v"(d[8]));
}

// The lanes of every 16-lane row that has a lane in the wave mask m.
__device__ __forceinline__ unsigned long long rows_with(unsigned long long m) {
    unsigned long long r = 0ull;
#pragma unroll
    for (int q = 0; q < 4; q++) r |= ((m >> (16 * q)) & 0xFFFFull) ? (0xFFFFull << (16 * q)) : 0ull;
    return r;
}

// Back-to-front over this block's list of the staged batch (positions j = jbase + k).  Every
// lane evaluates the step without branches; the results are kept where the pair contributes.
// BG: the background is not black (its term in dL/dalpha is needed).
template <bool BG>
__device__ __forceinline__ void bwd_walk(const RasterArgs& a, const TileCtx& c, const Batch& b, Log& log, Lists l,
                                         int32_t jbase, Bwd& s) {
    const float amax = a.p.alpha_max;
    const float l2amin = __log2f(a.p.alpha_min);
    const uint16_t* lst = b.list16[c.list_id];
    const int quad = (c.lane >> 2) & 3;
    // log row of the component this lane's quad stores as w0 after the reduce-scatter; its w1
    // component is two rows further
    float* const log_w0 = log.v[quad < 2 ? quad : quad + 3];
    uint32_t e_next = lst[max(l.max_len - 1, 0)];  // list entries are read one step ahead
    for (int i = l.max_len - 1; i >= 0; i--) {
        // past this lane's list: an earlier entry (a staged index), unused
        const int k = e_next & 0xFFu, slot = e_next >> 8;
        e_next = lst[max(i - 1, 0)];
        const int jk = jbase + k;
        // uniform over the row (the lists hold no entry past the row's largest n_contrib)
        const bool active = i < l.len;
        // ballots of single compares cost no vector instruction
        const unsigned long long am = __builtin_amdgcn_ballot_w64(active);
        if (am == 0ull) continue;
        const float2 xy = b.xy[k];
        const float4 q = b.q[k];
        const float4 oc = b.oc[k];
        // the forward's pair evaluation, for every lane
        const float dx = c.fpx - xy.x;
        const float dy = c.fpy - xy.y;
        const float bdx = q.y * dx;
        const float cdy = q.z * dy;
        const float p2 = fmaf(q.x * dx, dx, fmaf(bdx, dy, fmaf(cdy, dy, q.w)));
        const bool contrib = active & (jk < s.nc) & (p2 >= l2amin);
        const unsigned long long cm =
            am & __builtin_amdgcn_ballot_w64(jk < s.nc) & __builtin_amdgcn_ballot_w64(p2 >= l2amin);
        const float v = __builtin_amdgcn_exp2f(p2);              // o G, G = exp(-q/2)
        const bool unclamped = v <= amax;
        const float alpha = __builtin_amdgcn_fmed3f(v, 0.0f, amax);  // min(alpha_max, v)
        const float oma = 1.0f - alpha;
        const float inv = __builtin_amdgcn_rcpf(oma);  // 1 - alpha >= 1 - alpha_max > 0 where it counts
        const float Tj = s.T * inv;
        // dL/dalpha = T_j sum_ch g_ch (c_ch - B_ch) - T_final / (1 - alpha) sum_ch g_ch bg_ch
        const float ge = fmaf(s.g0, oc.x, fmaf(s.g1, oc.y, s.g2 * oc.z)) - s.GB;
        float dLda = Tj * ge;
        if (BG) dLda = fmaf(-s.Tfin * inv, s.gbg, dLda);
        // zero where the pair does not contribute (selects, so no garbage of other lanes leaks)
        const float wgt = contrib ? alpha * Tj : 0.0f;
        // o G dL/dalpha: dL/do times o, and the factor of the mean and conic gradients
        const float gv = (contrib && unclamped) ? v * dLda : 0.0f;
        // per-pixel sums whose entry-constant factors are applied once per entry when the batch
        // is flushed: dL/dmean2d = -ln2 (2 a, b; b, 2 c) (gv dx, gv dy) in the log2-scaled
        // conic, dL/d(A, B, C) = (-1/2, -1, -1/2) (gv dx dx, gv dx dy, gv dy dy), dL/do = gv / o
        const float gx = gv * dx, gy = gv * dy;
        float d[9];
        d[0] = gx;
        d[1] = gy;
        d[2] = gx * dx;
        d[3] = gx * dy;
        d[4] = gy * dy;
        d[5] = gv;
        d[6] = wgt * s.g0;
        d[7] = wgt * s.g1;
        d[8] = wgt * s.g2;
        if (contrib) {
            // colour behind the next entry: alpha c + (1 - alpha) B = B + alpha (c - B)
            s.GB = fmaf(alpha, ge, s.GB);
            s.T = Tj;
        }
        if (cm != 0ull) {
            float w0, w1, w2;
            row_reduce_scatter(d, w0, w1, w2);
            // the lanes that store: each quad's first lane, in rows with a contributing lane (the
            // lane mask is formed with scalar instructions and used directly as the exec mask);
            // the slots of other pairs stay zero
            const unsigned long long rm = rows_with(cm);
            if (__builtin_amdgcn_inverse_ballot_w64(rm & 0x1111111111111111ull)) {
                log_w0[slot] = w0;
                log_w0[slot + 2 * (kSlots + 1)] = w1;
            }
            // the first lane of a row is in quad 0, whose log_w0 is row 0: row 4 is 4 rows further
            if (__builtin_amdgcn_inverse_ballot_w64(rm & 0x0001000100010001ull)) log_w0[slot + 4 * (kSlots + 1)] = w2;
        }
    }
}

// Exclusive prefix over the staged batch of the entries' block counts (their (entry, block)
// pairs), stored in meta[k][1].  Contains workgroup barriers; the staged masks must be visible.
__device__ __forceinline__ void pair_prefix(const TileCtx& c, Batch& b, int cnt, int* s_wave) {
    const int k = threadIdx.x;
    const int pc = k < cnt ? __builtin_popcount((uint32_t)b.meta[k][0]) : 0;
    int incl = pc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (c.lane >= o) incl += y;
    }
    if (c.lane == kWave - 1) s_wave[c.w] = incl;
    __syncthreads();
    int off = 0;
#pragma unroll
    for (int q = 0; q < kWaves; q++) off += q < c.w ? s_wave[q] : 0;
    if (k < cnt) b.meta[k][1] = (uint16_t)(off + incl - pc);
    __syncthreads();
}

// The backward's sub-batch ending at batch index hi: the longest run of entries [lo, hi), at
// most kSub, whose (entry, block) pairs fit the log.  Every wavefront computes the same lo.
__device__ __forceinline__ int sub_batch(const TileCtx& c, const Batch& b, int hi) {
    const int last = hi - 1;
    const int end = (int)b.meta[last][1] + __builtin_popcount((uint32_t)b.meta[last][0]);  // pairs before hi
    const int e0 = hi - 1 - c.lane, e1 = e0 - kWave;
    const bool f0 = e0 >= 0 && end - (int)b.meta[max(e0, 0)][1] <= kSlots;
    const bool f1 = e1 >= 0 && end - (int)b.meta[max(e1, 0)][1] <= kSlots;
    // the entries that fit form a run down from hi: the prefix is non-decreasing
    return hi - __popcll(__builtin_amdgcn_ballot_w64(f0)) - __popcll(__builtin_amdgcn_ballot_w64(f1));
}

// Each wavefront compacts sub-batch entries [lo, hi) (at most kSub) into the lists of its four
// 4x4 blocks, in entry order, each list entry holding the batch index and the (entry, block)
// pair's log slot: the pairs of the sub-batch's entries before it (`first` is the pair position
// of entry lo) plus the block's rank among the entry's blocks.  Ends with a workgroup barrier:
// the previous sub-batch's gather must be done before the walk stores into the log again.
// Entries at batch index >= row_lim (this lane's row: the row's largest n_contrib minus the
// batch start) lie past every pixel of the row and stay out of its list.
__device__ __forceinline__ Lists build_sub_lists(const TileCtx& c, Batch& b, int lo, int hi, int first, int row_lim) {
    int len[kRowsPerWave] = {0, 0, 0, 0};
    int lim[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; r++) lim[r] = __builtin_amdgcn_readlane(row_lim, 16 * r);
    const unsigned long long lt = (1ull << c.lane) - 1ull;
#pragma unroll
    for (int half = 0; half < kSub / kWave; half++) {
        const int k = lo + half * kWave + c.lane;
        const uint32_t meta = k < hi ? *reinterpret_cast<const uint32_t*>(b.meta[k]) : 0u;
        const int pos = (int)(meta >> 16) - first;
#pragma unroll
        for (int r = 0; r < kRowsPerWave; r++) {
            const int bit = block_bit(c.w, r);
            const bool hit = ((meta >> bit) & 1u) && k < lim[r];
            const unsigned long long bal = __builtin_amdgcn_ballot_w64(hit);
            const int slot = pos + __builtin_popcount(meta & ((1u << bit) - 1u));
            if (hit) b.list16[c.w * kRowsPerWave + r][len[r] + __popcll(bal & lt)] = (uint16_t)(k | (slot << 8));
            len[r] += __popcll(bal);
        }
    }
    __syncthreads();
    Lists l;
    l.len = c.row == 0 ? len[0] : c.row == 1 ? len[1] : c.row == 2 ? len[2] : len[3];
    l.max_len = __builtin_amdgcn_readfirstlane(max(max(len[0], len[1]), max(len[2], len[3])));
    return l;
}

// After a sub-batch's walk (and a barrier): two threads per entry of [lo, hi) add up the entry's
// slots in slot order, clear them for the next sub-batch, apply the entry-constant factors and
// store the sums as the instance's partial record (plain stores: every instance belongs to
// exactly one tile).  Thread part 0 takes components 0-4 (mean and conic), part 1 takes 5-8
// (opacity and colour).  `first` is the slot position of entry lo.
__device__ __forceinline__ void gather_sub_batch(const RasterArgs& a, const Batch& b, Log& log, int lo, int hi,
                                                 int first) {
    const int k = lo + (int)(threadIdx.x >> 1), part = threadIdx.x & 1;
    if (k >= hi) return;
    const int c0 = part == 0 ? 0 : 5;
    const int nc = part == 0 ? 5 : 4;
    const uint32_t meta = *reinterpret_cast<const uint32_t*>(b.meta[k]);
    const int s0 = (int)(meta >> 16) - first, s1 = s0 + __builtin_popcount(meta & 0xFFFFu);
    float d[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int sl = s0; sl < s1; sl++) {
#pragma unroll
        for (int t = 0; t < 5; t++) {
            if (t < nc) {
                d[t] += log.v[c0 + t][sl];
                log.v[c0 + t][sl] = 0.0f;
            }
        }
    }
    // the bound only matters for bins and records of different calls (stale instance indices)
    if ((uint64_t)(uint32_t)b.inst[k] >= (uint64_t)a.num_instances) return;
    float* rec = a.partials + (size_t)b.inst[k] * 9 + c0;
    if (part == 0) {
        // the entry-constant factors of the mean and conic gradients (see bwd_walk)
        const float4 q = b.q[k];
        rec[0] = -kLn2 * fmaf(2.0f * q.x, d[0], q.y * d[1]);
        rec[1] = -kLn2 * fmaf(q.y, d[0], 2.0f * q.z * d[1]);
        rec[2] = d[2] * -0.5f;
        rec[3] = -d[3];
        rec[4] = d[4] * -0.5f;
    } else {
        const float o = b.oc[k].w;  // above alpha_min > 0 for every entry that reaches a pixel
        rec[0] = d[0] != 0.0f ? d[0] / o : 0.0f;
        rec[1] = d[1];
        rec[2] = d[2];
        rec[3] = d[3];
    }
}

__device__ __forceinline__ int row_max(int x) {
    for (int o = 8; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ int block_max(int x, int* s_red) {
    for (int o = kWave / 2; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
    if ((threadIdx.x & (kWave - 1)) == 0) s_red[threadIdx.x / kWave] = x;
    __syncthreads();
    int m = s_red[0];
    for (int k = 1; k < kWaves; k++) m = max(m, s_red[k]);
    __syncthreads();
    return m;
}

__device__ __forceinline__ void add_counters(int64_t* counters, Counts c) {
    for (int o = kWave / 2; o > 0; o >>= 1) {
        c.eval += __shfl_xor(c.eval, o);
        c.blend += __shfl_xor(c.blend, o);
        c.hit += __shfl_xor(c.hit, o);
        c.staged += __shfl_xor(c.staged, o);
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
        atomicAdd((unsigned long long*)&counters[0], (unsigned long long)c.eval);
        atomicAdd((unsigned long long*)&counters[1], (unsigned long long)c.blend);
        atomicAdd((unsigned long long*)&counters[2], (unsigned long long)c.hit);
        if (c.staged) atomicAdd((unsigned long long*)&counters[3], (unsigned long long)c.staged);
    }
}

// Zero the block lists once per workgroup, so that an index read past a list's end always names
// an entry that some batch staged (finite values).  Needs a barrier before the lists are read.
__device__ __forceinline__ void zero_lists(Batch& b) {
    static_assert(sizeof(b.list) == kBlock * sizeof(uint4), "one 16-byte store per thread");
    reinterpret_cast<uint4*>(&b.list[0][0])[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ void zero_log(Log& log) {
    static_assert(kSlots == kBlock, "one slot per thread");
#pragma unroll
    for (int t = 0; t < 9; t++) log.v[t][threadIdx.x] = 0.0f;
}

// Forward over the whole tile list.  On return *last_b0 is the list position of the last staged
// batch (-1 if none) and *last_cnt its entry count.
template <bool COUNT, bool INST>
__device__ __forceinline__ void forward_tile(const RasterArgs& a, const TileCtx& c, Batch& b, Fwd& f, Counts& cnt,
                                             int32_t* last_b0, int* last_cnt) {
    *last_b0 = -1;
    *last_cnt = 0;
    for (int32_t b0 = 0; b0 < c.n; b0 += kBatch) {
        if (__syncthreads_count(f.done != 0.0f) == kBlock) break;
        const int cnt_b = min(kBatch, c.n - b0);
        if ((int)threadIdx.x < cnt_b) stage<INST>(a, c, b, threadIdx.x, b0 + threadIdx.x);
        if (COUNT && threadIdx.x == 0) cnt.staged += cnt_b;
        __syncthreads();
        const Lists l = build_lists(c, b, cnt_b);
        fwd_walk<COUNT>(a, c, b, l, b0, f, cnt);
        *last_b0 = b0;
        *last_cnt = cnt_b;
    }
}

// Backward over list positions [0, maxnc); the batch starting at `resident_b0` (with
// `resident_cnt` entries) is already staged.  The log must be zero on entry; it is zero again on
// return.
template <bool BG, bool COUNT = false>
__device__ __forceinline__ void backward_tile(const RasterArgs& a, const TileCtx& c, Batch& b, Log& log, int* s_wave,
                                              int32_t maxnc, int32_t resident_b0, int resident_cnt, Bwd& s) {
    const int row_nc = row_max(s.nc);
    // the instances of list positions [maxnc, n) get zero records: the walk never reaches them
    for (int32_t j = maxnc + (int32_t)threadIdx.x; j < c.n; j += kBlock) {
        const int32_t slot = a.vals[c.start + j];
        const float4 r2 = a.rec[4 * (c.vbase + slot) + 2];
        const int lo = __float_as_int(r2.y), hi = __float_as_int(r2.z);
        const int tx0 = lo & 0xFFFF, ty0 = lo >> 16, tx1 = hi & 0xFFFF;
        const int inst = __float_as_int(r2.w) + (c.ty - ty0) * (tx1 - tx0 + 1) + (c.tx - tx0);
        if ((uint64_t)(uint32_t)inst < (uint64_t)a.num_instances) {
            float* rec = a.partials + (size_t)inst * 9;
#pragma unroll
            for (int t = 0; t < 9; t++) rec[t] = 0.0f;
        }
    }
    if (maxnc <= 0) return;
    for (int32_t b0 = ((maxnc - 1) / kBatch) * kBatch; b0 >= 0; b0 -= kBatch) {
        // entries past maxnc contribute nowhere
        int cnt_b = min(resident_cnt, maxnc - b0);
        __syncthreads();  // the previous batch's gather is done with the staged records
        if (b0 != resident_b0) {
            cnt_b = min(kBatch, maxnc - b0);
            if ((int)threadIdx.x < cnt_b) stage<true>(a, c, b, threadIdx.x, b0 + threadIdx.x);
            // the restaged entries (diagnostics of the counting variant)
            if (COUNT && threadIdx.x == 0) atomicAdd((unsigned long long*)&a.counters[3], (unsigned long long)cnt_b);
            __syncthreads();
        }
        pair_prefix(c, b, cnt_b, s_wave);
        for (int hi = cnt_b; hi > 0;) {
            const int lo = sub_batch(c, b, hi);
            const int first = __builtin_amdgcn_readfirstlane((int)b.meta[lo][1]);
            const Lists l = build_sub_lists(c, b, lo, hi, first, row_nc - b0);
            bwd_walk<BG>(a, c, b, log, l, b0, s);
            __syncthreads();
            gather_sub_batch(a, b, log, lo, hi, first);
            hi = lo;
        }
        resident_b0 = -1;
    }
}

template <bool COUNT>
__global__ __launch_bounds__(kBlock) void raster_fwd_kernel(RasterArgs a, float* image, float* t_final,
                                                            int32_t* n_contrib) {
    __shared__ Batch b;
    const TileCtx c = tile_ctx(a);
    Fwd f{1.0f, 0.0f, 0.0f, 0.0f, 0, c.inside ? 0.0f : 1.0f};
    Counts cnt{0, 0, 0, 0};
    int32_t last_b0;
    int last_cnt;
    zero_lists(b);
    forward_tile<COUNT, false>(a, c, b, f, cnt, &last_b0, &last_cnt);
    if (COUNT) add_counters(a.counters, cnt);
    if (!c.inside) return;
    const size_t plane = (size_t)a.width * a.height;
    const size_t p = (size_t)c.py * a.width + c.px;
    image[(size_t)(3 * c.v + 0) * plane + p] = fmaf(f.T, a.p.bg[0], f.C0);
    image[(size_t)(3 * c.v + 1) * plane + p] = fmaf(f.T, a.p.bg[1], f.C1);
    image[(size_t)(3 * c.v + 2) * plane + p] = fmaf(f.T, a.p.bg[2], f.C2);
    t_final[(size_t)c.v * plane + p] = f.T;
    n_contrib[(size_t)c.v * plane + p] = f.last;
}

__global__ __launch_bounds__(256) void loss_l1_kernel(int64_t n, const float* image, const float* target, float scale,
                                                      float* dl, float* loss_sum) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    float l = 0.0f;
    if (i < n) {
        const float d = image[i] - target[i];
        dl[i] = d > 0.0f ? scale : (d < 0.0f ? -scale : 0.0f);
        l = scale * fabsf(d);
    }
    if (loss_sum) {
        l = wave_sum(l);
        if ((threadIdx.x & (kWave - 1)) == 0 && l != 0.0f) atomicAdd(loss_sum, l);
    }
}

// The fused call's loss sum: an integer accumulator in units of 2^-20, cleared before the
// kernel and added to the caller's float afterwards.
constexpr double kLossFix = 1048576.0;

__global__ void loss_acc_clear_kernel(long long* acc) { *acc = 0; }

__global__ void loss_acc_finish_kernel(const long long* acc, float* loss_sum) {
    *loss_sum += (float)((double)*acc / kLossFix);
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

// Per-Gaussian gather of the backward: the gradient of a visible slot is the sum of its
// instances' partial records, which lie contiguously at [inst_base, inst_base + n_tiles).  A lane
// adds up the records of its own slot in instance order; a slot with more than kHeavy records
// (a large splat) is added up by the whole wavefront instead (each lane a strided share, then a
// fixed-order wavefront reduction), so that one large splat does not hold up 63 lanes.  A slot
// with more than kHugeSlot records is listed and added up by a workgroup of its own
// (reduce_huge_kernel): in a large scene such splats are many and neighbours in index order, and
// one wavefront would add them up one after another.  Every sum is taken in a fixed order.
constexpr int kHeavy = 16;

__device__ __forceinline__ void store_grad(const Grads& g, size_t i, const float d[9]) {
    g.d_mean2d[i] = make_float2(d[0], d[1]);
    g.d_conic[3 * i] = d[2];
    g.d_conic[3 * i + 1] = d[3];
    g.d_conic[3 * i + 2] = d[4];
    g.d_opacity[i] = d[5];
    g.d_color[3 * i] = d[6];
    g.d_color[3 * i + 1] = d[7];
    g.d_color[3 * i + 2] = d[8];
}

__global__ __launch_bounds__(256) void reduce_partials_kernel(const int32_t* vis_count, int32_t V, int32_t capacity,
                                                              const int32_t* inst_base, const int32_t* n_tiles,
                                                              const float* partials, int64_t num_instances,
                                                              int4* huge_slots, int32_t* huge_count, int32_t huge_cap,
                                                              Grads g) {
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t wave = (int32_t)(blockIdx.x * (256 / kWave) + threadIdx.x / kWave);
    const int32_t waves = (int32_t)(gridDim.x * (256 / kWave));
    for (int v = 0; v < V; v++) {
        const int32_t cnt = vis_count[v];
        const size_t base = (size_t)v * capacity;
        // wavefront-uniform loop over groups of 64 consecutive slots
        for (int32_t s0 = wave * kWave; s0 < cnt; s0 += waves * kWave) {
            const int32_t s = s0 + lane;
            const size_t i = base + s;
            int64_t off = 0;
            int n = 0;
            if (s < cnt) {
                off = inst_base[i];
                // clamped to the records that exist (only a stale projection could reach past them)
                n = (off < 0 || off > num_instances) ? 0 : (int)min((int64_t)n_tiles[i], num_instances - off);
            }
            bool heavy = n > kHeavy, listed = false;
            if (n > kHugeSlot) {
                const int h = atomicAdd(huge_count, 1);
                if (h < huge_cap) {
                    huge_slots[h] = make_int4((int)i, (int)off, n, 0);  // added up by reduce_huge_kernel
                    listed = true;
                    heavy = false;
                }
                // a full list (never, with the list sized for the instances): summed here
            }
            if (s < cnt && !heavy && !listed) {
                const float* rec = partials + (size_t)off * 9;
                float d[9];
#pragma unroll
                for (int t = 0; t < 9; t++) d[t] = 0.0f;
                for (int k = 0; k < n; k++)
#pragma unroll
                    for (int t = 0; t < 9; t++) d[t] += rec[9 * k + t];
                store_grad(g, i, d);
            }
            unsigned long long hm = __builtin_amdgcn_ballot_w64(heavy);
            while (hm != 0ull) {
                const int src = __ffsll((long long)hm) - 1;
                hm &= hm - 1ull;
                const int64_t off0 = __shfl((long long)off, src);
                const int n0 = __shfl(n, src);
                const float* rec = partials + (size_t)off0 * 9;
                float d[9];
#pragma unroll
                for (int t = 0; t < 9; t++) d[t] = 0.0f;
                for (int k = lane; k < n0; k += kWave)
#pragma unroll
                    for (int t = 0; t < 9; t++) d[t] += rec[9 * k + t];
#pragma unroll
                for (int t = 0; t < 9; t++)
                    for (int o = kWave / 2; o > 0; o >>= 1) d[t] += __shfl_xor(d[t], o);
                if (lane == src) store_grad(g, i, d);
            }
        }
    }
}

// A listed slot's records summed by one workgroup: each thread a strided share in record order,
// then a fixed pairwise tree over the threads.
__global__ __launch_bounds__(256) void reduce_huge_kernel(const int4* huge_slots, const int32_t* huge_count,
                                                          int32_t huge_cap, const float* partials, Grads g) {
    __shared__ float s_sum[9][256];
    const int32_t cnt = min(*huge_count, huge_cap);
    for (int32_t h = blockIdx.x; h < cnt; h += gridDim.x) {
        const int4 e = huge_slots[h];
        const float* rec = partials + (size_t)e.y * 9;
        float d[9];
#pragma unroll
        for (int t = 0; t < 9; t++) d[t] = 0.0f;
        for (int k = threadIdx.x; k < e.z; k += 256)
#pragma unroll
            for (int t = 0; t < 9; t++) d[t] += rec[9 * k + t];
#pragma unroll
        for (int t = 0; t < 9; t++) s_sum[t][threadIdx.x] = d[t];
        __syncthreads();
        for (int o = 128; o > 0; o >>= 1) {
            if ((int)threadIdx.x < o) {
#pragma unroll
                for (int t = 0; t < 9; t++) s_sum[t][threadIdx.x] += s_sum[t][threadIdx.x + o];
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
#pragma unroll
            for (int t = 0; t < 9; t++) d[t] = s_sum[t][0];
            store_grad(g, (size_t)e.x, d);
        }
        __syncthreads();
    }
}

template <bool BG>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(6))) void raster_bwd_kernel(
    RasterArgs a, const float* t_final, const int32_t* n_contrib, const float* dl, Grads gr) {
    __shared__ Batch b;
    __shared__ Log log;
    __shared__ int s_red[kWaves];
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.huge_count = 0;  // the gather appends after this kernel
    const TileCtx c = tile_ctx(a);
    const size_t plane = (size_t)a.width * a.height;
    const size_t p = (size_t)c.py * a.width + c.px;
    Bwd s{};
    if (c.inside) {
        s.T = t_final[(size_t)c.v * plane + p];
        s.nc = n_contrib[(size_t)c.v * plane + p];
        s.g0 = dl[(size_t)(3 * c.v + 0) * plane + p];
        s.g1 = dl[(size_t)(3 * c.v + 1) * plane + p];
        s.g2 = dl[(size_t)(3 * c.v + 2) * plane + p];
    } else {
        s.T = 1.0f;
        s.nc = 0;
        s.g0 = s.g1 = s.g2 = 0.0f;
    }
    s.Tfin = s.T;
    s.gbg = fmaf(s.g0, a.p.bg[0], fmaf(s.g1, a.p.bg[1], s.g2 * a.p.bg[2]));
    s.GB = 0.0f;
    zero_log(log);
    zero_lists(b);
    const int maxnc = block_max(s.nc, s_red);
    backward_tile<BG>(a, c, b, log, s_red, maxnc, -1, 0, s);
}

template <bool COUNT, bool BG>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(6))) void raster_fused_kernel(RasterArgs a, int mode, const float* tgt, float scale,
                                                              float* image, float* loss_sum, Grads gr) {
    __shared__ Batch b;
    __shared__ Log log;
    __shared__ int s_red[kWaves];
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.huge_count = 0;  // the gather appends after this kernel
    const TileCtx c = tile_ctx(a);
    Fwd f{1.0f, 0.0f, 0.0f, 0.0f, 0, c.inside ? 0.0f : 1.0f};
    Counts cnt{0, 0, 0, 0};
    int32_t last_b0;
    int last_cnt;
    zero_log(log);
    zero_lists(b);
    forward_tile<COUNT, true>(a, c, b, f, cnt, &last_b0, &last_cnt);
    if (COUNT) add_counters(a.counters, cnt);
    // loss gradient in registers
    const size_t plane = (size_t)a.width * a.height;
    const size_t p = (size_t)c.py * a.width + c.px;
    Bwd s{};
    s.T = f.T;
    s.Tfin = f.T;
    s.nc = c.inside ? f.last : 0;
    s.GB = 0.0f;
    s.g0 = s.g1 = s.g2 = 0.0f;
    float lsum = 0.0f;
    if (c.inside) {
        const float C0 = fmaf(f.T, a.p.bg[0], f.C0);
        const float C1 = fmaf(f.T, a.p.bg[1], f.C1);
        const float C2 = fmaf(f.T, a.p.bg[2], f.C2);
        if (image) {
            image[(size_t)(3 * c.v + 0) * plane + p] = C0;
            image[(size_t)(3 * c.v + 1) * plane + p] = C1;
            image[(size_t)(3 * c.v + 2) * plane + p] = C2;
        }
        const float t0 = tgt[(size_t)(3 * c.v + 0) * plane + p];
        const float t1 = tgt[(size_t)(3 * c.v + 1) * plane + p];
        const float t2 = tgt[(size_t)(3 * c.v + 2) * plane + p];
        if (mode == GS_LOSS_L1) {
            const float d0 = C0 - t0, d1 = C1 - t1, d2 = C2 - t2;
            s.g0 = d0 > 0.0f ? scale : (d0 < 0.0f ? -scale : 0.0f);
            s.g1 = d1 > 0.0f ? scale : (d1 < 0.0f ? -scale : 0.0f);
            s.g2 = d2 > 0.0f ? scale : (d2 < 0.0f ? -scale : 0.0f);
            lsum = scale * (fabsf(d0) + fabsf(d1) + fabsf(d2));
        } else {
            s.g0 = t0;
            s.g1 = t1;
            s.g2 = t2;
        }
    }
    if (loss_sum && mode == GS_LOSS_L1) {
        // in fixed point (2^-20): integer sums do not depend on the order of the workgroups
        lsum = wave_sum(lsum);
        if (c.lane == 0 && lsum != 0.0f)
            atomicAdd(reinterpret_cast<unsigned long long*>(a.loss_acc),
                      (unsigned long long)(long long)llrint((double)lsum * kLossFix));
    }
    const int maxnc = block_max(s.nc, s_red);
    // every pixel's last blended entry lies in the last staged batch, so it is still resident
    s.gbg = fmaf(s.g0, a.p.bg[0], fmaf(s.g1, a.p.bg[1], s.g2 * a.p.bg[2]));
    backward_tile<BG, COUNT>(a, c, b, log, s_red, maxnc, last_b0, last_cnt, s);
}

}  // namespace

int32_t fused_lds_entries() { return kBatch; }

// The carving order of the backward's workspace (256-byte aligned pieces): partial records,
// huge-slot count, huge-slot list.
size_t raster_ws_bytes(int64_t instances) {
    const auto a256 = [](size_t b) { return (b + 255) & ~size_t(255); };
    return a256(sizeof(float) * 9 * (size_t)instances) + a256(sizeof(int32_t)) +
           a256(sizeof(int4) * (size_t)huge_slot_cap(instances)) + a256(sizeof(long long));
}

hipError_t launch_raster_fwd(const RasterArgs& a, float* image, float* t_final, int32_t* n_contrib, hipStream_t s) {
    const unsigned nblocks = (unsigned)(a.V * a.tiles_x * a.tiles_y);
    if (a.counters)
        hipLaunchKernelGGL(raster_fwd_kernel<true>, dim3(nblocks), dim3(kBlock), 0, s, a, image, t_final, n_contrib);
    else
        hipLaunchKernelGGL(raster_fwd_kernel<false>, dim3(nblocks), dim3(kBlock), 0, s, a, image, t_final, n_contrib);
    return hipGetLastError();
}

hipError_t launch_loss_l1(int64_t n, const float* image, const float* target, float scale, float* dl, float* loss_sum,
                          hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(loss_l1_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, image, target, scale, dl,
                       loss_sum);
    return hipGetLastError();
}

static unsigned grid_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    if (b > 8192) b = 8192;
    if (b < 1) b = 1;
    return (unsigned)b;
}

// Run a backward kernel, then gather the partial records per Gaussian.  The backward stores the
// record of every instance in its lists; with capped lists the instances the cap dropped are in
// none, so the records are zeroed first.
template <typename Launch>
static hipError_t with_partials(const RasterArgs& a, Grads g, hipStream_t s, Launch launch) {
    const int64_t n = a.num_instances * 9;
    if (a.capped && n > 0) hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, a.partials, n);
    launch();
    hipLaunchKernelGGL(reduce_partials_kernel, dim3(grid_for(a.capacity)), dim3(256), 0, s, a.vis_count, a.V,
                       a.capacity, a.inst_base, a.n_tiles, a.partials, a.num_instances, a.huge_slots, a.huge_count,
                       a.huge_cap, g);
    const int32_t grid = a.huge_cap < 1024 ? a.huge_cap : 1024;
    hipLaunchKernelGGL(reduce_huge_kernel, dim3(grid), dim3(256), 0, s, a.huge_slots, a.huge_count, a.huge_cap,
                       a.partials, g);
    return hipGetLastError();
}

hipError_t launch_raster_bwd(const RasterArgs& a, const float* /*image*/, const float* t_final, const int32_t* n_contrib,
                             const float* dl, Grads g, hipStream_t s) {
    const unsigned nblocks = (unsigned)(a.V * a.tiles_x * a.tiles_y);
    const bool bg = a.p.bg[0] != 0.0f || a.p.bg[1] != 0.0f || a.p.bg[2] != 0.0f;
    return with_partials(a, g, s, [&] {
        if (bg)
            hipLaunchKernelGGL(raster_bwd_kernel<true>, dim3(nblocks), dim3(kBlock), 0, s, a, t_final, n_contrib, dl, g);
        else
            hipLaunchKernelGGL(raster_bwd_kernel<false>, dim3(nblocks), dim3(kBlock), 0, s, a, t_final, n_contrib, dl,
                               g);
    });
}

static hipError_t launch_raster_fused_kernels(const RasterArgs& a, int mode, const float* target_or_dl, float scale,
                                              float* image, float* loss_sum, Grads g, hipStream_t s,
                                              unsigned nblocks, bool bg) {
    return with_partials(a, g, s, [&] {
        if (a.counters && bg)
            hipLaunchKernelGGL((raster_fused_kernel<true, true>), dim3(nblocks), dim3(kBlock), 0, s, a, mode,
                               target_or_dl, scale, image, loss_sum, g);
        else if (a.counters)
            hipLaunchKernelGGL((raster_fused_kernel<true, false>), dim3(nblocks), dim3(kBlock), 0, s, a, mode,
                               target_or_dl, scale, image, loss_sum, g);
        else if (bg)
            hipLaunchKernelGGL((raster_fused_kernel<false, true>), dim3(nblocks), dim3(kBlock), 0, s, a, mode,
                               target_or_dl, scale, image, loss_sum, g);
        else
            hipLaunchKernelGGL((raster_fused_kernel<false, false>), dim3(nblocks), dim3(kBlock), 0, s, a, mode,
                               target_or_dl, scale, image, loss_sum, g);
    });
}

hipError_t launch_raster_fused(const RasterArgs& a, int mode, const float* target_or_dl, float scale, float* image,
                               float* loss_sum, Grads g, hipStream_t s) {
    const unsigned nblocks = (unsigned)(a.V * a.tiles_x * a.tiles_y);
    const bool bg = a.p.bg[0] != 0.0f || a.p.bg[1] != 0.0f || a.p.bg[2] != 0.0f;
    const bool lsum = loss_sum && mode == GS_LOSS_L1;
    if (lsum) hipLaunchKernelGGL(loss_acc_clear_kernel, dim3(1), dim3(1), 0, s, a.loss_acc);
    const hipError_t e = launch_raster_fused_kernels(a, mode, target_or_dl, scale, image, loss_sum, g, s, nblocks, bg);
    if (e != hipSuccess) return e;
    if (lsum) hipLaunchKernelGGL(loss_acc_finish_kernel, dim3(1), dim3(1), 0, s, a.loss_acc, loss_sum);
    return hipGetLastError();
}

}  // namespace gsmi
