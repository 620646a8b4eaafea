// Internal declarations of the gfx950 HIP implementation behind include/gsmi.h.
//
// Every kernel is compiled with -ffp-contract=off: multiply-adds are fused only where an
// explicit fmaf() says so, so that a formula evaluated in two kernels (the forward and the
// backward recompute of alpha) rounds identically in both.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gsmi.h"

namespace gsmi {

constexpr int kTile = GS_TILE;            // 16x16 pixels per tile
constexpr int kTileThreads = kTile * kTile;  // one thread per pixel, 4 wavefronts of 64
constexpr int kWave = 64;
// guard band of the per-view frustum cull, as a fraction of the image size beyond each edge
constexpr float kGuard = 0.15f;

// Camera as the kernels read it (kernel-argument struct, by value).
struct CamDev {
    int32_t width, height, tiles_x, tiles_y;
    float fx, fy, cx, cy;
    float R[9];
    float t[3];
    float campos[3];
};

struct CamArray {
    CamDev c[GS_MAX_VIEWS];
};

struct ParamsDev {
    float znear, eps2d, alpha_min, alpha_max, t_min;
    float bg[3];
    int32_t sh_degree, tile_cap;
};

// ---------------------------------------------------------------------------------------
// Pair evaluation shared by every rasterizer: the forward, the backward's recomputation and
// the fused kernel call this one function, so they take bit-identical decisions.
// q = A dx^2 + 2 B dx dy + C dy^2 with d = pixel centre - projected centre;
// G = exp(-q/2); v = o G; alpha = min(alpha_max, v).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float pair_power(float dx, float dy, float A, float B, float C) {
    const float cdy = C * dy;
    const float bdx = B * dx;
    const float q = fmaf(A * dx, dx, fmaf(2.0f * bdx, dy, cdy * dy));
    return -0.5f * q;
}

__device__ __forceinline__ float pair_gauss(float power) { return __expf(power); }

// 1 - alpha.  Unclamped (v = o G <= alpha_max) it is 1 - o G with a single rounding, which
// keeps the relative error of a small 1 - alpha (alpha near alpha_max) from growing by the
// rounding of alpha itself; clamped it is 1 - alpha_max.
__device__ __forceinline__ float one_minus_alpha(float o, float G, float v, float amax) {
    return v <= amax ? fmaf(-o, G, 1.0f) : 1.0f - amax;
}

// ---------------------------------------------------------------------------------------
// Launchers (defined next to their kernels).
// ---------------------------------------------------------------------------------------
// The counts the binning sizes its launches from, in the order they are copied to the host:
// instances and visible slots per view, and the smallest float32 bit pattern of the visible
// depths of all views with the complement of the largest.
struct CountSummary {
    int64_t inst[GS_MAX_VIEWS];
    int32_t vis[GS_MAX_VIEWS];
    uint32_t bits[2];
};

struct ProjectArgs {
    int32_t n, V, capacity;
    const float *means, *log_scales, *quats, *logits, *sh;
    CamArray cams;
    ParamsDev p;
    int32_t* vis_count;
    int64_t* inst_count;
    int32_t* vis_ids;
    float2* mean2d;          // optional (NULL: not written), as conic_opacity and color
    float4* conic_opacity;
    float* color;
    float* depth;
    ushort4* tile_rect;
    int32_t* n_tiles;
    int32_t* inst_base;
    float4* raster_rec;      // [V][capacity][4]
    // workspace
    int32_t* block_counts;   // [2V][nw]: visible slots per wavefront of 64 Gaussians (rows 0..V-1), then
                             // instances per wavefront
    int32_t* block_offsets;  // [2V][nw]: exclusive scans of the rows of block_counts
    int32_t* row_totals;     // [2V]: visible slots per view, then instances per view
    int32_t* scan_partials;  // scan workspace
    uint2* block_depth;      // [nw] (smallest, complement of largest) visible depth bits per wavefront;
                             // NULL: not computed
    CountSummary* summary;   // device copy of the counts (written when block_depth is set)
    uint8_t* seen;           // [nw * 64] 1 where some view sees the Gaussian (counting pass)
    int64_t* inst_partials;  // [V][project_partials()] partial instance sums
    uint2* depth_partials;   // [project_partials()] partial depth ranges
};
// The counting pass, the block scans and (with block_depth) the count summary: afterwards
// vis/inst counts are final and the summary may be copied out while the writing pass runs.
hipError_t launch_project_count(const ProjectArgs& a, hipStream_t s);
// The writing pass (records of the visible slots).
hipError_t launch_project_write(const ProjectArgs& a, hipStream_t s);
size_t project_ws_bytes(int32_t n, int32_t V);
int32_t project_count_waves(int32_t n);
int32_t project_partials();

// Backward of the projection: per-slot 2D gradients of V views -> per-Gaussian parameter
// gradients (summed over views), one thread per Gaussian.
struct ProjectBwdArgs {
    int32_t n, V, capacity;
    const float *means, *log_scales, *quats, *logits, *sh;
    CamArray cams;
    ParamsDev p;
    const int32_t* vis_count;
    const int32_t* vis_ids;
    const float2* d_mean2d;
    const float* d_conic;
    const float* d_opacity;
    const float* d_color;
    float *g_means, *g_log_scales, *g_quats, *g_logits, *g_sh;
    // null: every gradient row is written (zeros for Gaussians no view sees); otherwise
    // seen_out[i] = 1 for a Gaussian some view sees, 0 for the others, whose rows are not written
    uint8_t* seen_out;
};
hipError_t launch_project_bwd(const ProjectBwdArgs& a, hipStream_t s);

// Exclusive scan of `rows` independent int32 rows of length n (row r at in + r*n):
// out[r][i] = sum_{k<i} in[r][k]; totals[r] = sum of row r (totals may be null).
// In-place exclusive scan of n int32 values by one workgroup (n up to a few hundred thousand).
hipError_t launch_scan_small(int32_t* a, int32_t n, hipStream_t s);
hipError_t launch_scan_rows(const int32_t* in, int32_t* out, int32_t* totals, int32_t n, int32_t rows,
                            int32_t* partials, hipStream_t s);
size_t scan_partials_bytes(int32_t n, int32_t rows);

// LSD radix sort of (uint32 key, uint32 value) pairs over bits [0, bits).  Sorts keys/vals in
// place through the alternate buffers; the result lands in keys/vals when the number of
// passes is even and in keys_alt/vals_alt when it is odd (radix_passes() tells which).
int radix_passes(int bits);
hipError_t launch_radix_sort(uint32_t* keys, uint32_t* vals, uint32_t* keys_alt, uint32_t* vals_alt, int32_t n,
                             int bits, int32_t* hist, int32_t* partials, hipStream_t s);
size_t radix_hist_bytes(int32_t n);
size_t radix_partials_bytes(int32_t n);

// Binning helpers.
constexpr int kDepthRangeBlocks = 512;
struct BinReadback {
    int64_t inst[GS_MAX_VIEWS];
    int32_t vis[GS_MAX_VIEWS];
    uint32_t bits[2];  // smallest float32 bit pattern of the visible depths, complement of the largest
    uint2 partial[kDepthRangeBlocks];  // per-block partial depth ranges (device only; not read back)
};
hipError_t launch_bin_counts(const int32_t* vis_count, const int64_t* inst_count, int32_t V, const float* depth,
                             int32_t capacity, BinReadback* out, hipStream_t s);
// Also clears zero[0, n_zero).
hipError_t launch_depth_keys(const float* depth, const int64_t* view_first, int32_t V, int32_t capacity,
                             int32_t total, uint32_t key_min, uint32_t* keys, uint32_t* vals, int32_t* zero,
                             int32_t n_zero, hipStream_t s);
// Instances of the depth-sorted slots: chunk_offsets holds emit_chunks(total) ints of workspace.
int32_t emit_chunks(int32_t total);
// Rectangles of more than kHugeRect tiles are listed (huge_list, two int4 per entry, at most
// huge_rect_cap(M) entries; huge_count one int) and written by a workgroup each.
constexpr int kHugeRect = 256;
inline int32_t huge_rect_cap(int64_t instances) { return (int32_t)(instances / kHugeRect + 1); }
// rect_lo / rect_hi: total words each of workspace (the rectangles in depth order).
hipError_t launch_emit(const uint32_t* packed, const ushort4* rect, int32_t capacity, int32_t total, int32_t tiles_x,
                       int32_t tiles_per_view, int32_t M, int32_t* chunk_offsets, uint32_t* rect_lo, uint32_t* rect_hi,
                       int4* huge_list, int32_t* huge_count, int32_t huge_cap, uint32_t* tile_keys, int32_t* vals,
                       hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s);
hipError_t launch_ranges(const uint32_t* tile_keys, int32_t M, int32_t* ranges, hipStream_t s);
// Heavy-first permutation of the tiles (stable counting sort on a 5-bit length bucket); hist
// holds tile_order_hist_ints(n_tiles_total) ints of workspace.
size_t tile_order_hist_ints(int32_t n_tiles_total);
hipError_t launch_tile_order(const int32_t* ranges, int32_t n_tiles_total, int32_t* hist, int32_t* order,
                             hipStream_t s);
hipError_t launch_cap_count(const int32_t* ranges, int32_t n_tiles_total, int32_t K, int32_t* kept, hipStream_t s);
// slot_bits: V * capacity words of workspace (the visible slots' scores); scratch_bits: one word
// per instance (the scores of lists longer than the select keeps in LDS).  The scores come from
// conic_opacity, or from the packed records rec when conic_opacity is NULL.
hipError_t launch_cap_select(const int32_t* ranges, const int32_t* vals, const float4* conic_opacity,
                             const float4* rec, const int32_t* vis_count, int32_t V, int32_t capacity, int32_t tiles_per_view,
                             int32_t n_tiles_total, int32_t K, const int32_t* cap_offsets, const int32_t* tile_order,
                             int32_t* vals_capped, int32_t* ranges_capped, uint32_t* slot_bits,
                             uint32_t* scratch_bits, hipStream_t s);

// Rasterizers.
struct RasterArgs {
    int32_t V, width, height, tiles_x, tiles_y, capacity;
    ParamsDev p;
    const int32_t* ranges;   // [V*T][2]
    const int32_t* vals;
    const float4* rec;           // [V][capacity][4] packed records (x y A B | C o r g | b rect rect base | ...)
    const int32_t* vis_count;
    const int32_t* tile_order;   // optional: workgroup -> global tile (heavy tiles first)
    const int32_t* inst_base;    // backward: first instance index of each slot
    const int32_t* n_tiles;      // backward: instances per slot
    float* partials;             // backward: [instances][9] per-instance gradient records
    int64_t num_instances;       // backward: records in use
    int32_t capped;              // the lists are the top-K capped ones (some instances are in none)
    int64_t* counters;           // optional
    // backward: slots with more than kHugeSlot records, listed (int4 (slot index, first record,
    // records, 0)) for a workgroup each; the raster kernel clears the count
    int4* huge_slots;
    int32_t* huge_count;
    long long* loss_acc;         // fused call's loss sum in fixed point (workspace)
    int32_t huge_cap;
};
constexpr int kHugeSlot = 256;
inline int32_t huge_slot_cap(int64_t instances) { return (int32_t)(instances / kHugeSlot + 1); }
// Bytes of the backward's workspace for an instance count: partial records, then the huge-slot
// list and its count.
size_t raster_ws_bytes(int64_t instances);
hipError_t launch_raster_fwd(const RasterArgs& a, float* image, float* t_final, int32_t* n_contrib, hipStream_t s);
hipError_t launch_loss_l1(int64_t n, const float* image, const float* target, float scale, float* dl, float* loss_sum,
                          hipStream_t s);
struct Grads {
    float2* d_mean2d;
    float* d_conic;
    float* d_opacity;
    float* d_color;
};
hipError_t launch_raster_bwd(const RasterArgs& a, const float* image, const float* t_final, const int32_t* n_contrib,
                             const float* dl, Grads g, hipStream_t s);
hipError_t launch_raster_fused(const RasterArgs& a, int mode, const float* target_or_dl, float scale, float* image,
                               float* loss_sum, Grads g, hipStream_t s);

// F2: sparse 2D gradient records.  Slot-indexed inputs ([V][capacity]) and owner outputs
// ([V][n_owner]) in the layout of gs_grads2d.
struct GradsIn {
    const float* d_mean2d;  // [..][2]
    const float* d_conic;   // [..][3]
    const float* d_opacity;
    const float* d_color;   // [..][3]
};
struct GradsOut {
    float* d_mean2d;
    float* d_conic;
    float* d_opacity;
    float* d_color;
};
size_t encode_workspace_bytes(int32_t capacity, int32_t V);
hipError_t launch_grad_encode(int32_t V, int32_t capacity, const int32_t* vis_count, const int32_t* vis_ids,
                              GradsIn g, int32_t* keys, float* records, int32_t* view_offset, void* ws,
                              hipStream_t s);
hipError_t launch_grad_decode(int32_t V, int32_t n_owner, int64_t max_records, const int32_t* view_offset,
                              const int32_t* keys, const float* records, GradsOut o, hipStream_t s);

// F3: composition of P <= kMaxPartials partial renders (C [V][3][H][W], T [V][H][W]), front to back.
constexpr int kMaxPartials = 16;
struct ComposeArgs {
    const float* c[kMaxPartials];
    const float* t[kMaxPartials];
    float bg[3];
};
hipError_t launch_compose(int32_t P, int32_t V, int64_t plane, const ComposeArgs& a, float* image, float* t_out,
                          hipStream_t s);

// F4: Adam over parameter groups ([rows][n] float32 each), dense or deferred.
constexpr int kMaxAdamGroups = 8;
struct AdamGroup {
    float* param;
    const float* grad;
    float* m;
    float* v;
    int32_t rows;
    float lr;
};
struct AdamHyper {
    float beta1, beta2, eps;
};
struct AdamArgs {
    AdamGroup groups[kMaxAdamGroups];
    int32_t n_groups;
    AdamHyper h;
};
hipError_t launch_adam_step(const AdamArgs& a, int64_t n, int32_t t, int32_t* last_step, const int32_t* active,
                            int64_t n_active, hipStream_t s);
// Deferred step whose candidates are the Gaussians with seen[i] != 0 (the others' gradient rows
// are not read).
hipError_t launch_adam_step_seen(const AdamArgs& a, int64_t n, int32_t t, int32_t* last_step, const uint8_t* seen,
                                 hipStream_t s);
hipError_t launch_adam_flush(const AdamArgs& a, int64_t n, int32_t t, int32_t* last_step, hipStream_t s);
int32_t fused_lds_entries();

// GS_CHECK: device validation of tile lists (gs_check_bins).
struct CheckArgs {
    int32_t V, capacity, tpv, tiles_x;
    int64_t count;              // entries of the lists checked (instances, or the kept ones)
    const int32_t* vis_count;   // [V]
    const float* depth;         // [V][capacity]
    const ushort4* rect;        // [V][capacity]
    const int32_t* n_tiles;     // [V][capacity]
    const int32_t* inst_base;   // [V][capacity]
    const uint32_t* tile_keys;  // sorted tile keys of the full lists; NULL for the capped lists
    const int32_t* vals;
    const int32_t* ranges;      // [V * tpv][2]
    int32_t cap;                // the cap of capped lists, else 0
    unsigned long long* viol;   // [GS_CHECK_KINDS] violation counts
    long long* sums;            // [2V]: n_tiles summed over each view's slots, then list lengths per view
};
// slots: also the per-slot checks and sums (once per call, with the full lists)
hipError_t launch_check_bins(const CheckArgs& a, bool slots, hipStream_t s);

}  // namespace gsmi
