// Host side of the C ABI in gsmi.h: argument validation (before anything is enqueued),
// workspace carving, the single count read-back of gs_bin_tiles, and launch orchestration.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

using namespace gsmi;

namespace {

thread_local std::string g_last_error;

gs_status fail(gs_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

gs_status hip_check(hipError_t e, const char* what) {
    if (e == hipSuccess) return GS_OK;
    return fail(GS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Bump allocator over the caller's workspace.
struct Carver {
    char* base;
    size_t used = 0;
    explicit Carver(void* p) : base(static_cast<char*>(p)) {}
    template <typename T>
    T* take(size_t count) {
        T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
        used += align256(sizeof(T) * count);
        return p;
    }
};

int tiles_along(int px) { return (px + kTile - 1) / kTile; }

gs_status check_cams(const gs_camera* cams, int32_t V) {
    if (!cams) return fail(GS_ERR_INVALID_ARGUMENT, "cams is null");
    if (V < 1 || V > GS_MAX_VIEWS) return fail(GS_ERR_INVALID_ARGUMENT, "V=%d outside 1..%d", V, GS_MAX_VIEWS);
    for (int v = 0; v < V; v++) {
        const gs_camera& c = cams[v];
        if (c.width <= 0 || c.height <= 0 || c.width > 65535 * kTile || c.height > 65535 * kTile)
            return fail(GS_ERR_INVALID_ARGUMENT, "view %d: image size %dx%d", v, c.width, c.height);
        if (c.width != cams[0].width || c.height != cams[0].height)
            return fail(GS_ERR_INVALID_ARGUMENT, "view %d: image size differs from view 0", v);
        if ((int64_t)tiles_along(c.width) * tiles_along(c.height) * V >= (int64_t(1) << 31))
            return fail(GS_ERR_INVALID_ARGUMENT, "too many tiles");
    }
    return GS_OK;
}

gs_status check_params(const gs_render_params* p) {
    if (!p) return fail(GS_ERR_INVALID_ARGUMENT, "params is null");
    if (p->sh_degree < 0 || p->sh_degree > 3) return fail(GS_ERR_INVALID_ARGUMENT, "sh_degree=%d", p->sh_degree);
    if (p->tile_cap < 0) return fail(GS_ERR_INVALID_ARGUMENT, "tile_cap=%d", p->tile_cap);
    if (!(p->alpha_min > 0.0f) || !(p->alpha_max <= 1.0f) || !(p->alpha_min < p->alpha_max) || !(p->alpha_max < 1.0f))
        return fail(GS_ERR_INVALID_ARGUMENT, "alpha bounds must satisfy 0 < alpha_min < alpha_max < 1");
    if (!(p->t_min >= 0.0f) || !(p->t_min < 1.0f)) return fail(GS_ERR_INVALID_ARGUMENT, "t_min outside [0, 1)");
    if (!(p->eps2d >= 0.0f) || !std::isfinite(p->eps2d)) return fail(GS_ERR_INVALID_ARGUMENT, "eps2d outside [0, inf)");
    // the depth keys are float32 bit patterns, which order like the values only for positive depths
    if (!(p->znear >= 0.0f) || !std::isfinite(p->znear)) return fail(GS_ERR_INVALID_ARGUMENT, "znear outside [0, inf)");
    for (int c = 0; c < 3; c++)
        if (!std::isfinite(p->bg[c])) return fail(GS_ERR_INVALID_ARGUMENT, "background is not finite");
    return GS_OK;
}

CamArray to_dev(const gs_camera* cams, int32_t V) {
    CamArray a;
    std::memset(&a, 0, sizeof(a));
    for (int v = 0; v < V; v++) {
        CamDev& d = a.c[v];
        d.width = cams[v].width;
        d.height = cams[v].height;
        d.tiles_x = tiles_along(cams[v].width);
        d.tiles_y = tiles_along(cams[v].height);
        d.fx = cams[v].fx;
        d.fy = cams[v].fy;
        d.cx = cams[v].cx;
        d.cy = cams[v].cy;
        std::memcpy(d.R, cams[v].R, sizeof(d.R));
        std::memcpy(d.t, cams[v].t, sizeof(d.t));
        std::memcpy(d.campos, cams[v].campos, sizeof(d.campos));
    }
    return a;
}

ParamsDev to_dev(const gs_render_params* p) {
    ParamsDev d;
    d.znear = p->znear;
    d.eps2d = p->eps2d;
    d.alpha_min = p->alpha_min;
    d.alpha_max = p->alpha_max;
    d.t_min = p->t_min;
    d.bg[0] = p->bg[0];
    d.bg[1] = p->bg[1];
    d.bg[2] = p->bg[2];
    d.sh_degree = p->sh_degree;
    d.tile_cap = p->tile_cap;
    return d;
}

// mean2d, conic_opacity and color are optional everywhere: copies of values the packed record
// holds, written only when given.
gs_status check_projected(const gs_projected* pr) {
    if (!pr) return fail(GS_ERR_INVALID_ARGUMENT, "projected is null");
    if (pr->capacity < 0) return fail(GS_ERR_INVALID_ARGUMENT, "projected capacity < 0");
    if (!pr->vis_count || !pr->inst_count) return fail(GS_ERR_INVALID_ARGUMENT, "projected counts are null");
    return GS_OK;
}

// Workspace layout of gs_bin_tiles.
struct BinWs {
    uint32_t *dkey, *dval, *dkey_alt, *dval_alt;
    int32_t* emit_offsets;  // [emit_chunks(n * V)] instance offsets of the emission chunks
    uint32_t *tkey_alt, *tval_alt;
    int32_t *hist, *partials;
    int32_t *kept, *cap_offsets;
    int32_t* order_hist;    // tile-order bucket counts per chunk
    BinReadback* readback;  // counts and depth range read by the host
    int4* huge_rects;       // [2 * huge_rect_cap(inst_cap)] rectangles written by a workgroup each
    int32_t* huge_count;    // [1]
};

BinWs carve_bin(void* ws, int32_t n, int32_t V, int32_t tiles_total, int64_t inst_cap, size_t* bytes) {
    Carver c(ws);
    const int64_t nv = (int64_t)n * V;
    int64_t sort_n64 = nv > inst_cap ? nv : inst_cap;
    if (tiles_total > sort_n64) sort_n64 = tiles_total;
    const int32_t sort_n = (int32_t)sort_n64;
    BinWs w;
    w.dkey = c.take<uint32_t>(nv);
    w.dval = c.take<uint32_t>(nv);
    w.dkey_alt = c.take<uint32_t>(nv);
    w.dval_alt = c.take<uint32_t>(nv);
    w.emit_offsets = c.take<int32_t>(emit_chunks((int32_t)nv) + 1);
    w.tkey_alt = c.take<uint32_t>(inst_cap);
    w.tval_alt = c.take<uint32_t>(inst_cap);
    w.hist = c.take<int32_t>(radix_hist_bytes(sort_n) / sizeof(int32_t));
    size_t part = radix_partials_bytes(sort_n);
    const size_t p3 = scan_partials_bytes(tiles_total, 1);
    if (p3 > part) part = p3;
    w.partials = c.take<int32_t>(part / sizeof(int32_t));
    w.kept = c.take<int32_t>(tiles_total);
    w.cap_offsets = c.take<int32_t>(tiles_total);
    w.order_hist = c.take<int32_t>(tile_order_hist_ints(tiles_total) + 1);
    w.readback = c.take<BinReadback>(1);
    w.huge_rects = c.take<int4>(2 * (size_t)huge_rect_cap(inst_cap));
    w.huge_count = c.take<int32_t>(1);
    *bytes = c.used;
    return w;
}

int bits_for(int64_t count) {
    int b = 1;
    while ((int64_t(1) << b) < count) b++;
    return b;
}

gs_status check_raster(const gs_camera* cams, const gs_projected* proj, const gs_bins* bins, int32_t V,
                       const gs_render_params* p, int32_t use_capped, RasterArgs* ra) {
    gs_status st = check_cams(cams, V);
    if (st != GS_OK) return st;
    if ((st = check_params(p)) != GS_OK) return st;
    if ((st = check_projected(proj)) != GS_OK) return st;
    if (!proj->raster_rec) return fail(GS_ERR_INVALID_ARGUMENT, "projected raster_rec is null");
    if (!bins) return fail(GS_ERR_INVALID_ARGUMENT, "bins is null");
    const int32_t* ranges = use_capped ? bins->ranges_capped : bins->ranges;
    const int32_t* vals = use_capped ? bins->vals_capped : bins->vals;
    if (!ranges || !vals) return fail(GS_ERR_INVALID_ARGUMENT, "bins ranges/vals are null");
    if (bins->count < 0) return fail(GS_ERR_INVALID_ARGUMENT, "bins hold no lists (the last gs_bin_tiles failed)");
    ra->V = V;
    ra->width = cams[0].width;
    ra->height = cams[0].height;
    ra->tiles_x = tiles_along(cams[0].width);
    ra->tiles_y = tiles_along(cams[0].height);
    ra->capacity = proj->capacity;
    ra->p = to_dev(p);
    ra->ranges = ranges;
    ra->vals = vals;
    ra->rec = reinterpret_cast<const float4*>(proj->raster_rec);
    ra->vis_count = proj->vis_count;
    ra->tile_order = bins->tile_order;
    ra->inst_base = proj->inst_base;
    ra->n_tiles = proj->n_tiles;
    ra->partials = nullptr;
    ra->huge_slots = nullptr;
    ra->huge_count = nullptr;
    ra->huge_cap = 0;
    ra->num_instances = bins->count;
    ra->capped = use_capped ? 1 : 0;
    ra->counters = nullptr;
    return GS_OK;
}

// The backward's partial-record workspace and the bins/projection fields it needs.
gs_status check_partials(const gs_projected* proj, const gs_bins* bins, void* ws, size_t ws_bytes, RasterArgs* ra) {
    if (!proj->n_tiles || !proj->inst_base)
        return fail(GS_ERR_INVALID_ARGUMENT, "n_tiles / inst_base are null");
    if (bins->count < 0 || bins->count > bins->capacity)
        return fail(GS_ERR_INVALID_ARGUMENT, "bins->count %lld outside [0, capacity]", (long long)bins->count);
    const size_t need = raster_ws_bytes(bins->count);
    if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "raster workspace %zu < %zu bytes", ws_bytes, need);
    Carver c(ws);
    ra->partials = c.take<float>(9 * (size_t)bins->count);
    ra->huge_count = c.take<int32_t>(1);
    ra->huge_slots = c.take<int4>((size_t)huge_slot_cap(bins->count));
    ra->huge_cap = huge_slot_cap(bins->count);
    ra->loss_acc = c.take<long long>(1);
    return GS_OK;
}

gs_status check_grads(const gs_grads2d* g, Grads* out) {
    if (!g || !g->d_mean2d || !g->d_conic || !g->d_opacity || !g->d_color)
        return fail(GS_ERR_INVALID_ARGUMENT, "gradient outputs are null");
    out->d_mean2d = reinterpret_cast<float2*>(g->d_mean2d);
    out->d_conic = g->d_conic;
    out->d_opacity = g->d_opacity;
    out->d_color = g->d_color;
    return GS_OK;
}

}  // namespace

extern "C" {

const char* gs_version(void) { return "gsmi 0.1 (gfx950)"; }

const char* gs_status_string(gs_status s) {
    switch (s) {
        case GS_OK: return "ok";
        case GS_ERR_INVALID_ARGUMENT: return "invalid argument";
        case GS_ERR_CAPACITY: return "capacity exceeded";
        case GS_ERR_UNSUPPORTED: return "unsupported";
        case GS_ERR_HIP: return "HIP runtime error";
        case GS_ERR_INTERNAL: return "internal error";
        default: break;
    }
    return "unknown status";
}

const char* gs_last_error(void) { return g_last_error.c_str(); }

size_t gs_project_workspace_size(int32_t n, int32_t V) {
    if (n < 0 || V < 1) return 0;
    return project_ws_bytes(n, V);
}

// Pinned host copy of the count summary and the event gs_project records after copying it.
// `filled`: the buffer holds the counts of the last gs_project that named it, for V views and
// this capacity (set when the copy is enqueued; the event says when it has landed).
struct gs_readback {
    gsmi::CountSummary* host = nullptr;
    hipEvent_t done = nullptr;
    bool filled = false;
    int32_t V = 0, capacity = 0;
};

gs_status gs_readback_create(gs_readback** out) {
    g_last_error.clear();
    if (!out) return fail(GS_ERR_INVALID_ARGUMENT, "out is null");
    *out = nullptr;
    gs_readback* r = new gs_readback();
    void* h = nullptr;
    if (hipHostMalloc(&h, sizeof(gsmi::CountSummary), hipHostMallocDefault) != hipSuccess) {
        delete r;
        return fail(GS_ERR_HIP, "hipHostMalloc of the count buffer failed");
    }
    r->host = static_cast<gsmi::CountSummary*>(h);
    if (hipEventCreateWithFlags(&r->done, hipEventDisableTiming) != hipSuccess) {
        (void)hipHostFree(h);
        delete r;
        return fail(GS_ERR_HIP, "hipEventCreateWithFlags failed");
    }
    *out = r;
    return GS_OK;
}

void gs_readback_destroy(gs_readback* r) {
    if (!r) return;
    if (r->filled) (void)hipEventSynchronize(r->done);
    (void)hipEventDestroy(r->done);
    (void)hipHostFree(r->host);
    delete r;
}

gs_status gs_project(const gs_gaussians* g, const gs_camera* cams, int32_t V, const gs_render_params* p,
                     gs_projected* out, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (!g) return fail(GS_ERR_INVALID_ARGUMENT, "gaussians is null");
    gs_status st = check_cams(cams, V);
    if (st != GS_OK) return st;
    if ((st = check_params(p)) != GS_OK) return st;
    if (g->n < 0 || g->n >= (1 << 28)) return fail(GS_ERR_INVALID_ARGUMENT, "n=%d outside [0, 2^28)", g->n);
    if (g->n > 0 && (!g->means || !g->log_scales || !g->quats || !g->opacity_logits || !g->sh))
        return fail(GS_ERR_INVALID_ARGUMENT, "a parameter array is null");
    if ((st = check_projected(out)) != GS_OK) return st;
    if (!out->vis_ids || !out->depth || !out->tile_rect || !out->n_tiles || !out->inst_base || !out->raster_rec)
        return fail(GS_ERR_INVALID_ARGUMENT, "projected outputs are null");
    if (reinterpret_cast<uintptr_t>(out->raster_rec) % 64 != 0)
        return fail(GS_ERR_INVALID_ARGUMENT, "raster_rec is not 64-byte aligned");
    if (out->capacity < g->n) return fail(GS_ERR_INVALID_ARGUMENT, "capacity %d < n %d", out->capacity, g->n);
    if ((int64_t)out->capacity * V >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARGUMENT, "capacity * V must stay below 2^31");
    const size_t need = project_ws_bytes(g->n, V);
    if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "project workspace %zu < %zu bytes", ws_bytes, need);
    ProjectArgs a;
    a.n = g->n;
    a.V = V;
    a.capacity = out->capacity;
    a.means = g->means;
    a.log_scales = g->log_scales;
    a.quats = g->quats;
    a.logits = g->opacity_logits;
    a.sh = g->sh;
    a.cams = to_dev(cams, V);
    a.p = to_dev(p);
    a.vis_count = out->vis_count;
    a.inst_count = out->inst_count;
    a.vis_ids = out->vis_ids;
    a.mean2d = reinterpret_cast<float2*>(out->mean2d);
    a.conic_opacity = reinterpret_cast<float4*>(out->conic_opacity);
    a.color = out->color;
    a.depth = out->depth;
    a.tile_rect = reinterpret_cast<ushort4*>(out->tile_rect);
    a.n_tiles = out->n_tiles;
    a.inst_base = out->inst_base;
    a.raster_rec = reinterpret_cast<float4*>(out->raster_rec);
    const int32_t nw = project_count_waves(g->n);
    Carver c(ws);
    a.block_counts = c.take<int32_t>((size_t)nw * 2 * V);
    a.block_offsets = c.take<int32_t>((size_t)nw * 2 * V);
    a.row_totals = c.take<int32_t>((size_t)2 * V);
    a.scan_partials = c.take<int32_t>(scan_partials_bytes(nw, 2 * V) / sizeof(int32_t));
    gs_readback* rb = out->readback;
    uint2* block_depth = c.take<uint2>((size_t)nw);
    CountSummary* summary = c.take<CountSummary>(1);
    a.block_depth = rb ? block_depth : nullptr;
    a.summary = rb ? summary : nullptr;
    a.seen = c.take<uint8_t>((size_t)nw * 64);
    a.inst_partials = c.take<int64_t>((size_t)V * project_partials());
    a.depth_partials = c.take<uint2>((size_t)project_partials());
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (rb) rb->filled = false;
    gs_status st2 = hip_check(launch_project_count(a, s), "gs_project launch");
    if (st2 != GS_OK) return st2;
    if (rb) {
        // the counts are final here: copy them out while the writing pass runs
        if ((st2 = hip_check(hipMemcpyAsync(rb->host, a.summary, sizeof(CountSummary), hipMemcpyDeviceToHost, s),
                             "count copy")) != GS_OK)
            return st2;
        if ((st2 = hip_check(hipEventRecord(rb->done, s), "count event")) != GS_OK) return st2;
        rb->filled = true;
        rb->V = V;
        rb->capacity = out->capacity;
    }
    return hip_check(launch_project_write(a, s), "gs_project launch");
}

// gs_project_noalloc: gs_project with its workspace in a file-scope device array instead of a
// caller's buffer, for callers that cannot allocate.  The array's name is a host-side stand-in
// in host code; its device address is looked up once per device, with that device current, on
// the first call there, and only that address is used afterwards.  Every byte of the projection
// workspace is written before it is read within one call (the count pass writes the block
// counts, depth ranges and seen flags of every block it reads back), so the contents a previous
// call left behind need no clearing.  All calls on one device share the array: calls that
// overlap in time on one device (different host threads or streams) race.
namespace {
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

gs_status scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GS_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GS_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(GS_ERR_HIP, "hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GS_OK;
}
}  // namespace

size_t gs_project_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

gs_status gs_project_noalloc(const gs_gaussians* g, const gs_camera* cams, int32_t V, const gs_render_params* p,
                             gs_projected* out, void* stream) {
    g_last_error.clear();
    if (!g) return fail(GS_ERR_INVALID_ARGUMENT, "gaussians is null");
    gs_status st = check_cams(cams, V);
    if (st != GS_OK) return st;
    if (g->n < 0 || g->n >= (1 << 28)) return fail(GS_ERR_INVALID_ARGUMENT, "n=%d outside [0, 2^28)", g->n);
    const size_t need = project_ws_bytes(g->n, V);
    if (need > kNoAllocScratchBytes)
        return fail(GS_ERR_CAPACITY, "gs_project_noalloc: n=%d and V=%d need %zu workspace bytes, above the %zu-byte "
                                     "static scratch (use gs_project with a workspace)",
                    g->n, V, need, kNoAllocScratchBytes);
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != GS_OK) return st;
    return gs_project(g, cams, V, p, out, ws, kNoAllocScratchBytes, stream);
}

static gs_status project_bwd(const gs_gaussians* g, const gs_camera* cams, int32_t V, const gs_render_params* p,
                             const gs_projected* proj, const gs_grads2d* grads2d, gs_grads3d* out, uint8_t* seen_out,
                             void* stream, const char* what) {
    if (!g) return fail(GS_ERR_INVALID_ARGUMENT, "gaussians is null");
    gs_status st = check_cams(cams, V);
    if (st != GS_OK) return st;
    if ((st = check_params(p)) != GS_OK) return st;
    if (g->n < 0 || g->n >= (1 << 28)) return fail(GS_ERR_INVALID_ARGUMENT, "n=%d outside [0, 2^28)", g->n);
    if (g->n > 0 && (!g->means || !g->log_scales || !g->quats || !g->opacity_logits || !g->sh))
        return fail(GS_ERR_INVALID_ARGUMENT, "a parameter array is null");
    if (!proj || !proj->vis_count || !proj->vis_ids)
        return fail(GS_ERR_INVALID_ARGUMENT, "projected vis_count / vis_ids are null");
    if (proj->capacity < g->n) return fail(GS_ERR_INVALID_ARGUMENT, "capacity %d < n %d", proj->capacity, g->n);
    if ((int64_t)proj->capacity * V >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARGUMENT, "capacity * V must stay below 2^31");
    if (!grads2d || !grads2d->d_mean2d || !grads2d->d_conic || !grads2d->d_opacity || !grads2d->d_color)
        return fail(GS_ERR_INVALID_ARGUMENT, "2D gradients are null");
    if (!out || !out->d_means || !out->d_log_scales || !out->d_quats || !out->d_opacity_logits || !out->d_sh)
        return fail(GS_ERR_INVALID_ARGUMENT, "parameter gradient outputs are null");
    ProjectBwdArgs a;
    a.n = g->n;
    a.V = V;
    a.capacity = proj->capacity;
    a.means = g->means;
    a.log_scales = g->log_scales;
    a.quats = g->quats;
    a.logits = g->opacity_logits;
    a.sh = g->sh;
    a.cams = to_dev(cams, V);
    a.p = to_dev(p);
    a.vis_count = proj->vis_count;
    a.vis_ids = proj->vis_ids;
    a.d_mean2d = reinterpret_cast<const float2*>(grads2d->d_mean2d);
    a.d_conic = grads2d->d_conic;
    a.d_opacity = grads2d->d_opacity;
    a.d_color = grads2d->d_color;
    a.g_means = out->d_means;
    a.g_log_scales = out->d_log_scales;
    a.g_quats = out->d_quats;
    a.g_logits = out->d_opacity_logits;
    a.g_sh = out->d_sh;
    a.seen_out = seen_out;
    return hip_check(launch_project_bwd(a, static_cast<hipStream_t>(stream)), what);
}

gs_status gs_project_bwd(const gs_gaussians* g, const gs_camera* cams, int32_t V, const gs_render_params* p,
                         const gs_projected* proj, const gs_grads2d* grads2d, gs_grads3d* out, void* stream) {
    g_last_error.clear();
    return project_bwd(g, cams, V, p, proj, grads2d, out, nullptr, stream, "gs_project_bwd launch");
}

gs_status gs_project_bwd_seen(const gs_gaussians* g, const gs_camera* cams, int32_t V, const gs_render_params* p,
                              const gs_projected* proj, const gs_grads2d* grads2d, gs_grads3d* out, uint8_t* seen,
                              void* stream) {
    g_last_error.clear();
    if (!seen && g && g->n > 0) return fail(GS_ERR_INVALID_ARGUMENT, "seen is null");
    return project_bwd(g, cams, V, p, proj, grads2d, out, seen, stream, "gs_project_bwd_seen launch");
}

size_t gs_raster_workspace_size(int64_t instance_capacity) {
    if (instance_capacity < 0) return 0;
    return raster_ws_bytes(instance_capacity);
}

size_t gs_bin_workspace_size(int32_t n, int32_t V, int32_t width, int32_t height, int64_t instance_capacity) {
    if (n < 0 || V < 1 || width <= 0 || height <= 0 || instance_capacity < 0) return 0;
    size_t bytes = 0;
    carve_bin(nullptr, n, V, tiles_along(width) * tiles_along(height) * V, instance_capacity, &bytes);
    return bytes;
}

gs_status gs_bin_tiles(const gs_camera* cams, const gs_projected* proj, int32_t V, const gs_render_params* p,
                       gs_bins* bins, gs_bin_info* info, int64_t* required, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    gs_status st = check_cams(cams, V);
    if (st != GS_OK) return st;
    if ((st = check_params(p)) != GS_OK) return st;
    if ((st = check_projected(proj)) != GS_OK) return st;
    if (!proj->depth || !proj->tile_rect || !proj->n_tiles)
        return fail(GS_ERR_INVALID_ARGUMENT, "projected depth/rect/n_tiles are null");
    if (p->tile_cap > 0 && !proj->conic_opacity && !proj->raster_rec)
        return fail(GS_ERR_INVALID_ARGUMENT, "tile_cap > 0 needs conic_opacity or raster_rec");
    if (!bins || !bins->tile_keys || !bins->vals || !bins->ranges)
        return fail(GS_ERR_INVALID_ARGUMENT, "bins outputs are null");
    if (p->tile_cap > 0 && (!bins->vals_capped || !bins->ranges_capped || !bins->num_capped))
        return fail(GS_ERR_INVALID_ARGUMENT, "capped outputs are null while tile_cap > 0");
    if (!info) return fail(GS_ERR_INVALID_ARGUMENT, "info is null");
    if (bins->capacity < 0 || bins->capacity >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARGUMENT, "bins capacity outside [0, 2^31)");
    bins->count = -1;  // until the lists are complete
    const int tiles_x = tiles_along(cams[0].width), tiles_y = tiles_along(cams[0].height);
    const int32_t tpv = tiles_x * tiles_y;
    const int32_t tiles_total = tpv * V;
    size_t need = 0;
    carve_bin(nullptr, proj->capacity, V, tiles_total, bins->capacity, &need);
    if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "bin workspace %zu < %zu bytes", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);

    // the one read-back: visible and instance counts of every view and the visible depth range
    BinWs w = carve_bin(ws, proj->capacity, V, tiles_total, bins->capacity, &need);
    BinReadback rb;
    gs_readback* early = proj->readback;
    if (early && early->filled && early->V == V && early->capacity == proj->capacity) {
        // copied by gs_project before its writing pass: wait for that copy only
        if ((st = hip_check(hipEventSynchronize(early->done), "count copy wait")) != GS_OK) return st;
        for (int v = 0; v < V; v++) {
            rb.vis[v] = early->host->vis[v];
            rb.inst[v] = early->host->inst[v];
        }
        rb.bits[0] = early->host->bits[0];
        rb.bits[1] = early->host->bits[1];
    } else {
        if ((st = hip_check(launch_bin_counts(proj->vis_count, proj->inst_count, V, proj->depth, proj->capacity,
                                              w.readback, s),
                            "count launch")) != GS_OK)
            return st;
        if ((st = hip_check(hipMemcpyAsync(&rb, w.readback, offsetof(BinReadback, partial), hipMemcpyDeviceToHost,
                                           s),
                            "count read")) != GS_OK)
            return st;
        if ((st = hip_check(hipStreamSynchronize(s), "count read sync")) != GS_OK) return st;
    }
    const int32_t* vis = rb.vis;
    const int64_t* inst = rb.inst;
    std::memset(info, 0, sizeof(*info));
    int64_t total_vis = 0, M = 0;
    for (int v = 0; v < V; v++) {
        if (vis[v] < 0 || vis[v] > proj->capacity || inst[v] < 0)
            return fail(GS_ERR_INTERNAL, "view %d: implausible counts (%d, %lld)", v, vis[v], (long long)inst[v]);
        info->vis_count[v] = vis[v];
        info->view_offset[v] = M;
        total_vis += vis[v];
        M += inst[v];
    }
    info->view_offset[V] = M;
    info->num_instances = M;
    info->num_instances_capped = p->tile_cap > 0 ? -1 : M;
    if (required) *required = M;
    if (M >= (int64_t(1) << 31)) return fail(GS_ERR_CAPACITY, "%lld instances exceed 2^31 - 1", (long long)M);
    if (M > bins->capacity)
        return fail(GS_ERR_CAPACITY, "%lld instances exceed the bins capacity %lld", (long long)M,
                    (long long)bins->capacity);

    // the tile ranges start cleared: by the depth-key kernel when there are instances
    hipError_t e = M > 0 ? hipSuccess : launch_fill_i32(bins->ranges, 0, 2 * (int64_t)tiles_total, s);
    if (e == hipSuccess && M > 0) {
        // depth digits, one entry per visible slot
        int64_t first[GS_MAX_VIEWS + 1];
        int64_t acc = 0;
        for (int v = 0; v < V; v++) {
            first[v] = acc;
            acc += vis[v];
        }
        first[V] = acc;
        const int32_t nvis = (int32_t)total_vis;
        // keys relative to the smallest visible depth: as many bits as the depth range needs
        const uint32_t key_min = rb.bits[0], key_span = ~rb.bits[1] - rb.bits[0];
        const int dbits = key_span == 0 ? 0 : 32 - __builtin_clz(key_span);
        e = launch_depth_keys(proj->depth, first, V, proj->capacity, nvis, key_min, w.dkey, w.dval, bins->ranges,
                              2 * tiles_total, s);
        if (e == hipSuccess)
            e = launch_radix_sort(w.dkey, w.dval, w.dkey_alt, w.dval_alt, nvis, dbits, w.hist, w.partials, s);
        uint32_t* packed = (radix_passes(dbits) % 2 == 0) ? w.dval : w.dval_alt;
        // emit so that the tile sort's final pass lands in the output buffers
        const int tbits = bits_for(tiles_total);
        const bool odd = radix_passes(tbits) % 2 == 1;
        uint32_t* k0 = odd ? w.tkey_alt : bins->tile_keys;
        uint32_t* v0 = odd ? w.tval_alt : reinterpret_cast<uint32_t*>(bins->vals);
        uint32_t* k1 = odd ? bins->tile_keys : w.tkey_alt;
        uint32_t* v1 = odd ? reinterpret_cast<uint32_t*>(bins->vals) : w.tval_alt;
        // the depth keys are spent: their two buffers hold the rectangles in depth order
        if (e == hipSuccess)
            e = launch_emit(packed, reinterpret_cast<const ushort4*>(proj->tile_rect), proj->capacity, nvis, tiles_x, tpv,
                            (int32_t)M, w.emit_offsets, w.dkey, w.dkey_alt, w.huge_rects, w.huge_count,
                            huge_rect_cap(bins->capacity), k0, reinterpret_cast<int32_t*>(v0), s);
        if (e == hipSuccess) e = launch_radix_sort(k0, v0, k1, v1, (int32_t)M, tbits, w.hist, w.partials, s);
        if (e == hipSuccess) e = launch_ranges(bins->tile_keys, (int32_t)M, bins->ranges, s);
    }
    if (e == hipSuccess && bins->tile_order)
        e = launch_tile_order(bins->ranges, tiles_total, w.order_hist, bins->tile_order, s);
    if (e == hipSuccess && p->tile_cap > 0) {
        e = launch_cap_count(bins->ranges, tiles_total, p->tile_cap, w.kept, s);
        if (e == hipSuccess) e = launch_scan_rows(w.kept, w.cap_offsets, bins->num_capped, tiles_total, 1, w.partials, s);
        if (e == hipSuccess)
            // the depth sort's key buffer (capacity * V words) is free again: the slots' scores
            e = launch_cap_select(bins->ranges, bins->vals, reinterpret_cast<const float4*>(proj->conic_opacity),
                                  reinterpret_cast<const float4*>(proj->raster_rec), proj->vis_count, V, proj->capacity, tpv, tiles_total, p->tile_cap, w.cap_offsets,
                                  bins->tile_order, bins->vals_capped, bins->ranges_capped, w.dkey, w.tkey_alt, s);
    }
    if (e == hipSuccess) bins->count = M;
    return hip_check(e, "gs_bin_tiles launch");
}

gs_status gs_raster_fwd(const gs_camera* cams, const gs_projected* proj, const gs_bins* bins, int32_t V,
                        const gs_render_params* p, int32_t use_capped, float* image, float* t_final,
                        int32_t* n_contrib, gs_counters* counters, void* stream) {
    g_last_error.clear();
    RasterArgs ra;
    gs_status st = check_raster(cams, proj, bins, V, p, use_capped, &ra);
    if (st != GS_OK) return st;
    if (!image || !t_final || !n_contrib) return fail(GS_ERR_INVALID_ARGUMENT, "forward outputs are null");
    ra.counters = counters;
    return hip_check(launch_raster_fwd(ra, image, t_final, n_contrib, static_cast<hipStream_t>(stream)),
                     "gs_raster_fwd launch");
}

gs_status gs_loss_l1_grad(int32_t V, int32_t width, int32_t height, const float* image, const float* target,
                          float scale, float* dl_dimage, float* loss_sum, void* stream) {
    g_last_error.clear();
    if (V < 1 || width <= 0 || height <= 0) return fail(GS_ERR_INVALID_ARGUMENT, "bad image size");
    if (!image || !target || !dl_dimage) return fail(GS_ERR_INVALID_ARGUMENT, "loss buffers are null");
    const int64_t n = (int64_t)V * 3 * width * height;
    return hip_check(launch_loss_l1(n, image, target, scale, dl_dimage, loss_sum, static_cast<hipStream_t>(stream)),
                     "gs_loss_l1_grad launch");
}

gs_status gs_raster_bwd(const gs_camera* cams, const gs_projected* proj, const gs_bins* bins, int32_t V,
                        const gs_render_params* p, int32_t use_capped, const float* image, const float* t_final,
                        const int32_t* n_contrib, const float* dl_dimage, gs_grads2d* grads, void* ws,
                        size_t ws_bytes, void* stream) {
    g_last_error.clear();
    RasterArgs ra;
    gs_status st = check_raster(cams, proj, bins, V, p, use_capped, &ra);
    if (st != GS_OK) return st;
    if (!t_final || !n_contrib || !dl_dimage) return fail(GS_ERR_INVALID_ARGUMENT, "backward inputs are null");
    Grads g;
    if ((st = check_grads(grads, &g)) != GS_OK) return st;
    if ((st = check_partials(proj, bins, ws, ws_bytes, &ra)) != GS_OK) return st;
    return hip_check(launch_raster_bwd(ra, image, t_final, n_contrib, dl_dimage, g, static_cast<hipStream_t>(stream)),
                     "gs_raster_bwd launch");
}

gs_status gs_raster_fused(const gs_camera* cams, const gs_projected* proj, const gs_bins* bins, int32_t V,
                          const gs_render_params* p, int32_t use_capped, gs_loss_mode mode,
                          const float* target_or_dldc, float loss_scale, float* image_opt, float* loss_sum_opt,
                          gs_grads2d* grads, gs_counters* counters, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    RasterArgs ra;
    gs_status st = check_raster(cams, proj, bins, V, p, use_capped, &ra);
    if (st != GS_OK) return st;
    if (mode != GS_LOSS_L1 && mode != GS_LOSS_EXTERNAL) return fail(GS_ERR_INVALID_ARGUMENT, "loss mode %d", (int)mode);
    if (!target_or_dldc) return fail(GS_ERR_INVALID_ARGUMENT, "target_or_dldc is null");
    Grads g;
    if ((st = check_grads(grads, &g)) != GS_OK) return st;
    if ((st = check_partials(proj, bins, ws, ws_bytes, &ra)) != GS_OK) return st;
    ra.counters = counters;
    return hip_check(launch_raster_fused(ra, (int)mode, target_or_dldc, loss_scale, image_opt, loss_sum_opt, g,
                                         static_cast<hipStream_t>(stream)),
                     "gs_raster_fused launch");
}

gs_status gs_check_bins(const gs_camera* cams, const gs_projected* proj, int32_t V, const gs_render_params* p,
                        const gs_bins* bins, int64_t* violations, void* stream) {
    g_last_error.clear();
    gs_status st = check_cams(cams, V);
    if (st != GS_OK) return st;
    if ((st = check_params(p)) != GS_OK) return st;
    if ((st = check_projected(proj)) != GS_OK) return st;
    if (!proj->depth || !proj->tile_rect || !proj->n_tiles || !proj->inst_base)
        return fail(GS_ERR_INVALID_ARGUMENT, "projected depth/rect/n_tiles/inst_base are null");
    if (!bins || !bins->tile_keys || !bins->vals || !bins->ranges)
        return fail(GS_ERR_INVALID_ARGUMENT, "bins outputs are null");
    if (p->tile_cap > 0 && (!bins->vals_capped || !bins->ranges_capped || !bins->num_capped))
        return fail(GS_ERR_INVALID_ARGUMENT, "capped outputs are null while tile_cap > 0");
    if (bins->count < 0) return fail(GS_ERR_INVALID_ARGUMENT, "bins hold no successful gs_bin_tiles result");
    if (!violations) return fail(GS_ERR_INVALID_ARGUMENT, "violations is null");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int tiles_x = tiles_along(cams[0].width), tiles_y = tiles_along(cams[0].height);
    // device counters: violations, then [2V] sums of the full lists, then [2V] of the capped ones
    const size_t bytes = sizeof(unsigned long long) * GS_CHECK_KINDS + sizeof(long long) * 4 * V;
    void* dbuf = nullptr;
    if ((st = hip_check(hipMalloc(&dbuf, bytes), "check buffer")) != GS_OK) return st;
    struct Free {
        void* p;
        ~Free() { (void)hipFree(p); }
    } guard{dbuf};
    unsigned long long* viol = static_cast<unsigned long long*>(dbuf);
    long long* sums = reinterpret_cast<long long*>(viol + GS_CHECK_KINDS);
    if ((st = hip_check(hipMemsetAsync(dbuf, 0, bytes, s), "check clear")) != GS_OK) return st;
    CheckArgs a;
    a.V = V;
    a.capacity = proj->capacity;
    a.tpv = tiles_x * tiles_y;
    a.tiles_x = tiles_x;
    a.count = bins->count;
    a.vis_count = proj->vis_count;
    a.depth = proj->depth;
    a.rect = reinterpret_cast<const ushort4*>(proj->tile_rect);
    a.n_tiles = proj->n_tiles;
    a.inst_base = proj->inst_base;
    a.tile_keys = bins->tile_keys;
    a.vals = bins->vals;
    a.ranges = bins->ranges;
    a.cap = 0;
    a.viol = viol;
    a.sums = sums;
    if ((st = hip_check(launch_check_bins(a, true, s), "check launch")) != GS_OK) return st;
    int32_t kept = 0;
    if (p->tile_cap > 0) {
        if ((st = hip_check(hipMemcpyAsync(&kept, bins->num_capped, sizeof(kept), hipMemcpyDeviceToHost, s),
                            "check kept read")) != GS_OK)
            return st;
        if ((st = hip_check(hipStreamSynchronize(s), "check sync")) != GS_OK) return st;
        CheckArgs c = a;
        c.count = kept;
        c.tile_keys = nullptr;
        c.vals = bins->vals_capped;
        c.ranges = bins->ranges_capped;
        c.cap = p->tile_cap;
        c.sums = sums + 2 * V;
        if ((st = hip_check(launch_check_bins(c, false, s), "check launch")) != GS_OK) return st;
    }
    unsigned long long hv[GS_CHECK_KINDS];
    std::vector<long long> hs(4 * (size_t)V);
    std::vector<int32_t> vis(V), first(V, 0);
    if ((st = hip_check(hipMemcpyAsync(hv, viol, sizeof(hv), hipMemcpyDeviceToHost, s), "check read")) != GS_OK ||
        (st = hip_check(hipMemcpyAsync(hs.data(), sums, sizeof(long long) * 4 * V, hipMemcpyDeviceToHost, s),
                        "check read")) != GS_OK ||
        (st = hip_check(hipMemcpyAsync(vis.data(), proj->vis_count, sizeof(int32_t) * V, hipMemcpyDeviceToHost, s),
                        "check read")) != GS_OK)
        return st;
    if ((st = hip_check(hipStreamSynchronize(s), "check sync")) != GS_OK) return st;
    for (int v = 0; v < V; v++)
        if (vis[v] > 0 &&
            (st = hip_check(hipMemcpy(&first[v], proj->inst_base + (size_t)v * proj->capacity, sizeof(int32_t),
                                      hipMemcpyDeviceToHost),
                            "check read")) != GS_OK)
            return st;
    // host rules: per view, the full lists hold exactly the slots' instances, which the instance
    // bases number view after view; the capped lists are no longer than the full ones
    long long before = 0;
    for (int v = 0; v < V; v++) {
        if (hs[V + v] != hs[v]) hv[GS_CHECK_COUNT]++;
        if (vis[v] > 0 && first[v] != before) hv[GS_CHECK_SLOT_RECORD]++;
        before += hs[v];
        if (p->tile_cap > 0 && hs[3 * V + v] > hs[V + v]) hv[GS_CHECK_COUNT]++;
    }
    static const char* names[GS_CHECK_KINDS] = {"range", "key", "slot", "rect", "order", "count", "cap", "slot record"};
    std::string found;
    for (int k = 0; k < GS_CHECK_KINDS; k++) {
        violations[k] = (int64_t)hv[k];
        if (hv[k]) found += std::string(found.empty() ? "" : ", ") + names[k] + " x" + std::to_string(hv[k]);
    }
    if (!found.empty()) return fail(GS_ERR_INTERNAL, "bins violate: %s", found.c_str());
    return GS_OK;
}

gs_status gs_fused_max_cap(int32_t* k) {
    if (!k) return fail(GS_ERR_INVALID_ARGUMENT, "k is null");
    *k = fused_lds_entries();
    return GS_OK;
}

size_t gs_grad_encode_workspace_size(int32_t capacity, int32_t V) {
    if (capacity < 0 || V < 1 || V > GS_MAX_VIEWS) return 0;
    return encode_workspace_bytes(capacity, V);
}

gs_status gs_grad_encode(int32_t V, int32_t capacity, const int32_t* vis_count, const int32_t* vis_ids,
                         const gs_grads2d* grads, int32_t* keys, float* records, int32_t* view_offset, void* ws,
                         size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (V < 1 || V > GS_MAX_VIEWS) return fail(GS_ERR_INVALID_ARGUMENT, "V=%d outside 1..%d", V, GS_MAX_VIEWS);
    if (capacity < 0) return fail(GS_ERR_INVALID_ARGUMENT, "capacity < 0");
    if ((int64_t)capacity * V >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARGUMENT, "V * capacity records exceed 2^31 - 1");
    if (!vis_count || !vis_ids || !keys || !records || !view_offset)
        return fail(GS_ERR_INVALID_ARGUMENT, "encode buffers are null");
    if (!grads || !grads->d_mean2d || !grads->d_conic || !grads->d_opacity || !grads->d_color)
        return fail(GS_ERR_INVALID_ARGUMENT, "grads are null");
    const size_t need = encode_workspace_bytes(capacity, V);
    if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "encode workspace %zu < %zu bytes", ws_bytes, need);
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(GS_ERR_INVALID_ARGUMENT, "ws is not 256-byte aligned");
    if (capacity == 0) {
        // no slots: the offsets are all zero (a fill kernel, so that the call can be captured)
        return hip_check(launch_fill_i32(view_offset, 0, V + 1, static_cast<hipStream_t>(stream)), "gs_grad_encode");
    }
    GradsIn g{grads->d_mean2d, grads->d_conic, grads->d_opacity, grads->d_color};
    return hip_check(launch_grad_encode(V, capacity, vis_count, vis_ids, g, keys, records, view_offset, ws,
                                        static_cast<hipStream_t>(stream)),
                     "gs_grad_encode launch");
}

gs_status gs_grad_decode(int32_t V, int32_t n_owner, int64_t max_records, const int32_t* view_offset,
                         const int32_t* keys, const float* records, gs_grads2d* owner, void* stream) {
    g_last_error.clear();
    if (V < 1 || V > GS_MAX_VIEWS) return fail(GS_ERR_INVALID_ARGUMENT, "V=%d outside 1..%d", V, GS_MAX_VIEWS);
    if (n_owner < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n_owner < 0");
    if (max_records < 0 || max_records >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARGUMENT, "max_records outside [0, 2^31)");
    if (!view_offset || !keys || !records) return fail(GS_ERR_INVALID_ARGUMENT, "decode buffers are null");
    if (!owner || !owner->d_mean2d || !owner->d_conic || !owner->d_opacity || !owner->d_color)
        return fail(GS_ERR_INVALID_ARGUMENT, "owner arrays are null");
    if (max_records == 0 || n_owner == 0) return GS_OK;
    GradsOut o{owner->d_mean2d, owner->d_conic, owner->d_opacity, owner->d_color};
    return hip_check(launch_grad_decode(V, n_owner, max_records, view_offset, keys, records, o,
                                        static_cast<hipStream_t>(stream)),
                     "gs_grad_decode launch");
}

gs_status gs_compose(int32_t P, int32_t V, int32_t width, int32_t height, const float* const* colors,
                     const float* const* t_finals, const float* bg, float* image, float* t_out, void* stream) {
    g_last_error.clear();
    if (P < 1 || P > GS_MAX_PARTIALS) return fail(GS_ERR_INVALID_ARGUMENT, "P=%d outside 1..%d", P, GS_MAX_PARTIALS);
    if (V < 1 || V > GS_MAX_VIEWS) return fail(GS_ERR_INVALID_ARGUMENT, "V=%d outside 1..%d", V, GS_MAX_VIEWS);
    if (width <= 0 || height <= 0) return fail(GS_ERR_INVALID_ARGUMENT, "image size %dx%d", width, height);
    if (!colors || !t_finals || !bg || !image) return fail(GS_ERR_INVALID_ARGUMENT, "compose buffers are null");
    ComposeArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int k = 0; k < P; k++) {
        if (!colors[k] || !t_finals[k]) return fail(GS_ERR_INVALID_ARGUMENT, "partial %d is null", k);
        a.c[k] = colors[k];
        a.t[k] = t_finals[k];
    }
    for (int c = 0; c < 3; c++) {
        if (!std::isfinite(bg[c])) return fail(GS_ERR_INVALID_ARGUMENT, "bg is not finite");
        a.bg[c] = bg[c];
    }
    return hip_check(launch_compose(P, V, (int64_t)width * height, a, image, t_out, static_cast<hipStream_t>(stream)),
                     "gs_compose launch");
}

namespace {

gs_status adam_args(int32_t n, const gs_adam_group* groups, int32_t n_groups, const gs_adam_params* hp, int32_t t,
                    AdamArgs* a) {
    if (n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n < 0");
    if (!groups || n_groups < 1 || n_groups > GS_MAX_ADAM_GROUPS)
        return fail(GS_ERR_INVALID_ARGUMENT, "n_groups=%d outside 1..%d", n_groups, GS_MAX_ADAM_GROUPS);
    if (!hp) return fail(GS_ERR_INVALID_ARGUMENT, "hp is null");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) || !(hp->eps > 0.0f))
        return fail(GS_ERR_INVALID_ARGUMENT, "Adam needs 0 <= beta1, beta2 < 1 and eps > 0");
    if (t < 1) return fail(GS_ERR_INVALID_ARGUMENT, "step t=%d < 1", t);
    std::memset(a, 0, sizeof(*a));
    for (int k = 0; k < n_groups; k++) {
        const gs_adam_group& G = groups[k];
        if (!G.param || !G.grad || !G.m || !G.v) return fail(GS_ERR_INVALID_ARGUMENT, "group %d has a null array", k);
        if (G.rows < 1) return fail(GS_ERR_INVALID_ARGUMENT, "group %d: rows=%d", k, G.rows);
        if (!std::isfinite(G.lr)) return fail(GS_ERR_INVALID_ARGUMENT, "group %d: lr is not finite", k);
        if ((int64_t)G.rows * n >= (int64_t(1) << 40)) return fail(GS_ERR_INVALID_ARGUMENT, "group %d too large", k);
        a->groups[k] = AdamGroup{G.param, G.grad, G.m, G.v, G.rows, G.lr};
    }
    a->n_groups = n_groups;
    a->h = AdamHyper{hp->beta1, hp->beta2, hp->eps};
    return GS_OK;
}

}  // namespace

gs_status gs_adam_step(int32_t n, const gs_adam_group* groups, int32_t n_groups, const gs_adam_params* hp,
                       int32_t t, int32_t* last_step, const int32_t* active, int32_t n_active, void* stream) {
    g_last_error.clear();
    AdamArgs a;
    gs_status st = adam_args(n, groups, n_groups, hp, t, &a);
    if (st != GS_OK) return st;
    if (last_step && active && n_active < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n_active < 0");
    return hip_check(launch_adam_step(a, n, t, last_step, last_step ? active : nullptr, n_active,
                                      static_cast<hipStream_t>(stream)),
                     "gs_adam_step launch");
}

gs_status gs_adam_step_seen(int32_t n, const gs_adam_group* groups, int32_t n_groups, const gs_adam_params* hp,
                            int32_t t, int32_t* last_step, const uint8_t* seen, void* stream) {
    g_last_error.clear();
    AdamArgs a;
    gs_status st = adam_args(n, groups, n_groups, hp, t, &a);
    if (st != GS_OK) return st;
    if (n > 0 && (!last_step || !seen)) return fail(GS_ERR_INVALID_ARGUMENT, "last_step or seen is null");
    return hip_check(launch_adam_step_seen(a, n, t, last_step, seen, static_cast<hipStream_t>(stream)),
                     "gs_adam_step_seen launch");
}

gs_status gs_adam_flush(int32_t n, const gs_adam_group* groups, int32_t n_groups, const gs_adam_params* hp,
                        int32_t t, int32_t* last_step, void* stream) {
    g_last_error.clear();
    AdamArgs a;
    gs_status st = adam_args(n, groups, n_groups, hp, t, &a);
    if (st != GS_OK) return st;
    if (!last_step) return fail(GS_ERR_INVALID_ARGUMENT, "last_step is null");
    return hip_check(launch_adam_flush(a, n, t, last_step, static_cast<hipStream_t>(stream)), "gs_adam_flush launch");
}

}  // extern "C"
