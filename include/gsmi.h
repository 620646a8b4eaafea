/*
 * gsmi.h -- C ABI of a single-GPU (MI355X, gfx950) implementation of one training iteration of
 * tile-based differentiable 3D Gaussian splatting: EWA projection, tile binning with a
 * (tile, depth) radix sort, front-to-back alpha compositing, its reverse-order backward pass,
 * a fused forward+backward rasterizer and an optional per-tile cap.
 *
 * Where the operations come from.  ByteSplat (arXiv 2610.02851, English abstract) names the
 * forward and backward rasterization, their fusion into one kernel that keeps intermediates on
 * chip, and pruning under per-tile on-chip memory limits.  Grendel (arXiv 2406.18533, English
 * abstract) notes that each Gaussian touches a small, view-dependent subset of pixels, the
 * sparsity tile binning exploits, and trains on batches of views.  GS-Scale (arXiv 2509.15645,
 * English abstract) culls against each view's frustum.  No page writes out the formulas; the
 * library computes standard EWA splatting, with every open constant in gs_render_params.
 *
 * Conventions for every entry point.
 *  - Pointers inside the structs and the array arguments are DEVICE pointers unless a comment
 *    says "host".  All device memory is owned by the caller; the library never allocates
 *    device memory.  Scratch space comes from a caller-provided workspace whose size the
 *    matching *_workspace_size query returns; it must be 256-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues work on it
 *    and returns, except gs_bin_tiles, which performs one device-to-host read of the counts it
 *    needs to size its launches (and therefore synchronizes `stream`).
 *  - Arguments are validated on the host before anything is enqueued; a call that returns an
 *    error has enqueued nothing, except GS_ERR_HIP, which reports a failed launch or copy
 *    (asynchronous faults of earlier work surface as GS_ERR_HIP from a later call).
 *  - gs_last_error() returns a thread-local message describing the last failure.
 *  - Sizes: Gaussians per call n < 2^28; views per call 1 <= V <= GS_MAX_VIEWS; instances
 *    ((Gaussian, tile) pairs) per call < 2^31.
 *  - Images are float32 [V][3][H][W]; per-pixel maps [V][H][W]; all views of a call share
 *    one width and height.
 *  - The library keeps no state between calls other than the error message.
 */
#ifndef GSMI_H
#define GSMI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GS_MAX_VIEWS 16
#define GS_TILE 16 /* tile side in pixels */

typedef enum {
    GS_OK = 0,
    GS_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, inconsistent cameras, ... */
    GS_ERR_CAPACITY = 2,         /* an output buffer is too small; *required says how large */
    GS_ERR_UNSUPPORTED = 3,      /* a request the library does not serve (e.g. a device index past
                                    the ones it keeps state for) */
    GS_ERR_HIP = 4,              /* a HIP runtime call failed */
    GS_ERR_INTERNAL = 5,         /* a check of the library's own results failed */
    GS_STATUS_FORCE_INT32 = 0x7FFFFFFF /* not a status: makes every int32 value a valid gs_status
                                          (callers in C may pass any int) */
} gs_status;

/* Pinhole camera, OpenCV axes (x right, y down, z forward).  Host struct.
 * Pixel (u, v) covers [u, u+1) x [v, v+1); its centre is (u + 1/2, v + 1/2). */
typedef struct {
    int32_t width, height;
    float fx, fy, cx, cy;   /* focal lengths and principal point, pixels */
    float R[9];             /* world -> camera rotation, row-major */
    float t[3];             /* world -> camera translation: x_cam = R x_world + t */
    float campos[3];        /* camera centre in world coordinates (SH view direction origin) */
} gs_camera;

/* Constants the pages leave open.  Host struct.  Typical values in brackets.  Every call that
 * takes it returns GS_ERR_INVALID_ARGUMENT unless 0 < alpha_min < alpha_max < 1, 0 <= t_min < 1,
 * eps2d and znear are finite and >= 0 (depths must stay positive: their float32 bit patterns
 * are the sort keys), bg is finite, 0 <= sh_degree <= 3 and tile_cap >= 0. */
typedef struct {
    float znear;      /* [0.2]   Gaussians with camera-space z <= znear are culled */
    float eps2d;      /* [0.3]   low-pass dilation added to the 2D covariance diagonal, px^2 */
    float alpha_min;  /* [1/255] pairs with alpha below this are skipped */
    float alpha_max;  /* [0.99]  alpha = min(alpha_max, o * exp(-q/2)) */
    float t_min;      /* [1e-4]  a pixel stops before a blend that would take T below t_min */
    float bg[3];      /* [0,0,0] background colour, added as T_final * bg */
    int32_t sh_degree;/* 0..3 */
    int32_t tile_cap; /* 0 = off; else keep at most this many entries per tile (gs_bin_tiles) */
} gs_render_params;

/* Gaussian parameters, structure of arrays, float32, device. */
typedef struct {
    int32_t n;
    const float* means;          /* [3][n] world position */
    const float* log_scales;     /* [3][n] per-axis log standard deviation */
    const float* quats;          /* [4][n] rotation (w, x, y, z), need not be normalized */
    const float* opacity_logits; /* [n]    opacity = sigmoid(logit) */
    const float* sh;             /* [3*(d+1)^2][n], row k*3 + channel; row 0..2 = DC = base colour */
} gs_gaussians;

/* Opaque host-side buffer for the per-view counts: pinned host memory and an event (see
 * gs_readback_create).  Owned by the caller through create/destroy. */
typedef struct gs_readback gs_readback;

/* Per-view projected records, indexed by visible slot.  All arrays are [V][capacity][...]
 * with capacity >= n; slot s of view v lives at index v*capacity + s.  Visible Gaussians of
 * a view take slots 0..vis_count[v]-1 in ascending Gaussian index.  mean2d, conic_opacity and
 * color are optional (NULL: not written; the packed record holds the same values): no call
 * needs them, and gs_bin_tiles with tile_cap > 0 reads the conic and opacity from
 * conic_opacity when it is given, else from raster_rec. */
typedef struct {
    int32_t capacity;
    int32_t* vis_count;       /* [V]  number of visible Gaussians per view */
    int64_t* inst_count;      /* [V]  sum of n_tiles per view ((Gaussian, tile) instances) */
    int32_t* vis_ids;         /* [V][capacity]    Gaussian index of each slot */
    float* mean2d;            /* [V][capacity][2] projected centre, pixels (optional) */
    float* conic_opacity;     /* [V][capacity][4] (A, B, C, o): q = A dx^2 + 2B dx dy + C dy^2
                                 (optional) */
    float* color;             /* [V][capacity][3] RGB after the lower clamp at 0 (optional) */
    float* depth;             /* [V][capacity]    camera-space z */
    uint16_t* tile_rect;      /* [V][capacity][4] (tx0, ty0, tx1, ty1), inclusive */
    int32_t* n_tiles;         /* [V][capacity]    tiles in the rectangle */
    int32_t* inst_base;       /* [V][capacity]    first index of the slot's (Gaussian, tile) instances
                                 when the instances of all views are numbered view by view, slot by
                                 slot, and within a slot row-major over its tile rectangle: the sum
                                 of n_tiles over every earlier (view, slot) */
    float* raster_rec;        /* [V][capacity][16] the record the rasterizers read, packed into one
                                 64-byte line per slot (256-byte aligned array): x, y, A, B, C, o,
                                 r, g, b, then as 32-bit patterns tx0 | ty0 << 16, tx1 | ty1 << 16,
                                 inst_base, then depth, n_tiles (32-bit pattern), 0, 0 */
    gs_readback* readback;    /* optional (may be NULL): when set, gs_project copies the per-view
                                 visible and instance counts and the visible depth range into it
                                 as soon as they are known (before the records are written), and
                                 gs_bin_tiles takes them from there instead of reading the device;
                                 it holds the counts of the last gs_project call that named it */
} gs_projected;

/* Tile bins of all views of one call.  Global tile id = v * tiles_per_view + ty * tiles_x + tx.
 * ranges[g] = [start, end) into vals (positions over all views); empty tiles hold (0, 0). */
typedef struct {
    int64_t capacity;           /* instance capacity of tile_keys / vals / vals_capped */
    int64_t count;              /* written by gs_bin_tiles (host value): instances of all views on
                                   success, -1 after a failed call; the raster calls refuse
                                   bins whose count is negative */
    uint32_t* tile_keys;        /* [capacity] global tile id of each sorted instance */
    int32_t* vals;              /* [capacity] slot of each sorted instance */
    int32_t* ranges;            /* [V * tiles_per_view][2] */
    int32_t* vals_capped;       /* [capacity]  only written when tile_cap > 0 */
    int32_t* ranges_capped;     /* [V * tiles_per_view][2]  only written when tile_cap > 0 */
    int32_t* num_capped;        /* [1] instances kept by the cap, all views (tile_cap > 0) */
    int32_t* tile_order;        /* [V * tiles_per_view] optional (may be NULL): a permutation of
                                   the global tiles, longest lists first, written by gs_bin_tiles
                                   and used by the raster calls to schedule heavy tiles early;
                                   the order changes no result */
} gs_bins;

/* Host-side counts that gs_bin_tiles reports. */
typedef struct {
    int32_t vis_count[GS_MAX_VIEWS];
    int64_t view_offset[GS_MAX_VIEWS + 1]; /* first instance position of each view */
    int64_t num_instances;                 /* all views */
    int64_t num_instances_capped;          /* = num_instances when the cap is off; -1 when it is
                                              on (the count is then on the device, bins->num_capped) */
} gs_bin_info;

/* Per-slot 2D gradients, [V][capacity][k], float32, device.  The backward calls overwrite the
 * entries of every visible slot (slots >= vis_count are left untouched). */
typedef struct {
    float* d_mean2d;  /* [V][capacity][2] dL/d mean2d (pixels) */
    float* d_conic;   /* [V][capacity][3] dL/d (A, B, C) */
    float* d_opacity; /* [V][capacity]    dL/d o (activated opacity) */
    float* d_color;   /* [V][capacity][3] dL/d colour (post-clamp RGB) */
} gs_grads2d;

/* Per-Gaussian parameter gradients, float32, device, in the layout of gs_gaussians. */
typedef struct {
    float* d_means;          /* [3][n] */
    float* d_log_scales;     /* [3][n] */
    float* d_quats;          /* [4][n] with respect to the raw (unnormalized) quaternion */
    float* d_opacity_logits; /* [n] */
    float* d_sh;             /* [3*(d+1)^2][n], row k*3 + channel */
} gs_grads3d;

typedef enum {
    GS_LOSS_L1 = 0,
    GS_LOSS_EXTERNAL = 1,
    GS_LOSS_MODE_FORCE_INT32 = 0x7FFFFFFF /* not a mode: any int32 value is a valid gs_loss_mode,
                                             so that an unknown one is refused, not undefined */
} gs_loss_mode;

/* Optional per-call diagnostics: device int64 [4], accumulated (the caller zeroes them); pass
 * NULL to skip (counting selects a slower kernel variant).  [0] (pixel, list entry) pairs the
 * forward evaluated; [1] pairs blended; [2] evaluated pairs whose alpha reaches alpha_min (the
 * blended pairs plus, per pixel, at most the one at which it stops: every correct method must
 * evaluate these, whatever it culls); [3] list entries staged from the packed records into LDS
 * (every forward batch, and in gs_raster_fused every batch the backward stages again). */
typedef int64_t gs_counters;

const char* gs_version(void);
const char* gs_status_string(gs_status s);
const char* gs_last_error(void);

/*
 * Host-side count buffer for gs_projected.readback: page-locked host memory for the counts of
 * up to GS_MAX_VIEWS views and an event that gs_project records after its copy.  With it, the
 * one device-to-host read of an iteration overlaps the projection's record-writing pass, and
 * gs_bin_tiles waits for that copy only, not for the stream; the GPU keeps working while the
 * host sizes the binning launches.  *out is set on success.  A buffer serves one projection at
 * a time: calls that name the same buffer must not overlap.  Errors: GS_ERR_INVALID_ARGUMENT
 * for out == NULL; GS_ERR_HIP if the pinned allocation or the event cannot be created.
 */
gs_status gs_readback_create(gs_readback** out);
/* Releases a buffer from gs_readback_create (NULL is ignored).  Waits for a pending copy. */
void gs_readback_destroy(gs_readback* r);

/* Workspace bytes of gs_project for n Gaussians and V views. */
size_t gs_project_workspace_size(int32_t n, int32_t V);

/*
 * A1: project every Gaussian into each of V views.  Per Gaussian and view: activations
 * (sigmoid opacity, exp scales, normalized quaternion); camera transform and near cull; world
 * covariance R diag(s^2) R^T; EWA 2D covariance J W Sigma W^T J^T + eps2d I, conic = its
 * inverse; projected centre; colour from spherical harmonics along the view direction (DC is
 * the base colour; lower clamp at 0); the exact bounding box of the region where
 * o exp(-q/2) >= alpha_min (half extents 1.001 sqrt(2 ln(o/alpha_min) Sigma'_xx) etc.) clipped
 * to the image, and its tile rectangle.  Gaussians with any non-finite input or derived value,
 * det <= 0, o <= alpha_min or an empty box are culled (per-view frustum culling as in GS-Scale,
 * arXiv 2509.15645, English abstract).  Visible Gaussians are compacted into slots in ascending
 * index order.  Besides the per-field arrays (mean2d, conic_opacity and color only where given),
 * every visible slot gets its instance base and the packed 64-byte rasterizer record.
 * Parameters are read once for all V views.
 * Errors: GS_ERR_INVALID_ARGUMENT for null pointers, n < 0, V outside 1..GS_MAX_VIEWS,
 * capacity < n, sh_degree outside 0..3, non-positive image sizes or differing image sizes
 * between views; GS_ERR_CAPACITY if ws_bytes is too small.
 */
gs_status gs_project(const gs_gaussians* g, const gs_camera* cams /*host [V]*/, int32_t V,
                     const gs_render_params* p, gs_projected* out, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * gs_project without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * projection's scratch (per-wavefront counts and their scans, per-wavefront depth ranges, the
 * count summary, one flag byte per Gaussian: about 2.1 bytes per Gaussian at 4 views) lives in a
 * static device array of gs_project_noalloc_max_bytes() = 16 MiB that the library holds on every
 * device it runs on until the process ends.  Calls nothing that allocates.  Same arguments, outputs and errors
 * as gs_project, plus GS_ERR_CAPACITY when gs_project_workspace_size(n, V) exceeds that size
 * (about 7.8 million Gaussians at 4 views), and GS_ERR_HIP if the array's device address cannot
 * be found.  All calls on one device share the array: calls that overlap in time on one device
 * (from several host threads or streams) race and must be serialised by the caller.
 */
gs_status gs_project_noalloc(const gs_gaussians* g, const gs_camera* cams /*host [V]*/, int32_t V,
                             const gs_render_params* p, gs_projected* out, void* stream);

/* The static scratch of gs_project_noalloc, in bytes. */
size_t gs_project_noalloc_max_bytes(void);

/* Workspace bytes of gs_raster_bwd / gs_raster_fused for an instance capacity: one float32
 * partial-gradient record (9 values) per (Gaussian, tile) instance, then a short list of the
 * slots with more than 256 instances (16 bytes per 256 instances), whose records one workgroup
 * each adds up, then the fused call's fixed-point loss sum (8 bytes). */
size_t gs_raster_workspace_size(int64_t instance_capacity);

/* Workspace bytes of gs_bin_tiles for n Gaussians, V views and an instance capacity. */
size_t gs_bin_workspace_size(int32_t n, int32_t V, int32_t width, int32_t height, int64_t instance_capacity);

/*
 * A2-A6: bin the visible slots of all V views into 16x16 tiles.  Instances (one per slot and
 * tile of its rectangle) are ordered by (view, tile, depth, slot) with an LSD radix sort whose
 * low (depth) digits are sorted once per slot before the instances are emitted (the emission
 * keeps each slot's depth, so this is the same stable sort of the (tile, depth) key); the
 * result is a total order, so tile ids, order and ranges are exact.  With tile_cap K > 0,
 * every tile holding more than K entries keeps the K entries with the largest
 * score = o / sqrt(A C - B^2) (opacity times the square root of the dilated covariance's
 * determinant, evaluated in float32 with one rounding per operation), ties broken by
 * depth then slot, kept in depth order (ByteSplat's pruning under per-tile on-chip limits).
 * Reads the per-view counts back to the host once (info, host), then sizes its launches: from
 * proj->readback when the last gs_project filled it (waiting on that copy's event only), else
 * by its own copy from the device (synchronizing the stream).
 * Errors: GS_ERR_INVALID_ARGUMENT as for gs_project, and when tile_cap > 0 while both
 * proj->conic_opacity and proj->raster_rec are NULL; GS_ERR_CAPACITY (with *required, host,
 * set to the instances needed) when bins->capacity is too small, in which case the bins are
 * left undefined; GS_ERR_CAPACITY if the workspace is too small.
 */
gs_status gs_bin_tiles(const gs_camera* cams /*host [V]*/, const gs_projected* proj, int32_t V,
                       const gs_render_params* p, gs_bins* bins, gs_bin_info* info /*host*/,
                       int64_t* required /*host*/, void* ws, size_t ws_bytes, void* stream);

/*
 * A7: forward rasterization (ByteSplat, arXiv 2610.02851, English abstract: forward
 * rasterization, one of the two passes whose repeated off-chip accesses it names as a
 * bottleneck; the compositing rule is the plain front-to-back reading below, which no page
 * writes out).  One 256-thread workgroup per 16x16 tile and view; records of the tile list are
 * staged in LDS in batches.  Per pixel, front to back:
 * alpha = min(alpha_max, o exp(-q/2)); skip alpha < alpha_min; stop before a blend that would
 * take T below t_min; C += alpha T c; T *= (1 - alpha); at the end C += T bg.
 * n_contrib = 1 + list position of the last blended entry (0 if none).  `use_capped` selects
 * the capped lists.  Outputs: image [V][3][H][W], t_final [V][H][W], n_contrib [V][H][W].
 */
gs_status gs_raster_fwd(const gs_camera* cams /*host [V]*/, const gs_projected* proj, const gs_bins* bins,
                        int32_t V, const gs_render_params* p, int32_t use_capped, float* image,
                        float* t_final, int32_t* n_contrib, gs_counters* counters, void* stream);

/* A8: dL/dC of L = scale * sum |C - target| (L1): scale * sign(C - target), sign(0) = 0.
 * image, target, dl_dimage: [V][3][H][W].  loss_sum (optional, device float, accumulated with
 * float atomics: its last bits may differ between calls; gs_raster_fused's loss sum does not). */
gs_status gs_loss_l1_grad(int32_t V, int32_t width, int32_t height, const float* image, const float* target,
                          float scale, float* dl_dimage, float* loss_sum, void* stream);

/*
 * A9: backward rasterization (ByteSplat, arXiv 2610.02851, English abstract: backward
 * rasterization, the second of the two passes; the derivative is the chain rule of A7's
 * compositing, which no page writes out).  Per pixel, back to front from n_contrib: T is
 * recovered by division by (1 - alpha); with Bk the colour behind entry j,
 *   dL/dc_j = alpha_j T_j g,  dL/dalpha_j = sum_ch g_ch (T_j (c_j - Bk) - T_final bg / (1 - alpha_j)),
 * and unless alpha was clamped, dL/do = G dL/dalpha, dL/dmean2d = o G dL/dalpha (A dx + B dy,
 * B dx + C dy) with d = pixel centre - mean2d, dL/d(A,B,C) = o G dL/dalpha (-dx^2/2, -dx dy,
 * -dy^2/2).  Within a tile, each entry's contributions are summed over the pixels in LDS and
 * stored once, without atomics, as a partial record at the instance's index (see
 * gs_projected.inst_base) in the workspace; a per-Gaussian pass then sums each slot's partials
 * into grads.  Every sum is taken in a fixed order, so repeated calls give identical bits.
 * ws: gs_raster_workspace_size(bins->count) bytes or more, 256-byte aligned.
 */
gs_status gs_raster_bwd(const gs_camera* cams /*host [V]*/, const gs_projected* proj, const gs_bins* bins,
                        int32_t V, const gs_render_params* p, int32_t use_capped, const float* image,
                        const float* t_final, const int32_t* n_contrib, const float* dl_dimage,
                        gs_grads2d* grads, void* ws, size_t ws_bytes, void* stream);

/*
 * A10: fused forward + loss gradient + backward in one kernel per tile (ByteSplat, arXiv
 * 2610.02851, English abstract: forward and backward rasterization fused into one kernel that
 * keeps intermediates on chip).  Per-pixel colour, transmittance and n_contrib stay in
 * registers; records are staged through LDS in batches, and the last forward batch is reused as
 * the first backward batch.  mode GS_LOSS_L1: target_or_dldc is the target image and the
 * gradient is loss_scale * sign(C - target); GS_LOSS_EXTERNAL: target_or_dldc is dL/dC.
 * image_opt (optional) receives the rendered image; loss_sum_opt (optional, device float)
 * accumulates scale * sum |C - target| (L1 mode only), summed in fixed point (units of 2^-20
 * per wavefront's partial) so that repeated calls give identical bits.  Same gradients as A7+A8+A9, gathered the
 * same way (ws as for gs_raster_bwd).
 */
gs_status gs_raster_fused(const gs_camera* cams /*host [V]*/, const gs_projected* proj, const gs_bins* bins,
                          int32_t V, const gs_render_params* p, int32_t use_capped, gs_loss_mode mode,
                          const float* target_or_dldc, float loss_scale, float* image_opt,
                          float* loss_sum_opt, gs_grads2d* grads, gs_counters* counters, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Backward of A1 (the step that follows the rasterizer backward in training, which ByteSplat,
 * arXiv 2610.02851, English abstract, names as the workload; no page writes it out): the chain
 * rule of gs_project from the per-slot gradients `grads2d` of V views (dL/d mean2d, conic (A, B,
 * C), activated opacity and clamped colour, as gs_raster_bwd / gs_raster_fused write them) to
 * the parameters, summed over the views in which each Gaussian is visible:
 *   conic -> dilated 2D covariance -> J W and the world covariance R diag(s^2) R^T -> log-scales
 *   and the normalized quaternion -> raw quaternion; J(t) and the projected centre -> camera
 *   point t = W mu + t_cam -> mean; colour = max(0, DC + sum_k sh_k Y_k(dir)) -> SH rows (only
 *   for channels above zero) and, through dir = unit(mu - campos), the mean;
 *   opacity = sigmoid(logit) -> logit.
 * The culling and box decisions are piecewise constant and carry no gradient.  `proj` must be
 * the output of gs_project for the same parameters, cameras and params (its vis_count and vis_ids
 * are read: the slots of a view hold ascending Gaussian indices).  Every entry of `out` is
 * overwritten (zero for Gaussians that no view sees).  One thread per Gaussian; no workspace.
 * Errors: GS_ERR_INVALID_ARGUMENT for null pointers or sizes as for gs_project.
 */
gs_status gs_project_bwd(const gs_gaussians* g, const gs_camera* cams /*host [V]*/, int32_t V,
                         const gs_render_params* p, const gs_projected* proj, const gs_grads2d* grads2d,
                         gs_grads3d* out, void* stream);

/*
 * gs_project_bwd for training with frustum culling and deferred updates (GS-Scale, arXiv
 * 2509.15645, English abstract: frustum culling and a deferred optimizer update keep the
 * Gaussians outside the views from costing memory traffic): the same gradients for every
 * Gaussian that some view sees, but the gradient rows of the others are neither read nor written
 * (they keep whatever they held); seen (device uint8 [n], written) is 1 for a Gaussian that some
 * view's visible set holds and 0 otherwise, the flags gs_adam_step_seen takes.  The rows written
 * are bit-identical to gs_project_bwd's.  Errors: those of gs_project_bwd, and
 * GS_ERR_INVALID_ARGUMENT for a null seen with n > 0.
 */
gs_status gs_project_bwd_seen(const gs_gaussians* g, const gs_camera* cams /*host [V]*/, int32_t V,
                              const gs_render_params* p, const gs_projected* proj, const gs_grads2d* grads2d,
                              gs_grads3d* out, uint8_t* seen, void* stream);

/*
 * GS_CHECK, a debug aid: validates on the device what gs_bin_tiles wrote for `proj`, `V` views
 * and params `p` (the full lists, and the capped ones too when p->tile_cap > 0), against the
 * properties the (view, tile, depth, slot) order fixes.  violations (host [GS_CHECK_KINDS]) receives
 * the count of each kind:
 *   GS_CHECK_RANGE       a tile range reversed, outside [0, count), non-zero while empty, or not
 *                        where the partition of [0, count) in global tile order puts it;
 *   GS_CHECK_KEY         a full-list entry whose sorted tile key is not its range's tile;
 *   GS_CHECK_SLOT        an entry naming no visible slot of its tile's view;
 *   GS_CHECK_RECT        an entry whose tile lies outside its slot's tile rectangle;
 *   GS_CHECK_ORDER       a list that is not strictly increasing in (depth, slot);
 *   GS_CHECK_COUNT       list lengths that do not add up to each view's instances (the slots'
 *                        n_tiles; for capped lists, to *num_capped and at most the full lists);
 *   GS_CHECK_CAP         a capped list longer than the cap;
 *   GS_CHECK_SLOT_RECORD a slot rectangle off the tile grid, an n_tiles that is not its area, or
 *                        instance bases that do not follow the slots view by view.
 * Allocates a small device buffer and synchronizes the stream (never call it where allocation or
 * waiting is not allowed).  Returns GS_ERR_INTERNAL, naming the kinds found, when any count is
 * non-zero; GS_ERR_INVALID_ARGUMENT for null pointers or bins without a successful count.
 */
#define GS_CHECK_RANGE 0
#define GS_CHECK_KEY 1
#define GS_CHECK_SLOT 2
#define GS_CHECK_RECT 3
#define GS_CHECK_ORDER 4
#define GS_CHECK_COUNT 5
#define GS_CHECK_CAP 6
#define GS_CHECK_SLOT_RECORD 7
#define GS_CHECK_KINDS 8
gs_status gs_check_bins(const gs_camera* cams /*host [V]*/, const gs_projected* proj, int32_t V,
                        const gs_render_params* p, const gs_bins* bins, int64_t* violations /*host*/,
                        void* stream);

/*
 * The largest per-tile cap K (gs_render_params.tile_cap) under which gs_raster_fused keeps every
 * tile's list on chip from the forward through the backward: a list of at most K entries is
 * staged from the packed records into LDS once, in one batch, and the backward walks that same
 * batch (ByteSplat, English abstract: pruning that respects per-tile shared-memory limits).
 * Longer lists (a larger cap, or none) are still rendered exactly: they stream through LDS in
 * batches of K entries and the backward stages every batch but the last one again, which
 * diagnostics counter [3] shows.  *k (host) receives K.
 */
gs_status gs_fused_max_cap(int32_t* k);

/*
 * F2: sparse exchange of the per-view 2D gradient records (ByteSplat, English abstract: zero
 * partial gradients are left out of the exchange between GPUs; an encoder kernel compacts the
 * remaining records and a decoder kernel adds the received records directly into the arrays of
 * the Gaussians' owner).  On one GPU the pair is the encoder and decoder of that exchange.
 *
 * gs_grad_encode: a record is the nine 2D gradient components of one (view v, visible slot
 * s < vis_count[v]) of grads (d_mean2d x, y, d_conic A, B, C, d_opacity, d_color r, g, b, at
 * index v*capacity + s, the layout the backward calls write).  Every record with a component
 * other than zero (a NaN counts as non-zero, -0 as zero) is written as keys[k] =
 * vis_ids[v*capacity + s] (its Gaussian) and records[k*9 .. k*9+8] = the nine components in that
 * order, k increasing with (view, slot).  view_offset (device int32 [V+1]) receives the first
 * record of each view and, at [V], the number of records.  keys and records must hold
 * V*capacity records (all visible slots kept); view_offset must not overlap them.  ws:
 * gs_grad_encode_workspace_size(capacity, V) bytes or more, 256-byte aligned.  capacity and
 * vis_count/vis_ids are those of the gs_projected the gradients belong to.
 */
size_t gs_grad_encode_workspace_size(int32_t capacity, int32_t V);
gs_status gs_grad_encode(int32_t V, int32_t capacity, const int32_t* vis_count, const int32_t* vis_ids,
                         const gs_grads2d* grads, int32_t* keys, float* records, int32_t* view_offset, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * gs_grad_decode: adds every record k of an encoded stream into the owner arrays: for the view
 * v with view_offset[v] <= k < view_offset[v+1], owner entry v*n_owner + keys[k] of each
 * gs_grads2d array (owner->d_mean2d [V][n_owner][2], ...) is incremented by the record's
 * components; keys outside [0, n_owner) are skipped.  Within one stream every (view, Gaussian)
 * appears at most once, so a decode touches each entry at most once; decoding several streams in
 * sequence accumulates them.  max_records (host) bounds view_offset[V] (V*capacity of the
 * encode) and sizes the launch.
 */
gs_status gs_grad_decode(int32_t V, int32_t n_owner, int64_t max_records, const int32_t* view_offset,
                         const int32_t* keys, const float* records, gs_grads2d* owner, void* stream);

#define GS_MAX_PARTIALS 16

/*
 * F3: global composition of pixel-level partial renders (Splaxel, English abstract: each GPU
 * renders its local subset of the Gaussians and only partial pixel values are exchanged and
 * composed into the image).  A partial render of a subset of the Gaussians is gs_raster_fwd's
 * image and t_final for that subset drawn on a black background (bg = 0): its premultiplied
 * colour C and its final transmittance T.  Given P partials in front-to-back order, writes
 *   image = C_1 + T_1 (C_2 + T_2 (... + T_{P-1} C_P)) + (T_1 T_2 ... T_P) bg,
 *   t_out = T_1 T_2 ... T_P   (t_out may be NULL),
 * per view and pixel.  For subsets whose Gaussians are depth-separated in every view (all of
 * subset i in front of all of subset i+1 along every pixel's ray: per-pixel, every Gaussian of
 * subset i sorts before every Gaussian of subset i+1) and with t_min = 0 (no early stop), this
 * equals rendering the union up to float32 rounding.
 * colors (host [P]): device [V][3][H][W] each; t_finals (host [P]): device [V][H][W] each;
 * bg (host [3]); 1 <= P <= GS_MAX_PARTIALS.  image may alias colors[0] and t_out t_finals[0]
 * (each pixel is read before it is written by the same thread).
 */
gs_status gs_compose(int32_t P, int32_t V, int32_t width, int32_t height, const float* const* colors,
                     const float* const* t_finals, const float* bg, float* image, float* t_out, void* stream);

#define GS_MAX_ADAM_GROUPS 8

/* One parameter group of gs_adam_step / gs_adam_flush: rows x n float32 arrays (row r of
 * Gaussian i at r*n + i, the layout of gs_gaussians / gs_grads3d), device pointers. */
typedef struct {
    float* param;       /* [rows][n] parameters, updated in place */
    const float* grad;  /* [rows][n] gradients of this step */
    float* m;           /* [rows][n] first moments (start at 0) */
    float* v;           /* [rows][n] second moments (start at 0) */
    int32_t rows;
    float lr;           /* learning rate of the group */
} gs_adam_group;

typedef struct {
    float beta1, beta2, eps; /* [0.9, 0.999, 1e-15..1e-8] */
} gs_adam_params;

/*
 * F4: one Adam step t >= 1 (textbook Adam per component: m = b1 m + (1 - b1) g,
 * v = b2 v + (1 - b2) g^2, p -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps), in float32),
 * dense or deferred (GS-Scale, English abstract: a deferred optimizer update avoids the memory
 * accesses of Gaussians with zero gradients).
 *  - last_step == NULL: dense; every Gaussian takes step t (active is ignored).
 *  - last_step != NULL (device int32 [n], 0 before the first step): deferred.  The candidates are
 *    all n Gaussians when active == NULL, and a candidate whose gradient is zero in every row of
 *    every group is left untouched; with active (device int32 [n_active]) the candidates are the
 *    listed Gaussians, each updated even if its gradient is zero, and the caller guarantees that
 *    every unlisted Gaussian has a zero gradient at step t.  An updated Gaussian first replays
 *    steps last_step+1 .. t-1 with a zero gradient, then takes step t; last_step becomes t.
 *    Gaussians with last_step >= t are left alone.
 * The replay performs the dense step's float32 operations in the same order, so after
 * gs_adam_flush(t) the parameters and moments equal those of t dense steps bit for bit.
 * groups (host [n_groups], 1 <= n_groups <= GS_MAX_ADAM_GROUPS), hp (host).
 */
gs_status gs_adam_step(int32_t n, const gs_adam_group* groups, int32_t n_groups, const gs_adam_params* hp,
                       int32_t t, int32_t* last_step, const int32_t* active, int32_t n_active, void* stream);

/*
 * F4, deferred, with the Gaussians to update named by flags (GS-Scale, English abstract, as for
 * gs_adam_step): the candidates are the Gaussians with seen[i] != 0 (device uint8 [n], as
 * gs_project_bwd_seen writes it), each updated as in gs_adam_step's deferred form even if its
 * gradient is zero; a Gaussian with seen[i] == 0 is left untouched and its gradient rows are not
 * read (the caller guarantees its gradient is zero at step t, which holds for a Gaussian no view
 * sees).  last_step (device int32 [n]) as for gs_adam_step; after gs_adam_flush(t) the parameters
 * and moments equal those of t dense steps bit for bit.  Errors: those of gs_adam_step, and
 * GS_ERR_INVALID_ARGUMENT for a null last_step or seen with n > 0.
 */
gs_status gs_adam_step_seen(int32_t n, const gs_adam_group* groups, int32_t n_groups, const gs_adam_params* hp,
                            int32_t t, int32_t* last_step, const uint8_t* seen, void* stream);

/* F4: bring every Gaussian of a deferred state to step t (replay of its steps after last_step
 * with a zero gradient; last_step becomes t).  Same arguments as gs_adam_step. */
gs_status gs_adam_flush(int32_t n, const gs_adam_group* groups, int32_t n_groups, const gs_adam_params* hp,
                        int32_t t, int32_t* last_step, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GSMI_H */
