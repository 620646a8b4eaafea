/* One training iteration of the hot path driven from plain C through the C ABI and the HIP
 * runtime's C API (no Python, no PyTorch): gs_project -> gs_bin_tiles (grown and retried once on
 * GS_ERR_CAPACITY) -> gs_raster_fwd and gs_raster_fused (L1 against a target).  Reads the scene
 * from argv[1] and writes every output the checks need to argv[2]; both files are raw
 * little-endian arrays in the order read_input / main write them. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gsmi.h"

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

#define GS_OK_(call)                                                                  \
    do {                                                                              \
        gs_status s_ = (call);                                                        \
        if (s_ != GS_OK) {                                                            \
            fprintf(stderr, "%s failed: %s (%s)\n", #call, gs_status_string(s_), gs_last_error()); \
            return 3;                                                                 \
        }                                                                             \
    } while (0)

static int read_all(FILE* f, void* p, size_t bytes) { return fread(p, 1, bytes, f) == bytes; }

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    if (hipMalloc(&p, bytes ? bytes : 4) != hipSuccess) return NULL;
    return p;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s scene.bin out.bin\n", argv[0]);
        return 1;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) return 1;
    int32_t hdr[4]; /* n, width, height, sh degree */
    float camf[19]; /* fx fy cx cy R[9] t[3] campos[3] */
    if (!read_all(in, hdr, sizeof(hdr)) || !read_all(in, camf, sizeof(camf))) return 1;
    const int32_t n = hdr[0], W = hdr[1], H = hdr[2], deg = hdr[3];
    if (n <= 0 || n > (1 << 20) || W <= 0 || H <= 0 || W > 4096 || H > 4096 || deg < 0 || deg > 3) return 1;
    const int32_t nk3 = 3 * (deg + 1) * (deg + 1);
    const size_t params = (size_t)(3 + 3 + 4 + 1 + nk3) * n, npx = (size_t)W * H;
    float* host = (float*)malloc(sizeof(float) * (params + 3 * npx));
    if (!host || !read_all(in, host, sizeof(float) * (params + 3 * npx))) return 1;
    fclose(in);

    gs_camera cam;
    memset(&cam, 0, sizeof(cam));
    cam.width = W;
    cam.height = H;
    cam.fx = camf[0];
    cam.fy = camf[1];
    cam.cx = camf[2];
    cam.cy = camf[3];
    memcpy(cam.R, camf + 4, sizeof(cam.R));
    memcpy(cam.t, camf + 13, sizeof(cam.t));
    memcpy(cam.campos, camf + 16, sizeof(cam.campos));
    gs_render_params p;
    memset(&p, 0, sizeof(p));
    p.znear = 0.2f;
    p.eps2d = 0.3f;
    p.alpha_min = 1.0f / 255.0f;
    p.alpha_max = 0.99f;
    p.t_min = 1e-4f;
    p.sh_degree = deg;

    /* parameters and target on the device */
    float* d_params = (float*)dev_alloc(sizeof(float) * params);
    float* d_target = (float*)dev_alloc(sizeof(float) * 3 * npx);
    if (!d_params || !d_target) return 2;
    HIP_OK(hipMemcpy(d_params, host, sizeof(float) * params, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_target, host + params, sizeof(float) * 3 * npx, hipMemcpyHostToDevice));
    gs_gaussians g;
    g.n = n;
    g.means = d_params;
    g.log_scales = d_params + 3 * (size_t)n;
    g.quats = d_params + 6 * (size_t)n;
    g.opacity_logits = d_params + 10 * (size_t)n;
    g.sh = d_params + 11 * (size_t)n;

    /* projected records (capacity n, one view) */
    gs_projected pr;
    memset(&pr, 0, sizeof(pr));
    pr.capacity = n;
    pr.vis_count = (int32_t*)dev_alloc(sizeof(int32_t));
    pr.inst_count = (int64_t*)dev_alloc(sizeof(int64_t));
    pr.vis_ids = (int32_t*)dev_alloc(sizeof(int32_t) * n);
    pr.mean2d = (float*)dev_alloc(sizeof(float) * 2 * n);
    pr.conic_opacity = (float*)dev_alloc(sizeof(float) * 4 * n);
    pr.color = (float*)dev_alloc(sizeof(float) * 3 * n);
    pr.depth = (float*)dev_alloc(sizeof(float) * n);
    pr.tile_rect = (uint16_t*)dev_alloc(sizeof(uint16_t) * 4 * n);
    pr.n_tiles = (int32_t*)dev_alloc(sizeof(int32_t) * n);
    pr.inst_base = (int32_t*)dev_alloc(sizeof(int32_t) * n);
    pr.raster_rec = (float*)dev_alloc(sizeof(float) * 16 * n); /* hipMalloc: 256-byte aligned */
    const size_t ws_p_bytes = gs_project_workspace_size(n, 1);
    void* ws_p = dev_alloc(ws_p_bytes);
    if (!pr.raster_rec || !ws_p) return 2;
    GS_OK_(gs_project(&g, &cam, 1, &p, &pr, ws_p, ws_p_bytes, NULL));

    /* bins: a first guess of 4 instances per Gaussian, grown once if too small */
    const int32_t tiles = ((W + 15) / 16) * ((H + 15) / 16);
    gs_bins b;
    memset(&b, 0, sizeof(b));
    b.ranges = (int32_t*)dev_alloc(sizeof(int32_t) * 2 * tiles);
    int64_t cap = 4 * (int64_t)n, required = 0;
    gs_bin_info info;
    gs_status st = GS_ERR_CAPACITY;
    void* ws_b = NULL;
    for (int attempt = 0; attempt < 2 && st == GS_ERR_CAPACITY; attempt++) {
        if (attempt == 1) {
            HIP_OK(hipFree(b.tile_keys));
            HIP_OK(hipFree(b.vals));
            HIP_OK(hipFree(ws_b));
            cap = required;
        }
        b.capacity = cap;
        b.tile_keys = (uint32_t*)dev_alloc(sizeof(uint32_t) * cap);
        b.vals = (int32_t*)dev_alloc(sizeof(int32_t) * cap);
        const size_t ws_b_bytes = gs_bin_workspace_size(n, 1, W, H, cap);
        ws_b = dev_alloc(ws_b_bytes);
        if (!b.tile_keys || !b.vals || !ws_b) return 2;
        st = gs_bin_tiles(&cam, &pr, 1, &p, &b, &info, &required, ws_b, ws_b_bytes, NULL);
    }
    GS_OK_(st);
    const int64_t m = b.count;

    /* separate forward, then the fused forward + L1 gradient + backward */
    float* image = (float*)dev_alloc(sizeof(float) * 3 * npx);
    float* image_fused = (float*)dev_alloc(sizeof(float) * 3 * npx);
    float* t_final = (float*)dev_alloc(sizeof(float) * npx);
    int32_t* n_contrib = (int32_t*)dev_alloc(sizeof(int32_t) * npx);
    gs_grads2d gr;
    gr.d_mean2d = (float*)dev_alloc(sizeof(float) * 2 * n);
    gr.d_conic = (float*)dev_alloc(sizeof(float) * 3 * n);
    gr.d_opacity = (float*)dev_alloc(sizeof(float) * n);
    gr.d_color = (float*)dev_alloc(sizeof(float) * 3 * n);
    const size_t ws_r_bytes = gs_raster_workspace_size(m);
    void* ws_r = dev_alloc(ws_r_bytes);
    if (!image || !image_fused || !t_final || !n_contrib || !gr.d_color || !ws_r) return 2;
    GS_OK_(gs_raster_fwd(&cam, &pr, &b, 1, &p, 0, image, t_final, n_contrib, NULL, NULL));
    GS_OK_(gs_raster_fused(&cam, &pr, &b, 1, &p, 0, GS_LOSS_L1, d_target, 1.0f, image_fused, NULL, &gr, NULL, ws_r,
                           ws_r_bytes, NULL));
    HIP_OK(hipDeviceSynchronize());

    /* everything back to the host, in the order the checks read it */
    FILE* out = fopen(argv[2], "wb");
    if (!out) return 1;
    int32_t vis = 0;
    HIP_OK(hipMemcpy(&vis, pr.vis_count, sizeof(vis), hipMemcpyDeviceToHost));
    fwrite(&vis, sizeof(vis), 1, out);
    fwrite(&m, sizeof(m), 1, out);
    fwrite(&tiles, sizeof(tiles), 1, out);
    struct {
        const void* dev;
        size_t bytes;
    } outs[] = {
        {pr.vis_ids, sizeof(int32_t) * vis},         {pr.mean2d, sizeof(float) * 2 * vis},
        {pr.conic_opacity, sizeof(float) * 4 * vis}, {pr.color, sizeof(float) * 3 * vis},
        {pr.depth, sizeof(float) * vis},             {pr.tile_rect, sizeof(uint16_t) * 4 * vis},
        {pr.n_tiles, sizeof(int32_t) * vis},         {b.ranges, sizeof(int32_t) * 2 * tiles},
        {b.tile_keys, sizeof(uint32_t) * m},         {b.vals, sizeof(int32_t) * m},
        {image, sizeof(float) * 3 * npx},            {t_final, sizeof(float) * npx},
        {n_contrib, sizeof(int32_t) * npx},          {image_fused, sizeof(float) * 3 * npx},
        {gr.d_mean2d, sizeof(float) * 2 * vis},      {gr.d_conic, sizeof(float) * 3 * vis},
        {gr.d_opacity, sizeof(float) * vis},         {gr.d_color, sizeof(float) * 3 * vis},
    };
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); i++) {
        void* h = malloc(outs[i].bytes ? outs[i].bytes : 1);
        if (!h) return 1;
        HIP_OK(hipMemcpy(h, outs[i].dev, outs[i].bytes, hipMemcpyDeviceToHost));
        fwrite(h, 1, outs[i].bytes, out);
        free(h);
    }
    fclose(out);
    printf("iteration from C: %d visible, %lld instances\n", vis, (long long)m);
    return 0;
}
