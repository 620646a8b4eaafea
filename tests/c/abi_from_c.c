/* A plain C99 caller of the library: the public header compiles as C, the library links and
 * loads without any Python or PyTorch, and calls that validation refuses return their status
 * without touching a device (so this runs on a machine without a GPU). */
#include <stdio.h>
#include <string.h>

#include "gsmi.h"

static int failures = 0;

static void expect(int cond, const char* what) {
    if (!cond) {
        printf("FAIL: %s\n", what);
        failures++;
    }
}

int main(void) {
    const char* v = gs_version();
    expect(v != NULL && strlen(v) > 0, "gs_version");
    expect(strlen(gs_status_string(GS_ERR_INVALID_ARGUMENT)) > 0, "gs_status_string");

    /* workspace queries are pure host arithmetic */
    expect(gs_project_workspace_size(1000, 4) > 0, "gs_project_workspace_size");
    expect(gs_raster_workspace_size(-1) == 0, "gs_raster_workspace_size(-1)");
    int32_t k = 0;
    expect(gs_fused_max_cap(&k) == GS_OK && k > 0, "gs_fused_max_cap");

    /* refused before anything is enqueued */
    gs_render_params p;
    memset(&p, 0, sizeof(p));
    p.znear = 0.2f;
    p.eps2d = 0.3f;
    p.alpha_min = 1.0f / 255.0f;
    p.alpha_max = 0.99f;
    p.t_min = 1e-4f;
    p.sh_degree = 0;
    gs_camera cam;
    memset(&cam, 0, sizeof(cam));
    cam.width = 64;
    cam.height = 48;
    gs_status st = gs_project(NULL, &cam, 1, &p, NULL, NULL, 0, NULL);
    expect(st == GS_ERR_INVALID_ARGUMENT, "gs_project(NULL gaussians)");
    expect(strstr(gs_last_error(), "null") != NULL, "gs_last_error names the null argument");
    p.znear = -1.0f;
    gs_gaussians g;
    memset(&g, 0, sizeof(g));
    st = gs_project(&g, &cam, 1, &p, NULL, NULL, 0, NULL);
    expect(st == GS_ERR_INVALID_ARGUMENT, "gs_project(znear < 0)");
    st = gs_adam_step_seen(10, NULL, 1, NULL, 1, NULL, NULL, NULL);
    expect(st == GS_ERR_INVALID_ARGUMENT, "gs_adam_step_seen(NULL groups)");

    printf("%s: %d failure(s)\n", v ? v : "?", failures);
    return failures == 0 ? 0 : 1;
}
