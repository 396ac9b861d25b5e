/*
 * The C ABI's host-side argument checks under AddressSanitizer and UndefinedBehaviorSanitizer, on a host-only
 * build of the library (tests/test_abi_sanitizers.py compiles and runs it; no GPU). Every call below must be
 * rejected on the host with the documented status before anything is launched; the pointers are never
 * dereferenced. Test infrastructure.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gs_raster.h"

static int failures = 0;
static void expect(gs_status got, gs_status want, const char *what) {
    if (got != want) {
        printf("%s: got %d, want %d (%s)\n", what, (int)got, (int)want, gs_last_error());
        ++failures;
    } else if (strlen(gs_last_error()) == 0) {
        printf("%s: no message\n", what);
        ++failures;
    }
}

int main(void) {
    void *f = (void *)0x1000; /* never dereferenced */
    const float *cf = (const float *)f;
    const int32_t *ci = (const int32_t *)f;
    int64_t nout = 0;
    /* workspace queries: degenerate and huge sizes must not overflow */
    size_t w = gs_isect_workspace_bytes(0, 10, 0, 4, 4, 1);
    w += gs_isect_workspace_bytes(1, 1 << 30, (int64_t)1 << 40, 1 << 14, 1 << 14, 1);
    w += gs_sort_workspace_bytes(0, 64) + gs_sort_workspace_bytes((int64_t)1 << 40, 64);
    w += gs_sort_workspace_bytes(-5, 10) + gs_tile_ranges_workspace_bytes();
    w += gs_rasterize_workspace_bytes(0, 1, 1) + gs_rasterize_workspace_bytes(4, 100, 67);
    (void)w;
    /* gs_isect_tiles */
    int32_t *fi = (int32_t *)f;
    expect(gs_isect_tiles(cf, cf, 3, cf, 1, 10, 16, 4, 4, 1, fi, fi, &nout, NULL, NULL, 0, f, 1 << 20, NULL),
           GS_ERR_INVALID_ARG, "isect radii_per_gauss");
    expect(gs_isect_tiles(cf, cf, 1, cf, 1, 10, 0, 4, 4, 1, fi, fi, &nout, NULL, NULL, 0, f, 1 << 20, NULL),
           GS_ERR_INVALID_ARG, "isect tile_size");
    expect(gs_isect_tiles(cf, cf, 1, cf, (int64_t)1 << 16, (int64_t)1 << 16, 16, 4, 4, 1, (int32_t *)f, (int32_t *)f,
                          &nout, NULL, NULL, 0, f, 1 << 20, NULL), GS_ERR_INVALID_ARG, "isect C*N");
    expect(gs_isect_tiles(cf, cf, 1, cf, 1, 10, 16, 4, 4, 1, fi, fi, &nout, NULL, NULL, 0, NULL, 0, NULL),
           GS_ERR_WORKSPACE, "isect workspace");
    /* gs_sort_keys */
    expect(gs_sort_keys((uint64_t *)f, (int32_t *)f, 10, 65, f, 1 << 20, NULL), GS_ERR_INVALID_ARG, "sort end_bit");
    expect(gs_sort_keys((uint64_t *)f, (int32_t *)f, -1, 64, f, 1 << 20, NULL), GS_ERR_INVALID_ARG, "sort n");
    expect(gs_sort_keys((uint64_t *)f, (int32_t *)f, 10, 64, f, 16, NULL), GS_ERR_WORKSPACE, "sort workspace");
    /* gs_tile_ranges */
    expect(gs_tile_ranges((const uint64_t *)f, 10, 0, 4, 4, (int32_t *)f, 0, f, 256, NULL), GS_ERR_INVALID_ARG,
           "ranges C");
    expect(gs_tile_ranges((const uint64_t *)f, 10, 1, 4, 4, (int32_t *)f, 0, NULL, 0, NULL), GS_ERR_WORKSPACE,
           "ranges workspace");
    /* the composite entry points */
    float *ff = (float *)f;
    const float cut = 1 / 255.0f;
    expect(gs_rasterize_fwd(cf, cf, cf, cf, NULL, 1, 4, 5, 64, 64, 16, 4, 4, ci, ci, 10, NULL, cut, 0.99f, 1e-4f, ff,
                            ff, NULL, NULL, NULL, NULL, 0, NULL), GS_ERR_INVALID_ARG, "fwd K");
    expect(gs_rasterize_fwd(cf, cf, cf, cf, NULL, 1, 4, 3, 64, 64, 16, 5, 4, ci, ci, 10, NULL, cut, 0.99f, 1e-4f, ff,
                            ff, NULL, NULL, NULL, NULL, 0, NULL), GS_ERR_INVALID_ARG, "fwd grid");
    expect(gs_rasterize_fwd_traced(cf, cf, cf, cf, NULL, 1, 4, 3, 64, 64, 16, 4, 4, ci, ci, 10, NULL, 1 / 255.0f,
                                   0.99f, 1e-4f, -1, -1, (float *)f, (float *)f, NULL, NULL, (int32_t *)f,
                                   (int32_t *)f, NULL, NULL, 0, NULL), GS_ERR_INVALID_ARG, "traced steps");
    expect(gs_rasterize_fwd_hwexp(cf, cf, cf, cf, NULL, 1, 4, 3, 64, 64, 33, 2, 2, ci, ci, 10, NULL, cut, 0.99f,
                                  1e-4f, ff, ff, NULL, NULL, NULL, NULL), GS_ERR_INVALID_ARG, "hwexp tile_size");
    expect(gs_rasterize_fwd_bins(cf, cf, cf, cf, NULL, 1, 4, 3, 64, 64, 16, 4, 4, ci, ci, 0, cut, 0.99f, 1e-4f, ff,
                                 ff, NULL, NULL, NULL, NULL), GS_ERR_INVALID_ARG, "bins capacity");
    expect(gs_bin_tiles(cf, cf, 1, cf, 1, 4, 16, 1 << 12, 1 << 12, 256, (int32_t *)f, (int32_t *)f, NULL),
           GS_ERR_INVALID_ARG, "bin_tiles slots");
    expect(gs_rasterize_bwd(cf, cf, cf, cf, NULL, 1, 4, 3, 32, 32, 16, 2, 2, ci, ci, 10, NULL, 1 / 255.0f, 0.0f, cf,
                            ci, cf, cf, (float *)f, (float *)f, (float *)f, (float *)f, NULL, NULL, NULL),
           GS_ERR_INVALID_ARG, "bwd clamp");
    expect(gs_project_fwd(cf, cf, cf, cf, 0, 10, 64, 64, 0.3f, 0.01f, 1e10f, 0.0f, 0, (int32_t *)f, (float *)f,
                          (float *)f, (float *)f, NULL, NULL), GS_ERR_INVALID_ARG, "project C");
    if (failures) return 1;
    printf("abi sanitizer run ok\n");
    return 0;
}
