/*
 * Runs every oracle routine on small seeded scenes, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py compiles and runs it). It checks no values: the
 * other CPU tests pin those; this run only has to finish without a sanitizer report. Test infrastructure.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_bits_for(int64_t count);
int64_t orc_isect_count(const float *, const float *, int, int64_t, int64_t, int, int, int, int32_t *, int64_t *);
int orc_isect_emit(const float *, const float *, int, const float *, int64_t, int64_t, int, int, int, uint64_t *,
                   int32_t *);
int orc_sort_pairs(uint64_t *, int32_t *, int64_t);
int orc_tile_offsets(const uint64_t *, int64_t, int64_t, int, int, int32_t *);
float orc_exp_neg(float);
int64_t orc_rasterize_fwd_traced(const float *, const float *, const float *, const float *, const float *, int64_t,
                                 int, int, int, int, int, int, const int32_t *, const int32_t *, int64_t,
                                 const int32_t *, float, float, float, const int64_t *, int64_t, int64_t, int64_t,
                                 float *, float *, float *, int32_t *, int32_t *, int32_t *);
int64_t orc_rasterize_tile(const float *, const float *, const float *, const float *, const float *, int, int, int,
                           int, int, int, int64_t, const int32_t *, int64_t, float, float, float, float *, float *,
                           int64_t *);
int orc_rasterize_bwd(const float *, const float *, const float *, const float *, const float *, int64_t, int64_t,
                      int, int, int, int, int, int, const int32_t *, const int32_t *, int64_t, const int32_t *, float,
                      float, const float *, const int32_t *, const float *, const float *, double *, double *,
                      double *, double *, double *, double *, double *, double *, double *, double *, double *,
                      double *, double *, double *, double *, double *);
void orc_project(const float *, const float *, const float *, const float *, int64_t, int64_t, int, int, float,
                 float, float, float, int, int32_t *, float *, float *, float *, float *);
int64_t orc_tile_lists(const float *, const float *, int, const float *, int64_t, int64_t, int, int, int,
                       const int64_t *, int64_t, int64_t *, int32_t *);
int64_t orc_bin_tiles(const float *, const float *, int, const float *, int64_t, int64_t, int, int, int, int64_t,
                      int32_t *, int32_t *);
int64_t orc_rasterize_bins(const float *, const float *, const float *, const float *, const float *, int64_t, int,
                           int, int, int, int, int, const int32_t *, int64_t, float, float, float, float *, float *,
                           float *, int32_t *);

static uint64_t state = 0x853c49e6748fea9bull;
static float uniform(float lo, float hi) {  /* a 64-bit LCG's top 24 bits */
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (float)(state >> 40) / 16777216.0f;
}
#define NEW(T, n) ((T *)calloc((size_t)((n) > 0 ? (n) : 1), sizeof(T)))

static int run_scene(int64_t C, int64_t N, int W, int H, int ts, int K, int rpg) {
    const int tw = (W + ts - 1) / ts, th = (H + ts - 1) / ts;
    const int64_t M = C * N, T = C * tw * th, P = C * (int64_t)W * H;
    float *means = NEW(float, 2 * M), *radii = NEW(float, rpg * M), *depths = NEW(float, M);
    float *conics = NEW(float, 3 * M), *colors = NEW(float, K * M), *ops = NEW(float, M), *bg = NEW(float, C * K);
    for (int64_t i = 0; i < M; ++i) {
        means[2 * i] = uniform(-8.0f, W + 8.0f);
        means[2 * i + 1] = uniform(-8.0f, H + 8.0f);
        for (int r = 0; r < rpg; ++r) radii[rpg * i + r] = i % 9 == 0 ? 0.0f : uniform(0.2f, 14.0f);
        depths[i] = i % 5 == 0 && i > 0 ? depths[i - 1] : uniform(0.5f, 10.0f);
        const float s1 = uniform(0.5f, 5.0f), s2 = uniform(0.5f, 5.0f), rho = uniform(-0.6f, 0.6f);
        const float det = s1 * s1 * s2 * s2 * (1.0f - rho * rho);
        conics[3 * i] = s2 * s2 / det;
        conics[3 * i + 1] = -rho * s1 * s2 / det;
        conics[3 * i + 2] = s1 * s1 / det;
        for (int k = 0; k < K; ++k) colors[K * i + k] = uniform(0.0f, 1.0f);
        ops[i] = i % 7 == 0 ? 0.999f : uniform(0.0f, 1.0f);
    }
    for (int64_t i = 0; i < C * K; ++i) bg[i] = uniform(0.0f, 1.0f);
    int32_t *tpg = NEW(int32_t, M);
    int64_t *goff = NEW(int64_t, M);
    const int64_t n = orc_isect_count(means, radii, rpg, C, N, ts, tw, th, tpg, goff);
    uint64_t *keys = NEW(uint64_t, n);
    int32_t *ids = NEW(int32_t, n), *off = NEW(int32_t, T), *masks = NEW(int32_t, T);
    orc_isect_emit(means, radii, rpg, depths, C, N, ts, tw, th, keys, ids);
    if (orc_sort_pairs(keys, ids, n) != 0) return 1;
    if (orc_tile_offsets(keys, n, C, tw, th, off) != 0) return 1;
    for (int64_t t = 0; t < T; ++t) masks[t] = t % 3 != 0;
    float *col = NEW(float, P * K), *alp = NEW(float, P), *Tr = NEW(float, P);
    int32_t *last = NEW(int32_t, P), *cnt = NEW(int32_t, P);
    const int S = 5;
    int32_t *trace = NEW(int32_t, P * S);
    if (orc_rasterize_fwd_traced(means, conics, colors, ops, bg, C, K, W, H, ts, tw, th, off, ids, n, NULL,
                                 1.0f / 255.0f, 0.99f, 1e-4f, NULL, 0, -1, -1, col, alp, Tr, last, NULL, NULL) < 0)
        return 1;
    if (orc_rasterize_fwd_traced(means, conics, colors, ops, bg, C, K, W, H, ts, tw, th, off, ids, n, masks,
                                 1.0f / 255.0f, 0.99f, 1e-4f, NULL, 0, 3, S, col, alp, Tr, last, trace, cnt) < 0)
        return 1;
    /* the backward on the capped, masked forward's outputs, every optional output on */
    float *gc = NEW(float, P * K), *ga = NEW(float, P);
    for (int64_t i = 0; i < P * K; ++i) gc[i] = uniform(-1.0f, 1.0f);
    for (int64_t i = 0; i < P; ++i) ga[i] = uniform(-1.0f, 1.0f);
    double *g = NEW(double, M * ((2 + 3 + K + 1) * 3 + 2) + C * K * 3);
    double *gm = g, *gq = gm + 2 * M, *gcol = gq + 3 * M, *go = gcol + K * M, *gabs = go + M, *am = gabs + 2 * M;
    double *aq = am + 2 * M, *acol = aq + 3 * M, *ao = acol + K * M, *em = ao + M, *eq = em + 2 * M;
    double *ecol = eq + 3 * M, *eo = ecol + K * M, *gbg = eo + M, *abg = gbg + C * K, *ebg = abg + C * K;
    if (orc_rasterize_bwd(means, conics, colors, ops, bg, C, N, K, W, H, ts, tw, th, off, ids, n, masks,
                          1.0f / 255.0f, 0.99f, alp, last, gc, ga, gm, gq, gcol, go, gbg, gabs, am, aq, acol, ao,
                          abg, em, eq, ecol, eo, ebg) != 0)
        return 1;
    /* one tile over an explicit list, the brute-force lists and the bins */
    float *tc = NEW(float, ts * ts * K), *tT = NEW(float, ts * ts);
    int64_t *tl = NEW(int64_t, ts * ts), tiles[2] = {0, T - 1}, counts[2];
    const int64_t total = orc_tile_lists(means, radii, rpg, depths, C, N, ts, tw, th, tiles, 2, counts, NULL);
    int32_t *lists = NEW(int32_t, total);
    orc_tile_lists(means, radii, rpg, depths, C, N, ts, tw, th, tiles, 2, counts, lists);
    orc_rasterize_tile(means, conics, colors, ops, bg, K, W, H, ts, tw, th, T - 1, lists + counts[0], counts[1],
                       1.0f / 255.0f, 0.99f, 1e-4f, tc, tT, tl);
    const int64_t cap = 6;
    int32_t *bins = NEW(int32_t, T * cap), *bcnt = NEW(int32_t, T);
    if (orc_bin_tiles(means, radii, rpg, depths, C, N, ts, tw, th, cap, bins, bcnt) < 0) return 1;
    if (orc_rasterize_bins(means, conics, colors, ops, bg, C, K, W, H, ts, tw, th, bins, cap, 1.0f / 255.0f, 0.99f,
                           1e-4f, col, alp, Tr, last) < 0)
        return 1;
    free(means); free(radii); free(depths); free(conics); free(colors); free(ops); free(bg); free(tpg); free(goff);
    free(keys); free(ids); free(off); free(masks); free(col); free(alp); free(Tr); free(last); free(cnt);
    free(trace); free(gc); free(ga); free(g); free(tc); free(tT); free(tl); free(lists); free(bins); free(bcnt);
    return 0;
}

static int run_projection(void) {
    const int64_t C = 2, N = 300;
    float *means = NEW(float, 3 * N), *cov = NEW(float, 9 * N), view[32] = {0}, Ks[18] = {0};
    for (int64_t i = 0; i < N; ++i) {
        for (int d = 0; d < 3; ++d) means[3 * i + d] = uniform(-3.0f, 3.0f) + (d == 2 ? 4.0f : 0.0f);
        const float s = uniform(0.0f, 0.3f);
        cov[9 * i] = cov[9 * i + 4] = cov[9 * i + 8] = i % 11 == 0 ? 0.0f : s * s;
        cov[9 * i + 1] = cov[9 * i + 3] = i % 13 == 0 ? 1.0f : 0.0f; /* some indefinite */
    }
    for (int c = 0; c < 2; ++c) {
        view[16 * c] = view[16 * c + 5] = view[16 * c + 10] = view[16 * c + 15] = 1.0f;
        view[16 * c + 11] = c ? 1.0f : 0.0f;
        Ks[9 * c] = 500.0f;
        Ks[9 * c + 4] = 450.0f;
        Ks[9 * c + 2] = 160.0f;
        Ks[9 * c + 5] = 120.0f;
        Ks[9 * c + 8] = 1.0f;
    }
    int32_t *r = NEW(int32_t, 2 * C * N);
    float *m2 = NEW(float, 2 * C * N), *dep = NEW(float, C * N), *con = NEW(float, 3 * C * N);
    float *comp = NEW(float, C * N);
    for (int ortho = 0; ortho < 2; ++ortho)
        orc_project(means, cov, view, Ks, C, N, 320, 240, 0.3f, 0.5f, 100.0f, 1.0f, ortho, r, m2, dep, con, comp);
    free(means); free(cov); free(r); free(m2); free(dep); free(con); free(comp);
    return 0;
}

int main(void) {
    float probe[] = {-1.0f, 0.0f, 1e-30f, 0.5f, 17.0f, 79.9f, 80.0f, 80.1f, 1e30f, INFINITY, NAN};
    volatile float sink = 0.0f;
    for (unsigned i = 0; i < sizeof probe / sizeof probe[0]; ++i) sink += orc_exp_neg(probe[i]);
    for (int64_t c = 0; c < 70; ++c) sink += (float)orc_bits_for(c);
    if (run_scene(2, 200, 70, 45, 16, 3, 1)) return 1;
    if (run_scene(1, 150, 37, 29, 8, 1, 2)) return 1;
    if (run_scene(1, 60, 40, 33, 32, 4, 1)) return 1;
    if (run_scene(1, 0, 20, 20, 16, 3, 1)) return 1; /* no splats */
    if (run_projection()) return 1;
    printf("oracle sanitizer run ok\n");
    return 0;
}
