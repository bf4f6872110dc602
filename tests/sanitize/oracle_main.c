/* Driver of the oracle's C functions for AddressSanitizer / UndefinedBehavior-
 * Sanitizer builds (CPU only): Philox4x32-10 against the published known-answer
 * vectors (argv[1], the golden file), then the noise and head estimators on
 * small and ragged shapes, empty sizes included, with internal consistency
 * checks.  Prints "ok" and exits 0 when every check holds; a sanitizer finding
 * aborts the program. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
void orc_noise_raw(uint64_t seed, uint32_t layer, uint32_t draw, uint32_t token, int64_t n, uint32_t *raw);
void orc_noise(uint64_t seed, uint32_t layer, uint32_t draw, uint32_t token, int64_t n, double *a);
void orc_noise_block(uint64_t seed, uint32_t layer, uint32_t draw_offset, int64_t K, uint32_t token_offset,
                     int64_t T, int64_t n, double *out);
void orc_head_estimate(const double *logits, const int32_t *labels, int64_t T, int64_t V, int64_t K, double sigma,
                       uint64_t seed, uint32_t layer, uint32_t token_offset, uint32_t draw_offset, double *ghat,
                       double *rewards, double *ce0);
void orc_head_estimate_subset(const double *logits, const int32_t *labels, int64_t T, int64_t V, int64_t K,
                              int64_t m, double sigma, uint64_t seed, uint32_t layer, uint32_t token_offset,
                              uint32_t draw_offset, double *ghat, double *rewards, double *ce0);

static int fails = 0;
#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } \
    } while (0)

static void kat(const char *path)
{
    FILE *f = fopen(path, "r");
    CHECK(f != NULL);
    if (!f) return;
    char line[512];
    int n = 0;
    while (fgets(line, sizeof line, f)) {
        if (line[0] == '#' || line[0] == '\n') continue;
        unsigned v[10];
        if (sscanf(line, "%x %x %x %x %x %x %x %x %x %x", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5], &v[6], &v[7],
                   &v[8], &v[9]) != 10)
            continue;
        uint32_t ctr[4] = {v[0], v[1], v[2], v[3]}, key[2] = {v[4], v[5]}, out[4];
        orc_philox4x32_10(ctr, key, out);
        for (int j = 0; j < 4; ++j) CHECK(out[j] == v[6 + j]);
        ++n;
    }
    fclose(f);
    CHECK(n >= 3);
}

static void noise(void)
{
    const int64_t K = 3, T = 5, n = 7;   /* ragged: n not a multiple of 4 */
    double *blk = malloc(sizeof(double) * K * T * n), a[7];
    uint32_t raw[8];
    orc_noise_block(11, 2, 4, K, 9, T, n, blk);
    for (int64_t i = 0; i < K; ++i)
        for (int64_t t = 0; t < T; ++t) {
            orc_noise(11, 2, 4 + (uint32_t)i, 9 + (uint32_t)t, n, a);
            CHECK(memcmp(a, blk + (i * T + t) * n, sizeof a) == 0);
            for (int c = 0; c < n; ++c) CHECK(isfinite(a[c]) && fabs(a[c]) <= 5.7683);
        }
    orc_noise_raw(11, 2, 4, 9, n, raw);
    orc_noise_block(11, 2, 0, 0, 0, T, n, blk);   /* empty */
    orc_noise_block(11, 2, 0, K, 0, 0, n, blk);
    free(blk);
}

static void head(void)
{
    const int64_t T = 3, V = 5, K = 4;   /* V not a multiple of 4 */
    double z[15], g[15], gs[15], r[12], rs[12], c0[3], c1[3];
    int32_t y[3] = {0, 4, 2};
    for (int i = 0; i < 15; ++i) z[i] = sin(1.7 * i) * 2.0;
    orc_head_estimate(z, y, T, V, K, 1e-2, 5, 1, 3, 7, g, r, c0);
    for (int i = 0; i < 15; ++i) CHECK(isfinite(g[i]));
    for (int i = 0; i < 3; ++i) CHECK(c0[i] > 0.0);
    /* a window covering the vocabulary is the full estimator */
    orc_head_estimate_subset(z, y, T, V, K, 8, 1e-2, 5, 1, 3, 7, gs, rs, c1);
    CHECK(memcmp(g, gs, sizeof g) == 0 && memcmp(r, rs, sizeof r) == 0 && memcmp(c0, c1, sizeof c0) == 0);
    /* a narrow window: finite, and the rewards of a one-quad window still well defined */
    orc_head_estimate_subset(z, y, T, V, K, 4, 1e-2, 5, 1, 3, 7, gs, rs, NULL);
    for (int i = 0; i < 15; ++i) CHECK(isfinite(gs[i]));
    /* empty sizes and optional outputs */
    orc_head_estimate(z, y, 0, V, K, 1e-2, 5, 1, 0, 0, g, NULL, NULL);
    orc_head_estimate(z, y, T, V, 0, 1e-2, 5, 1, 0, 0, g, NULL, NULL);
    orc_head_estimate(z, y, 1, 1, 2, 1e-2, 5, 1, 0, 0, g, r, NULL);   /* one-entry vocabulary */
    CHECK(g[0] == 0.0 || fabs(g[0]) < 1e-12);
}

int main(int argc, char **argv)
{
    if (argc < 2) { fprintf(stderr, "usage: %s KAT_FILE\n", argv[0]); return 2; }
    kat(argv[1]);
    noise();
    head();
    if (fails) return 1;
    printf("ok\n");
    return 0;
}
