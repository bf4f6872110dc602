/* Driver of the library's host-side argument checks for AddressSanitizer /
 * UndefinedBehaviorSanitizer builds (host code instrumented, no GPU needed):
 * every call below is rejected on the host before any device work, with the
 * status the header documents; the size queries are plain host arithmetic.
 * Prints "ok" and exits 0 when every check holds; a sanitizer finding aborts. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dust.h"

static int fails = 0;
#define EXPECT(call, st, msg)                                                                  \
    do {                                                                                       \
        dust_status s_ = (call);                                                               \
        const char *e_ = dust_last_error();                                                    \
        if ((int)s_ != (st) || (msg && !strstr(e_, msg))) {                                    \
            fprintf(stderr, "line %d: status %d (want %d): %s\n", __LINE__, (int)s_, (st), e_); \
            ++fails;                                                                           \
        }                                                                                      \
    } while (0)

#define FAKE ((void *)(uintptr_t)0x10000)
#define FAKEF ((float *)(uintptr_t)0x10000)
#define FAKEI ((const int32_t *)(uintptr_t)0x10000)

int main(void)
{
    if (dust_abi_version() != 2) ++fails;
    /* head estimator */
    EXPECT(dust_estimate_head(NULL, 0, FAKEF, FAKEI, 4, 8, 2, 3, 0.01f, 1, 0, 0, 0, FAKEF, FAKEF, NULL, NULL, 0, NULL),
           1, "non-NULL");
    EXPECT(dust_estimate_head(FAKE, 7, FAKEF, FAKEI, 4, 8, 2, 3, 0.01f, 1, 0, 0, 0, FAKEF, FAKEF, NULL, NULL, 0, NULL),
           2, "logits_dtype");
    EXPECT(dust_estimate_head(FAKE, 0, FAKEF, FAKEI, 0, 8, 2, 3, 0.01f, 1, 0, 0, 0, FAKEF, FAKEF, NULL, NULL, 0, NULL),
           1, "T must be");
    EXPECT(dust_estimate_head(FAKE, 0, FAKEF, FAKEI, 4, 8, 2, 3, -1.0f, 1, 0, 0, 0, FAKEF, FAKEF, NULL, NULL, 0, NULL),
           1, "sigma");
    EXPECT(dust_estimate_head(FAKE, 0, FAKEF, FAKEI, 4, 8, 2, 3, 0.01f, 1, 0, (uint64_t)1 << 40, 0, FAKEF, FAKEF, NULL,
                              NULL, 0, NULL),
           1, "token counter");
    EXPECT(dust_estimate_head(FAKE, 1, FAKEF, FAKEI, 4, 70000, 2, 3, 0.01f, 1, 0, 0, 0, FAKEF, FAKEF, NULL, NULL, 0,
                              NULL),
           2, "65536");
    EXPECT(dust_estimate_head(FAKE, 0, FAKEF, FAKEI, 4, 8, 2, 3, 0.01f, 1, 0, 0, 0, FAKEF, NULL, NULL, NULL, 0, NULL),
           3, "workspace");
    EXPECT(dust_estimate_head_noalloc(FAKE, 1, FAKEF, FAKEI, 4096, 8192, 512, 4, 0.01f, 1, 1, 0, 0, FAKEF, NULL, NULL,
                                      NULL),
           2, "static scratch");
    EXPECT(dust_estimate_head_subset(FAKE, 0, FAKEF, FAKEI, 4, 1000, 8, 3, 6, 0.01f, 1, 0, 0, 0, FAKEF, FAKEF, NULL,
                                     NULL, 0, NULL),
           1, "multiple of 4");
    /* interior linear: W_head offsets past 2^31 */
    EXPECT(dust_estimate_linear(FAKEF, FAKEF, FAKEF, FAKE, FAKE, FAKEI, 4, 512, 2048, ((int64_t)1 << 31) / 512, 2, 0.01f, 1e-5f,
                                1, 0, 0, 0, FAKEF, NULL, NULL, NULL, 0, NULL),
           2, "2^31");
    /* noise and outer product */
    EXPECT(dust_noise(1, 0, 0, 1, 0, 1, 4, NULL, NULL, NULL), 1, NULL);
    EXPECT(dust_noise(1, 0, 0, 1, (uint64_t)1 << 33, 1, 4, NULL, FAKEF, NULL), 1, NULL);
    EXPECT(dust_debug_noise(1, 0, 0, (uint64_t)1 << 32, 4, NULL, FAKEF, NULL), 1, "2^32");
    EXPECT(dust_outer_product(NULL, FAKEF, 4, 4, 4, FAKEF, NULL, 0, NULL), 1, NULL);
    EXPECT(dust_outer_product(FAKEF, FAKEF, 4096, 2048, 512, FAKEF, NULL, 0, NULL), 3, NULL);
    /* attention */
    EXPECT(dust_estimate_attn_v(FAKEF, FAKEF, FAKEF, FAKEF, 128, 64, 96, 2, 3, 0.01f, 1, 2, 0, 0, FAKEF, NULL, NULL,
                                FAKE, (size_t)1 << 30, NULL),
           2, NULL);
    EXPECT(dust_estimate_attn(3, FAKEF, FAKEF, FAKEF, FAKEF, FAKEF, 128, 64, 128, 2, 3, 0.01f, 1, 2, 0, 0, FAKEF, NULL,
                              NULL, FAKE, (size_t)1 << 30, NULL),
           1, NULL);
    /* size queries */
    if (dust_head_workspace_bytes(4096, 8192, 512, 256) == 0) ++fails;
    if (dust_linear_workspace_bytes(4096, 512, 2048, 8192, 64) == 0) ++fails;
    if (dust_outer_workspace_bytes(4096, 2048, 512) == 0) ++fails;
    if (dust_head_noalloc_max_bytes() != ((size_t)64 << 20)) ++fails;
    if (fails) return 1;
    printf("ok\n");
    return 0;
}
