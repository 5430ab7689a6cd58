/*
 * Host-side checks of libssd under AddressSanitizer and UndefinedBehavior-
 * Sanitizer (test infrastructure): the library's host code is built with
 * the sanitizers (no device code) and this driver calls every entry point on
 * the paths that need no GPU: the plan and workspace sizes over a sweep of
 * shapes (huge ones included, where the size arithmetic could overflow), the
 * status texts, and argument checks that must fail before any pointer is
 * read. Pointers passed here are never dereferenced: each call is expected to
 * return an error first. Exit status 0 when every expectation holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssd.h"

static int failures = 0;
#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
                    __LINE__, #cond);                                         \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

int main(void) {
    void *fake = (void *)(uintptr_t)0x100000;      /* aligned, never read */
    void *fake_odd = (void *)(uintptr_t)0x100004;  /* a dt that is not 16-byte aligned */
    float *ffake = (float *)fake;

    for (int s = -9; s <= 1; ++s) {
        const char *t = ssd_strerror(s);
        EXPECT(t != NULL && strlen(t) > 0);
    }

    /* plans and workspace sizes over a sweep of shapes */
    const int bts[] = {1, 2, 8, 64, 4096};
    const int lens[] = {1, 37, 64, 2048, 65536, 1 << 22};
    const int heads[] = {1, 4, 8, 80, 1024};
    const int states[] = {0, 15, 16, 48, 64, 96, 128, 192, 256, 272};
    const int chunks[] = {0, 32, 64, 128, 256, 512};
    int checked = 0;
    for (size_t a = 0; a < sizeof bts / sizeof *bts; ++a)
        for (size_t b = 0; b < sizeof lens / sizeof *lens; ++b)
            for (size_t c = 0; c < sizeof heads / sizeof *heads; ++c)
                for (size_t d = 0; d < sizeof states / sizeof *states; ++d)
                    for (size_t e = 0; e < sizeof chunks / sizeof *chunks; ++e)
                        for (int dtype = 0; dtype <= 2; ++dtype)
                            for (int al = 0; al < 2; ++al) {
                                const int Bt = bts[a], L = lens[b], H = heads[c], N = states[d],
                                          Q = chunks[e];
                                const int G = H % 4 == 0 ? 4 : 1;
                                ssd_plan p;
                                memset(&p, 0xAB, sizeof p);
                                const int rc = ssd_forward_plan_info(Bt, L, H, 64, G, N, Q, dtype,
                                                                     al ? fake : fake_odd, &p);
                                const size_t ws = ssd_forward_workspace_size(Bt, L, H, 64, G, N, Q, dtype);
                                const int plan = ssd_forward_plan(Bt, L, H, 64, G, N, Q, dtype,
                                                                  al ? fake : fake_odd);
                                if (rc == SSD_OK) {
                                    EXPECT(p.path == SSD_PATH_STAGES || p.path == SSD_PATH_SINGLE_PASS);
                                    EXPECT(p.kernel_dstate >= N && p.kernel_dstate <= 256);
                                    EXPECT(plan == (p.path == SSD_PATH_SINGLE_PASS ? p.segments : 0));
                                    if (al) EXPECT(ws == p.workspace_bytes);
                                } else {
                                    EXPECT(rc < 0 && p.workspace_bytes == 0 && ws == 0 && plan == rc);
                                }
                                (void)ssd_backward_workspace_size(Bt, L, H, 64, G, N, dtype);
                                (void)ssd_forward_varlen_workspace_size(L, H, 64, G, N, Q, dtype);
                                (void)ssd_chunk_cb_size(Bt, L, G, Q, dtype);
                                ++checked;
                            }
    EXPECT(checked > 0);
    EXPECT(ssd_forward_plan_info(1, 10, 8, 64, 1, 64, 64, 1, fake, NULL) == SSD_ERR_NULL);

    /* argument checks, each before any pointer is used */
    EXPECT(ssd_forward(NULL, fake, ffake, fake, fake, NULL, 1, 128, 4, 64, 1, 64, 64, 1, NULL,
                       fake, NULL, fake, (size_t)1 << 40, NULL) == SSD_ERR_NULL);
    EXPECT(ssd_forward(fake, fake, ffake, fake, fake, NULL, 0, 128, 4, 64, 1, 64, 64, 1, NULL,
                       fake, NULL, fake, (size_t)1 << 40, NULL) == SSD_ERR_SHAPE);
    EXPECT(ssd_forward(fake, fake, ffake, fake, fake, NULL, 1, 128, 4, 64, 3, 64, 64, 1, NULL,
                       fake, NULL, fake, (size_t)1 << 40, NULL) == SSD_ERR_SHAPE);
    EXPECT(ssd_forward(fake, fake, ffake, fake, fake, NULL, 1, 128, 4, 64, 1, 40, 64, 1, NULL,
                       fake, NULL, fake, (size_t)1 << 40, NULL) == SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_forward(fake, fake, ffake, fake, fake, NULL, 1, 128, 4, 64, 1, 64, 64, 1, NULL,
                       fake, NULL, fake, 1, NULL) == SSD_ERR_WORKSPACE);
    ssd_options bad = {NULL, 0, 1, 2.0f, 1.0f, SSD_DISC_EULER};  /* dt_min > dt_max */
    EXPECT(ssd_forward_ex(fake, fake, ffake, fake, fake, NULL, 1, 128, 4, 64, 1, 64, 64, 1, NULL,
                          fake, NULL, fake, (size_t)1 << 40, &bad, NULL, NULL) == SSD_ERR_OPTION);
    ssd_options bad_disc = {NULL, 0, 0, 0.0f, 0.0f, 7};
    EXPECT(ssd_forward_ex(fake, fake, ffake, fake, fake, NULL, 1, 128, 4, 64, 1, 64, 64, 1, NULL,
                          fake, NULL, fake, (size_t)1 << 40, &bad_disc, NULL, NULL) == SSD_ERR_OPTION);
    EXPECT(ssd_forward_static(fake, fake, ffake, fake, fake, NULL, 1, 128, 4, 64, 1, 40, 64, 1,
                              NULL, fake, NULL, NULL, NULL) == SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_forward_static(fake, fake, ffake, fake, fake, NULL, 1, 128, 4, 64, 1, 64, 64, 1,
                              NULL, fake, NULL, &bad, NULL) == SSD_ERR_OPTION);
    EXPECT(ssd_step(NULL, fake, fake, ffake, fake, fake, NULL, 1, 4, 64, 1, 64, 1, fake, NULL) ==
           SSD_ERR_NULL);
    EXPECT(ssd_step(ffake, fake, fake, ffake, fake, fake, NULL, 1, 4, 64, 3, 64, 1, fake, NULL) ==
           SSD_ERR_SHAPE);
    EXPECT(ssd_forward_varlen(fake, fake, ffake, fake, fake, NULL, (const int *)fake, 0, 128, 4, 64,
                              1, 64, 64, 1, fake, NULL, fake, (size_t)1 << 40, NULL, NULL) ==
           SSD_ERR_SHAPE);
    EXPECT(ssd_forward_varlen(fake, fake, ffake, fake, fake, NULL, NULL, 2, 128, 4, 64, 1, 64, 64, 1,
                              fake, NULL, fake, (size_t)1 << 40, NULL, NULL) == SSD_ERR_NULL);
    EXPECT(ssd_backward(fake, fake, ffake, fake, fake, NULL, NULL, NULL, NULL, 1, 128, 4, 64, 1, 64, 1,
                        fake, fake, ffake, fake, fake, NULL, NULL, NULL, fake, (size_t)1 << 40, NULL,
                        NULL) == SSD_ERR_NULL);
    EXPECT(ssd_backward(fake, fake, ffake, fake, fake, NULL, NULL, fake, NULL, 1, 128, 4, 64, 1, 64, 1,
                        fake, fake, ffake, fake, fake, NULL, NULL, NULL, fake, 1, NULL, NULL) ==
           SSD_ERR_WORKSPACE);
    EXPECT(ssd_chunk_cumsum(NULL, ffake, 1, 128, 4, 64, 1, ffake, ffake, NULL, NULL) == SSD_ERR_NULL);

    if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
    else printf("abi driver: %d shape combinations, every check passed\n", checked);
    return failures ? 1 : 0;
}
