/* Plain-C99 consumer of include/ttsbb.h.  Built with -std=c99 -Wall -Werror -pedantic
 * and run on the CPU: every entry point is called through its argument-check path, which
 * must return before touching a device. */
#include <stdio.h>
#include <string.h>

#include "ttsbb.h"

static int fails = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++fails;                                                   \
        }                                                              \
    } while (0)

int main(void) {
    ttsbb_config cfg;
    ttsbb_ctx *ctx = NULL;
    int32_t sched[4];
    float dummy = 0.f;

    ttsbb_default_config(&cfg);
    EXPECT(cfg.n_layers == 28 && cfg.hidden == 1024 && cfg.n_heads == 16 && cfg.n_kv_heads == 8);
    EXPECT(cfg.head_dim == 128 && cfg.ffn == 3072 && cfg.kv_page == 16 && cfg.dtype == TTSBB_BF16);
    ttsbb_default_config(NULL);

    EXPECT(ttsbb_create(NULL, NULL, NULL, NULL, &ctx) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_create(&cfg, NULL, NULL, NULL, NULL) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_create(&cfg, NULL, NULL, NULL, &ctx) == TTSBB_INVALID_ARG); /* 28 layers, none given */
    cfg.n_layers = 0;
    cfg.head_dim = 64;
    EXPECT(ttsbb_create(&cfg, NULL, NULL, NULL, &ctx) == TTSBB_UNSUPPORTED);
    cfg.head_dim = 128;
    cfg.n_kv_heads = 5;
    EXPECT(ttsbb_create(&cfg, NULL, NULL, NULL, &ctx) == TTSBB_UNSUPPORTED);
    cfg.n_kv_heads = 8;
    cfg.max_rows = 0;
    EXPECT(ttsbb_create(&cfg, NULL, NULL, NULL, &ctx) == TTSBB_INVALID_ARG);
    EXPECT(ctx == NULL);

    ttsbb_destroy(NULL);
    EXPECT(ttsbb_sync(NULL) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_codebook_embed(NULL, 1, 1, NULL, NULL, 1, NULL, NULL, NULL, 0, &dummy) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_decode_step(NULL, 1, &dummy, NULL, NULL, 1, NULL, 1, NULL, 0, 0, NULL, NULL) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_decode_step_noalloc(NULL, 1, &dummy, NULL, NULL, 1, NULL, 1, NULL, 0, 0, NULL, NULL) ==
           TTSBB_INVALID_ARG);
    EXPECT(ttsbb_maskgit_pass(NULL, 0, NULL, NULL, 0, 1, 1, 2, 1, NULL, NULL, NULL, 0, 5.0f, NULL, NULL,
                              NULL) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_maskgit_pass_cfg(NULL, 0, NULL, NULL, 0, 4, 2, 1, 2, 1, NULL, NULL, NULL, 0, 5.0f, 2.0f, NULL,
                                  NULL, NULL) == TTSBB_INVALID_ARG);
    {
        ttsbb_maskgit_step_args sa;
        memset(&sa, 0, sizeof sa);
        EXPECT(ttsbb_maskgit_step(NULL, &sa) == TTSBB_INVALID_ARG);
    }
    EXPECT(ttsbb_rvq_decode(NULL, 1, 8, 1024, 64, 1024, NULL, NULL, NULL, NULL, &dummy) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_philox_words(NULL, 42u, 0u, 1u, 0u, 1, NULL) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_prefill(NULL, 1, &dummy, NULL, NULL, 1, NULL, 1, NULL, 0, 0, NULL, NULL) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_set_tap_layer(NULL, 0) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_read_tap(NULL, 0, &dummy, 1, NULL, NULL) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_profile_start(NULL, 1u, 16) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_profile_stop(NULL, NULL, NULL) == TTSBB_INVALID_ARG);

    EXPECT(ttsbb_unmask_schedule(10, 2, sched) == TTSBB_OK && sched[0] == 3 && sched[1] == 7);
    EXPECT(ttsbb_unmask_schedule(10, 0, sched) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_unmask_schedule(-1, 2, sched) == TTSBB_INVALID_ARG);
    EXPECT(ttsbb_unmask_schedule(10, 2, NULL) == TTSBB_INVALID_ARG);

    EXPECT(strcmp(ttsbb_status_str(TTSBB_OK), "ok") == 0);
    EXPECT(ttsbb_status_str(TTSBB_DEVICE_ERROR) != NULL);
    EXPECT(ttsbb_status_str((ttsbb_status)42) != NULL);

    if (fails) return 1;
    printf("abi ok\n");
    return 0;
}
