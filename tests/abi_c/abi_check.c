/*
 * Plain C11 client of include/cfz.h, linked against libcfz.so: the header is
 * self-contained C, the library exports what it declares, and the host-side
 * entry points behave as documented without touching a GPU (size queries,
 * status strings, argument validation -- every call below fails validation or
 * reads host memory only).  Prints "OK" on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "cfz.h"

#define EXPECT(cond)                                                     \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond);   \
            return 1;                                                    \
        }                                                                \
    } while (0)

static int run(void)
{
    EXPECT(cfz_abi_version() == CFZ_ABI_VERSION);

    cfz_desc d;
    memset(&d, 0, sizeof d);
    d.rows = 1024;
    d.cols = 3072;
    d.bits = 4;
    d.group = 64;
    d.ef_mode = CFZ_EF_DELTA;
    d.role = CFZ_SENDER;
    d.state_dtype = CFZ_STATE_F32;
    EXPECT(cfz_codes_bytes(&d) == (size_t)1024 * 3072 / 2);
    EXPECT(cfz_scales_bytes(&d) == (size_t)1024 * 3072 / 64 * 4);
    d.bits = 3;
    EXPECT(cfz_codes_bytes(&d) == 0);
    d.bits = 4;

    for (int st = CFZ_OK; st <= CFZ_ERR_HIP; ++st)
        EXPECT(cfz_status_string((cfz_status)st) != NULL);

    /* validation before any device work: fake, never dereferenced addresses */
    cfz_buffers b;
    b.prev_bf16 = (uint16_t *)(uintptr_t)0x10000;
    b.base = NULL;
    b.err = (void *)(uintptr_t)0x20000;
    cfz_state *s = (cfz_state *)(uintptr_t)0xdead;
    EXPECT(cfz_state_create(NULL, &b, NULL, NULL, &s) == CFZ_ERR_NULL);
    EXPECT(s == (cfz_state *)(uintptr_t)0xdead);
    d.group = 48;
    EXPECT(cfz_state_create(&d, &b, NULL, NULL, &s) == CFZ_ERR_UNSUPPORTED);
    d.group = 64;
    b.err = (void *)(uintptr_t)0x20008;
    EXPECT(cfz_state_create(&d, &b, NULL, NULL, &s) == CFZ_ERR_ALIGN);
    EXPECT(strlen(cfz_last_error()) > 0);

    /* resume enqueues nothing: a live handle on host memory only */
    b.err = (void *)(uintptr_t)0x20000;
    EXPECT(cfz_state_resume(&d, &b, 7, &s) == CFZ_OK);
    EXPECT(cfz_state_steps(s) == 7);
    EXPECT(cfz_compress(s, NULL, NULL, NULL, NULL) == CFZ_ERR_NULL);
    EXPECT(cfz_decompress(s, (const uint8_t *)(uintptr_t)0x30000,
                          (const float *)(uintptr_t)0x40000, NULL, NULL) == CFZ_ERR_MODE);
    EXPECT(cfz_state_destroy(s) == CFZ_OK);
    EXPECT(cfz_state_destroy(NULL) == CFZ_OK);
    EXPECT(cfz_state_steps(NULL) == -1);

    EXPECT(cfz_lowrank_workspace_bytes(57, 1024, 3072, 16) > 0);
    EXPECT(cfz_lowrank_workspace_bytes(57, 1024, 3072, 33) == 0);
    EXPECT(cfz_lowrank_ef_workspace_bytes(57, 1024, 3072, 16) >
           cfz_lowrank_workspace_bytes(57, 1024, 3072, 16));
    EXPECT(cfz_lowrank(2, 128, 192, 0, 2, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
           CFZ_ERR_SHAPE);
    EXPECT(cfz_lowrank_ef_warmup(12, NULL, NULL, NULL, NULL, NULL) == CFZ_ERR_SHAPE);
    EXPECT(cfz_lowrank_ef_compress_deferred(2, 128, 192, 8, 2, 2, NULL, NULL, NULL, NULL, NULL,
                                            NULL, NULL, NULL, 0, NULL) == CFZ_ERR_SHAPE);
    EXPECT(cfz_lowrank_ef_flush(2, 128, 192, 8, NULL, NULL, NULL, NULL, NULL) == CFZ_ERR_NULL);
    EXPECT(cfz_stream_copy(NULL, NULL, 0, NULL) == CFZ_OK);
    return 0;
}

int main(void)
{
    if (run() != 0)
        return 1;
    printf("OK\n");
    return 0;
}
