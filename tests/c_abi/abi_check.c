/* Compiled as C99 against include/gdr.h and linked with libgdr.so by
 * tests/test_abi_cpu.py: the boundary is plain C (no C++ or torch types), and
 * the calls that need no GPU behave as the header states. Prints "ok" and
 * exits 0, or names the first failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "gdr.h"

#define CHECK(cond)                                         \
    do {                                                    \
        if (!(cond)) {                                      \
            printf("failed: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                       \
        }                                                   \
    } while (0)

int main(void) {
    gdr_desc d;
    size_t bytes = 0;
    char fake_storage[64];
    void *p = fake_storage; /* never dereferenced: every call below is rejected or empty */

    CHECK(gdr_version() == 1);
    CHECK(gdr_state_bytes(1, 48, 128, 128) == (size_t)3145728);
    CHECK(gdr_state_bytes(0, 48, 128, 128) == 0);

    memset(&d, 0, sizeof d);
    d.B = 1; d.T = 4096; d.H_qk = 16; d.H_v = 48; d.d_k = 128; d.d_v = 128;
    d.io_dtype = GDR_BF16; d.decay = GDR_DECAY_SCALAR; d.chunk = 64; d.scale = 1.0f;
    CHECK(gdr_chunk_workspace_bytes(&d, &bytes) == GDR_OK && bytes > 0);

    d.H_v = 47; /* not a multiple of H_qk */
    CHECK(gdr_chunk_workspace_bytes(&d, &bytes) == GDR_E_INVAL);
    CHECK(strlen(gdr_last_error()) > 0);
    d.H_v = 48;

    d.d_k = d.d_v = 96; /* unsupported head dimension */
    CHECK(gdr_chunk_fwd(&d, p, p, p, (const float *)p, (const float *)p, NULL, NULL, NULL, p, (float *)p, p,
                        (size_t)1 << 40, NULL) == GDR_E_UNSUPPORTED);
    d.d_k = d.d_v = 128;

    /* Gates: beta together with b and w is rejected before any HIP call. */
    CHECK(gdr_recurrent_fwd(&d, p, p, p, (const float *)p, (const float *)p, p, p, NULL, p, (float *)p, NULL) ==
          GDR_E_INVAL);
    CHECK(gdr_decode_step(&d, p, p, p, (const float *)p, (const float *)p, p, p, (float *)p, p, NULL) ==
          GDR_E_INVAL);
    CHECK(gdr_recurrent_fwd_in(&d, NULL, p, p, p, (const float *)p, (const float *)p, NULL, NULL, NULL, p,
                               (float *)p, NULL) == GDR_E_INVAL);
    {
        gdr_input_stage st;
        memset(&st, 0, sizeof st);
        CHECK(gdr_chunk_fwd_in(&d, &st, p, p, p, (const float *)p, (const float *)p, NULL, NULL, NULL, p,
                               (float *)p, p, (size_t)1 << 40, NULL) == GDR_E_INVAL); /* no taps */
    }

    /* No sequences: a valid no-op that needs no GPU. */
    d.B = 0;
    CHECK(gdr_chunk_fwd(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, (float *)p, NULL, 0, NULL) ==
          GDR_OK);
    CHECK(strcmp(gdr_last_error(), "") == 0);
    CHECK(gdr_state_free(NULL) == GDR_OK);

    printf("ok\n");
    return 0;
}
