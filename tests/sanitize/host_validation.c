/*
 * Host-side validation of the C ABI (include/gdn2.h) under AddressSanitizer
 * and UndefinedBehaviorSanitizer.  Linked against a host-only, sanitized
 * build of the library; every call below is rejected (or has nothing to
 * enqueue) before any HIP call, so no GPU is needed.  The pointers are fake,
 * well-separated device addresses: validation only compares them.
 * Prints one line per failed expectation and exits with their count.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn2.h"

static int failures = 0;

#define EXPECT(expr, want)                                                          \
    do {                                                                            \
        const long got_ = (long)(expr);                                             \
        if (got_ != (long)(want)) {                                                 \
            printf("FAIL line %d: %s -> %ld, want %ld\n", __LINE__, #expr, got_, (long)(want)); \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

#define P(i) ((void *)(uintptr_t)((UINT64_C(1) << 40) + (uint64_t)(i) * (UINT64_C(1) << 32)))
#define F(i) ((float *)P(i))

static gdn2_desc good(void) {
    gdn2_desc d;
    memset(&d, 0, sizeof d);
    d.batch = 2; d.seqlen = 128; d.heads = 4; d.dk = 128; d.dv = 128; d.chunk = 64;
    d.qkv_dtype = GDN2_BF16; d.decay_kind = GDN2_GATE_KEY; d.erase_kind = GDN2_GATE_KEY;
    d.write_kind = GDN2_GATE_KEY; d.q_scale = 1.f;
    return d;
}

static int fwd(const gdn2_desc *d, void *q, void *o, void *so, void *ws, size_t wsb) {
    return gdn2_chunk_fwd(d, q, P(1), P(2), F(3), F(4), F(5), F(6), (float *)o, (float *)so, ws, wsb, NULL);
}

static int bwd(const gdn2_desc *d, void *d_o, void *dq, void *ws, size_t wsb) {
    return gdn2_chunk_bwd(d, P(0), P(1), P(2), F(3), F(4), F(5), F(6), (const float *)d_o, F(11),
                          (float *)dq, F(13), F(14), F(15), F(16), F(17), F(18), ws, wsb, NULL);
}

int main(void) {
    size_t n = 0;
    gdn2_desc d = good();

    EXPECT(gdn2_abi_version(), GDN2_ABI_VERSION);
    for (int s = -3; s < 12; ++s) EXPECT(gdn2_status_str(s) != NULL, 1);

    /* workspace queries, valid and invalid */
    EXPECT(gdn2_chunk_fwd_workspace(&d, &n), GDN2_OK);
    EXPECT(n > 0, 1);
    EXPECT(gdn2_chunk_fwd_workspace(NULL, &n), GDN2_ERR_NULL);
    EXPECT(gdn2_chunk_fwd_workspace(&d, NULL), GDN2_ERR_NULL);
    d.qkv_dtype = GDN2_F32;
    EXPECT(gdn2_chunk_fwd_workspace(&d, &n), GDN2_OK);
    EXPECT(n, 0);
    d = good(); d.seqlen = 65536; d.batch = 1; d.heads = 16;  /* two-level scan */
    EXPECT(gdn2_chunk_fwd_workspace(&d, &n), GDN2_OK);
    EXPECT(gdn2_chunk_bwd_workspace(&d, &n), GDN2_OK);
    EXPECT(gdn2_chunk_fwd_varlen_workspace(&d, &n), GDN2_OK);
    EXPECT(gdn2_chunk_bwd_varlen_workspace(&d, &n), GDN2_OK);

    /* descriptors: every field out of range, and sizes whose products overflow */
    const struct { int field; int64_t value; int want; } bad[] = {
        {0, -1, GDN2_ERR_SHAPE}, {1, -5, GDN2_ERR_SHAPE}, {2, 0, GDN2_ERR_SHAPE}, {3, 0, GDN2_ERR_SHAPE},
        {4, 0, GDN2_ERR_SHAPE}, {3, 129, GDN2_ERR_UNSUPPORTED}, {4, 256, GDN2_ERR_UNSUPPORTED},
        {5, 8, GDN2_ERR_UNSUPPORTED}, {5, 128, GDN2_ERR_UNSUPPORTED}, {6, 7, GDN2_ERR_DTYPE},
        {7, 2, GDN2_ERR_SHAPE}, {8, -1, GDN2_ERR_SHAPE}, {9, 2, GDN2_ERR_DTYPE},
        {10, INT64_MAX / 2, GDN2_ERR_SHAPE}, {11, INT64_MAX, GDN2_ERR_SHAPE}, {12, INT64_MAX, GDN2_ERR_SHAPE},
    };
    for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
        d = good();
        switch (bad[i].field) {
            case 0: d.batch = bad[i].value; break;
            case 1: d.seqlen = bad[i].value; break;
            case 2: d.heads = bad[i].value; break;
            case 3: d.dk = bad[i].value; break;
            case 4: d.dv = bad[i].value; break;
            case 5: d.chunk = bad[i].value; break;
            case 6: d.qkv_dtype = (int32_t)bad[i].value; break;
            case 7: d.decay_kind = (int32_t)bad[i].value; break;
            case 8: d.erase_kind = (int32_t)bad[i].value; break;
            case 9: d.o_dtype = (int32_t)bad[i].value; break;
            case 10: d.batch = bad[i].value; d.seqlen = 1 << 30; break;
            case 11: d.seqlen = bad[i].value; break;
            case 12: d.heads = bad[i].value; break;
        }
        EXPECT(fwd(&d, P(0), P(7), P(8), NULL, 0), bad[i].want);
        EXPECT(gdn2_chunk_fwd_workspace(&d, &n), bad[i].want);
        EXPECT(gdn2_chunk_fwd_static(&d, P(0), P(1), P(2), F(3), F(4), F(5), F(6), F(7), F(8), NULL),
               bad[i].want);
    }

    /* null arguments and aliasing */
    d = good();
    EXPECT(fwd(NULL, P(0), P(7), P(8), NULL, 0), GDN2_ERR_NULL);
    EXPECT(fwd(&d, NULL, P(7), P(8), NULL, 0), GDN2_ERR_NULL);
    EXPECT(fwd(&d, P(0), NULL, P(8), NULL, 0), GDN2_ERR_NULL);
    EXPECT(fwd(&d, P(0), (char *)P(0) + 16, P(8), NULL, 0), GDN2_ERR_ALIAS);
    EXPECT(fwd(&d, P(0), P(7), (char *)P(6) + 64, NULL, 0), GDN2_ERR_ALIAS);
    EXPECT(fwd(&d, P(0), P(7), P(8), P(7), 1 << 30), GDN2_ERR_ALIAS);
    EXPECT(fwd(&d, P(0), P(7), P(8), P(9), 16), GDN2_ERR_WORKSPACE);
    EXPECT(fwd(&d, P(0), P(7), P(8), (char *)P(9) + 8, 1 << 30), GDN2_ERR_WORKSPACE);

    /* nothing to enqueue: T == 0 with the state updated in place, B == 0 */
    d = good(); d.seqlen = 0;
    EXPECT(fwd(&d, P(0), P(7), P(6), NULL, 0), GDN2_OK);
    EXPECT(fwd(&d, P(0), P(7), NULL, NULL, 0), GDN2_OK);
    d = good(); d.batch = 0;
    EXPECT(fwd(&d, P(0), P(7), NULL, NULL, 0), GDN2_OK);

    /* the static entry point: too large for its scratch */
    d = good(); d.batch = 244; d.heads = 4; d.seqlen = 64 * 100;
    EXPECT(gdn2_chunk_fwd_static(&d, P(0), P(1), P(2), F(3), F(4), F(5), F(6), F(7), F(8), NULL),
           GDN2_ERR_SCRATCH);

    /* decode */
    d = good(); d.seqlen = 2;
    EXPECT(gdn2_recurrent_step(&d, P(0), P(1), P(2), F(3), F(4), F(5), F(6), F(7), NULL), GDN2_ERR_SHAPE);
    d.seqlen = 1;
    EXPECT(gdn2_recurrent_step(&d, P(0), P(1), P(2), F(3), F(4), F(5), F(6), (float *)((char *)P(6) + 8), NULL),
           GDN2_ERR_ALIAS);
    EXPECT(gdn2_recurrent_step(NULL, P(0), P(1), P(2), F(3), F(4), F(5), F(6), F(7), NULL), GDN2_ERR_NULL);

    /* backward */
    d = good();
    EXPECT(gdn2_chunk_bwd_workspace(&d, &n), GDN2_OK);
    const size_t bws = n;
    EXPECT(bwd(&d, NULL, P(12), P(19), bws), GDN2_ERR_NULL);
    EXPECT(bwd(&d, P(10), P(12), P(19), bws - 256), GDN2_ERR_WORKSPACE);
    EXPECT(bwd(&d, P(10), P(10), P(19), bws), GDN2_ERR_ALIAS);
    d.o_dtype = GDN2_BF16;  /* d_o is fp32 whatever o_dtype says: its whole span is checked */
    EXPECT(bwd(&d, P(10), (char *)P(10) + 2 * 128 * 4 * 128 * 4 - 4, P(19), bws), GDN2_ERR_ALIAS);

    /* packed sequences */
    d = good(); d.batch = 3;
    EXPECT(gdn2_chunk_fwd_varlen(&d, NULL, P(0), P(1), P(2), F(3), F(4), F(5), F(6), F(7), F(8), NULL, 0, NULL),
           GDN2_ERR_NULL);
    EXPECT(gdn2_chunk_fwd_varlen(&d, (const int32_t *)P(7), P(0), P(1), P(2), F(3), F(4), F(5), F(6), F(7), F(8),
                                 NULL, 0, NULL),
           GDN2_ERR_ALIAS);

    printf("%d failures\n", failures);
    return failures;
}
