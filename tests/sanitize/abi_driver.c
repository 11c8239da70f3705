/*
 * Sanitizer driver for the host side of the C ABI (test infrastructure):
 * every entry point of include/pda.h through its host-side checks, with the
 * library's host code built under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Needs no GPU: the calls either return an
 * error before touching the device or are no-ops (num_seqs == 0); device
 * pointers are aligned stand-ins that are never dereferenced.
 * Exit status 0 when every call returned the status its arguments call for.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pda.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        const pda_status got_ = (call);                                                 \
        if (got_ != (want)) {                                                           \
            fprintf(stderr, "FAIL line %d: %s -> %d, want %d (%s)\n", __LINE__, #call,  \
                    (int)got_, (int)(want), pda_last_error() ? pda_last_error() : "");  \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

/* aligned stand-ins for device buffers (never dereferenced by host code) */
#define FAKE ((void *)(uintptr_t)0x100000)
#define FAKEI ((const int32_t *)(uintptr_t)0x100000)

static pda_dims mk(int32_t ms, int32_t hq, int32_t hkv, int32_t d, int32_t bs, int32_t cap) {
    pda_dims x = {ms, hq, hkv, d, bs, cap};
    return x;
}

static void sizes_sweep(void) {
    /* sizes and strides over a grid, extreme values included: no overflow,
       every call returns */
    const int32_t ms[] = {0, 1, 4, 1000, 1 << 20, 0x7fffffff};
    const int32_t hq[] = {1, 8, 32, 128, 0x7fffffff};
    const int32_t hkv[] = {1, 2, 8};
    const int32_t hd[] = {0, 8, 64, 128, 136, 256, 264};
    const int32_t bs[] = {0, 1, 16, 5, 1 << 16};
    const int32_t cap[] = {0, 1, 64, 4096, 0x7fffffff};
    const int32_t bps[] = {-1, 0, 1, 3, 64, 1 << 30};
    size_t sink = 0;
    for (size_t a = 0; a < sizeof ms / 4; ++a)
        for (size_t b = 0; b < sizeof hq / 4; ++b)
            for (size_t c = 0; c < sizeof hkv / 4; ++c)
                for (size_t e = 0; e < sizeof hd / 4; ++e)
                    for (size_t f = 0; f < sizeof bs / 4; ++f)
                        for (size_t g = 0; g < sizeof cap / 4; ++g) {
                            pda_dims d = mk(ms[a], hq[b], hkv[c], hd[e], bs[f], cap[g]);
                            const pda_status v = pda_dims_validate(&d);
                            sink += (size_t)v + pda_state_bytes(&d);
                            size_t off[3] = {0, 0, 0};
                            (void)pda_state_offsets(&d, off);
                            sink += off[2];
                            for (size_t h = 0; h < sizeof bps / 4; ++h) {
                                sink += (size_t)pda_blocks_per_split(&d, bps[h]);
                                sink += pda_workspace_bytes(&d, bps[h]);
                                sink += pda_prefill_workspace_bytes(&d, 1 + (int32_t)h * 7, bps[h]);
                            }
                            if (v == PDA_OK) {
                                const pda_strides p = pda_paged_strides(&d), s = pda_scratch_pool_strides(&d);
                                sink += (size_t)(p.blk + s.blk + pda_scratch_pool_v_offset(&d));
                            }
                        }
    printf("sizes sweep done (%zu)\n", sink);
}

static void validation(void) {
    pda_dims d = mk(4, 8, 2, 64, 16, 32);
    EXPECT(pda_dims_validate(&d), PDA_OK);
    pda_dims b = d;
    b.num_q_heads = 6; b.num_kv_heads = 4;
    EXPECT(pda_dims_validate(&b), PDA_ERR_GQA);
    b = d; b.head_dim = 264;
    EXPECT(pda_dims_validate(&b), PDA_ERR_HEAD_DIM);
    b = d; b.head_dim = 12;
    EXPECT(pda_dims_validate(&b), PDA_ERR_HEAD_DIM);
    b = d; b.block_size = 0;
    EXPECT(pda_dims_validate(&b), PDA_ERR_DIMS);
    EXPECT(pda_dims_validate(NULL), PDA_ERR_NULL);

    const pda_strides st = {16 * 2 * 64, 2 * 64, 64};
    const size_t ws = pda_workspace_bytes(&d, 0);
    /* decode: each check fires before anything is enqueued */
    EXPECT(pda_decode(&d, NULL, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, FAKE, ws, FAKE, 0, NULL), PDA_ERR_NULL);
    EXPECT(pda_decode(&d, (char *)FAKE + 2, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, FAKE, ws, FAKE, 0, NULL),
           PDA_ERR_ALIGN);
    pda_strides bad = st;
    bad.tok += 4;
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, bad, FAKE, ws, FAKE, 0, NULL), PDA_ERR_ALIGN);
    bad = st;
    bad.tok = (int64_t)1 << 30;
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, bad, FAKE, ws, FAKE, 0, NULL), PDA_ERR_DIMS);
    bad = st;
    bad.blk = INT64_MAX - 7;
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, bad, FAKE, ws, FAKE, 0, NULL), PDA_ERR_DIMS);
    bad = st;
    bad.tok = INT64_MAX - 7;
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, bad, FAKE, ws, FAKE, 0, NULL), PDA_ERR_DIMS);
    bad = st;
    bad.blk = (int64_t)1 << 32;
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, bad, FAKE, ws, FAKE, 0, NULL), PDA_ERR_DIMS);
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 5, st, FAKE, ws, FAKE, 0, NULL), PDA_ERR_MAX_SEQS);
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, -1, st, FAKE, ws, FAKE, 0, NULL), PDA_ERR_MAX_SEQS);
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, FAKE, 16, FAKE, 0, NULL), PDA_ERR_WORKSPACE);
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, FAKE, ws, FAKE, -1, NULL), PDA_ERR_DIMS);
    EXPECT(pda_decode(&b, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, FAKE, ws, FAKE, 0, NULL), PDA_ERR_DIMS);
    EXPECT(pda_decode(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 0, st, FAKE, ws, FAKE, 0, NULL), PDA_OK);
    EXPECT(pda_decode_noalloc(&d, NULL, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, FAKE, 0, NULL), PDA_ERR_NULL);
    EXPECT(pda_decode_noalloc(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 5, st, FAKE, 0, NULL), PDA_ERR_MAX_SEQS);
    /* valid dims whose partials need far more than the built-in scratch */
    pda_dims huge = mk(60000, 64, 8, 256, 16, 64);
    const pda_strides hst = pda_paged_strides(&huge);
    EXPECT(pda_dims_validate(&huge), PDA_OK);
    EXPECT(pda_decode_noalloc(&huge, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, hst, FAKE, 1, NULL),
           PDA_ERR_WORKSPACE);
    EXPECT(pda_decode_masked(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, NULL, 64, FAKE, ws, FAKE, 0, NULL),
           PDA_ERR_NULL);
    EXPECT(pda_decode_masked(&d, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, (const uint8_t *)FAKE, 0, FAKE, ws,
                             FAKE, 0, NULL),
           PDA_ERR_DIMS);

    /* prefill */
    const size_t pws = pda_prefill_workspace_bytes(&d, 8, 0);
    EXPECT(pda_prefill(&d, 0, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, 1, NULL, 0, 0, FAKE, pws, FAKE, 0, 0,
                       NULL),
           PDA_ERR_DIMS);
    EXPECT(pda_prefill(&d, 8, NULL, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 4, st, 1, NULL, 0, 0, FAKE, pws, FAKE, 0, 0,
                       NULL),
           PDA_ERR_NULL);
    EXPECT(pda_prefill(&d, 8, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 5, st, 1, NULL, 0, 0, FAKE, pws, FAKE, 0, 0,
                       NULL),
           PDA_ERR_MAX_SEQS);
    EXPECT(pda_prefill(&d, 8, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 0, st, 1, NULL, 0, 0, FAKE, pws, FAKE, 0, 0,
                       NULL),
           PDA_OK);

    /* rotary */
    const float *tab = (const float *)FAKE;
    EXPECT(pda_rope(NULL, FAKE, 4, 2, 64, tab, tab, 16, FAKEI, NULL), PDA_ERR_NULL);
    EXPECT(pda_rope(FAKE, FAKE, 4, 2, 60, tab, tab, 16, FAKEI, NULL), PDA_ERR_HEAD_DIM);
    EXPECT(pda_rope(FAKE, FAKE, -1, 2, 64, tab, tab, 16, FAKEI, NULL), PDA_ERR_DIMS);
    EXPECT(pda_rope(FAKE, FAKE, 0, 2, 64, tab, tab, 16, FAKEI, NULL), PDA_OK);
    EXPECT(pda_rope_append_kv(&d, FAKE, FAKE, 4, FAKEI, FAKEI, tab, tab, 16, NULL, FAKE, FAKE, st, NULL),
           PDA_ERR_NULL);
    EXPECT(pda_rope_append_kv(&d, FAKE, FAKE, 0, FAKEI, FAKEI, tab, tab, 16, FAKEI, FAKE, FAKE, st, NULL), PDA_OK);

    /* plans */
    pda_plan *plan = NULL;
    EXPECT(pda_create(&d, NULL, FAKE, ws, 0, &plan), PDA_ERR_NULL);
    EXPECT(pda_create(&d, FAKE, FAKE, ws - 4, 0, &plan), PDA_ERR_WORKSPACE);
    EXPECT(pda_create(&d, (char *)FAKE + 4, FAKE, ws, 0, &plan), PDA_ERR_ALIGN);
    EXPECT(pda_create(&d, FAKE, FAKE, ws, 0, &plan), PDA_OK);
    if (plan) {
        EXPECT(pda_begin_step(plan, 5, NULL), PDA_ERR_MAX_SEQS);
        EXPECT(pda_step_tile(plan, FAKE, FAKE, NULL, FAKEI, FAKEI, NULL, 16, 4, st, NULL), PDA_ERR_NULL);
        EXPECT(pda_step_tile(plan, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 9, st, NULL), PDA_ERR_MAX_SEQS);
        EXPECT(pda_finalize(plan, NULL, 4, NULL), PDA_ERR_NULL);
        EXPECT(pda_finalize(plan, FAKE, 5, NULL), PDA_ERR_MAX_SEQS);
        EXPECT(pda_begin_step(plan, 0, NULL), PDA_OK);
        EXPECT(pda_step_tile(plan, FAKE, FAKE, FAKE, FAKEI, FAKEI, NULL, 16, 0, st, NULL), PDA_OK);
        EXPECT(pda_finalize(plan, FAKE, 0, NULL), PDA_OK);
        pda_destroy(plan);
    }
    pda_destroy(NULL);
    EXPECT(pda_debug_time_attention(NULL, NULL), PDA_OK);
    EXPECT(pda_debug_time_attention(FAKE, NULL), PDA_ERR_NULL);

    for (int s = -1; s <= 9; ++s) {
        const char *t = pda_status_string((pda_status)s);
        if (!t || !t[0]) {
            fprintf(stderr, "FAIL: no status string for %d\n", s);
            ++failures;
        }
    }
    const char *le = pda_last_error();
    if (!le) {
        fprintf(stderr, "FAIL: pda_last_error returned NULL\n");
        ++failures;
    }
}

int main(void) {
    sizes_sweep();
    validation();
    printf("abi sanitizer driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
