/*
 * Sanitizer driver for the fp64 oracle (test infrastructure): the oracle's
 * three entry points over seeded random small problems, built together with
 * oracle/pda_oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer.
 * Values are checked elsewhere (the oracle's pins); here every call must stay
 * within its buffers, return the code its inputs call for, and give finite
 * outputs for finite inputs.
 *
 * Cases: both pool layouts' stride shapes, block sizes 1..32, empty and
 * one-token sequences, counts and last-valid counts out of range (clamped),
 * page ids outside the pool (must return -1), keep-masks, row selections,
 * several tiles, prefill causal and not, rotary with positions out of the
 * table (clamped).  Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int pda_oracle_attend(int32_t, int32_t, int32_t, int32_t, int32_t, const uint16_t *, const uint16_t *,
                      int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int32_t, int32_t,
                      const int32_t *, const int32_t *, const int32_t *, const uint8_t *, int64_t,
                      const int32_t *, int64_t, double *, double *, double *, double *, int);
int pda_oracle_prefill(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, const uint16_t *,
                       const uint16_t *, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int32_t,
                       const int32_t *, const int32_t *, const int32_t *, int32_t, const uint8_t *,
                       int64_t, int64_t, const int64_t *, int64_t, double *, double *, double *,
                       double *, int);
int pda_oracle_rope(int64_t, int32_t, int32_t, const uint16_t *, const float *, const float *, int32_t,
                    const int32_t *, double *);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {   /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int rnd(int n) { return (int)(next_u64() % (uint64_t)n); }
static uint16_t rnd_bf16(void) {   /* finite values in [-2, 2) */
    float f = (float)((double)(next_u64() >> 11) / 9007199254740992.0 * 4.0 - 2.0);
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static int failures = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fprintf(stderr, "\n");                        \
            ++failures;                                   \
        }                                                 \
    } while (0)

static int all_finite(const double *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

/* One random paged problem: pool with every listed page plus a poison page. */
static void attend_case(int trial) {
    const int S = 1 + rnd(4), Hkv = 1 + rnd(3), G = 1 + rnd(4), Hq = Hkv * G;
    const int D = 2 * (1 + rnd(40)), bs = 1 + rnd(32), T = 1 + rnd(3);
    const int scratch = rnd(2);
    int ctx[4];
    int pages_needed = 0;
    for (int s = 0; s < S; ++s) {
        ctx[s] = rnd(4) == 0 ? rnd(2) : rnd(200);
        pages_needed += (ctx[s] + bs - 1) / bs;
    }
    const int P = pages_needed + 2;
    int64_t blk, tok, kvh;
    if (scratch) { blk = 2LL * Hkv * bs * D; tok = D; kvh = (int64_t)bs * D; }
    else { blk = (int64_t)bs * Hkv * D; tok = (int64_t)Hkv * D; kvh = D; }
    const int64_t v_base = scratch ? (int64_t)Hkv * bs * D : (int64_t)P * blk;
    const int64_t pool_elems = scratch ? (int64_t)P * blk : 2 * (int64_t)P * blk;
    uint16_t *pool = malloc(sizeof(uint16_t) * (size_t)pool_elems);
    for (int64_t i = 0; i < pool_elems; ++i) pool[i] = rnd_bf16();
    /* split each sequence's pages over T tiles */
    int cap = 1;
    int *seq_first = malloc(sizeof(int) * S), *seq_np = malloc(sizeof(int) * S);
    int next_page = 1;   /* page 0 is left out (never listed) */
    for (int s = 0; s < S; ++s) {
        seq_first[s] = next_page;
        seq_np[s] = (ctx[s] + bs - 1) / bs;
        next_page += seq_np[s];
        if (seq_np[s] > cap) cap = seq_np[s];
    }
    int32_t *blocks = calloc((size_t)T * S * cap, sizeof(int32_t));
    int32_t *counts = calloc((size_t)T * S, sizeof(int32_t));
    int32_t *lastv = calloc((size_t)T * S, sizeof(int32_t));
    for (int s = 0; s < S; ++s) {
        int done = 0;
        for (int t = 0; t < T; ++t) {
            const int n = t == T - 1 ? seq_np[s] - done : rnd(seq_np[s] - done + 1);
            for (int j = 0; j < n; ++j) blocks[((int64_t)t * S + s) * cap + j] = seq_first[s] + done + j;
            counts[t * S + s] = n;
            const int last_page_tokens = (done + n == seq_np[s] && ctx[s] % bs) ? ctx[s] % bs : bs;
            lastv[t * S + s] = n ? last_page_tokens : 0;
            done += n;
        }
    }
    /* out-of-range counts and last-valid values are clamped by the oracle */
    if (trial % 5 == 0) { counts[0] = cap + 3; lastv[0] = bs + 7; }
    if (trial % 7 == 0) { counts[0] = -2; lastv[0] = -1; }
    uint16_t *q = malloc(sizeof(uint16_t) * (size_t)S * Hq * D);
    for (int64_t i = 0; i < (int64_t)S * Hq * D; ++i) q[i] = rnd_bf16();
    const int64_t mstride = (int64_t)T * cap * bs + 3;
    uint8_t *mask = NULL;
    if (rnd(2)) {
        mask = malloc((size_t)S * mstride);
        for (int64_t i = 0; i < S * mstride; ++i) mask[i] = (uint8_t)(rnd(4) != 0);
    }
    int32_t pairs[5];
    int64_t npairs = (int64_t)S * Hq;
    const int32_t *pp = NULL;
    if (rnd(3) == 0) {
        npairs = 1 + rnd(5);
        for (int i = 0; i < npairs; ++i) pairs[i] = rnd(S * Hq);
        pp = pairs;
    }
    double *m = malloc(sizeof(double) * npairs), *l = malloc(sizeof(double) * npairs);
    double *o = malloc(sizeof(double) * npairs * D), *out = malloc(sizeof(double) * npairs * D);
    int rc = pda_oracle_attend(S, Hq, Hkv, D, bs, q, pool, pool_elems, 0, v_base, blk, tok, kvh, T, cap,
                               blocks, counts, lastv, mask, mstride, pp, npairs, m, l, o, out, 1 + rnd(3));
    CHECK(rc == 0, "attend trial %d returned %d", trial, rc);
    if (rc == 0) {
        CHECK(all_finite(l, npairs) && all_finite(o, npairs * D) && all_finite(out, npairs * D),
              "attend trial %d: non-finite output", trial);
    }
    /* a page id past the pool must be refused with -1 (when the page is
       read: every row computed, no mask) */
    if (S > 0 && counts[0] > 0 && counts[0] <= cap && pp == NULL && mask == NULL) {
        const int32_t keep = blocks[0];
        blocks[0] = P + 5;
        rc = pda_oracle_attend(S, Hq, Hkv, D, bs, q, pool, pool_elems, 0, v_base, blk, tok, kvh, T, cap,
                               blocks, counts, lastv, mask, mstride, pp, npairs, m, l, o, out, 1);
        CHECK(rc == -1, "attend trial %d: page outside the pool returned %d", trial, rc);
        blocks[0] = -3;
        rc = pda_oracle_attend(S, Hq, Hkv, D, bs, q, pool, pool_elems, 0, v_base, blk, tok, kvh, T, cap,
                               blocks, counts, lastv, mask, mstride, pp, npairs, m, l, o, out, 1);
        CHECK(rc == -1, "attend trial %d: negative page returned %d", trial, rc);
        blocks[0] = keep;
    }
    /* bad dimensions: 3 q heads over 2 kv heads is no whole ratio */
    rc = pda_oracle_attend(S, 3, 2, D, bs, q, pool, pool_elems, 0, v_base, blk, tok, kvh, T, cap,
                           blocks, counts, lastv, mask, mstride, NULL, 0, m, l, o, out, 1);
    CHECK(rc == -2, "attend: bad GQA ratio accepted (%d)", rc);

    /* prefill over tile 0 as the sequence's one page list */
    const int Q = 1 + rnd(6);
    uint16_t *qc = malloc(sizeof(uint16_t) * (size_t)S * Q * Hq * D);
    for (int64_t i = 0; i < (int64_t)S * Q * Hq * D; ++i) qc[i] = rnd_bf16();
    const int64_t nrows_all = (int64_t)S * Q * Hq;
    int64_t rows[4];
    int64_t nrows = nrows_all;
    const int64_t *rs = NULL;
    if (rnd(2)) {
        nrows = 1 + rnd(4);
        for (int i = 0; i < nrows; ++i) rows[i] = (int64_t)rnd((int)nrows_all);
        rs = rows;
    }
    const int64_t mq = cap * bs + 1, ms = Q * mq;
    uint8_t *pmask = NULL;
    if (rnd(2)) {
        pmask = malloc((size_t)S * ms);
        for (int64_t i = 0; i < S * ms; ++i) pmask[i] = (uint8_t)(rnd(3) != 0);
    }
    double *pm = malloc(sizeof(double) * nrows), *pl = malloc(sizeof(double) * nrows);
    double *po = malloc(sizeof(double) * nrows * D), *pout = malloc(sizeof(double) * nrows * D);
    for (int causal = 0; causal < 2; ++causal) {
        rc = pda_oracle_prefill(S, Q, Hq, Hkv, D, bs, qc, pool, pool_elems, 0, v_base, blk, tok, kvh, cap,
                                blocks, counts, lastv, causal, pmask, ms, mq, rs, nrows, pm, pl, po, pout,
                                1 + rnd(3));
        CHECK(rc == 0, "prefill trial %d causal %d returned %d", trial, causal, rc);
        if (rc == 0) CHECK(all_finite(pout, nrows * D), "prefill trial %d: non-finite output", trial);
    }
    free(pm); free(pl); free(po); free(pout); free(pmask); free(qc);
    free(m); free(l); free(o); free(out); free(mask); free(q);
    free(blocks); free(counts); free(lastv); free(seq_first); free(seq_np); free(pool);
}

static void rope_case(int trial) {
    const int64_t Tn = rnd(20);
    const int H = 1 + rnd(5), D = 2 * (1 + rnd(33)), MP = 1 + rnd(50);
    uint16_t *x = malloc(sizeof(uint16_t) * (size_t)(Tn * H * D + 1));
    for (int64_t i = 0; i < Tn * H * D; ++i) x[i] = rnd_bf16();
    float *ct = malloc(sizeof(float) * (size_t)MP * (D / 2)), *st = malloc(sizeof(float) * (size_t)MP * (D / 2));
    for (int64_t i = 0; i < (int64_t)MP * (D / 2); ++i) {
        ct[i] = (float)cos((double)i);
        st[i] = (float)sin((double)i);
    }
    int32_t *pos = malloc(sizeof(int32_t) * (size_t)(Tn + 1));
    for (int64_t i = 0; i < Tn; ++i) pos[i] = rnd(MP + 10) - 5;   /* some out of the table */
    double *out = malloc(sizeof(double) * (size_t)(Tn * H * D + 1));
    int rc = pda_oracle_rope(Tn, H, D, x, ct, st, MP, pos, out);
    CHECK(rc == 0, "rope trial %d returned %d", trial, rc);
    if (rc == 0) CHECK(all_finite(out, Tn * H * D), "rope trial %d: non-finite output", trial);
    rc = pda_oracle_rope(Tn, H, D + 1, x, ct, st, MP, pos, out);
    CHECK(rc == -2, "rope: odd head_dim accepted (%d)", rc);
    free(x); free(ct); free(st); free(pos); free(out);
}

int main(int argc, char **argv) {
    const int trials = argc > 1 ? atoi(argv[1]) : 300;
    for (int t = 0; t < trials; ++t) {
        attend_case(t);
        rope_case(t);
    }
    printf("oracle sanitizer driver: %d trials, %d failures\n", trials, failures);
    return failures ? 1 : 0;
}
