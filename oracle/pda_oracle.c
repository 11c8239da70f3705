/*
 * fp64 CPU oracle for paged grouped-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path calls this code: only
 * the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
 * shares no code, header or table with the GPU library.
 *
 * What it computes is the plain definition of single-token attention, written
 * out directly -- two passes over each (sequence, q head)'s gathered token
 * list -- with no online update, no splitting and no blocking:
 *
 *   score_t = (sum_d q[d] * K_t[d]) * (1 / sqrt(head_dim))
 *   M = max_t score_t,  w_t = exp(score_t - M),  L = sum_t w_t,
 *   O[d] = sum_t w_t * V_t[d],  out[d] = O[d] / L   (0 when L == 0)
 *
 * Sources (the pages that define the operation):
 *  - AstrAI "CUDA Kernels" page, section "Python Wrappers": q/k/v are laid out
 *    [batch, seq_len, n_heads, head_dim] and the scale is 1/sqrt(head_dim).
 *  - spark_storage "tiled_attention.rs" page, file header comment: a running
 *    (m, l, o) state, reset to (-inf, 0, 0), folded tile by tile, then o / l
 *    stored as bf16.  (M, L, O) above is that state after every tile listed.
 *  - same page, TiledAttention::paged_strides / scratch_pool_strides: the
 *    (blk, tok, kvh) stride triple, in bf16 elements, addresses element d of
 *    token slot j of kv head g in page b at b*blk + j*tok + g*kvh + d, for K
 *    and for V alike.
 *  - same page, TiledAttentionDims::validate and gqa_ratio: q heads are a
 *    whole multiple of kv heads, their ratio G being passed to the kernel.
 *  - AstrAI "CUDA Kernels" page, section "Python Wrappers": an optional
 *    boolean mask over the kv positions of each sequence, True keeping the
 *    position ([batch, kv_len] for a single query, [batch, q_len, kv_len]
 *    for a chunk of queries), and the is_causal switch.
 *  - same page, "Overview" table and section "Attention Backend": prefill
 *    attention (a chunk of q_len > 1 query tokens per sequence) next to
 *    decode, dispatched by q_len.
 *  - same page, "Rotary Embedding Kernel" and "Rotary Backend": rotary
 *    embedding from fp32 cos/sin tables, defined by its complex-multiply
 *    form (consecutive element pairs as complex numbers times cos + i sin).
 *
 * Readings where the pages are silent:
 *  - q head h reads kv head g = h / G (contiguous groups of G q heads).
 *  - the last-valid count is given per sequence and per tile; it applies to the
 *    last page that tile lists for the sequence, every other page being full.
 *    Counts are clamped to [0, tile_capacity], last-valid counts to
 *    [0, block_size].
 *  - a sequence with no token gives M = -inf, L = 0, O = 0 and out = 0.
 *  - the state's m is in natural-log units (the max of the scaled scores).
 *  - the mask indexes a sequence's tokens in logical order (over all tiles
 *    given); a position it does not keep is left out of the softmax entirely,
 *    exactly as if the token were not listed.
 *  - prefill: the q_len queries of a sequence are its newest tokens, already
 *    in the cache, so query i of a sequence listing P tokens sits at position
 *    P - q_len + i.  Causal attention keeps the keys at positions up to and
 *    including the query's own; a query whose position is negative (more
 *    queries than listed tokens) keeps none.  A mask, when given, removes
 *    positions on top of that.
 *
 * Inputs are bf16 bit patterns; each is widened exactly to binary64 and all
 * arithmetic is binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int32_t clamp_i32(int32_t x, int32_t lo, int32_t hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

/*
 * Element offsets (relative to a pool base) of every token row that sequence
 * s lists for kv head g, in logical order: tile by tile, page by page, slot by
 * slot, keeping only logical positions up to and including `last_pos` and,
 * with a mask row, only positions whose mask byte is non-zero.  Returns the
 * number of rows, or -1 if a kept row would leave the pool.
 */
static int64_t gather_rows(int32_t s, int32_t g, int32_t num_seqs, int32_t block_size,
                           int64_t blk, int64_t tok, int64_t kvh, int32_t head_dim,
                           int32_t n_tiles, int32_t capacity, const int32_t *blocks,
                           const int32_t *counts, const int32_t *last_valid,
                           const uint8_t *mask_row, int64_t last_pos,
                           int64_t pool_rows_limit, int64_t *rows) {
    int64_t n = 0, pos = 0;
    for (int32_t t = 0; t < n_tiles; ++t) {
        int32_t cnt = clamp_i32(counts[(int64_t)t * num_seqs + s], 0, capacity);
        const int32_t *list = blocks + ((int64_t)t * num_seqs + s) * capacity;
        for (int32_t i = 0; i < cnt; ++i) {
            int32_t valid = block_size;
            if (i == cnt - 1)
                valid = clamp_i32(last_valid[(int64_t)t * num_seqs + s], 0, block_size);
            for (int32_t j = 0; j < valid; ++j) {
                const int keep = pos <= last_pos && (mask_row == NULL || mask_row[pos] != 0);
                ++pos;
                if (!keep) continue;
                int64_t r = (int64_t)list[i] * blk + (int64_t)j * tok + (int64_t)g * kvh;
                if (list[i] < 0 || r < 0 || r + head_dim > pool_rows_limit) return -1;
                rows[n++] = r;
            }
        }
    }
    return n;
}

/* Tokens sequence s lists over the tiles (counts and last-valid clamped). */
static int64_t listed_tokens(int32_t s, int32_t num_seqs, int32_t block_size, int32_t n_tiles,
                             int32_t capacity, const int32_t *counts, const int32_t *last_valid) {
    int64_t n = 0;
    for (int32_t t = 0; t < n_tiles; ++t) {
        int32_t cnt = clamp_i32(counts[(int64_t)t * num_seqs + s], 0, capacity);
        if (cnt > 0)
            n += (int64_t)(cnt - 1) * block_size +
                 clamp_i32(last_valid[(int64_t)t * num_seqs + s], 0, block_size);
    }
    return n;
}

/*
 * The definition for one query row qh over the n gathered token rows: two
 * passes (scaled scores and their maximum; then weights, their sum and the
 * weighted sum of V rows), then out = O / L (0 when L == 0).  `score` has room
 * for n values.
 */
static void attend_rows(const uint16_t *qh, const uint16_t *kpool, const uint16_t *vpool,
                        const int64_t *rows, int64_t n, int32_t head_dim, double scale,
                        double *score, double *m, double *l, double *op, double *outp) {
    /* pass 1: scaled scores and their maximum */
    double M = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        const uint16_t *kr = kpool + rows[t];
        double acc = 0.0;
        for (int32_t d = 0; d < head_dim; ++d) acc += bf16_to_f64(qh[d]) * bf16_to_f64(kr[d]);
        score[t] = acc * scale;
        if (score[t] > M) M = score[t];
    }
    /* pass 2: weights, their sum and the weighted sum of V rows */
    double L = 0.0;
    for (int32_t d = 0; d < head_dim; ++d) op[d] = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const uint16_t *vr = vpool + rows[t];
        double w = exp(score[t] - M);
        L += w;
        for (int32_t d = 0; d < head_dim; ++d) op[d] += w * bf16_to_f64(vr[d]);
    }
    *m = M;
    *l = L;
    for (int32_t d = 0; d < head_dim; ++d) outp[d] = L > 0.0 ? op[d] / L : 0.0;
}

/*
 * Attention of one query token per sequence over the tokens listed by
 * `n_tiles` tiles (the state after those tiles, and its finalised output).
 *
 *   q           bf16 [num_seqs, num_q_heads, head_dim]
 *   pool        flat bf16 buffer of pool_elems elements; K rows start at
 *               k_base, V rows at v_base, both addressed with (blk, tok, kvh)
 *   blocks      int32 [n_tiles, num_seqs, capacity]
 *   counts      int32 [n_tiles, num_seqs]
 *   last_valid  int32 [n_tiles, num_seqs]
 *   mask        optional uint8 [num_seqs, mask_stride]: position t of sequence
 *               s (in logical order over the tiles) is kept where
 *               mask[s * mask_stride + t] != 0 (NULL: every position kept)
 *   pairs       optional list of n_pairs indices s*num_q_heads + h to compute
 *               (NULL: all num_seqs*num_q_heads, in order)
 *   m, l        fp64 [n_pairs]; o, out fp64 [n_pairs, head_dim]
 *
 * Returns 0, or -1 on a page id or row outside the pool, -2 on bad
 * dimensions, -3 on allocation failure.
 */
int pda_oracle_attend(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, const uint16_t *q,
                      const uint16_t *pool, int64_t pool_elems, int64_t k_base, int64_t v_base,
                      int64_t blk, int64_t tok, int64_t kvh, int32_t n_tiles, int32_t capacity,
                      const int32_t *blocks, const int32_t *counts, const int32_t *last_valid,
                      const uint8_t *mask, int64_t mask_stride,
                      const int32_t *pairs, int64_t n_pairs, double *m, double *l, double *o,
                      double *out, int nthreads) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || n_tiles < 0 || capacity < 0 || num_q_heads % num_kv_heads != 0)
        return -2;
    if (pairs == NULL) n_pairs = (int64_t)num_seqs * num_q_heads;
    const int32_t G = num_q_heads / num_kv_heads;
    const double scale = 1.0 / sqrt((double)head_dim);
    const int64_t max_rows = (int64_t)n_tiles * capacity * block_size;
    const int64_t k_limit = pool_elems - k_base, v_limit = pool_elems - v_base;
    const int64_t row_limit = k_limit < v_limit ? k_limit : v_limit;
    int status = 0;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel num_threads(nthreads)
    {
        int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(max_rows > 0 ? max_rows : 1));
        double *score = (double *)malloc(sizeof(double) * (size_t)(max_rows > 0 ? max_rows : 1));
        if (!rows || !score) {
#pragma omp atomic write
            status = -3;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < n_pairs; ++p) {
            if (!rows || !score) continue;
            const int64_t sh = pairs ? pairs[p] : p;
            const int32_t s = (int32_t)(sh / num_q_heads), h = (int32_t)(sh % num_q_heads);
            const int32_t g = h / G;
            double *op = o + p * head_dim, *outp = out + p * head_dim;
            int64_t n = gather_rows(s, g, num_seqs, block_size, blk, tok, kvh, head_dim, n_tiles,
                                    capacity, blocks, counts, last_valid,
                                    mask ? mask + (int64_t)s * mask_stride : NULL, INT64_MAX,
                                    row_limit, rows);
            if (n < 0) {
#pragma omp atomic write
                status = -1;
                continue;
            }
            const uint16_t *qh = q + ((int64_t)s * num_q_heads + h) * head_dim;
            attend_rows(qh, pool + k_base, pool + v_base, rows, n, head_dim, scale, score, &m[p],
                        &l[p], op, outp);
        }
        free(rows);
        free(score);
    }
    return status;
}

/*
 * Prefill: a chunk of q_len query tokens per sequence attends over the tokens
 * its one page list holds (the chunk's own keys included, as its newest
 * q_len tokens).  Query i of sequence s sits at position P_s - q_len + i,
 * P_s being the tokens the sequence lists; with `causal` it keeps the keys at
 * positions 0 .. P_s - q_len + i, without it every listed key.
 *
 *   q           bf16 [num_seqs, q_len, num_q_heads, head_dim]
 *   pool, k_base, v_base, blk, tok, kvh   as pda_oracle_attend
 *   blocks      int32 [num_seqs, capacity];  counts, last_valid int32 [num_seqs]
 *   mask        optional uint8: position t is kept for query i of sequence s
 *               where mask[s * mask_seq_stride + i * mask_q_stride + t] != 0
 *               (NULL: no mask)
 *   rows_sel    optional list of n_rows indices (s * q_len + i) * num_q_heads + h
 *               (NULL: all num_seqs * q_len * num_q_heads, in order)
 *   m, l        fp64 [n_rows]; o, out fp64 [n_rows, head_dim]
 *
 * Returns as pda_oracle_attend.
 */
int pda_oracle_prefill(int32_t num_seqs, int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, const uint16_t *q,
                       const uint16_t *pool, int64_t pool_elems, int64_t k_base, int64_t v_base,
                       int64_t blk, int64_t tok, int64_t kvh, int32_t capacity,
                       const int32_t *blocks, const int32_t *counts, const int32_t *last_valid,
                       int32_t causal, const uint8_t *mask, int64_t mask_seq_stride,
                       int64_t mask_q_stride, const int64_t *rows_sel, int64_t n_rows, double *m,
                       double *l, double *o, double *out, int nthreads) {
    if (num_seqs < 0 || q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || capacity < 0 || num_q_heads % num_kv_heads != 0)
        return -2;
    if (rows_sel == NULL) n_rows = (int64_t)num_seqs * q_len * num_q_heads;
    const int32_t G = num_q_heads / num_kv_heads;
    const double scale = 1.0 / sqrt((double)head_dim);
    const int64_t max_rows = (int64_t)capacity * block_size;
    const int64_t k_limit = pool_elems - k_base, v_limit = pool_elems - v_base;
    const int64_t row_limit = k_limit < v_limit ? k_limit : v_limit;
    int status = 0;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel num_threads(nthreads)
    {
        int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(max_rows > 0 ? max_rows : 1));
        double *score = (double *)malloc(sizeof(double) * (size_t)(max_rows > 0 ? max_rows : 1));
        if (!rows || !score) {
#pragma omp atomic write
            status = -3;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < n_rows; ++p) {
            if (!rows || !score) continue;
            const int64_t sih = rows_sel ? rows_sel[p] : p;
            const int32_t h = (int32_t)(sih % num_q_heads);
            const int64_t si = sih / num_q_heads;
            const int32_t s = (int32_t)(si / q_len), i = (int32_t)(si % q_len);
            const int32_t g = h / G;
            const int64_t P = listed_tokens(s, num_seqs, block_size, 1, capacity, counts, last_valid);
            const int64_t last_pos = causal ? P - q_len + i : INT64_MAX;
            const uint8_t *mrow = mask ? mask + (int64_t)s * mask_seq_stride + (int64_t)i * mask_q_stride
                                       : NULL;
            int64_t n = gather_rows(s, g, num_seqs, block_size, blk, tok, kvh, head_dim, 1, capacity,
                                    blocks, counts, last_valid, mrow, last_pos, row_limit, rows);
            if (n < 0) {
#pragma omp atomic write
                status = -1;
                continue;
            }
            const uint16_t *qh = q + (si * num_q_heads + h) * head_dim;
            attend_rows(qh, pool + k_base, pool + v_base, rows, n, head_dim, scale, score, &m[p],
                        &l[p], o + p * head_dim, out + p * head_dim);
        }
        free(rows);
        free(score);
    }
    return status;
}

/*
 * Rotary embedding, the complex-multiply form: element pair j of a row,
 * (x[2j], x[2j+1]), read as the complex number x[2j] + i x[2j+1], times
 * cos + i sin of the token's position:
 *
 *   out[2j]     = x[2j] cos_j - x[2j+1] sin_j
 *   out[2j + 1] = x[2j] sin_j + x[2j+1] cos_j
 *
 * with cos_j = cos_table[p * (head_dim / 2) + j] (fp32, widened exactly) and
 * p = positions[token], clamped to [0, max_positions - 1].
 *
 *   x          bf16 [num_tokens, num_heads, head_dim]
 *   out        fp64 [num_tokens, num_heads, head_dim] (unrounded)
 *
 * Returns 0, or -2 on bad dimensions (odd head_dim, non-positive sizes).
 */
int pda_oracle_rope(int64_t num_tokens, int32_t num_heads, int32_t head_dim, const uint16_t *x,
                    const float *cos_table, const float *sin_table, int32_t max_positions,
                    const int32_t *positions, double *out) {
    if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || head_dim % 2 != 0 || max_positions <= 0)
        return -2;
    const int32_t half = head_dim / 2;
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int32_t p = clamp_i32(positions[t], 0, max_positions - 1);
        const float *c = cos_table + (int64_t)p * half;
        const float *sn = sin_table + (int64_t)p * half;
        for (int32_t h = 0; h < num_heads; ++h) {
            const int64_t row = (t * num_heads + h) * head_dim;
            for (int32_t j = 0; j < half; ++j) {
                const double re = bf16_to_f64(x[row + 2 * j]), im = bf16_to_f64(x[row + 2 * j + 1]);
                const double cj = (double)c[j], sj = (double)sn[j];
                out[row + 2 * j] = re * cj - im * sj;
                out[row + 2 * j + 1] = re * sj + im * cj;
            }
        }
    }
    return 0;
}
