/*
 * pda.h -- paged grouped-query decode attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpda.so.  One query token per sequence attends over a bf16 K/V
 * cache stored in fixed-size pages ("blocks") that each sequence reaches
 * through its own list of page ids.  The work runs as split-KV partial passes
 * that keep an online-softmax (m, l, o) state, merged by log-sum-exp, then a
 * finalize step that stores o / l as bf16.
 *
 * Sources, by page and section:
 *  [TA]  spark_storage "tiled_attention.rs": the header comment (state
 *        lifecycle: reset, one launch per tile, finalize), TiledAttentionDims
 *        and its validate / gqa_ratio / *_bytes, TiledAttention::begin_step,
 *        paged_strides, scratch_pool_strides, step_tile, finalize, and the
 *        constant NEG_INF_F32_BITS.
 *  [CK]  AstrAI "CUDA Kernels": section "Python Wrappers" (q/k/v layout
 *        [batch, seq_len, n_heads, head_dim]; scale 1/sqrt(head_dim); the
 *        optional boolean mask [batch, kv_len], true keeping a position;
 *        wrappers fail loudly when the compiled library is absent), section
 *        "Attention Backend" (decode through the paged kernel with page
 *        size 1) and the "Overview" table (GQA decode with split-KV; paged
 *        KV-cache decode; GQA prefill), the is_causal switch and the
 *        [batch, q_len, kv_len] mask of "Python Wrappers" for prefill;
 *        "Rotary Embedding Kernel" and "Rotary Backend" (fused cos/sin
 *        lookup and rotation, fp32 tables, bf16 rows; its complex-multiply
 *        form defines the pairing).
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device memory owned by the caller; the
 *    library never allocates, frees or retains device memory and keeps no
 *    global device state, except the fixed scratch array of
 *    pda_decode_noalloc (PDA_NOALLOC_SCRATCH_BYTES per GPU, part of the
 *    library's code object).  pda_plan is a small host-side handle.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued on it and the call returns without synchronising; a device
 *    fault therefore surfaces at the caller's next synchronisation.
 *  - Every argument is checked on the host before anything is enqueued: a
 *    call that returns a status other than PDA_OK has enqueued nothing
 *    (PDA_ERR_HIP excepted, which reports a failed launch).  A thread-local
 *    text with details is available from pda_last_error().
 *  - bf16 tensors hold raw bfloat16 bit patterns (uint16).  q, the pools, the
 *    output, the state and the workspace must be 16-byte aligned; strides must
 *    be non-negative multiples of 8 elements (PDA_ERR_ALIGN) below 2^32
 *    elements each, with a token row's offset inside a page below 2^31
 *    (PDA_ERR_DIMS); page-id, count and last-valid arrays must be
 *    4-byte aligned.
 *  - Device-side data contract (not checkable on the host): counts are read
 *    clamped to [0, tile_capacity] and last-valid counts to [0, block_size];
 *    every listed page id must address a page inside the pools.
 */
#ifndef PDA_H
#define PDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pda_status {
    PDA_OK = 0,
    PDA_ERR_NULL = 1,      /* a required pointer is NULL */
    PDA_ERR_DIMS = 2,      /* a dimension is out of range (non-positive, or an index would overflow) */
    PDA_ERR_GQA = 3,       /* num_q_heads is not a whole multiple of num_kv_heads ([TA] validate) */
    PDA_ERR_HEAD_DIM = 4,  /* head_dim above 256 ([TA] validate) or not a multiple of 8 */
    PDA_ERR_MAX_SEQS = 5,  /* num_seqs above max_seqs ([TA] begin_step) or negative */
    PDA_ERR_ALIGN = 6,     /* pointer or stride misaligned, or stride negative */
    PDA_ERR_WORKSPACE = 7, /* workspace smaller than pda_workspace_bytes requires */
    PDA_ERR_HIP = 8        /* a HIP launch failed ([TA] begin_step memset status checks) */
} pda_status;

/* Sizes fixed for the lifetime of a plan ([TA] TiledAttentionDims).
 * max_seqs bounds num_seqs of every call; tile_capacity is the row length of
 * the page-id arrays, i.e. the most pages one sequence lists per call. */
typedef struct pda_dims {
    int32_t max_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t tile_capacity;
} pda_dims;

/* Stride triple in bf16 elements selecting the K/V layout ([TA] paged_strides,
 * scratch_pool_strides): element d of token slot j of kv head g in page b is
 * at pool[b*blk + j*tok + g*kvh + d].  K and V share the triple. */
typedef struct pda_strides {
    int64_t blk;
    int64_t tok;
    int64_t kvh;
} pda_strides;

typedef struct pda_plan pda_plan;

/* Checks dims: every field >= 1; num_q_heads % num_kv_heads == 0
 * (PDA_ERR_GQA); head_dim <= 256 and head_dim % 8 == 0 (PDA_ERR_HEAD_DIM);
 * tile_capacity * block_size <= 2^24 and tile_capacity * block_size^2 <= 2^32
 * (PDA_ERR_DIMS).  [TA] TiledAttentionDims::validate. */
pda_status pda_dims_validate(const pda_dims *dims);

/* Bytes of the fp32 running state ([TA] m_bytes + l_bytes + o_bytes): m and l
 * are [max_seqs, num_q_heads], o is [max_seqs, num_q_heads, head_dim], stored
 * in that order in one caller-owned device buffer, each starting on a 16-byte
 * boundary (m and l padded up to a multiple of 16 bytes; pda_state_offsets).  m is in
 * natural-log units (the running max of the scaled scores), l the running sum
 * of exp(score - m), o the running sum of exp(score - m) * V.  0 if dims are
 * invalid. */
size_t pda_state_bytes(const pda_dims *dims);

/* Byte offsets of m, l and o inside the state buffer (offsets[0..2]). */
pda_status pda_state_offsets(const pda_dims *dims, size_t offsets[3]);

/* Pages per split-KV partition that a call with `blocks_per_split` uses:
 * the request clamped to [1, tile_capacity], or the library's own choice
 * when the request is 0 (never fewer than ceil(tile_capacity / 256) pages). */
int32_t pda_blocks_per_split(const pda_dims *dims, int32_t blocks_per_split);

/* Device workspace bytes for max_seqs sequences with the given
 * blocks_per_split (0 = the library's choice, sized for any device): 256 bytes
 * of control words (the work-item counter), one 64-bit arrival counter per
 * (sequence, kv head, chunk of 16 q heads) padded to a multiple of 16 bytes,
 * then the fp32 split partials: the (m, l) pairs, rows * slots * 2 * 4 bytes
 * padded up to a multiple of 16, then the o rows, rows * slots * head_dim * 4,
 * where rows = max_seqs * num_q_heads and slots = ceil(tile_capacity / bps),
 * one per split (the kernel may group splits into larger work items, which
 * then share a slot, or, in a launch with too little work for more than one
 * round of split items, lengthen every split up to twice bps pages: splits
 * only grow, so a sequence never needs more slots than this).
 * The workspace needs no clearing, before its first use or ever: every
 * counter is tagged with the launch that counts in it, and a launch restarts
 * any counter another launch (or leftover content) left behind.  Calls that
 * share a workspace must not run concurrently (order them on one stream).  0
 * if dims are invalid. */
size_t pda_workspace_bytes(const pda_dims *dims, int32_t blocks_per_split);

/* ([TA] paged_strides) layout [num_blocks, block_size, num_kv_heads, head_dim]:
 * (block_size*num_kv_heads*head_dim, num_kv_heads*head_dim, head_dim). */
pda_strides pda_paged_strides(const pda_dims *dims);

/* ([TA] scratch_pool_strides) layout [slot, K|V, kv_head, block_size, head_dim]:
 * with kv_stripe = num_kv_heads*block_size*head_dim,
 * (2*kv_stripe, head_dim, block_size*head_dim).  The V pool pointer is the K
 * pool pointer plus pda_scratch_pool_v_offset() elements. */
pda_strides pda_scratch_pool_strides(const pda_dims *dims);
int64_t pda_scratch_pool_v_offset(const pda_dims *dims);

/* Creates a plan over caller-owned device buffers ([TA] TiledAttention::new,
 * which allocates its own state; here the caller does):
 *   state      device, pda_state_bytes(dims) bytes
 *   workspace  device, at least pda_workspace_bytes(dims, blocks_per_split)
 *   blocks_per_split  0 = the library's choice
 * The buffers must outlive the plan.  *out receives the handle. */
pda_status pda_create(const pda_dims *dims, void *state, void *workspace, size_t workspace_bytes,
                      int32_t blocks_per_split, pda_plan **out);
void pda_destroy(pda_plan *plan);

/* Resets state rows [0, num_seqs) to m = -inf (bits 0xFF800000), l = 0,
 * o = 0 ([TA] begin_step, NEG_INF_F32_BITS).  Rows >= num_seqs are left
 * untouched.  Fails with PDA_ERR_MAX_SEQS if num_seqs > max_seqs. */
pda_status pda_begin_step(pda_plan *plan, int32_t num_seqs, void *stream);

/* Folds one tile of pages into the running state ([TA] step_tile; split-KV
 * per [CK] Overview).
 *   q                  device bf16 [num_seqs, num_q_heads, head_dim]
 *   k_pool, v_pool     device bf16 pools addressed with `strides`
 *   tile_blocks        device int32 [num_seqs, tile_capacity]: page ids, in
 *                      logical token order
 *   tile_block_counts  device int32 [num_seqs]: pages listed per sequence
 *   last_block_valid   device int32 [num_seqs], or NULL to use
 *                      last_block_valid_default for every sequence: valid
 *                      token slots in the last page this tile lists for the
 *                      sequence (block_size when the sequence continues in a
 *                      later tile)
 * q head h attends with kv head h / (num_q_heads / num_kv_heads); scores are
 * scaled by 1/sqrt(head_dim) ([CK] Python Wrappers).  A sequence with count
 * 0 leaves its state rows bit-unchanged.  Rows >= num_seqs are untouched. */
pda_status pda_step_tile(pda_plan *plan, const void *q, const void *k_pool, const void *v_pool,
                         const int32_t *tile_blocks, const int32_t *tile_block_counts,
                         const int32_t *last_block_valid, int32_t last_block_valid_default,
                         int32_t num_seqs, pda_strides strides, void *stream);

/* out[s, h, :] = bf16(o / l), rounded to nearest even; 0 where l == 0
 * ([TA] finalize).  out: device bf16 [num_seqs, num_q_heads, head_dim]. */
pda_status pda_finalize(pda_plan *plan, void *out, int32_t num_seqs, void *stream);

/* One-shot decode: split-KV partials, their log-sum-exp merge and o / l to
 * bf16, with the split partials in `workspace` ([CK] Overview: paged decode,
 * split-KV).
 * Arguments as pda_step_tile plus:
 *   dims        as for pda_create (num_seqs <= dims->max_seqs)
 *   workspace   device, at least pda_workspace_bytes(dims, blocks_per_split)
 *   out         device bf16 [num_seqs, num_q_heads, head_dim]
 * A sequence with no token gets an all-zero output row. */
pda_status pda_decode(const pda_dims *dims, const void *q, const void *k_pool, const void *v_pool,
                      const int32_t *block_tables, const int32_t *block_counts,
                      const int32_t *last_block_valid, int32_t last_block_valid_default,
                      int32_t num_seqs, pda_strides strides, void *workspace,
                      size_t workspace_bytes, void *out, int32_t blocks_per_split, void *stream);

/* Bytes of the scratch array built into the library for pda_decode_noalloc
 * (one array per GPU, from the library's load until the process ends). */
#define PDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* pda_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no workspace: the split partials and control words live in a scratch
 * array with static storage inside the library, PDA_NOALLOC_SCRATCH_BYTES on
 * each GPU, whose device address is looked up once per device (on the first
 * call with that device current).  The call allocates nothing and calls no
 * allocating routine; q, the pools, the tables and `out` are the caller's.
 * Arguments, results and errors as pda_decode, with the scratch in place of
 * `workspace`; the current device must be the one `stream` belongs to.
 *   PDA_ERR_WORKSPACE  if these dims and blocks_per_split need more than
 *                      PDA_NOALLOC_SCRATCH_BYTES (pda_workspace_bytes(dims,
 *                      blocks_per_split) > the limit); raise
 *                      blocks_per_split, lower max_seqs / tile_capacity or
 *                      call pda_decode with a workspace
 *   PDA_ERR_HIP        if the scratch address cannot be looked up
 * Every call on a GPU shares that GPU's scratch and keeps the last call's
 * contents there; nothing in it needs clearing (its counters are tagged with
 * the launch that counts in them, as in any workspace).  Calls that overlap on
 * one GPU (different streams or threads without ordering) race on the scratch
 * and give wrong results: order them, for example on one stream. */
pda_status pda_decode_noalloc(const pda_dims *dims, const void *q, const void *k_pool,
                              const void *v_pool, const int32_t *block_tables,
                              const int32_t *block_counts, const int32_t *last_block_valid,
                              int32_t last_block_valid_default, int32_t num_seqs,
                              pda_strides strides, void *out, int32_t blocks_per_split,
                              void *stream);

/* pda_decode with a boolean keep-mask over each sequence's kv positions
 * ([CK] Python Wrappers: mask [batch, kv_len], true = keep).
 *   kv_mask      device uint8 [num_seqs, mask_stride]: position t of sequence
 *                s (its t-th listed token, in list order) takes part where
 *                kv_mask[s * mask_stride + t] != 0
 *   mask_stride  bytes per sequence row, >= 1 (PDA_ERR_DIMS otherwise)
 * Other arguments as pda_decode.  A dropped position is left out of the
 * softmax as if its token were not listed; a sequence whose every position is
 * dropped gets an all-zero output row.  Device-side contract: each row holds
 * at least as many bytes as its sequence lists tokens.  PDA_ERR_NULL if
 * kv_mask is NULL. */
pda_status pda_decode_masked(const pda_dims *dims, const void *q, const void *k_pool,
                             const void *v_pool, const int32_t *block_tables,
                             const int32_t *block_counts, const int32_t *last_block_valid,
                             int32_t last_block_valid_default, int32_t num_seqs,
                             pda_strides strides, const uint8_t *kv_mask, int64_t mask_stride,
                             void *workspace, size_t workspace_bytes, void *out,
                             int32_t blocks_per_split, void *stream);

/* Device workspace bytes for pda_prefill with chunks of q_len queries and the
 * given blocks_per_split (0 = the library's choice, sized for any device):
 * the fp32 split partials of max_seqs * q_len * num_q_heads rows, slots =
 * ceil(tile_capacity / bps) each, (m, l) pairs then o rows,
 * rows * slots * (head_dim + 2) * 4 + 16 bytes; 0 when no call with these
 * sizes splits (one split covers tile_capacity pages), and 0 if dims are
 * invalid or q_len < 1.  Needs no clearing; calls sharing a workspace must
 * not run concurrently. */
size_t pda_prefill_workspace_bytes(const pda_dims *dims, int32_t q_len, int32_t blocks_per_split);

/* Prefill / chunked prefill ([CK] Overview: GQA prefill; Python Wrappers:
 * is_causal and the [batch, q_len, kv_len] mask; Attention Backend: prefill
 * next to decode).  Each sequence brings a chunk of q_len query tokens that
 * are its newest tokens, their keys and values already written to the pages
 * it lists: query i of a sequence listing P tokens sits at position
 * P - q_len + i.
 *   dims, k_pool, v_pool, block_tables, block_counts, last_block_valid,
 *   last_block_valid_default, num_seqs, strides   as pda_decode
 *   q_len         queries per sequence, >= 1 (PDA_ERR_DIMS otherwise)
 *   q             device bf16 [num_seqs, q_len, num_q_heads, head_dim] (blhd)
 *   causal        non-zero: query i keeps keys at positions 0 .. P - q_len + i
 *                 (none if that is negative); zero: every listed key
 *   kv_mask       NULL, or device uint8: key t takes part for query i of
 *                 sequence s only where kv_mask[s * mask_seq_stride +
 *                 i * mask_q_stride + t] != 0 (mask_q_stride 0 shares one
 *                 [batch, kv_len] row across the chunk), on top of causal;
 *                 strides >= 0 (PDA_ERR_DIMS otherwise)
 *   workspace     device, pda_prefill_workspace_bytes(dims, q_len,
 *                 blocks_per_split) bytes (may be NULL when that is 0)
 *   out           device bf16 [num_seqs, q_len, num_q_heads, head_dim]
 *   blocks_per_split  pages per split-KV partition, 0 = the library's choice
 *   rows_per_wave     16, 32 or 64 query rows (q_len x q-head pairs of one kv
 *                 head) per wavefront, 0 = the library's choice (16 when a kv
 *                 head has at most 16 rows, else 32); capped at 16 for
 *                 head_dim > 128 and at 32 for head_dim > 64 with a mask
 * q head h attends with kv head h / (num_q_heads / num_kv_heads), scale
 * 1/sqrt(head_dim).  A query that keeps no key gets an all-zero row.
 * Device-side contract as pda_decode; with a mask, every row covers the
 * tokens its sequence lists. */
pda_status pda_prefill(const pda_dims *dims, int32_t q_len, const void *q, const void *k_pool,
                       const void *v_pool, const int32_t *block_tables,
                       const int32_t *block_counts, const int32_t *last_block_valid,
                       int32_t last_block_valid_default, int32_t num_seqs, pda_strides strides,
                       int32_t causal, const uint8_t *kv_mask, int64_t mask_seq_stride,
                       int64_t mask_q_stride, void *workspace, size_t workspace_bytes, void *out,
                       int32_t blocks_per_split, int32_t rows_per_wave, void *stream);

/* Rotary embedding ([CK] Rotary Embedding Kernel, Rotary Backend): element
 * pair j of each row, (x[2j], x[2j+1]), read as a complex number, times
 * cos + i sin of the token's position:
 *   out[2j] = x[2j] cos_j - x[2j+1] sin_j,  out[2j+1] = x[2j] sin_j + x[2j+1] cos_j
 * computed in fp32 and rounded once to bf16 (nearest even).
 *   x, out        device bf16 [num_tokens, num_heads, head_dim] (blhd rows with
 *                 batch and seq_len flattened); out may equal x (in place)
 *   cos_table, sin_table  device fp32 [max_positions, head_dim / 2]
 *   positions     device int32 [num_tokens]: each token's position, clamped to
 *                 [0, max_positions - 1] on the device
 * head_dim a multiple of 8 in [8, 256] (PDA_ERR_HEAD_DIM); x, out and the
 * tables 16-byte aligned, positions 4-byte aligned (PDA_ERR_ALIGN). */
pda_status pda_rope(const void *x, void *out, int64_t num_tokens, int32_t num_heads,
                    int32_t head_dim, const float *cos_table, const float *sin_table,
                    int32_t max_positions, const int32_t *positions, void *stream);

/* Rotary embedding fused with the paged-cache write of new tokens: token t's
 * K row is rotated as pda_rope does and stored, with its V row unchanged, at
 * slot positions[t] % block_size of page
 * block_tables[token_seq[t] * tile_capacity + positions[t] / block_size] of
 * the pools addressed with `strides` (the layouts of pda_decode).
 *   dims          num_kv_heads, head_dim, block_size, tile_capacity of the cache;
 *                 max_seqs bounds token_seq
 *   k_new, v_new  device bf16 [num_tokens, num_kv_heads, head_dim]
 *   token_seq     device int32 [num_tokens]: the sequence each token belongs to
 *   positions     device int32 [num_tokens]: its position in that sequence
 *   block_tables  device int32 [max_seqs, tile_capacity]
 *   k_pool, v_pool  device bf16 pools, written
 * A token whose sequence is outside [0, max_seqs), whose position is
 * negative or whose page index reaches tile_capacity is not written; the
 * cos/sin row is the position clamped to the table.  Device-side contract:
 * the page ids used address pages inside the pools, and no two tokens of a
 * call share a slot. */
pda_status pda_rope_append_kv(const pda_dims *dims, const void *k_new, const void *v_new,
                              int64_t num_tokens, const int32_t *token_seq,
                              const int32_t *positions, const float *cos_table,
                              const float *sin_table, int32_t max_positions,
                              const int32_t *block_tables, void *k_pool, void *v_pool,
                              pda_strides strides, void *stream);

/* Timing diagnostics, for benchmarks that need the attention kernel's own
 * duration: arms the calling thread's next pda_decode, pda_decode_masked,
 * pda_step_tile or pda_prefill call to record `before` and `after`
 * (hipEvent_t handles owned by the caller, passed as void*) on that call's
 * stream right before and right after its attention kernel, ahead of the
 * split merge.  The next call that launches
 * the attention kernel consumes the pair; NULL, NULL disarms.  PDA_ERR_NULL
 * if exactly one of them is NULL. */
pda_status pda_debug_time_attention(void *before, void *after);

/* Static name of a status code. */
const char *pda_status_string(pda_status status);

/* Details of the last failure on the calling thread ("" if none). */
const char *pda_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PDA_H */
