// Internal interface between the C-ABI host code (pda_api.hip) and the
// rotary-embedding kernels (pda_rope.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pda {

struct RopeArgs {
    const uint16_t *x;        // bf16 [T, H, D]: rows to rotate (new K rows for the append)
    uint16_t *out;            // bf16 [T, H, D] (rope; may equal x)
    const uint16_t *v_new;    // bf16 [T, H, D] (append: new V rows)
    uint16_t *k_pool, *v_pool;  // append: the paged cache pools
    const float *cos_t, *sin_t;  // fp32 [max_pos, D / 2]
    const int32_t *positions;    // int32 [T]
    const int32_t *token_seq;    // int32 [T] (append: each token's sequence)
    const int32_t *blocks;       // int32 [S, cap] (append: page lists)
    int64_t T;
    int64_t blk, tok, kvh;       // append: pool strides in bf16 elements
    int32_t H, D, max_pos, S, cap, bs;
};

hipError_t launch_rope(const RopeArgs &a, int cus, hipStream_t st);
hipError_t launch_rope_append_kv(const RopeArgs &a, int cus, hipStream_t st);

}  // namespace pda
