// Internal interface between the C-ABI host code (pda_api.hip) and the gfx950
// kernels (pda_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pda {

// Everything the split-KV partial kernel needs, passed by value.
struct PartialArgs {
    const uint16_t *q;        // bf16 [S, Hq, D]
    const uint16_t *k;        // bf16 K pool base
    const uint16_t *v;        // bf16 V pool base
    const int32_t *blocks;    // int32 [S, cap] page ids
    const int32_t *counts;    // int32 [S]
    const int32_t *lastv;     // int32 [S] or null
    float *part_ml;           // fp32 [S, Hq, nsplit, 2]: (m in log2 units, l)
    float *part_o;            // fp32 [S, Hq, nsplit, D]
    int64_t blk, tok, kvh;    // strides in bf16 elements
    uint64_t bs_magic;        // ceil(2^32 / bs): t / bs == (t * bs_magic) >> 32 for t < 2^24
    int32_t Hq, Hkv, G, D, bs, cap, bps, nhc, nsplit, lv_default;
    float scale_log2;         // log2(e) / sqrt(D)
};

// Merge of split partials: into the output (decode) or into the state (tile).
struct CombineArgs {
    const int32_t *counts;
    const int32_t *lastv;
    const float *part_ml;
    const float *part_o;
    float *m, *l, *o;         // state (tile merge) or null
    uint16_t *out;            // bf16 output (decode) or null
    int32_t S, Hq, D, bs, cap, bps, nsplit, lv_default;
};

// Choices the host makes before launching.
struct Plan {
    int dp;     // padded head dim: 64, 128 or 256
    int gc;     // q heads per workgroup: 1, 2, 4 or 8
    int nhc;    // head chunks per kv head: ceil(G / gc)
    bool p16;   // block_size % 16 == 0: every 16-token group lies inside one page
};

Plan choose_plan(int G, int D, int bs);

hipError_t launch_partial(const Plan &p, const PartialArgs &a, int S, hipStream_t st);
hipError_t launch_combine(const CombineArgs &a, int dp, hipStream_t st);
hipError_t launch_reset(float *m, float *l, float *o, int64_t rows, int D, hipStream_t st);
hipError_t launch_finalize(const float *l, const float *o, uint16_t *out, int64_t rows, int D,
                           hipStream_t st);

}  // namespace pda
