// Internal interface between the C-ABI host code (pda_api.hip) and the gfx950
// kernels (pda_attend.hip, pda_kernels.hip, pda_prefill.hip, pda_rope.hip).
// Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pda {

// Layout of the caller's decode workspace, in this order:
//   ctrl      256 bytes; ctrl[0] (64-bit) is the work-item counter
//   arrive    uint64 [max_seqs, units]: per (sequence, kv head + head chunk),
//             the number of its split items that have left their partials
//   part_ml   fp32 [max_seqs, Hq, nsplit, 2]: (m in log2 units, l) per split,
//             padded to a multiple of 16 bytes
//   part_o    fp32 [max_seqs, Hq, nsplit, D]
// The counters are 64-bit words (epoch << 32 | count): the high half names
// the launch that last counted in it (AttendArgs::epoch, unique per launch),
// and the first claim of a launch that finds another launch's epoch (or any
// leftover content) restarts the word at its own epoch.  So the workspace
// needs no clearing, before its first use or after a failed launch.
constexpr int kCtrlBytes = 256;

// Everything the attention kernel needs, passed by value.
struct AttendArgs {
    const uint16_t *q;        // bf16 [S, Hq, D]
    const uint16_t *k;        // bf16 K pool base
    const uint16_t *v;        // bf16 V pool base
    const int32_t *blocks;    // int32 [S, cap] page ids
    const int32_t *counts;    // int32 [S]
    const int32_t *lastv;     // int32 [S] or null
    unsigned long long *work;     // workspace: the work-item counter
    unsigned long long *arrive;   // workspace: arrival counters [S, units]
    float *part_ml;           // workspace partials
    float *part_o;
    uint16_t *out;            // bf16 [S, Hq, D] (decode) or null
    float *m, *l, *o;         // running state (tile) or null
    const uint8_t *mask;      // decode: kv keep-mask [S, mask_stride] (nonzero = keep) or null
    int64_t mask_stride;      // bytes per sequence row of the mask
    int64_t blk, tok, kvh;    // strides in bf16 elements
    uint64_t bs_magic;        // ceil(2^32 / bs): t / bs == (t * bs_magic) >> 32 for t < 2^24
    int32_t S, Hq, Hkv, G, D, bs, cap, bps, nhc, nsplit, lv_default;
    int32_t prefix_mode;      // 1: enumerate only non-empty splits (needs 2 (S + 1) ints of LDS)
    uint32_t epoch;           // this launch's counter epoch (never reused by a recent launch)
    int32_t restart;          // 1: a launch that makes claims restarts the counters after its
                              // enumeration (0 only to test the claims' own restart:
                              // PDA_DEBUG_NO_COUNTER_RESTART set)
    float scale_log2;         // log2(e) / sqrt(D)
};

// Choices the host makes before launching.
struct Plan {
    int dp;     // padded head dim: 64, 128 or 256
    int nhc;    // head chunks per kv head: ceil(G / kHeadsPerItem)
    bool p16;   // block_size % 16 == 0: every 16-token group lies inside one page
};

// q heads of one kv head that a decode work item takes (the columns of the
// matrix-core products).
constexpr int kHeadsPerItem = 16;

Plan choose_plan(int G, int D, int bs);

// Sequences up to this count enumerate work items through LDS prefix sums
// (3 (S + 1) ints next to the kernel's V tiles, up to 37 KB, within gfx950's
// 160 KB of LDS per workgroup).
constexpr int kPrefixMaxSeqs = 10240;

// Work-item sizing with the prefix enumeration (decided in the attention
// kernel from the total work): with at least kBigTokensLarge tokens of work
// per wave, "big" items span kBigTokensLarge tokens (at least one split) and
// take kEighthsLarge / 8 of a sequence's splits; with less, every split is an
// item of its own when that makes no more items than waves (one round, equal
// lengths); failing that, splits of as many pages as a bound on the item
// count says make no more items than waves, if that is at most kWidenMax
// times the launch's pages per split; failing that too, kEighthsPaired / 8 of
// the splits go in
// pairs (measured on MI355X for batch 16, contexts 512-4096, 256-token
// splits: 0, 2, 4, 6, 7, 8 eighths paired gave 54.6, 51.6, 47.7, 44.4, 43.3,
// 43.7 us per step; fewer, longer items keep HBM as busy and leave shorter
// merges; the same batch with one round of 304- to 416-token splits took
// 35.2-36.8 us against 39.4 paired).
constexpr int kBigTokensLarge = 1024;
constexpr int kEighthsLarge = 7;
constexpr int kEighthsPaired = 7;
constexpr int kWidenMax = 2;
// With at least kBigTokensLarge tokens of work per wave, the splits that a
// sequence with big items has left go kSinglesLarge at a time (the last item
// takes what remains): measured on MI355X, items of 512 tokens there beat 256
// (fewer items and partial slots per sequence, so shorter merges), while the
// short sequences that end the queue keep one split per item.
constexpr int kSinglesLarge = 2;

// Optional events recorded on the launch stream right before and right after
// the attention kernel (timing diagnostics); null members are skipped.
struct AttendEvents {
    hipEvent_t before = nullptr;
    hipEvent_t after = nullptr;
};

// Launches the persistent decode attention kernel (decode when a.out is set,
// else a tile folded into the running state); the split merge runs inside it.
// `cus` is the device's compute-unit count.
hipError_t launch_attend(const Plan &p, const AttendArgs &a, int cus, hipStream_t st,
                         const AttendEvents &ev);

// Prefill: a chunk of Q query tokens per sequence (the sequence's newest
// tokens), rows (i, h) of kv head g ordered r = i G + (h - g G).
struct PrefillArgs {
    const uint16_t *q;        // bf16 [S, Q, Hq, D]
    const uint16_t *k;        // bf16 K pool base
    const uint16_t *v;        // bf16 V pool base
    const int32_t *blocks;    // int32 [S, cap] page ids
    const int32_t *counts;    // int32 [S]
    const int32_t *lastv;     // int32 [S] or null
    const uint8_t *mask;      // keep-mask, byte (s, i, t) at s mask_ss + i mask_qs + t, or null
    int64_t mask_ss, mask_qs;
    uint16_t *out;            // bf16 [S, Q, Hq, D]
    float *part_ml;           // fp32 [S Q Hq, nsplit, 2]: (m in log2 units, l) per split
    float *part_o;            // fp32 [S Q Hq, nsplit, D]
    int64_t blk, tok, kvh;    // strides in bf16 elements
    uint64_t bs_magic;        // ceil(2^32 / bs)
    int32_t S, Q, Hq, Hkv, G, D, bs, cap, lv_default;
    int32_t span;             // tokens per kv split (a whole number of pages)
    int32_t nsplit;           // split slots per sequence: ceil(cap bs / span)
    int32_t ntiles;           // row tiles per kv head: ceil(Q G / (16 rb))
    int32_t causal;
    int32_t cus;              // the device's compute units
    int32_t longest_first;    // set by the launcher: rank units by length (more workgroups than fit at once)
    float scale_log2;         // log2(e) / sqrt(D)
};

// dp: padded head dim (64, 128, 256); rb: 16-row blocks per wave (1, 2, 4,
// at most prefill_max_rb(dp, with a mask)).  Launches the attention kernel,
// then the split merge when nsplit > 1.
int prefill_max_rb(int dp, bool mask);
hipError_t launch_prefill(const PrefillArgs &a, int dp, int rb, hipStream_t st, const AttendEvents &ev);
hipError_t launch_reset(float *m, float *l, float *o, int64_t rows, int D, hipStream_t st);
hipError_t launch_finalize(const float *l, const float *o, uint16_t *out, int64_t rows, int D,
                           hipStream_t st);


}  // namespace pda
