// gfx950 (CDNA4) persistent decode attention, both products on the matrix
// cores, with the split-KV merge inside the same launch.
//
// The operation: for each sequence s and q head h, the single query
// q[s, h, :] attends over the tokens the sequence's page list names, scale
// 1/sqrt(head_dim) (AstrAI "CUDA Kernels", section "Python Wrappers"), with
// the online-softmax (m, l, o) state of the spark_storage "tiled_attention.rs"
// page (header comment: reset, one launch per tile, finalize as o / l) and
// split-KV partials merged by log-sum-exp (the "Overview" table of the AstrAI
// page: GQA decode with split-KV, paged KV-cache decode, tensor-core MMA
// variants).
//
// Work items are (sequence, split, kv head + head chunk), kv head fastest, so
// the waves reading one page's interleaved kv-head rows run together.  Every
// wave takes items from one launch-tagged atomic counter on its own and
// streams its items' 16-token groups as one stream with NBUF - 1 groups in
// flight (the next item's first groups are requested during the current
// item's last round).  A sequence whose tokens fit one split gets its result
// directly (bf16 o / l for decode, folded into the running state for a
// tile); otherwise each item leaves an (m, l, o) partial in its slot and
// counts its arrival on its unit's launch-tagged counter, and the item that
// arrives last merges the unit's slots in token order (the ticket decides who
// merges, never the order).  Per group:
//   scores, transposed: S^T (16 tokens x 16 heads) = K (A operand, the 16 K
//      rows as loaded: lane l holds token l%16, elements 32 c + 8 (l/16) ..
//      + 8) x Q^T (B operand, the item's q heads, up to 16, the rest zero),
//      v_mfma_f32_16x16x32_bf16 x D/32.  Lane l receives head l%16 and tokens
//      4 (l/16) + i, i = 0..3.
//   online softmax per head in base 2: the lane's four tokens, then the four
//      lanes of a head (l, l^16, l^32, l^48) through gfx950 lane swaps; the
//      running max and the accumulator rescale of a head never leave its
//      lanes.  The weights, in exactly the B-operand layout of the next
//      product (head l%16, tokens 4 (l/16) .. + 3), are split into a bf16
//      pair p = hi + lo (|p - hi - lo| <= 2^-18 p), so the product carries
//      the fp32 weights' precision.
//   P.V, transposed: O^T (16 head-dim elements x 16 heads) += V^T (A operand)
//      x P^T (B operand), 16 tokens deep, v_mfma_f32_16x16x16_bf16 twice (hi,
//      lo) per 16-element block of the head dim.  V is loaded 16 bytes per
//      lane (whole 16-byte chunks of whole rows), written to LDS row-major
//      and read back transposed with ds_read_b64_tr_b16, which hands lane
//      (q, c) column 16 n + c of tokens 4 q .. + 3.  Lane l accumulates head
//      l%16, elements 16 n + 4 (l/16) + i.
// So no weight goes through LDS and the VALU work per group is the softmax
// of four scores per lane and the weight split: one wave streams a group in
// far fewer instructions than with fp32 P.V on the VALU, which shortens the
// launch's tail (a few waves finishing their last items) and the small
// batches bound by one wave's rate.
#include "pda_internal.h"
#include "pda_device.h"

namespace pda {
namespace {

constexpr int kMWaves = 4;
constexpr int kMThreads = 64 * kMWaves;

// Scores on the VALU (v_dot2c_f32_bf16) instead of the matrix cores, for
// items of up to kValuScoreHeads q heads: the measured alternative to the
// MFMA score product, kept buildable for that comparison (off: the kernel
// computes every score on the matrix cores).
constexpr bool kValuScores = false;
constexpr int kValuScoreHeads = 4;

typedef __bf16 bf16x8_m __attribute__((ext_vector_type(8)));
typedef float f32x4_m __attribute__((ext_vector_type(4)));
typedef short i16x4_m __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_m lds_i16x4_m;
typedef __attribute__((address_space(3))) unsigned char lds_u8_m;

template <int DP>
struct MShape {
    static constexpr int NCK = DP / 32;        // 32-element chunks of the head dim (score products)
    static constexpr int NDB = DP / 16;        // 16-element blocks of the head dim (output products)
    static constexpr int CPR = DP / 8;         // 16-byte chunks per V row
    static constexpr int RPI = 64 / CPR;       // V rows per load instruction: 8, 4, 2
    static constexpr int NV = 16 / RPI;        // V load instructions per 16-token group: 2, 4, 8
    // LDS bytes per V row: 32 bytes of padding start each row an odd multiple
    // of 8 banks after the previous one, so the 16 rows a transposing read
    // touches (32 bytes each) take disjoint bank groups.
    static constexpr int PITCH = 2 * DP + 32;
    static constexpr int TILE = 16 * PITCH;    // one group's V tile
    static constexpr int NTB = DP <= 128 ? 2 : 1;   // tiles per wave (double-buffered by group parity)
};

// Registers of one 16-token group in flight.
template <int DP>
struct MGroup {
    u32x4 k[MShape<DP>::NCK];   // K: token lane%16, elements 32 c + 8 (lane/16) .. + 8
    u32x4 v[MShape<DP>::NV];    // V: token RPI i + lane / CPR, elements 8 (lane % CPR) .. + 8
    uint32_t keep;              // with a kv mask: the mask byte of token lane%16
    uint64_t kept;              // with a kv mask: bit t set when token t takes part
};

// One work item as a wave holds it (everything wave-uniform except bidvec and q).
template <int DP>
struct MItem {
    int kind;        // 0: attend tokens [t0, t1); 1: zero the decode output rows; 2: nothing
    int s, g, unit, h0, nh, split, nspl, slot;
    int cnt, t0, t1, ng, nsp;
    int cb;          // first page (index into the sequence's list) of the page-id window
    int bidvec;      // the window: lane i holds the id of page cb + i
    u32x4 q[MShape<DP>::NCK];   // B operand: head lane%16, elements 32 c + 8 (lane/16) .. + 8
    // VALU scores: q heads 0 .. kValuScoreHeads - 1 of the item, elements
    // 32 c + 8 (lane/16) .. + 8 (the K elements the lane holds)
    u32x4 qv[kValuScores ? kValuScoreHeads : 1][kValuScores ? MShape<DP>::NCK : 1];
};

// One claim on a launch-tagged counter (epoch << 32 | count), made by one
// lane: returns the count before this claim within launch `epoch`.  A word
// that holds another launch's epoch (or anything else) is restarted at this
// epoch, with this claim as its first, by a compare-and-swap against the
// value the claim saw; a claim that loses that race to another claim of the
// launch counts on the restarted word.  Counts within a launch are therefore
// 0, 1, 2, ... whatever the word held before the launch.
// epoch_claim_after takes over from a fetch-and-add of 1 that returned v.
__device__ __forceinline__ uint32_t epoch_claim_after(unsigned long long *p, uint32_t epoch, unsigned long long v) {
    for (;;) {
        if ((uint32_t)(v >> 32) == epoch) return (uint32_t)v;
        unsigned long long cur = v + 1;   // the word right after this claim's add
        for (;;) {
            if ((uint32_t)(cur >> 32) == epoch) break;   // restarted by another claim
            unsigned long long expected = cur;
            if (__hip_atomic_compare_exchange_strong(p, &expected, ((unsigned long long)epoch << 32) | 1ull,
                                                     __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT))
                return 0;
            cur = expected;
        }
        v = __hip_atomic_fetch_add(p, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}
__device__ __forceinline__ uint32_t epoch_claim(unsigned long long *p, uint32_t epoch) {
    return epoch_claim_after(p, epoch, __hip_atomic_fetch_add(p, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Restarts a counter at this launch's epoch with count 0 unless it already
// holds this epoch (a later claim of the launch may have restarted it:
// the compare-and-swap against the other epoch's value then fails, and
// changes nothing).  The result is not waited for.
__device__ __forceinline__ void epoch_restart(unsigned long long *p, uint32_t epoch) {
    unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(v >> 32) != epoch)
        __hip_atomic_compare_exchange_strong(p, &v, (unsigned long long)epoch << 32, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The split partials travel between waves of different XCDs, whose L2
// caches are not coherent with each other.  They are written with
// device-scope stores (gfx950: sc1, written through to the device coherence
// point) and read with device-scope loads (sc1, served from that point), so
// neither side needs a whole-cache write-back or invalidate (an agent-scope
// fence would do one of those per item).
__device__ __forceinline__ void st_dev2(float *p, float x, float y) {
    const unsigned long long v = (unsigned long long)__float_as_uint(x) | ((unsigned long long)__float_as_uint(y) << 32);
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ld_dev2(const float *p, float &x, float &y) {
    const unsigned long long v = __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    x = __uint_as_float((uint32_t)v);
    y = __uint_as_float((uint32_t)(v >> 32));
}
// 16-byte device-scope accesses through a buffer resource over one unit's
// partial rows (gfx950 buffer_load/store_dwordx4 with sc1; cache policy 16 is
// sc1 on this target).  Word 3 of the resource selects 32-bit elements, as
// every gfx9-family resource for raw byte-offset access; an offset past
// num_records reads zero and writes nothing.
constexpr int kBufWord3 = 0x00020000;
constexpr int kPolicySc1 = 16;
// The base and size are wave-uniform; they are read into scalars here so the
// resource lives in SGPRs (a resource in VGPRs makes the compiler wrap every
// access in a loop over its distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t unit_rsrc(const float *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    float *ub = reinterpret_cast<float *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, 0, (int)__builtin_amdgcn_readfirstlane(bytes), kBufWord3);
}
__device__ __forceinline__ f32x4_m ld_dev4b(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4_m, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicySc1));
}
__device__ __forceinline__ void st_dev4b(__amdgpu_buffer_rsrc_t r, uint32_t off, const f32x4_m &x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, kPolicySc1);
}

template <int DP, bool P16, int NBUF, bool TILE, bool MASK>
__global__ void __launch_bounds__(kMThreads) attend_kernel(const AttendArgs a) {
    using SH = MShape<DP>;
    constexpr int NCK = SH::NCK, NDB = SH::NDB, CPR = SH::CPR, RPI = SH::RPI, NV = SH::NV;
    constexpr int PITCH = SH::PITCH;
    constexpr int HPI = kHeadsPerItem;   // q heads per work item (MFMA columns)
    static_assert(HPI == 16, "the products' columns are 16 q heads");
    static_assert(NBUF >= 2, "at least 2 ring slots");

    __shared__ __attribute__((aligned(16))) unsigned char vt_all[kMWaves][SH::NTB][SH::TILE];
    __shared__ int scan[3 * kMWaves];
    __shared__ float vsc_all[kValuScores ? kMWaves : 1][kValuScores ? 256 : 1];   // VALU scores: [token][head]
    __shared__ float wsum_f[2 * kMWaves];
    extern __shared__ int prefix[];   // 3 (S + 1) ints when a.prefix_mode

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int units = a.Hkv * a.nhc;
    // pages and tokens per split: the launch's, or longer ones chosen below
    int bpsx = a.bps, span = a.bps * a.bs;
    const int qd = lane >> 4, col = lane & 15;


    // Work items.  With the prefix (up to kPrefixMaxSeqs sequences), each
    // sequence's splits are grouped: a share of them, `big` at a time, form
    // "big" items queued first; the rest (the "single" items: one split, or,
    // for sequences with big items when the work is large, `sgl` splits) are
    // queued after all big ones, so the queue ends with short work.  The single items of
    // sequences that also have big items (long sequences, whose merges take
    // many slots) come before those of the others, so that the launch ends
    // with items whose merges are short.  Decode keeps one small item for an
    // empty sequence so that its zero output row gets written.
    int nbig_pairs = 0, nlong_pairs = 0, npairs;
    int *pbig = prefix;                  // big items before sequence s
    int *plong = prefix + a.S + 1;       // single items of sequences with big items, before s
    int *pshort = prefix + 2 * (a.S + 1);   // single items of the others, before s
    const int nsp_max = (a.cap + a.bps - 1) / a.bps;
    int big = 1, eighths = 0, sgl = 1;
    if (a.prefix_mode) {
        // Sizing (every workgroup takes the same decision from the same
        // totals): with at least kBigTokensLarge tokens of work per wave, big
        // items span kBigTokensLarge tokens and take kEighthsLarge / 8 of the
        // splits; with less, every split is an item as long as there are no
        // more split items than waves (one round, equal lengths), else
        // longer splits (up to kWidenMax times the launch's) if some make no
        // more items than waves, else
        // kEighthsPaired / 8 of the splits go in pairs.  Splits only grow,
        // so a sequence never has more items than partial slots.
        float tot = 0.f, nspl = 0.f;
        for (int s = tid; s < a.S; s += kMThreads) {
            const int nt = seq_tokens(a.counts, a.lastv, a.lv_default, s, a.cap, a.bs);
            pshort[s + 1] = nt;   // kept for the scan below
            tot += (float)nt;
            nspl += (float)splits_of(nt, span);
        }
        tot = wave_sum(tot);
        nspl = wave_sum(nspl);
        if (lane == 0) {
            wsum_f[w] = tot;
            wsum_f[kMWaves + w] = nspl;
        }
        __syncthreads();
        tot = 0.f;
        nspl = 0.f;
        for (int ww = 0; ww < kMWaves; ++ww) {
            tot += wsum_f[ww];
            nspl += wsum_f[kMWaves + ww];
        }
        const float waves = (float)((int)gridDim.x * kMWaves);
        if (tot * (float)units >= (float)kBigTokensLarge * waves) {
            big = max(1, kBigTokensLarge / span);
            eighths = kEighthsLarge;
            sgl = kSinglesLarge;
        } else if (nspl * (float)units > waves) {
            // A sequence of n tokens makes at most n / L + 1 items of L
            // tokens (an empty one makes one), so L >= tot / (waves / units
            // - S) makes no more items than waves; the fewest pages that
            // reach that bound, if no more than kWidenMax times the launch's.
            const float room = waves / (float)units - (float)a.S;
            const float need = room >= 1.f ? ceilf(tot / (room * (float)a.bs)) : 3e9f;
            if (need <= (float)(kWidenMax * a.bps)) {
                bpsx = max(a.bps + 1, (int)need);
                span = bpsx * a.bs;
                big = 1;
                eighths = 0;
            } else {
                big = 2;
                eighths = kEighthsPaired;
            }
        } else {
            big = 1;
            eighths = 0;
        }
        int carry_b = 0, carry_l = 0, carry_s = 0;
        for (int base = 0; base < a.S; base += kMThreads) {
            const int s = base + tid;
            int nb = 0, nl = 0, ns = 0;
            if (s < a.S) {
                const int nsp = splits_of(pshort[s + 1], span);
                nb = big_items_of(nsp, big, eighths);
                const int sg = nb > 0 ? sgl : 1;   // only long sequences pair their singles
                ns = (nsp - nb * big + sg - 1) / sg;
                if (!TILE && nsp == 0) ns = 1;
                if (nb > 0) {
                    nl = ns;
                    ns = 0;
                }
            }
            // inclusive scan over the wave's lanes that hold sequences (the
            // first nsw): offsets below nsw only, the total in lane nsw - 1
            const int nsw = min(64, a.S - base - 64 * w);
            int xb = nb, xl = nl, xs = ns;
            for (int off = 1; off < nsw; off <<= 1) {
                const int yb = __shfl_up(xb, off, 64);
                const int yl = __shfl_up(xl, off, 64);
                const int ys = __shfl_up(xs, off, 64);
                if (lane >= off) {
                    xb += yb;
                    xl += yl;
                    xs += ys;
                }
            }
            if (lane == (nsw > 0 ? nsw - 1 : 0)) {
                scan[w] = xb;
                scan[kMWaves + w] = xl;
                scan[2 * kMWaves + w] = xs;
            }
            __syncthreads();
            int wb = 0, wl = 0, wsum = 0;
            for (int ww = 0; ww < w; ++ww) {
                wb += scan[ww];
                wl += scan[kMWaves + ww];
                wsum += scan[2 * kMWaves + ww];
            }
            if (s < a.S) {
                pbig[s + 1] = carry_b + wb + xb;
                plong[s + 1] = carry_l + wl + xl;
                pshort[s + 1] = carry_s + wsum + xs;
            }
            for (int ww = 0; ww < kMWaves; ++ww) {
                carry_b += scan[ww];
                carry_l += scan[kMWaves + ww];
                carry_s += scan[2 * kMWaves + ww];
            }
            __syncthreads();
        }
        if (tid == 0) {
            pbig[0] = 0;
            plong[0] = 0;
            pshort[0] = 0;
        }
        nbig_pairs = __builtin_amdgcn_readfirstlane(carry_b);
        nlong_pairs = __builtin_amdgcn_readfirstlane(carry_l);
        npairs = nbig_pairs + nlong_pairs + __builtin_amdgcn_readfirstlane(carry_s);
    } else {
        npairs = a.S * nsp_max;
    }
    const int nitems = npairs * units;
    __syncthreads();

    const int nwaves = (int)gridDim.x * kMWaves;
    // A launch that makes claims restarts its counters at its epoch before
    // its first items end, so that claims and arrival counts take the
    // one-atomic path: the waves claiming after their first items would
    // otherwise contend for the compare-and-swap that restarts a word found
    // with another launch's epoch (measured: 7 % of a step on ragged batches).
    // Without claims, the few arrivals on each word restart it themselves,
    // and the pass's round trips are saved.  Either order of a restart and a
    // claim or arrival on a word is correct (epoch_restart changes only a word
    // of another epoch).
    if (a.restart && nitems > nwaves) {
        const int64_t gsize = (int64_t)gridDim.x * kMThreads;
        const int64_t gtid = (int64_t)blockIdx.x * kMThreads + tid;
        if (gtid == 0) epoch_restart(a.work, a.epoch);
        for (int64_t i = gtid; i < (int64_t)a.S * units; i += gsize) epoch_restart(a.arrive + i, a.epoch);
    }
    const int tok32 = (int)a.tok;
    const int32_t *lv_src = a.lastv ? a.lastv : a.counts;

    // Lane-invariant offsets.  K chunks past head_dim re-read chunk 0 of the
    // same row (q is zero there); V chunks past head_dim re-read chunk 0 (in
    // bounds) and land in LDS columns whose output rows are never stored.
    int kd[NCK];
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
        const int d0 = 32 * c + 8 * qd;
        kd[c] = d0 < a.D ? d0 : 0;
    }
    const int vrow = lane / CPR;              // V row within a load instruction
    const int vch = lane % CPR;               // V 16-byte chunk of the lane
    const int vofs = 8 * vch < a.D ? 8 * vch : 0;
    const int vlane = vrow * tok32 + vofs;
    unsigned char *vt = &vt_all[w][0][0];
    lds_u8_m *vt_lds = (lds_u8_m *)&vt_all[0][0][0] + w * (SH::NTB * SH::TILE);
    // transposing read: lane (qd, c) points at row 4 qd + c/4, elements 4 (c%4) .. + 3 of a block
    const uint32_t tr_off = (uint32_t)((4 * qd + (col >> 2)) * PITCH + 8 * (col & 3));
    const uint32_t wr_off = (uint32_t)(vrow * PITCH + 16 * vch);

    auto locate = [&](int it, MItem<DP> &x) {
        x.kind = it < nitems ? 0 : 2;
        if (it >= nitems) it = 0;
        int pair = it / units;
        const int unit = it - pair * units;
        if (a.prefix_mode) {
            const bool is_big = pair < nbig_pairs;
            const bool is_long = !is_big && pair < nbig_pairs + nlong_pairs;
            // the array by index, not by a select of pointers (a select among
            // three LDS pointers makes the compiler keep the kernel's
            // arguments in private memory and address through flat pointers)
            const int *pf = prefix + (is_big ? 0 : (is_long ? a.S + 1 : 2 * (a.S + 1)));
            if (!is_big) pair -= is_long ? nbig_pairs : nbig_pairs + nlong_pairs;
            int lo = 0, hi = a.S;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (pf[mid] <= pair) lo = mid;
                else hi = mid;
            }
            x.s = __builtin_amdgcn_readfirstlane(lo);
            const int j = pair - __builtin_amdgcn_readfirstlane(pf[x.s]);
            if (is_big) {
                x.split = j * big;
                x.nspl = big;
                x.slot = j;
            } else {
                const int nb_s = __builtin_amdgcn_readfirstlane(pbig[x.s + 1] - pbig[x.s]);
                const int sg = is_long ? sgl : 1;
                x.split = nb_s * big + j * sg;
                x.nspl = sg;
                x.slot = nb_s + j;
            }
        } else {
            x.s = pair / nsp_max;
            x.split = pair - x.s * nsp_max;
            x.nspl = 1;
            x.slot = x.split;
        }
        x.unit = unit;
        x.g = unit / a.nhc;
        const int hc = unit - x.g * a.nhc;
        x.h0 = x.g * a.G + hc * HPI;
        x.nh = min(HPI, a.G - hc * HPI);
        x.cb = x.split * bpsx;
    };

    auto fetch = [&](MItem<DP> &x, int &cnt_raw, int &lv_raw) {
        cnt_raw = a.counts[x.s];
        lv_raw = lv_src[x.s];
        const uint16_t *qp = a.q + ((int64_t)x.s * a.Hq + x.h0 + min(col, x.nh - 1)) * a.D;
#pragma unroll
        for (int c = 0; c < NCK; ++c) x.q[c] = ld16(qp + kd[c]);
        if constexpr (kValuScores) {
#pragma unroll
            for (int h = 0; h < kValuScoreHeads; ++h) {
                const uint16_t *qh = a.q + ((int64_t)x.s * a.Hq + x.h0 + min(h, x.nh - 1)) * a.D;
#pragma unroll
                for (int c = 0; c < NCK; ++c) x.qv[h][c] = ld16(qh + kd[c]);
            }
        }
        x.bidvec = a.blocks[(int64_t)x.s * a.cap + min(x.cb + lane, a.cap - 1)];
    };

    auto resolve = [&](MItem<DP> &x, int cnt_raw, int lv_raw) {
        x.t0 = x.t1 = x.ng = 0;
        x.cnt = clampi(__builtin_amdgcn_readfirstlane(cnt_raw), 0, a.cap);
        const int lv = clampi(a.lastv ? __builtin_amdgcn_readfirstlane(lv_raw) : a.lv_default, 0, a.bs);
        const int ntok = x.cnt > 0 ? (x.cnt - 1) * a.bs + lv : 0;
        x.nsp = splits_of(ntok, span);
#pragma unroll
        for (int c = 0; c < NCK; ++c)
            x.q[c] = (col < x.nh && 32 * c + 8 * qd < a.D) ? x.q[c] : u32x4{0, 0, 0, 0};
        if constexpr (kValuScores) {
#pragma unroll
            for (int h = 0; h < kValuScoreHeads; ++h)
#pragma unroll
                for (int c = 0; c < NCK; ++c)
                    x.qv[h][c] = (32 * c + 8 * qd < a.D) ? x.qv[h][c] : u32x4{0, 0, 0, 0};
        }
        if (x.kind != 0) return;
        if (ntok == 0) {
            x.kind = (!TILE && (a.prefix_mode || x.split == 0)) ? 1 : 2;
            return;
        }
        if (x.split >= x.nsp) {
            x.kind = 2;
            return;
        }
        x.t0 = x.split * span;
        x.t1 = min(x.t0 + x.nspl * span, ntok);
        x.ng = (x.t1 - x.t0 + 15) >> 4;
    };

    // Items past the first wave's-worth come from the work counter; when
    // there are no more items than waves, every wave's first item is its
    // last and no claim is made (a claim is an atomic on one word: a
    // thousand of them at once, as at the end of a one-round launch, queue
    // for microseconds).
    const bool claims = nitems > nwaves;
    auto claim_next = [&]() {
        if (!claims) return nitems;
        const int grabbed = lane == 0 ? (int)epoch_claim(a.work, a.epoch) : 0;
        return nwaves + readlane(grabbed, 0);
    };

    auto zero_rows = [&](const MItem<DP> &x) {
        const int64_t row0 = (int64_t)x.s * a.Hq + x.h0;
        for (int idx = lane; idx < x.nh * a.D; idx += 64) a.out[row0 * a.D + idx] = 0;
    };

    auto take_sync = [&](int it, MItem<DP> &x) {
        for (;;) {
            int cr, lr;
            locate(it, x);
            fetch(x, cr, lr);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            resolve(x, cr, lr);
            if (x.kind == 0 || it >= nitems) return;
            if (x.kind == 1) zero_rows(x);
            it = claim_next();
        }
    };

    // Loads of group n of item x (indices past the last group re-read it: in
    // bounds, never computed).
    auto issue = [&](MItem<DP> &x, int n, MGroup<DP> &r) {
        n = min(n, x.ng - 1);
        const int gs = x.t0 + 16 * n;
        const int64_t gk = (int64_t)x.g * a.kvh;
        const int32_t *brow = a.blocks + (int64_t)x.s * a.cap;
        if constexpr (P16) {
            const int page = page_of((uint32_t)gs, a.bs_magic);
            if (page - x.cb >= 64) {   // move the window (at most once per 64 pages)
                x.cb = page;
                x.bidvec = brow[min(page + lane, x.cnt - 1)];
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
            const int bid = readlane(x.bidvec, page - x.cb);
            const int64_t off = (int64_t)bid * a.blk + gk + (int64_t)(gs - page * a.bs) * a.tok;
            const uint16_t *kb = a.k + off;
            const uint16_t *vb = a.v + off;
#pragma unroll
            for (int c = 0; c < NCK; ++c) r.k[c] = ld16(kb + (col * tok32 + kd[c]));
            if constexpr (MASK) {
                const int tk = gs + col < x.t1 ? gs + col : gs;
                r.keep = a.mask[(int64_t)x.s * a.mask_stride + tk];
            }
#pragma unroll
            for (int i = 0; i < NV; ++i)
                r.v[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(vb + (int64_t)(RPI * i) * a.tok + vlane));
        } else {
            const int last = min(gs + 15, x.t1 - 1);
            if (page_of((uint32_t)last, a.bs_magic) - x.cb >= 64) {
                x.cb = page_of((uint32_t)gs, a.bs_magic);
                x.bidvec = brow[min(x.cb + lane, x.cnt - 1)];
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
            const int tk = gs + col < x.t1 ? gs + col : gs;
            const int pk = page_of((uint32_t)tk, a.bs_magic);
            const int bk = __shfl(x.bidvec, pk - x.cb, 64);
            const uint16_t *kp = a.k + ((int64_t)bk * a.blk + gk + (int64_t)(tk - pk * a.bs) * a.tok);
#pragma unroll
            for (int c = 0; c < NCK; ++c) r.k[c] = ld16(kp + kd[c]);
            if constexpr (MASK) r.keep = a.mask[(int64_t)x.s * a.mask_stride + tk];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int tv = gs + RPI * i + vrow < x.t1 ? gs + RPI * i + vrow : gs;
                const int pv = page_of((uint32_t)tv, a.bs_magic);
                const int bv = __shfl(x.bidvec, pv - x.cb, 64);
                const uint16_t *vp = a.v + ((int64_t)bv * a.blk + gk + (int64_t)(tv - pv * a.bs) * a.tok);
                r.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + vofs));
            }
        }
    };

    float m2;            // running max of the lane's head (base 2), the same in its four lanes
    float ls;            // running sum of the lane's own token weights
    f32x4_m acc[NDB];    // O^T blocks: head col, elements 16 n + 4 qd + i

    // Per group, two stages, software-pipelined across groups: scores(g + 1)
    // (MFMA, online max, weights) runs next to pv(g) (V into LDS, transposed
    // reads, MFMA), and the rescale of the accumulators by the max change of
    // group g + 1 follows pv(g).
    bool grow_next = false;     // wave-uniform
    float alpha_next = 1.f;     // per lane (its head)
    // weights as bf16 pairs (tokens 4 qd .. + 3 of head col): those of the
    // group pv() consumes, and those scores() just produced
    u32x2 pw_hi = {0u, 0u}, pw_lo = {0u, 0u}, pn_hi = {0u, 0u}, pn_lo = {0u, 0u};

    auto scores = [&](const MItem<DP> &x, MGroup<DP> &r, int n) {
        const int gs = x.t0 + 16 * n;
        f32x4_m sacc = {0.f, 0.f, 0.f, 0.f};
        bool valu = false;
        if constexpr (kValuScores) valu = x.nh <= kValuScoreHeads;
        if constexpr (kValuScores) if (valu) {
            // lane (t, qd) = (lane % 16, lane / 16): the dot products of its
            // quarter of K row t with the same quarter of each q head, summed
            // over the four quarters' lanes, then transposed through LDS to
            // the product's layout (lane: head lane % 16, tokens 4 qd + i)
            float part[kValuScoreHeads];
#pragma unroll
            for (int h = 0; h < kValuScoreHeads; ++h) {
                part[h] = 0.f;
#pragma unroll
                for (int c = 0; c < NCK; ++c)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // the elements go through scalars: a bit cast of a
                        // vector element indexed in an unrolled loop compiles
                        // to element 0 every time (seen with this hipcc)
                        const uint32_t kk = r.k[c][j], qq = x.qv[h][c][j];
                        part[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kk),
                                                                 __builtin_bit_cast(bf16x2, qq), part[h], false);
                    }
                part[h] = sum4(part[h]);
            }
            float *vs = &vsc_all[kValuScores ? w : 0][0];
            if (qd == 0) {
#pragma unroll
                for (int h = 0; h < kValuScoreHeads; ++h) vs[col * 16 + h] = part[h];
            }
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[i] = col < kValuScoreHeads ? vs[(4 * qd + i) * 16 + col] : 0.f;
            wave_lds_sync();
        }
        if (!valu) {
#pragma unroll
            for (int c = 0; c < NCK; ++c)
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_m, r.k[c]),
                                                               __builtin_bit_cast(bf16x8_m, x.q[c]), sacc, 0, 0, 0);
        }
        // token validity: bit t of `ok` set when token gs + t takes part
        uint32_t okbits;
        if constexpr (MASK) {
            const bool valid = gs + col < x.t1 && r.keep != 0;
            r.kept = __builtin_amdgcn_ballot_w64(valid);
            okbits = (uint32_t)r.kept & 0xffffu;
        } else {
            const int nvalid = x.t1 - gs;   // >= 1
            okbits = nvalid >= 16 ? 0xffffu : ((1u << nvalid) - 1u);
        }
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sc[i] = ((okbits >> (4 * qd + i)) & 1u) ? sacc[i] * a.scale_log2 : -INFINITY;
        const float mx = max4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
        const float mn = fmaxf(m2, mx);
        const bool grow = mn > m2;
        alpha_next = grow ? exp2_fast(m2 - mn) : 1.f;   // mn is finite when grow
        m2 = mn;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = ((okbits >> (4 * qd + i)) & 1u) ? exp2_fast(sc[i] - mn) : 0.f;
        ls = fmaf(ls, alpha_next, (p[0] + p[1]) + (p[2] + p[3]));
        const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
        const uint32_t l01 = pack_bf16(p[0] - bf_lo(h01), p[1] - bf_hi(h01));
        const uint32_t l23 = pack_bf16(p[2] - bf_lo(h23), p[3] - bf_hi(h23));
        pn_hi = u32x2{h01, h23};
        pn_lo = u32x2{l01, l23};
        grow_next = __builtin_amdgcn_ballot_w64(grow) != 0;
    };

    auto pv = [&](const MItem<DP> &x, MGroup<DP> &r, int n) {
        const int gs = x.t0 + 16 * n;
        unsigned char *tile = vt + (SH::NTB == 2 ? (n & 1) * SH::TILE : 0);
        // rows that take no part (past t1, or dropped by the mask) get V = 0,
        // so that 0 * (NaN or Inf) never reaches the sums
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int row = RPI * i + vrow;
            bool ok;
            if constexpr (MASK) ok = (r.kept >> row) & 1;
            else ok = gs + row < x.t1;
            const u32x4 val = ok ? r.v[i] : u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4 *>(tile + wr_off + (RPI * i) * PITCH) = val;
        }
        wave_lds_sync();
        const lds_u8_m *tl = vt_lds + (SH::NTB == 2 ? (n & 1) * SH::TILE : 0);
        const i16x4_m bh = __builtin_bit_cast(i16x4_m, pw_hi);
        const i16x4_m bl = __builtin_bit_cast(i16x4_m, pw_lo);
#pragma unroll
        for (int j = 0; j < NDB; ++j) {
            const i16x4_m av = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_m *)(tl + tr_off + 32 * j));
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bh, acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bl, acc[j], 0, 0, 0);
        }
    };

    auto rescale = [&]() {
        if (grow_next) {
#pragma unroll
            for (int j = 0; j < NDB; ++j) acc[j] *= alpha_next;
        }
    };

    // Group g: scores(g + 1) from ring slot NEXT, pv(g) from slot THIS, then
    // the rescale for group g + 1.  With two ring slots the stages stay in
    // group order.
    constexpr bool kPipelined = NBUF >= 3;
    auto step = [&](const MItem<DP> &x, MGroup<DP> &rthis, MGroup<DP> &rnext, int g) {
        grow_next = false;
        if constexpr (kPipelined) {
            if (g + 1 < x.ng) scores(x, rnext, g + 1);
            pv(x, rthis, g);
            rescale();
            pw_hi = pn_hi;
            pw_lo = pn_lo;
        } else {
            scores(x, rthis, g);
            rescale();
            pw_hi = pn_hi;
            pw_lo = pn_lo;
            pv(x, rthis, g);
        }
    };

    // Log-sum-exp merge of a unit's partial slots 0 .. nslot - 1 in token
    // order (after the running state, for a tile) into the bf16 output or the
    // state; run by the wave that left the unit's last partial, after an
    // acquire fence.  The wave's V-tile LDS (free between items) holds the
    // slot weights of 64 slots at a time.  Lanes take the (m, l) pairs LPH
    // lanes per head, and the o rows as flat 4-float chunks of the unit's
    // [nh, D] block, two per lane per pass, U slots of loads in flight.
    // The merge is a chain of dependent device-scope round trips at the end
    // of the launch's last items, so when every lane's pairs fit R registers
    // (the usual case) each pair is loaded once, together with the first U
    // slots' o chunks.
    auto merge = [&](const MItem<DP> &x, int nslot) {
        constexpr int U = 8;
        constexpr int R = 4;
        float *wl = reinterpret_cast<float *>(vt);   // [HPI][64] weights of one chunk of slots
        float *lsm = wl + HPI * 64;                  // [HPI] L per head
        float *fsm = lsm + HPI;                      // [HPI] tile: the state's weight per head
        const int nh = x.nh;
        const int64_t row0 = (int64_t)x.s * a.Hq + x.h0;
        int lph = 64;   // lanes per head for the (m, l) pairs
        while (lph > 4 && lph * nh > 64) lph >>= 1;
        const int hh = lane / lph, jl = lane - (lane / lph) * lph;
        const bool hok = hh < nh;
        const float *mlh = a.part_ml + (row0 + (hok ? hh : 0)) * a.nsplit * 2;
        // 16-byte reads through a buffer resource over the unit's o rows
        // (under 2 GiB: the host refuses larger ones)
        const __amdgpu_buffer_rsrc_t urs =
            unit_rsrc(a.part_o + row0 * a.nsplit * a.D, (uint32_t)((int64_t)nh * a.nsplit * a.D * 4));
        const int D4 = a.D >> 2;
        const int F4 = nh * D4;
        // this lane's output chunk p0 + lane (+ 64 for the second): head,
        // first element, byte offset of slot 0 (past F4: head 0, element 0,
        // unused)
        struct Chunk {
            bool ok;
            int h, d;
            uint32_t obo;
        };
        auto chunk = [&](int c) {
            Chunk k;
            k.ok = c < F4;
            k.h = k.ok ? c / D4 : 0;
            k.d = k.ok ? 4 * (c - k.h * D4) : 0;
            k.obo = (uint32_t)(((int64_t)k.h * a.nsplit * a.D + k.d) * 4);
            return k;
        };
        // a tile's state chunk (read before the merge's arithmetic, so that
        // its load travels with the partials')
        auto state_chunk = [&](const Chunk &k) {
            f32x4_m st = {0.f, 0.f, 0.f, 0.f};
            if (TILE && k.ok) st = *reinterpret_cast<const f32x4_m *>(a.o + (row0 + k.h) * a.D + k.d);
            return st;
        };
        auto store = [&](const Chunk &k, const f32x4_m &ov, const f32x4_m &st) {
            if (!k.ok) return;
            const int64_t r = row0 + k.h;
            const float L = lsm[k.h];
            if (TILE) {
                const float fs = fsm[k.h];
                float *po = a.o + r * a.D + k.d;
                *reinterpret_cast<f32x4_m *>(po) = fs > 0.f ? st * fs + ov : ov;
            } else {
                u32x2 packed = {0u, 0u};
                if (L > 0.f) {
                    packed[0] = (uint32_t)f32_to_bf16(ov[0] / L) | ((uint32_t)f32_to_bf16(ov[1] / L) << 16);
                    packed[1] = (uint32_t)f32_to_bf16(ov[2] / L) | ((uint32_t)f32_to_bf16(ov[3] / L) << 16);
                }
                *reinterpret_cast<u32x2 *>(a.out + r * a.D + k.d) = packed;
            }
        };
        // a tile's state (l, m) of head hh (read for every lane, used only
        // where hok: no branch, and no arithmetic on it before the merge's
        // other loads are issued)
        float ls_st = 0.f, ms_raw = 0.f;
        if (TILE) {
            const int64_t rr = row0 + (hok ? hh : 0);
            ls_st = a.l[rr];
            ms_raw = a.m[rr];
        }

        if (nslot <= 64 && nslot <= R * lph) {
            // 1. the lane's pairs (slots jl + lph k) and the first U slots'
            // o chunks of the first pass, in flight together
            float mr[R], lr[R];
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int j = jl + lph * k;
                mr[k] = -INFINITY;
                lr[k] = 0.f;
                if (j < nslot) ld_dev2(mlh + 2 * j, mr[k], lr[k]);
            }
            const Chunk k0 = chunk(lane), k1 = chunk(64 + lane);
            f32x4_m x0[U], x1[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t jo = (uint32_t)min(u, nslot - 1) * (uint32_t)a.D * 4u;
                x0[u] = ld_dev4b(urs, k0.obo + jo);
                x1[u] = ld_dev4b(urs, k1.obo + jo);
            }
            const f32x4_m s0 = state_chunk(k0), s1 = state_chunk(k1);
            // every load above issued before the first wait (the scheduler
            // would otherwise start the arithmetic on the pairs, and wait for
            // them, before issuing the o chunks)
            __builtin_amdgcn_sched_barrier(0);
            const float ms_st = ms_raw * kLog2e;
            // 2. each head's maximum over the slots holding tokens (and the
            // state), the weights into LDS, L
            float mx = -INFINITY;
#pragma unroll
            for (int k = 0; k < R; ++k)
                if (lr[k] > 0.f) mx = fmaxf(mx, mr[k]);
            if (TILE && hok && ls_st > 0.f) mx = fmaxf(mx, ms_st);
            for (int off = 1; off < lph; off <<= 1) mx = fmaxf(mx, shfl_xor(mx, off));
            const float M = mx;
            float lacc = 0.f;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int j = jl + lph * k;
                const float wgt = lr[k] > 0.f ? exp2_fast(mr[k] - M) : 0.f;
                if (hok && j < nslot) wl[hh * 64 + j] = wgt;
                lacc = fmaf(wgt, lr[k], lacc);
            }
            for (int off = 1; off < lph; off <<= 1) lacc += shfl_xor(lacc, off);
            if (hok && jl == 0) {
                const float fs = TILE && ls_st > 0.f ? exp2_fast(ms_st - M) : 0.f;
                if (TILE) fsm[hh] = fs;
                lsm[hh] = TILE ? fmaf(ls_st, fs, lacc) : lacc;
            }
            wave_lds_sync();
            // 3. the weighted o rows, pass by pass (the weights stay in LDS)
            for (int p0 = 0; p0 < F4; p0 += 128) {
                const Chunk c0 = chunk(p0 + lane), c1 = chunk(p0 + 64 + lane);
                f32x4_m o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
                for (int j0 = 0; j0 < nslot; j0 += U) {
                    if (p0 != 0 || j0 != 0) {
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const uint32_t jo = (uint32_t)min(j0 + u, nslot - 1) * (uint32_t)a.D * 4u;
                            x0[u] = ld_dev4b(urs, c0.obo + jo);
                            x1[u] = ld_dev4b(urs, c1.obo + jo);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool in = j0 + u < nslot;
                        const int jj = min(j0 + u, nslot - 1);
                        o0 += (in ? wl[c0.h * 64 + jj] : 0.f) * x0[u];
                        o1 += (in ? wl[c1.h * 64 + jj] : 0.f) * x1[u];
                    }
                }
                store(c0, o0, p0 == 0 ? s0 : state_chunk(c0));
                store(c1, o1, p0 == 0 ? s1 : state_chunk(c1));
            }
            if (TILE && hok && jl == 0) {
                const float L = lsm[hh];
                a.l[row0 + hh] = L;
                a.m[row0 + hh] = L > 0.f ? M * kLn2 : -INFINITY;
            }
            wave_lds_sync();   // the tile LDS is the next groups' V tiles
            return;
        }

        // More pairs than registers: the same, the pairs read again per chunk
        // of 64 slots and per pass.
        const float ms_st = ms_raw * kLog2e;
        // 1. each head's maximum over the slots holding tokens (and the state)
        float mx = -INFINITY;
#pragma unroll 4
        for (int j = jl; j < nslot; j += lph) {
            float t[2];
            ld_dev2(mlh + 2 * j, t[0], t[1]);
            if (t[1] > 0.f) mx = fmaxf(mx, t[0]);
        }
        if (TILE && hok && ls_st > 0.f) mx = fmaxf(mx, ms_st);
        for (int off = 1; off < lph; off <<= 1) mx = fmaxf(mx, shfl_xor(mx, off));
        const float M = mx;   // the head's maximum, in its LPH lanes
        if (TILE && hok && jl == 0) fsm[hh] = ls_st > 0.f ? exp2_fast(ms_st - M) : 0.f;

        // 2. passes of 128 chunks: weights, L, weighted o rows
        float lacc = 0.f;
        for (int p0 = 0; p0 < F4; p0 += 128) {
            const Chunk c0 = chunk(p0 + lane), c1 = chunk(p0 + 64 + lane);
            f32x4_m o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
            for (int cb = 0; cb < nslot; cb += 64) {
                const int n = min(64, nslot - cb);
                for (int j = jl; j < n; j += lph) {
                    float t[2];
                    ld_dev2(mlh + 2 * (cb + j), t[0], t[1]);
                    const float wgt = t[1] > 0.f ? exp2_fast(t[0] - M) : 0.f;
                    if (hok) wl[hh * 64 + j] = wgt;
                    if (p0 == 0) lacc = fmaf(wgt, t[1], lacc);
                }
                wave_lds_sync();
                // U slots of loads in flight; slots past n re-read slot n - 1
                // and take weight 0
                for (int j0 = 0; j0 < n; j0 += U) {
                    f32x4_m x0[U], x1[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const uint32_t jo = (uint32_t)(cb + min(j0 + u, n - 1)) * (uint32_t)a.D * 4u;
                        x0[u] = ld_dev4b(urs, c0.obo + jo);
                        x1[u] = ld_dev4b(urs, c1.obo + jo);
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool in = j0 + u < n;
                        const int jj = min(j0 + u, n - 1);
                        o0 += (in ? wl[c0.h * 64 + jj] : 0.f) * x0[u];
                        o1 += (in ? wl[c1.h * 64 + jj] : 0.f) * x1[u];
                    }
                }
                wave_lds_sync();   // the next chunk's weights overwrite these
            }
            if (p0 == 0) {   // each head's L (the state first, for a tile)
                for (int off = 1; off < lph; off <<= 1) lacc += shfl_xor(lacc, off);
                if (hok && jl == 0) lsm[hh] = TILE ? fmaf(ls_st, ls_st > 0.f ? fsm[hh] : 0.f, lacc) : lacc;
                wave_lds_sync();
            }
            store(c0, o0, state_chunk(c0));
            store(c1, o1, state_chunk(c1));
        }
        if (TILE && hok && jl == 0) {
            const float L = lsm[hh];
            a.l[row0 + hh] = L;
            a.m[row0 + hh] = L > 0.f ? M * kLn2 : -INFINITY;
        }
        wave_lds_sync();   // the tile LDS is the next groups' V tiles
    };

    // The item's totals: its result directly, or a partial (and, for the
    // unit's last partial, the merge).  Lane (qd, h) holds head h, elements
    // 16 n + 4 qd + i.
    auto finish = [&](const MItem<DP> &x) {
        const float L = sum4(ls);
        const int h = col;
        const bool hv = h < x.nh;
        const int64_t r = (int64_t)x.s * a.Hq + x.h0 + (hv ? h : 0);
        if (x.nsp == 1) {
            if (!hv) return;
            if (TILE) {
                const float lsd = a.l[r], msd = a.m[r] * kLog2e;
                float Mt = m2, fs = 0.f, fp = 1.f;
                if (lsd > 0.f) {
                    Mt = fmaxf(msd, m2);
                    fs = exp2_fast(msd - Mt);
                    fp = exp2_fast(m2 - Mt);
                }
#pragma unroll
                for (int j = 0; j < NDB; ++j) {
                    const int d = 16 * j + 4 * qd;
                    if (d >= a.D) continue;
                    float *po = a.o + r * a.D + d;
                    float t[4];
                    ld_f<4>(po, t);
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[e] = fmaf(t[e], fs, acc[j][e] * fp);
                    st_f<4>(po, t);
                }
                if (qd == 0) {
                    const float Lt = fmaf(lsd, fs, L * fp);
                    a.l[r] = Lt;
                    a.m[r] = Lt > 0.f ? Mt * kLn2 : -INFINITY;
                }
            } else {
#pragma unroll
                for (int j = 0; j < NDB; ++j) {
                    const int d = 16 * j + 4 * qd;
                    if (d >= a.D) continue;
                    u32x2 packed = {0u, 0u};
                    if (L > 0.f) {
                        packed[0] = (uint32_t)f32_to_bf16(acc[j][0] / L) | ((uint32_t)f32_to_bf16(acc[j][1] / L) << 16);
                        packed[1] = (uint32_t)f32_to_bf16(acc[j][2] / L) | ((uint32_t)f32_to_bf16(acc[j][3] / L) << 16);
                    }
                    *reinterpret_cast<u32x2 *>(a.out + r * a.D + d) = packed;
                }
            }
            return;
        }
        if (hv) {
            const int64_t pi = r * a.nsplit + x.slot;
            const int64_t row0 = (int64_t)x.s * a.Hq + x.h0;
            const __amdgpu_buffer_rsrc_t urs =
                unit_rsrc(a.part_o + row0 * a.nsplit * a.D, (uint32_t)((int64_t)x.nh * a.nsplit * a.D * 4));
            const uint32_t po = (uint32_t)((pi - row0 * a.nsplit) * a.D * 4);
#pragma unroll
            for (int j = 0; j < NDB; ++j) {
                const int d = 16 * j + 4 * qd;
                if (d < a.D) st_dev4b(urs, po + 4 * d, acc[j]);
            }
            if (qd == 0) {
                st_dev2(a.part_ml + 2 * pi, m2, L);
            }
        }
        // the partial's device-scope stores complete before its arrival is
        // counted; the unit's last arrival merges
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const int before = lane == 0 ? (int)epoch_claim(a.arrive + (int64_t)x.s * units + x.unit, a.epoch) : 0;
        const int nslot = slots_of(x.nsp, a.prefix_mode != 0, big, eighths, sgl);
        if (readlane(before, 0) == nslot - 1) {
            // this XCD's L2 may hold stale copies of the partials' lines
            // (from whatever last touched the workspace): invalidate it
            // before reading them
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            merge(x, nslot);
        }
    };

    MItem<DP> cur, nxt;
    MGroup<DP> rb[NBUF];
    take_sync((int)blockIdx.x * kMWaves + w, cur);
    if (cur.kind == 0) {
#pragma unroll
        for (int j = 0; j < NBUF - 1; ++j) issue(cur, j, rb[j]);
    }
    while (cur.kind == 0) {
        asm volatile("" ::"v"(cur.bidvec));
#pragma unroll
        for (int c = 0; c < NCK; ++c) asm volatile("" ::"v"(cur.q[c]));
        m2 = -INFINITY;
        ls = 0.f;
#pragma unroll
        for (int j = 0; j < NDB; ++j) acc[j] = f32x4_m{0.f, 0.f, 0.f, 0.f};

        const int nr = (cur.ng + NBUF - 1) / NBUF;
        const bool staged = nr >= 3;
        const int rA = staged ? nr - 3 : -1, rB = staged ? nr - 2 : -1;
        // Staged items claim the next item with one atomic at round rA and
        // prefetch it at round rB; a claim that finds another launch's epoch
        // (rare: the counter is restarted at the launch's start) is completed
        // after the rounds.
        unsigned long long claim_raw = 0ull;   // lane 0: the work counter before this wave's add
        bool fetched = false;
        int it_next = nitems, cnt_raw = 0, lv_raw = 0;
        nxt.kind = 2;
        if (!staged) {
            it_next = claim_next();
            locate(it_next, nxt);
            fetch(nxt, cnt_raw, lv_raw);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            resolve(nxt, cnt_raw, lv_raw);
        }
        if constexpr (kPipelined) {   // the pipeline's first stage for group 0
            scores(cur, rb[0], 0);
            pw_hi = pn_hi;
            pw_lo = pn_lo;
        }
        // One round: NBUF groups, each issued NBUF - 1 groups ahead of its
        // step.
        auto round = [&](int n) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NBUF; ++j) {
                issue(cur, n + j + NBUF - 1, rb[(j + NBUF - 1) % NBUF]);
                if (n + j < cur.ng) step(cur, rb[j], rb[(j + 1) % NBUF], n + j);
            }
        };
        // The rounds before rA in a loop of their own, rounds rA (the claim)
        // and rB (the next item's fetch) written out after it: with the
        // work-counter atomic inside the loop's body, the compiler drained
        // every load in flight once per round (measured: wide-head and small
        // batches 1.5-3 % faster without that drain).
        int n = 0;
        for (int r = 0; r < (staged ? rA : nr - 1); ++r, n += NBUF) round(n);
        if (staged) {
            claim_raw = !claims ? ((unsigned long long)a.epoch << 32) | (unsigned)(nitems - nwaves)
                        : lane == 0 ? __hip_atomic_fetch_add(a.work, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                    : 0ull;
            round(n);
            n += NBUF;
            const uint32_t chi = (uint32_t)readlane((int)(uint32_t)(claim_raw >> 32), 0);
            if (chi == a.epoch) {
                it_next = nwaves + readlane((int)(uint32_t)claim_raw, 0);
                locate(it_next, nxt);
                fetch(nxt, cnt_raw, lv_raw);
                fetched = true;
            }
            round(n);
            n += NBUF;
        }
        if (staged) {
            if (!fetched) {
                const int g = lane == 0 ? (int)epoch_claim_after(a.work, a.epoch, claim_raw) : 0;
                it_next = nwaves + readlane(g, 0);
                locate(it_next, nxt);
                fetch(nxt, cnt_raw, lv_raw);
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
            resolve(nxt, cnt_raw, lv_raw);
        }
        issue(cur, n + NBUF - 1, rb[NBUF - 1]);
        if (n < cur.ng) step(cur, rb[0], rb[1], n);
#pragma unroll
        for (int j = 1; j < NBUF; ++j) {
            if (nxt.kind == 0) issue(nxt, j - 1, rb[j - 1]);
            else issue(cur, cur.ng - 1, rb[j - 1]);
            if (n + j < cur.ng) step(cur, rb[j], rb[(j + 1) % NBUF], n + j);
        }
        finish(cur);
        if (nxt.kind != 0 && it_next < nitems) {
            if (nxt.kind == 1) zero_rows(nxt);
            take_sync(claim_next(), nxt);
            if (nxt.kind == 0) {
#pragma unroll
                for (int j = 0; j < NBUF - 1; ++j) issue(nxt, j, rb[j]);
            }
        }
        cur = nxt;
    }

}

// Ring slots (16-token groups, all but one in flight per wave): four, two at
// head dim 256 (16 KB per group; measured on MI355X, three or four slots run
// slower there).
constexpr int attend_nbuf(int dp) { return dp == 256 ? 2 : 4; }

template <int DP, bool P16, bool TILE, bool MASK>
hipError_t launch_t(const AttendArgs &a, int cus, hipStream_t st, const AttendEvents &ev) {
    auto kernel = attend_kernel<DP, P16, attend_nbuf(DP), TILE, MASK>;
    const size_t dyn = a.prefix_mode ? 3 * sizeof(int) * ((size_t)a.S + 1) : 0;
    // One workgroup (four waves) per compute unit: measured on MI355X, the
    // paged row streams of one wave per SIMD reach a higher HBM rate than two.
    const int64_t nsp_max = (a.cap + a.bps - 1) / a.bps;
    const int64_t upper = ((int64_t)a.S * nsp_max * a.Hkv * a.nhc + kMWaves - 1) / kMWaves;
    int64_t nwg = cus;
    if (nwg > upper) nwg = upper;
    if (nwg < 1) nwg = 1;
    if (ev.before) {
        const hipError_t r = hipEventRecord(ev.before, st);
        if (r != hipSuccess) return r;
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)nwg), dim3(kMThreads), dyn, st, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && ev.after) e = hipEventRecord(ev.after, st);
    return e;
}

template <int DP>
hipError_t launch_d(const Plan &p, const AttendArgs &a, int cus, hipStream_t st, const AttendEvents &ev) {
    const bool tile = a.out == nullptr;   // the kv mask comes with decode only
    if (p.p16) {
        if (tile) return launch_t<DP, true, true, false>(a, cus, st, ev);
        return a.mask ? launch_t<DP, true, false, true>(a, cus, st, ev) : launch_t<DP, true, false, false>(a, cus, st, ev);
    }
    if (tile) return launch_t<DP, false, true, false>(a, cus, st, ev);
    return a.mask ? launch_t<DP, false, false, true>(a, cus, st, ev) : launch_t<DP, false, false, false>(a, cus, st, ev);
}

}  // namespace

Plan choose_plan(int G, int D, int bs) {
    Plan p;
    p.dp = D <= 64 ? 64 : (D <= 128 ? 128 : 256);
    p.nhc = G / kHeadsPerItem + (G % kHeadsPerItem != 0);   // ceil, without overflow for any G
    p.p16 = (bs % 16) == 0;
    return p;
}

hipError_t launch_attend(const Plan &p, const AttendArgs &a, int cus, hipStream_t st, const AttendEvents &ev) {
    switch (p.dp) {
        case 64: return launch_d<64>(p, a, cus, st, ev);
        case 128: return launch_d<128>(p, a, cus, st, ev);
        default: return launch_d<256>(p, a, cus, st, ev);
    }
}

}  // namespace pda
