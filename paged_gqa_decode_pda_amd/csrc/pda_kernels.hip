// gfx950 (CDNA4) kernels for paged grouped-query decode attention.
//
// The operation: for each sequence s and q head h, attend the single query
// q[s, h, :] over the tokens listed by the sequence's page list, with scale
// 1/sqrt(head_dim) (AstrAI "CUDA Kernels", section "Python Wrappers") and the
// online-softmax (m, l, o) running state of the spark_storage
// "tiled_attention.rs" page (header comment: reset, one launch per tile,
// finalize as o / l in bf16).  Split-KV partitions follow the "Overview" table
// of the AstrAI page (GQA decode with split-KV, paged KV cache).
//
// Kernels:
//   attend_kernel    persistent: every wave64 takes work items (sequence,
//                    split, kv head + head chunk) from an atomic counter on
//                    its own.  For its split it gathers K/V rows from their
//                    pages, scores the head chunk's q heads against them and
//                    keeps a base-2 online softmax; a single-split sequence's
//                    result is written directly, other splits leave (m, l, o)
//                    partials in the workspace.
//   combine_kernel   one wave per (sequence, q head) row with several splits:
//                    log-sum-exp merge in split order into the bf16 output
//                    (decode) or into the fp32 running state (tile).
//   reset_kernel / finalize_kernel  state fill and o / l -> bf16.
//
// Lane layouts of a wave (D_PAD = padded head dim, 64/128/256):
//   q, K: operands of v_mfma_f32_16x16x32_bf16 (16 heads x 16 tokens per
//      instruction, 32 elements of the head dim deep).  Lane l holds the
//      16-byte chunk 32c + 8(l/16) of head l%16 (q) and of token l%16 (K), so
//      each K load instruction reads 64 contiguous bytes of 16 rows.  The
//      scores come back with lane = token and heads 4(l/16) + i.
//   V: 16 lanes per token row, 4 rows per wave; lane (r = lane/16, c =
//      lane%16) holds elements [c*D_PAD/16, (c+1)*D_PAD/16) of token 4i + r.
//      Softmax weights move from the score layout to the V layout through LDS.
#include "pda_internal.h"
#include "pda_device.h"

namespace pda {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Control words shared across XCDs (the work counter, rewound for the next
// launch; the item sizing, passed to the merge kernel) are written with
// agent-scope stores (gfx950: sc1, written through to the device coherence
// point) and the sizing is read back with agent-scope vector loads.
__device__ __forceinline__ void st_coherent_i(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The matching vector load from the coherence point (never the scalar cache).
__device__ __forceinline__ int ld_coherent_i(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// VE / 2 dwords of bf16 pairs (VE = 2 or 4 elements) of a V row.  V rows
// are streamed once per call and each load covers whole cache lines, so they
// are read non-temporally (measured on MI355X: 5-7 % faster steps).  K rows
// are not: each 128-byte line of a K row is read by two load instructions
// (64 bytes of 16 rows each), and the second must still find the line.
template <int VE>
__device__ __forceinline__ void ld_v(const uint16_t *p, uint32_t (&r)[VE / 2]) {
    if constexpr (VE == 2) {
        r[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
    } else {
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        r[0] = x[0];
        r[1] = x[1];
    }
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
template <int N>
__device__ __forceinline__ void ld_f(const float *p, float (&t)[N]) {
    if constexpr (N == 2) {
        const f32x2 x = *reinterpret_cast<const f32x2 *>(p);
        t[0] = x[0];
        t[1] = x[1];
    } else {
        const f32x4v x = *reinterpret_cast<const f32x4v *>(p);
        t[0] = x[0];
        t[1] = x[1];
        t[2] = x[2];
        t[3] = x[3];
    }
}
template <int N>
__device__ __forceinline__ void st_f(float *p, const float (&t)[N]) {
    if constexpr (N == 2) *reinterpret_cast<f32x2 *>(p) = f32x2{t[0], t[1]};
    else *reinterpret_cast<f32x4v *>(p) = f32x4v{t[0], t[1], t[2], t[3]};
}
template <int N>
__device__ __forceinline__ void st_u(uint16_t *p, const uint32_t (&t)[N]) {
    if constexpr (N == 1) *reinterpret_cast<uint32_t *>(p) = t[0];
    else *reinterpret_cast<u32x2 *>(p) = u32x2{t[0], t[1]};
}

// Tokens of sequence s: the first `cnt` listed pages, all full except the
// last, which holds `lv` valid slots.
__device__ __forceinline__ int seq_tokens(const int32_t *counts, const int32_t *lastv, int lv_default,
                                          int s, int cap, int bs) {
    int cnt = clampi(counts[s], 0, cap);
    if (cnt == 0) return 0;
    int lv = clampi(lastv ? lastv[s] : lv_default, 0, bs);
    return (cnt - 1) * bs + lv;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// V lane layout: a row step covers VR token rows, VL lanes per row, VE
// consecutive elements per lane (one dword or two), so each load instruction
// reads whole rows and every lane accumulates its own elements.
template <int DP>
struct VLayout {
    static constexpr int VE = DP == 256 ? 4 : 2;
    static constexpr int VL = DP / VE;   // 32, 64, 64
    static constexpr int VR = 64 / VL;   // 2, 1, 1
    static constexpr int NS = 16 / VR;   // row steps per 16-token group
};

// Registers of one 16-token group in flight.
template <int DP>
struct GroupRegs {
    u32x4 k[DP / 32];   // K, MFMA B-operand layout: token lane % 16, elements 32 c + 8 (lane / 16) .. + 8
    uint32_t v[VLayout<DP>::NS][VLayout<DP>::VE / 2];   // V: token VR i + lane / VL, elements VE (lane % VL) .. + VE
    uint32_t keep;      // with a kv mask: the mask byte of token lane % 16
    uint64_t kept;      // with a kv mask: bit t set when token t takes part (filled by the scores stage)
};

__device__ __forceinline__ int readlane(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }
__device__ __forceinline__ float readlanef(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

constexpr int kRowRor1 = 0x121;   // row_ror:1
constexpr int kRowRor2 = 0x122;   // row_ror:2

// Maximum / sum over each 16-lane row, left in every lane of the row.
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<kRowRor8>(x));
    x = fmaxf(x, dpp<kRowRor4>(x));
    x = fmaxf(x, dpp<kRowRor2>(x));
    return fmaxf(x, dpp<kRowRor1>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<kRowRor8>(x);
    x += dpp<kRowRor4>(x);
    x += dpp<kRowRor2>(x);
    return x + dpp<kRowRor1>(x);
}

// Maximum / sum over the whole wave (every lane active), wave-uniform: DPP
// inside each 16-lane row, then the four row results read into scalars, in
// one fixed order (no LDS round trip on the chain).
__device__ __forceinline__ float wave_max(float x) {
    x = row_max16(x);
    return fmaxf(fmaxf(readlanef(x, 0), readlanef(x, 16)), fmaxf(readlanef(x, 32), readlanef(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
    x = row_sum16(x);
    return (readlanef(x, 0) + readlanef(x, 16)) + (readlanef(x, 32) + readlanef(x, 48));
}

// Softmax weights of one group, moving from the score layout (lane = token)
// to the V layout (16 lanes per token row).
template <int GC>
struct WaveSmem {
    float p[2][16][GC];   // double-buffered by group parity
};

// Splits of a sequence: ceil(ntok / span), 0 for an empty sequence.
__device__ __forceinline__ int splits_of(int ntok, int span) { return ntok > 0 ? (ntok + span - 1) / span : 0; }

// Work items of a sequence with nsp splits (prefix mode): nb "big" items of
// `big` consecutive splits cover about eighths / 8 of the splits, then one
// item per remaining split.  Items are numbered in token order; item k of the
// sequence owns partial slot k, so a sequence has nb + (nsp - nb * big) slots.
__device__ __forceinline__ int big_items_of(int nsp, int big, int eighths) { return (eighths * nsp) / (8 * big); }
__device__ __forceinline__ int slots_of(int nsp, bool prefix_mode, int big, int eighths) {
    return prefix_mode ? nsp - (big - 1) * big_items_of(nsp, big, eighths) : nsp;
}

// One work item as a wave holds it.  Everything is wave-uniform except bidvec
// and q.
template <int DP>
struct Item {
    int kind;        // 0: attend tokens [t0, t1); 1: zero the decode output rows; 2: nothing
    int s, g, h0, nh, split, nspl, slot;
    int cnt, t0, t1, ng, nsp;
    int cb;          // first page (index into the sequence's list) of the page-id window
    int bidvec;      // the window: lane i holds the id of page cb + i
    u32x4 q[DP / 32];  // MFMA A operand: head lane % 16, elements 32 c + 8 (lane / 16) .. + 8
};

// Persistent attention kernel.  Work items are (sequence, split, unit), unit =
// (kv head, head chunk) fastest, so the waves reading the interleaved kv-head
// rows of the same pages run together.  Every wave takes items from an atomic
// counter on its own and never waits for another wave.
//
// A wave's items form one stream of 16-token groups with NBUF - 1 groups in
// flight: the last ring slots of an item already load the next item's first
// groups.  The next item is claimed three ring rounds before the end of the
// current one, located and its counts, q rows and page ids requested two
// rounds before, and resolved at the start of the last round, so every wait
// lands on loads issued a round earlier and the stream does not drain between
// items (items of fewer than three rounds take the next item synchronously).
//
// Per group: q.K^T as DP/32 v_mfma_f32_16x16x32_bf16 (A = the head chunk's q
// rows, B = 16 K rows loaded straight into the operand layout, 64 contiguous
// bytes of 16 rows per load); the scores land with lane = token and heads
// 4 (lane / 16) + i in the four result registers.  A base-2 online softmax
// per head uses 16-lane DPP maxima and a wave-uniform running max; the weights
// move to the V layout through LDS and P.V accumulates in fp32 FMAs.  A
// sequence with one split gets its result written directly (bf16 o / l for
// decode, folded into the running state for a tile); otherwise every item
// leaves an (m, l, o) partial in its slot for combine_kernel.
template <int DP, int GC, bool P16, int NBUF, bool TILE, bool MASK>
__global__ void __launch_bounds__(kThreads) attend_kernel(const AttendArgs a) {
    constexpr int NCK = DP / 32;
    constexpr int VE = VLayout<DP>::VE, VL = VLayout<DP>::VL, VR = VLayout<DP>::VR, NS = VLayout<DP>::NS;
    constexpr int HR = (GC + 3) / 4;   // score rows (of 16 lanes) that hold real heads
    constexpr int NI = GC < 4 ? GC : 4;
    static_assert(GC <= 8 && NBUF >= 2, "at most 8 q heads per item, at least 2 ring slots");

    __shared__ WaveSmem<GC> wsm[kWaves];
    __shared__ int scan[2 * kWaves];
    __shared__ float wsum_f[2 * kWaves];
    extern __shared__ int prefix[];   // 2 (S + 1) ints when a.prefix_mode

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int units = a.Hkv * a.nhc;
    const int span = a.bps * a.bs;
    const int row = lane >> 4, col = lane & 15;

    // Work items.  With the prefix (sequences up to kPrefixMaxSeqs), each
    // sequence's splits are grouped: a share of them, `big` at a time,
    // form "big" items queued first; the rest are single-split items queued
    // after all big ones, so the queue ends with short work.  Decode keeps
    // one small item for an empty sequence so that its zero output row gets
    // written.
    int nbig_pairs = 0, npairs;
    int *pbig = prefix;                 // big items before sequence s
    int *psmall = prefix + a.S + 1;     // small items before sequence s
    const int nsp_max = (a.cap + a.bps - 1) / a.bps;
    int big = 1, eighths = 0;
    if (a.prefix_mode) {
        // Sizing (every workgroup takes the same decision from the same
        // totals): with at least kBigTokensLarge tokens of work per wave, big
        // items span kBigTokensLarge tokens and take kEighthsLarge / 8 of the
        // splits; with less, every split is an item as long as there are no
        // more split items than waves (one round, equal lengths), else
        // kEighthsPaired / 8 of the splits go in pairs.
        float tot = 0.f, nspl = 0.f;
        for (int s = tid; s < a.S; s += kThreads) {
            const int nt = seq_tokens(a.counts, a.lastv, a.lv_default, s, a.cap, a.bs);
            psmall[s + 1] = nt;   // kept for the scan below
            tot += (float)nt;
            nspl += (float)splits_of(nt, span);
        }
        tot = wave_sum(tot);
        nspl = wave_sum(nspl);
        if (lane == 0) {
            wsum_f[w] = tot;
            wsum_f[kWaves + w] = nspl;
        }
        __syncthreads();
        tot = wsum_f[0] + wsum_f[1] + wsum_f[2] + wsum_f[3];
        nspl = wsum_f[4] + wsum_f[5] + wsum_f[6] + wsum_f[7];
        const float waves = (float)((int)gridDim.x * kWaves);
        if (tot * (float)units >= (float)kBigTokensLarge * waves) {
            big = max(1, kBigTokensLarge / span);
            eighths = kEighthsLarge;
        } else if (nspl * (float)units > waves) {
            big = 2;
            eighths = kEighthsPaired;
        } else {
            big = 1;
            eighths = 0;
        }
        if (blockIdx.x == 0 && tid == 0) {   // for the merge kernel
            st_coherent_i(&a.ctrl[kCtrlSizing], big);
            st_coherent_i(&a.ctrl[kCtrlSizing + 1], eighths);
        }
        int carry_b = 0, carry_s = 0;
        for (int base = 0; base < a.S; base += kThreads) {
            const int s = base + tid;
            int nb = 0, ns = 0;
            if (s < a.S) {
                const int nsp = splits_of(psmall[s + 1], span);
                nb = big_items_of(nsp, big, eighths);
                ns = nsp - nb * big;
                if (!TILE && nsp == 0) ns = 1;
            }
            int xb = nb, xs = ns;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int yb = __shfl_up(xb, off, 64);
                const int ys = __shfl_up(xs, off, 64);
                if (lane >= off) {
                    xb += yb;
                    xs += ys;
                }
            }
            if (lane == 63) {
                scan[w] = xb;
                scan[kWaves + w] = xs;
            }
            __syncthreads();
            int wb = 0, wsum = 0;
            for (int ww = 0; ww < w; ++ww) {
                wb += scan[ww];
                wsum += scan[kWaves + ww];
            }
            if (s < a.S) {
                pbig[s + 1] = carry_b + wb + xb;
                psmall[s + 1] = carry_s + wsum + xs;
            }
            carry_b += scan[0] + scan[1] + scan[2] + scan[3];
            carry_s += scan[4] + scan[5] + scan[6] + scan[7];
            __syncthreads();
        }
        if (tid == 0) {
            pbig[0] = 0;
            psmall[0] = 0;
        }
        nbig_pairs = __builtin_amdgcn_readfirstlane(carry_b);
        npairs = nbig_pairs + __builtin_amdgcn_readfirstlane(carry_s);
    } else {
        npairs = a.S * nsp_max;
    }
    const int nitems = npairs * units;
    __syncthreads();

    WaveSmem<GC> &ws = wsm[w];
    const int nwaves = (int)gridDim.x * kWaves;
    const int tok32 = (int)a.tok;
    // without per-sequence last-valid counts, any in-bounds int array stands in
    // (its values are not used)
    const int32_t *lv_src = a.lastv ? a.lastv : a.counts;

    // Lane-invariant element offsets.  K chunks past head_dim re-read chunk 0
    // of the same row (in bounds; q is zero there); V lanes past head_dim are
    // never stored.
    int kd[NCK];
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
        const int d0 = 32 * c + 8 * row;
        kd[c] = d0 < a.D ? d0 : 0;
    }
    const int vr = VR == 1 ? 0 : lane / VL;   // V row within a step
    const int ve0 = (lane % VL) * VE;          // first V element of the lane
    const bool vok = ve0 < a.D;                // head_dim is a multiple of 8: all VE elements in, or all out
    const int vofs = vok ? ve0 : 0;
    const int vlane = vr * (int)a.tok + vofs;

    // Step 1 of taking item `it`: where it is, from LDS only.  An index past
    // the last item becomes kind 2 with in-bounds coordinates.
    auto locate = [&](int it, Item<DP> &x) {
        x.kind = it < nitems ? 0 : 2;
        if (it >= nitems) it = 0;
        int pair = it / units;
        const int unit = it - pair * units;
        if (a.prefix_mode) {
            const bool is_big = pair < nbig_pairs;
            const int *pf = is_big ? pbig : psmall;
            if (!is_big) pair -= nbig_pairs;
            int lo = 0, hi = a.S;   // the largest s with pf[s] <= pair
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
                x.split = nb_s * big + j;
                x.nspl = 1;
                x.slot = nb_s + j;
            }
        } else {
            x.s = pair / nsp_max;
            x.split = pair - x.s * nsp_max;
            x.nspl = 1;
            x.slot = x.split;
        }
        x.g = unit / a.nhc;
        const int hc = unit - x.g * a.nhc;
        x.h0 = x.g * a.G + hc * GC;
        x.nh = min(GC, a.G - hc * GC);
        x.cb = x.split * a.bps;   // the split's first page (< tile_capacity)
    };

    // Step 2: request the sequence's counts, the q rows and the page-id
    // window (page ids past the list are read but never used).
    auto fetch = [&](Item<DP> &x, int &cnt_raw, int &lv_raw) {
        cnt_raw = a.counts[x.s];
        lv_raw = lv_src[x.s];
        const uint16_t *qp = a.q + ((int64_t)x.s * a.Hq + x.h0 + min(col, x.nh - 1)) * a.D;
#pragma unroll
        for (int c = 0; c < NCK; ++c) x.q[c] = ld16(qp + kd[c]);
        x.bidvec = a.blocks[(int64_t)x.s * a.cap + min(x.cb + lane, a.cap - 1)];
    };

    // Step 3: the token range, from the counts.
    auto resolve = [&](Item<DP> &x, int cnt_raw, int lv_raw) {
        x.t0 = x.t1 = x.ng = 0;   // no token range unless it attends
        x.cnt = clampi(__builtin_amdgcn_readfirstlane(cnt_raw), 0, a.cap);
        const int lv = clampi(a.lastv ? __builtin_amdgcn_readfirstlane(lv_raw) : a.lv_default, 0, a.bs);
        const int ntok = x.cnt > 0 ? (x.cnt - 1) * a.bs + lv : 0;
        x.nsp = splits_of(ntok, span);
#pragma unroll
        for (int c = 0; c < NCK; ++c)
            x.q[c] = (col < x.nh && 32 * c + 8 * row < a.D) ? x.q[c] : u32x4{0, 0, 0, 0};
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

    auto claim_next = [&]() {
        const int grabbed = lane == 0 ? atomicAdd(&a.ctrl[0], 1) : 0;
        return nwaves + readlane(grabbed, 0);
    };

    // Takes items from `it` on until one has tokens or the queue is empty,
    // writing the zero rows of empty decode sequences on the way.
    auto take_sync = [&](int it, Item<DP> &x) {
        for (;;) {
            int cr, lr;
            locate(it, x);
            fetch(x, cr, lr);
            // complete every request here, so that none is left pending into
            // the ring loop
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            resolve(x, cr, lr);
            if (x.kind == 0 || it >= nitems) return;
            if (x.kind == 1) {
                const int64_t row0 = (int64_t)x.s * a.Hq + x.h0;
                for (int idx = lane; idx < x.nh * a.D; idx += 64) a.out[row0 * a.D + idx] = 0;
            }
            it = claim_next();
        }
    };

    // Loads of group n of item x (indices past the last group re-read it: in
    // bounds, never computed).
    auto issue = [&](Item<DP> &x, int n, GroupRegs<DP> &r) {
        n = min(n, x.ng - 1);
        const int gs = x.t0 + 16 * n;
        const int64_t gk = (int64_t)x.g * a.kvh;
        const int32_t *brow = a.blocks + (int64_t)x.s * a.cap;
        if constexpr (P16) {
            const int page = page_of((uint32_t)gs, a.bs_magic);
            if (page - x.cb >= 64) {   // move the window (at most once per 64 pages)
                x.cb = page;
                x.bidvec = brow[min(page + lane, x.cnt - 1)];
                // wait here, so that the path without a move carries no wait
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
            const int bid = readlane(x.bidvec, page - x.cb);
            const int64_t off = (int64_t)bid * a.blk + gk + (int64_t)(gs - page * a.bs) * a.tok;
            const uint16_t *kb = a.k + off;
            const uint16_t *vb = a.v + off;
#pragma unroll
            for (int c = 0; c < NCK; ++c) r.k[c] = ld16(kb + (col * tok32 + kd[c]));
            if constexpr (MASK) {   // tokens past t1 read the group's first token's byte (in bounds)
                const int tk = gs + col < x.t1 ? gs + col : gs;
                r.keep = a.mask[(int64_t)x.s * a.mask_stride + tk];
            }
            // uniform row pointer per step, one lane offset for all steps
#pragma unroll
            for (int i = 0; i < NS; ++i) ld_v<VE>(vb + (int64_t)(VR * i) * a.tok + vlane, r.v[i]);
        } else {
            const int last = min(gs + 15, x.t1 - 1);
            if (page_of((uint32_t)last, a.bs_magic) - x.cb >= 64) {
                x.cb = page_of((uint32_t)gs, a.bs_magic);
                x.bidvec = brow[min(x.cb + lane, x.cnt - 1)];
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
            // tokens past t1 read the group's first token instead (in bounds)
            const int tk = gs + col < x.t1 ? gs + col : gs;
            const int pk = page_of((uint32_t)tk, a.bs_magic);
            const int bk = __shfl(x.bidvec, pk - x.cb, 64);
            const uint16_t *kp = a.k + ((int64_t)bk * a.blk + gk + (int64_t)(tk - pk * a.bs) * a.tok);
#pragma unroll
            for (int c = 0; c < NCK; ++c) r.k[c] = ld16(kp + kd[c]);
            if constexpr (MASK) r.keep = a.mask[(int64_t)x.s * a.mask_stride + tk];
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int tv = gs + VR * i + vr < x.t1 ? gs + VR * i + vr : gs;
                const int pv = page_of((uint32_t)tv, a.bs_magic);
                const int bv = VR == 1 ? readlane(x.bidvec, pv - x.cb) : __shfl(x.bidvec, pv - x.cb, 64);
                const uint16_t *vp = a.v + ((int64_t)bv * a.blk + gk + (int64_t)(tv - pv * a.bs) * a.tok);
                ld_v<VE>(vp + vofs, r.v[i]);
            }
        }
    };

    float m2[GC];          // running max per head (base 2, wave-uniform)
    float ls4[4];          // running sum of this lane's token weights, head 4 (lane / 16) + i
    float acc_o[GC][VE];   // running P.V of the lane's elements (partial over its V rows when VR > 1)

    // Per group, two stages, software-pipelined across groups: scores(g + 1)
    // (MFMA, online max, weights into LDS buffer (g + 1) & 1) runs next to
    // pv(g) (weights of group g from buffer g & 1, times V), so the latency
    // chain of one overlaps the FMAs of the other.  The rescale of the P.V
    // sums by the max change of group g + 1 is applied after pv(g).
    bool grow_next = false;   // wave-uniform
    float alpha_next[GC];

    auto scores = [&](const Item<DP> &x, GroupRegs<DP> &r, int n) {
        const int gs = x.t0 + 16 * n;
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCK; ++c)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x.q[c]),
                                                           __builtin_bit_cast(bf16x8, r.k[c]), sacc, 0, 0, 0);
        const bool valid = gs + col < x.t1 && (!MASK || r.keep != 0);
        if constexpr (MASK) r.kept = __builtin_amdgcn_ballot_w64(valid);
        float sc[4], rm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = valid ? sacc[i] * a.scale_log2 : -INFINITY;
#pragma unroll
        for (int i = 0; i < NI; ++i) rm[i] = row_max16(sc[i]);
        bool grow = false;
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            const float mn = fmaxf(m2[h], readlanef(rm[h & 3], 16 * (h >> 2)));
            grow |= mn > m2[h];
            alpha_next[h] = exp2_fast(m2[h] - mn);   // 0 while m2 is still -inf
            m2[h] = mn;
        }
        grow_next = grow;
        if (grow) {
#pragma unroll
            for (int i = 0; i < NI; ++i) ls4[i] *= (HR > 1 && row == 1) ? alpha_next[(4 + i) % GC] : alpha_next[i];
        }
        float p[4];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float mh = (HR > 1 && row == 1) ? m2[(4 + i) % GC] : m2[i];
            p[i] = valid ? exp2_fast(sc[i] - mh) : 0.f;
            ls4[i] += p[i];
        }
        if (row < HR) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
                if (4 * row + i < GC) ws.p[n & 1][col][4 * row + i] = p[i];
        }
    };

    auto pv = [&](const Item<DP> &x, GroupRegs<DP> &r, int n) {
        const int gs = x.t0 + 16 * n;
        // rows that take no part (past t1, or dropped by the mask) get V = 0,
        // so that 0 * (NaN or Inf) never reaches the sums
        if constexpr (MASK) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const bool ok = (r.kept >> (VR * i + vr)) & 1;
#pragma unroll
                for (int e = 0; e < VE / 2; ++e) r.v[i][e] = ok ? r.v[i][e] : 0u;
            }
        } else if (gs + 16 > x.t1) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const bool ok = gs + VR * i + vr < x.t1;
#pragma unroll
                for (int e = 0; e < VE / 2; ++e) r.v[i][e] = ok ? r.v[i][e] : 0u;
            }
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            float pw[GC];
#pragma unroll
            for (int h = 0; h < GC; ++h) pw[h] = ws.p[n & 1][VR * i + vr][h];
#pragma unroll
            for (int e = 0; e < VE / 2; ++e) {
                const float f0 = bf_lo(r.v[i][e]);
                const float f1 = bf_hi(r.v[i][e]);
#pragma unroll
                for (int h = 0; h < GC; ++h) {
                    acc_o[h][2 * e] = fmaf(pw[h], f0, acc_o[h][2 * e]);
                    acc_o[h][2 * e + 1] = fmaf(pw[h], f1, acc_o[h][2 * e + 1]);
                }
            }
        }
    };

    // Group g of the current item: scores(g + 1) from ring slot NEXT, pv(g)
    // from ring slot THIS, then the rescale for group g + 1.  With a ring of
    // two slots the next group is the one just requested, so there the
    // stages stay in group order (scores(g), then pv(g)).
    constexpr bool kPipelined = NBUF >= 3;
    auto step = [&](const Item<DP> &x, GroupRegs<DP> &rthis, GroupRegs<DP> &rnext, int g) {
        grow_next = false;
        if constexpr (kPipelined) {
            if (g + 1 < x.ng) scores(x, rnext, g + 1);
        } else {
            scores(x, rthis, g);
            if (grow_next) {
#pragma unroll
                for (int h = 0; h < GC; ++h) {
#pragma unroll
                    for (int e = 0; e < VE; ++e) acc_o[h][e] *= alpha_next[h];
                }
            }
            grow_next = false;
            wave_lds_sync();
        }
        pv(x, rthis, g);
        if (grow_next) {
#pragma unroll
            for (int h = 0; h < GC; ++h) {
#pragma unroll
                for (int e = 0; e < VE; ++e) acc_o[h][e] *= alpha_next[h];
            }
        }
        wave_lds_sync();
    };

    // The item's totals: its result directly, or a partial.
    auto finish = [&](const Item<DP> &x) {
        const int64_t row0 = (int64_t)x.s * a.Hq + x.h0;
        float rs[4], lsum[GC];
#pragma unroll
        for (int i = 0; i < NI; ++i) rs[i] = row_sum16(ls4[i]);
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            lsum[h] = readlanef(rs[h & 3], 16 * (h >> 2));
            if constexpr (VR > 1) {
#pragma unroll
                for (int e = 0; e < VE; ++e) acc_o[h][e] += shfl_xor(acc_o[h][e], 32);
            }
        }
        // lanes of V row 0 hold the item's totals for elements ve0 .. ve0 + VE - 1
        const bool store = vr == 0 && vok;
        if (x.nsp == 1) {
#pragma unroll
            for (int h = 0; h < GC; ++h) {
                if (h >= x.nh) continue;
                const int64_t r = row0 + h;
                if (TILE) {
                    const float ls = a.l[r], ms = a.m[r] * kLog2e;
                    float Mt = m2[h], fs = 0.f, fp = 1.f;
                    if (ls > 0.f) {
                        Mt = fmaxf(ms, m2[h]);
                        fs = exp2_fast(ms - Mt);
                        fp = exp2_fast(m2[h] - Mt);
                    }
                    if (store) {
                        float *po = a.o + r * a.D + ve0;
                        float t[VE];
                        ld_f<VE>(po, t);
#pragma unroll
                        for (int e = 0; e < VE; ++e) t[e] = fmaf(t[e], fs, acc_o[h][e] * fp);
                        st_f<VE>(po, t);
                    }
                    if (lane == 0) {
                        const float Lt = fmaf(ls, fs, lsum[h] * fp);
                        a.l[r] = Lt;
                        a.m[r] = Lt > 0.f ? Mt * kLn2 : -INFINITY;
                    }
                } else if (store) {
                    const float L = lsum[h];
                    uint32_t packed[VE / 2];
#pragma unroll
                    for (int e = 0; e < VE / 2; ++e)
                        packed[e] = L > 0.f ? (uint32_t)f32_to_bf16(acc_o[h][2 * e] / L) |
                                                  ((uint32_t)f32_to_bf16(acc_o[h][2 * e + 1] / L) << 16)
                                            : 0u;
                    st_u<VE / 2>(a.out + r * a.D + ve0, packed);
                }
            }
        } else {
#pragma unroll
            for (int h = 0; h < GC; ++h) {
                if (h >= x.nh) continue;
                const int64_t pi = (row0 + h) * a.nsplit + x.slot;
                if (store) st_f<VE>(a.part_o + pi * a.D + ve0, acc_o[h]);
                if (lane == 0) {
                    a.part_ml[2 * pi] = m2[h];
                    a.part_ml[2 * pi + 1] = lsum[h];
                }
            }
        }
    };

    Item<DP> cur, nxt;
    GroupRegs<DP> rb[NBUF];
    take_sync((int)blockIdx.x * kWaves + w, cur);
    if (cur.kind == 0) {
#pragma unroll
        for (int j = 0; j < NBUF - 1; ++j) issue(cur, j, rb[j]);
    }
    while (cur.kind == 0) {
        // The item's q rows and page-id window were requested a round before
        // the previous item ended.  Consume them here, once per item, so that
        // no wait for them is left inside the ring loop.
        asm volatile("" ::"v"(cur.bidvec));
#pragma unroll
        for (int c = 0; c < NCK; ++c) asm volatile("" ::"v"(cur.q[c]));
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            m2[h] = -INFINITY;
#pragma unroll
            for (int e = 0; e < VE; ++e) acc_o[h][e] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ls4[i] = 0.f;

        // rounds of NBUF groups; the item's group count is padded to whole
        // rounds (padding re-reads the last group and is not computed)
        const int nr = (cur.ng + NBUF - 1) / NBUF;
        const bool staged = nr >= 3;
        const int rA = staged ? nr - 3 : -1, rB = staged ? nr - 2 : -1;
        int grabbed = 0, it_next = nitems, cnt_raw = 0, lv_raw = 0;
        nxt.kind = 2;
        if (!staged) {
            // a short item takes the next one at once, waiting at each step
            it_next = claim_next();
            locate(it_next, nxt);
            fetch(nxt, cnt_raw, lv_raw);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            resolve(nxt, cnt_raw, lv_raw);
        }
        if constexpr (kPipelined) {
            scores(cur, rb[0], 0);   // the pipeline's first stage for group 0
            wave_lds_sync();
        }
        int n = 0;
        for (int r = 0; r < nr - 1; ++r, n += NBUF) {
            // Stage B (locate the claimed item, request its counts, q rows and
            // page ids) sits before stage A (the claim) in program order, so
            // every path from the claim to its use, and from the requests to
            // theirs, crosses a full round of ring loads and the compiler's
            // waits leave the ring in flight.
            if (r == rB) {
                it_next = nwaves + readlane(grabbed, 0);
                locate(it_next, nxt);
                fetch(nxt, cnt_raw, lv_raw);
            }
            if (r == rA) grabbed = lane == 0 ? atomicAdd(&a.ctrl[0], 1) : 0;
#pragma unroll
            for (int j = 0; j < NBUF; ++j) {
                issue(cur, n + j + NBUF - 1, rb[(j + NBUF - 1) % NBUF]);
                if (n + j < cur.ng) step(cur, rb[j], rb[(j + 1) % NBUF], n + j);
            }
        }
        if (staged) resolve(nxt, cnt_raw, lv_raw);   // stage C
        // last round: its issues after the first carry the next item's first
        // groups into the ring slots that item starts from
        issue(cur, n + NBUF - 1, rb[NBUF - 1]);
        if (n < cur.ng) step(cur, rb[0], rb[1], n);
#pragma unroll
        for (int j = 1; j < NBUF; ++j) {
            // both paths issue the same loads, so that the waits of the
            // computes that follow keep their in-flight allowance
            if (nxt.kind == 0) issue(nxt, j - 1, rb[j - 1]);
            else issue(cur, cur.ng - 1, rb[j - 1]);
            if (n + j < cur.ng) step(cur, rb[j], rb[(j + 1) % NBUF], n + j);
        }
        finish(cur);
        if (nxt.kind != 0 && it_next < nitems) {
            // the claimed item had no tokens: take items synchronously
            if (nxt.kind == 1) {
                const int64_t row0 = (int64_t)nxt.s * a.Hq + nxt.h0;
                for (int idx = lane; idx < nxt.nh * a.D; idx += 64) a.out[row0 * a.D + idx] = 0;
            }
            take_sync(claim_next(), nxt);
            if (nxt.kind == 0) {
#pragma unroll
                for (int j = 0; j < NBUF - 1; ++j) issue(nxt, j, rb[j]);
            }
        }
        cur = nxt;
    }

    // The last wave to finish rewinds the work counter for the next launch.
    if (lane == 0) {
        const int done = atomicAdd(&a.ctrl[1], 1);
        if (done == (int)gridDim.x * kWaves - 1) {
            st_coherent_i(&a.ctrl[0], 0);
            st_coherent_i(&a.ctrl[1], 0);
        }
    }
}

// One wave per (sequence, q head) row whose sequence has more than one split:
// log-sum-exp merge of the split partials in split order (after the running
// state when folding a tile), into the bf16 output or the state.  Slot weights
// are formed lane-parallel (lane i <-> slot cb + i).  The weighted sum reads
// 16 bytes per lane: a load instruction covers SPI slot rows of DP/4 lanes
// each, U instructions are in flight, and the SPI lane groups are summed at
// the end.
template <int DP, bool TILE>
__global__ void __launch_bounds__(kThreads) combine_kernel(const AttendArgs a) {
    constexpr int LPS = DP / 4;     // lanes per slot row
    constexpr int SPI = 64 / LPS;   // slot rows per load instruction: 4, 2, 1
    constexpr int U = 8;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t sh = (int64_t)blockIdx.x * kWaves + w;
    if (sh >= (int64_t)a.S * a.Hq) return;
    const int s = (int)(sh / a.Hq);
    const int span = a.bps * a.bs;
    const int nsp = splits_of(seq_tokens(a.counts, a.lastv, a.lv_default, s, a.cap, a.bs), span);
    if (nsp <= 1) return;   // written by the attention kernel (or an untouched empty tile)
    const bool pm = a.prefix_mode != 0;
    const int big = pm ? ld_coherent_i(&a.ctrl[kCtrlSizing]) : 1;
    const int eighths = pm ? ld_coherent_i(&a.ctrl[kCtrlSizing + 1]) : 0;
    const int nslot = slots_of(nsp, pm, big, eighths);
    const int sub = lane / LPS;
    const int d0 = (lane % LPS) * 4;
    const bool dok = d0 < a.D;   // head_dim is a multiple of 8: a lane's 4 elements are all in or all out
    const int dofs = dok ? d0 : 0;
    const float *ml = a.part_ml + sh * a.nsplit * 2;
    const float *po = a.part_o + sh * a.nsplit * a.D;

    // Rows of slots j0 + u SPI + sub (u < U) of a chunk with n slots; slots
    // past n re-read slot n - 1 and get weight 0.
    float t[U][4];
    auto load_block = [&](int cb, int j0, int n) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(j0 + u * SPI + sub, n - 1);
            ld_f<4>(po + (int64_t)(cb + j) * a.D + dofs, t[u]);
        }
    };
    // (m, l) of slot lane + 64 c
    auto load_ml = [&](int cb) {
        float x[2];
        ld_f<2>(ml + 2 * min(cb + lane, nslot - 1), x);
        return f32x2{x[0], cb + lane < nslot ? x[1] : 0.f};
    };
    // the first chunk's (m, l) and first block of rows do not depend on the
    // weights: request them before the maximum is known
    f32x2 ml_c = load_ml(0);
    load_block(0, 0, min(64, nslot));

    const float ls = TILE ? a.l[sh] : 0.f;
    const float ms = TILE ? a.m[sh] * kLog2e : -INFINITY;
    float M = ls > 0.f ? ms : -INFINITY;
    if (ml_c[1] > 0.f) M = fmaxf(M, ml_c[0]);
    for (int cb = 64; cb < nslot; cb += 64) {
        const f32x2 x = load_ml(cb);
        if (x[1] > 0.f) M = fmaxf(M, x[0]);
    }
    M = wave_max(M);

    float L = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
    if (ls > 0.f) {
        const float f = exp2_fast(ms - M);
        L = ls * f;
        if (sub == 0 && dok) {   // counted once: lane group 0 only
            float st[4];
            ld_f<4>(a.o + sh * a.D + d0, st);
#pragma unroll
            for (int e = 0; e < 4; ++e) O[e] = st[e] * f;
        }
    }
    for (int cb = 0; cb < nslot; cb += 64) {
        if (cb > 0) ml_c = load_ml(cb);
        const float wi = ml_c[1] > 0.f ? exp2_fast(ml_c[0] - M) : 0.f;
        L += wave_sum(wi * ml_c[1]);
        const int n = min(64, nslot - cb);
        for (int j0 = 0; j0 < n; j0 += SPI * U) {
            if (cb > 0 || j0 > 0) load_block(cb, j0, n);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + u * SPI + sub;
                const float f = __shfl(wi, min(j, n - 1), 64);
                const float fw = j < n ? f : 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) O[e] = fmaf(t[u][e], fw, O[e]);
            }
        }
    }
#pragma unroll
    for (int off = LPS; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] += shfl_xor(O[e], off);
    }
    if (sub != 0 || !dok) return;
    if (TILE) {
        st_f<4>(a.o + sh * a.D + d0, O);
        if (lane == 0) {
            a.l[sh] = L;
            a.m[sh] = L > 0.f ? M * kLn2 : -INFINITY;
        }
    } else {
        uint32_t packed[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
            packed[e] = L > 0.f ? (uint32_t)f32_to_bf16(O[2 * e] / L) | ((uint32_t)f32_to_bf16(O[2 * e + 1] / L) << 16)
                                : 0u;
        st_u<2>(a.out + sh * a.D + d0, packed);
    }
}

__global__ void __launch_bounds__(256) reset_kernel(float *m, float *l, float *o, int64_t rows, int D) {
    const int64_t n = rows * D;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        o[i] = 0.f;
        if (i < rows) {
            m[i] = -INFINITY;
            l[i] = 0.f;
        }
    }
}

__global__ void __launch_bounds__(256) zero_ints_kernel(int32_t *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

__global__ void __launch_bounds__(256) finalize_kernel(const float *l, const float *o, uint16_t *out,
                                                       int64_t rows, int D) {
    const int64_t n = rows * D;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float li = l[i / D];
        out[i] = li > 0.f ? f32_to_bf16(o[i] / li) : 0;
    }
}

// Ring slots (16-token K/V groups; all but one in flight per wave): four,
// two for head dim 256 (measured faster there: 16 KB per group).
constexpr int nbuf_for(int dp) { return dp == 256 ? 2 : 4; }

template <int DP, int GC, bool P16, bool TILE, bool MASK>
hipError_t launch_attend_t(const AttendArgs &a, int cus, hipStream_t st, const AttendEvents &ev) {
    auto kernel = attend_kernel<DP, GC, P16, nbuf_for(DP), TILE, MASK>;
    const size_t dyn = a.prefix_mode ? 2 * sizeof(int) * ((size_t)a.S + 1) : 0;
    // One workgroup (four waves) per compute unit: measured on MI355X, the
    // paged row streams of one wave per SIMD reach a higher HBM rate than two
    // (or an uneven split of workgroups over the CUs).
    const int64_t nsp_max = (a.cap + a.bps - 1) / a.bps;
    const int64_t upper = ((int64_t)a.S * nsp_max * a.Hkv * a.nhc + kWaves - 1) / kWaves;
    int64_t nwg = cus;
    if (nwg > upper) nwg = upper;
    if (nwg < 1) nwg = 1;
    if (ev.before) {
        const hipError_t r = hipEventRecord(ev.before, st);
        if (r != hipSuccess) return r;
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)nwg), dim3(kThreads), dyn, st, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && ev.after) e = hipEventRecord(ev.after, st);
    if (e != hipSuccess || a.bps >= a.cap) return e;   // one split per sequence: nothing to combine
    const int64_t rows = (int64_t)a.S * a.Hq;
    hipLaunchKernelGGL((combine_kernel<DP, TILE>), dim3((unsigned)((rows + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int DP, int GC>
hipError_t launch_attend_p(const Plan &p, const AttendArgs &a, int cus, hipStream_t st, const AttendEvents &ev) {
    const bool tile = a.out == nullptr;   // the kv mask comes with decode only
    if (p.p16) {
        if (tile) return launch_attend_t<DP, GC, true, true, false>(a, cus, st, ev);
        return a.mask ? launch_attend_t<DP, GC, true, false, true>(a, cus, st, ev)
                      : launch_attend_t<DP, GC, true, false, false>(a, cus, st, ev);
    }
    if (tile) return launch_attend_t<DP, GC, false, true, false>(a, cus, st, ev);
    return a.mask ? launch_attend_t<DP, GC, false, false, true>(a, cus, st, ev)
                  : launch_attend_t<DP, GC, false, false, false>(a, cus, st, ev);
}

template <int DP>
hipError_t launch_attend_g(const Plan &p, const AttendArgs &a, int cus, hipStream_t st, const AttendEvents &ev) {
    switch (p.gc) {
        case 1: return launch_attend_p<DP, 1>(p, a, cus, st, ev);
        case 2: return launch_attend_p<DP, 2>(p, a, cus, st, ev);
        case 4: return launch_attend_p<DP, 4>(p, a, cus, st, ev);
        default:
            if constexpr (DP <= 128) return launch_attend_p<DP, 8>(p, a, cus, st, ev);
            return hipErrorInvalidValue;
    }
}

int grid_1d(int64_t n, int per) {
    int64_t b = (n + per - 1) / per;
    if (b > 65536) b = 65536;
    return b < 1 ? 1 : (int)b;
}

}  // namespace

Plan choose_plan(int G, int D, int bs) {
    Plan p;
    p.dp = D <= 64 ? 64 : (D <= 128 ? 128 : 256);
    const int gmax = p.dp == 256 ? 4 : 8;
    int gc = 1;
    while (gc < G && gc < gmax) gc *= 2;
    p.gc = gc;
    p.nhc = (G + gc - 1) / gc;
    p.p16 = (bs % 16) == 0;
    return p;
}

hipError_t launch_attend(const Plan &p, const AttendArgs &a, int cus, hipStream_t st,
                         const AttendEvents &ev) {
    switch (p.dp) {
        case 64: return launch_attend_g<64>(p, a, cus, st, ev);
        case 128: return launch_attend_g<128>(p, a, cus, st, ev);
        default: return launch_attend_g<256>(p, a, cus, st, ev);
    }
}

hipError_t launch_reset(float *m, float *l, float *o, int64_t rows, int D, hipStream_t st) {
    hipLaunchKernelGGL(reset_kernel, dim3(grid_1d(rows * D, 256)), dim3(256), 0, st, m, l, o, rows, D);
    return hipGetLastError();
}

hipError_t launch_zero_ints(int32_t *p, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL(zero_ints_kernel, dim3(grid_1d(n, 256)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_finalize(const float *l, const float *o, uint16_t *out, int64_t rows, int D,
                           hipStream_t st) {
    hipLaunchKernelGGL(finalize_kernel, dim3(grid_1d(rows * D, 256)), dim3(256), 0, st, l, o, out,
                       rows, D);
    return hipGetLastError();
}

}  // namespace pda
