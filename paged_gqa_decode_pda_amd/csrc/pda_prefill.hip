// gfx950 (CDNA4) kernels for paged grouped-query prefill: a chunk of q_len
// query tokens per sequence, the sequence's newest tokens (their keys already
// in the paged cache), attends over the sequence's listed tokens.  Query i of
// a sequence listing P tokens sits at position P - q_len + i; with the causal
// switch it keeps keys up to its own position, and an optional keep-mask
// [batch, q_len, kv_len] removes positions on top of that (AstrAI "CUDA
// Kernels": the "Overview" table's prefill kernel, section "Python Wrappers"
// for is_causal, the mask and the blhd layout, section "Attention Backend"
// for prefill next to decode).
//
// With q_len * G query rows per kv head the scores are a dense contraction,
// so both products run on v_mfma_f32_16x16x32_bf16:
//   scores, transposed: S^T (16 tokens x 16 rows) = K (A operand, 16 token
//      rows from the ring below) x Q^T (B operand, the q rows).
//      Lane l gets rows l%16 and tokens 4(l/16) + i, i = 0..3, so two
//      16-token halves leave lane l exactly the 8 weights that the B operand
//      of the next product needs from row l%16: no transpose of P.
//   output, transposed: O^T (16 head-dim elements x 16 rows) += V^T (A
//      operand) x P^T (B operand), 32 tokens deep, with the 32 tokens taken in
//      the order (4(l/16) .. +3 of half 0, the same of half 1) that the
//      scores left in the lanes.  V^T's lanes need 8 tokens of one column,
//      so V is read back from LDS with 2-byte transposed reads (the 16-byte
//      chunks of a V row stored XOR-swizzled by the row, so the rows one
//      read covers fall on disjoint banks).  O^T's lanes hold row l%16, so
//      the online softmax rescale of a row never leaves its lane.
//
// Work items: (sequence, kv split, kv head, group of four row tiles); a
// workgroup takes one, each of its four waves one row tile (RB row blocks of
// 16 query rows, rows r = i * G + (h - g G) of kv head g), and they stream
// the split's tokens in steps of 32 through three-stage rings in LDS: K and
// V of a step are loaded once for the four waves, straight from memory into
// LDS (gfx950's global_load_lds_dwordx4, a quarter of the loads per wave),
// and every wave reads them from the rings (K in exactly the product's
// operand layout).  The step loop is pipelined across steps: iteration st
// computes P.V of step st - 1 and the scores of step st + 1 on the matrix
// cores beside the weights of step st on the vector ALU, so each wave
// interleaves the two kinds of work; K is loaded two steps ahead and V
// one.  One barrier per iteration: behind it every wave's loads that the
// iteration reads have landed and every wave is done with the stages that
// the iteration's loads overwrite.  Units (sequence, kv split, kv head) are
// dealt round-robin to the eight XCDs, longest first when there are few
// enough (sequence, split) pairs to rank in each workgroup, and a unit's row
// tiles, which read the same pages, run on consecutive waves of one XCD.
// A sequence whose tokens fit one split gets its bf16 result directly;
// otherwise each item leaves (m, l, o) partials for prefill_merge_kernel.
#include <type_traits>

#include "pda_internal.h"
#include "pda_device.h"

namespace pda {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfSortPairs = 64 * kPfWaves;   // one (sequence, split) pair per thread
constexpr int kPfThreads = 64 * kPfWaves;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;

// One stage of the ring: a 32-token step's K, [half][chunk] blocks of 64
// lanes x 16 bytes in the score product's A-operand layout (lane l: token
// l % 16 of the half, elements 32 c + 8 (l / 16) .. + 7), then its V, 32
// rows of 2 DP bytes whose 16-byte chunk c of row r sits at chunk position
// c ^ 2 (r % 4): a transposing read takes 8 bytes of the same 32-byte piece
// from each of 4 consecutive rows per 16 lanes, and the swizzle puts those
// four pieces on disjoint groups of 8 banks whatever the pitch.
template <int DP>
struct PfStage {
    static constexpr int NCK = DP / 32;          // 32-element chunks of the head dim
    static constexpr int CPR = DP / 8;           // 16-byte chunks per V row
    static constexpr int RPI = 64 / CPR;         // V rows per load instruction
    static constexpr int NV = 32 / RPI;          // V load instructions per step
    static constexpr int NJ = 2 * NCK + NV;      // load instructions per step (of 1 KB each)
    static constexpr int KBYTES = 2 * NCK * 1024;
    static constexpr int PITCH = 2 * DP;
    static constexpr int BYTES = KBYTES + 32 * PITCH;
};
constexpr int kPfStages = 3;
__device__ __forceinline__ int vswz(int row) { return 2 * (row & 3); }

// s_waitcnt vmcnt(n) (expcnt, lgkmcnt left at their maxima), n < 64.
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }

// A step's K from its ring stage: N reads of 16 bytes per lane at p + 1024 j
// (p = the stage plus 16 * lane), waited for inside the block.  The ring's
// data comes from DMA loads the caller has waited for (its own) and fenced
// with a barrier (everyone's); written as asm because the compiler, which
// cannot tell the stages apart, would otherwise wait for every load in
// flight, the later steps' too, before the first read.  The outputs are
// early-clobber: a read's result may land before a later read of the block
// has taken its address, so no output may share the address register.
#define PF_RD(j) "ds_read_b128 %" #j ", %[p] offset:" #j "*1024\n"
__device__ __forceinline__ void lds_read_k(u32x4 (&k)[4], const lds_u8_t *p) {
    asm volatile(PF_RD(0) PF_RD(1) PF_RD(2) PF_RD(3) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
                 : [p] "v"(p));
}
__device__ __forceinline__ void lds_read_k(u32x4 (&k)[8], const lds_u8_t *p) {
    asm volatile(PF_RD(0) PF_RD(1) PF_RD(2) PF_RD(3) PF_RD(4) PF_RD(5) PF_RD(6) PF_RD(7)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]),
                   "=&v"(k[7])
                 : [p] "v"(p));
}
__device__ __forceinline__ void lds_read_k(u32x4 (&k)[16], const lds_u8_t *p) {
    asm volatile(PF_RD(0) PF_RD(1) PF_RD(2) PF_RD(3) PF_RD(4) PF_RD(5) PF_RD(6) PF_RD(7) PF_RD(8)
                 PF_RD(9) PF_RD(10) PF_RD(11) PF_RD(12) PF_RD(13) PF_RD(14) PF_RD(15)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]),
                   "=&v"(k[7]), "=&v"(k[8]), "=&v"(k[9]), "=&v"(k[10]), "=&v"(k[11]), "=&v"(k[12]),
                   "=&v"(k[13]), "=&v"(k[14]), "=&v"(k[15])
                 : [p] "v"(p));
}
#undef PF_RD

// Transposed V reads of head-dim blocks 4 m .. 4 m + 3 from a ring stage:
// block 4 m + j at b[j] + OFF (rows 0 .. 15) and b[j] + OFF + HI (rows 16 ..
// 31), waited for inside the block (for the reason given at lds_read_k).
template <int OFF, int HI>
__device__ __forceinline__ void lds_read_vt4(i16x4_t (&lo)[4], i16x4_t (&hi)[4], const lds_u8_t *b0,
                                             const lds_u8_t *b1, const lds_u8_t *b2, const lds_u8_t *b3) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%c12\n"
        "ds_read_b64_tr_b16 %1, %9 offset:%c12\n"
        "ds_read_b64_tr_b16 %2, %10 offset:%c12\n"
        "ds_read_b64_tr_b16 %3, %11 offset:%c12\n"
        "ds_read_b64_tr_b16 %4, %8 offset:%c13\n"
        "ds_read_b64_tr_b16 %5, %9 offset:%c13\n"
        "ds_read_b64_tr_b16 %6, %10 offset:%c13\n"
        "ds_read_b64_tr_b16 %7, %11 offset:%c13\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]),
          "=&v"(hi[3])
        : "v"(b0), "v"(b1), "v"(b2), "v"(b3), "n"(OFF), "n"(OFF + HI));
}

// 16 bytes per lane from global memory into LDS at dst + 16 * lane (dst
// wave-uniform; gfx950 global_load_lds_dwordx4, counted on vmcnt like a load).
__device__ __forceinline__ void ld16_lds(const void *src, lds_u8_t *dst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

// The running max a row's weights are taken against moves only when the
// row's true max exceeds it by more than this (log2 units): weights stay
// below 2^kRescaleSlack, and the rescale of the accumulators is rare.
constexpr float kRescaleSlack = 8.f;

__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = max(x, __shfl_xor(x, m, 64));
    return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = min(x, __shfl_xor(x, m, 64));
    return x;
}
__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, shfl_xor(x, m));
    return x;
}

// Tokens sequence s lists: its first `cnt` pages, all full except the last.
__device__ __forceinline__ int seq_tokens_pf(const PrefillArgs &a, int s) {
    const int cnt = clampi(a.counts[s], 0, a.cap);
    if (cnt == 0) return 0;
    return (cnt - 1) * a.bs + clampi(a.lastv ? a.lastv[s] : a.lv_default, 0, a.bs);
}

__device__ __forceinline__ int or16(int x) {   // OR over the 16 lanes of a row
    x |= __shfl_xor(x, 1, 64);
    x |= __shfl_xor(x, 2, 64);
    x |= __shfl_xor(x, 4, 64);
    return x | __shfl_xor(x, 8, 64);
}

// 16-byte load at a byte offset (under 2^32) from a wave-uniform base, so the
// address is a scalar base plus a 32-bit lane offset.
__device__ __forceinline__ u32x4 ld16_at(const uint16_t *base, uint32_t byte_off) {
    return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(base) + byte_off);
}

// Up to 32 rows per wave (head dim up to 128) the registers fit two waves
// per SIMD (two workgroups per CU): while one computes at raised priority
// the other issues its loads or waits at its barrier; 64 rows need the whole
// register file of one wave.
template <int DP, int RB, bool MASK, bool P16, bool LAPS>
__global__ void __launch_bounds__(kPfThreads, (DP <= 128 && RB <= 2) ? 2 : 1) prefill_kernel(const PrefillArgs a) {
    using SG = PfStage<DP>;
    constexpr int NCK = SG::NCK, CPR = SG::CPR, RPI = SG::RPI, NV = SG::NV, NJ = SG::NJ;
    constexpr int NDB = DP / 16;          // 16-element blocks of the head dim (output)
    constexpr int PITCH = SG::PITCH;
    constexpr int SHARE = NJ / kPfWaves;  // load instructions per wave and step
    static_assert(NJ % kPfWaves == 0, "every wave takes the same share of a step's loads");
    __shared__ __attribute__((aligned(16))) unsigned char ring[kPfStages * SG::BYTES];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qd = lane >> 4, col = lane & 15;
    const u32x4 kOnes = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0 pairs
    lds_u8_t *ring_lds = (lds_u8_t *)&ring[0];   // the LDS address space
    // transposing reads of V: lane (qd, c) reads row 4 qd + c/4 (of each
    // half), bytes 8 (c % 4) .. + 8 of the 32-byte piece of head-dim block n,
    // which the swizzle stores at piece n ^ (c/4) of the row (row % 4 ==
    // c/4); for n = 4 m + j that is 128 m + 32 (j ^ c/4): four lane offsets
    // plus an immediate
    uint32_t tr_b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        tr_b[j] = (uint32_t)(SG::KBYTES + (4 * qd + (col >> 2)) * PITCH + 8 * (col & 3) + 32 * (j ^ (col >> 2)));

    // Work assignment.  Hardware workgroup b runs on XCD b % 8 (the grid is
    // a multiple of 8).  Units (sequence, split, kv head), kv head fastest,
    // are dealt round-robin to the XCDs, so each XCD gets an even share of
    // every sequence; XCD x runs its units in turn, a unit's tile groups on
    // its workgroups (they read the same pages through one L2).
    // When the workgroups take more than one round of the CUs and there are
    // at most kPfSortPairs (sequence, split) pairs, the units are taken
    // longest first, so the launch ends with short work.
    __shared__ int pair_len[kPfSortPairs];
    __shared__ int pair_order[kPfSortPairs];
    const int b = (int)blockIdx.x;
    const int npairs = a.S * a.nsplit;
    const bool sorted = a.longest_first != 0 && npairs <= kPfSortPairs;
    if (sorted) {
        const int t = threadIdx.x;
        int len = -1;
        if (t < npairs) {
            const int st_ = t / a.nsplit;
            len = clampi(seq_tokens_pf(a, st_) - (t - st_ * a.nsplit) * a.span, 0, a.span);
            pair_len[t] = len;
        }
        __syncthreads();
        if (t < npairs) {   // rank by length, descending; ties in index order
            int rank = 0;
            for (int j = 0; j < npairs; ++j) {
                const int lj = pair_len[j];
                rank += (lj > len || (lj == len && j < t)) ? 1 : 0;
            }
            pair_order[rank] = t;
        }
        __syncthreads();
    }
    // Each workgroup walks its XCD's list of tile groups: position r, then
    // 2R - 1 - r, then 2R + r, ... (R workgroups per XCD, at most as many as
    // are resident), so no workgroup waits for dispatch and, with the list
    // longest first, each pairs long work with short.  Without LAPS (the list
    // fits the resident workgroups) there is one lap.  Every wave of the
    // workgroup takes the same path through these loops (the barriers).
    const int R = (int)(gridDim.x >> 3);
    const int ntg = (a.ntiles + kPfWaves - 1) / kPfWaves;   // tile groups per unit
    for (int64_t lap = 0; LAPS || lap == 0; ++lap) {
        const int64_t r = (lap & 1) ? (R - 1 - (b >> 3)) : (b >> 3);
        const int64_t pos = lap * R + r;   // position in XCD b % 8's list of tile groups
        const int64_t k = pos / ntg;
        const int tg = (int)(pos - k * ntg);
        const int rt = tg * kPfWaves + w;   // this wave's row tile
        const bool have = rt < a.ntiles;    // a wave past the unit's last tile only loads
        const int64_t u = (b & 7) + 8 * k;
        if (u >= (int64_t)npairs * a.Hkv) break;   // positions only grow with lap
        const int g = (int)(u % a.Hkv);
        int pair = (int)(u / a.Hkv);
        if (sorted) pair = pair_order[pair];
        const int sp = pair % a.nsplit;
        const int s = pair / a.nsplit;

        const int P = seq_tokens_pf(a, s);
        const int span = a.span;
        const int nsp = P > 0 ? (P + span - 1) / span : 0;
        if (sp >= (nsp > 0 ? nsp : 1)) continue;
        const bool direct = nsp <= 1;

        // this lane's rows, one per row block: r = rt 16 RB + 16 b + col
        const int QG = a.Q * a.G;
        int lim[RB];            // last key position the row keeps (-1: none)
        int64_t rowid[RB];      // (s Q + i) Hq + h, or -1 past the chunk
        const uint8_t *mrow[RB];  // the row's keep-mask bytes (with a mask)
        int lim_min = 0x7fffffff;
        u32x4 qb[RB][NCK];
    #pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = rt * 16 * RB + 16 * rb + col;
            const bool ok = have && r < QG;
            const int i = ok ? r / a.G : 0;
            const int h = g * a.G + (ok ? r - i * a.G : 0);
            rowid[rb] = ok ? ((int64_t)s * a.Q + i) * a.Hq + h : -1;
            lim[rb] = ok ? (a.causal ? P - a.Q + i : P - 1) : -1;
            mrow[rb] = MASK ? a.mask + (int64_t)s * a.mask_ss + (int64_t)i * a.mask_qs : nullptr;
            if (ok) lim_min = min(lim_min, lim[rb]);
            const uint16_t *qp = a.q + (ok ? rowid[rb] : 0) * a.D;
    #pragma unroll
            for (int c = 0; c < NCK; ++c) {
                const int d0 = 32 * c + 8 * qd;
                qb[rb][c] = (ok && d0 < a.D) ? ld16(qp + d0) : u32x4{0, 0, 0, 0};
            }
        }
        lim_min = __builtin_amdgcn_readfirstlane(wave_min_i(lim_min));
        // the workgroup's steps go as far as its last row keeps keys (the same
        // in every wave); a wave's rows past their own limit mask the tokens
        const int rlast = min((tg + 1) * kPfWaves * 16 * RB, QG) - 1;
        const int lim_g = a.causal ? P - a.Q + rlast / a.G : P - 1;
        const int t0 = sp * span;
        const int t1 = min(min(t0 + span, P), lim_g + 1);
        const int nst = t1 > t0 ? (t1 - t0 + 31) >> 5 : 0;

        // Online-softmax state per row block: the reference max m2 (log2
        // units), the threshold thr = m2 + slack, the offset the weights are
        // taken against (mw: m2, or 0 while the row has kept nothing, so that
        // its -inf scores still give weight 0), the pending rescale factor,
        // the weight sum (every element of lacc) and O.
        float m2[RB], thr[RB], mw[RB], alpha[RB];
        f32x4_t lacc[RB];
        f32x4_t acc[RB][NDB];
    #pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            m2[rb] = -INFINITY;
            thr[rb] = -INFINITY;
            mw[rb] = 0.f;
            alpha[rb] = 1.f;
            lacc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
            for (int n = 0; n < NDB; ++n) acc[rb][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

        const int32_t *brow = a.blocks + (int64_t)s * a.cap;
        const int64_t gk = (int64_t)g * a.kvh;
        // This wave's share of a step's loads: instructions j = w + 4 i.  The
        // first NKI are K instructions (j < 2 NCK): half j / NCK, chunk j %
        // NCK, lane l loading token l % 16 of the half, elements kdc[i] (32
        // chunk + 8 (l / 16); past head_dim it re-reads chunk 0, where q is
        // 0).  The other NVI are V instructions v = w + 4 (i - NKI): rows RPI
        // v .. + RPI - 1 of the step, lane l at chunk position l % CPR of row
        // RPI v + l / CPR, so it loads that row's chunk (l % CPR) ^ 2 (row %
        // 4) (past head_dim chunk 0, never stored out).  Offsets in bytes
        // from the first row of the instruction's half, for steps whose two
        // 16-token halves each lie inside one page.
        constexpr int NKI = NCK / 2, NVI = NV / 4;
        static_assert(NKI + NVI == SHARE && NKI >= 1 && NVI >= 1, "load shares");
        int khf[NKI], kdc[NKI], vhf[NVI], vtok[NVI], vdc[NVI];
        uint32_t kob[NKI], vob[NVI];
    #pragma unroll
        for (int i = 0; i < NKI; ++i) {
            const int j = w + kPfWaves * i;
            khf[i] = j / NCK;
            const int d0 = 32 * (j - khf[i] * NCK) + 8 * qd;
            kdc[i] = d0 < a.D ? d0 : 0;
            kob[i] = 2u * (uint32_t)(col * (int)a.tok + kdc[i]);
        }
    #pragma unroll
        for (int i = 0; i < NVI; ++i) {
            const int row = RPI * (w + kPfWaves * i) + lane / CPR;   // row of the step
            vhf[i] = (RPI * (w + kPfWaves * i)) / 16;
            vtok[i] = row;
            const int vd = 8 * ((lane % CPR) ^ vswz(row));
            vdc[i] = vd < a.D ? vd : 0;
            vob[i] = 2u * (uint32_t)((row - 16 * vhf[i]) * (int)a.tok + vdc[i]);
        }

        // Steps that address rows one by one (a half crossing a page, or the
        // partial last step) take page ids from a 64-page window held one id
        // per lane.  The K loads run two steps ahead of the V loads, so each
        // has its own window; a window moves forward only (steps come in
        // order) and waits for its load where it moves.
        int cbk = t0 / a.bs, cbv = cbk;   // first page of each window
        int bidk = brow[min(cbk + lane, a.cap - 1)];
        int bidv = bidk;
        auto window_for = [&](int st, int &cb, int &bidvec) __attribute__((always_inline)) {
            const int tb = t0 + 32 * st;
            const int last = min(tb + 31, t1 - 1);
            if (page_of((uint32_t)last, a.bs_magic) - cb >= 64) {
                cb = page_of((uint32_t)tb, a.bs_magic);
                bidvec = brow[min(cb + lane, a.cap - 1)];
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
        };
        // element offset of token t's row (kv head g); t must be listed and
        // inside the window
        auto row_in = [&](int t, int bidvec, int cb) __attribute__((always_inline)) -> int64_t {
            const int pg = page_of((uint32_t)t, a.bs_magic);
            const int bid = __shfl(bidvec, pg - cb, 64);
            return (int64_t)bid * a.blk + gk + (int64_t)(t - pg * a.bs) * a.tok;
        };

        // Steps whose halves each lie inside one page address their loads
        // from the halves' first rows.  Their page ids come through the
        // scalar cache (the block table is read-only here, so the constant
        // address space may serve it), fetched at the end of the iteration
        // before the one that issues the step's K: the fetch is in flight
        // through the barrier wait, not in front of the LDS reads, which wait
        // for every scalar load too.  The half bases are computed once, for
        // the K loads, and kept for the V loads one iteration later.
        const __attribute__((address_space(4))) int32_t *brow_c =
            (const __attribute__((address_space(4))) int32_t *)brow;
        int pf_st = -1, pf_b[2] = {0, 0}, pf_r[2] = {0, 0};   // prefetched: step, page ids, rows in page
        auto prefetch = [&](int st) __attribute__((always_inline)) {
            const int tb = t0 + 32 * st;
    #pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int pg = page_of((uint32_t)(tb + 16 * hf), a.bs_magic);
                pf_b[hf] = brow_c[pg];
                pf_r[hf] = tb + 16 * hf - pg * a.bs;
            }
            pf_st = st;
        };
        // first element of each half's first row (kv head g); the strides are
        // below 2^32 and in-page offsets below 2^31 (checked by the host), so
        // 32-bit factors suffice
        int64_t hk[2] = {0, 0}, hv[2] = {0, 0};   // of the K step last issued, of the next V step
        const uint32_t blk32 = (uint32_t)a.blk, tok32 = (uint32_t)a.tok;
        auto uniform_step = [&](int st) __attribute__((always_inline)) { return P16 && t0 + 32 * st + 32 <= t1; };
        auto shift_q = [&]() __attribute__((always_inline)) {
            hv[0] = hk[0];
            hv[1] = hk[1];
        };
        // This wave's share of step j's K loads into stage j % kPfStages (its
        // half bases into hk), and of step j's V loads (its half bases in hv).
        auto issue_k = [&](int j) __attribute__((always_inline)) {
            lds_u8_t *stg = ring_lds + (j % kPfStages) * SG::BYTES;
            if (uniform_step(j)) {
                if (pf_st != j) prefetch(j);
    #pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    hk[hf] = (int64_t)((uint64_t)(uint32_t)pf_b[hf] * blk32 + (uint32_t)pf_r[hf] * tok32) + gk;
    #pragma unroll
                for (int i = 0; i < NKI; ++i)
                    ld16_lds(reinterpret_cast<const char *>(a.k + (khf[i] ? hk[1] : hk[0])) + kob[i],
                             stg + 1024 * (w + kPfWaves * i));
            } else {   // rows past t1 read a listed row (weight 0)
                const int tb = t0 + 32 * j;
                window_for(j, cbk, bidk);
    #pragma unroll
                for (int i = 0; i < NKI; ++i) {
                    const int t = min(tb + 16 * khf[i] + col, t1 - 1);
                    ld16_lds(a.k + row_in(t, bidk, cbk) + kdc[i], stg + 1024 * (w + kPfWaves * i));
                }
            }
        };
        auto issue_v = [&](int j) __attribute__((always_inline)) {
            lds_u8_t *stg = ring_lds + (j % kPfStages) * SG::BYTES + SG::KBYTES;
            if (uniform_step(j)) {
    #pragma unroll
                for (int i = 0; i < NVI; ++i)
                    ld16_lds(reinterpret_cast<const char *>(a.v + (vhf[i] ? hv[1] : hv[0])) + vob[i],
                             stg + 1024 * (w + kPfWaves * i));
            } else {
                const int tb = t0 + 32 * j;
                window_for(j, cbv, bidv);
    #pragma unroll
                for (int i = 0; i < NVI; ++i) {
                    const int t = min(tb + vtok[i], t1 - 1);
                    ld16_lds(a.v + row_in(t, bidv, cbv) + vdc[i], stg + 1024 * (w + kPfWaves * i));
                }
            }
        };
        // Wait until at most nk steps' K loads and nv steps' V loads of this
        // wave are in flight (loads complete in order).
        auto wait_loads = [&](int nk, int nv) __attribute__((always_inline)) {
            const int n = nk * NKI + nv * NVI;
            if (n == 0) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            else if (n == NKI) __builtin_amdgcn_s_waitcnt(vmcnt_wait(NKI));
            else if (n == NVI) __builtin_amdgcn_s_waitcnt(vmcnt_wait(NVI));
            else if (n == NKI + NVI) __builtin_amdgcn_s_waitcnt(vmcnt_wait(NKI + NVI));
            else __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * NKI + NVI));
        };
        auto barrier = [&]() __attribute__((always_inline)) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        };

        // The step loop is pipelined across steps: iteration st computes
        // P.V of step st - 1 and the scores of step st + 1 on the matrix
        // cores and the weights of step st on the vector ALU, all independent
        // of one another, so each wave interleaves the two kinds of work (a
        // wave's matrix-core and vector work overlap; two waves' on one SIMD
        // mostly do not).  Iteration st issues K(st + 2) and V(st + 1) and
        // reads K(st + 1) and V(st - 1), all from stage (step % 3) of the K
        // and V rings: K loads have one iteration to land, V loads two.
        f32x4_t s_cur[RB][2], s_nxt[RB][2];   // scores (transposed) of steps st and st + 1
        u32x4 pb_prev[RB], pb_cur[RB];        // bf16 weights of steps st - 1 and st
        int kp_prev = 0xff, kp_cur = 0xff, kp_nxt = 0xff;   // with a mask: tokens some row keeps
        bool resc = false;                    // a rescale by alpha is pending
    #pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            s_cur[rb][0] = s_cur[rb][1] = s_nxt[rb][0] = s_nxt[rb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            pb_prev[rb] = pb_cur[rb] = u32x4{0, 0, 0, 0};
        }

        // scores of step st from its K (already in registers), transposed:
        // lane -> row col, tokens 16 hf + 4 qd + i
        auto scores = [&](f32x4_t (&sc)[RB][2], const u32x4 (&kf)[2 * NCK]) __attribute__((always_inline)) {
    #pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
    #pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    f32x4_t x = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                    for (int c = 0; c < NCK; ++c)
                        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[hf * NCK + c]),
                                                                    __builtin_bit_cast(bf16x8_t, qb[rb][c]), x,
                                                                    0, 0, 0);
                    sc[rb][hf] = x;
                }
            }
        };
        // The scan of step st's scores: tokens a row does not keep get -inf
        // (a step inside every row's range, and the split's, keeps all and
        // skips the tests); each lane's maximum scaled score against its rows'
        // thresholds.  The reference max of a row moves only when the row's
        // max passes it by more than the slack (a row with nothing kept so far
        // keeps (m, l, o) = (-inf, 0, 0)); while no lane of the wave passes,
        // no row moves and the cross-lane maxima are skipped.  A move takes
        // effect for the weights of step st; the rescale of O and l by alpha
        // waits for P.V of step st - 1 (resc).
        auto scan = [&](int st, f32x4_t (&sc)[RB][2], int &keep_any) __attribute__((always_inline)) {
            const int tb = t0 + 32 * st;
            const bool full = !MASK && tb + 32 <= t1 && tb + 31 <= lim_min;
            keep_any = 0xff;
            if (!full) {
                int ka = 0;
    #pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
    #pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
    #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int t = tb + 16 * hf + 4 * qd + i;
                            bool ok = t < t1 && t <= lim[rb];
                            if constexpr (MASK) ok = ok && mrow[rb][t] != 0;
                            ka |= ok ? 1 << (4 * hf + i) : 0;
                            sc[rb][hf][i] = ok ? sc[rb][hf][i] : -INFINITY;
                        }
                    }
                }
                keep_any = or16(ka);
            }
            float lmx[RB];
            bool pass = false;
    #pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const f32x4_t s0 = sc[rb][0], s1 = sc[rb][1];
                lmx[rb] = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                                fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3]))) *
                          a.scale_log2;
                pass |= lmx[rb] > thr[rb];
            }
            if (__builtin_amdgcn_ballot_w64(pass) != 0) {
    #pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const float mx = max4(lmx[rb]);
                    const bool mv = mx > thr[rb];
                    const float mn = mv ? mx : m2[rb];
                    alpha[rb] = mv ? exp2_fast(m2[rb] - mn) : 1.f;
                    m2[rb] = mn;
                    thr[rb] = mn + kRescaleSlack;
                    mw[rb] = mn == -INFINITY ? 0.f : mn;
                }
                resc = true;
            }
        };
        // bf16 weights of step st (masked scores are -inf: weight 0), for
        // the (row block, half) pairs k0 .. k1 - 1 of the 2 RB
        auto weights = [&](const f32x4_t (&sc)[RB][2], u32x4 (&pb)[RB], auto k0c, auto k1c) __attribute__((always_inline)) {
            constexpr int K0 = decltype(k0c)::value, K1 = decltype(k1c)::value;
    #pragma unroll
            for (int k = K0; k < K1; ++k) {
                const int rb = k >> 1, hf = k & 1;
                float p[4];
    #pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = exp2_fast(fmaf(sc[rb][hf][i], a.scale_log2, -mw[rb]));
                pb[rb][2 * hf] = pack_bf16(p[0], p[1]);
                pb[rb][2 * hf + 1] = pack_bf16(p[2], p[3]);
                // computed here, beside the matrix-core work of the phase (the
                // compiler would otherwise sink it to the end of the iteration)
                asm volatile("" ::"v"(pb[rb][2 * hf]), "v"(pb[rb][2 * hf + 1]));
            }
        };
        // P.V of the step in ring stage stg with weights pb (keep_any: with a
        // mask, the tokens some row keeps; the others' V may hold anything
        // and is zeroed).  l: the same product with a block of ones for V^T
        // sums each row's weights exactly as rounded for P.V.
        auto pv = [&](const lds_u8_t *stg, const u32x4 (&pb)[RB], int keep_any) __attribute__((always_inline)) {
    #pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                lacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kOnes),
                                                                   __builtin_bit_cast(bf16x8_t, pb[rb]), lacc[rb],
                                                                   0, 0, 0);
            uint32_t vkeep = 0xffffffffu;
            if constexpr (MASK) {
                if (__builtin_amdgcn_ballot_w64(keep_any != 0xff) != 0) vkeep = 0;   // decided per element
            }
            // A = V^T block n, lane (qd, col) holding column 16 n + col of
            // tokens 4 qd .. 4 qd + 3 of each half.  A transposing LDS read
            // (ds_read_b64_tr_b16) gives lane i of each 16-lane group element
            // i % 4 of the 8-byte chunks read by lanes i / 4 + 4 j, j = 0..3;
            // so lane (qd, c) points at row 4 qd + c / 4 (of each half),
            // elements 16 n + 4 (c % 4) .. + 3.  Head-dim blocks four at a
            // time: their transposed reads, then their products.
            auto pv4 = [&](auto mc) {
                constexpr int M = decltype(mc)::value;
                i16x4_t lo4[4], hi4[4];
                lds_read_vt4<128 * M, 16 * PITCH>(lo4, hi4, stg + tr_b[0], stg + tr_b[1], stg + tr_b[2],
                                                  stg + tr_b[3]);
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = 4 * M + j;
                    u32x4 A = {__builtin_bit_cast(u32x2, lo4[j])[0], __builtin_bit_cast(u32x2, lo4[j])[1],
                               __builtin_bit_cast(u32x2, hi4[j])[0], __builtin_bit_cast(u32x2, hi4[j])[1]};
                    if constexpr (MASK) {
                        if (vkeep == 0) {
    #pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const uint32_t m = ((keep_any >> (2 * e)) & 1 ? 0xffffu : 0u) |
                                                   ((keep_any >> (2 * e + 1)) & 1 ? 0xffff0000u : 0u);
                                A[e] &= m;
                            }
                        }
                    }
    #pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        acc[rb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A),
                                                                             __builtin_bit_cast(bf16x8_t, pb[rb]),
                                                                             acc[rb][n], 0, 0, 0);
                }
            };
            static_assert(NDB % 4 == 0 && NDB <= 16, "head-dim blocks in groups of four");
            pv4(std::integral_constant<int, 0>{});
            if constexpr (NDB > 4) pv4(std::integral_constant<int, 1>{});
            if constexpr (NDB > 8) {
                pv4(std::integral_constant<int, 2>{});
                pv4(std::integral_constant<int, 3>{});
            }
        };

        // Iteration st of the pipeline; PV, NEXT, W: whether step st - 1, st
        // + 1, st exist (the same in every wave).
        auto iter = [&](int st, auto pv_c, auto next_c, auto w_c) __attribute__((always_inline)) {
            constexpr bool PV = decltype(pv_c)::value, NEXT = decltype(next_c)::value, W = decltype(w_c)::value;
            // this wave's loads of K(st + 1) and V(st - 1) have landed (those
            // of V(st), issued after K(st + 1), may still be in flight), then
            // everyone's; every wave is past iteration st - 1, which read the
            // stages that K(st + 2) and V(st + 1) take
            wait_loads(0, st < nst ? 1 : 0);
            barrier();
            if (st + 2 < nst) issue_k(st + 2);
            if (st + 1 < nst) issue_v(st + 1);
            shift_q();
            if (have) {
                // two phases, each pairing matrix-core work with half of the
                // weights: P.V of step st - 1, then the scores of step st + 1
                // (the phase boundaries keep the compiler from hoisting the K
                // read, and with it 2 NCK registers, into the first)
                constexpr std::integral_constant<int, 0> k0{};
                constexpr std::integral_constant<int, RB> kh{};
                constexpr std::integral_constant<int, 2 * RB> k2{};
                // the compute runs at raised wave priority: a SIMD's other
                // wave, while it issues its loads or waits at the barrier,
                // takes the issue cycles this one leaves (measured: 7 % faster
                // than equal priorities)
                __builtin_amdgcn_s_setprio(1);
                if constexpr (PV) pv(ring_lds + ((st + 2) % kPfStages) * SG::BYTES, pb_prev, kp_prev);
                if constexpr (W) weights(s_cur, pb_cur, k0, kh);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (NEXT) {
                    u32x4 kflat[2 * NCK];
                    lds_read_k(kflat, ring_lds + ((st + 1) % kPfStages) * SG::BYTES + 16 * lane);
                    scores(s_nxt, kflat);
                }
                if constexpr (W) weights(s_cur, pb_cur, kh, k2);
                __builtin_amdgcn_sched_barrier(0);
                // the rescale a move at step st asks for, after P.V of step st - 1
                if (resc) {
    #pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
    #pragma unroll
                        for (int n = 0; n < NDB; ++n) acc[rb][n] *= alpha[rb];
                        lacc[rb] *= alpha[rb];
                    }
                    resc = false;
                }
                if constexpr (NEXT) scan(st + 1, s_nxt, kp_nxt);
    #pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    pb_prev[rb] = pb_cur[rb];
                    s_cur[rb][0] = s_nxt[rb][0];
                    s_cur[rb][1] = s_nxt[rb][1];
                }
                kp_prev = kp_cur;
                kp_cur = kp_nxt;
                __builtin_amdgcn_s_setprio(0);
            }
            // the page ids of the K step the next iteration issues
            if (st + 3 < nst && uniform_step(st + 3)) prefetch(st + 3);
        };

        // the item's q rows and page ids in registers before the ring's loads
        // start (the compiler would otherwise wait for all loads in flight at
        // every use of them)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        if (nst > 0) {
            // K(0), K(1) and V(0) in flight; wait for K(0)
            issue_k(0);
            shift_q();
            if (1 < nst) issue_k(1);
            issue_v(0);
            shift_q();
            wait_loads(1 < nst ? 1 : 0, 1);
            barrier();
            if (have) {
                u32x4 kflat[2 * NCK];
                lds_read_k(kflat, ring_lds + 16 * lane);
                scores(s_cur, kflat);
                scan(0, s_cur, kp_cur);
            }
            if (2 < nst && uniform_step(2)) prefetch(2);
            const std::true_type T{};
            const std::false_type F{};
            if (nst == 1) {
                iter(0, F, F, T);
                iter(1, T, F, F);
            } else {
                iter(0, F, T, T);
                for (int st = 1; st < nst - 1; ++st) iter(st, T, T, T);
                iter(nst - 1, T, F, T);
                iter(nst, T, F, F);
            }
        }
        // every wave done with the ring before the next item's loads
        barrier();

        // totals: lane l holds O[row col][16 n + 4 qd + i]
    #pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float L = lacc[rb][0];
            if (rowid[rb] < 0) continue;
            if (direct) {
                uint16_t *op = a.out + rowid[rb] * a.D;
                const float inv = L > 0.f ? 1.f / L : 0.f;
    #pragma unroll
                for (int n = 0; n < NDB; ++n) {
                    const int d = 16 * n + 4 * qd;
                    if (d >= a.D) continue;
                    const f32x4_t x = acc[rb][n];
                    *reinterpret_cast<u32x2 *>(op + d) =
                        u32x2{pack_bf16(x[0] * inv, x[1] * inv), pack_bf16(x[2] * inv, x[3] * inv)};
                }
            } else {
                const int64_t pi = rowid[rb] * a.nsplit + sp;
                if (L > 0.f) {
                    float *po = a.part_o + pi * a.D;
    #pragma unroll
                    for (int n = 0; n < NDB; ++n) {
                        const int d = 16 * n + 4 * qd;
                        if (d < a.D) *reinterpret_cast<f32x4_t *>(po + d) = acc[rb][n];
                    }
                }
                if (qd == 0) {
                    a.part_ml[2 * pi] = m2[rb];
                    a.part_ml[2 * pi + 1] = L;
                }
            }
        }
    }
}

// One wave per output row (s, i, h) of a sequence with several splits:
// log-sum-exp merge of its split partials (slots with l = 0 hold no token
// and are skipped, their o never read) into the bf16 output.
template <int DP>
__global__ void __launch_bounds__(kPfThreads) prefill_merge_kernel(const PrefillArgs a) {
    constexpr int E = DP / 64;   // elements per lane
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kPfWaves + (threadIdx.x >> 6);
    const int64_t nrows = (int64_t)a.S * a.Q * a.Hq;
    if (row >= nrows) return;
    const int s = (int)(row / ((int64_t)a.Q * a.Hq));
    const int P = seq_tokens_pf(a, s);
    const int nsp = P > 0 ? (P + a.span - 1) / a.span : 0;
    if (nsp <= 1) return;
    const float *ml = a.part_ml + row * a.nsplit * 2;
    float M = -INFINITY;
    for (int k = lane; k < nsp; k += 64)
        if (ml[2 * k + 1] > 0.f) M = fmaxf(M, ml[2 * k]);
    M = __builtin_amdgcn_readfirstlane(wave_max_f(M));
    float o[E], L = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.f;
    const int d0 = lane * E;
    for (int k = 0; k < nsp; ++k) {
        const float lk = ml[2 * k + 1];
        if (!(lk > 0.f)) continue;
        const float wk = exp2_fast(ml[2 * k] - M);
        L = fmaf(wk, lk, L);
        if (d0 < a.D) {
            const float *po = a.part_o + (row * a.nsplit + k) * a.D + d0;
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = fmaf(wk, po[e], o[e]);
        }
    }
    if (d0 < a.D) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        uint16_t *op = a.out + row * a.D + d0;
#pragma unroll
        for (int e = 0; e < E; ++e) op[e] = f32_to_bf16(o[e] * inv);
    }
}

template <int DP, int RB, bool MASK, bool P16>
hipError_t launch_prefill_t(const PrefillArgs &args, hipStream_t st, const AttendEvents &ev) {
    PrefillArgs a = args;
    // every XCD holds at most ceil(units / 8) units of ceil(ntiles / 4)
    // tile groups each; at most as many workgroups as are resident, each
    // looping over positions
    const int64_t units = (int64_t)a.S * a.nsplit * a.Hkv;
    const int64_t need = (units + 7) / 8 * ((a.ntiles + kPfWaves - 1) / kPfWaves);   // positions per XCD
    const int64_t per_cu = (DP <= 128 && RB <= 2) ? 2 : 1;      // as the launch bounds allow
    const int64_t resident = (a.cus >= 8 ? a.cus / 8 : 1) * per_cu;   // per XCD
    const int64_t nwg = 8 * (need < resident ? need : resident);
    a.longest_first = need > resident ? 1 : 0;
    if (ev.before) {
        hipError_t e = hipEventRecord(ev.before, st);
        if (e != hipSuccess) return e;
    }
    if (need > resident)
        hipLaunchKernelGGL((prefill_kernel<DP, RB, MASK, P16, true>), dim3((unsigned)nwg), dim3(kPfThreads), 0, st, a);
    else
        hipLaunchKernelGGL((prefill_kernel<DP, RB, MASK, P16, false>), dim3((unsigned)nwg), dim3(kPfThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev.after) {
        e = hipEventRecord(ev.after, st);
        if (e != hipSuccess) return e;
    }
    if (a.nsplit > 1) {
        const int64_t rows = (int64_t)a.S * a.Q * a.Hq;
        hipLaunchKernelGGL((prefill_merge_kernel<DP>), dim3((unsigned)((rows + kPfWaves - 1) / kPfWaves)),
                           dim3(kPfThreads), 0, st, a);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

// Instantiated shapes: head dims up to 128 take 1, 2 or 4 row blocks per wave
// (4 only without a mask at 128: with one it would spill), 256 takes one.
int prefill_max_rb(int dp, bool mask) {
    if (dp == 256) return 1;
    if (dp == 128 && mask) return 2;
    return 4;
}

template <int DP, int RB, bool MASK>
hipError_t launch_prefill_p(const PrefillArgs &a, hipStream_t st, const AttendEvents &ev) {
    return a.bs % 16 == 0 ? launch_prefill_t<DP, RB, MASK, true>(a, st, ev)
                          : launch_prefill_t<DP, RB, MASK, false>(a, st, ev);
}

hipError_t launch_prefill(const PrefillArgs &a, int dp, int rb, hipStream_t st, const AttendEvents &ev) {
    const bool m = a.mask != nullptr;
    switch (dp) {
        case 64:
            if (rb == 1) return m ? launch_prefill_p<64, 1, true>(a, st, ev) : launch_prefill_p<64, 1, false>(a, st, ev);
            if (rb == 2) return m ? launch_prefill_p<64, 2, true>(a, st, ev) : launch_prefill_p<64, 2, false>(a, st, ev);
            return m ? launch_prefill_p<64, 4, true>(a, st, ev) : launch_prefill_p<64, 4, false>(a, st, ev);
        case 128:
            if (rb == 1) return m ? launch_prefill_p<128, 1, true>(a, st, ev) : launch_prefill_p<128, 1, false>(a, st, ev);
            if (rb == 2 || m) return m ? launch_prefill_p<128, 2, true>(a, st, ev) : launch_prefill_p<128, 2, false>(a, st, ev);
            return launch_prefill_p<128, 4, false>(a, st, ev);
        default:
            return m ? launch_prefill_p<256, 1, true>(a, st, ev) : launch_prefill_p<256, 1, false>(a, st, ev);
    }
}

}  // namespace pda
