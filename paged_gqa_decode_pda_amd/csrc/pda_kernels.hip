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
//   K: 4 lanes per token, 16 tokens per wave; lane (t = lane/4, j = lane%4)
//      holds the 16-byte chunks 4c + j (c < D_PAD/32) of token t's K row, so
//      each load instruction reads 64 contiguous bytes of 16 rows.  Scores use
//      v_dot2c_f32_bf16 on bf16 pairs and a 2-step quad DPP reduction.
//   V: 16 lanes per token row, 4 rows per wave; lane (r = lane/16, c =
//      lane%16) holds elements [c*D_PAD/16, (c+1)*D_PAD/16) of token 4i + r.
//      Softmax weights move from the K layout to the V layout through LDS.
#include "pda_internal.h"

#include <map>
#include <mutex>
#include <utility>

namespace pda {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWaves = 4;
constexpr int kBigSplits = 4;   // splits per big work item
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// The two bf16 halves of a dword, widened exactly to fp32.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// DPP lane permutations (all source lanes valid for the controls used).
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;   // row_ror:4 (within 16-lane rows)
constexpr int kRowRor8 = 0x128;   // row_ror:8

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Split partials travel between workgroups (possibly on different XCDs, each
// with its own L2) through device-coherent accesses: agent-scope relaxed
// atomic stores and loads, which gfx950 issues with sc1 (written through to,
// and read from, the device coherence point).  No L2 writeback or invalidate
// is needed; a writer only waits for its stores to complete before counting
// its split in.
__device__ __forceinline__ void st_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent_i(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int kWaitVmcnt0 = 0x0F70;   // s_waitcnt vmcnt(0): this wave's loads and stores completed

// Lanes of one wave exchange data through LDS: make prior LDS writes visible
// to the wave's other lanes before the reads that follow.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// binary32 -> bf16, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x2 ld8(const uint16_t *p) { return *reinterpret_cast<const u32x2 *>(p); }

// Tokens of sequence s: the first `cnt` listed pages, all full except the
// last, which holds `lv` valid slots.
__device__ __forceinline__ int seq_tokens(const int32_t *counts, const int32_t *lastv, int lv_default,
                                          int s, int cap, int bs) {
    int cnt = clampi(counts[s], 0, cap);
    if (cnt == 0) return 0;
    int lv = clampi(lastv ? lastv[s] : lv_default, 0, bs);
    return (cnt - 1) * bs + lv;
}

__device__ __forceinline__ int page_of(uint32_t t, uint64_t magic) {
    return (int)(((uint64_t)t * magic) >> 32);
}

// Per-wave registers of one 16-token group.
template <int DP>
struct GroupRegs {
    static constexpr int NCK = DP / 32;   // 16-byte K chunks per lane
    static constexpr int VW = DP / 32;    // V dwords per lane per row step (DP/16 bf16)
    u32x4 k[NCK];
    uint32_t v[4][VW];
};

__device__ __forceinline__ int readlane(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }
__device__ __forceinline__ float readlanef(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Maximum over the 64 lanes of a value that is already equal within each
// 16-lane row: four lane reads, result in a scalar register.
__device__ __forceinline__ float row_values_max(float x) {
    return fmaxf(fmaxf(readlanef(x, 0), readlanef(x, 16)), fmaxf(readlanef(x, 32), readlanef(x, 48)));
}

// Per-wave shared memory.
template <int GC>
struct WaveSmem {
    float p[16][GC];       // softmax weights, K lane layout -> V lane layout
    float wt[GC][64];      // merge: weights of one 64-split chunk
};

// One wave streams the 16-token groups of the token range [t0, t1) of
// sequence s for kv head g and the q heads h0 .. h0 + nh - 1, NBUF groups of
// K/V in flight in registers while it computes.  The page ids are read once
// per 64 pages into one VGPR (lane i holds page cb + i of the sequence's list)
// and picked with readlane (pages of 16k tokens) or a lane shuffle (other
// block sizes), so no table load sits between a group's address and its data.
// On return m2 (log2 units), lsum and acc_o hold the wave's totals in every
// lane: acc_o[h][e] is element col * DP/16 + e of head h.
template <int DP, int GC, bool P16, int NBUF>
__device__ __forceinline__ void wave_pass(const AttendArgs &a, WaveSmem<GC> &ws, int lane, int s,
                                          int g, int h0, int nh, int t0, int t1, int cnt,
                                          float (&m2)[GC], float (&lsum)[GC],
                                          float (&acc_o)[GC][DP / 16]) {
    constexpr int NCK = DP / 32;
    constexpr int VW = DP / 32;      // V dwords per lane per row step
    constexpr int VPL = DP / 16;     // V elements per lane
    constexpr int VC = DP == 64 ? 1 : VW / 4;

    const int ngroups = (t1 - t0 + 15) >> 4;
    const int32_t *brow = a.blocks + (int64_t)s * a.cap;
    const int quad = lane >> 2, ql = lane & 3;
    const int row = lane >> 4, col = lane & 15;

    // Lane-invariant element offsets.  Chunks past head_dim re-read chunk 0
    // of the same row (in bounds); q is zero there, and V lanes past head_dim
    // are never stored.
    int kd[NCK];
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
        const int d0 = 8 * (4 * c + ql);
        kd[c] = d0 < a.D ? d0 : 0;
    }
    int vd[VC];
#pragma unroll
    for (int c = 0; c < VC; ++c) {
        const int e0 = col * VPL + 8 * c;
        vd[c] = e0 < a.D ? e0 : 0;
    }
    const int tok32 = (int)a.tok;
    const int64_t gk = (int64_t)g * a.kvh;

    // q chunks in the K lane layout, zero past head_dim.  Padding heads of a
    // short last head chunk (h >= nh) repeat head nh - 1; their results are
    // never stored.
    u32x4 qr[GC][NCK];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
        const uint16_t *qp = a.q + ((int64_t)s * a.Hq + h0 + min(h, nh - 1)) * a.D;
#pragma unroll
        for (int c = 0; c < NCK; ++c) {
            const u32x4 x = ld16(qp + kd[c]);
            qr[h][c] = 8 * (4 * c + ql) < a.D ? x : u32x4{0, 0, 0, 0};
        }
    }

#pragma unroll
    for (int h = 0; h < GC; ++h) {
        m2[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < VPL; ++e) acc_o[h][e] = 0.f;
    }

    int cb = 0, bidvec = 0;   // page-id window: lane i holds brow[cb + i]
    auto load_window = [&](int first) {
        cb = first;
        bidvec = brow[min(first + lane, cnt - 1)];
    };

    auto issue = [&](int n, GroupRegs<DP> &r) {
        const int gs = t0 + 16 * n;
        if constexpr (P16) {
            const int page = page_of((uint32_t)gs, a.bs_magic);
            const int bid = readlane(bidvec, page - cb);
            const int64_t off = (int64_t)bid * a.blk + gk + (int64_t)(gs - page * a.bs) * a.tok;
            const uint16_t *kb = a.k + off;
            const uint16_t *vb = a.v + off;
#pragma unroll
            for (int c = 0; c < NCK; ++c) r.k[c] = ld16(kb + (quad * tok32 + kd[c]));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ro = (4 * i + row) * tok32;
                if constexpr (DP == 64) {
                    const u32x2 x = ld8(vb + (ro + vd[0]));
                    r.v[i][0] = x[0];
                    r.v[i][1] = x[1];
                } else {
#pragma unroll
                    for (int c = 0; c < VC; ++c) {
                        const u32x4 x = ld16(vb + (ro + vd[c]));
                        r.v[i][4 * c + 0] = x[0];
                        r.v[i][4 * c + 1] = x[1];
                        r.v[i][4 * c + 2] = x[2];
                        r.v[i][4 * c + 3] = x[3];
                    }
                }
            }
        } else {
            // tokens past t1 read the group's first token instead (in bounds)
            const int tk = gs + quad < t1 ? gs + quad : gs;
            const int pk = page_of((uint32_t)tk, a.bs_magic);
            const int bk = __shfl(bidvec, pk - cb, 64);
            const uint16_t *kp = a.k + ((int64_t)bk * a.blk + gk + (int64_t)(tk - pk * a.bs) * a.tok);
#pragma unroll
            for (int c = 0; c < NCK; ++c) r.k[c] = ld16(kp + kd[c]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tv = gs + 4 * i + row < t1 ? gs + 4 * i + row : gs;
                const int pv = page_of((uint32_t)tv, a.bs_magic);
                const int bv = __shfl(bidvec, pv - cb, 64);
                const uint16_t *vp = a.v + ((int64_t)bv * a.blk + gk + (int64_t)(tv - pv * a.bs) * a.tok);
                if constexpr (DP == 64) {
                    const u32x2 x = ld8(vp + vd[0]);
                    r.v[i][0] = x[0];
                    r.v[i][1] = x[1];
                } else {
#pragma unroll
                    for (int c = 0; c < VC; ++c) {
                        const u32x4 x = ld16(vp + vd[c]);
                        r.v[i][4 * c + 0] = x[0];
                        r.v[i][4 * c + 1] = x[1];
                        r.v[i][4 * c + 2] = x[2];
                        r.v[i][4 * c + 3] = x[3];
                    }
                }
            }
        }
    };

    auto compute = [&](GroupRegs<DP> &r, int n) {
        const int gs = t0 + 16 * n;
        // scores of token gs + quad for every head of the chunk
        float acc[GC];
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            float x = 0.f;
#pragma unroll
            for (int c = 0; c < NCK; ++c) {
                x = dot2(qr[h][c][0], r.k[c][0], x);
                x = dot2(qr[h][c][1], r.k[c][1], x);
                x = dot2(qr[h][c][2], r.k[c][2], x);
                x = dot2(qr[h][c][3], r.k[c][3], x);
            }
            x += dpp<kQuadSwap1>(x);
            x += dpp<kQuadSwap2>(x);
            acc[h] = x;
        }
        const bool valid = gs + quad < t1;
        float sc[GC];
        bool grow = false;
        float alpha[GC];
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            sc[h] = valid ? acc[h] * a.scale_log2 : -INFINITY;
            float x = sc[h];
            x = fmaxf(x, dpp<kRowRor4>(x));
            x = fmaxf(x, dpp<kRowRor8>(x));
            const float mn = fmaxf(m2[h], row_values_max(x));
            grow |= mn > m2[h];
            alpha[h] = (mn == -INFINITY) ? 1.f : exp2_fast(m2[h] - mn);
            m2[h] = mn;
        }
        if (grow) {  // uniform: m2 is identical in every lane
#pragma unroll
            for (int h = 0; h < GC; ++h) {
                lsum[h] *= alpha[h];
#pragma unroll
                for (int e = 0; e < VPL; ++e) acc_o[h][e] *= alpha[h];
            }
        }
        float p[GC];
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            p[h] = valid ? exp2_fast(sc[h] - m2[h]) : 0.f;
            lsum[h] += p[h];
        }
        if (ql == 0) {
#pragma unroll
            for (int h = 0; h < GC; ++h) ws.p[quad][h] = p[h];
        }
        // the last group of a range may hold tokens past t1: zero their V so
        // that 0 * (NaN or Inf) never reaches the sums
        if (gs + 16 > t1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = gs + 4 * i + row < t1;
#pragma unroll
                for (int e = 0; e < VW; ++e) r.v[i][e] = ok ? r.v[i][e] : 0u;
            }
        }
        wave_lds_sync();
        // o += p * V, token 4i + row per row step
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float pv[GC];
#pragma unroll
            for (int h = 0; h < GC; ++h) pv[h] = ws.p[4 * i + row][h];
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                const float f0 = bf_lo(r.v[i][e]);
                const float f1 = bf_hi(r.v[i][e]);
#pragma unroll
                for (int h = 0; h < GC; ++h) {
                    acc_o[h][2 * e] = fmaf(pv[h], f0, acc_o[h][2 * e]);
                    acc_o[h][2 * e + 1] = fmaf(pv[h], f1, acc_o[h][2 * e + 1]);
                }
            }
        }
        wave_lds_sync();
    };

    // groups covered by one 64-page window
    const int per_window = P16 ? 4 * a.bs : max(1, (62 * a.bs + 1) / 16);
    for (int c0 = 0; c0 < ngroups; c0 += per_window) {
        const int nc = min(per_window, ngroups - c0);
        load_window(page_of((uint32_t)(t0 + 16 * c0), a.bs_magic));
        // Loads are issued unconditionally (indices past the window re-read
        // its last group, an L2 hit) so that every wait for a group's data
        // counts exactly the younger loads; only the compute is skipped.
        GroupRegs<DP> rb[NBUF];
#pragma unroll
        for (int j = 0; j < NBUF - 1; ++j) issue(c0 + min(j, nc - 1), rb[j]);
        for (int n = 0; n < nc; n += NBUF) {
#pragma unroll
            for (int j = 0; j < NBUF; ++j) {
                issue(c0 + min(n + j + NBUF - 1, nc - 1), rb[(j + NBUF - 1) % NBUF]);
                if (n + j < nc) compute(rb[j], c0 + n + j);
            }
        }
    }

    // Wave totals in every lane: o over the 4 rows, l over the 16 token quads.
#pragma unroll
    for (int h = 0; h < GC; ++h) {
#pragma unroll
        for (int e = 0; e < VPL; ++e) {
            float x = acc_o[h][e];
            x += shfl_xor(x, 16);
            x += shfl_xor(x, 32);
            acc_o[h][e] = x;
        }
        float y = lsum[h];
        y += shfl_xor(y, 4);
        y += shfl_xor(y, 8);
        y += shfl_xor(y, 16);
        y += shfl_xor(y, 32);
        lsum[h] = y;
    }
}

__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, shfl_xor(x, 1));
    x = fmaxf(x, shfl_xor(x, 2));
    x = fmaxf(x, shfl_xor(x, 4));
    x = fmaxf(x, shfl_xor(x, 8));
    x = fmaxf(x, shfl_xor(x, 16));
    return fmaxf(x, shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += shfl_xor(x, 1);
    x += shfl_xor(x, 2);
    x += shfl_xor(x, 4);
    x += shfl_xor(x, 8);
    x += shfl_xor(x, 16);
    return x + shfl_xor(x, 32);
}

// Splits of a sequence: ceil(ntok / span), 0 for an empty sequence.
__device__ __forceinline__ int splits_of(int ntok, int span) { return ntok > 0 ? (ntok + span - 1) / span : 0; }

// Work items of a sequence with nsp splits (prefix mode): nb "big" items of
// kBigSplits consecutive splits cover about 3/4 of the splits, then one item
// per remaining split.  Items are numbered in token order; item k of the
// sequence owns partial slot k, so a sequence has nb + (nsp - nb * kBigSplits)
// slots.
__device__ __forceinline__ int big_items_of(int nsp) { return (3 * nsp) / (4 * kBigSplits); }
__device__ __forceinline__ int slots_of(int nsp, bool prefix_mode) {
    return prefix_mode ? nsp - (kBigSplits - 1) * big_items_of(nsp) : nsp;
}

// Persistent attention kernel.  Work items are (sequence, split, unit), unit =
// (kv head, head chunk) fastest, and every wave takes items on its own from an
// atomic counter, so the waves reading the interleaved kv-head rows of the
// same pages run together and no wave ever waits for another.  A sequence
// with one split gets its result written directly (bf16 o / l for decode, the
// running state folded for a tile); otherwise every split leaves an (m, l, o)
// partial in the workspace for combine_kernel.
template <int DP, int GC, bool P16, int NBUF, bool TILE>
__global__ void __launch_bounds__(kThreads) attend_kernel(const AttendArgs a) {
    constexpr int VPL = DP / 16;
    __shared__ WaveSmem<GC> wsm[kWaves];
    __shared__ int scan[2 * kWaves];
    extern __shared__ int prefix[];   // 2 (S + 1) ints when a.prefix_mode

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int units = a.Hkv * a.nhc;
    const int span = a.bps * a.bs;
    const int row = lane >> 4, col = lane & 15;

    // Work items.  With the prefix (sequences up to kPrefixMaxSeqs), each
    // sequence's splits are grouped: about 3/4 of them, kBigSplits at a time,
    // form "big" items queued first; the rest are single-split items queued
    // after all big ones, so the queue ends with short work.  Decode keeps
    // one small item for an empty sequence so that its zero output row gets
    // written.
    int nbig_pairs = 0, npairs;
    int *pbig = prefix;                 // big items before sequence s
    int *psmall = prefix + a.S + 1;     // small items before sequence s
    if (a.prefix_mode) {
        int carry_b = 0, carry_s = 0;
        for (int base = 0; base < a.S; base += kThreads) {
            const int s = base + tid;
            int nb = 0, ns = 0;
            if (s < a.S) {
                const int nsp = splits_of(seq_tokens(a.counts, a.lastv, a.lv_default, s, a.cap, a.bs), span);
                nb = big_items_of(nsp);
                ns = nsp - nb * kBigSplits;
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
        npairs = a.S * ((a.cap + a.bps - 1) / a.bps);
    }
    const int nitems = npairs * units;
    __syncthreads();

    // Wave gw starts on item gw; later items come from the counter (which
    // counts from the number of waves).  An item is claimed only when the
    // previous one is done, so no item waits behind a busy wave.
    WaveSmem<GC> &ws = wsm[w];
    const int nwaves = (int)gridDim.x * kWaves;
    int it = (int)blockIdx.x * kWaves + w;
    while (it < nitems) {
        int pair = it / units;
        const int unit = it - pair * units;
        int s, split, nspl = 1, slot;   // first split, splits covered, partial slot
        if (a.prefix_mode) {
            const bool big = pair < nbig_pairs;
            const int *pf = big ? pbig : psmall;
            if (!big) pair -= nbig_pairs;
            int lo = 0, hi = a.S;   // the largest s with pf[s] <= pair
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (pf[mid] <= pair) lo = mid;
                else hi = mid;
            }
            s = __builtin_amdgcn_readfirstlane(lo);
            const int j = pair - __builtin_amdgcn_readfirstlane(pf[s]);
            if (big) {
                split = j * kBigSplits;
                nspl = kBigSplits;
                slot = j;
            } else {
                const int nb_s = big_items_of(splits_of(seq_tokens(a.counts, a.lastv, a.lv_default, s, a.cap, a.bs), span));
                split = nb_s * kBigSplits + j;
                slot = nb_s + j;
            }
        } else {
            const int nsp_max = (a.cap + a.bps - 1) / a.bps;
            s = pair / nsp_max;
            split = pair - s * nsp_max;
            slot = split;
        }
        const int g = unit / a.nhc;
        const int hc = unit - g * a.nhc;
        const int h0 = g * a.G + hc * GC;
        const int nh = min(GC, a.G - hc * GC);
        const int cnt = clampi(a.counts[s], 0, a.cap);
        const int ntok = seq_tokens(a.counts, a.lastv, a.lv_default, s, a.cap, a.bs);
        const int nsp = splits_of(ntok, span);
        const int64_t row0 = (int64_t)s * a.Hq + h0;   // first (sequence, q head) row

        if (ntok == 0) {
            // only decode gets here (an empty sequence's single item): zero rows
            if (!TILE && split == 0) {
                for (int idx = lane; idx < nh * a.D; idx += 64) a.out[row0 * a.D + idx] = 0;
            }
        } else if (split < nsp) {
            const int t0 = split * span;
            const int t1 = min(t0 + nspl * span, ntok);
            float m2[GC], lsum[GC], acc_o[GC][VPL];
            wave_pass<DP, GC, P16, NBUF>(a, ws, lane, s, g, h0, nh, t0, t1, cnt, m2, lsum, acc_o);
            // row-0 lanes store elements e0 .. e0 + VPL - 1; with a padded
            // head dim of 256 a lane's slice may straddle head_dim, so every
            // element is checked
            const int e0 = col * VPL;
            const bool store = row == 0 && e0 < a.D;
            if (nsp == 1) {
#pragma unroll
                for (int h = 0; h < GC; ++h) {
                    if (h >= nh) continue;
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
#pragma unroll
                            for (int e = 0; e < VPL; ++e) {
                                if (e0 + e >= a.D) continue;
                                float *po = a.o + r * a.D + e0 + e;
                                *po = fmaf(*po, fs, acc_o[h][e] * fp);
                            }
                        }
                        if (lane == 0) {
                            const float Lt = fmaf(ls, fs, lsum[h] * fp);
                            a.l[r] = Lt;
                            a.m[r] = Lt > 0.f ? Mt * kLn2 : -INFINITY;
                        }
                    } else if (store) {
                        const float L = lsum[h];
#pragma unroll
                        for (int e = 0; e < VPL; ++e)
                            if (e0 + e < a.D) a.out[r * a.D + e0 + e] = L > 0.f ? f32_to_bf16(acc_o[h][e] / L) : 0;
                    }
                }
            } else {
                // a split partial for the combine kernel
#pragma unroll
                for (int h = 0; h < GC; ++h) {
                    if (h >= nh) continue;
                    const int64_t pi = (row0 + h) * a.nsplit + slot;
                    if (store) {
#pragma unroll
                        for (int e = 0; e < VPL; ++e)
                            if (e0 + e < a.D) a.part_o[pi * a.D + e0 + e] = acc_o[h][e];
                    }
                    if (lane == 0) {
                        a.part_ml[2 * pi] = m2[h];
                        a.part_ml[2 * pi + 1] = lsum[h];
                    }
                }
            }
        }
        const int grabbed = lane == 0 ? atomicAdd(&a.ctrl[0], 1) : 0;
        it = nwaves + readlane(grabbed, 0);
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
// state when folding a tile), into the bf16 output or the state.  Split
// weights are formed lane-parallel (lane i <-> split cbase + i); lanes own
// DP/64 consecutive elements of the weighted sums.
template <int DP, bool TILE>
__global__ void __launch_bounds__(kThreads) combine_kernel(const AttendArgs a) {
    constexpr int EPL = DP / 64;
    __shared__ float wts[kWaves][64];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t sh = (int64_t)blockIdx.x * kWaves + w;
    if (sh >= (int64_t)a.S * a.Hq) return;
    const int s = (int)(sh / a.Hq);
    const int span = a.bps * a.bs;
    const int nsp = splits_of(seq_tokens(a.counts, a.lastv, a.lv_default, s, a.cap, a.bs), span);
    if (nsp <= 1) return;   // written by the attention kernel (or an untouched empty tile)
    const int nslot = slots_of(nsp, a.prefix_mode != 0);
    const int d0 = lane * EPL;
    const bool dok = d0 < a.D;   // head_dim is a multiple of 8: a lane's elements are all in or all out
    const float *ml = a.part_ml + sh * a.nsplit * 2;
    const float *po = a.part_o + sh * a.nsplit * a.D;

    const float ls = TILE ? a.l[sh] : 0.f;
    const float ms = TILE ? a.m[sh] * kLog2e : -INFINITY;
    float M = ls > 0.f ? ms : -INFINITY;
    for (int i = lane; i < nslot; i += 64) {
        const float li = ml[2 * i + 1], mi = ml[2 * i];
        if (li > 0.f) M = fmaxf(M, mi);
    }
    M = wave_max(M);

    float L = 0.f, O[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[e] = 0.f;
    if (ls > 0.f) {
        const float f = exp2_fast(ms - M);
        L = ls * f;
        if (dok) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) O[e] = a.o[sh * a.D + d0 + e] * f;
        }
    }
    for (int cb = 0; cb < nslot; cb += 64) {
        const int i = cb + lane;
        float wi = 0.f, li = 0.f;
        if (i < nslot) {
            li = ml[2 * i + 1];
            const float mi = ml[2 * i];
            wi = li > 0.f ? exp2_fast(mi - M) : 0.f;
        }
        wts[w][lane] = wi;
        L += wave_sum(wi * li);
        wave_lds_sync();
        const int n = min(64, nslot - cb);
        if (dok) {
#pragma unroll 8
            for (int j = 0; j < n; ++j) {
                const float f = wts[w][j];
                const float *src = po + (int64_t)(cb + j) * a.D + d0;
#pragma unroll
                for (int e = 0; e < EPL; ++e) O[e] = fmaf(src[e], f, O[e]);
            }
        }
        wave_lds_sync();
    }
    if (TILE) {
        if (dok) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) a.o[sh * a.D + d0 + e] = O[e];
        }
        if (lane == 0) {
            a.l[sh] = L;
            a.m[sh] = L > 0.f ? M * kLn2 : -INFINITY;
        }
    } else if (dok) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) a.out[sh * a.D + d0 + e] = L > 0.f ? f32_to_bf16(O[e] / L) : 0;
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

__global__ void __launch_bounds__(256) finalize_kernel(const float *l, const float *o, uint16_t *out,
                                                       int64_t rows, int D) {
    const int64_t n = rows * D;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float li = l[i / D];
        out[i] = li > 0.f ? f32_to_bf16(o[i] / li) : 0;
    }
}

// Workgroups per compute unit the kernel can hold, cached per (kernel, LDS).
int blocks_per_cu(const void *kernel, size_t dyn_lds) {
    static std::mutex mu;
    static std::map<std::pair<const void *, size_t>, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto key = std::make_pair(kernel, dyn_lds);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, dyn_lds) != hipSuccess || n < 1) n = 1;
    cache[key] = n;
    return n;
}

constexpr int nbuf_for(int dp) { return dp == 256 ? 2 : 3; }   // 16-token K/V groups in flight per wave

template <int DP, int GC, bool P16, bool TILE>
hipError_t launch_attend_t(const AttendArgs &a, int cus, hipStream_t st) {
    auto kernel = attend_kernel<DP, GC, P16, nbuf_for(DP), TILE>;
    const size_t dyn = a.prefix_mode ? 2 * sizeof(int) * ((size_t)a.S + 1) : 0;
    const int64_t per_cu = blocks_per_cu(reinterpret_cast<const void *>(kernel), dyn);
    const int64_t nsp_max = (a.cap + a.bps - 1) / a.bps;
    const int64_t upper = ((int64_t)a.S * nsp_max * a.Hkv * a.nhc + kWaves - 1) / kWaves;
    int64_t nwg = per_cu * cus;
    if (nwg > upper) nwg = upper;
    if (nwg < 1) nwg = 1;
    hipLaunchKernelGGL(kernel, dim3((unsigned)nwg), dim3(kThreads), dyn, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.bps >= a.cap) return e;   // one split per sequence: nothing to combine
    const int64_t rows = (int64_t)a.S * a.Hq;
    hipLaunchKernelGGL((combine_kernel<DP, TILE>), dim3((unsigned)((rows + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int DP, int GC>
hipError_t launch_attend_p(const Plan &p, const AttendArgs &a, int cus, hipStream_t st) {
    const bool tile = a.out == nullptr;
    if (p.p16) return tile ? launch_attend_t<DP, GC, true, true>(a, cus, st) : launch_attend_t<DP, GC, true, false>(a, cus, st);
    return tile ? launch_attend_t<DP, GC, false, true>(a, cus, st) : launch_attend_t<DP, GC, false, false>(a, cus, st);
}

template <int DP>
hipError_t launch_attend_g(const Plan &p, const AttendArgs &a, int cus, hipStream_t st) {
    switch (p.gc) {
        case 1: return launch_attend_p<DP, 1>(p, a, cus, st);
        case 2: return launch_attend_p<DP, 2>(p, a, cus, st);
        case 4: return launch_attend_p<DP, 4>(p, a, cus, st);
        default:
            if constexpr (DP <= 128) return launch_attend_p<DP, 8>(p, a, cus, st);
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

hipError_t launch_attend(const Plan &p, const AttendArgs &a, int cus, hipStream_t st) {
    switch (p.dp) {
        case 64: return launch_attend_g<64>(p, a, cus, st);
        case 128: return launch_attend_g<128>(p, a, cus, st);
        default: return launch_attend_g<256>(p, a, cus, st);
    }
}

hipError_t launch_reset(float *m, float *l, float *o, int64_t rows, int D, hipStream_t st) {
    hipLaunchKernelGGL(reset_kernel, dim3(grid_1d(rows * D, 256)), dim3(256), 0, st, m, l, o, rows, D);
    return hipGetLastError();
}

hipError_t launch_finalize(const float *l, const float *o, uint16_t *out, int64_t rows, int D,
                           hipStream_t st) {
    hipLaunchKernelGGL(finalize_kernel, dim3(grid_1d(rows * D, 256)), dim3(256), 0, st, l, o, out,
                       rows, D);
    return hipGetLastError();
}

}  // namespace pda
