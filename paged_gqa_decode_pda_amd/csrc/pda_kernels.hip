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
//   partial_kernel  one workgroup (4 wave64) per (split, kv head, head chunk,
//                   sequence): gathers the split's K/V rows from their pages,
//                   computes the scores of the head chunk's q heads, keeps a
//                   base-2 online softmax per wave and merges the 4 waves;
//                   writes one (m, l, o) partial per q head.
//   combine_kernel  one wave per (sequence, q head): log-sum-exp merge of the
//                   partials in split order, into bf16 output (decode) or
//                   into the running state (tile).
//   reset_kernel / finalize_kernel  state fill and o / l -> bf16.
//
// Lane layouts inside partial_kernel (D_PAD = padded head dim, 64/128/256):
//   K: 4 lanes per token, 16 tokens per wave; lane (t = lane/4, j = lane%4)
//      holds the 16-byte chunks 4c + j (c < D_PAD/32) of token t's K row, so
//      each load instruction reads 64 contiguous bytes of 16 rows.  Scores use
//      v_dot2c_f32_bf16 on bf16 pairs and a 2-step quad DPP reduction.
//   V: 16 lanes per token row, 4 rows per wave; lane (r = lane/16, c =
//      lane%16) holds elements [c*D_PAD/16, (c+1)*D_PAD/16) of token 4i + r.
//      Softmax weights move from the K layout to the V layout through LDS.
#include "pda_internal.h"

namespace pda {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWaves = 4;
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

// One workgroup = 4 waves = one (split, kv head, head chunk, sequence).  The
// split's 16-token groups are dealt to the waves in contiguous runs; each wave
// keeps NBUF groups of K/V in flight in registers while it computes.  The page
// ids a wave needs are read once into one VGPR (lane i holds page cb + i of
// the sequence's list) and picked out with readlane (pages of 16k tokens) or a
// lane shuffle (other block sizes), so no table load sits between a group's
// address and its data.
template <int DP, int GC, bool P16, int NBUF>
__global__ void __launch_bounds__(kThreads) partial_kernel(const PartialArgs a) {
    constexpr int NCK = DP / 32;
    constexpr int VW = DP / 32;      // V dwords per lane per row step
    constexpr int VPL = DP / 16;     // V elements per lane
    constexpr int VC = DP == 64 ? 1 : VW / 4;   // V loads per row step (8 B for DP 64, else 16 B each)

    __shared__ float p_lds[kWaves][16][GC];
    __shared__ float m_lds[kWaves][GC];
    __shared__ float l_lds[kWaves][GC];
    __shared__ float o_lds[kWaves][GC][DP];

    const int lane = threadIdx.x & 63;
    // wave index as a scalar: everything derived from it is wave-uniform
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // kv head (and head chunk) is the fastest grid dimension: the workgroups
    // that read the interleaved kv-head rows of the same pages are dispatched
    // together and stream those pages at the same time.
    const int g = blockIdx.x / a.nhc;
    const int hc = blockIdx.x - g * a.nhc;
    const int split = blockIdx.y;
    const int s = blockIdx.z;
    const int h0 = g * a.G + hc * GC;
    const int nh = min(GC, a.G - hc * GC);

    const int cnt = clampi(a.counts[s], 0, a.cap);
    if (cnt == 0) return;
    const int lv = clampi(a.lastv ? a.lastv[s] : a.lv_default, 0, a.bs);
    const int ntok = (cnt - 1) * a.bs + lv;
    const int span = a.bps * a.bs;
    const int t0 = split * span;
    if (t0 >= ntok) return;  // uniform over the workgroup
    const int t1 = min(t0 + span, ntok);
    const int ngroups = (t1 - t0 + 15) >> 4;
    const int gpw = (ngroups + kWaves - 1) / kWaves;
    const int g_lo = w * gpw;
    const int n_my = max(0, min(ngroups - g_lo, gpw));
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

    float m2[GC], lsum[GC], acc_o[GC][VPL];
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
        const int gs = t0 + 16 * (g_lo + n);
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
        const int gs = t0 + 16 * (g_lo + n);
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
            for (int h = 0; h < GC; ++h) p_lds[w][quad][h] = p[h];
        }
        // the last group of a split may hold tokens past t1: zero their V so
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
            for (int h = 0; h < GC; ++h) pv[h] = p_lds[w][4 * i + row][h];
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

    if (n_my > 0) {
        // groups covered by one 64-page window
        const int per_window = P16 ? 4 * a.bs : max(1, (62 * a.bs + 1) / 16);
        for (int c0 = 0; c0 < n_my; c0 += per_window) {
            const int nc = min(per_window, n_my - c0);
            load_window(page_of((uint32_t)(t0 + 16 * (g_lo + c0)), a.bs_magic));
            // Loads are issued unconditionally (indices past the chunk re-read
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
    }

    // Wave totals: o over the 4 rows, l over the 16 token quads.
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
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            m_lds[w][h] = m2[h];
            l_lds[w][h] = lsum[h];
        }
    }
    if (row == 0) {
#pragma unroll
        for (int h = 0; h < GC; ++h)
#pragma unroll
            for (int e = 0; e < VPL; ++e) o_lds[w][h][col * VPL + e] = acc_o[h][e];
    }
    __syncthreads();

    // Merge the 4 waves in fixed order and write the split's partial.
    const int64_t pbase = ((int64_t)s * a.Hq + h0) * a.nsplit + split;
    for (int idx = threadIdx.x; idx < GC * DP; idx += kThreads) {
        const int h = idx / DP, d = idx - h * DP;
        if (h >= nh || d >= a.D) continue;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, m_lds[ww][h]);
        float O = 0.f, L = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float mw = m_lds[ww][h];
            if (mw == -INFINITY) continue;
            const float f = exp2_fast(mw - M);
            O = fmaf(o_lds[ww][h][d], f, O);
            L = fmaf(l_lds[ww][h], f, L);
        }
        const int64_t pi = pbase + (int64_t)h * a.nsplit;
        a.part_o[pi * a.D + d] = O;
        if (d == 0) {
            a.part_ml[2 * pi] = M;
            a.part_ml[2 * pi + 1] = L;
        }
    }
}

// One wave per (sequence, q head); lanes own DP/64 consecutive elements.
// Split weights are formed lane-parallel (lane i <-> split cbase + i); the
// weighted sum of the o partials runs in split order, state first when
// merging into the running state.
template <int DP>
__global__ void __launch_bounds__(kThreads) combine_kernel(const CombineArgs a) {
    constexpr int EPL = DP / 64;
    const int lane = threadIdx.x & 63;
    const int64_t sh = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (sh >= (int64_t)a.S * a.Hq) return;
    const int s = (int)(sh / a.Hq);
    const int ntok = seq_tokens(a.counts, a.lastv, a.lv_default, s, a.cap, a.bs);
    const int span = a.bps * a.bs;
    const int nsp = ntok > 0 ? (ntok + span - 1) / span : 0;
    const int d0 = lane * EPL;
    const bool dok = d0 < a.D;   // D is a multiple of 8, so a lane's elements are all in or all out

    if (nsp == 0) {
        if (a.out && dok) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) a.out[sh * a.D + d0 + e] = 0;
        }
        return;  // empty tile: the running state stays bit-identical
    }

    const float *ml = a.part_ml + sh * a.nsplit * 2;
    const float *po = a.part_o + sh * a.nsplit * a.D;

    float ms = -INFINITY, ls = 0.f;
    if (a.m) {
        ms = a.m[sh] * kLog2e;
        ls = a.l[sh];
    }
    float M = ls > 0.f ? ms : -INFINITY;
    for (int i = lane; i < nsp; i += 64) {
        const float li = ml[2 * i + 1];
        if (li > 0.f) M = fmaxf(M, ml[2 * i]);
    }
    M = fmaxf(M, shfl_xor(M, 1));
    M = fmaxf(M, shfl_xor(M, 2));
    M = fmaxf(M, shfl_xor(M, 4));
    M = fmaxf(M, shfl_xor(M, 8));
    M = fmaxf(M, shfl_xor(M, 16));
    M = fmaxf(M, shfl_xor(M, 32));

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
    for (int cbase = 0; cbase < nsp; cbase += 64) {
        const int i = cbase + lane;
        float wi = 0.f, li = 0.f;
        if (i < nsp) {
            li = ml[2 * i + 1];
            wi = li > 0.f ? exp2_fast(ml[2 * i] - M) : 0.f;
        }
        float x = wi * li;
        x += shfl_xor(x, 1);
        x += shfl_xor(x, 2);
        x += shfl_xor(x, 4);
        x += shfl_xor(x, 8);
        x += shfl_xor(x, 16);
        x += shfl_xor(x, 32);
        L += x;
        const int n = min(64, nsp - cbase);
        if (dok) {
#pragma unroll 8
            for (int j = 0; j < n; ++j) {
                const float f = readlanef(wi, j);
                const float *src = po + (int64_t)(cbase + j) * a.D + d0;
#pragma unroll
                for (int e = 0; e < EPL; ++e) O[e] = fmaf(src[e], f, O[e]);
            }
        }
    }
    if (a.out) {
        if (dok) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) a.out[sh * a.D + d0 + e] = L > 0.f ? f32_to_bf16(O[e] / L) : 0;
        }
    } else {
        if (dok) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) a.o[sh * a.D + d0 + e] = O[e];
        }
        if (lane == 0) {
            a.l[sh] = L;
            a.m[sh] = L > 0.f ? M * kLn2 : -INFINITY;
        }
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

constexpr int kNbuf = 3;   // 16-token groups of K/V in flight per wave

template <int DP, int GC, bool P16>
hipError_t launch_partial_t(const PartialArgs &a, int S, hipStream_t st) {
    dim3 grid(a.Hkv * a.nhc, a.nsplit, S);
    hipLaunchKernelGGL((partial_kernel<DP, GC, P16, kNbuf>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int DP, int GC>
hipError_t launch_partial_p(const PartialArgs &a, bool p16, int S, hipStream_t st) {
    return p16 ? launch_partial_t<DP, GC, true>(a, S, st) : launch_partial_t<DP, GC, false>(a, S, st);
}

template <int DP>
hipError_t launch_partial_g(const Plan &p, const PartialArgs &a, int S, hipStream_t st) {
    switch (p.gc) {
        case 1: return launch_partial_p<DP, 1>(a, p.p16, S, st);
        case 2: return launch_partial_p<DP, 2>(a, p.p16, S, st);
        case 4: return launch_partial_p<DP, 4>(a, p.p16, S, st);
        default:
            if constexpr (DP <= 128) return launch_partial_p<DP, 8>(a, p.p16, S, st);
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

hipError_t launch_partial(const Plan &p, const PartialArgs &a, int S, hipStream_t st) {
    switch (p.dp) {
        case 64: return launch_partial_g<64>(p, a, S, st);
        case 128: return launch_partial_g<128>(p, a, S, st);
        default: return launch_partial_g<256>(p, a, S, st);
    }
}

hipError_t launch_combine(const CombineArgs &a, int dp, hipStream_t st) {
    const int64_t waves = (int64_t)a.S * a.Hq;
    dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
    switch (dp) {
        case 64: hipLaunchKernelGGL((combine_kernel<64>), grid, dim3(kThreads), 0, st, a); break;
        case 128: hipLaunchKernelGGL((combine_kernel<128>), grid, dim3(kThreads), 0, st, a); break;
        default: hipLaunchKernelGGL((combine_kernel<256>), grid, dim3(kThreads), 0, st, a); break;
    }
    return hipGetLastError();
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
