// Device helpers shared by the gfx950 kernel files.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pda {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// The two bf16 halves of a dword, widened exactly to fp32.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// DPP lane permutations (all source lanes valid for the controls used).
constexpr int kRowRor4 = 0x124;   // row_ror:4 (within 16-lane rows)
constexpr int kRowRor8 = 0x128;   // row_ror:8

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kWaitVmcnt0 = 0x0F70;   // s_waitcnt vmcnt(0): this wave's vector memory operations completed

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

__device__ __forceinline__ int page_of(uint32_t t, uint64_t magic) {
    return (int)(((uint64_t)t * magic) >> 32);
}

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

// Tokens of sequence s: the first `cnt` listed pages, all full except the
// last, which holds `lv` valid slots.
__device__ __forceinline__ int seq_tokens(const int32_t *counts, const int32_t *lastv, int lv_default,
                                          int s, int cap, int bs) {
    int cnt = clampi(counts[s], 0, cap);
    if (cnt == 0) return 0;
    int lv = clampi(lastv ? lastv[s] : lv_default, 0, bs);
    return (cnt - 1) * bs + lv;
}

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

// Splits of a sequence: ceil(ntok / span), 0 for an empty sequence.
__device__ __forceinline__ int splits_of(int ntok, int span) { return ntok > 0 ? (ntok + span - 1) / span : 0; }

// Work items of a sequence with nsp splits (prefix mode): nb "big" items of
// `big` consecutive splits cover about eighths / 8 of the splits, then one
// item per `sgl` remaining splits when nb > 0, else per split (the last item
// takes what is left).  Items are numbered in token order; item k of the
// sequence owns partial slot k.
__device__ __forceinline__ int big_items_of(int nsp, int big, int eighths) { return (eighths * nsp) / (8 * big); }
__device__ __forceinline__ int slots_of(int nsp, bool prefix_mode, int big, int eighths, int sgl) {
    if (!prefix_mode) return nsp;
    const int nb = big_items_of(nsp, big, eighths);
    const int sg = nb > 0 ? sgl : 1;
    return nb + (nsp - nb * big + sg - 1) / sg;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values to a bf16 pair, round to nearest even (one
// v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// x of lanes l and l^16 (gfx950 v_permlane16_swap of x with itself: the two
// results hold, per lane, the values of lanes l & ~16 and l | 16), and the
// same for l^32 (v_permlane32_swap).  VALU lane swaps, no LDS round trip.
__device__ __forceinline__ void pair16(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Maximum of x over the four lanes l, l^16, l^32, l^48 (one row of the
// transposed scores).
__device__ __forceinline__ float max4(float x) {
    float a, b;
    pair16(x, a, b);
    pair32(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}
// Sum over the same four lanes, in an order that is the same in every lane
// (lanes with bit 4 clear first, then bit 5 clear first).
__device__ __forceinline__ float sum4(float x) {
    float a, b;
    pair16(x, a, b);
    pair32(a + b, a, b);
    return a + b;
}

}  // namespace
}  // namespace pda
