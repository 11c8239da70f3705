// gfx950 kernels for rotary embedding (AstrAI "CUDA Kernels", sections
// "Rotary Embedding Kernel" and "Rotary Backend"): element pair j of a row,
// (x[2j], x[2j+1]), read as a complex number, times cos + i sin of the
// token's position, with cos/sin looked up in fp32 tables
// [max_positions, head_dim / 2]:
//
//   out[2j]     = x[2j] cos_j - x[2j+1] sin_j
//   out[2j + 1] = x[2j] sin_j + x[2j+1] cos_j
//
// computed in fp32 and rounded once to bf16 (round to nearest even).
//
//   rope_kernel            rows of a [tokens, heads, head_dim] tensor, in place
//                          or into another buffer (q before attention)
//   rope_append_kv_kernel  new K rows rotated and new V rows copied into the
//                          paged cache at each token's page and slot (K as it
//                          is written to the cache)
//
// Both are elementwise and HBM-bound: a thread takes 16 bytes of a row (four
// pairs), the matching 16 bytes of cos and of sin, and stores 16 bytes; the
// grid strides over the rows' 16-byte chunks.
#include "pda_device.h"
#include "pda_rope.h"

namespace pda {
namespace {

typedef float f32x4r __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2r __attribute__((ext_vector_type(2)));

constexpr int kRopeThreads = 256;

__device__ __forceinline__ uint32_t rot_pair(uint32_t ab, float c, float s) {
    const float a = bf_lo(ab), b = bf_hi(ab);
    const float re = fmaf(a, c, -(b * s));
    const float im = fmaf(a, s, b * c);
    const bf16x2r v = {(__bf16)re, (__bf16)im};
    return __builtin_bit_cast(uint32_t, v);
}

// Four pairs of one 16-byte chunk, starting at pair j0 of the token's table row.
__device__ __forceinline__ u32x4 rotate_chunk(u32x4 x, const float *cos_row, const float *sin_row, int j0) {
    const f32x4r c = *reinterpret_cast<const f32x4r *>(cos_row + j0);
    const f32x4r s = *reinterpret_cast<const f32x4r *>(sin_row + j0);
    return u32x4{rot_pair(x[0], c[0], s[0]), rot_pair(x[1], c[1], s[1]), rot_pair(x[2], c[2], s[2]),
                 rot_pair(x[3], c[3], s[3])};
}

__global__ void __launch_bounds__(kRopeThreads) rope_kernel(const RopeArgs a) {
    const int cpr = a.D / 8;                       // 16-byte chunks per row
    const int64_t per_token = (int64_t)a.H * cpr;
    const int64_t n = a.T * per_token;
    const int half = a.D / 2;
    for (int64_t e = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * kRopeThreads) {
        const int64_t t = e / per_token;
        const int k = (int)(e % cpr);
        const int p = clampi(a.positions[t], 0, a.max_pos - 1);
        const u32x4 x = ld16(a.x + e * 8);
        *reinterpret_cast<u32x4 *>(a.out + e * 8) =
            rotate_chunk(x, a.cos_t + (int64_t)p * half, a.sin_t + (int64_t)p * half, 4 * k);
    }
}

__global__ void __launch_bounds__(kRopeThreads) rope_append_kv_kernel(const RopeArgs a) {
    const int cpr = a.D / 8;
    const int64_t per_token = (int64_t)a.H * cpr;
    const int64_t n = a.T * per_token;
    const int half = a.D / 2;
    for (int64_t e = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * kRopeThreads) {
        const int64_t t = e / per_token;
        const int rem = (int)(e - t * per_token);
        const int h = rem / cpr, k = rem - h * cpr;
        const int s = a.token_seq[t];
        const int pos = a.positions[t];
        if (s < 0 || s >= a.S || pos < 0) continue;   // outside the tables: not written
        const int pi = pos / a.bs;
        if (pi >= a.cap) continue;
        const int bid = a.blocks[(int64_t)s * a.cap + pi];
        const int64_t dst = (int64_t)bid * a.blk + (int64_t)(pos - pi * a.bs) * a.tok + (int64_t)h * a.kvh + 8 * k;
        const int p = min(pos, a.max_pos - 1);
        const u32x4 kx = ld16(a.x + e * 8);
        const u32x4 vx = ld16(a.v_new + e * 8);
        *reinterpret_cast<u32x4 *>(a.k_pool + dst) =
            rotate_chunk(kx, a.cos_t + (int64_t)p * half, a.sin_t + (int64_t)p * half, 4 * k);
        *reinterpret_cast<u32x4 *>(a.v_pool + dst) = vx;
    }
}

int rope_grid(int64_t n, int cus) {
    const int64_t want = (n + kRopeThreads - 1) / kRopeThreads;
    const int64_t cap = (int64_t)cus * 8;   // eight 256-thread workgroups per CU, then stride
    return (int)(want < 1 ? 1 : (want < cap ? want : cap));
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, int cus, hipStream_t st) {
    const int64_t n = a.T * a.H * (a.D / 8);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_kernel, dim3(rope_grid(n, cus)), dim3(kRopeThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_rope_append_kv(const RopeArgs &a, int cus, hipStream_t st) {
    const int64_t n = a.T * a.H * (a.D / 8);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_append_kv_kernel, dim3(rope_grid(n, cus)), dim3(kRopeThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace pda
