// gfx950 (CDNA4) kernels for the running state of tiled decode (spark_storage
// "tiled_attention.rs" page: header comment, TiledAttention::begin_step and
// finalize): the reset of (m, l, o) before the first tile and the final
// o / l to bf16.  The attention itself (decode and each tile) is in
// pda_attend.hip.
#include "pda_internal.h"
#include "pda_device.h"

namespace pda {
namespace {

// m = -inf (bits 0xFF800000), l = 0, o = 0 for `rows` rows (a fill kernel,
// not driver memsets: safe inside captured graphs).
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

// out = bf16(o / l), rounded to nearest even; 0 where l == 0.
__global__ void __launch_bounds__(256) finalize_kernel(const float *l, const float *o, uint16_t *out,
                                                       int64_t rows, int D) {
    const int64_t n = rows * D;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float li = l[i / D];
        out[i] = li > 0.f ? f32_to_bf16(o[i] / li) : 0;
    }
}

int grid_1d(int64_t n, int per) {
    int64_t b = (n + per - 1) / per;
    if (b > 65536) b = 65536;
    return b < 1 ? 1 : (int)b;
}

}  // namespace

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
