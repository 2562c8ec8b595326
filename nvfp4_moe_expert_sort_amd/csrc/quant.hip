// quant.hip -- NVFP4 row quantizer on gfx950.
//
// miniTE summary page, "how it differs": per-row FP32 outer scale
// g = max|row| / (6*448), one E4M3 scale per 16 elements, E2M1 codes, round
// to nearest, no Hadamard transform, no stochastic rounding.  One wavefront
// owns one row: the row amax is a wave reduction, each lane then quantizes
// 8-element groups (a 16-element block spans two neighbouring lanes, whose
// maxima meet in one shuffle).  Loads are 16 B per lane, so a wave reads 1 KiB
// contiguous per step; HBM-bound.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"
#include "nvfp4_quant_row.h"

namespace nvfp4 {

// Generic quantizer: one wave per row, four rows per 256-thread block.
__global__ void __launch_bounds__(256) quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                         int64_t ld, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, float* __restrict__ g,
                                                         int gemm, int round_up) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    int64_t dst = row;
    quant_row_wave(x + row * ld, cols, -1.0f, round_up != 0, gemm != 0, &dst, 1, codes, scales, g);
}

// FC2 input: quantize h of every (token, slot) pair.  The row amax is the max
// of the per-column-tile maxima the FC1 producer emitted for this row (the
// maxima of the tensor FC2 actually consumes, miniTE page "how to use it").
__global__ void __launch_bounds__(256) quant_h_kernel(const uint16_t* __restrict__ h, int64_t P, int64_t I,
                                                      const int32_t* __restrict__ pair2row,
                                                      const float* __restrict__ amax2_part, int n_part,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                      float* __restrict__ g, int round_up) {
    const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= P) return;
    const int32_t row = pair2row[p];
    if (row < 0) return;
    float amax = 0.0f;
    for (int i = 0; i < n_part; i++) amax = fmaxf(amax, amax2_part[(int64_t)row * n_part + i]);
    int64_t dst = row;
    quant_row_wave(h + (int64_t)row * I, I, amax, round_up != 0, true, &dst, 1, codes, scales, g);
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                             uint8_t* scales, float* g, bool gemm, bool round_up, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, cols, ld, codes,
                       scales, g, gemm ? 1 : 0, round_up ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_quant_h(const uint16_t* h, int64_t P, int64_t I, const int32_t* pair2row, const float* amax2_part,
                          int n_part, uint8_t* codes, uint8_t* scales, float* g, bool round_up, hipStream_t stream) {
    if (P <= 0) return hipSuccess;
    const int64_t blocks = (P + 3) / 4;
    hipLaunchKernelGGL(quant_h_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, h, P, I, pair2row, amax2_part,
                       n_part, codes, scales, g, round_up ? 1 : 0);
    return hipGetLastError();
}

}  // namespace nvfp4
