// producer.hip -- the router-weighted SwiGLU producer as a kernel of its own,
// for the unfused forward (FC1 writes y1, then this kernel makes h).
//
// miniTE summary page, "how it differs": the router probability multiplies
// the SwiGLU output before FC2; "how to use it": that producer also emits the
// maxima FC2's quantizer takes; "assumptions and limits": the fused path is
// checked bit for bit against the unfused quantization/GEMM steps.  Article
// section 4.4: SiLU(gate) * up formed in FP32 and rounded once.
//
// Per sorted row r holding a pair (row2pair[r] >= 0):
//   h[r][n] = bf16(silu(f32(y1[r][n])) * f32(y1[r][I + n]) * p[r])
//   amax_part[r][j] = max |h[r][n]| over the 32 columns n of group j
// with the element arithmetic of the fused FC1 epilogue (swiglu_prob_bf16),
// so both give the same bits.  Padding rows are not written, as in the fused
// path.  One thread per (row, 32-column group): 64-byte loads of gate and up,
// 64-byte store of h.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

__global__ void __launch_bounds__(256) swiglu_producer_kernel(const uint16_t* __restrict__ y1, int64_t rows,
                                                              int32_t I, const int32_t* __restrict__ row2pair,
                                                              const float* __restrict__ row_prob,
                                                              const int32_t* __restrict__ expert_off, int32_t E,
                                                              uint16_t* __restrict__ h,
                                                              float* __restrict__ amax_part) {
    const int32_t n_part = I / 32;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t r = i / n_part;
    const int32_t j = (int32_t)(i % n_part);
    if (r >= rows || r >= expert_off[E]) return;
    if (row2pair[r] < 0) return;  // padding row
    const float p = row_prob[r];
    const u32x4* g4 = reinterpret_cast<const u32x4*>(y1 + r * 2 * I + 32 * j);
    const u32x4* u4 = reinterpret_cast<const u32x4*>(y1 + r * 2 * I + I + 32 * j);
    u32x4* h4 = reinterpret_cast<u32x4*>(h + r * I + 32 * j);
    uint32_t mx = 0u;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const u32x4 gv = g4[q], uv = u4[q];
        u32x4 hv;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const uint32_t lo = swiglu_prob_bf16(bf16_to_f32(gv[w] & 0xFFFFu), bf16_to_f32(uv[w] & 0xFFFFu), p);
            const uint32_t hi = swiglu_prob_bf16(bf16_to_f32(gv[w] >> 16), bf16_to_f32(uv[w] >> 16), p);
            hv[w] = lo | (hi << 16);
            // BF16 bit patterns of |h| order like their values
            mx = max(mx, max(lo & 0x7FFFu, hi & 0x7FFFu));
        }
        h4[q] = hv;
    }
    amax_part[r * n_part + j] = __uint_as_float(mx << 16);
}

hipError_t launch_swiglu_producer(const uint16_t* y1, int64_t rows_bound, int32_t I, const int32_t* row2pair,
                                  const float* row_prob, const int32_t* expert_off, int32_t E, uint16_t* h,
                                  float* amax_part, hipStream_t stream) {
    const int64_t n = rows_bound * (I / 32);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(swiglu_producer_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, y1,
                       rows_bound, I, row2pair, row_prob, expert_off, E, h, amax_part);
    return hipGetLastError();
}

}  // namespace nvfp4
