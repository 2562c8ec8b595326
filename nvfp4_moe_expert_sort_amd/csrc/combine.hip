// combine.hip -- deterministic combine of each token's K expert outputs.
//
// Article section 4.5: the owner of a token accumulates its expert outputs in
// FP32 in top-k slot order, so the result does not depend on which expert
// finished first.  miniTE summary page, "how it differs": the combine order is
// preserved through padding, quantization and cast.  Here
//   out[t] = bf16( (((0.0f + y2[row(t,0)]) + y2[row(t,1)]) + ...) )
// with no weighting (the router probability was applied before FC2).
// HBM-bound streaming kernel: one block per token, 16-byte loads and stores.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ y2,
                                                      const int32_t* __restrict__ pair2row, int32_t H, int32_t K,
                                                      uint16_t* __restrict__ out) {
    const int64_t t = blockIdx.x;
    __shared__ int32_t rows[kMaxTopK];
    if (threadIdx.x < K) rows[threadIdx.x] = pair2row[t * K + threadIdx.x];
    __syncthreads();
    for (int64_t c = threadIdx.x; c < H / 8; c += blockDim.x) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; j++) acc[j] = 0.0f;
        for (int k = 0; k < K; k++) {
            const int32_t r = rows[k];
            if (r < 0) continue;  // only for ids outside the contract (reported by the error word)
            const u32x4 v = *reinterpret_cast<const u32x4*>(y2 + (int64_t)r * H + c * 8);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                acc[2 * j] = acc[2 * j] + bf16_to_f32(v[j] & 0xFFFFu);
                acc[2 * j + 1] = acc[2 * j + 1] + bf16_to_f32(v[j] >> 16);
            }
        }
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; j++) o[j] = f32_to_bf16_rne(acc[2 * j]) | (f32_to_bf16_rne(acc[2 * j + 1]) << 16);
        *reinterpret_cast<u32x4*>(out + t * H + c * 8) = o;
    }
}

hipError_t launch_combine(const uint16_t* y2, const int32_t* pair2row, int32_t T, int32_t H, int32_t K,
                          uint16_t* out, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, stream, y2, pair2row, H, K, out);
    return hipGetLastError();
}

}  // namespace nvfp4
