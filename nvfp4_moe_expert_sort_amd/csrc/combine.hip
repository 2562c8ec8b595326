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
        // All K rows are loaded before the first add (K <= kMaxTopK, in
        // groups of 8 to bound the registers), so the loads are in flight
        // together instead of one round trip per slot.  A pair with no row
        // (ids outside the contract, reported by the error word) reads row 0
        // and contributes +0: acc starts at +0 and an FP32 sum of that form
        // is never -0, so adding +0 leaves every bit unchanged.
        for (int k0 = 0; k0 < K; k0 += 8) {
            u32x4 v[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int32_t r = k0 + i < K ? rows[k0 + i] : -1;
                v[i] = *reinterpret_cast<const u32x4*>(y2 + (int64_t)max(r, 0) * H + c * 8);
                if (r < 0) v[i] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < 8; i++) {
                if (k0 + i >= K) break;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    acc[2 * j] = acc[2 * j] + bf16_to_f32(v[i][j] & 0xFFFFu);
                    acc[2 * j + 1] = acc[2 * j + 1] + bf16_to_f32(v[i][j] >> 16);
                }
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
