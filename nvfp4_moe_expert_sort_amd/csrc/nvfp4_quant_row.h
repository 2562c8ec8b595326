// nvfp4_quant_row.h -- one wavefront quantizes one row to NVFP4 (shared by the
// generic quantizer, the sort/scatter kernel and the FC2-input quantizer).
//
// miniTE summary page, "how it differs": g = max|row| / (6*448) per row, one
// E4M3 scale per 16 elements, E2M1 codes, round to nearest, no stochastic
// rounding.  Binary32 operations in this order, IEEE division throughout:
//   g = amax / 2688; d = 6 g; per block s = E4M3(amax_b / d); per element
//   q = |x| / (s g) and the code is the E2M1 magnitude of q with the input's
//   sign bit (magnitude 0 when s g == 0).
#pragma once

#include "nvfp4_device.h"

namespace nvfp4 {

// Quantize row `x` (cols BF16 values, cols % 16 == 0) with the calling wave and
// write the result to each of the n_dst rows in dst_rows.  amax < 0 asks for
// the row amax to be computed here; otherwise it is the caller's max|x|.
__device__ __forceinline__ void quant_row_wave(const uint16_t* __restrict__ x, int64_t cols, float amax, bool round_up, bool gemm,
                               const int64_t* dst_rows, int n_dst, uint8_t* __restrict__ codes,
                               uint8_t* __restrict__ scales, float* __restrict__ gout) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t groups = cols >> 3;
    if (amax < 0.0f) {
        float m = 0.0f;
        for (int64_t gi = lane; gi < groups; gi += kWave) {
            u32x4 v = *reinterpret_cast<const u32x4*>(x + gi * 8);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                m = fmaxf(m, fabsf(bf16_to_f32(v[j] & 0xFFFFu)));
                m = fmaxf(m, fabsf(bf16_to_f32(v[j] >> 16)));
            }
        }
        amax = wave_max(m);
    }
    const float g = amax / 2688.0f;  // IEEE binary32 division (2688 = 6 * 448)
    const float d = 6.0f * g;
    const int64_t iters = (groups + kWave - 1) / kWave;
    for (int64_t it = 0; it < iters; it++) {
        const int64_t gi = it * kWave + lane;
        const bool live = gi < groups;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (live) v = *reinterpret_cast<const u32x4*>(x + gi * 8);
        float lm = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            lm = fmaxf(lm, fabsf(bf16_to_f32(v[j] & 0xFFFFu)));
            lm = fmaxf(lm, fabsf(bf16_to_f32(v[j] >> 16)));
        }
        const float bmax = fmaxf(lm, __shfl_xor(lm, 1, kWave));  // partner lane holds the other 8 of the block
        uint32_t sbyte = 0u;
        if (amax > 0.0f) sbyte = e4m3_encode(bmax / d, round_up);
        const float s = e4m3_decode(sbyte);
        const float sg = s * g;
        uint32_t word = 0u;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t b = (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            uint32_t mag = 0u;
            if (sg != 0.0f) mag = e2m1_magnitude(fabsf(bf16_to_f32(b)) / sg);
            word |= (((b >> 15) << 3) | mag) << (4 * j);
        }
        if (live) {
            const int64_t k = gi * 8;
            for (int i = 0; i < n_dst; i++) {
                const int64_t r = dst_rows[i];
                if (gemm) {
                    *reinterpret_cast<uint32_t*>(codes + gemm_code_off(r, k, cols)) = word;
                    if ((lane & 1) == 0) scales[gemm_scale_off(r, k, cols)] = (uint8_t)sbyte;
                } else {
                    *reinterpret_cast<uint32_t*>(codes + r * (cols >> 1) + gi * 4) = word;
                    if ((lane & 1) == 0) scales[r * (cols >> 4) + (gi >> 1)] = (uint8_t)sbyte;
                }
            }
        }
    }
    if (lane == 0)
        for (int i = 0; i < n_dst; i++) gout[dst_rows[i]] = g;
}

}  // namespace nvfp4
