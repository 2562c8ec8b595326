// nvfp4_quant_row.h -- NVFP4 quantization of 32-element groups by one lane,
// and of whole rows by one wavefront.
//
// miniTE summary page, "how it differs": g = max|row| / (6*448) per row, one
// E4M3 scale per 16 elements, E2M1 codes, round to nearest, no stochastic
// rounding.  Binary32 operations in this order, IEEE division throughout:
//   g = amax / 2688; d = 6 g; per block s = E4M3(amax_b / d); per element
//   q = |x| / (s g) and the code is the E2M1 magnitude of q with the input's
//   sign bit (magnitude 0 when s g == 0).
//
// A lane owns 32 consecutive elements (two blocks): it reads 64 bytes and
// writes 16 bytes of codes (element 2i in the low nibble of byte i) and two
// scale bytes.  In the GEMM layout those 16 bytes are exactly one lane slot of
// a 1 KiB tile-chunk, so tile-wise writers emit whole contiguous chunks.
#pragma once

#include "nvfp4_device.h"

namespace nvfp4 {

// Row scale g and block divisor d from the row amax.
struct RowScale {
    float g, d;
    bool zero;
};

__device__ __forceinline__ RowScale row_scale(float amax) {
    RowScale r;
    r.g = amax / 2688.0f;  // IEEE binary32 division (2688 = 6 * 448)
    r.d = 6.0f * r.g;
    r.zero = !(amax > 0.0f);
    return r;
}

// Max |x| over the 8 BF16 values packed in one u32x4.
__device__ __forceinline__ float absmax8(u32x4 v) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        m = fmaxf(m, fabsf(bf16_to_f32(v[j] & 0xFFFFu)));
        m = fmaxf(m, fabsf(bf16_to_f32(v[j] >> 16)));
    }
    return m;
}

// Quantize one 16-element block (two u32x4 of BF16 pairs) -> two code words and the scale byte.
__device__ __forceinline__ void quant_block16(u32x4 lo, u32x4 hi, const RowScale& rs, bool round_up, uint32_t& w0,
                                              uint32_t& w1, uint32_t& sbyte) {
    const float bmax = fmaxf(absmax8(lo), absmax8(hi));
    sbyte = rs.zero ? 0u : e4m3_encode(bmax / rs.d, round_up);
    const float sg = e4m3_decode(sbyte) * rs.g;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int half = 0; half < 2; half++) {
        const u32x4 v = half ? hi : lo;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t b = (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            uint32_t mag = 0u;
            if (sg != 0.0f) mag = e2m1_magnitude(fabsf(bf16_to_f32(b)) / sg);
            w[half] |= (((b >> 15) << 3) | mag) << (4 * j);
        }
    }
    w0 = w[0];
    w1 = w[1];
}

// Quantize 32 consecutive elements (v[0..3]); with only_first, just the first
// block (v[0], v[1]) is real and the second's outputs are zero.
__device__ __forceinline__ void quant32(const u32x4 (&v)[4], const RowScale& rs, bool round_up, bool only_first,
                                        u32x4& codes, uint32_t& scales2) {
    uint32_t s0 = 0u, s1 = 0u, w0 = 0u, w1 = 0u, w2 = 0u, w3 = 0u;
    quant_block16(v[0], v[1], rs, round_up, w0, w1, s0);
    if (!only_first) quant_block16(v[2], v[3], rs, round_up, w2, w3, s1);
    codes = u32x4{w0, w1, w2, w3};
    scales2 = s0 | (s1 << 8);
}

__device__ __forceinline__ void load32(const uint16_t* p, bool only_first, u32x4 (&v)[4]) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    v[0] = q[0];
    v[1] = q[1];
    if (only_first) {
        v[2] = u32x4{0u, 0u, 0u, 0u};
        v[3] = u32x4{0u, 0u, 0u, 0u};
    } else {
        v[2] = q[2];
        v[3] = q[3];
    }
}

// One wavefront quantizes the row x[0..cols) (cols % 16 == 0; x 16-byte
// aligned) into row `r` of the output planes.  Logical layout: codes
// [*][cols/2], scales [*][cols/16]; GEMM layout (cols % 128 == 0): the tiled
// map of include/nvfp4moe.h.  amax < 0: computed here (first pass).
__device__ __forceinline__ void quant_row_wave(const uint16_t* __restrict__ x, int64_t cols, float amax, bool round_up,
                                               bool gemm, int64_t r, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales, float* __restrict__ gout) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t groups = (cols + 31) >> 5;  // 32-element groups; the last may hold one block
    if (amax < 0.0f) {
        float m = 0.0f;
        for (int64_t gi = lane; gi < groups; gi += kWave) {
            const bool one = (gi + 1) * 32 > cols;
            u32x4 v[4];
            load32(x + gi * 32, one, v);
            m = fmaxf(m, fmaxf(fmaxf(absmax8(v[0]), absmax8(v[1])), fmaxf(absmax8(v[2]), absmax8(v[3]))));
        }
        amax = wave_max(m);
    }
    const RowScale rs = row_scale(amax);
    for (int64_t gi = lane; gi < groups; gi += kWave) {
        const bool one = (gi + 1) * 32 > cols;
        u32x4 v[4];
        load32(x + gi * 32, one, v);
        u32x4 c;
        uint32_t s2;
        quant32(v, rs, round_up, one, c, s2);
        const int64_t k = gi * 32;
        if (gemm) {
            *reinterpret_cast<u32x4*>(codes + gemm_code_off(r, k, cols)) = c;
            *reinterpret_cast<uint16_t*>(scales + gemm_scale_off(r, k, cols)) = (uint16_t)s2;
        } else {
            // Rows start 8-byte aligned (codes) and byte aligned (scales) when
            // cols % 32 == 16, 16- and 2-byte aligned when cols % 32 == 0.
            uint8_t* cr = codes + r * (cols >> 1) + gi * 16;
            uint8_t* sr = scales + r * (cols >> 4) + gi * 2;
            if ((cols & 31) == 0) {
                *reinterpret_cast<u32x4*>(cr) = c;
                *reinterpret_cast<uint16_t*>(sr) = (uint16_t)s2;
            } else {
                *reinterpret_cast<u32x2*>(cr) = u32x2{c[0], c[1]};
                sr[0] = (uint8_t)s2;
                if (!one) {
                    *reinterpret_cast<u32x2*>(cr + 8) = u32x2{c[2], c[3]};
                    sr[1] = (uint8_t)(s2 >> 8);
                }
            }
        }
    }
    if (lane == 0) gout[r] = rs.g;
}

}  // namespace nvfp4
