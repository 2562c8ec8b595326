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

// Max of |x| over the 8 BF16 values packed in one u32x4, as a BF16 bit
// pattern: for finite values the bits of |x| order like the values, so the
// integer max is exact.
// The two halves of each word are maxed as a pair of 16-bit integers.
typedef uint16_t u16x2q __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t absmax8_bits(u32x4 v) {
    u16x2q m = __builtin_bit_cast(u16x2q, v[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int j = 1; j < 4; j++) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2q, v[j] & 0x7FFF7FFFu));
    return max((uint32_t)m[0], (uint32_t)m[1]);
}

__device__ __forceinline__ float absmax8(u32x4 v) { return bf16_to_f32(absmax8_bits(v)); }

// fl32(a / b) from y = fl32(1 / b) with two FMAs (Markstein's correction
// step).  Equal to the IEEE quotient for every binary32 b and every BF16 a
// whose quotient lies in [2^-5, 2^5): checked exhaustively (all 2^23 divisor
// significands x all BF16 dividend significands over that quotient range).
// Quotients below 2^-5 or above 2^5 are far from every E2M1 decision
// threshold (0.25 .. 5), so the code they give is the same either way.
__device__ __forceinline__ float quot(float a, float b, float y) {
    const float q0 = a * y;
    const float r = __builtin_fmaf(-q0, b, a);
    return __builtin_fmaf(r, y, q0);
}

// Two E2M1 codes into byte SEL of `old`: the hardware conversion
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to the nearest E2M1 value,
// ties to the even code, saturating at 6, and keeps the sign bit.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t old, float q0, float q1) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, q0, q1, 1.0f, SEL);
}

// Signed quotient x / sg, from x's BF16 pattern in the high half of a word
// (low half zero), carrying x's sign bit.  Every step of quot() is odd in x
// under round-to-nearest, so for x != 0 this is sign(x) * (|x| / sg) bit for
// bit; the correction step turns a -0 quotient into +0, so the sign bit is
// put back from x (one bit-field insert).
template <bool FAST>
__device__ __forceinline__ float signed_q(uint32_t xw, float sg, float y) {
    const float x = __uint_as_float(xw);
    const float q = FAST ? quot(x, sg, y) : x / sg;
    return __uint_as_float((__float_as_uint(q) & 0x7FFFFFFFu) | (xw & 0x80000000u));
}

// Eight E2M1 codes (one word) of the eight BF16 values in v.
template <bool FAST>
__device__ __forceinline__ uint32_t codes8(u32x4 v, float sg, float y) {
    uint32_t acc = 0u;
    acc = fp4_pair<0>(acc, signed_q<FAST>(v[0] << 16, sg, y), signed_q<FAST>(v[0] & 0xFFFF0000u, sg, y));
    acc = fp4_pair<1>(acc, signed_q<FAST>(v[1] << 16, sg, y), signed_q<FAST>(v[1] & 0xFFFF0000u, sg, y));
    acc = fp4_pair<2>(acc, signed_q<FAST>(v[2] << 16, sg, y), signed_q<FAST>(v[2] & 0xFFFF0000u, sg, y));
    acc = fp4_pair<3>(acc, signed_q<FAST>(v[3] << 16, sg, y), signed_q<FAST>(v[3] & 0xFFFF0000u, sg, y));
    return acc;
}

// Quantize one 16-element block (two u32x4 of BF16 pairs) -> two code words and the scale byte.
__device__ __forceinline__ void quant_block16(u32x4 lo, u32x4 hi, const RowScale& rs, bool round_up, uint32_t& w0,
                                              uint32_t& w1, uint32_t& sbyte) {
    const float bmax = bf16_to_f32(max(absmax8_bits(lo), absmax8_bits(hi)));
    sbyte = rs.zero ? 0u : e4m3_encode(bmax / rs.d, round_up);
    const float sg = e4m3_decode(sbyte) * rs.g;
    if (sg == 0.0f) {  // zero block or scale underflow: codes keep only the sign
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int half = 0; half < 2; half++) {
            const u32x4 v = half ? hi : lo;
#pragma unroll
            for (int j = 0; j < 8; j++) w[half] |= (((v[j >> 1] >> (16 * (j & 1))) >> 15) & 1u) << (4 * j + 3);
        }
        w0 = w[0];
        w1 = w[1];
        return;
    }
    const float y = 1.0f / sg;  // IEEE division, once per block
    // The reciprocal overflows only for sg < 2^-128 (blocks of subnormal
    // values).  The choice between the reciprocal path and IEEE division is
    // taken once for the whole wavefront, so no element carries a branch;
    // both give the IEEE quotient wherever the reciprocal is finite.
    if (__all(y < __builtin_huge_valf())) {
        w0 = codes8<true>(lo, sg, y);
        w1 = codes8<true>(hi, sg, y);
    } else {
        w0 = codes8<false>(lo, sg, y);
        w1 = codes8<false>(hi, sg, y);
    }
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
        uint32_t m = 0u;
        for (int64_t gi = lane; gi < groups; gi += kWave) {
            const bool one = (gi + 1) * 32 > cols;
            u32x4 v[4];
            load32(x + gi * 32, one, v);
            m = max(m, max(max(absmax8_bits(v[0]), absmax8_bits(v[1])), max(absmax8_bits(v[2]), absmax8_bits(v[3]))));
        }
        amax = bf16_to_f32(wave_max_u32(m));
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

// max |x| over a row of cols (cols % 16 == 0) BF16 values, one wavefront
// (quant_row_wave's first pass).
__device__ __forceinline__ float row_amax_wave(const uint16_t* __restrict__ x, int64_t cols) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t groups = (cols + 31) >> 5;
    uint32_t m = 0u;
    for (int64_t gi = lane; gi < groups; gi += kWave) {
        const bool one = (gi + 1) * 32 > cols;
        u32x4 v[4];
        load32(x + gi * 32, one, v);
        m = max(m, max(max(absmax8_bits(v[0]), absmax8_bits(v[1])), max(absmax8_bits(v[2]), absmax8_bits(v[3]))));
    }
    return bf16_to_f32(wave_max_u32(m));
}

template <int G>
struct RowRegs {
    u32x4 v[G][4];
};

// The loads of quant_row_regs alone: lane l's groups l, l + 64, ... of the
// row into registers (issued, not waited for).  No branch: a lane past the
// row's last group re-reads that group (row_quant ignores it).
template <int G>
__device__ __forceinline__ void row_load(const uint16_t* __restrict__ x, int64_t cols, RowRegs<G>& rr) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t groups = cols >> 5;
#pragma unroll
    for (int gg = 0; gg < G; gg++) {
        const int64_t gi = lane + kWave * gg;
        load32(x + (gi < groups ? gi : groups - 1) * 32, false, rr.v[gg]);
    }
}

// max |x| over a row loaded by row_load (a BF16 value, exact in FP32).
template <int G>
__device__ __forceinline__ float row_amax(const RowRegs<G>& rr, int64_t cols) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t groups = cols >> 5;
    uint32_t m = 0u;
#pragma unroll
    for (int gg = 0; gg < G; gg++) {
        const int64_t gi = lane + kWave * gg;
        if (gi < groups)
            m = max(m, max(max(absmax8_bits(rr.v[gg][0]), absmax8_bits(rr.v[gg][1])),
                           max(absmax8_bits(rr.v[gg][2]), absmax8_bits(rr.v[gg][3]))));
    }
    return bf16_to_f32(wave_max_u32(m));
}

// The rest of quant_row_regs on a row loaded by row_load.
template <int G>
__device__ __forceinline__ void row_quant(const RowRegs<G>& rr, int64_t cols, bool round_up, bool gemm, int64_t r,
                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                          float* __restrict__ gout) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t groups = cols >> 5;
    const RowScale rs = row_scale(row_amax<G>(rr, cols));
#pragma unroll
    for (int gg = 0; gg < G; gg++) {
        const int64_t gi = lane + kWave * gg;
        if (gi < groups) {
            u32x4 c;
            uint32_t s2;
            quant32(rr.v[gg], rs, round_up, false, c, s2);
            const int64_t k = gi * 32;
            if (gemm) {
                *reinterpret_cast<u32x4*>(codes + gemm_code_off(r, k, cols)) = c;
                *reinterpret_cast<uint16_t*>(scales + gemm_scale_off(r, k, cols)) = (uint16_t)s2;
            } else {
                *reinterpret_cast<u32x4*>(codes + r * (cols >> 1) + gi * 16) = c;
                *reinterpret_cast<uint16_t*>(scales + r * (cols >> 4) + gi * 2) = (uint16_t)s2;
            }
        }
    }
    if (lane == 0) gout[r] = rs.g;
}

// One row per wavefront, held in registers: lane l owns the 32-element groups
// l, l + 64, ... (G of them, cols <= 2048 G, cols % 32 == 0), so the row is
// read once for its amax and its quantization.  Same arithmetic and outputs
// as quant_row_wave.
template <int G>
__device__ __forceinline__ void quant_row_regs(const uint16_t* __restrict__ x, int64_t cols, bool round_up, bool gemm,
                                               int64_t r, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                               float* __restrict__ gout) {
    RowRegs<G> rr;
    row_load<G>(x, cols, rr);
    row_quant<G>(rr, cols, round_up, gemm, r, codes, scales, gout);
}

// Several short rows per wavefront (cols % 32 == 0, at most LPR 32-element
// groups per row): lane l quantizes group l % LPR of row r0 + l / LPR (rows at
// or past `rows` are skipped), and a row's amax is reduced over its own LPR
// lanes.  Same arithmetic and outputs as quant_row_regs; a row of 24 groups
// (768 columns) then keeps 48 of 64 lanes busy instead of 24.
template <int LPR>
__device__ __forceinline__ void quant_rows_packed(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                  int64_t ld, int64_t r0, bool round_up, bool gemm,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  float* __restrict__ gout) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t r = r0 + lane / LPR;
    const int gi = lane % LPR;
    const bool on = r < rows && gi < (cols >> 5);
    u32x4 v[4];
    uint32_t m = 0u;
    if (on) {
        load32(x + r * ld + gi * 32, false, v);
        m = max(max(absmax8_bits(v[0]), absmax8_bits(v[1])), max(absmax8_bits(v[2]), absmax8_bits(v[3])));
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, kWave));
    const RowScale rs = row_scale(bf16_to_f32(m));
    if (on) {
        u32x4 c;
        uint32_t s2;
        quant32(v, rs, round_up, false, c, s2);
        const int64_t k = (int64_t)gi * 32;
        if (gemm) {
            *reinterpret_cast<u32x4*>(codes + gemm_code_off(r, k, cols)) = c;
            *reinterpret_cast<uint16_t*>(scales + gemm_scale_off(r, k, cols)) = (uint16_t)s2;
        } else {
            *reinterpret_cast<u32x4*>(codes + r * (cols >> 1) + gi * 16) = c;
            *reinterpret_cast<uint16_t*>(scales + r * (cols >> 4) + gi * 2) = (uint16_t)s2;
        }
    }
    if (gi == 0 && r < rows) gout[r] = rs.g;
}

}  // namespace nvfp4
