// nvfp4_device.h -- device helpers shared by the gfx950 kernels: NVFP4 format
// encoders, the GEMM-layout address map and wave reductions.
//
// Formats (miniTE summary page, section "how it differs"): E2M1 element codes,
// one OCP E4M3FN scale per 16 elements, one FP32 outer scale per row
// g = max|row| / (6*448), round to nearest, no stochastic rounding.  The E4M3
// rounding of the block scale is a build-time reading (round up by default,
// RNE selectable); both are exact integer/bit manipulations below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_kernels.h"

namespace nvfp4 {

constexpr int kWave = 64;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// float -> BF16 bits with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t bf16_hw(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// silu(a) = a / (1 + e^-a) in FP32 with the hardware base-2 exponential
// (v_exp_f32, on a * -log2(e)) and reciprocal (v_rcp_f32).  Used by the FC1
// epilogue and by the separate SwiGLU producer, so both give the same bits.
__device__ __forceinline__ float silu_fast(float a) {
    const float e = __builtin_amdgcn_exp2f(a * -1.4426950408889634f);
    return a * __builtin_amdgcn_rcpf(1.0f + e);
}

// The router-weighted SwiGLU output of one element: gate and up are the BF16
// FC1 outputs (as FP32), p the router probability; one BF16 rounding.
__device__ __forceinline__ uint32_t swiglu_prob_bf16(float gate, float up, float p) {
    return bf16_hw(silu_fast(gate) * up * p);
}

// E4M3FN byte of a non-negative block scale v.  round_up: the smallest E4M3FN
// value >= v; otherwise nearest with ties to an even mantissa.  Clamped to
// 448 (0x7E); 0 for v <= 0.  The hardware conversion v_cvt_pk_fp8_f32 rounds
// to nearest even (subnormal codes included); round-up takes the next code
// when that value lies below v (codes of non-negative values are monotone).
// Checked on the GPU against an integer encoder written from the format
// (exponent, 3-bit mantissa, ceil/rint) for every non-negative binary32
// pattern below 512, both modes: no difference.
__device__ __forceinline__ uint32_t e4m3_encode(float v, bool round_up) {
    if (!(v > 0.0f)) return 0u;
    const float c = fminf(v, 448.0f);
    uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
    if (round_up && __builtin_amdgcn_cvt_f32_fp8(code, 0) < c) code += 1u;
    return code;
}

// E4M3FN byte -> float (gfx950 converts the OCP E4M3FN format in hardware).
__device__ __forceinline__ float e4m3_decode(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8(byte, 0); }

// --- GEMM layout (see include/nvfp4moe.h) -------------------------------------------------------
// Byte offset of the 4-byte group holding columns [k, k+8) (k % 8 == 0) of row r.
__device__ __forceinline__ size_t gemm_code_off(int64_t r, int64_t k, int64_t cols) {
    int64_t rt = r >> 5, rl = r & 31, c = k >> 6, h = (k >> 5) & 1;
    return (size_t)((rt * (cols >> 6) + c) * 1024 + (h * 32 + rl) * 16 + ((k & 31) >> 1));
}
// Byte offset of the scale of the 16-column block starting at column k of row r.
__device__ __forceinline__ size_t gemm_scale_off(int64_t r, int64_t k, int64_t cols) {
    int64_t rt = r >> 5, rl = r & 31, c = k >> 6, h = (k >> 5) & 1;
    return (size_t)((rt * (cols >> 7) + (c >> 1)) * 256 + (h * 32 + rl) * 4 + (c & 1) * 2 + ((k & 31) >> 4));
}

// --- XCD-aware block order ---------------------------------------------------------------------
// A 1-D grid over (row-tile quad q, column group j) with j fastest within an
// XCD: workgroups are dispatched round-robin over the 8 XCDs (block b runs on
// XCD b % 8), so block b takes item b / 8 of XCD b % 8's list, whose items
// are its quads x, x + 8, x + 16, ... each followed by all its column groups.
// The column groups of one row-tile quad then run together on one XCD and
// share its L2 for the per-row data they all read.  Returns false for the
// padding blocks past the last quad.
__device__ __forceinline__ bool xcd_quad_group(int64_t n_quads, int64_t groups, int64_t& quad, int64_t& group) {
    const int64_t b = blockIdx.x, x = b & 7, i = b >> 3;
    quad = (i / groups) * 8 + x;
    group = i % groups;
    return quad < n_quads;
}
inline unsigned xcd_quad_group_blocks(int64_t n_quads, int64_t groups) {
    return (unsigned)(((n_quads + 7) / 8) * 8 * groups);
}

// --- wave reductions ----------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
    return v;
}

}  // namespace nvfp4
