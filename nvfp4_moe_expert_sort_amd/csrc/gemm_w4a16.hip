// gemm_w4a16.hip -- grouped GEMMs of the W4A16 variant: NVFP4 weights, BF16
// activations left unquantized (the article, section 6: NVFP4 W4A16 routed
// experts).  Same grouping, same per-row contract as the W4A4 GEMM: FC1 is
// followed by the router-weighted SwiGLU producer, each output is one FP32
// accumulation in one fixed K order, and the epilogue multiplies by g^w only
// (the activations carry no outer scale) before the BF16 cast.
//
// Design (gfx950): one workgroup per (32-row subtile, column tile); each of
// its 4 waves owns 2 MFMA column tiles (FC1: 32 gate and the matching 32 up
// rows of W1; FC2: 64 output columns).  Both operands go straight from memory
// into registers in the MFMA operand layout: in the GEMM layout lane
// (h*32 + r) holds weight row r, columns [64c + 32h, 64c + 32h + 32), and the
// MFMA of k-step j of chunk c takes its columns 8j .. 8j + 7, so the matching
// BF16 activations are 16 contiguous bytes of row r.  Weights are decoded
// exactly: E2M1 x E4M3 has at most 6 significant bits, exact in BF16; the
// products of BF16 values are exact in FP32.  FC1 reads each sorted row's
// token row of x through row2pair (no sorted copy of x is built).  No LDS,
// no split-K, no configuration chosen by the token count.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

typedef __bf16 w16_bf16x8 __attribute__((ext_vector_type(8)));
typedef float w16_f32x2 __attribute__((ext_vector_type(2)));

// 8 E2M1 codes (one 32-bit word, code i in bits 4i..4i+3) times an E4M3 scale
// value s, as BF16 (exact).  The hardware conversion applies only the
// exponent of its scale operand, so it runs at 1.0 and s multiplies in FP32.
__device__ __forceinline__ w16_bf16x8 w16_decode8(uint32_t codes, float s) {
    const w16_f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    const w16_f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    const w16_f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    const w16_f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    return w16_bf16x8{(__bf16)(v0[0] * s), (__bf16)(v0[1] * s), (__bf16)(v1[0] * s), (__bf16)(v1[1] * s),
                      (__bf16)(v2[0] * s), (__bf16)(v2[1] * s), (__bf16)(v3[0] * s), (__bf16)(v3[1] * s)};
}

// E4M3 scale byte `sel` (0..3) of a scale word, as FP32 (exact).
__device__ __forceinline__ float w16_scale(uint32_t sw, int sel) {
    switch (sel) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8(sw, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8(sw, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8(sw, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8(sw, 3);
    }
}

__device__ __forceinline__ uint32_t w16_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float w16_silu(float a) {
    const float e = __builtin_amdgcn_exp2f(a * -1.4426950408889634f);
    return a * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int MODE>
__global__ void __launch_bounds__(256) gemm_w4a16_kernel(W16Params P) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nt = blockIdx.x % P.n_tiles_n, rest = blockIdx.x / P.n_tiles_n;
    const int64_t sub = rest % 4, mt = rest / 4;
    if (mt >= *P.n_mtiles) return;
    const int4 d = P.mtiles[mt];
    if (sub >= d.z) return;
    const int32_t row0 = d.x + 32 * (int32_t)sub, expert = d.y, row_end = d.w;

    int32_t bcol[2];
    bool active;
    if (MODE == kGemmSwiGLU) {
        const int32_t hc = (int32_t)nt * 128 + 32 * wave;
        active = hc < P.inter;
        bcol[0] = hc;
        bcol[1] = P.inter + hc;
    } else {
        const int32_t c = (int32_t)nt * 256 + 64 * wave;
        active = c < P.N;
        bcol[0] = c;
        bcol[1] = c + 32;
    }
    if (!active) return;

    const int r = lane & 31, h = lane >> 5;
    const int64_t K = P.K, kc64 = K >> 6, kc128 = K >> 7;
    // this lane's activation row
    const int64_t arow = row0 + r;
    int64_t src = arow;
    if (P.row2pair) {
        const int32_t pair = P.row2pair[arow];
        src = pair >= 0 ? pair / P.top_k : 0;  // padding rows read token 0 and are not stored
    }
    const uint16_t* a = P.a + src * K + 32 * h;
    const uint8_t* bc[2];
    const uint8_t* bs[2];
#pragma unroll
    for (int jt = 0; jt < 2; jt++) {
        const int64_t rt = ((int64_t)expert * P.N + bcol[jt]) >> 5;
        bc[jt] = P.b_codes + rt * kc64 * 1024 + lane * 16;
        bs[jt] = P.b_scales + rt * kc128 * 256 + lane * 4;
    }

    f32x16 acc[2] = {f32x16{}, f32x16{}};
    for (int64_t cp = 0; cp < kc128; cp++) {  // 128 columns: two 64-column chunks
        u32x4 av[2][4], bv[2][2];
        uint32_t sw[2];
#pragma unroll
        for (int ch = 0; ch < 2; ch++) {
#pragma unroll
            for (int j = 0; j < 4; j++) av[ch][j] = *reinterpret_cast<const u32x4*>(a + 128 * cp + 64 * ch + 8 * j);
#pragma unroll
            for (int jt = 0; jt < 2; jt++) bv[ch][jt] = *reinterpret_cast<const u32x4*>(bc[jt] + (2 * cp + ch) * 1024);
        }
#pragma unroll
        for (int jt = 0; jt < 2; jt++) sw[jt] = *reinterpret_cast<const uint32_t*>(bs[jt] + cp * 256);
#pragma unroll
        for (int ch = 0; ch < 2; ch++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int jt = 0; jt < 2; jt++) {
                    // scale byte (ch*2 + j/2) of the dword: the 16-column block of k-step j
                    const float s = w16_scale(sw[jt], ch * 2 + (j >> 1));
                    const w16_bf16x8 bw = w16_decode8(bv[ch][jt][j], s);
                    acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(w16_bf16x8, av[ch][j]), bw,
                                                                      acc[jt], 0, 0, 0);
                }
    }

    // Register i of an MFMA tile: row (i/4)*8 + h*4 + i%4, column r.
    const int64_t wrow0 = (int64_t)expert * P.N;
    if (MODE == kGemmSwiGLU) {
        const float gg = P.b_g[wrow0 + bcol[0] + r], gu = P.b_g[wrow0 + bcol[1] + r];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int32_t row = row0 + (i >> 2) * 8 + h * 4 + (i & 3);
            if (row >= row_end) continue;
            const float yg = __uint_as_float(w16_bf16_rne(acc[0][i] * gg) << 16);
            const float yu = __uint_as_float(w16_bf16_rne(acc[1][i] * gu) << 16);
            P.out[(int64_t)row * P.ld_out + bcol[0] + r] = (uint16_t)w16_bf16_rne(w16_silu(yg) * yu * P.row_prob[row]);
        }
    } else {
#pragma unroll
        for (int jt = 0; jt < 2; jt++) {
            const float gw = P.b_g[wrow0 + bcol[jt] + r];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int32_t row = row0 + (i >> 2) * 8 + h * 4 + (i & 3);
                if (row < row_end) P.out[(int64_t)row * P.ld_out + bcol[jt] + r] = (uint16_t)w16_bf16_rne(acc[jt][i] * gw);
            }
        }
    }
}

hipError_t launch_gemm_w4a16(int mode, const W16Params& P, int64_t mt_bound, hipStream_t stream) {
    const int64_t blocks = mt_bound * 4 * P.n_tiles_n;
    if (blocks <= 0) return hipSuccess;
    if (mode == kGemmSwiGLU)
        hipLaunchKernelGGL(gemm_w4a16_kernel<kGemmSwiGLU>, dim3((unsigned)blocks), dim3(256), 0, stream, P);
    else
        hipLaunchKernelGGL(gemm_w4a16_kernel<kGemmPlain>, dim3((unsigned)blocks), dim3(256), 0, stream, P);
    return hipGetLastError();
}

}  // namespace nvfp4
