// gemm.hip -- grouped NVFP4 GEMM on gfx950 with the FP32 epilogue.
//
// miniTE summary page, "how it differs": the GEMM consumes E2M1 codes with
// 16-element E4M3 block scales, accumulates in FP32, and its epilogue
// multiplies by g^x * g^w and casts to BF16; the router probability scales the
// SwiGLU output before FC2.  "How to use it": the GEMM reads the quantizer's
// contiguous buffer directly, expert boundaries are device offsets, and FC1
// and FC2 have separate GEMM configurations.  Article section 4.4: each row is
// accumulated in one fixed order, SiLU(gate) * up is formed in FP32 and
// rounded once.
//
// Design (gfx950):
//  * Exact dequantization to f16.  s * c with c in E2M1 and s in E4M3 has at
//    most 6 significant bits and lies in [2^-10, 2688], so it is exact in f16;
//    every f16 x f16 product is exact in FP32, so the only rounding is the
//    FP32 accumulation inside v_mfma_f32_32x32x16_f16.  The hardware FP4
//    conversion (v_cvt_scalef32_pk_f16_fp4) applies only the exponent of its
//    scale operand, so it runs with scale 1.0 and the E4M3 block scale is
//    applied by one packed f16 multiply (exact).
//  * Operands go from HBM/L2 straight to registers: in the GEMM layout one
//    16-byte load per lane fetches 32 rows x 64 columns contiguously, and a
//    lane's 32 codes feed four MFMAs.  Both operands use the same column
//    permutation inside a 64-column chunk, so the dot product is unchanged.
//  * One wavefront per workgroup owns a 128 x 128 output tile (4 x 4 MFMA
//    tiles, 256 FP32 accumulators): decode work per MFMA is halved relative
//    to 64-wide tiles, which keeps the VALU decode inside the MFMA shadow.
//  * Persistent waves walk a tile list whose length is read on the device (no
//    host sync).  Waves with blockIdx % 8 == x (the same XCD under round-robin
//    dispatch) take one contiguous range of tiles, so an expert's weight slab
//    is fetched from HBM into that XCD's L2 once and reused by its row tiles.
//  * No split-K, one K order, one instruction sequence per row for every
//    batch size: a row's bits depend only on its own inputs.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

__device__ __forceinline__ half8 decode8(uint32_t codes, half2v s2) {
    const half2v v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
    const half2v v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
    const half2v v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
    const half2v v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
    return half8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

template <int SEL>
__device__ __forceinline__ half2v scale2(uint32_t sdw) {
    const _Float16 s = (_Float16)__builtin_amdgcn_cvt_f32_fp8(sdw, SEL);  // exact: E4M3 values are f16-normal
    return half2v{s, s};
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

template <int MODE, int NSUB>
__device__ __forceinline__ void gemm_tile(const GemmParams& P, int32_t row0, int32_t expert, int32_t row_end,
                                          int32_t nt) {
    const int lane = threadIdx.x & 63;
    const int64_t K = P.K;
    const int64_t kc64 = K >> 6, kc128 = K >> 7;
    // Row tiles (32 rows each) of A and B.
    int64_t rta[NSUB], rtb[4];
    int32_t bcol0[4];
#pragma unroll
    for (int i = 0; i < NSUB; i++) rta[i] = (row0 >> 5) + i;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        bcol0[j] = MODE == kGemmSwiGLU ? nt * 64 + 32 * (j & 1) + (j >> 1) * P.inter : nt * 128 + 32 * j;
        rtb[j] = ((int64_t)expert * P.N + bcol0[j]) >> 5;
    }
    const uint8_t* a_c = P.a_codes + lane * 16;
    const uint8_t* b_c = P.b_codes + lane * 16;
    const uint8_t* a_s = P.a_scales + lane * 4;
    const uint8_t* b_s = P.b_scales + lane * 4;

    f32x16 acc[NSUB][4];
#pragma unroll
    for (int i = 0; i < NSUB; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x16{};

    // Raw operands for one 128-column step (two 64-column chunks).
    u32x4 ca[2][NSUB], cb[2][4];
    uint32_t sa[NSUB], sb[4];
    auto load = [&](int64_t cp, u32x4 (&xa)[2][NSUB], u32x4 (&xb)[2][4], uint32_t (&ya)[NSUB],
                    uint32_t (&yb)[4]) {
#pragma unroll
        for (int ch = 0; ch < 2; ch++) {
#pragma unroll
            for (int i = 0; i < NSUB; i++)
                xa[ch][i] = *reinterpret_cast<const u32x4*>(a_c + (rta[i] * kc64 + 2 * cp + ch) * 1024);
#pragma unroll
            for (int j = 0; j < 4; j++)
                xb[ch][j] = *reinterpret_cast<const u32x4*>(b_c + (rtb[j] * kc64 + 2 * cp + ch) * 1024);
        }
#pragma unroll
        for (int i = 0; i < NSUB; i++) ya[i] = *reinterpret_cast<const uint32_t*>(a_s + (rta[i] * kc128 + cp) * 256);
#pragma unroll
        for (int j = 0; j < 4; j++) yb[j] = *reinterpret_cast<const uint32_t*>(b_s + (rtb[j] * kc128 + cp) * 256);
    };

    load(0, ca, cb, sa, sb);
    for (int64_t cp = 0; cp < kc128; cp++) {
        u32x4 na[2][NSUB], nb[2][4];
        uint32_t nsa[NSUB], nsb[4];
        if (cp + 1 < kc128) load(cp + 1, na, nb, nsa, nsb);
#pragma unroll
        for (int ch = 0; ch < 2; ch++) {
            // scale of the block holding k-steps 0,1 (sel ch*2) and 2,3 (sel ch*2+1) of this chunk
            half2v as0[NSUB], as1[NSUB], bs0[4], bs1[4];
#pragma unroll
            for (int i = 0; i < NSUB; i++) {
                as0[i] = ch == 0 ? scale2<0>(sa[i]) : scale2<2>(sa[i]);
                as1[i] = ch == 0 ? scale2<1>(sa[i]) : scale2<3>(sa[i]);
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                bs0[j] = ch == 0 ? scale2<0>(sb[j]) : scale2<2>(sb[j]);
                bs1[j] = ch == 0 ? scale2<1>(sb[j]) : scale2<3>(sb[j]);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                half8 av[NSUB], bv[4];
#pragma unroll
                for (int i = 0; i < NSUB; i++) av[i] = decode8(ca[ch][i][ks], ks < 2 ? as0[i] : as1[i]);
#pragma unroll
                for (int j = 0; j < 4; j++) bv[j] = decode8(cb[ch][j][ks], ks < 2 ? bs0[j] : bs1[j]);
#pragma unroll
                for (int i = 0; i < NSUB; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
            }
        }
        if (cp + 1 < kc128) {
#pragma unroll
            for (int ch = 0; ch < 2; ch++) {
#pragma unroll
                for (int i = 0; i < NSUB; i++) ca[ch][i] = na[ch][i];
#pragma unroll
                for (int j = 0; j < 4; j++) cb[ch][j] = nb[ch][j];
            }
#pragma unroll
            for (int i = 0; i < NSUB; i++) sa[i] = nsa[i];
#pragma unroll
            for (int j = 0; j < 4; j++) sb[j] = nsb[j];
        }
    }

    // Epilogue.  Lane l holds, for register r of an MFMA tile, row
    // (r/4)*8 + (l/32)*4 + r%4 and column l%32 of that 32x32 tile.
    const int colL = lane & 31;
    const int rowL = (lane >> 5) * 4;
    if (MODE == kGemmSwiGLU) {
        const float gwg0 = P.b_g[(int64_t)expert * P.N + bcol0[0] + colL];
        const float gwg1 = P.b_g[(int64_t)expert * P.N + bcol0[1] + colL];
        const float gwu0 = P.b_g[(int64_t)expert * P.N + bcol0[2] + colL];
        const float gwu1 = P.b_g[(int64_t)expert * P.N + bcol0[3] + colL];
#pragma unroll
        for (int i = 0; i < NSUB; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int32_t row = row0 + 32 * i + (r >> 2) * 8 + rowL + (r & 3);
                const bool valid = row < row_end;
                const float gx = valid ? P.a_g[row] : 0.0f;
                const float pr = valid ? P.row_prob[row] : 0.0f;
                float m = 0.0f;
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const float gg = gx * (j == 0 ? gwg0 : gwg1);
                    const float gu = gx * (j == 0 ? gwu0 : gwu1);
                    const float yg = bf16_to_f32(f32_to_bf16_rne(acc[i][j][r] * gg));
                    const float yu = bf16_to_f32(f32_to_bf16_rne(acc[i][j + 2][r] * gu));
                    const uint32_t hb = f32_to_bf16_rne(silu(yg) * yu * pr);
                    m = fmaxf(m, fabsf(bf16_to_f32(hb)));
                    if (valid) P.out[(int64_t)row * P.ld_out + nt * 64 + 32 * j + colL] = (uint16_t)hb;
                }
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
                if (valid && colL == 0) P.amax_part[(int64_t)row * P.n_tiles_n + nt] = m;
            }
        }
    } else {
        float gw[4];
#pragma unroll
        for (int j = 0; j < 4; j++) gw[j] = P.b_g[(int64_t)expert * P.N + bcol0[j] + colL];
#pragma unroll
        for (int i = 0; i < NSUB; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int32_t row = row0 + 32 * i + (r >> 2) * 8 + rowL + (r & 3);
                if (row < row_end) {
                    const float ga = P.a_g[row];
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const uint32_t y = f32_to_bf16_rne(acc[i][j][r] * (ga * gw[j]));
                        P.out[(int64_t)row * P.ld_out + bcol0[j] + colL] = (uint16_t)y;
                    }
                }
            }
        }
    }
}

template <int MODE>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_kernel(GemmParams P) {
    const int64_t n_mt = P.dense_m >= 0 ? (P.dense_m + kTileRows - 1) / kTileRows : *P.n_mtiles;
    const int64_t total = n_mt * P.n_tiles_n;
    const int64_t nw = gridDim.x;          // a multiple of 8
    const int64_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = nw >> 3;
    const int64_t t_begin = total * xcd / 8, t_end = total * (xcd + 1) / 8;
    for (int64_t t = t_begin + slot; t < t_end; t += per) {
        const int64_t mt = t / P.n_tiles_n;
        const int32_t nt = (int32_t)(t % P.n_tiles_n);
        int32_t row0, expert, nsub, row_end;
        if (P.dense_m >= 0) {
            row0 = (int32_t)(mt * kTileRows);
            expert = 0;
            nsub = min(4, (P.dense_m - row0 + kMAlign - 1) / kMAlign);
            row_end = P.dense_m;
        } else {
            const int4 d = P.mtiles[mt];
            row0 = d.x;
            expert = d.y;
            nsub = d.z;
            row_end = d.w;
        }
        switch (nsub) {
            case 4: gemm_tile<MODE, 4>(P, row0, expert, row_end, nt); break;
            case 3: gemm_tile<MODE, 3>(P, row0, expert, row_end, nt); break;
            case 2: gemm_tile<MODE, 2>(P, row0, expert, row_end, nt); break;
            default: gemm_tile<MODE, 1>(P, row0, expert, row_end, nt); break;
        }
    }
}

hipError_t launch_gemm(int mode, const GemmParams& P, int grid_waves, hipStream_t stream) {
    const int g = (grid_waves + 7) / 8 * 8;
    if (mode == kGemmSwiGLU)
        hipLaunchKernelGGL(gemm_kernel<kGemmSwiGLU>, dim3(g), dim3(64), 0, stream, P);
    else
        hipLaunchKernelGGL(gemm_kernel<kGemmPlain>, dim3(g), dim3(64), 0, stream, P);
    return hipGetLastError();
}

}  // namespace nvfp4
