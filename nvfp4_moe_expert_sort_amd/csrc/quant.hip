// quant.hip -- NVFP4 quantizers on gfx950.
//
// miniTE summary page, "how it differs": per-row FP32 outer scale
// g = max|row| / (6*448), one E4M3 scale per 16 elements, E2M1 codes, round
// to nearest, no Hadamard transform, no stochastic rounding.  Both kernels are
// HBM-bound streaming kernels: each lane reads 64 contiguous bytes of one row
// and writes 16 bytes of codes.
//   quant_rows_kernel  one wave per row (generic entry point, weights, dense X);
//                      rows of up to 8192 columns are read once into registers,
//                      longer ones in two passes (amax, then quantize); rows of
//                      at most 1024 columns (a multiple of 32) go 2, 4 or 8 to
//                      a wave;
//   quant_h_kernel     FC2 input: one wave per (32-row tile, 128 columns) of
//                      the sorted buffer, writing whole 1 KiB GEMM chunks; the
//                      row amax is the max of the per-32-column maxima the FC1
//                      producer emitted (miniTE page, "how to use it": FC2
//                      maxima come from the router-weighted producer).
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"
#include "nvfp4_quant_row.h"

namespace nvfp4 {

__global__ void __launch_bounds__(256) quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                         int64_t ld, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, float* __restrict__ g,
                                                         int gemm, int round_up, int rows_per_wave) {
    const bool ru = round_up != 0, gm = gemm != 0;
    if (rows_per_wave > 1) {  // short rows, several per wavefront
        const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * rows_per_wave;
        if (r0 >= rows) return;
        switch (rows_per_wave) {
            case 2: quant_rows_packed<32>(x, rows, cols, ld, r0, ru, gm, codes, scales, g); break;
            case 4: quant_rows_packed<16>(x, rows, cols, ld, r0, ru, gm, codes, scales, g); break;
            default: quant_rows_packed<8>(x, rows, cols, ld, r0, ru, gm, codes, scales, g); break;
        }
        return;
    }
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint16_t* xr = x + row * ld;
    // Rows of up to 8192 columns (cols % 32 == 0) are read once into registers.
    const int64_t per_lane = (cols % 32 == 0) ? (cols / 32 + kWave - 1) / kWave : 0;
    switch (per_lane) {
        case 1: quant_row_regs<1>(xr, cols, ru, gm, row, codes, scales, g); break;
        case 2: quant_row_regs<2>(xr, cols, ru, gm, row, codes, scales, g); break;
        case 3: quant_row_regs<3>(xr, cols, ru, gm, row, codes, scales, g); break;
        case 4: quant_row_regs<4>(xr, cols, ru, gm, row, codes, scales, g); break;
        default: quant_row_wave(xr, cols, -1.0f, ru, gm, row, codes, scales, g); break;
    }
}

// 128-column steps per wave (measured at T = 4096: 1 step 26 us, 2 steps 30, 3 steps 33)
constexpr int kQuantHSteps = 1;

__global__ void __launch_bounds__(256) quant_h_kernel(const uint16_t* __restrict__ h, int64_t I,
                                                      const int32_t* __restrict__ expert_off, int32_t E,
                                                      int32_t capacity, const int32_t* __restrict__ expert_count,
                                                      const int32_t* __restrict__ row2pair,
                                                      const float* __restrict__ amax2_part, int n_part,
                                                      int64_t n_row_tiles, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, float* __restrict__ g,
                                                      int round_up) {
    // Block: four 32-row tiles (one per wave) x one column group of
    // kQuantHSteps 128-column steps; the groups of a quad run together on one
    // XCD (xcd_quad_group), so its rows' maxima and pairs are fetched once.
    const int lane = threadIdx.x & 63;
    const int64_t cps = I / 128;
    int64_t quad, grp;
    if (!xcd_quad_group((n_row_tiles + 3) / 4, (cps + kQuantHSteps - 1) / kQuantHSteps, quad, grp)) return;
    const int64_t rt = quad * 4 + (threadIdx.x >> 6);
    if (rt >= n_row_tiles) return;
    const int64_t cp0 = grp * kQuantHSteps;
    const int hh = lane >> 5, rl = lane & 31;
    const int64_t row = rt * 32 + rl;
    // Every load is issued before the test of whether this row tile holds an
    // expert's rows (all rows below the launch bound are in-bounds; a tile
    // past the last expert's rows reads values that are never used), so the
    // test's own load does not delay them.  The h loads go out first (padding
    // rows read in-bounds values that are never used), then the row's pair
    // and partial maxima: n_part = I / 32 floats, 16-byte aligned since
    // I % 128 == 0.
    u32x4 v[kQuantHSteps][2][4];
#pragma unroll
    for (int s = 0; s < kQuantHSteps; s++) {
        const int64_t cp = min(cp0 + s, cps - 1);  // a step past the end re-reads the last one (not stored)
#pragma unroll
        for (int ch = 0; ch < 2; ch++) load32(h + row * I + 64 * (2 * cp + ch) + 32 * hh, false, v[s][ch]);
    }
    const int32_t pr = row2pair[row];
    // Row amax: the maxima are non-negative floats, which order like their
    // bit patterns, so an integer max is exact.  The two lanes of a row
    // (lanes rl and rl + 32) each read half of every eight 16-byte vectors,
    // all in flight together (indices past the row's last vector re-read
    // it), and swap their partial maxima.
    const u32x4* part = reinterpret_cast<const u32x4*>(amax2_part + row * n_part);
    const int n4 = n_part / 4;
    uint32_t mbits = 0u;
    for (int i0 = 0; i0 < n4; i0 += 8) {
        u32x4 q[4];
#pragma unroll
        for (int j = 0; j < 4; j++) q[j] = part[min(i0 + 4 * hh + j, n4 - 1)];
#pragma unroll
        for (int j = 0; j < 4; j++) mbits = max(mbits, max(max(q[j][0], q[j][1]), max(q[j][2], q[j][3])));
    }
    mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, 32, kWave));
    if (!row_tile_used(rt, E, capacity, expert_off, expert_count)) return;
    const bool valid = pr >= 0;  // padding rows are written as zeros
    const float amax = valid ? __uint_as_float(mbits) : 0.0f;
    const RowScale rs = row_scale(amax);
#pragma unroll
    for (int s = 0; s < kQuantHSteps; s++) {
        const int64_t cp = cp0 + s;
        if (cp >= cps) break;
        uint32_t sc = 0u;
#pragma unroll
        for (int ch = 0; ch < 2; ch++) {
            const int64_t c = 2 * cp + ch;
            u32x4 cw = {0u, 0u, 0u, 0u};
            uint32_t s2 = 0u;
            if (valid) quant32(v[s][ch], rs, round_up != 0, false, cw, s2);
            *reinterpret_cast<u32x4*>(codes + (rt * (I / 64) + c) * 1024 + lane * 16) = cw;
            sc |= s2 << (16 * ch);
        }
        *reinterpret_cast<uint32_t*>(scales + (rt * (I / 128) + cp) * 256 + lane * 4) = sc;
    }
    if (cp0 == 0 && hh == 0) g[row] = valid ? rs.g : 0.0f;
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                             uint8_t* scales, float* g, bool gemm, bool round_up, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    // Rows of at most 32 groups of 32 elements share a wavefront: 2, 4 or 8
    // rows of up to 32, 16 or 8 groups.
    const int64_t groups = cols / 32;
    const int rpw = (cols % 32 != 0 || groups > 32) ? 1 : groups > 16 ? 2 : groups > 8 ? 4 : 8;
    const int64_t blocks = (rows + 4 * rpw - 1) / (4 * rpw);
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, cols, ld, codes,
                       scales, g, gemm ? 1 : 0, round_up ? 1 : 0, rpw);
    return hipGetLastError();
}

hipError_t launch_quant_h(const uint16_t* h, int64_t rows_bound, int64_t I, const int32_t* expert_off, int32_t E,
                          int32_t capacity, const int32_t* expert_count, const int32_t* row2pair,
                          const float* amax2_part, int n_part, uint8_t* codes, uint8_t* scales, float* g,
                          bool round_up, hipStream_t stream) {
    const int64_t n_row_tiles = rows_bound / 32, groups = (I / 128 + kQuantHSteps - 1) / kQuantHSteps;
    if (n_row_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(quant_h_kernel, dim3(xcd_quad_group_blocks((n_row_tiles + 3) / 4, groups)), dim3(256), 0, stream,
                       h, I, expert_off, E, capacity, expert_count, row2pair, amax2_part, n_part, n_row_tiles, codes,
                       scales, g, round_up ? 1 : 0);
    return hipGetLastError();
}

}  // namespace nvfp4
