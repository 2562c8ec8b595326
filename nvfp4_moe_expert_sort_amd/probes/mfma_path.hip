// mfma_path.hip -- the two exact ways to run an NVFP4 x NVFP4 GEMM on gfx950,
// timed side by side (the GEMM path choice: exact dequantization to a 16-bit
// MFMA format vs the scaled FP4 MFMA).
//
// An NVFP4 element is c * s: c an E2M1 code value, s the E4M3 scale of its
// 16-element block (miniTE summary page, "how it differs").
//
//  * f16 path (what gemm.hip does): c * s has at most 6 significant bits and
//    is exact in f16, so each operand fragment is decoded to f16 (hardware
//    FP4 -> f16 conversion, then one packed multiply by the f16 block scale)
//    and v_mfma_f32_32x32x16_f16 takes one 16-element block per instruction.
//  * scaled FP4 path: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies raw E2M1
//    codes and applies one power-of-two (E8M0) scale per lane, i.e. per 32
//    K values of a row or column.  An E4M3 scale is 2^e * m with a 3-bit
//    mantissa m, so only its exponent can ride in the instruction; m_a * m_b
//    differs per (row, column, block) and must be applied to the block's
//    partial sum in FP32 before it joins the accumulator.  Exactness
//    therefore takes one instruction per 16-element block (16 of its 64 K
//    slots used, the rest zero) plus, per output element and block, one
//    multiply (m_a * m_b) and one FMA.
//
// Both loops below use the production wave tile (128 rows x 64 columns: 4 x 2
// MFMA tiles, 8 MFMAs per 16-element K step) and two waves per SIMD, with
// operands in registers so that only instruction issue is measured:
//   f16 path     8 MFMAs + 24 VALU per K step (two weight fragments decoded
//                by the wave, its quarter of the shared activation decode);
//   scaled FP4   8 MFMAs + 256 VALU per K step (16 multiplies and 16 FMAs per
//                MFMA for the mantissa rescale; the row mantissas are not
//                refetched per block, which favours this path).
// Useful flops are 2 * 32 * 32 * 16 per MFMA in both.  Run it under
// `rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU
// SQ_ACTIVE_INST_VALU SQ_BUSY_CYCLES` for the pipe utilisation.
//
// First, a one-wave check that the scaled FP4 instruction's lane layout is
// the one assumed (lane l: row or column l % 32, K values 32 (l / 32) + i in
// nibble i of its 16 bytes, low nibble first) by comparing one 32x32x64
// product with exact host arithmetic.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

static const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
static float e2m1(unsigned nib) { return (nib & 8 ? -1.0f : 1.0f) * kE2M1[nib & 7]; }

// One wave: C (32x32) = A (32x64 FP4 codes) * B (64x32 FP4 codes), scales 2^0.
__global__ void layout_check(const int* a, const int* b, float* c) {
    const int lane = threadIdx.x;
    i32x8 va = {a[lane * 4 + 0], a[lane * 4 + 1], a[lane * 4 + 2], a[lane * 4 + 3], 0, 0, 0, 0};
    i32x8 vb = {b[lane * 4 + 0], b[lane * 4 + 1], b[lane * 4 + 2], b[lane * 4 + 3], 0, 0, 0, 0};
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 4, 4, 0, 127, 0, 127);
    for (int r = 0; r < 16; r++) c[lane * 16 + r] = acc[r];
}

__device__ __forceinline__ half8 decode8(uint32_t codes, half2v s2) {
    const half2v v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
    const half2v v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
    const half2v v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
    const half2v v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
    return half8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// MODE 0: f16 MFMAs only; 1: f16 path (decode + MFMA); 2: scaled FP4 MFMAs
// only; 3: exact scaled FP4 path (MFMA + mantissa rescale).
template <int MODE>
__global__ void __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
path_loop(float* out, int steps, uint32_t seed) {
    const int lane = threadIdx.x & 63;
    uint32_t code = seed * 2654435761u + lane * 40503u + 0x12345u;
    f32x16 acc[4][2];
    for (int i = 0; i < 4; i++) acc[i][0] = acc[i][1] = f32x16{};
    if (MODE <= 1) {
        half8 a[4], b[2];
        const half2v s2 = {(_Float16)0.5f, (_Float16)0.5f};
        for (int i = 0; i < 4; i++) a[i] = decode8(code ^ (0x01010101u * i), s2);
        for (int j = 0; j < 2; j++) b[j] = decode8(code ^ (0x10101010u * j), s2);
        for (int st0 = 0; st0 < steps; st0 += 4) {
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int st = st0 + u;
                if (MODE == 1) {
                    // the wave's per-step decode work: two weight fragments and a
                    // quarter of the activation tile's (one fragment)
                    const half2v sc = {(_Float16)(0.5f + (st & 1)), (_Float16)(0.5f + (st & 1))};
                    b[0] = decode8(code + st, sc);
                    b[1] = decode8(code ^ st, sc);
                    a[u] = decode8(code - st, sc);
                }
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
    } else {
        // 16 of the 64 K slots carry codes: the first 8 bytes of lanes 0..31
        const bool lo = lane < 32;
        i32x8 a[4], b[2];
        for (int i = 0; i < 4; i++) a[i] = i32x8{lo ? (int)(code ^ i) : 0, lo ? (int)(code + i) : 0, 0, 0, 0, 0, 0, 0};
        for (int j = 0; j < 2; j++) b[j] = i32x8{lo ? (int)(code * 3 + j) : 0, lo ? (int)(code * 5 ^ j) : 0, 0, 0, 0, 0, 0, 0};
        // mantissa factors (1 + f/8) of the E4M3 scales: per row register for A, per lane column for B
        // (the A side's are kept fixed across blocks here, which leaves out the
        // per-block fetch of 16 row mantissas a real kernel would need)
        float ma[4][16];
        for (int i = 0; i < 4; i++)
            for (int r = 0; r < 16; r++) ma[i][r] = 1.0f + (float)(((code * (2 * i + 1)) >> r) & 7) * 0.125f;
        for (int st = 0; st < steps; st++) {
            const int ea = 127 + (st & 3), eb = 127 - (st & 1);  // E8M0 exponents of this block's scales
            // this block's column mantissas, one per column tile (lane = column)
            const float mb[2] = {1.0f + (float)(((uint32_t)st ^ code) & 7u) * 0.125f,
                                 1.0f + (float)(((uint32_t)st ^ (code >> 3)) & 7u) * 0.125f};
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    if (MODE == 2) {
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, ea, 0,
                                                                                     eb);
                    } else {
                        const f32x16 part =
                            __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], f32x16{}, 4, 4, 0, ea, 0, eb);
#pragma unroll
                        for (int r = 0; r < 16; r++) acc[i][j][r] = __builtin_fmaf(part[r], ma[i][r] * mb[j], acc[i][j][r]);
                    }
                }
        }
    }
    float s = 0.0f;
    for (int i = 0; i < 4; i++)
        for (int j = 0; j < 2; j++)
            for (int r = 0; r < 16; r++) s += acc[i][j][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

#define CHECK(x)                                                                       \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(1);                                                                   \
        }                                                                              \
    } while (0)

template <int MODE>
static void run(const char* name, float* d, int blocks, int steps, int vpm) {
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    hipLaunchKernelGGL(path_loop<MODE>, dim3(blocks), dim3(256), 0, 0, d, 64, 1u);
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(path_loop<MODE>, dim3(blocks), dim3(256), 0, 0, d, steps, 1u);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double useful = 2.0 * 32 * 32 * 16 * 8.0 * steps * blocks * 4;
    printf("%-36s %8.3f ms  %7.1f TFLOP/s useful  (%d VALU per 8 MFMAs)\n", name, ms, useful / ms / 1e9, vpm);
}

int main() {
    // (1) layout check on one wave
    std::vector<int> ha(64 * 4), hb(64 * 4);
    srand(7);
    for (auto& v : ha) v = rand() ^ (rand() << 15);
    for (auto& v : hb) v = rand() ^ (rand() << 15);
    int *da, *db;
    float* dc;
    CHECK(hipMalloc(&da, ha.size() * 4));
    CHECK(hipMalloc(&db, hb.size() * 4));
    CHECK(hipMalloc(&dc, 64 * 16 * 4));
    CHECK(hipMemcpy(da, ha.data(), ha.size() * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(db, hb.data(), hb.size() * 4, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(layout_check, dim3(1), dim3(64), 0, 0, da, db, dc);
    CHECK(hipGetLastError());
    std::vector<float> hc(64 * 16);
    CHECK(hipMemcpy(hc.data(), dc, hc.size() * 4, hipMemcpyDeviceToHost));
    auto nib = [](const std::vector<int>& v, int lane, int i) {
        return ((unsigned)v[lane * 4 + i / 8] >> (4 * (i % 8))) & 0xFu;
    };
    int bad = 0;
    for (int lane = 0; lane < 64; lane++)
        for (int r = 0; r < 16; r++) {
            const int row = (r / 4) * 8 + (lane / 32) * 4 + r % 4, col = lane % 32;
            double ref = 0.0;
            for (int k = 0; k < 64; k++) {
                const int la = row + 32 * (k / 32), lb = col + 32 * (k / 32);
                ref += (double)e2m1(nib(ha, la, k % 32)) * (double)e2m1(nib(hb, lb, k % 32));
            }
            if ((double)hc[lane * 16 + r] != ref) bad++;
        }
    printf("scaled FP4 MFMA lane layout check: %d of 1024 outputs differ from exact host arithmetic\n", bad);
    if (bad) return 2;

    // (2) throughput of the two exact paths at the production wave tile, two waves per SIMD
    int dev = 0, cus = 256;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    const int blocks = 2 * cus, steps = 20000;  // a multiple of 4
    float* d;
    CHECK(hipMalloc(&d, (size_t)blocks * 256 * 4));
    run<0>("f16 MFMA only", d, blocks, steps, 0);
    run<1>("f16 path (decode + MFMA)", d, blocks, steps, 24);
    run<2>("scaled FP4 MFMA only (16 of 64 K)", d, blocks, steps, 0);
    run<3>("exact scaled FP4 path (MFMA + rescale)", d, blocks, steps, 256);
    CHECK(hipDeviceSynchronize());
    return 0;
}
