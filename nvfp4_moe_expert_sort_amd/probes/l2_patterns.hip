// l2_patterns.hip -- L2 -> CU read bandwidth of operand-fetch patterns on
// gfx950 (a stand-alone measurement program, not part of the library).
//
// Every workgroup (1024 of them, 256 threads) reads the same 2 MiB buffer,
// which stays in each XCD's L2, with one 16-byte load per lane.  One wave
// instruction covers `rows` rows of `bpr` bytes each (bpr = 1024: 1 KiB
// contiguous), the rows `pitch` bytes apart -- the shapes in which the GEMM
// kernels fetch a row-major operand tile (for example 8 rows x 128 bytes of
// a KC operand's 64-deep chunk, or 2 rows x 512 bytes of a 256-wide MC
// chunk).  Each wave keeps eight loads in flight; nothing is written except
// one word per thread that the compiler cannot prove unused.  Prints one
// line per pattern: bytes per row, pitch, time and TB/s.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kBytes = 2u << 20;
constexpr int kBlocks = 1024;
constexpr int kSteps = 256;  // load instructions per wave and repetition

__global__ void __launch_bounds__(256) read_pattern(const uint8_t* __restrict__ buf, int bpr, int pitch, int reps,
                                                    uint32_t* __restrict__ out) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lanes_per_row = bpr / 16;
    const int r = lane / lanes_per_row, c = lane % lanes_per_row;
    const uint32_t span = (uint32_t)(64 / lanes_per_row) * (uint32_t)pitch;  // bytes one instruction spans
    const uint32_t nblk = (kBytes - 4096) / span;
    // column window of a wave inside the row (several waves, several windows)
    const uint32_t win = pitch > bpr ? (uint32_t)(pitch - bpr) : 0u;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int rep = 0; rep < reps; rep++) {
        for (int it = 0; it < kSteps; it += 8) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const uint32_t blk = (uint32_t)(it + u + blockIdx.x * 7 + wave * 3) % nblk;
                const uint32_t col = win ? ((uint32_t)((wave + u) % 4) * (uint32_t)bpr) % (win + 16u) : 0u;
                uint32_t off = blk * span + (uint32_t)r * (uint32_t)pitch + (col & ~15u) + (uint32_t)c * 16u;
                off = (off % (kBytes - 16u)) & ~15u;  // in bounds: off + 16 <= kBytes
                v[u] = *reinterpret_cast<const u32x4*>(buf + off);
            }
#pragma unroll
            for (int u = 0; u < 8; u++) acc += v[u];
        }
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x12345678u) out[blockIdx.x * 256 + tid] = acc[0];
}

static int check(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return 1;
    }
    return 0;
}

int main() {
    uint8_t* buf = nullptr;
    uint32_t* out = nullptr;
    if (check(hipMalloc(&buf, kBytes), "hipMalloc") || check(hipMalloc(&out, (size_t)kBlocks * 256 * 4), "hipMalloc") ||
        check(hipMemset(buf, 1, kBytes), "hipMemset"))
        return 1;
    // {bytes per row, row pitch}: 1 KiB contiguous, then the GEMM fetch shapes
    // at the pitches of the operands (H = 2048 and I = 768 BF16 rows: 4096 and
    // 1536 bytes; 2I: 3072) and at pitches off a multiple of 1 KiB.
    const int cases[][2] = {{1024, 1024}, {128, 4096}, {128, 4224}, {128, 3072}, {128, 1536},
                            {256, 4096},  {256, 4352}, {256, 3072}, {256, 1536}, {512, 4096},
                            {512, 4608},  {512, 1536}, {64, 4096},  {32, 4096}};
    hipEvent_t a, b;
    if (check(hipEventCreate(&a), "hipEventCreate") || check(hipEventCreate(&b), "hipEventCreate")) return 1;
    for (const auto& cs : cases) {
        const int bpr = cs[0], pitch = cs[1], reps = 8;
        hipLaunchKernelGGL(read_pattern, dim3(kBlocks), dim3(256), 0, 0, buf, bpr, pitch, 1, out);  // warm-up
        hipEventRecord(a);
        hipLaunchKernelGGL(read_pattern, dim3(kBlocks), dim3(256), 0, 0, buf, bpr, pitch, reps, out);
        hipEventRecord(b);
        if (check(hipEventSynchronize(b), "kernel")) return 1;
        float ms = 0.0f;
        hipEventElapsedTime(&ms, a, b);
        const double bytes = (double)kBlocks * 256 * kSteps * 16 * reps;
        printf("bytes/row %4d pitch %5d: %8.1f us  %.2f TB/s\n", bpr, pitch, ms * 1e3, bytes / (ms * 1e-3) / 1e12);
        fflush(stdout);
    }
    hipFree(buf);
    hipFree(out);
    return 0;
}
