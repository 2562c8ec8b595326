// gemm_w4a16.hip -- grouped GEMMs of the W4A16 variant: NVFP4 weights, BF16
// activations left unquantized (the article, section 6: NVFP4 W4A16 routed
// experts).  Same grouping, same per-row contract as the W4A4 GEMM: FC1 is
// followed by the router-weighted SwiGLU producer, each output is one FP32
// accumulation in one fixed K order, and the epilogue multiplies by g^w only
// (the activations carry no outer scale) before the BF16 cast.
//
// Design (gfx950): one workgroup of 4 waves per (row tile of up to 128 rows,
// column tile); each wave owns 2 MFMA column tiles (FC1: 32 gate and the
// matching 32 up rows of W1; FC2: 64 output columns) for all the tile's rows.
// For every 128-column step wave w loads the BF16 rows of 32-row subtile w
// into LDS in the MFMA operand layout (in the GEMM layout lane (h*32 + r)
// holds weight row r, columns [64c + 32h, 64c + 32h + 32), and the MFMA of
// k-step j of chunk c takes its columns 8j .. 8j + 7, so the matching
// activations are 16 contiguous bytes of row r); every wave reads its A
// operands there and decodes its own weight columns in registers, exactly:
// E2M1 x E4M3 has at most 6 significant bits, exact in BF16, and products of
// BF16 values are exact in FP32.  FC1 reads each sorted row's token row of x
// through row2pair (no sorted copy of x is built).  No split-K, no
// configuration chosen by the token count.
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


// Workgroup barrier ordering LDS accesses only: global loads in flight (the
// next step's weights) stay in flight; the compiler waits for loaded values
// where they are used.  The memory clobber keeps accesses on their side.
__device__ __forceinline__ void w16_barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS: this step's and the next step's activation fragments,
// [buffer][32-row subtile][64-column chunk][k-step][lane] x 16 bytes.
struct W16SharedA {
    u32x4 a[2][4][2][4][64];
};

template <int MODE, int NSUB>
__device__ __forceinline__ void w16_tile(const W16Params& P, W16SharedA& S, int32_t row0, int32_t expert,
                                         int32_t row_end, int32_t nt) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int32_t bcol[2];
    bool active;
    if (MODE == kGemmSwiGLU) {
        const int32_t hc = nt * 128 + 32 * wave;
        active = hc < P.inter;
        bcol[0] = hc;
        bcol[1] = P.inter + hc;
    } else {
        const int32_t c = nt * 256 + 64 * wave;
        active = c < P.N;
        bcol[0] = c;
        bcol[1] = c + 32;
    }
    // An idle wave still loads its subtile's activations (the others need
    // them) and reads wave 0's weight columns, which it never uses.
    const int32_t wcol = active ? 0 : (MODE == kGemmSwiGLU ? 32 : 64) * wave;
    const int r = lane & 31, h = lane >> 5;
    // The weight global scales of this wave's columns (column r of each
    // column tile), for the epilogue, loaded before the K loop.
    const int64_t wrow0 = (int64_t)expert * P.N;
    const float cg0 = P.b_g[wrow0 + bcol[0] - wcol + r], cg1 = P.b_g[wrow0 + bcol[1] - wcol + r];
    const int64_t K = P.K, kc64 = K >> 6, kc128 = K >> 7;
    // activation row of this wave's subtile (a wave past the tile's subtiles
    // re-reads subtile 0 and stores nothing)
    const bool aload = wave < NSUB;
    const int64_t arow = row0 + 32 * (aload ? wave : 0) + r;
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
        const int64_t rt = ((int64_t)expert * P.N + bcol[jt] - wcol) >> 5;
        bc[jt] = P.b_codes + rt * kc64 * 1024 + lane * 16;
        bs[jt] = P.b_scales + rt * kc128 * 256 + lane * 4;
    }
    auto load_a = [&](int64_t cp, int ch, u32x4 (&v)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ks++) v[ks] = *reinterpret_cast<const u32x4*>(a + 128 * cp + 64 * ch + 8 * ks);
    };
    auto load_b = [&](int64_t cp, u32x4 (&v)[2][2], uint32_t (&sw)[2]) {
#pragma unroll
        for (int ch = 0; ch < 2; ch++)
#pragma unroll
            for (int jt = 0; jt < 2; jt++) v[ch][jt] = *reinterpret_cast<const u32x4*>(bc[jt] + (2 * cp + ch) * 1024);
#pragma unroll
        for (int jt = 0; jt < 2; jt++) sw[jt] = *reinterpret_cast<const uint32_t*>(bs[jt] + cp * 256);
    };
    auto store_a = [&](int buf, int ch, const u32x4 (&v)[4]) {
        if (!aload) return;
#pragma unroll
        for (int ks = 0; ks < 4; ks++) S.a[buf][wave][ch][ks][lane] = v[ks];
    };

    f32x16 acc[NSUB][2];
#pragma unroll
    for (int i = 0; i < NSUB; i++) {
        acc[i][0] = f32x16{};
        acc[i][1] = f32x16{};
    }
    // The next step's activations pass through registers one 64-column chunk
    // at a time: chunk 0 is loaded at the step's start and stored to LDS
    // halfway, chunk 1 is loaded then and stored at the step's end.
    u32x4 av[4], bcur[2][2], bnxt[2][2];
    uint32_t scur[2], snxt[2];
    load_a(0, 0, av);
    load_b(0, bcur, scur);
    store_a(0, 0, av);
    load_a(0, 1, av);
    store_a(0, 1, av);
    w16_barrier_lds();
    // The K loop's MFMA stream outranks a co-resident workgroup's epilogue.
    __builtin_amdgcn_s_setprio(2);
    for (int64_t cp = 0; cp < kc128; cp++) {
        const int buf = (int)(cp & 1);
        const int64_t cn = cp + 1 < kc128 ? cp + 1 : cp;  // the last step re-reads its own operands
        load_a(cn, 0, av);
        load_b(cn, bnxt, snxt);
#pragma unroll
        for (int st = 0; st < 8; st++) {
            const int ch = st >> 2, ks = st & 3;
            if (st == 4) {
                store_a(buf ^ 1, 0, av);
                load_a(cn, 1, av);
            }
            w16_bf16x8 af[NSUB];
#pragma unroll
            for (int i = 0; i < NSUB; i++) af[i] = __builtin_bit_cast(w16_bf16x8, S.a[buf][i][ch][ks][lane]);
            w16_bf16x8 bw[2];
#pragma unroll
            for (int jt = 0; jt < 2; jt++) bw[jt] = w16_decode8(bcur[ch][jt][ks], w16_scale(scur[jt], 2 * ch + (ks >> 1)));
#pragma unroll
            for (int i = 0; i < NSUB; i++)
#pragma unroll
                for (int jt = 0; jt < 2; jt++)
                    acc[i][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bw[jt], acc[i][jt], 0, 0, 0);
        }
        store_a(buf ^ 1, 1, av);  // step cp+1's fragments are in the other buffer
        w16_barrier_lds();
#pragma unroll
        for (int ch = 0; ch < 2; ch++)
#pragma unroll
            for (int jt = 0; jt < 2; jt++) bcur[ch][jt] = bnxt[ch][jt];
        scur[0] = snxt[0];
        scur[1] = snxt[1];
    }
    __builtin_amdgcn_s_setprio(0);
    if (!active) return;

    // Register i of MFMA tile (t, jt): row 32t + (i/4)*8 + h*4 + i%4 of the
    // tile, column r of column tile jt.  Each 32-row subtile goes through this
    // wave's own slice of the (now idle) LDS buffer, so a lane stores 16-byte
    // pieces of one row; the slices are wave-private and one wave's LDS
    // accesses complete in order.
    constexpr int kPitch = 72;  // halves per staged row: 64 columns + 8 pad
    uint16_t* E = reinterpret_cast<uint16_t*>(&S) + wave * (32 * kPitch);
    const int rowL = h * 4;
    if (MODE == kGemmSwiGLU) {
        // h leaves in whole 128-byte lines: each wave stages its 32 columns of
        // all the tile's rows, then the workgroup stores the tile's 128 columns
        // (256 bytes of each row), 16 lanes per row.  (All four waves get
        // here: the inner size is a multiple of 128, so every wave has h
        // columns.)
        constexpr int kPitchH = 40;  // halves per staged row: 32 columns + 8 pad (80 B, conflict-free)
        uint16_t* EH = reinterpret_cast<uint16_t*>(&S) + wave * (128 * kPitchH);
        const float gg = cg0, gu = cg1;
#pragma unroll
        for (int t = 0; t < NSUB; t++) {
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int rr = (i >> 2) * 8 + rowL + (i & 3);
                const int32_t row = min(row0 + 32 * t + rr, row_end - 1);  // rows past the end are not stored
                const float yg = __uint_as_float(bf16_hw(acc[t][0][i] * gg) << 16);
                const float yu = __uint_as_float(bf16_hw(acc[t][1][i] * gu) << 16);
                EH[(32 * t + rr) * kPitchH + r] = (uint16_t)swiglu_prob_bf16(yg, yu, P.row_prob[row]);
            }
        }
        w16_barrier_lds();
        // (the thread index passes through an empty asm after the barrier, so
        // the store addresses are not computed early and held in registers)
        int tid = (int)threadIdx.x;
        asm volatile("" : "+v"(tid));
        const uint16_t* E0 = reinterpret_cast<const uint16_t*>(&S);
        const int32_t hc0 = bcol[0] - 32 * wave;  // the tile's first h column
#pragma unroll
        for (int q = 0; q < 2 * NSUB; q++) {
            const int c = q * 256 + tid;
            const int rl = c >> 4, cc = c & 15;  // row of the tile, 8-column chunk (wave cc / 4's slice)
            const u32x4 v = *reinterpret_cast<const u32x4*>(E0 + (cc >> 2) * (128 * kPitchH) + rl * kPitchH + 8 * (cc & 3));
            const int32_t row = row0 + rl;
            if (row < row_end) *reinterpret_cast<u32x4*>(P.out + (int64_t)row * P.ld_out + hc0 + 8 * cc) = v;
        }
    } else {
        const float g0 = cg0, g1 = cg1;
#pragma unroll
        for (int t = 0; t < NSUB; t++) {
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int rr = (i >> 2) * 8 + rowL + (i & 3);
                E[rr * kPitch + r] = (uint16_t)bf16_hw(acc[t][0][i] * g0);
                E[rr * kPitch + 32 + r] = (uint16_t)bf16_hw(acc[t][1][i] * g1);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
            // lane l: row l % 32, columns 32 (l / 32) .. + 32 of the wave's 64
            const int32_t row = row0 + 32 * t + r;
            if (row < row_end) {
                const u32x4* src = reinterpret_cast<const u32x4*>(E + r * kPitch + 32 * h);
                u32x4* dst = reinterpret_cast<u32x4*>(P.out + (int64_t)row * P.ld_out + bcol[0] + 32 * h);
#pragma unroll
                for (int q = 0; q < 4; q++) dst[q] = src[q];
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// One workgroup of 4 waves per (row tile of up to 128 rows, column tile):
// the activation tile is loaded once per 128-column step (wave w loads
// subtile w) into LDS, from where every wave reads its MFMA operands; each
// wave decodes its own weight columns in registers.  Workgroup b runs on XCD
// b % 8 (round-robin dispatch), and XCD x takes the contiguous range
// [x * span, (x + 1) * span) of the device's tile list, so a row tile's
// column tiles and an expert's row tiles -- which share activations and a
// weight slab -- meet in one XCD's L2.  The grid (a multiple of 8) covers
// the static tile bound.
template <int MODE>
__global__ void __launch_bounds__(256, 2) gemm_w4a16_kernel(W16Params P) {
    __shared__ W16SharedA S;
    const int64_t total = (int64_t)(*P.n_mtiles) * P.n_tiles_n;
    const int64_t span = (total + 7) / 8, slot = blockIdx.x >> 3;
    if (slot >= span) return;
    const int64_t tile = (int64_t)(blockIdx.x & 7) * span + slot;
    if (tile >= total) return;
    const int32_t nt = (int32_t)(tile % P.n_tiles_n);
    const int64_t mt = tile / P.n_tiles_n;
    const int4 d = P.mtiles[mt];
    switch (d.z) {
        case 4: w16_tile<MODE, 4>(P, S, d.x, d.y, d.w, nt); break;
        case 3: w16_tile<MODE, 3>(P, S, d.x, d.y, d.w, nt); break;
        case 2: w16_tile<MODE, 2>(P, S, d.x, d.y, d.w, nt); break;
        default: w16_tile<MODE, 1>(P, S, d.x, d.y, d.w, nt); break;
    }
}

hipError_t launch_gemm_w4a16(int mode, const W16Params& P, int64_t mt_bound, hipStream_t stream) {
    const int64_t blocks = (mt_bound * P.n_tiles_n + 7) / 8 * 8;
    if (blocks <= 0) return hipSuccess;
    if (mode == kGemmSwiGLU)
        hipLaunchKernelGGL(gemm_w4a16_kernel<kGemmSwiGLU>, dim3((unsigned)blocks), dim3(256), 0, stream, P);
    else
        hipLaunchKernelGGL(gemm_w4a16_kernel<kGemmPlain>, dim3((unsigned)blocks), dim3(256), 0, stream, P);
    return hipGetLastError();
}

}  // namespace nvfp4
