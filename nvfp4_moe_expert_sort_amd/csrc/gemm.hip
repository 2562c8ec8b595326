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
//  * A workgroup of 4 wavefronts (one per SIMD; two workgroups share each CU,
//    so every SIMD runs two independent waves at 256 registers each) owns a
//    tile of 128 rows x 256 B-rows (FC2: 256 output columns; FC1: 128 gate
//    and the matching 128 up rows, i.e. 128 columns of h).  Each wave owns 128
//    rows x 2 MFMA column tiles (128 FP32 accumulators).  The two workgroups
//    on a CU drift apart, so one's epilogue and barriers overlap the other's
//    MFMAs.
//  * The activation tile is decoded once per workgroup: for every 128-column
//    step wave w decodes the 32-row tile w (both 64-column chunks) into LDS,
//    and all four waves read their MFMA A operands from there.  Each wave
//    decodes its own weight columns in registers.  In the GEMM layout one
//    16-byte load per lane fetches 32 rows x 64 columns as one contiguous
//    1 KiB; both operands use the same column permutation inside a 64-column
//    chunk, which leaves the dot product unchanged.
//  * Double-buffered LDS, one barrier per 128-column step; loads for the next
//    step are issued before the current step's MFMAs.
//  * Workgroups walk a tile list whose length is read on the device (no host
//    sync).  Workgroups with blockIdx % 8 == x (one XCD under round-robin
//    dispatch) take one contiguous range of tiles, so an expert's weight slab
//    and its row tiles meet in that XCD's L2.  The grid is either persistent
//    (two workgroups per CU, each walking its share of the range) or hybrid:
//    persistent workgroups walk a static bulk of equal tile counts and one
//    workgroup per tile takes the last rounds (the hardware dispatcher then
//    balances those tiles over the CU slots as they free up).
//  * No split-K, one K order, one instruction sequence per row for every batch
//    size: a row's bits depend only on its own inputs.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"
#include "nvfp4_quant_row.h"

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

// Scale of k-steps {0,1} (first) and {2,3} (second) of chunk CH of a 128-column step.
template <int CH>
__device__ __forceinline__ void scales_of(uint32_t sdw, half2v& lo, half2v& hi) {
    lo = scale2<2 * CH>(sdw);
    hi = scale2<2 * CH + 1>(sdw);
}

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// LDS: decoded A operands, [buffer][32-row tile][chunk][k-step][lane] x 16 bytes.
// After the K loop the same 64 KiB stage the epilogue (per-wave slices).
struct SharedA {
    half8 a[2][4][2][4][64];
};

// LDS: the next 128-column step's raw weight codes, written by direct
// global->LDS loads, [wave][chunk][column tile][lane] x 16 bytes.
struct SharedB {
    u32x4 b[kWaves][2][2][64];
};

// s_waitcnt immediates (gfx9 encoding): vmcnt(0), and lgkmcnt(0).
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// Workgroup barrier that orders this wave's LDS reads and writes only: the
// next steps' global and global->LDS loads stay in flight (their wave-private
// destinations are waited for separately).  The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ADEC false: this wave has no activation subtile of its own (wave >= NSUB)
// and is compiled without the K loop's activation decodes; the choice is made
// once per tile by a wave-uniform branch, so the MFMA stream has no branch.
// AQ true (FC1 only): the activations arrive in BF16 and are quantized here,
// one 32-element group per lane and chunk, just before their decode.
template <int MODE, int NSUB, bool ADEC, bool AQ>
__device__ __forceinline__ void block_tile(const GemmParams& P, SharedA& S, SharedB& SB, int32_t row0, int32_t expert,
                                           int32_t row_end, int32_t nt) {
    // wave index as a scalar, so per-wave conditions are scalar branches
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = P.K;
    const int64_t kc64 = K >> 6, kc128 = K >> 7;

    // This wave's two weight column tiles (wave 0's always exist).
    int32_t bcol0[2];
    bool active;
    if (MODE == kGemmSwiGLU) {
        const int32_t hc = nt * 128 + 32 * wave;
        active = hc < P.inter;
        bcol0[0] = hc;            // gate rows
        bcol0[1] = P.inter + hc;  // the matching up rows
    } else {
        const int32_t c = nt * 256 + 64 * wave;
        active = c < P.N;
        bcol0[0] = c;
        bcol0[1] = c + 32;
    }
    // Every load below is issued unconditionally from an in-bounds address
    // (an idle wave reads wave 0's columns or row tile 0; the last step
    // re-reads its own operands), so no loaded value joins a conditional
    // default and the compiler never has to wait for it early.
    const int32_t wcol = active ? 0 : (MODE == kGemmSwiGLU ? 32 : 64) * wave;
    int64_t rtb[2];
#pragma unroll
    for (int j = 0; j < 2; j++) rtb[j] = ((int64_t)expert * P.N + bcol0[j] - wcol) >> 5;

    // The activation units this wave decodes for every 128-column step: its
    // 32-row tile `wave`, both 64-column chunks.
    const int ai = wave;
    const bool adec = ai < NSUB;
    const int64_t rta = (row0 >> 5) + (adec ? ai : 0);

    const uint8_t* a_c = P.a_codes + lane * 16;
    const uint8_t* a_s = P.a_scales + lane * 4;

    // AQ: lane l of wave `ai` owns row row0 + 32 ai + l % 32 and, in every
    // 64-column chunk, the 32 columns of half l / 32 -- exactly the GEMM
    // layout's 16-byte unit of that lane -- which it quantizes with the
    // library's 32-element quantizer against its token's outer scale: the
    // codes and scales the sort's quantizer and gather put in that unit.
    const uint16_t* xrow = P.a_bf16;
    RowScale rsa{0.0f, 0.0f, true};
    if (AQ && ADEC) {
        const int32_t arow = row0 + 32 * ai + (lane & 31);
        const int32_t pr = P.a_row2pair[arow];
        // padding rows read token 0 (their results are never stored)
        const int64_t tok = pr >= 0 ? (int64_t)((uint32_t)pr / (uint32_t)P.a_top_k) : 0;
        rsa = row_scale(P.a_amax[tok]);
        xrow = P.a_bf16 + tok * K + 32 * (lane >> 5);
    }
    auto load_xa = [&](int64_t cp, u32x4 (&vb)[2][4]) {
#pragma unroll
        for (int ch = 0; ch < 2; ch++) load32(xrow + 128 * cp + 64 * ch, false, vb[ch]);
    };
    // chunk ch's codes into xa, its two block scales into bytes 2ch, 2ch + 1 of ya
    auto quant_xa = [&](int ch, const u32x4 (&vb)[4], u32x4& xa, uint32_t& ya) {
        uint32_t s2;
        quant32(vb, rsa, P.a_round_up != 0, false, xa, s2);
        ya = ch == 0 ? s2 : (ya | (s2 << 16));
    };
    const uint8_t* b_c = P.b_codes + lane * 16;
    const uint8_t* b_s = P.b_scales + lane * 4;

    // Plain mode: row scales of the tile's rows for the epilogue, fetched before
    // the K loop; lane l holds rows l and 64 + l (clamped to the tile's rows).
    const int colL = lane & 31;
    constexpr int kLastRow = 32 * NSUB - 1;
    float rg0 = 0.0f, rg1 = 0.0f;
    if (MODE == kGemmPlain) {
        rg0 = P.a_g[row0 + min(lane, kLastRow)];
        rg1 = NSUB > 2 ? P.a_g[row0 + min(64 + lane, kLastRow)] : 0.0f;
    }

    // The weight global scales of this wave's columns (column l % 32 of each
    // column tile), for the epilogue, loaded before the K loop.
    float cg[2];
#pragma unroll
    for (int j = 0; j < 2; j++) cg[j] = P.b_g[(int64_t)expert * P.N + bcol0[j] - wcol + (lane & 31)];
    f32x16 acc[NSUB][2];
#pragma unroll
    for (int i = 0; i < NSUB; i++) {
        acc[i][0] = f32x16{};
        acc[i][1] = f32x16{};
    }

    auto load_a = [&](int64_t cp, u32x4 (&xa)[2], uint32_t& ya) {
#pragma unroll
        for (int ch = 0; ch < 2; ch++) xa[ch] = *reinterpret_cast<const u32x4*>(a_c + (rta * kc64 + 2 * cp + ch) * 1024);
        ya = *reinterpret_cast<const uint32_t*>(a_s + (rta * kc128 + cp) * 256);
    };
    auto load_bs = [&](int64_t cp, uint32_t (&yb)[2]) {
#pragma unroll
        for (int j = 0; j < 2; j++) yb[j] = *reinterpret_cast<const uint32_t*>(b_s + (rtb[j] * kc128 + cp) * 256);
    };
    // Weight codes of step cp straight into this wave's LDS slice (lane l's
    // 16 bytes land at slice + 16 l); no registers are held while in flight.
    auto dma_b = [&](int64_t cp) {
#pragma unroll
        for (int ch = 0; ch < 2; ch++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(b_c + (rtb[j] * kc64 + 2 * cp + ch) * 1024),
                    (__attribute__((address_space(3))) void*)&SB.b[wave][ch][j][0], 16, 0, 0);
    };
    auto decode_a = [&](int buf, const u32x4 (&xa)[2], uint32_t ya) {
        if (!adec) return;
        half2v lo0, hi0, lo1, hi1;
        scales_of<0>(ya, lo0, hi0);
        scales_of<1>(ya, lo1, hi1);
#pragma unroll
        for (int ks = 0; ks < 4; ks++) S.a[buf][ai][0][ks][lane] = decode8(xa[0][ks], ks < 2 ? lo0 : hi0);
#pragma unroll
        for (int ks = 0; ks < 4; ks++) S.a[buf][ai][1][ks][lane] = decode8(xa[1][ks], ks < 2 ? lo1 : hi1);
    };

    u32x4 ub[2][2];  // this step's weight codes [chunk][column tile]
    uint32_t usb[2];
    {
        u32x4 ua[2] = {};
        uint32_t usa = 0u;
        if (AQ) {
            if (ADEC) {
                u32x4 vb[2][4];
                load_xa(0, vb);
                quant_xa(0, vb[0], ua[0], usa);
                quant_xa(1, vb[1], ua[1], usa);
            }
        } else {
            load_a(0, ua, usa);
        }
#pragma unroll
        for (int ch = 0; ch < 2; ch++)
#pragma unroll
            for (int j = 0; j < 2; j++) ub[ch][j] = *reinterpret_cast<const u32x4*>(b_c + (rtb[j] * kc64 + ch) * 1024);
        load_bs(0, usb);
        if (kc128 > 1) dma_b(1);
        decode_a(0, ua, usa);
    }
    barrier_lds();
    // Issue priority: the K loop's MFMA stream outranks a neighbouring
    // wave's epilogue (VALU-heavy), so the two waves that share a SIMD keep
    // its matrix pipe busy while one of them finishes a tile.
    __builtin_amdgcn_s_setprio(2);
    for (int64_t cp = 0; cp < kc128; cp++) {
        const int buf = (int)(cp & 1);
        const bool more = cp + 1 < kc128;
        const int64_t cpn = more ? cp + 1 : cp;
        u32x4 na[2];
        uint32_t nsa, nsb[2];
        u32x4 nv[2][4];  // AQ: the next step's BF16 activations
        if (AQ) {
            if (ADEC) load_xa(cpn, nv);
        } else {
            load_a(cpn, na, nsa);
        }
        load_bs(cpn, nsb);
        if (active) {
            half2v bsc[2][2][2];  // [chunk][column tile][lo/hi]
#pragma unroll
            for (int j = 0; j < 2; j++) {
                scales_of<0>(usb[j], bsc[0][j][0], bsc[0][j][1]);
                scales_of<1>(usb[j], bsc[1][j][0], bsc[1][j][1]);
            }
            half8 acur[NSUB];
#pragma unroll
            for (int i = 0; i < NSUB; i++) acur[i] = S.a[buf][i][0][0][lane];
            // Eight k-steps of 16 columns; the A operands of k-step s+1 are read
            // from LDS and its weights decoded while the MFMAs of k-step s run.
            half8 bv[2];
#pragma unroll
            for (int j = 0; j < 2; j++) bv[j] = decode8(ub[0][j][0], bsc[0][j][0]);
#pragma unroll
            for (int st = 0; st < 8; st++) {
                half8 anxt[NSUB];
                if (st < 7) {
#pragma unroll
                    for (int i = 0; i < NSUB; i++) anxt[i] = S.a[buf][i][(st + 1) >> 2][(st + 1) & 3][lane];
                }
                half8 bn[2];
                const int sn = st < 7 ? st + 1 : 7, chn = sn >> 2, ksn = sn & 3;
#pragma unroll
                for (int i = 0; i < NSUB; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(acur[i], bv[j], acc[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 2; j++) bn[j] = decode8(ub[chn][j][ksn], bsc[chn][j][ksn >> 1]);
                // AQ: the next step's activations quantized on k-steps 2 and 3
                // (one chunk each), ahead of their decode on k-steps 4..7
                if (AQ && ADEC && st == 2) quant_xa(0, nv[0], na[0], nsa);
                if (AQ && ADEC && st == 3) quant_xa(1, nv[1], na[1], nsa);
                if (st < 7) {
#pragma unroll
                    for (int i = 0; i < NSUB; i++) acur[i] = anxt[i];
                }
                // The next step's activation fragments (loaded at this step's
                // start, arrived by its second half) are decoded two per
                // k-step on k-steps 4..7, into the other LDS buffer; the
                // barrier at the step's end orders them before any reader.  On
                // the last step they re-decode this step's codes into a buffer
                // nobody reads.  A wave with no activation tile of its own
                // (wave >= NSUB) is compiled without them.
                if (ADEC && st >= 4) {
                    half2v sl, sh;
                    if ((st - 4) < 2)
                        scales_of<0>(nsa, sl, sh);
                    else
                        scales_of<1>(nsa, sl, sh);
#pragma unroll
                    for (int ff = 0; ff < 2; ff++) {
                        const int f = 2 * (st - 4) + ff, fch = f >> 2, fks = f & 3;
                        S.a[buf ^ 1][ai][fch][fks][lane] = decode8(na[fch][fks], fks < 2 ? sl : sh);
                    }
                }
                // The next k-step's A-operand reads and decodes (its weights;
                // on k-steps 4..7 also the next step's activations) issue in
                // the shadow of this k-step's MFMAs -- after each MFMA one LDS
                // read (the first NSUB) and four VALU slots -- instead of in a
                // burst between two k-steps: a lone wave on its SIMD keeps its
                // matrix pipe fed.
#pragma unroll
                for (int q = 0; q < NSUB * 2; q++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    if (q < NSUB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 2; j++) bv[j] = bn[j];
            }
        } else {
            if (AQ && ADEC) {
                quant_xa(0, nv[0], na[0], nsa);
                quant_xa(1, nv[1], na[1], nsa);
            }
            decode_a(buf ^ 1, na, nsa);
        }
        // Step cp+1's weight codes: landed in LDS (wait for this wave's
        // loads), into registers, then the slice is refilled for step cp+2.
        // On the last step this re-reads the slice; the values go unused.
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
        for (int ch = 0; ch < 2; ch++)
#pragma unroll
            for (int j = 0; j < 2; j++) ub[ch][j] = SB.b[wave][ch][j][lane];
        usb[0] = nsb[0];
        usb[1] = nsb[1];
        if (cp + 2 < kc128) {
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // slice read before it is overwritten
            dma_b(cp + 2);
        }
        barrier_lds();
    }
    __builtin_amdgcn_s_setprio(0);  // epilogue at the lowest priority
    if (!active) return;

    // Epilogue.  Lane l holds, for register r of an MFMA tile, row
    // (r/4)*8 + (l/32)*4 + r%4 and column l%32 of that 32x32 tile.  Results go
    // through this wave's own slice of the (now idle) LDS operand buffers, so
    // global stores are 16 bytes per lane and each row's max |h| is a
    // lane-local reduction.  In plain mode the tile's row scales go to the
    // wave's raw-weight slice, from where the four consecutive rows of a
    // register group are one broadcast read.  Both slices are wave-private and
    // LDS accesses of one wave complete in order; the barrier at the end of
    // the tile loop orders them against the next tile's LDS writes.  Nothing
    // here waits for the global stores.
    const int rowL = (lane >> 5) * 4;
    float* RS = reinterpret_cast<float*>(&SB.b[wave][0][0][0]);
    if (MODE == kGemmPlain) {
        RS[lane] = rg0;
        RS[64 + lane] = rg1;
    }
    if (MODE == kGemmSwiGLU) {
        constexpr int kPitch = 40;  // halves per staged row: 32 columns + 8 pad (80 B, conflict-free)
        uint16_t* E = reinterpret_cast<uint16_t*>(&S) + wave * (128 * kPitch);
#pragma unroll
        for (int i = 0; i < NSUB; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                // Rows past row_end (an expert's padding) are computed from
                // in-bounds scale/probability entries and never stored.
                const int rl = 32 * i + (r >> 2) * 8 + rowL + (r & 3);
                const int32_t row = row0 + rl;
                const float gx = P.a_g[row];
                const float pr = P.row_prob[row];
                const float yg = bf16_to_f32(bf16_hw(acc[i][0][r] * (gx * cg[0])));
                const float yu = bf16_to_f32(bf16_hw(acc[i][1][r] * (gx * cg[1])));
                E[rl * kPitch + colL] = (uint16_t)swiglu_prob_bf16(yg, yu, pr);
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        const int32_t part = bcol0[0] >> 5;
#pragma unroll
        for (int half = 0; half < 2; half++) {
            const int rl = lane + 64 * half;
            if (rl < 32 * NSUB) {
                const u32x4* src = reinterpret_cast<const u32x4*>(E + rl * kPitch);
                u16x2 m = {0, 0};
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const u32x4 v = src[q];
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v[j] & 0x7FFF7FFFu));
                }
                const int32_t row = row0 + rl;
                if (row < row_end) {
                    // max |h| over these 32 columns: BF16 bit patterns of |h|
                    // order like their values, so the integer max is exact.
                    const uint32_t mb = max((uint32_t)m[0], (uint32_t)m[1]);
                    P.amax_part[(int64_t)row * P.n_part + part] = __uint_as_float(mb << 16);
                }
            }
        }
        // h leaves in whole 128-byte lines: once all four waves have staged
        // their 32 columns, the workgroup stores its 128 columns (256 bytes
        // of each row), 16 lanes per row, 16-byte chunk c of row r going to
        // thread (16 r + c) % 256.  (All four waves reach this barrier: the
        // inner size is a multiple of 128, so every wave has h columns.)
        barrier_lds();
        // (the thread index passes through an empty asm after the barrier, so
        // the store addresses are not computed before the K loop and held
        // in registers across it)
        int tid = (int)threadIdx.x;
        asm volatile("" : "+v"(tid));
        const uint16_t* E0 = reinterpret_cast<const uint16_t*>(&S);
        const int32_t hc0 = nt * 128;
#pragma unroll
        for (int q = 0; q < 2 * NSUB; q++) {
            const int c = q * kThreads + tid;
            const int rl = c >> 4, cc = c & 15;
            const u32x4 v = *reinterpret_cast<const u32x4*>(E0 + (cc >> 2) * (128 * kPitch) + rl * kPitch + 8 * (cc & 3));
            const int32_t row = row0 + rl;
            if (row < row_end) *reinterpret_cast<u32x4*>(P.out + (int64_t)row * P.ld_out + hc0 + 8 * cc) = v;
        }
    } else {
        constexpr int kPitch = 72;  // halves per staged row: 64 columns + 8 pad (144 B, conflict-free)
        uint16_t* E = reinterpret_cast<uint16_t*>(&S) + wave * (32 * kPitch);
        // one 32-row MFMA tile per pass; the wave's 64 columns of a row are 128
        // contiguous bytes of the output, so eight lanes store one row (lane l:
        // row 8q + l/8 of the pass, bytes 16 (l % 8)) and each store
        // instruction writes eight whole 128-byte lines
#pragma unroll
        for (int i = 0; i < NSUB; i++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int rb = 8 * q + rowL;  // first of this lane's four rows in the pass
                const float4 g4 = *reinterpret_cast<const float4*>(RS + 32 * i + rb);  // rows past row_end are not stored
                const float ga[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 4 * q + e;
                    E[(rb + e) * kPitch + colL] = (uint16_t)bf16_hw(acc[i][0][r] * (ga[e] * cg[0]));
                    E[(rb + e) * kPitch + 32 + colL] = (uint16_t)bf16_hw(acc[i][1][r] * (ga[e] * cg[1]));
                }
            }
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int r = 8 * q + (lane >> 3), pc = 8 * (lane & 7);
                const int32_t row = row0 + 32 * i + r;
                const u32x4 v = *reinterpret_cast<const u32x4*>(E + r * kPitch + pc);
                if (row < row_end)
                    *reinterpret_cast<u32x4*>(P.out + (int64_t)row * P.ld_out + bcol0[0] + pc) = v;
            }
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // slice read before the next pass overwrites it
            __builtin_amdgcn_wave_barrier();
        }
    }
}

template <int MODE, bool AQ = false>
__global__ void __launch_bounds__(kThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_kernel(GemmParams P) {
    __shared__ SharedA S;
    __shared__ SharedB SB;
    const int64_t n_mt = P.dense_m >= 0 ? (P.dense_m + kTileRows - 1) / kTileRows : *P.n_mtiles;
    const int64_t total = n_mt * P.n_tiles_n;
    const int64_t nb = gridDim.x;  // a multiple of 8
    const int64_t xcd = blockIdx.x & 7;
    int64_t slot = blockIdx.x >> 3, per = nb >> 3;
    int64_t t_begin = total * xcd / 8, t_end = total * (xcd + 1) / 8;
    if (P.persist > 0) {
        // Hybrid grid: workgroups [0, persist) walk a static bulk of
        // (tiles / persist - 1) rounds, exactly that many tiles each; the
        // remaining one to two rounds go one tile per workgroup to the rest of
        // the grid, which the dispatcher starts as the persistent ones finish.
        const int64_t np = P.persist;
        const int64_t S = (total / np > 1 ? total / np - 1 : 0) * np;
        if (blockIdx.x < np) {
            t_begin = S * xcd / 8;
            t_end = S * (xcd + 1) / 8;
            per = np >> 3;
        } else {
            t_begin = S + (total - S) * xcd / 8;
            t_end = S + (total - S) * (xcd + 1) / 8;
            slot = (blockIdx.x - np) >> 3;
            per = (nb - np) >> 3;
        }
    }
    // Each tile's descriptor is loaded one tile ahead, so a tile's first
    // operand loads do not wait for it.
    auto tile_desc = [&](int64_t t) -> int4 {
        const int64_t mt = (uint32_t)t / (uint32_t)P.n_tiles_n;  // tile indices are < 2^31
        if (P.dense_m >= 0) {
            const int32_t row0 = (int32_t)(mt * kTileRows);
            return make_int4(row0, 0, min(4, (P.dense_m - row0 + kMAlign - 1) / kMAlign), P.dense_m);
        }
        return P.mtiles[mt];
    };
    int64_t t = t_begin + slot;
    if (t >= t_end || per <= 0) return;
    int4 d = tile_desc(t);
    for (; t < t_end; t += per) {
        const int32_t nt = (int32_t)((uint32_t)t % (uint32_t)P.n_tiles_n);
        const int4 cur = d;
        if (t + per < t_end) d = tile_desc(t + per);
        const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
        switch (cur.z) {
            case 4: block_tile<MODE, 4, true, AQ>(P, S, SB, cur.x, cur.y, cur.w, nt); break;
            case 3:
                if (wv < 3)
                    block_tile<MODE, 3, true, AQ>(P, S, SB, cur.x, cur.y, cur.w, nt);
                else
                    block_tile<MODE, 3, false, AQ>(P, S, SB, cur.x, cur.y, cur.w, nt);
                break;
            case 2:
                if (wv < 2)
                    block_tile<MODE, 2, true, AQ>(P, S, SB, cur.x, cur.y, cur.w, nt);
                else
                    block_tile<MODE, 2, false, AQ>(P, S, SB, cur.x, cur.y, cur.w, nt);
                break;
            default:
                if (wv < 1)
                    block_tile<MODE, 1, true, AQ>(P, S, SB, cur.x, cur.y, cur.w, nt);
                else
                    block_tile<MODE, 1, false, AQ>(P, S, SB, cur.x, cur.y, cur.w, nt);
                break;
        }
        barrier_lds();  // the next tile's prologue overwrites LDS buffer 0
    }
}

int gemm_cols_per_tile(int mode) { return mode == kGemmSwiGLU ? 128 : 256; }

hipError_t launch_gemm(int mode, const GemmParams& P, int grid_blocks, hipStream_t stream, bool aq) {
    const int g = (grid_blocks + 7) / 8 * 8;
    if (mode == kGemmSwiGLU && aq)
        hipLaunchKernelGGL((gemm_kernel<kGemmSwiGLU, true>), dim3(g), dim3(kThreads), 0, stream, P);
    else if (mode == kGemmSwiGLU)
        hipLaunchKernelGGL(gemm_kernel<kGemmSwiGLU>, dim3(g), dim3(kThreads), 0, stream, P);
    else
        hipLaunchKernelGGL(gemm_kernel<kGemmPlain>, dim3(g), dim3(kThreads), 0, stream, P);
    return hipGetLastError();
}

}  // namespace nvfp4
