// backward.hip -- BF16 straight-through backward of the expert forward.
//
// miniTE summary page, "how it differs": the backward takes quantization as
// the identity (straight-through) and runs BF16 GEMMs on the stored original
// BF16 activations and weights, so nothing is quantized on the way back; the
// router probability multiplies the SwiGLU output, and the combine is a plain
// sum over the top-k slots.  With sorted row r holding pair p = t*K + k of
// expert e (the forward's sort), the steps are
//   dh[r]      = bf16(dout[t] . W2[e])                     grouped GEMM, K = H
//   dgate, dup = bf16(dh p up silu'(gate)), bf16(dh p silu(gate))
//   dprob[p]   = sum_n dh silu(gate) up                    FP32, one fixed order
//   dxp[r]     = bf16([dgate | dup] . W1[e])               grouped GEMM, K = 2I
//   dx[t]      = bf16(FP32 slot-order sum of dxp)          the forward's combine
//   dW2[e]     = sum over e's rows of dout[t]^T h[r]       FP32, K = e's rows
//   dW1[e]     = sum over e's rows of [dgate|dup]^T x[t]   FP32, K = e's rows
// with gate, up the forward's BF16 FC1 output y1 and h its BF16 FC2 input.
//
// One GEMM kernel serves the four products: a workgroup of 4 wavefronts owns
// an output tile -- 128 x 256 for dh and dxp (each wave all 128 rows x 64
// columns, 4 x 2 MFMA tiles, so each A fragment feeds two MFMAs and each B
// fragment four), 128 x 128 for the weight gradients (each wave 64 x 64) --
// of v_mfma_f32_32x32x16_bf16 with FP32 accumulation, and walks K in chunks
// of 64 through LDS, each operand staged as memory gives it (16-byte stores).  An
// operand whose memory rows run along k (the activations of dh and dxp) gives
// each MFMA fragment in one 16-byte LDS read; one whose rows run along the
// output index (the weights; both operands of the weight gradients, whose k
// is the expert's rows) is transposed by the fragment reads (the LDS
// transpose read ds_read_b64_tr_b16).  Rows are gathered through the forward's row -> pair map
// where the operand is a token's row (dout, x).  Every output element is one
// MFMA chain in increasing k: no split-K, so the results are deterministic,
// and each row of dh, dxp and dx depends only on its own inputs.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

typedef __bf16 bf16x8b __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBwdThreads = 256;
constexpr int kBwdTile = 128;   // output rows and columns per workgroup
constexpr int kBwdChunk = 64;   // k per LDS chunk (four MFMA k-steps)
constexpr int kKcPitch = kBwdChunk + 8;  // halves per LDS row of a KC operand, [index][k]
// An MC operand's LDS rows are padded by 32 halves: the 32 lanes of one
// transposing fragment read cover four rows of 64 bytes, which a row pitch of
// 64 mod 256 bytes puts on disjoint banks (with 8 halves of padding they
// overlap 2-4 ways).
constexpr int kMcPad = 32;
constexpr int kBwdOperandLds = kBwdTile * kKcPitch > kBwdChunk * (kBwdTile + kMcPad)
                                   ? kBwdTile * kKcPitch
                                   : kBwdChunk * (kBwdTile + kMcPad);  // a KC operand, or an MC operand 128 wide
constexpr int kBwdOperandLdsWide = kBwdChunk * (2 * kBwdTile + kMcPad);  // an MC operand 256 wide
constexpr int kBwdWaitLgkm0 = 0xC07F;  // s_waitcnt lgkmcnt(0)

// Token of a sorted row from its row2pair entry (padding rows, -1, read token
// 0 and are never stored or are zero-filled).
__device__ __forceinline__ int32_t bwd_token(int32_t p, int32_t K) {
    return p >= 0 ? (int32_t)((uint32_t)p / (uint32_t)K) : 0;
}

// One 64-deep chunk of an operand tile W wide, staged in LDS as memory gives
// it, 16 bytes per store.  KC (memory rows run along k): LDS [index][k], and
// an MFMA fragment (8 consecutive k of one index) is one 16-byte read.  MC
// (memory rows run along the index): LDS [k][index], and a fragment is two
// transposing 8-byte reads.  Row and column indices are 32-bit (sorted rows
// < 2^30); a piece's offset is one 32 x 32 -> 64-bit multiply-add.
template <bool KC, int W = kBwdTile>
struct BwdLoad {
    static constexpr int kMcPitch = W + kMcPad;  // halves per LDS row of an MC operand, [k][index]
    static constexpr int kBwdPieces = W * kBwdChunk / 8 / kBwdThreads;  // 16-byte pieces per thread
    static constexpr int kRowsPerWave = 512 / W;  // MC: k rows a wave's pieces share per h
    u32x4 v[kBwdPieces];
    // Memory rows of this thread's pieces: KC, the tile's index rows (the same
    // for every chunk, looked up once per tile); MC, the k rows of a chunk.
    int32_t mrow[kBwdPieces];
    int32_t praw;  // a gathered MC operand: row2pair entry of this lane's row of the next chunk
    // KC: the tile's rows, once per tile (gathered ones looked up per piece).
    __device__ __forceinline__ void kc_rows(bool gather, const int32_t* row2pair, int32_t K, int32_t idx0,
                                            int32_t idx_end) {
#pragma unroll
        for (int h = 0; h < kBwdPieces; h++) {
            const int piece = threadIdx.x + h * kBwdThreads;
            const int32_t i = idx0 + piece / (kBwdChunk / 8);  // 128 index rows x 8 pieces of 8 k
            const int32_t ii = i < idx_end ? i : idx0;
            mrow[h] = gather ? bwd_token(row2pair[ii], K) : ii;
        }
    }
    // MC: piece h of thread (wave w, lane l) is k row
    // k0 + R w + l / (W / 8) + (2048 / W) h with R = 512 / W, so a wave
    // touches 16 rows.  Rows past the end (or of an empty range) take an
    // in-bounds row; never used.
    __device__ __forceinline__ void mc_rows(int32_t k0, int32_t k_end) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int h = 0; h < kBwdPieces; h++) {
            const int32_t k = k0 + kRowsPerWave * wave + lane / (W / 8) + (2048 / W) * h;
            const int32_t kk = k < k_end ? k : k_end - 1;
            mrow[h] = kk > 0 ? kk : 0;
        }
    }
    // A gathered MC operand: lane s < 16 (and its copies s + 16 j) looks up
    // row k0 + R w + s % R + (2048 / W) (s / R) of chunk k0 a chunk ahead of
    // its use ...
    __device__ __forceinline__ void mc_prefetch(const int32_t* row2pair, int32_t k0, int32_t k_end) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, s = lane & 15;
        const int32_t k = k0 + kRowsPerWave * wave + s % kRowsPerWave + (2048 / W) * (s / kRowsPerWave);
        const int32_t kk = k < k_end ? k : k_end - 1;
        praw = row2pair[kk > 0 ? kk : 0];
    }
    // ... and piece h of lane l takes the token from lane l / (W / 8) + R h.
    __device__ __forceinline__ void mc_gathered_rows(int32_t K) {
        const int lane = threadIdx.x & 63;
        const int32_t t = bwd_token(praw, K);
#pragma unroll
        for (int h = 0; h < kBwdPieces; h++) mrow[h] = __shfl(t, lane / (W / 8) + kRowsPerWave * h, kWave);
    }
    __device__ __forceinline__ void fetch(const uint16_t* base, int64_t ld, int32_t idx0, int32_t idx_end,
                                          int32_t k0) {
#pragma unroll
        for (int h = 0; h < kBwdPieces; h++) {
            const int piece = threadIdx.x + h * kBwdThreads;
            int32_t col;
            if (KC) {
                col = k0 + 8 * (piece % (kBwdChunk / 8));
            } else {
                col = idx0 + 8 * (piece % (W / 8));
                col = col < idx_end ? col : idx_end - 8;  // columns past the end (a partial tile) re-read the last 8
            }
            const uint64_t off = (uint64_t)(uint32_t)mrow[h] * (uint32_t)ld + (uint32_t)col;
            v[h] = *reinterpret_cast<const u32x4*>(base + off);
        }
    }
    // Pieces of rows past the end are stored as zeros (mask: the chunk or tile
    // has such rows; a uniform test, so full chunks skip the selects).
    __device__ __forceinline__ static int lds_at(int piece) {
        return KC ? (piece / (kBwdChunk / 8)) * kKcPitch + 8 * (piece % (kBwdChunk / 8))
                  : (piece / (W / 8)) * kMcPitch + 8 * (piece % (W / 8));
    }
    __device__ __forceinline__ void store(uint16_t* lds, bool mask, int32_t idx0, int32_t idx_end, int32_t k0,
                                          int32_t k_end) const {
        if (__builtin_expect(mask, 0)) {
#pragma unroll
            for (int h = 0; h < kBwdPieces; h++) {
                const int piece = threadIdx.x + h * kBwdThreads;
                const bool live = KC ? idx0 + piece / (kBwdChunk / 8) < idx_end : k0 + piece / (W / 8) < k_end;
                *reinterpret_cast<u32x4*>(lds + lds_at(piece)) = live ? v[h] : u32x4{0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int h = 0; h < kBwdPieces; h++)
                *reinterpret_cast<u32x4*>(lds + lds_at(threadIdx.x + h * kBwdThreads)) = v[h];
        }
    }
    // MFMA fragment of the 32 indices [base, base + 32) at k = kb .. kb + 15:
    // lane (kh*32 + c) gets k = kb + 8 kh .. kb + 8 kh + 7 of index base + c.
    // MC uses the LDS transpose read ds_read_b64_tr_b16: within each group of
    // 16 lanes, source lane s reads 4 consecutive halves and output lane L
    // receives half L % 4 of source lanes L / 4, 4 + L / 4, 8 + L / 4 and
    // 12 + L / 4 (checked on the GPU by reading an index-filled array), so
    // source lane s reads row k0 + s / 4 at indices 4 (s % 4) .. + 3 of the
    // group's 16 and each output lane gets 4 consecutive k of one index; two
    // reads give the 8.
    __device__ __forceinline__ bf16x8b frag(uint16_t* lds, int base, int kb) const {
        const int lane = threadIdx.x & 63;
        if (KC)
            return __builtin_bit_cast(
                bf16x8b, *reinterpret_cast<const u32x4*>(lds + (base + (lane & 31)) * kKcPitch + kb + 8 * (lane >> 5)));
        const int g = lane >> 4, sl = lane & 15;
        const int row = kb + 8 * (g >> 1) + (sl >> 2), col = base + 16 * (g & 1) + 4 * (sl & 3);
        typedef short v4s __attribute__((ext_vector_type(4)));
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(lds + row * kMcPitch + col));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(lds + (row + 4) * kMcPitch + col));
        const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(bf16x8b, u32x4{a[0], a[1], b[0], b[1]});
    }
};

struct BwdGemmParams {
    const uint16_t* a;
    int64_t lda;
    bool a_gather;
    const uint16_t* b;
    int64_t ldb;
    int64_t b_estride;  // elements between experts' B matrices (weights), 0 for activations
    bool b_gather;
    const int32_t* row2pair;
    int32_t top_k;
    // cases by row tile (dh, dxp): tiles from the forward's row-tile table
    const int4* mtiles;
    const int32_t* n_mtiles;
    // cases by expert (weight gradients): K = the expert's rows
    const int32_t* expert_off;
    const int32_t* expert_count;
    int32_t M, N, Kd;
    int32_t n_tiles_n, n_tiles_m;
    int64_t n_tiles;  // cases by expert: E * n_tiles_m * n_tiles_n (by row tile: read on the device)
    void* out;
    int64_t ldc;
    int64_t c_estride;
};

// BY_EXPERT false: C[r][n] = sum_k A[r][k] B[k][n] over k < Kd for the rows r
// of a row tile (A KC, BF16 output, rows past the expert's end not stored).
// BY_EXPERT true: C_e[m][n] = sum over e's rows r of A[r][m] B[r][n] (A and B
// MC, FP32 output).
template <bool BY_EXPERT>
__global__ void __launch_bounds__(kBwdThreads, 2) bwd_gemm_kernel(BwdGemmParams P) {
    // (row-tile cases: 128 x 256 tiles, each wave all 128 rows x 64 columns;
    // weight gradients: 128 x 128 tiles, waves 2 x 2 of 64 x 64)
    constexpr int TN = BY_EXPERT ? kBwdTile : 2 * kBwdTile;
    constexpr int NI = BY_EXPERT ? 2 : 4;  // 32-row MFMA tiles per wave
    // the two operand buffers, and after the K loop the output staging
    constexpr int kSA = kBwdOperandLds, kSB = BY_EXPERT ? kBwdOperandLds : kBwdOperandLdsWide;
    __shared__ __attribute__((aligned(16))) uint16_t LDS[kSA + kSB];
    uint16_t* const SA = LDS;
    uint16_t* const SB = LDS + kSA;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = BY_EXPERT ? (wave & 1) : 0, wn = BY_EXPERT ? (wave >> 1) : wave;
    // Workgroup b runs on XCD b % 8 (round-robin dispatch), and XCD x takes
    // the contiguous range [x * span, (x + 1) * span) of the tile list, in
    // which tiles that share an expert's operands (its weights, or its rows of
    // the activations) are neighbours: they meet in that XCD's L2 instead of
    // being fetched by all eight.  The grid is a multiple of 8 covering
    // 8 * span workgroups.
    const int64_t total = BY_EXPERT ? P.n_tiles : (int64_t)(*P.n_mtiles) * P.n_tiles_n;
    const int64_t span = (total + 7) / 8, slot = blockIdx.x >> 3;
    if (slot >= span) return;
    const int64_t tile = (int64_t)(blockIdx.x & 7) * span + slot;
    if (tile >= total) return;
    int32_t m0, m_end, n0, k_begin, k_end, row_end = 0;
    int64_t expert;
    if (!BY_EXPERT) {
        const int64_t mt = tile / P.n_tiles_n;
        const int4 d = P.mtiles[mt];
        m0 = d.x;
        m_end = d.x + 32 * d.z;
        row_end = d.w;
        expert = d.y;
        n0 = (int32_t)(tile % P.n_tiles_n) * TN;
        k_begin = 0;
        k_end = P.Kd;
    } else {
        const int64_t per_e = (int64_t)P.n_tiles_m * P.n_tiles_n;
        expert = tile / per_e;
        const int32_t rem = (int32_t)(tile % per_e);
        m0 = (rem / P.n_tiles_n) * kBwdTile;
        m_end = P.M;
        n0 = (rem % P.n_tiles_n) * kBwdTile;
        k_begin = P.expert_off[expert];
        k_end = k_begin + P.expert_count[expert];
    }
    const uint16_t* bbase = P.b + expert * P.b_estride;
    BwdLoad<!BY_EXPERT> la;
    BwdLoad<false, TN> lb;
    // A: BY_EXPERT false, KC with memory rows m (sorted rows, or the tokens
    // of dout's rows, looked up once per tile); true, MC with memory rows k
    // (sorted rows, or their tokens).  B: MC with memory rows k -- an
    // expert's weight rows, or sorted rows.  A gathered MC operand's row2pair
    // entries are loaded a chunk ahead, so a chunk's data loads never wait
    // for its lookups.
    const bool ga = BY_EXPERT && P.a_gather, gb = P.b_gather;
    auto prefetch_rows = [&](int32_t k0) {
        if (ga) la.mc_prefetch(P.row2pair, k0, k_end);
        if (gb) lb.mc_prefetch(P.row2pair, k0, k_end);
    };
    auto fetch = [&](int32_t k0) {
        if (BY_EXPERT) {
            if (ga) la.mc_gathered_rows(P.top_k);
            else la.mc_rows(k0, k_end);
        }
        if (gb) lb.mc_gathered_rows(P.top_k);
        else lb.mc_rows(k0, k_end);
        la.fetch(P.a, P.lda, m0, m_end, k0);
        lb.fetch(bbase, P.ldb, n0, P.N, k0);
    };
    f32x16 acc[NI][2];
#pragma unroll
    for (int i = 0; i < NI; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = f32x16{};
    const int r = lane & 31, kh = lane >> 5;
    if (!BY_EXPERT) la.kc_rows(P.a_gather, P.row2pair, P.top_k, m0, m_end);
    const bool mask_rows = !BY_EXPERT && m_end - m0 < kBwdTile;  // a row tile of fewer than 128 rows
    if (k_begin < k_end) {
        prefetch_rows(k_begin);
        fetch(k_begin);
        if (k_begin + kBwdChunk < k_end) prefetch_rows(k_begin + kBwdChunk);
    }
    for (int32_t k0 = k_begin; k0 < k_end; k0 += kBwdChunk) {
        __syncthreads();  // the previous chunk's fragments are read
        const bool mask_k = k0 + kBwdChunk > k_end;  // the last, partial chunk
        la.store(SA, BY_EXPERT ? mask_k : mask_rows, m0, m_end, k0, k_end);
        lb.store(SB, mask_k, n0, P.N, k0, k_end);
        __syncthreads();
        if (k0 + kBwdChunk < k_end) {  // next chunk in flight during the MFMAs
            fetch(k0 + kBwdChunk);
            if (k0 + 2 * kBwdChunk < k_end) prefetch_rows(k0 + 2 * kBwdChunk);
        }
#pragma unroll
        for (int ks = 0; ks < kBwdChunk / 16; ks++) {
            bf16x8b af[NI], bfr[2];
#pragma unroll
            for (int i = 0; i < NI; i++) af[i] = la.frag(SA, 64 * wm + 32 * i, 16 * ks);
#pragma unroll
            for (int j = 0; j < 2; j++) bfr[j] = lb.frag(SB, 64 * wn + 32 * j, 16 * ks);
#pragma unroll
            for (int i = 0; i < NI; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
    // Epilogue.  Register q of MFMA tile (i, j) holds row 64 wm + 32 i +
    // (q/4)*8 + kh*4 + q%4 and column 64 wn + 32 j + r of the wave's part of
    // the tile.  The values pass through the wave's own slice of the operand
    // buffers, one 32-row MFMA tile at a time, so that every global store is
    // 16 bytes per lane over whole rows of 128 (BF16) or 256 (FP32) bytes:
    // a quarter to an eighth of the store instructions of per-element stores,
    // which compete with the operand loads for the CU's address unit.
    __syncthreads();  // every wave's last fragment reads are done
    if (!BY_EXPERT) {
        constexpr int kP = 64;  // halves per staged row
        uint16_t* const E = LDS + wave * (32 * kP);
#pragma unroll
        for (int i = 0; i < NI; i++) {
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int q = 0; q < 16; q++)
                    E[((q >> 2) * 8 + kh * 4 + (q & 3)) * kP + 32 * j + r] = (uint16_t)bf16_hw(acc[i][j][q]);
            __builtin_amdgcn_s_waitcnt(kBwdWaitLgkm0);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int u = 0; u < 4; u++) {  // 8 lanes per row of 64 columns
                const int rl = 8 * u + (lane >> 3), cl = 8 * (lane & 7);
                const u32x4 v = *reinterpret_cast<const u32x4*>(E + rl * kP + cl);
                const int64_t row = m0 + 32 * i + rl;
                const int64_t col = n0 + 64 * wn + cl;
                if (row < row_end && row < m_end && col < P.N)  // rows past the expert's end, a partial column tile
                    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(P.out) + row * P.ldc + col) = v;
            }
            __builtin_amdgcn_s_waitcnt(kBwdWaitLgkm0);  // the slice is read before the next tile overwrites it
            __builtin_amdgcn_wave_barrier();
        }
    } else {
        constexpr int kP = 72;  // floats per staged row: rows 4 apart on disjoint banks
        float* const E = reinterpret_cast<float*>(LDS) + wave * (32 * kP);
#pragma unroll
        for (int i = 0; i < NI; i++) {
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int q = 0; q < 16; q++) E[((q >> 2) * 8 + kh * 4 + (q & 3)) * kP + 32 * j + r] = acc[i][j][q];
            __builtin_amdgcn_s_waitcnt(kBwdWaitLgkm0);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int u = 0; u < 8; u++) {  // 16 lanes per row of 64 columns
                const int rl = 4 * u + (lane >> 4), cl = 4 * (lane & 15);
                const f32x4 v = *reinterpret_cast<const f32x4*>(E + rl * kP + cl);
                const int64_t row = m0 + 64 * wm + 32 * i + rl;
                const int64_t col = n0 + 64 * wn + cl;
                // the weight gradients (2.4 GB at the Qwen3 shape) are written
                // once and not read here: non-temporal stores
                if (row < m_end && col < P.N)
                    __builtin_nontemporal_store(
                        v, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(P.out) + expert * P.c_estride +
                                                    row * P.ldc + col));
            }
            __builtin_amdgcn_s_waitcnt(kBwdWaitLgkm0);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// SwiGLU backward per sorted row holding a pair (one wavefront per row):
// dgate = bf16(((dh p) up) silu'(gate)), dup = bf16((dh p) silu(gate)),
// dprob = FP32 sum of dh silu(gate) up, each lane over its columns in
// increasing order, then a fixed butterfly.  silu and silu' use the hardware
// exp2 and reciprocal: sig = 1 / (1 + e^-g), silu = g sig,
// silu' = sig (1 + g (1 - sig)).  Lane l takes the 8 columns 8 l + 512 j
// (16-byte loads and stores; I is a multiple of 128).
__global__ void __launch_bounds__(256) swiglu_backward_kernel(const uint16_t* __restrict__ dh,
                                                              const uint16_t* __restrict__ y1, int64_t rows,
                                                              int32_t I, const int32_t* __restrict__ row2pair,
                                                              const float* __restrict__ row_prob,
                                                              const int32_t* __restrict__ expert_off, int32_t E,
                                                              uint16_t* __restrict__ dy1, float* __restrict__ dprobs) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows || r >= expert_off[E]) return;
    const int32_t p = row2pair[r];
    if (p < 0) return;
    const float pr = row_prob[r];
    float dp = 0.0f;
    for (int n0 = 8 * lane; n0 < I; n0 += 8 * kWave) {
        const u32x4 dv = *reinterpret_cast<const u32x4*>(dh + r * I + n0);
        const u32x4 gv = *reinterpret_cast<const u32x4*>(y1 + r * 2 * I + n0);
        const u32x4 uv = *reinterpret_cast<const u32x4*>(y1 + r * 2 * I + I + n0);
        u32x4 dg, du;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int w = e >> 1, sh = 16 * (e & 1);
            const float d = bf16_to_f32((uint16_t)(dv[w] >> sh));
            const float g = bf16_to_f32((uint16_t)(gv[w] >> sh));
            const float u = bf16_to_f32((uint16_t)(uv[w] >> sh));
            const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
            const float sv = g * sig;
            const float ds = sig * (1.0f + g * (1.0f - sig));
            const float dpr = d * pr;
            const uint32_t a = bf16_hw(dpr * u * ds), b = bf16_hw(dpr * sv);
            if (e & 1) {
                dg[w] |= a << 16;
                du[w] |= b << 16;
            } else {
                dg[w] = a;
                du[w] = b;
            }
            dp = dp + d * sv * u;
        }
        *reinterpret_cast<u32x4*>(dy1 + r * 2 * I + n0) = dg;
        *reinterpret_cast<u32x4*>(dy1 + r * 2 * I + I + n0) = du;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dp += __shfl_xor(dp, o, kWave);
    if (lane == 0) dprobs[p] = dp;
}

hipError_t launch_bwd_gemm(bool by_expert, const BwdGemmParams& P, int64_t tiles, hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((tiles + 7) / 8 * 8);  // XCD ranges of ceil(tiles / 8)
    if (by_expert) {
        BwdGemmParams Q = P;
        Q.n_tiles = tiles;
        hipLaunchKernelGGL(bwd_gemm_kernel<true>, dim3(grid), dim3(kBwdThreads), 0, stream, Q);
    } else {
        hipLaunchKernelGGL(bwd_gemm_kernel<false>, dim3(grid), dim3(kBwdThreads), 0, stream, P);
    }
    return hipGetLastError();
}

hipError_t launch_moe_backward(const BwdArgs& A, hipStream_t stream) {
    const int64_t E = A.E, H = A.H, I = A.I;
    // dh = dout (gathered) . W2[e]: A KC (rows of dout, through row2pair), B MC (W2[e] rows: k = m).
    BwdGemmParams g{};
    g.row2pair = A.row2pair;
    g.top_k = A.top_k;
    g.mtiles = A.mtiles;
    g.n_mtiles = A.n_mtiles;
    g.expert_off = A.expert_off;
    g.expert_count = A.expert_count;
    g.a = A.dout;
    g.lda = H;
    g.a_gather = true;
    g.b = A.w2;
    g.ldb = I;
    g.b_estride = H * I;
    g.b_gather = false;
    g.N = (int32_t)I;
    g.Kd = (int32_t)H;
    g.n_tiles_n = (int32_t)((I + 2 * kBwdTile - 1) / (2 * kBwdTile));
    g.out = A.dh;
    g.ldc = I;
    hipError_t e = launch_bwd_gemm(false, g, A.mt_bound * g.n_tiles_n, stream);
    if (e != hipSuccess) return e;
    // the SwiGLU backward and the router-probability gradient
    hipLaunchKernelGGL(swiglu_backward_kernel, dim3((unsigned)((A.rows_bound + 3) / 4)), dim3(256), 0, stream, A.dh,
                       A.y1, A.rows_bound, (int32_t)I, A.row2pair, A.row_prob, A.expert_off, (int32_t)E, A.dy1,
                       A.dprobs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dxp = dy1 . W1[e]: A KC (dy1 rows), B MC (W1[e] rows: k = j)
    BwdGemmParams x1 = g;
    x1.a = A.dy1;
    x1.lda = 2 * I;
    x1.a_gather = false;
    x1.b = A.w1;
    x1.ldb = H;
    x1.b_estride = 2 * I * H;
    x1.N = (int32_t)H;
    x1.Kd = (int32_t)(2 * I);
    x1.n_tiles_n = (int32_t)((H + 2 * kBwdTile - 1) / (2 * kBwdTile));
    x1.out = A.dxp;
    x1.ldc = H;
    e = launch_bwd_gemm(false, x1, A.mt_bound * x1.n_tiles_n, stream);
    if (e != hipSuccess) return e;
    // dx = FP32 slot-order sum of each token's dxp rows (the forward's
    // combine), while dxp is still in the last-level cache (the weight
    // gradients' 2.4 GB of writes would evict it)
    e = launch_combine(A.dxp, A.pair2row, A.T, (int32_t)H, A.top_k, A.dx, stream);
    if (e != hipSuccess) return e;
    // dW2[e] = dout(rows of e)^T h(rows of e): A MC (dout rows, gathered), B MC (h rows)
    BwdGemmParams w2 = g;
    w2.a = A.dout;
    w2.lda = H;
    w2.a_gather = true;
    w2.b = A.h;
    w2.ldb = I;
    w2.b_estride = 0;
    w2.b_gather = false;
    w2.M = (int32_t)H;
    w2.N = (int32_t)I;
    w2.n_tiles_m = (int32_t)(H / kBwdTile);
    w2.n_tiles_n = (int32_t)(I / kBwdTile);
    w2.out = A.dw2;
    w2.ldc = I;
    w2.c_estride = H * I;
    e = launch_bwd_gemm(true, w2, E * w2.n_tiles_m * w2.n_tiles_n, stream);
    if (e != hipSuccess) return e;
    // dW1[e] = dy1(rows of e)^T x(rows of e): A MC (dy1 rows), B MC (x rows, gathered)
    BwdGemmParams w1 = g;
    w1.a = A.dy1;
    w1.lda = 2 * I;
    w1.a_gather = false;
    w1.b = A.x;
    w1.ldb = H;
    w1.b_estride = 0;
    w1.b_gather = true;
    w1.M = (int32_t)(2 * I);
    w1.N = (int32_t)H;
    w1.n_tiles_m = (int32_t)(2 * I / kBwdTile);
    w1.n_tiles_n = (int32_t)(H / kBwdTile);
    w1.out = A.dw1;
    w1.ldc = H;
    w1.c_estride = 2 * I * H;
    e = launch_bwd_gemm(true, w1, E * w1.n_tiles_m * w1.n_tiles_n, stream);
    return e;
}

}  // namespace nvfp4
