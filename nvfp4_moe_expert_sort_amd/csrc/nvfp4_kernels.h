// nvfp4_kernels.h -- internal launchers of the gfx950 kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kMAlign = 32;      // each expert's rows are padded to a multiple of this (one MFMA row tile)
constexpr int kTileRows = 128;   // rows per GEMM wave tile (4 MFMA row tiles)
constexpr int kTokPerBlk = 16;   // tokens per block in the sort kernels
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kGemmPlain = 0;   // y = bf16(acc * g_a * g_b)
constexpr int kGemmSwiGLU = 1;  // FC1 + router-weighted SwiGLU producer (h and per-tile |h| maxima)

struct GemmParams {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const float* a_g;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const float* b_g;
    int32_t K;          // reduction length, multiple of 128
    int32_t N;          // rows of one expert's weight matrix
    int32_t n_tiles_n;  // column tiles per row tile
    const int4* mtiles;        // row tiles {row0, expert, 32-row subtiles, end of valid rows}
    const int32_t* n_mtiles;   // device count of row tiles
    int32_t dense_m;           // >= 0: one matrix with this many rows; row tiles implied
    int32_t persist;           // > 0 (a multiple of 8): hybrid grid, see gemm_kernel
    uint16_t* out;
    int64_t ld_out;
    const float* row_prob;     // SwiGLU mode: router probability per row
    float* amax_part;          // SwiGLU mode: [rows][n_part] max |h| of each 32-column group
    int32_t n_part;            // SwiGLU mode: I / 32
    int32_t inter;             // SwiGLU mode: I (gate rows [0, I), up rows [I, 2I))
    // Activations quantized inside the GEMM (gemm_kernel<kGemmSwiGLU, true>):
    // row r's A operand is its token's BF16 row a_bf16[row2pair[r] / top_k]
    // (K wide), quantized with the outer scale of a_amax[token] (max |x|);
    // a_g[r] holds that row's g.
    const uint16_t* a_bf16;
    const float* a_amax;
    const int32_t* a_row2pair;
    int32_t a_top_k;
    int32_t a_round_up;
};

struct RouteBuffers {
    int32_t* blk_counts;   // [nblk][E]; exclusive per-expert prefix after the scan
    int32_t* blk_err;      // [nblk]
    int32_t* expert_count; // [E]
    int32_t* expert_off;   // [E+1]
    int4* mtiles;          // [mtiles_cap] 4-subtile row tiles, an expert's remainder last (FC2)
    int4* mtiles_even;     // [mtiles_cap] the same tiles with each expert's subtiles spread evenly (FC1)
    int32_t* n_mtiles;     // [1]
    int32_t* err_word;     // [1]
    int32_t* pair2row;     // [T*K]
    int32_t* row2pair;     // [rows_cap]
    float* row_prob;       // [rows_cap]
    uint8_t* xq_codes;     // [T][H/2] token-major quantized X (logical layout)
    uint8_t* xq_scales;    // [T][H/16]
    float* gx;             // [T]
    uint8_t* a_codes;      // sorted, padded A1 (GEMM layout)
    uint8_t* a_scales;
    float* a_g;
};

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                             uint8_t* scales, float* g, bool gemm, bool round_up, hipStream_t stream);
hipError_t launch_quant_h(const uint16_t* h, int64_t rows_bound, int64_t I, const int32_t* expert_off, int32_t E,
                          int32_t capacity, const int32_t* expert_count, const int32_t* row2pair,
                          const float* amax2_part, int n_part, uint8_t* codes, uint8_t* scales, float* g,
                          bool round_up, hipStream_t stream);
// capacity 0: contiguous row layout; > 0: masked layout, expert e's rows in
// the chunk [e * capacity, (e + 1) * capacity) (capacity % kMAlign == 0).
// quant_x false: X is not quantized and no sorted A1 is built (the W4A16
// variant reads the BF16 rows of x itself).
hipError_t launch_route(const uint16_t* x, const int32_t* ids, const float* probs, int32_t T, int32_t H, int32_t K,
                        int32_t E, int32_t capacity, bool round_up, const RouteBuffers& rb, int64_t rows_cap,
                        hipStream_t stream, bool quant_x = true, bool online = false);

// W4A16 grouped GEMM (NVFP4 weights, BF16 activations): one workgroup per
// (32-row subtile of a row tile, column tile).
struct W16Params {
    const uint16_t* a;         // BF16 activation rows, K columns each
    const int32_t* row2pair;   // non-null: sorted row r reads row row2pair[r] / top_k of `a` (FC1)
    int32_t top_k;
    const uint8_t* b_codes;    // weights, GEMM layout, [E][N][K]
    const uint8_t* b_scales;
    const float* b_g;
    int32_t K, N;
    int32_t n_tiles_n;         // column tiles (FC1: 128 columns of h; FC2: 256 output columns)
    const int4* mtiles;
    const int32_t* n_mtiles;
    uint16_t* out;
    int64_t ld_out;
    const float* row_prob;     // SwiGLU mode: router probability per sorted row
    int32_t inter;             // SwiGLU mode: I
};
hipError_t launch_gemm_w4a16(int mode, const W16Params& P, int64_t mt_bound, hipStream_t stream);

// Router scores logits [T, E] (FP32) and the top-K ids / probabilities per token.
hipError_t launch_router(const uint16_t* x, int32_t T, int32_t H, const uint16_t* w, int32_t E, int32_t K,
                         bool renorm, float* logits, int32_t* ids, float* probs, hipStream_t stream);

#ifdef __HIPCC__
// Whether the 32-row tile rt of the sorted buffers holds rows of an expert:
// below off[E] in the contiguous layout (capacity 0); inside its expert's
// padded rows in the masked layout (a chunk holds whole tiles, capacity being
// a multiple of kMAlign).  Row tiles that hold none are never written.
__device__ __forceinline__ bool row_tile_used(int64_t rt, int32_t E, int32_t capacity,
                                              const int32_t* __restrict__ expert_off,
                                              const int32_t* __restrict__ expert_count) {
    const int64_t r = rt * kMAlign;
    if (capacity <= 0) return r < expert_off[E];
    const int64_t e = r / capacity;
    if (e >= E) return false;
    const int64_t kept = min(expert_count[e], capacity);
    return r - e * capacity < (kept + kMAlign - 1) / kMAlign * kMAlign;
}
#endif
// The BF16 straight-through backward (backward.hip): buffers from the
// forward (sort metadata, row probabilities, h, y1) and its own.
struct BwdArgs {
    int32_t T, top_k;
    int64_t E, H, I;
    const uint16_t* x;       // [T, H]
    const uint16_t* w1;      // [E, 2I, H] BF16
    const uint16_t* w2;      // [E, H, I] BF16
    const uint16_t* y1;      // [rows, 2I] the forward's FC1 output per sorted row
    const uint16_t* h;       // [rows, I] the forward's FC2 input per sorted row
    const uint16_t* dout;    // [T, H]
    const int32_t* row2pair;
    const int32_t* pair2row;
    const float* row_prob;
    const int4* mtiles;
    const int32_t* n_mtiles;
    const int32_t* expert_off;
    const int32_t* expert_count;
    int64_t mt_bound, rows_bound;
    uint16_t* dh;            // [rows, I]
    uint16_t* dy1;           // [rows, 2I]
    uint16_t* dxp;           // [rows, H]
    uint16_t* dx;            // [T, H]
    float* dprobs;           // [T, K]
    float* dw1;              // [E, 2I, H]
    float* dw2;              // [E, H, I]
};
hipError_t launch_moe_backward(const BwdArgs& args, hipStream_t stream);

int gemm_cols_per_tile(int mode);  // output columns per tile: 256 (plain) or 128 of h (128 gate + 128 up rows)
hipError_t launch_gemm(int mode, const GemmParams& P, int grid_blocks, hipStream_t stream, bool aq = false);
// The router-weighted SwiGLU producer on its own (unfused forward): h and the
// per-32-column maxima of |h| from y1 [rows, 2I] (gate | up), for sorted rows
// below min(rows_bound, expert_off[E]) that hold a pair.
hipError_t launch_swiglu_producer(const uint16_t* y1, int64_t rows_bound, int32_t I, const int32_t* row2pair,
                                  const float* row_prob, const int32_t* expert_off, int32_t E, uint16_t* h,
                                  float* amax_part, hipStream_t stream);
hipError_t launch_combine(const uint16_t* y2, const int32_t* pair2row, int32_t T, int32_t H, int32_t K,
                          uint16_t* out, hipStream_t stream);

}  // namespace nvfp4
