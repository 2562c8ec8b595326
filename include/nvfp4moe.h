/*
 * nvfp4moe.h -- C ABI of the MI355X (gfx950) NVFP4 MoE expert forward.
 *
 * The operation (sources: the miniTE summary page, "miniTE diagnoses and
 * narrows the cross-engine execution gap of NVFP4 RL", sections "how it
 * differs" and "how to use it"; the article "Finish RL training faster:
 * bitwise consistent, high-performance, agent-driven", sections 4.4-4.6):
 *
 *   sort tokens by expert (device offsets mark each expert's rows) and take
 *   the row amax in the same pass over X; pad each expert's rows; quantize
 *   every row to NVFP4 -- E2M1 codes, one E4M3 scale per 16 elements, one
 *   FP32 outer scale per row g = max|row| / (6*448), no Hadamard transform,
 *   no stochastic rounding; grouped GEMM FC1 whose FP32 epilogue multiplies
 *   by g^x * g^w and casts to BF16; h = SiLU(gate) * up * p (router
 *   probability) in FP32 rounded once to BF16, and that producer also emits
 *   the FC2 amax; quantize h; grouped GEMM FC2 with the same epilogue; sum
 *   each token's K expert outputs in FP32 in top-k slot order, round to BF16.
 *
 * Every token's output is bitwise identical whatever else is in the batch:
 * quantization is per row, each output row is accumulated in one fixed order
 * with one instruction sequence for every batch size (no split-K, no
 * configuration chosen by the token count), and the combine order is fixed.
 *
 * Conventions
 *   - All pointers are DEVICE pointers unless marked (host).  BF16 tensors
 *     are passed as uint16_t bit patterns, row-major.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; nothing here synchronises except the calls marked "syncs".
 *   - The library never allocates on the forward path: every buffer is the
 *     caller's.  It keeps no mutable global state, so calls on different
 *     streams with different workspaces are independent.
 *   - Errors found on the host return before anything is launched.  No
 *     exception crosses the ABI and nothing is printed.
 *   - NaN or Inf inputs are outside the contract (results undefined).
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define NVFP4MOE_API __attribute__((visibility("default")))
#else
#define NVFP4MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
    NVFP4_OK = 0,
    NVFP4_E_NULL = 1,      /* a required pointer is NULL */
    NVFP4_E_SHAPE = 2,     /* a size is negative, too large, or not a multiple the layout needs */
    NVFP4_E_ALIGN = 3,     /* a pointer is not aligned as documented */
    NVFP4_E_WORKSPACE = 4, /* workspace_bytes smaller than the size function returned */
    NVFP4_E_CAPACITY = 5,  /* T > cfg->max_tokens */
    NVFP4_E_HIP = 6,       /* a HIP launch or runtime call failed */
    NVFP4_E_MISMATCH = 7,  /* self-test found differing bits */
    NVFP4_E_DEVICE = 8,    /* the device reported a contract violation (see nvfp4moe_device_error) */
    NVFP4_E_ARG = 9,       /* an enum argument is out of range */
    NVFP4_E_SCRATCH = 10   /* the allocation-free forward's input exceeds its static scratch */
};

/* Rounding of the E4M3 block scale v = amax_block / (6 g).  The pages fix the
 * formats but not this rounding.  ROUND_UP (default) is the smallest E4M3
 * value >= v, so scale * 6 * g always covers the block maximum; RNE rounds to
 * the nearest E4M3 value (ties to an even mantissa).  Both clamp at 448. */
enum { NVFP4_SCALE_RU = 0, NVFP4_SCALE_RNE = 1 };

/* Layout of a quantized [rows, cols] matrix (three planes: codes, scales, g).
 *
 * LOGICAL: codes [rows][cols/2] bytes, element 2i in the low nibble of byte i;
 *          scales [rows][cols/16] E4M3FN bytes; g [rows] FP32.
 * GEMM:    the layout the grouped GEMM reads directly (rows % 32 == 0,
 *          cols % 128 == 0).  Rows are grouped in tiles of 32, columns in
 *          chunks of 64.  For row r (tile rt = r/32, rl = r%32) and column k
 *          (chunk c = k/64, half h = (k%64)/32):
 *            code byte  = (rt*(cols/64) + c)*1024 + (h*32 + rl)*16 + (k%32)/2,
 *                         element k in the low nibble when k is even;
 *            scale byte = (rt*(cols/128) + c/2)*256 + (h*32 + rl)*4
 *                         + (c%2)*2 + (k%32)/16;
 *            g[r] as in LOGICAL.
 *          One 64-lane load of 16 bytes per lane then fetches one contiguous
 *          1 KiB: 32 rows x 64 columns, lane (h*32 + rl) holding row rl,
 *          columns [64c + 32h, 64c + 32h + 32). */
enum { NVFP4_LAYOUT_LOGICAL = 0, NVFP4_LAYOUT_GEMM = 1 };

/* Layer configuration (host struct). */
typedef struct {
    int32_t hidden;      /* H: multiple of 128 */
    int32_t inter;       /* I: expert intermediate size, multiple of 128 */
    int32_t n_experts;   /* E: 1..1024 */
    int32_t top_k;       /* K: 1..n_experts (and <= 32) */
    int32_t max_tokens;  /* bound on T; sizes the workspace (static capacity) */
    int32_t scale_round; /* NVFP4_SCALE_RU or NVFP4_SCALE_RNE */
} nvfp4moe_config;

/* A quantized tensor of n_mats matrices [rows, cols] (host struct, device
 * pointers).  Plane sizes: codes n_mats*rows*cols/2 bytes, scales
 * n_mats*rows*cols/16 bytes, g n_mats*rows floats.  Matrices are stacked
 * along rows, so matrix e's row n is row e*rows + n of the planes. */
typedef struct {
    uint8_t* codes;
    uint8_t* scales;
    float* g;
    int32_t n_mats;
    int32_t rows;
    int32_t cols;
    int32_t layout; /* NVFP4_LAYOUT_* */
} nvfp4_qtensor;

/* Human-readable name of a status code (static string). */
NVFP4MOE_API const char* nvfp4_status_str(int status);

/* Quantize each row of x [rows, cols] (row stride ld elements) into NVFP4
 * (miniTE page, "how it differs": per-row outer scale g = max|row|/(6*448),
 * 16-element E4M3 block scales, E2M1 codes, round to nearest even, no
 * stochastic rounding).  Numeric contract, in binary32 with IEEE division:
 *   g = amax/2688; d = 6*g; per block v = amax_b/d, s = E4M3(v) per
 *   scale_round (0 if amax_b == 0); per element q = |x|/(s*g) and the code is
 *   the nearest E2M1 value, ties to even, saturating at 6, carrying the input
 *   sign bit; if s*g == 0 the code keeps only the sign.  A zero row gets
 *   g = 0 and all scales 0.
 * Requirements: cols % 16 == 0 (LOGICAL) or rows % 32 == 0 and
 * cols % 128 == 0 (GEMM); ld >= cols; x 16-byte aligned and ld % 8 == 0;
 * codes 16-byte, scales 2-byte and g 4-byte aligned.
 * Output planes as described for the layout. */
NVFP4MOE_API int nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                   float* g, int32_t layout, int32_t scale_round, void* stream);

/* Bytes of one quantized expert-weight tensor: which = 1 for W1 [E, 2I, H]
 * (rows 0..I-1 of each expert are the gate projection, I..2I-1 the up
 * projection), which = 2 for W2 [E, H, I].  Sum of the three planes (E2M1
 * codes, one E4M3 scale per 16 elements, one FP32 outer scale per row: the
 * weight format of the miniTE page, "how it differs"), each rounded up to
 * 256 bytes.  The caller allocates them once and the weights are re-quantized
 * into the same buffers on every update (article, section 4.6: weights
 * updated in place, addresses kept).  Returns 0 for an invalid config. */
NVFP4MOE_API size_t nvfp4moe_weight_bytes(const nvfp4moe_config* cfg, int32_t which);

/* Quantize BF16 expert weights (w1 [E, 2I, H], w2 [E, H, I]) in place into
 * caller-owned GEMM-layout tensors (W1q: n_mats E, rows 2I, cols H; W2q:
 * n_mats E, rows H, cols I).  Used once per weight update; writing into the
 * same buffers keeps their addresses (article, section 4.6). */
NVFP4MOE_API int nvfp4moe_quantize_weights(const nvfp4moe_config* cfg, const uint16_t* w1, const uint16_t* w2,
                              const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q, void* stream);

/* Workspace bytes for the forward; depends on cfg only (max_tokens bounds T),
 * so one allocation serves every batch size (article, section 4.6: buffers of
 * static capacity sized once, no read-back of per-expert counts to size them;
 * miniTE page, "how to use it": the quantizer writes and the GEMM reads one
 * contiguous buffer).  It holds the sort metadata, the quantized sorted
 * activations, h, the quantized h and the expert outputs
 * (nvfp4moe_workspace_layout).  Returns 0 for an invalid cfg. */
NVFP4MOE_API size_t nvfp4moe_workspace_bytes(const nvfp4moe_config* cfg);

/* The NVFP4 MoE expert forward for T tokens.
 *   x      [T, H] BF16 activations (16-byte aligned)
 *   ids    [T, K] int32 expert ids, each in [0, E), distinct within a token
 *   probs  [T, K] float32 router probabilities (applied to the SwiGLU output)
 *   W1q, W2q quantized weights in GEMM layout (nvfp4moe_quantize_weights)
 *   out    [T, H] BF16; out[t] = bf16(FP32 sum over k = 0..K-1, in the order
 *          the columns of ids list them, of expert ids[t,k]'s FC2 output)
 * T == 0 is a no-op.  An expert with no tokens reads none of its weights.
 * No host synchronisation; the launch grids depend on cfg and T only.
 * Out-of-range or repeated ids do not fault: they set the device error word
 * (nvfp4moe_device_error); the outputs are then unspecified. */
NVFP4MOE_API int nvfp4moe_moe_expert_forward(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T, const int32_t* ids,
                                const float* probs, const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q,
                                uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* The same forward with FC1 and the SwiGLU producer unfused, as a reference
 * for the fused path (miniTE page, "assumptions and limits": the fused
 * kernels are checked bit for bit against the unfused quantization and
 * grouped-GEMM steps).  FC1 runs as a plain grouped GEMM whose epilogue
 * writes y1 = bf16(acc * g^x * g^w1) for all 2I weight rows, then a separate
 * kernel forms h = bf16(silu(gate) * up * p) and its per-32-column maxima
 * from y1; every later step is the fused forward's.  Each value it writes
 * (h, the maxima, A2, y2, out) has the fused forward's bits.
 *   y1       [y1_rows, 2I] BF16, caller-owned (16-byte aligned); sorted row r
 *            holds y1 of the pair in row r (columns 0..I-1 gate, I..2I-1 up);
 *            padding rows are not written
 *   y1_rows  >= rows_cap of nvfp4moe_workspace_layout (else NVFP4_E_SHAPE)
 * Every other argument, the workspace and the errors are those of
 * nvfp4moe_moe_expert_forward.  Slower than the fused forward (y1 makes a
 * round trip through memory); meant for checking and inspection. */
NVFP4MOE_API int nvfp4moe_moe_expert_forward_unfused(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T,
                                                     const int32_t* ids, const float* probs, const nvfp4_qtensor* W1q,
                                                     const nvfp4_qtensor* W2q, uint16_t* out, uint16_t* y1,
                                                     int64_t y1_rows, void* workspace, size_t workspace_bytes,
                                                     void* stream);

/* The BF16 straight-through backward of the expert forward (miniTE page,
 * "how it differs": the backward takes quantization as the identity and runs
 * BF16 GEMMs on the stored original BF16 activations and weights, avoiding
 * any quantization on the way back).  It follows a call of
 * nvfp4moe_moe_expert_forward_unfused on the same cfg, x and T, whose
 * workspace (sort metadata, row probabilities, h) and y1 it reads.  With
 * p = t*K + k, e = ids[t,k], gate/up = y1 of pair p and h its FC2 input:
 *   dh[p]     = bf16(dout[t] . W2[e])             FP32 accumulation
 *   dgate[p]  = bf16(dh prob up silu'(gate)),  dup[p] = bf16(dh prob silu(gate))
 *   dprobs[t,k] = sum_n dh silu(gate) up         FP32
 *   dx[t]     = bf16(FP32 sum over k = 0..K-1, in slot order, of
 *               bf16([dgate | dup] . W1[e]))
 *   dw1[e]    = sum over e's pairs of [dgate | dup]^T x[t]      FP32 [2I, H]
 *   dw2[e]    = sum over e's pairs of dout[t]^T h[p]            FP32 [H, I]
 * (the combine passes dout[t] to every slot).  Every sum is one fixed order
 * (deterministic); dx[t] depends only on token t's inputs.
 *   x, dout   [T, H] BF16; w1 [E, 2I, H] and w2 [E, H, I] the BF16 weights
 *             the quantized ones were made from (16-byte aligned)
 *   y1        the forward's y1 buffer, y1_rows >= rows_cap
 *   fwd_workspace   the forward's workspace (read only)
 *   dx [T, H] BF16, dprobs [T, K] FP32, dw1, dw2 FP32: caller-owned outputs
 *             (dw1, dw2 overwritten, experts without tokens get zeros)
 *   workspace nvfp4moe_backward_workspace_bytes(cfg) bytes (dh, dgate|dup
 *             and each pair's FC1 input gradient), 256-byte aligned
 * Contiguous row layout only; errors as for the forward; no synchronisation. */
NVFP4MOE_API size_t nvfp4moe_backward_workspace_bytes(const nvfp4moe_config* cfg);
NVFP4MOE_API int nvfp4moe_moe_expert_backward(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T,
                                              const uint16_t* w1, const uint16_t* w2, const uint16_t* y1,
                                              int64_t y1_rows, const void* fwd_workspace, size_t fwd_workspace_bytes,
                                              const uint16_t* dout, uint16_t* dx, float* dprobs, float* dw1,
                                              float* dw2, void* workspace, size_t workspace_bytes, void* stream);

/* The W4A16 variant of the expert forward (the article, section 6: NVFP4
 * W4A16 routed experts): the same sort, SwiGLU producer, combine, arguments,
 * workspace and errors as nvfp4moe_moe_expert_forward, with the activations
 * left in BF16 instead of quantized (x into FC1, h into FC2; cfg->scale_round
 * is unused), so each epilogue multiplies by g^w only:
 *   y1 = bf16((x . W1q[e]^T) g^w1), h = bf16(silu(gate) * up * p),
 *   y2 = bf16((h . W2q[e]^T) g^w2), out[t] = bf16(FP32 slot-order sum of y2).
 * Per-token results are bitwise independent of the batch, as for the W4A4
 * forward.  The workspace's quantized-activation buffers are not written. */
NVFP4MOE_API int nvfp4moe_moe_expert_forward_w4a16(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T,
                                                   const int32_t* ids, const float* probs, const nvfp4_qtensor* W1q,
                                                   const nvfp4_qtensor* W2q, uint16_t* out, void* workspace,
                                                   size_t workspace_bytes, void* stream);

/* The expert forward with the activations' max, quantization and FC1 GEMM
 * fused (miniTE summary page, "assumptions and limits": the online
 * amax-quantization-GEMM fusion, whose numerical and performance validation
 * the page leaves open).  The sort records each token's max |x| instead of a
 * quantized copy of X (no gather); FC1 loads each sorted row's BF16 token
 * row and quantizes it as it goes, 32 elements per lane, with the outer scale
 * g = max|x| / 2688, the E4M3 block scales (cfg->scale_round) and the E2M1
 * codes of nvfp4moe_moe_expert_forward's quantizer, so every output is
 * bitwise that entry point's.  g is known before the GEMM starts (the sort
 * takes the max over the whole row), so no accumulator is ever rescaled.
 * Same arguments, workspace and errors as nvfp4moe_moe_expert_forward;
 * contiguous row layout only; no synchronisation. */
NVFP4MOE_API int nvfp4moe_moe_expert_forward_online(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T,
                                                    const int32_t* ids, const float* probs, const nvfp4_qtensor* W1q,
                                                    const nvfp4_qtensor* W2q, uint16_t* out, void* workspace,
                                                    size_t workspace_bytes, void* stream);

/* The same forward, recording caller-created hipEvent_t events[i] on `stream`
 * at each stage boundary, for timing the stages inside a timed region
 * (events[0] before the sort, [1] after the sort and the quantization of X,
 * [2] after the FC1 GEMM with its SwiGLU producer, [3] after the quantization
 * of h, [4] after the FC2 GEMM, [5] after the combine).  events (host array)
 * must hold NVFP4MOE_N_STAGE_EVENTS non-null events.  No synchronisation. */
#define NVFP4MOE_N_STAGE_EVENTS 6
NVFP4MOE_API int nvfp4moe_moe_expert_forward_events(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T,
                                                    const int32_t* ids, const float* probs, const nvfp4_qtensor* W1q,
                                                    const nvfp4_qtensor* W2q, uint16_t* out, void* workspace,
                                                    size_t workspace_bytes, void* const* events, void* stream);

/* Device error word of the last forward that used `workspace`: 0 if clean,
 * else a bitwise OR of 1 (an id outside [0, E)), 2 (an id repeated within a
 * token) and 4 (masked layout only: an expert received more pairs than its
 * capacity).  The routing (ids and probabilities) is an input decided
 * upstream (article, section 4.4: the router's top-k is fixed before the
 * expert path); the forward checks it on the device without a host read-back
 * (section 4.6) and reports violations here instead of faulting.
 * Syncs `stream`.  *code_host (host) receives the word. */
NVFP4MOE_API int nvfp4moe_device_error(const nvfp4moe_config* cfg, const void* workspace, int32_t* code_host, void* stream);

/* The forward with no workspace argument and no allocation, for callers that
 * cannot allocate device memory on the way: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Its intermediates
 * live in one static device array of NVFP4MOE_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the library's load until the process ends; its address is
 * looked up once per device on the first call there.  Arguments and results
 * are those of nvfp4moe_moe_expert_forward (same kernels, same bits), and:
 *   err_word  optional (may be NULL) device int32: receives the call's
 *             device error word (see nvfp4moe_device_error) by a 4-byte
 *             device-to-device copy at the end of the call
 * The intermediates need size nvfp4moe_workspace_bytes of cfg with
 * max_tokens = T; a call whose T needs more than the scratch returns
 * NVFP4_E_SCRATCH before any launch (at the Qwen3-30B-A3B layer shape,
 * H 2048, I 768, E 128, K 8, that is T above about 600 tokens).  T above
 * cfg->max_tokens returns NVFP4_E_CAPACITY.  Nothing in the scratch needs
 * clearing between calls: every call writes what it reads.  All calls on one
 * GPU share its scratch: calls that overlap in time on one GPU (different
 * streams, or host threads) race and their results are undefined; serialise
 * them (one stream, or events). */
#define NVFP4MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
NVFP4MOE_API int nvfp4moe_moe_expert_forward_noalloc(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T,
                                                     const int32_t* ids, const float* probs, const nvfp4_qtensor* W1q,
                                                     const nvfp4_qtensor* W2q, uint16_t* out, int32_t* err_word,
                                                     void* stream);

/* Byte offsets of the forward's intermediates inside the workspace, for
 * inspection (host struct).  Row-indexed buffers are indexed by sorted row r
 * in [0, off[E]); pair p = t*K + k. */
typedef struct {
    size_t err;          /* int32 error word */
    size_t expert_count; /* int32 [E] tokens routed to each expert */
    size_t expert_off;   /* int32 [E+1] padded row offsets (device offsets of expert boundaries) */
    size_t pair2row;     /* int32 [T*K] sorted row of each pair */
    size_t row2pair;     /* int32 [rows_cap] pair of each sorted row, -1 for padding */
    size_t a1_codes, a1_scales, a1_g;  /* quantized sorted X, GEMM layout, rows_cap rows x H */
    size_t h;            /* BF16 [rows_cap, I] router-weighted SwiGLU output */
    size_t amax2_part;   /* float [rows_cap, n_part] max |h| of each 32-column group of h, per row */
    size_t a2_codes, a2_scales, a2_g;  /* quantized h, GEMM layout, rows_cap rows x I */
    size_t y2;           /* BF16 [rows_cap, H] FC2 output per sorted row */
    int64_t rows_cap;    /* max_tokens*K + E*(m_align-1), rounded up to m_align (masked layout: E*capacity) */
    int32_t m_align;     /* each expert's rows are padded to a multiple of this */
    int32_t n_part;      /* I / 32: entries of amax2_part per row */
} nvfp4moe_ws_layout;

NVFP4MOE_API int nvfp4moe_workspace_layout(const nvfp4moe_config* cfg, nvfp4moe_ws_layout* layout_host);

/* The masked fixed-capacity row layout (article, section 4.4, "two layouts,
 * same row results": the decode side feeds the expert GEMMs per-expert chunks
 * of a fixed capacity, the training side packed contiguous rows, and the
 * same (token, slot) must get the same bits in both).  Expert e owns sorted
 * rows [e*capacity, (e+1)*capacity): its pairs take rows e*capacity + i in
 * the contiguous layout's order (i = the pair's rank within the expert), the
 * rows up to the next multiple of m_align are padding, and the rest of the
 * chunk is never read or written.  Every other rule of
 * nvfp4moe_moe_expert_forward holds, and each pair's quantized rows, h, y2
 * and each token's output are bitwise those of the contiguous layout.
 *   capacity  rows per expert chunk: a positive multiple of m_align (32) with
 *             E*capacity < 2^30, chosen by the caller independently of T
 * A pair ranked >= capacity within its expert gets no row (pair2row -1, its
 * term left out of its token's sum) and sets bit 4 of the device error word;
 * the outputs of the tokens it belongs to are then unspecified.
 * The workspace (bytes and layout from the _masked size functions, which
 * return 0 / NVFP4_E_SHAPE for a bad capacity) holds E*capacity rows:
 * rows_cap = E*capacity and off[e] = e*capacity, off[E] = E*capacity. */
NVFP4MOE_API size_t nvfp4moe_workspace_bytes_masked(const nvfp4moe_config* cfg, int32_t capacity);
NVFP4MOE_API int nvfp4moe_workspace_layout_masked(const nvfp4moe_config* cfg, int32_t capacity,
                                                  nvfp4moe_ws_layout* layout_host);
NVFP4MOE_API int nvfp4moe_moe_expert_forward_masked(const nvfp4moe_config* cfg, int32_t capacity, const uint16_t* x,
                                                    int32_t T, const int32_t* ids, const float* probs,
                                                    const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q, uint16_t* out,
                                                    void* workspace, size_t workspace_bytes, void* stream);

/* Router: the step that produces ids and probs for the expert forward.
 * Article, section 4.4 ("R3 unnecessary": the scoring GEMM is one
 * FP32-output kernel for every batch size, so routing recomputed on another
 * side matches) and section 2 (the same discrete choice needs the same
 * tie-breaking and output order).
 *   x         [T, H] BF16 tokens; w_router [E, H] BF16 (16-byte aligned)
 *   logits    [T, E] FP32 out: sum_h x[t,h] * w[e,h], accumulated in FP32
 *             by one instruction sequence for every T and every position of
 *             the token in the batch (bitwise batch-invariant)
 *   ids       [T, K] int32 out: the K highest-scoring experts, higher score
 *             first, equal scores (-0 equals +0) to the lower expert id
 *   probs     [T, K] FP32 out: exp(l_k - l_0) / D, with D the FP32 sum of
 *             exp(l_j - l_0) over the K selected in slot order (renormalize
 *             1) or over all E experts (renormalize 0)
 * Requirements: H % 16 == 0, 1 <= E <= 1024, 1 <= K <= min(E, 32);
 * T == 0 is a no-op.  NaN scores are outside the contract.  The outputs are
 * the caller's buffers; no workspace, no synchronisation. */
NVFP4MOE_API int nvfp4moe_router_topk(const uint16_t* x, int32_t T, int32_t H, const uint16_t* w_router, int32_t E,
                                      int32_t K, int32_t renormalize, float* logits, int32_t* ids, float* probs,
                                      void* stream);

/* Dense NVFP4 linear (miniTE page, "how it differs": the NVFP4 linear with a
 * per-token outer scale g^x and a per-weight-row g^w, whose FP32 epilogue
 * multiplies the FP32 accumulator by g^x * g^w and casts to BF16; "how to
 * use it": the quantizer's buffer is the GEMM's input):
 *   out [M, N] = bf16((Q(x) . Wq^T) * g^x * g^w)
 * with x [M, K] BF16 (16-byte aligned), Wq one GEMM-layout matrix [N, K]
 * (n_mats 1), out [M, N] BF16 caller-owned.  Q(x) per row uses scale_round
 * and goes to the workspace (nvfp4_linear_workspace_bytes(M, K) bytes,
 * 256-byte aligned, caller-owned).  M >= 0, K % 128 == 0, N % 128 == 0; M = 0
 * is a no-op.  Each output row depends on its own x row only (one K order,
 * no split-K).  Errors as for the forward; no synchronisation. */
NVFP4MOE_API size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t K);
NVFP4MOE_API int nvfp4_linear(const uint16_t* x, int64_t M, int64_t K, const nvfp4_qtensor* Wq, uint16_t* out,
                 int32_t scale_round, void* workspace, size_t workspace_bytes, void* stream);

/* Bitwise batch-invariance self-test (article, section 4.4: a row's result
 * must not depend on its neighbours).  Draws n_probe probe tokens and filler
 * tokens from `seed` on the host (a counter-based generator), runs every probe
 * alone, in decode batches of every size 1..max_decode_batch with the probe
 * at a varying position among fillers, and inside one prefill batch of
 * prefill_tokens tokens holding all probes, and that prefill batch once more
 * through the masked layout (capacity: the largest expert count rounded up to
 * 32; article section 4.4, two layouts, same row results); then compares each
 * probe's output bits with its batch-1 result.  Allocates its own device
 * buffers (it is not a forward-path call) and syncs.  report_host (host, may
 * be NULL) receives {n_compared, n_mismatched_tokens, first_bad_probe,
 * first_bad_batch}, the batch being its token count, negated for the masked
 * layout.
 * Returns NVFP4_OK when every bit matches, NVFP4_E_MISMATCH otherwise. */
NVFP4MOE_API int nvfp4moe_selftest_batch_invariance(const nvfp4moe_config* cfg, const nvfp4_qtensor* W1q,
                                       const nvfp4_qtensor* W2q, uint64_t seed, int32_t n_probe,
                                       int32_t max_decode_batch, int32_t prefill_tokens, int64_t* report_host,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
