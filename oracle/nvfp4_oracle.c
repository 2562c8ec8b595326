/*
 * nvfp4_oracle.c -- plain, slow, CPU reference of the NVFP4 MoE expert forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under nvfp4_moe_expert_sort_amd/) never calls it, and the two
 * share no source: every format helper below is written here a second time,
 * on purpose, from the format definitions.
 *
 * Source of the method: the miniTE summary page ("miniTE diagnoses and
 * narrows the cross-engine execution gap of NVFP4 RL"), sections "how it
 * differs" (per-token outer scale, 16-long E4M3 block scales, E2M1 codes,
 * no Hadamard, no stochastic rounding, g = max|row|/(6*448), FP32 epilogue
 * multiply by g^x g^w then BF16 cast, router probability on the SwiGLU output
 * before FC2, combine order preserved) and "how to use it" (sort+amax, pad,
 * quantize; FC2 maxima taken from the router-weighted producer).  The article
 * "Finish RL training faster: bitwise consistent, high-performance,
 * agent-driven", section 4.4 (elementwise round-to-nearest, one rounding of
 * SiLU(gate)*up) and section 4.5 (FP32 accumulation in top-k slot order).
 *
 * Numeric contract pinned where the pages are silent:
 *   g  = fl32(amax / 2688)            (2688 = 6 * 448)
 *   d  = fl32(6 * g)
 *   v  = fl32(amax_block / d)
 *   s  = E4M3FN, round-up (default) or round-to-nearest-even, clamped to 448
 *   sg = fl32(s * g);  q = fl32(|x| / sg);  code = E2M1 nearest, ties to even,
 *        saturating at 6; if sg == 0 (a zero block) the code keeps only the sign
 *   zero row: g = 0, every scale 0, codes keep the sign bit
 * GEMMs accumulate in FP64 (products of dequantized values are exact in FP64);
 * every BF16 result is one correctly rounded RNE conversion of an FP64 value,
 * except the combine, which sums in FP32 in slot order (section 4.5 of the
 * article) and rounds that FP32 sum once.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (SSE arithmetic on x86-64: every float operation is a true IEEE binary32 op).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FLT_EVAL_METHOD__) && __FLT_EVAL_METHOD__ != 0
#error "the oracle needs IEEE binary32 evaluation of float expressions (FLT_EVAL_METHOD 0)"
#endif

/* ------------------------------------------------------------------------ */
/* BF16                                                                      */
/* ------------------------------------------------------------------------ */

/* BF16 bit pattern -> value (BF16 is the top half of an IEEE binary32). */
double orc_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round an FP64 value once, to nearest with ties to even, onto the BF16 grid
 * (8 significant bits, binary32 exponent range, subnormal spacing 2^-133). */
uint16_t orc_double_to_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    double ax = fabs(x);
    int ex;
    frexp(ax, &ex);               /* ax in [2^(ex-1), 2^ex) */
    int qexp = ex - 8;            /* spacing of 8-bit significands in that binade */
    if (qexp < -133) qexp = -133; /* BF16 subnormal spacing */
    double r = nearbyint(ldexp(ax, -qexp)); /* default rounding mode: ties to even */
    r = ldexp(r, qexp);
    if (r > 3.3895313892515355e38) r = INFINITY; /* beyond the largest finite BF16 */
    float f = (float)r;          /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    u >>= 16;
    if (signbit(x)) u |= 0x8000;
    return (uint16_t)u;
}

/* ------------------------------------------------------------------------ */
/* E2M1 (FP4) and E4M3FN (FP8) from their definitions                         */
/* ------------------------------------------------------------------------ */

/* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
 * Exponent field 0 is subnormal: value = 0.m * 2^0. */
double orc_e2m1_value(int code) {
    int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* E4M3FN (OCP): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; the
 * all-ones pattern S.1111.111 is NaN, there is no infinity, max is 448.
 * Exponent field 0 is subnormal: value = (m/8) * 2^-6. */
double orc_e4m3_value(int byte) {
    int sign = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Nearest E2M1 magnitude code (0..7) to q >= 0; a tie goes to the code with
 * an even mantissa bit; values past 6 saturate to 6.  Plain search over the
 * eight magnitudes. */
int orc_e2m1_encode(float q) {
    double x = (double)q;
    if (!(x > 0.0)) return 0;           /* 0 (and NaN, which never reaches here) */
    if (x >= 6.0) return 7;             /* saturation (also keeps huge q out of the search) */
    int best = 0;
    double bestd = fabs(x - orc_e2m1_value(0));
    for (int c = 1; c < 8; c++) {
        double d = fabs(x - orc_e2m1_value(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* E4M3FN encoding of a non-negative block scale v.
 *   mode 0 (round up):  the smallest E4M3FN value >= v, clamped to 448.
 *   mode 1 (RNE):       the nearest E4M3FN value, ties to an even mantissa,
 *                       clamped to 448.
 * Plain scan of the 127 non-negative finite codes, which increase with the
 * code. */
int orc_e4m3_encode(float v, int mode) {
    double x = (double)v;
    if (!(x > 0.0)) return 0;
    if (x >= 448.0) return 0x7E;
    int up = 0;
    while (up < 0x7E && orc_e4m3_value(up) < x) up++;
    if (mode == 0) return up;
    if (orc_e4m3_value(up) == x || up == 0) return up;
    int lo = up - 1;
    double dl = x - orc_e4m3_value(lo), du = orc_e4m3_value(up) - x;
    if (dl < du) return lo;
    if (du < dl) return up;
    return (lo & 1) == 0 ? lo : up;
}

/* ------------------------------------------------------------------------ */
/* Quantizer Q                                                               */
/* ------------------------------------------------------------------------ */

static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Q of one row of `cols` BF16 values (cols % 16 == 0), logical layout:
 * codes: cols/2 bytes, element 2i in the low nibble of byte i;
 * scales: cols/16 E4M3FN bytes; *g: the FP32 outer scale. */
void orc_quantize_row(const uint16_t* x, int64_t cols, int mode, uint8_t* codes, uint8_t* scales,
                      float* g_out) {
    float amax = 0.0f;
    for (int64_t j = 0; j < cols; j++) {
        float a = fabsf(bf16_to_float(x[j]));
        if (a > amax) amax = a;
    }
    memset(codes, 0, (size_t)(cols / 2));
    if (amax == 0.0f) {
        *g_out = 0.0f;
        memset(scales, 0, (size_t)(cols / 16));
        for (int64_t j = 0; j < cols; j++) {
            int sign = (x[j] >> 15) & 1;
            codes[j / 2] |= (uint8_t)((sign << 3) << (4 * (j & 1)));
        }
        return;
    }
    volatile float g = amax / 2688.0f; /* volatile: keep each step a separate binary32 op */
    volatile float d = 6.0f * g;
    *g_out = g;
    for (int64_t b = 0; b < cols / 16; b++) {
        float bmax = 0.0f;
        for (int j = 0; j < 16; j++) {
            float a = fabsf(bf16_to_float(x[16 * b + j]));
            if (a > bmax) bmax = a;
        }
        int sbyte = 0;
        if (bmax > 0.0f) {
            volatile float v = bmax / d;
            sbyte = orc_e4m3_encode(v, mode);
        }
        scales[b] = (uint8_t)sbyte;
        volatile float s = (float)orc_e4m3_value(sbyte);
        volatile float sg = s * g;
        for (int j = 0; j < 16; j++) {
            int64_t k = 16 * b + j;
            int sign = (x[k] >> 15) & 1;
            int mag = 0;
            if (sg != 0.0f) {
                volatile float q = fabsf(bf16_to_float(x[k])) / sg;
                mag = orc_e2m1_encode(q);
            }
            codes[k / 2] |= (uint8_t)(((sign << 3) | mag) << (4 * (k & 1)));
        }
    }
}

void orc_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int mode, uint8_t* codes,
                  uint8_t* scales, float* g) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        orc_quantize_row(x + r * ld, cols, mode, codes + r * (cols / 2), scales + r * (cols / 16), g + r);
}

/* Dequantized block values s * E2M1(code) (exact in FP64), logical layout,
 * WITHOUT the outer scale g (which the GEMM epilogue applies). */
void orc_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t k = 0; k < cols; k++) {
            int code = (codes[r * (cols / 2) + k / 2] >> (4 * (k & 1))) & 15;
            double s = orc_e4m3_value(scales[r * (cols / 16) + k / 16]);
            out[r * cols + k] = s * orc_e2m1_value(code);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* GEMM with the NVFP4 epilogue                                              */
/* ------------------------------------------------------------------------ */

/* out[m][n] = bf16( (sum_k A[m][k] * B[n][k]) * ga[m] * gb[n] ), where A and B
 * are dequantized block values (s * E2M1), the sum runs over k ascending in
 * FP64 (every product is exact) and the epilogue product is formed in FP64
 * and rounded once. */
void orc_gemm_epilogue(const double* A, const float* ga, int64_t M, const double* B, const float* gb, int64_t N,
                       int64_t K, uint16_t* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            const double* a = A + m * K;
            const double* b = B + n * K;
            for (int64_t k = 0; k < K; k++) acc += a[k] * b[k];
            out[m * N + n] = orc_double_to_bf16(acc * (double)ga[m] * (double)gb[n]);
        }
    }
}

/* Dense NVFP4 linear: out = bf16((Xq . Wq^T) g^x g^w), both operands given
 * quantized (logical layout). */
void orc_linear(const uint8_t* xc, const uint8_t* xs, const float* gx, int64_t M, const uint8_t* wc,
                const uint8_t* ws, const float* gw, int64_t N, int64_t K, uint16_t* out) {
    double* A = (double*)malloc(sizeof(double) * (size_t)(M * K));
    double* B = (double*)malloc(sizeof(double) * (size_t)(N * K));
    orc_dequantize(xc, xs, M, K, A);
    orc_dequantize(wc, ws, N, K, B);
    orc_gemm_epilogue(A, gx, M, B, gw, N, K, out);
    free(A);
    free(B);
}

/* ------------------------------------------------------------------------ */
/* Router-weighted SwiGLU producer and the slot-order combine                */
/* ------------------------------------------------------------------------ */

double orc_silu(double a) { return a / (1.0 + exp(-a)); }

/* h[r][n] = bf16( silu(gate) * up * p[r] ) with gate = y1[r][n], up = y1[r][I+n]
 * (the two BF16 halves of the FC1 output), all in FP64, rounded once.
 * amax2[r] = max_n |h[r][n]| over the BF16 values (the tensor FC2 consumes). */
void orc_swiglu_prob(const uint16_t* y1, const float* p, int64_t R, int64_t I, uint16_t* h, float* amax2) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        float mx = 0.0f;
        for (int64_t n = 0; n < I; n++) {
            double gate = orc_bf16_to_double(y1[r * 2 * I + n]);
            double up = orc_bf16_to_double(y1[r * 2 * I + I + n]);
            uint16_t v = orc_double_to_bf16(orc_silu(gate) * up * (double)p[r]);
            h[r * I + n] = v;
            float a = fabsf(bf16_to_float(v));
            if (a > mx) mx = a;
        }
        amax2[r] = mx;
    }
}

/* out[t][m] = bf16( ((0.0f + y2[t,0][m]) + y2[t,1][m]) + ... ) in FP32, slots
 * k = 0..K-1 in the order the routing lists them.  y2 is indexed per (t, k). */
void orc_combine(const uint16_t* y2, int64_t T, int64_t K, int64_t H, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        for (int64_t m = 0; m < H; m++) {
            volatile float acc = 0.0f;
            for (int64_t k = 0; k < K; k++) acc = acc + bf16_to_float(y2[(t * K + k) * H + m]);
            out[t * H + m] = orc_double_to_bf16((double)acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Expert sort (the layout the hot path must produce, from its definition)  */
/* ------------------------------------------------------------------------ */

/* Pairs p = t*K + k.  Expert e owns rows [off[e], off[e+1]) of the sorted
 * buffer; its n_e pairs come first in increasing p (a stable sort by expert),
 * followed by padding up to a multiple of m_align.  Returns P_pad = off[E].
 * row2pair[r] = p for a pair row and -1 for a padding row (sized by P_pad).
 * Returns -1 if an id is outside [0, E). */
int64_t orc_route(const int32_t* ids, int64_t T, int64_t K, int64_t E, int64_t m_align, int64_t* off,
                  int32_t* pair2row, int32_t* row2pair, int64_t row2pair_cap) {
    int64_t P = T * K;
    int64_t* cnt = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    for (int64_t p = 0; p < P; p++) {
        if (ids[p] < 0 || ids[p] >= E) {
            free(cnt);
            return -1;
        }
        cnt[ids[p]]++;
    }
    off[0] = 0;
    for (int64_t e = 0; e < E; e++) off[e + 1] = off[e] + (cnt[e] + m_align - 1) / m_align * m_align;
    int64_t P_pad = off[E];
    if (row2pair) {
        int64_t n = P_pad < row2pair_cap ? P_pad : row2pair_cap;
        for (int64_t r = 0; r < n; r++) row2pair[r] = -1;
    }
    for (int64_t e = 0; e < E; e++) cnt[e] = 0;
    for (int64_t p = 0; p < P; p++) {
        int64_t e = ids[p];
        int64_t r = off[e] + cnt[e]++;
        pair2row[p] = (int32_t)r;
        if (row2pair && r < row2pair_cap) row2pair[r] = (int32_t)p;
    }
    free(cnt);
    return P_pad;
}

/* The masked fixed-capacity layout (article, section 4.4, "two layouts, same
 * row results": the decode side hands the expert GEMMs per-expert chunks of a
 * fixed capacity, the training side packed rows).  Expert e owns the chunk of
 * rows [e*capacity, (e+1)*capacity), so off[e] = e*capacity.  Its pairs take
 * the chunk's rows in increasing p, as in the contiguous layout; a pair whose
 * rank within its expert is capacity or more gets no row (pair2row = -1).
 * The kept rows are followed by padding rows (-1) up to a multiple of
 * m_align; row_used[r] is 1 for kept and padding rows, 0 for the rest of the
 * chunk, which holds nothing.  row2pair and row_used have E*capacity entries.
 * Returns the number of pairs left without a row, -1 if an id is outside
 * [0, E), -2 if capacity is not a positive multiple of m_align. */
int64_t orc_route_masked(const int32_t* ids, int64_t T, int64_t K, int64_t E, int64_t m_align, int64_t capacity,
                         int64_t* off, int32_t* pair2row, int32_t* row2pair, uint8_t* row_used) {
    int64_t P = T * K;
    if (capacity <= 0 || capacity % m_align != 0) return -2;
    for (int64_t p = 0; p < P; p++)
        if (ids[p] < 0 || ids[p] >= E) return -1;
    int64_t* rank = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    for (int64_t e = 0; e <= E; e++) off[e] = e * capacity;
    for (int64_t r = 0; r < E * capacity; r++) {
        row2pair[r] = -1;
        row_used[r] = 0;
    }
    int64_t dropped = 0;
    for (int64_t p = 0; p < P; p++) {
        int64_t e = ids[p];
        int64_t i = rank[e]++;
        if (i >= capacity) {
            pair2row[p] = -1;
            dropped++;
            continue;
        }
        pair2row[p] = (int32_t)(off[e] + i);
        row2pair[off[e] + i] = (int32_t)p;
    }
    for (int64_t e = 0; e < E; e++) {
        int64_t kept = rank[e] < capacity ? rank[e] : capacity;
        int64_t padded = (kept + m_align - 1) / m_align * m_align;
        for (int64_t i = 0; i < padded; i++) row_used[off[e] + i] = 1;
    }
    free(rank);
    return dropped;
}

/* ------------------------------------------------------------------------ */
/* Router (the step before the path)                                         */
/* ------------------------------------------------------------------------ */

/* Router scores: logits[t][e] = sum_h x[t][h] * w[e][h] over the BF16 values,
 * in FP64 (every product of two BF16 values is exact in FP64).  The article,
 * section 4.4 ("R3 unnecessary"): the scoring GEMM is one FP32-output kernel
 * for every batch size; this is the exact value that kernel approximates. */
void orc_router_logits(const uint16_t* x, int64_t T, int64_t H, const uint16_t* w, int64_t E, double* logits) {
    for (int64_t t = 0; t < T; t++)
        for (int64_t e = 0; e < E; e++) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; h++) acc += orc_bf16_to_double(x[t * H + h]) * orc_bf16_to_double(w[e * H + h]);
            logits[t * E + e] = acc;
        }
}

/* Top-k of given FP32 router scores (the article, section 2: the same
 * discrete choice needs the same tie-breaking and output order).  Experts are
 * ranked by score, higher first, equal scores by the lower expert id: a total
 * order, so the K selected and their order are unique.  Slot k holds the k-th
 * expert of that order.  Probabilities (softmax; the softmax is increasing in
 * the score, so it selects the same experts): p_k = exp(l_k - l_0) / D with D
 * the sum of exp(l_j - l_0) over the K selected (renormalize != 0) or over
 * all E experts, in FP64, stored as FP32. */
void orc_router_topk(const float* logits, int64_t T, int64_t E, int64_t K, int renormalize, int32_t* ids,
                     float* probs) {
    char* taken = (char*)malloc((size_t)E);
    for (int64_t t = 0; t < T; t++) {
        const float* l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int64_t k = 0; k < K; k++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++) /* strict '>' keeps the lower id on equal scores */
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            ids[t * K + k] = (int32_t)best;
        }
        const double top = l[ids[t * K]];
        double den = 0.0;
        if (renormalize)
            for (int64_t k = 0; k < K; k++) den += exp((double)l[ids[t * K + k]] - top);
        else
            for (int64_t e = 0; e < E; e++) den += exp((double)l[e] - top);
        for (int64_t k = 0; k < K; k++) probs[t * K + k] = (float)(exp((double)l[ids[t * K + k]] - top) / den);
    }
    free(taken);
}

/* ------------------------------------------------------------------------ */
/* The layer                                                                 */
/* ------------------------------------------------------------------------ */

/* FC2 of one pair: y2 = bf16((a . W2[e]^T) g^a g^w2) over the H rows of W2[e].
 * quantize_h != 0 (the NVFP4 layer): a = Q(h) dequantized and g^a its outer
 * scale, Q taken on the BF16 h that FC2 consumes; quantize_h == 0 (W4A16):
 * a = the BF16 values of h and g^a = 1.  w2d: E matrices [H][I] of
 * dequantized weights, w2g their outer scales.  hc, hs, hd: scratch of I/2,
 * I/16 bytes and I doubles. */
static void fc2_pair(const uint16_t* h, int64_t I, int64_t H, int64_t e, const double* w2d, const float* w2g,
                     int quantize_h, int mode, uint8_t* hc, uint8_t* hs, double* hd, uint16_t* y2) {
    double gh = 1.0;
    if (quantize_h) {
        float g;
        orc_quantize_row(h, I, mode, hc, hs, &g);
        orc_dequantize(hc, hs, 1, I, hd);
        gh = (double)g;
    } else {
        for (int64_t k = 0; k < I; k++) hd[k] = orc_bf16_to_double(h[k]);
    }
    for (int64_t m = 0; m < H; m++) {
        int64_t wr = e * H + m;
        const double* w = w2d + wr * I;
        double acc = 0.0;
        for (int64_t k = 0; k < I; k++) acc += hd[k] * w[k];
        y2[m] = orc_double_to_bf16(acc * gh * (double)w2g[wr]);
    }
}

/* The FC2 step alone, from a given h: y2[p] = fc2_pair(h[p], expert ids[p])
 * for P pairs (h [P][I] BF16, y2 [P][H] BF16), with the same arithmetic as
 * the layers below.  Lets a test run FC2 on another implementation's h. */
void orc_moe_fc2(const uint16_t* h, int64_t P, int64_t I, int64_t H, const int32_t* ids, const double* w2d,
                 const float* w2g, int quantize_h, int mode, uint16_t* y2) {
#pragma omp parallel
    {
        uint8_t* hc = (uint8_t*)malloc((size_t)(I / 2));
        uint8_t* hs = (uint8_t*)malloc((size_t)(I / 16));
        double* hd = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 16)
        for (int64_t p = 0; p < P; p++)
            fc2_pair(h + p * I, I, H, ids[p], w2d, w2g, quantize_h, mode, hc, hs, hd, y2 + p * H);
        free(hc);
        free(hs);
        free(hd);
    }
}

/* NVFP4 MoE expert forward for T tokens, computed per (token, slot) pair with
 * no sorting (the sorted layout changes no value):
 *   Xq = Q(x[t])                                   per token
 *   y1 = bf16((Xq . W1q[e]^T) g^x g^w1)            [2I] per pair, FP64 GEMM
 *   h  = bf16(silu(gate) * up * p),  amax2 = max|h|
 *   y2 = bf16((Q(h) . W2q[e]^T) g^h g^w2)          [H] per pair
 *   out[t] = bf16(FP32 sum over k of y2[t,k])
 * The weights come dequantized (s * E2M1 values from orc_dequantize, exact in
 * FP64) with their outer scales: w1d holds E matrices [2I][H] (rows 0..I-1
 * gate, I..2I-1 up), w2d E matrices [H][I].  Optional outputs (NULL to skip),
 * indexed per pair p = t*K+k: y1 [P][2I], h [P][I], amax2 [P], y2 [P][H]. */
void orc_moe_forward_deq(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t K, const int32_t* ids,
                         const float* probs, const double* w1d, const float* w1g, const double* w2d,
                         const float* w2g, int mode, uint16_t* out, uint16_t* y1_out, uint16_t* h_out,
                         float* amax2_out, uint16_t* y2_out) {
    int64_t P = T * K;
    uint8_t* xc = (uint8_t*)malloc((size_t)(T * H / 2));
    uint8_t* xs = (uint8_t*)malloc((size_t)(T * H / 16));
    float* gx = (float*)malloc(sizeof(float) * (size_t)T);
    orc_quantize(x, T, H, H, mode, xc, xs, gx);
    double* xd = (double*)malloc(sizeof(double) * (size_t)(T * H));
    orc_dequantize(xc, xs, T, H, xd);

    uint16_t* y2 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(P * H));
#pragma omp parallel
    {
        double* hd = (double*)malloc(sizeof(double) * (size_t)I);
        uint16_t* y1 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(2 * I));
        uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
        uint8_t* hc = (uint8_t*)malloc((size_t)(I / 2));
        uint8_t* hs = (uint8_t*)malloc((size_t)(I / 16));
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < P; p++) {
            int64_t t = p / K, e = ids[p];
            const double* a = xd + t * H;
            /* FC1 */
            for (int64_t n = 0; n < 2 * I; n++) {
                int64_t wr = e * 2 * I + n;
                const double* w = w1d + wr * H;
                double acc = 0.0;
                for (int64_t k = 0; k < H; k++) acc += a[k] * w[k];
                y1[n] = orc_double_to_bf16(acc * (double)gx[t] * (double)w1g[wr]);
            }
            /* router-weighted SwiGLU producer */
            float amax2;
            orc_swiglu_prob(y1, probs + p, 1, I, h, &amax2);
            /* FC2 on Q(h), Q taken on the BF16 h that FC2 consumes */
            fc2_pair(h, I, H, e, w2d, w2g, 1, mode, hc, hs, hd, y2 + p * H);
            if (y1_out) memcpy(y1_out + p * 2 * I, y1, sizeof(uint16_t) * (size_t)(2 * I));
            if (h_out) memcpy(h_out + p * I, h, sizeof(uint16_t) * (size_t)I);
            if (amax2_out) amax2_out[p] = amax2;
        }
        free(hd);
        free(y1);
        free(h);
        free(hc);
        free(hs);
    }
    orc_combine(y2, T, K, H, out);
    if (y2_out) memcpy(y2_out, y2, sizeof(uint16_t) * (size_t)(P * H));
    free(y2);
    free(xd);
    free(xc);
    free(xs);
    free(gx);
}

/* The same layer with the weights given quantized (logical layout): they are
 * dequantized once, then the layer runs as above. */
/* The W4A16 variant (the article, section 6: NVFP4 W4A16 routed experts):
 * the same layer with NVFP4 weights and BF16 activations left unquantized,
 * computed per (token, slot) pair:
 *   y1 = bf16((x[t] . W1q[e]^T) g^w1)            [2I], FP64 GEMM
 *   h  = bf16(silu(gate) * up * p)
 *   y2 = bf16((h . W2q[e]^T) g^w2)               [H]
 *   out[t] = bf16(FP32 sum over k of y2[t,k])
 * Weights as for orc_moe_forward_deq; optional per-pair outputs (NULL to
 * skip): y1 [P][2I], h [P][I], y2 [P][H]. */
void orc_moe_forward_w4a16(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t K, const int32_t* ids,
                           const float* probs, const double* w1d, const float* w1g, const double* w2d,
                           const float* w2g, uint16_t* out, uint16_t* y1_out, uint16_t* h_out, uint16_t* y2_out) {
    int64_t P = T * K;
    uint16_t* y2 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(P * H));
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)H);
        double* hd = (double*)malloc(sizeof(double) * (size_t)I);
        uint16_t* y1 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(2 * I));
        uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < P; p++) {
            int64_t t = p / K, e = ids[p];
            for (int64_t k = 0; k < H; k++) a[k] = orc_bf16_to_double(x[t * H + k]);
            for (int64_t n = 0; n < 2 * I; n++) {
                int64_t wr = e * 2 * I + n;
                const double* w = w1d + wr * H;
                double acc = 0.0;
                for (int64_t k = 0; k < H; k++) acc += a[k] * w[k];
                y1[n] = orc_double_to_bf16(acc * (double)w1g[wr]);
            }
            float amax2;
            orc_swiglu_prob(y1, probs + p, 1, I, h, &amax2);
            fc2_pair(h, I, H, e, w2d, w2g, 0, 0, NULL, NULL, hd, y2 + p * H);
            if (y1_out) memcpy(y1_out + p * 2 * I, y1, sizeof(uint16_t) * (size_t)(2 * I));
            if (h_out) memcpy(h_out + p * I, h, sizeof(uint16_t) * (size_t)I);
        }
        free(a);
        free(hd);
        free(y1);
        free(h);
    }
    orc_combine(y2, T, K, H, out);
    if (y2_out) memcpy(y2_out, y2, sizeof(uint16_t) * (size_t)(P * H));
    free(y2);
}

void orc_moe_forward(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                     const int32_t* ids, const float* probs, const uint8_t* w1c, const uint8_t* w1s,
                     const float* w1g, const uint8_t* w2c, const uint8_t* w2s, const float* w2g, int mode,
                     uint16_t* out, uint16_t* y1_out, uint16_t* h_out, float* amax2_out, uint16_t* y2_out) {
    double* w1d = (double*)malloc(sizeof(double) * (size_t)(E * 2 * I * H));
    double* w2d = (double*)malloc(sizeof(double) * (size_t)(E * H * I));
    orc_dequantize(w1c, w1s, E * 2 * I, H, w1d);
    orc_dequantize(w2c, w2s, E * H, I, w2d);
    orc_moe_forward_deq(x, T, H, I, K, ids, probs, w1d, w1g, w2d, w2g, mode, out, y1_out, h_out, amax2_out,
                        y2_out);
    free(w1d);
    free(w2d);
}

/* ------------------------------------------------------------------------ */
/* BF16 straight-through backward                                            */
/* ------------------------------------------------------------------------ */

/* d silu / d a = sigmoid(a) (1 + a (1 - sigmoid(a))), in FP64. */
double orc_silu_grad(double a) {
    double sg = 1.0 / (1.0 + exp(-a));
    return sg * (1.0 + a * (1.0 - sg));
}

/* SwiGLU backward of R rows (miniTE page, "how it differs": router
 * probability on the SwiGLU output): from dh [R][I] (BF16), the forward's
 * y1 [R][2I] = [gate | up] (BF16) and p [R]:
 *   dgate = bf16(dh p up silu'(gate)),  dup = bf16(dh p silu(gate))   in dy1 [R][2I]
 *   dprob = fl32(sum_n dh silu(gate) up)                               in dprob [R]
 * all in FP64. */
void orc_swiglu_backward(const uint16_t* dh, const uint16_t* y1, const float* p, int64_t R, int64_t I, uint16_t* dy1,
                         float* dprob) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        double pr = (double)p[r], dp = 0.0;
        for (int64_t n = 0; n < I; n++) {
            double g = orc_bf16_to_double(y1[r * 2 * I + n]);
            double u = orc_bf16_to_double(y1[r * 2 * I + I + n]);
            double d = orc_bf16_to_double(dh[r * I + n]);
            dy1[r * 2 * I + n] = orc_double_to_bf16(d * pr * u * orc_silu_grad(g));
            dy1[r * 2 * I + I + n] = orc_double_to_bf16(d * pr * orc_silu(g));
            dp += d * orc_silu(g) * u;
        }
        dprob[r] = (float)dp;
    }
}

/* Weight gradients from given per-pair gradients: for each expert e, over its
 * pairs p = t*K + k in increasing p, in FP64, stored as FP32:
 *   dw1[e] = sum dy1[p]^T x[t]   [2I][H],    dw2[e] = sum dy2[t]^T h[p]   [H][I]
 * with dy2[t] = dout[t] (the combine's gradient).  All inputs BF16. */
void orc_moe_weight_grads(const uint16_t* x, const uint16_t* dout, int64_t T, int64_t H, int64_t I, int64_t E,
                          int64_t K, const int32_t* ids, const uint16_t* dy1, const uint16_t* h, float* dw1,
                          float* dw2) {
    int64_t P = T * K;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t e = 0; e < E; e++) {
        double* a1 = (double*)calloc((size_t)(2 * I * H), sizeof(double));
        double* a2 = (double*)calloc((size_t)(H * I), sizeof(double));
        for (int64_t p = 0; p < P; p++) {
            if (ids[p] != e) continue;
            int64_t t = p / K;
            for (int64_t j = 0; j < 2 * I; j++) {
                double d = orc_bf16_to_double(dy1[p * 2 * I + j]);
                for (int64_t m = 0; m < H; m++) a1[j * H + m] += d * orc_bf16_to_double(x[t * H + m]);
            }
            for (int64_t m = 0; m < H; m++) {
                double d = orc_bf16_to_double(dout[t * H + m]);
                for (int64_t n = 0; n < I; n++) a2[m * I + n] += d * orc_bf16_to_double(h[p * I + n]);
            }
        }
        for (int64_t i = 0; i < 2 * I * H; i++) dw1[e * 2 * I * H + i] = (float)a1[i];
        for (int64_t i = 0; i < H * I; i++) dw2[e * H * I + i] = (float)a2[i];
        free(a1);
        free(a2);
    }
}

/* The backward of the expert forward (miniTE page, "how it differs": the
 * backward is the straight-through approximation -- quantization is taken as
 * the identity -- computed by BF16 GEMMs on the stored original BF16
 * activations and weights, so nothing is quantized in the backward).  With
 * p = t*K + k, e = ids[p], gate/up the forward's BF16 FC1 outputs y1[p] and
 * h[p] its BF16 FC2 input, per pair:
 *   dh[p]     = bf16( dout[t] . W2[e] )                       FP64 sum over H
 *   dgate[p]  = bf16( dh * prob * up * silu'(gate) )          FP64, elementwise
 *   dup[p]    = bf16( dh * prob * silu(gate) )
 *   dprob[p]  = fl32( sum_n dh[n] silu(gate[n]) up[n] )       FP64 sum over I
 *   dxp[p]    = bf16( [dgate | dup] . W1[e] )                 FP64 sum over 2I
 * and per token and expert:
 *   dx[t]     = bf16( FP32 sum of dxp[t, k] over k = 0..K-1, from +0.0f )
 *   dW2[e]    = fl32( sum over the pairs of e of dout[t]^T h[p] )      [H][I]
 *   dW1[e]    = fl32( sum over the pairs of e of [dgate|dup]^T x[t] )  [2I][H]
 * (the combine out[t] = sum_k y2[t, k] passes dout[t] to every slot; the
 * router probability multiplies the SwiGLU output, so its gradient is the dot
 * product of dh with silu(gate) up).  Weights w1 [E][2I][H], w2 [E][H][I] and
 * x, y1, h, dout are BF16 bit patterns; dh_out [P][I] and dy1_out [P][2I]
 * (BF16, may be NULL) return the intermediates. */
void orc_moe_backward(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, const int32_t* ids,
                      const float* probs, const uint16_t* w1, const uint16_t* w2, const uint16_t* y1,
                      const uint16_t* h, const uint16_t* dout, uint16_t* dx, float* dprobs, float* dw1, float* dw2,
                      uint16_t* dh_out, uint16_t* dy1_out) {
    int64_t P = T * K;
    uint16_t* dh = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(P * I));
    uint16_t* dy1 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(P * 2 * I));
    uint16_t* dxp = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(P * H));
    /* per pair: dh */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t p = 0; p < P; p++) {
        int64_t t = p / K, e = ids[p];
        const uint16_t* w2e = w2 + e * H * I;
        for (int64_t n = 0; n < I; n++) {
            double acc = 0.0;
            for (int64_t m = 0; m < H; m++)
                acc += orc_bf16_to_double(dout[t * H + m]) * orc_bf16_to_double(w2e[m * I + n]);
            dh[p * I + n] = orc_double_to_bf16(acc);
        }
    }
    /* the SwiGLU backward and the router-probability gradient */
    orc_swiglu_backward(dh, y1, probs, P, I, dy1, dprobs);
    /* per pair: the FC1 input gradient; per token: the slot-order sum */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t p = 0; p < P; p++) {
        const uint16_t* w1e = w1 + (int64_t)ids[p] * 2 * I * H;
        for (int64_t m = 0; m < H; m++) {
            double acc = 0.0;
            for (int64_t j = 0; j < 2 * I; j++)
                acc += orc_bf16_to_double(dy1[p * 2 * I + j]) * orc_bf16_to_double(w1e[j * H + m]);
            dxp[p * H + m] = orc_double_to_bf16(acc);
        }
    }
    orc_combine(dxp, T, K, H, dx); /* FP32 slot-order sum, one BF16 rounding */
    /* weight gradients: per expert, its pairs in increasing p */
    orc_moe_weight_grads(x, dout, T, H, I, E, K, ids, dy1, h, dw1, dw2);
    if (dh_out) memcpy(dh_out, dh, sizeof(uint16_t) * (size_t)(P * I));
    if (dy1_out) memcpy(dy1_out, dy1, sizeof(uint16_t) * (size_t)(P * 2 * I));
    free(dh);
    free(dy1);
    free(dxp);
}
