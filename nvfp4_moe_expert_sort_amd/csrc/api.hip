// api.hip -- host side of the C ABI declared in include/nvfp4moe.h: argument
// checks (before any launch), workspace carving, launch order, self-test.
//
// The forward enqueues, on the caller's stream and with no host sync:
//   route_count -> route_scan -> route_place (route_small alone up to 1024
//   pairs) -> route_gather (sort + amax + quantize X into the padded
//   GEMM-layout buffer) -> FC1 grouped GEMM with the router-weighted SwiGLU
//   producer (h and its per-32-column maxima) -> quantize h -> FC2 grouped
//   GEMM -> slot-order combine.
// (miniTE summary page, "how to use it"; article sections 4.4-4.6.)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/nvfp4moe.h"
#include "nvfp4_kernels.h"

using namespace nvfp4;

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool cfg_ok(const nvfp4moe_config* c) {
    if (!c) return false;
    if (c->hidden <= 0 || c->hidden % 128 != 0) return false;
    if (c->inter <= 0 || c->inter % 128 != 0) return false;
    if (c->n_experts < 1 || c->n_experts > kMaxExperts) return false;
    if (c->top_k < 1 || c->top_k > kMaxTopK || c->top_k > c->n_experts) return false;
    if (c->max_tokens < 0) return false;
    if (c->scale_round != NVFP4_SCALE_RU && c->scale_round != NVFP4_SCALE_RNE) return false;
    const int64_t rows = (int64_t)c->max_tokens * c->top_k + (int64_t)c->n_experts * (kMAlign - 1);
    if (rows >= (int64_t)1 << 30) return false;  // sorted row indices are int32
    return true;
}

struct Layout {
    nvfp4moe_ws_layout pub;
    size_t blk_err, blk_counts, mtiles, mtiles_even, n_mtiles, row_prob, xq_codes, xq_scales, gx;
    int64_t nblk_cap, mtiles_cap;
    size_t total;
};

// Masked layout: a positive multiple of kMAlign, with E * capacity rows
// addressable by int32 row indices.
bool capacity_ok(const nvfp4moe_config* c, int32_t capacity) {
    return capacity > 0 && capacity % kMAlign == 0 && (int64_t)c->n_experts * capacity < ((int64_t)1 << 30);
}

// capacity 0: contiguous layout (rows bounded by max_tokens); > 0: masked
// layout, E chunks of `capacity` rows.
Layout make_layout(const nvfp4moe_config* c, int32_t capacity = 0) {
    Layout L{};
    const int64_t E = c->n_experts, K = c->top_k, H = c->hidden, I = c->inter, Tm = c->max_tokens;
    const int64_t P = Tm * K;
    const int64_t rows = capacity > 0 ? E * capacity : (int64_t)up((size_t)(P + E * (kMAlign - 1)), kMAlign);
    L.nblk_cap = std::max<int64_t>(1, (Tm + kTokPerBlk - 1) / kTokPerBlk);
    L.mtiles_cap = rows / kTileRows + E + 1;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = up(o + std::max<size_t>(bytes, 1), kAlign);
        return at;
    };
    L.pub.err = take(4);
    L.blk_err = take(4 * L.nblk_cap);
    L.blk_counts = take(4 * L.nblk_cap * E);
    L.pub.expert_count = take(4 * E);
    L.pub.expert_off = take(4 * (E + 1));
    L.n_mtiles = take(4);
    L.mtiles = take(16 * L.mtiles_cap);
    L.mtiles_even = take(16 * L.mtiles_cap);
    L.pub.pair2row = take(4 * std::max<int64_t>(P, 1));
    L.pub.row2pair = take(4 * rows);
    L.row_prob = take(4 * rows);
    L.xq_codes = take(std::max<int64_t>(Tm, 1) * H / 2);
    L.xq_scales = take(std::max<int64_t>(Tm, 1) * H / 16);
    L.gx = take(4 * std::max<int64_t>(Tm, 1));
    L.pub.a1_codes = take(rows * H / 2);
    L.pub.a1_scales = take(rows * H / 16);
    L.pub.a1_g = take(4 * rows);
    L.pub.h = take(2 * rows * I);
    L.pub.amax2_part = take(4 * rows * (I / 32));
    L.pub.a2_codes = take(rows * I / 2);
    L.pub.a2_scales = take(rows * I / 16);
    L.pub.a2_g = take(4 * rows);
    L.pub.y2 = take(2 * rows * H);
    L.pub.rows_cap = rows;
    L.pub.m_align = kMAlign;
    L.pub.n_part = (int32_t)(I / 32);
    L.total = o;
    return L;
}

bool qt_ok(const nvfp4_qtensor* q, int64_t n_mats, int64_t rows, int64_t cols) {
    return q && q->codes && q->scales && q->g && q->n_mats == n_mats && q->rows == rows && q->cols == cols &&
           q->layout == NVFP4_LAYOUT_GEMM;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_E_HIP; }

// Persistent GEMM grid: two 4-wave workgroups per CU, at most one per tile
// (FC2 and the dense linear; FC1 uses the hybrid grid below).
int grid_blocks(int64_t tiles_bound) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    return (int)std::max<int64_t>(8, std::min<int64_t>(tiles_bound, 2 * (int64_t)cus));
}

// Hybrid GEMM grid (gemm_kernel with persist > 0): `persist` = two
// workgroups per CU walking a static bulk, then enough one-tile workgroups for
// the one to two rounds left over (tiles_bound bounds the tail).
int hybrid_persist() { return std::max(8, grid_blocks(1 << 30) / 8 * 8); }
int hybrid_grid(int64_t tiles_bound) {
    const int64_t np = hybrid_persist();
    return (int)(np + std::min<int64_t>(2 * np + 8, tiles_bound));
}

int32_t col_tiles(int64_t n, int mode) {
    const int64_t w = gemm_cols_per_tile(mode);
    return (int32_t)((n + w - 1) / w);
}

}  // namespace

// Scratch of the allocation-free forward: one static array per GPU the
// library runs on.  Host code never passes `scratch` itself to a kernel or a
// copy (on the host it names a stand-in, not device memory): it uses the
// device address hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kNoAllocScratchBytes = NVFP4MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on its first use
// there, with that device current).
int noalloc_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return NVFP4_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return NVFP4_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NVFP4_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_status_str(int s) {
    switch (s) {
        case NVFP4_OK: return "ok";
        case NVFP4_E_NULL: return "null pointer";
        case NVFP4_E_SHAPE: return "invalid shape";
        case NVFP4_E_ALIGN: return "misaligned pointer";
        case NVFP4_E_WORKSPACE: return "workspace too small";
        case NVFP4_E_CAPACITY: return "token count exceeds max_tokens";
        case NVFP4_E_HIP: return "HIP error";
        case NVFP4_E_MISMATCH: return "batch-invariance mismatch";
        case NVFP4_E_DEVICE: return "device-side contract violation";
        case NVFP4_E_ARG: return "invalid enum argument";
        case NVFP4_E_SCRATCH: return "token count too large for the allocation-free forward's static scratch";
        default: return "unknown status";
    }
}

int nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                   float* g, int32_t layout, int32_t scale_round, void* stream) {
    if (layout != NVFP4_LAYOUT_LOGICAL && layout != NVFP4_LAYOUT_GEMM) return NVFP4_E_ARG;
    if (scale_round != NVFP4_SCALE_RU && scale_round != NVFP4_SCALE_RNE) return NVFP4_E_ARG;
    if (rows < 0 || cols <= 0 || cols % 16 != 0 || ld < cols) return NVFP4_E_SHAPE;
    if (layout == NVFP4_LAYOUT_GEMM && (rows % 32 != 0 || cols % 128 != 0)) return NVFP4_E_SHAPE;
    if (rows >= ((int64_t)1 << 31)) return NVFP4_E_SHAPE;
    if (rows == 0) return NVFP4_OK;
    if (!x || !codes || !scales || !g) return NVFP4_E_NULL;
    if (!aligned(x, 16) || ld % 8 != 0 || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(g, 4))
        return NVFP4_E_ALIGN;
    return hip_status(launch_quant_rows(x, rows, cols, ld, codes, scales, g, layout == NVFP4_LAYOUT_GEMM,
                                        scale_round == NVFP4_SCALE_RU, (hipStream_t)stream));
}

size_t nvfp4moe_weight_bytes(const nvfp4moe_config* cfg, int32_t which) {
    if (!cfg_ok(cfg) || (which != 1 && which != 2)) return 0;
    const size_t E = cfg->n_experts, H = cfg->hidden, I = cfg->inter;
    const size_t rows = which == 1 ? E * 2 * I : E * H;
    const size_t cols = which == 1 ? H : I;
    return up(rows * cols / 2, kAlign) + up(rows * cols / 16, kAlign) + up(rows * 4, kAlign);
}

int nvfp4moe_quantize_weights(const nvfp4moe_config* cfg, const uint16_t* w1, const uint16_t* w2,
                              const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q, void* stream) {
    if (!cfg) return NVFP4_E_NULL;
    if (!cfg_ok(cfg)) return NVFP4_E_SHAPE;
    const int64_t E = cfg->n_experts, H = cfg->hidden, I = cfg->inter;
    if (!w1 || !w2 || !W1q || !W2q) return NVFP4_E_NULL;
    if (!qt_ok(W1q, E, 2 * I, H) || !qt_ok(W2q, E, H, I)) return NVFP4_E_SHAPE;
    const bool ru = cfg->scale_round == NVFP4_SCALE_RU;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_quant_rows(w1, E * 2 * I, H, H, W1q->codes, W1q->scales, W1q->g, true, ru, s);
    if (e != hipSuccess) return NVFP4_E_HIP;
    return hip_status(launch_quant_rows(w2, E * H, I, I, W2q->codes, W2q->scales, W2q->g, true, ru, s));
}

size_t nvfp4moe_workspace_bytes(const nvfp4moe_config* cfg) {
    if (!cfg_ok(cfg)) return 0;
    return make_layout(cfg).total;
}

int nvfp4moe_workspace_layout(const nvfp4moe_config* cfg, nvfp4moe_ws_layout* out) {
    if (!cfg || !out) return NVFP4_E_NULL;
    if (!cfg_ok(cfg)) return NVFP4_E_SHAPE;
    *out = make_layout(cfg).pub;
    return NVFP4_OK;
}

size_t nvfp4moe_workspace_bytes_masked(const nvfp4moe_config* cfg, int32_t capacity) {
    if (!cfg_ok(cfg) || !capacity_ok(cfg, capacity)) return 0;
    return make_layout(cfg, capacity).total;
}

int nvfp4moe_workspace_layout_masked(const nvfp4moe_config* cfg, int32_t capacity, nvfp4moe_ws_layout* out) {
    if (!cfg || !out) return NVFP4_E_NULL;
    if (!cfg_ok(cfg) || !capacity_ok(cfg, capacity)) return NVFP4_E_SHAPE;
    *out = make_layout(cfg, capacity).pub;
    return NVFP4_OK;
}

}  // extern "C"

namespace {

// The forward; when `events` is non-null, events[i] is recorded on the stream
// at each stage boundary (before the sort, after the sort, after FC1, after
// the FC2-input quantizer, after FC2, after the combine).
// capacity 0: the contiguous row layout; > 0: the masked layout.
// y1 non-null: the unfused forward -- FC1 as a plain grouped GEMM writing
// y1 [rows_cap, 2I], then the SwiGLU producer as a kernel of its own.
int forward_impl(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T, const int32_t* ids, const float* probs,
                 const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q, uint16_t* out, void* workspace,
                 size_t workspace_bytes, void* stream, void* const* events, int32_t capacity = 0,
                 bool w4a16 = false, uint16_t* y1 = nullptr, bool online = false) {
    if (!cfg) return NVFP4_E_NULL;
    if (!cfg_ok(cfg)) return NVFP4_E_SHAPE;
    if (capacity != 0 && !capacity_ok(cfg, capacity)) return NVFP4_E_SHAPE;
    if (T < 0) return NVFP4_E_SHAPE;
    if (T > cfg->max_tokens) return NVFP4_E_CAPACITY;
    const int64_t E = cfg->n_experts, K = cfg->top_k, H = cfg->hidden, I = cfg->inter;
    if (!W1q || !W2q) return NVFP4_E_NULL;
    if (!qt_ok(W1q, E, 2 * I, H) || !qt_ok(W2q, E, H, I)) return NVFP4_E_SHAPE;
    if (!workspace) return NVFP4_E_NULL;
    const Layout L = make_layout(cfg, capacity);
    if (workspace_bytes < L.total) return NVFP4_E_WORKSPACE;
    if (!aligned(workspace, kAlign)) return NVFP4_E_ALIGN;
    if (T == 0) return NVFP4_OK;
    if (!x || !ids || !probs || !out) return NVFP4_E_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ids, 4) || !aligned(probs, 4)) return NVFP4_E_ALIGN;

    hipStream_t s = (hipStream_t)stream;
    auto mark = [&](int i) -> bool {
        return !events || hipEventRecord((hipEvent_t)events[i], s) == hipSuccess;
    };
    uint8_t* ws = (uint8_t*)workspace;
    RouteBuffers rb;
    rb.blk_counts = (int32_t*)(ws + L.blk_counts);
    rb.blk_err = (int32_t*)(ws + L.blk_err);
    rb.expert_count = (int32_t*)(ws + L.pub.expert_count);
    rb.expert_off = (int32_t*)(ws + L.pub.expert_off);
    rb.mtiles = (int4*)(ws + L.mtiles);
    rb.mtiles_even = (int4*)(ws + L.mtiles_even);
    rb.n_mtiles = (int32_t*)(ws + L.n_mtiles);
    rb.err_word = (int32_t*)(ws + L.pub.err);
    rb.pair2row = (int32_t*)(ws + L.pub.pair2row);
    rb.row2pair = (int32_t*)(ws + L.pub.row2pair);
    rb.row_prob = (float*)(ws + L.row_prob);
    rb.xq_codes = ws + L.xq_codes;
    rb.xq_scales = ws + L.xq_scales;
    rb.gx = (float*)(ws + L.gx);
    rb.a_codes = ws + L.pub.a1_codes;
    rb.a_scales = ws + L.pub.a1_scales;
    rb.a_g = (float*)(ws + L.pub.a1_g);
    const bool ru = cfg->scale_round == NVFP4_SCALE_RU;

    if (!mark(0)) return NVFP4_E_HIP;
    hipError_t e = launch_route(x, ids, probs, T, (int32_t)H, (int32_t)K, (int32_t)E, capacity, ru, rb, L.pub.rows_cap, s,
                                !w4a16, online);
    if (e != hipSuccess || !mark(1)) return NVFP4_E_HIP;

    // Static bounds for this T (the device counts are <= these): at most
    // min(E, T*K) experts receive pairs, each padded by at most kMAlign - 1
    // rows and ending in at most one partial row tile.
    const int64_t P = (int64_t)T * K, used = std::min<int64_t>(E, P);
    const int64_t mt_bound = (P + used * (kMAlign - 1)) / kTileRows + used + 1;

    if (w4a16) {
        // NVFP4 weights x BF16 activations: FC1 reads x's rows through
        // row2pair, FC2 reads h as FC1 wrote it; no activation quantizer.
        W16Params g1{};
        g1.a = x;
        g1.row2pair = rb.row2pair;
        g1.top_k = (int32_t)K;
        g1.b_codes = W1q->codes;
        g1.b_scales = W1q->scales;
        g1.b_g = W1q->g;
        g1.K = (int32_t)H;
        g1.N = (int32_t)(2 * I);
        g1.n_tiles_n = col_tiles(I, kGemmSwiGLU);
        g1.mtiles = rb.mtiles_even;  // each expert's subtiles spread evenly over its row tiles (as the W4A4 FC1)
        g1.n_mtiles = rb.n_mtiles;
        g1.out = (uint16_t*)(ws + L.pub.h);
        g1.ld_out = I;
        g1.row_prob = rb.row_prob;
        g1.inter = (int32_t)I;
        e = launch_gemm_w4a16(kGemmSwiGLU, g1, mt_bound, s);
        if (e != hipSuccess || !mark(2) || !mark(3)) return NVFP4_E_HIP;
        W16Params g2{};
        g2.a = g1.out;
        g2.b_codes = W2q->codes;
        g2.b_scales = W2q->scales;
        g2.b_g = W2q->g;
        g2.K = (int32_t)I;
        g2.N = (int32_t)H;
        g2.n_tiles_n = col_tiles(H, kGemmPlain);
        g2.mtiles = rb.mtiles;
        g2.n_mtiles = rb.n_mtiles;
        g2.out = (uint16_t*)(ws + L.pub.y2);
        g2.ld_out = H;
        e = launch_gemm_w4a16(kGemmPlain, g2, mt_bound, s);
        if (e != hipSuccess || !mark(4)) return NVFP4_E_HIP;
        e = launch_combine(g2.out, rb.pair2row, T, (int32_t)H, (int32_t)K, out, s);
        if (e != hipSuccess || !mark(5)) return NVFP4_E_HIP;
        return NVFP4_OK;
    }

    GemmParams f1{};
    f1.a_codes = rb.a_codes;
    f1.a_scales = rb.a_scales;
    f1.a_g = rb.a_g;
    f1.b_codes = W1q->codes;
    f1.b_scales = W1q->scales;
    f1.b_g = W1q->g;
    f1.K = (int32_t)H;
    f1.N = (int32_t)(2 * I);
    f1.n_tiles_n = col_tiles(I, kGemmSwiGLU);
    f1.mtiles = rb.mtiles_even;  // (the unfused plain GEMM below takes the 4-subtile table)
    f1.n_mtiles = rb.n_mtiles;
    f1.dense_m = -1;
    f1.out = (uint16_t*)(ws + L.pub.h);
    f1.ld_out = I;
    f1.row_prob = rb.row_prob;
    f1.amax_part = (float*)(ws + L.pub.amax2_part);
    f1.n_part = (int32_t)(I / 32);
    f1.inter = (int32_t)I;
    if (online) {
        // X quantized inside FC1 from its BF16 rows (the sort recorded each
        // token's max |x| in gx and each sorted row's g in a1_g)
        f1.a_bf16 = x;
        f1.a_amax = rb.gx;
        f1.a_row2pair = rb.row2pair;
        f1.a_top_k = (int32_t)K;
        f1.a_round_up = ru ? 1 : 0;
    }
    if (y1) {
        // Unfused: y1 = bf16(acc * g^x * g^w1) for all 2I weight rows (the
        // plain epilogue, whose arithmetic per element is the fused one's),
        // then h and its maxima from y1 in a separate kernel.
        GemmParams u = f1;
        u.mtiles = rb.mtiles;
        u.N = (int32_t)(2 * I);
        u.n_tiles_n = col_tiles(2 * I, kGemmPlain);
        u.out = y1;
        u.ld_out = 2 * I;
        e = launch_gemm(kGemmPlain, u, grid_blocks(mt_bound * u.n_tiles_n), s);
        if (e != hipSuccess) return NVFP4_E_HIP;
        const int64_t rb1 = std::min<int64_t>(L.pub.rows_cap, mt_bound * kTileRows);
        e = launch_swiglu_producer(y1, rb1, (int32_t)I, rb.row2pair, rb.row_prob, rb.expert_off, (int32_t)E, f1.out,
                                   f1.amax_part, s);
        if (e != hipSuccess || !mark(2)) return NVFP4_E_HIP;
    } else {
        // FC1: hybrid grid -- two workgroups per CU walk a static bulk of
        // equal tile counts, and the last one to two rounds of tiles go one
        // per workgroup to the rest of the grid, which the hardware
        // dispatcher hands to whichever CU slot frees first.  Measured on the
        // Qwen3-30B-A3B-shaped layer at T = 4096: about 8 us faster than
        // persistent workgroups alone and 2-3 us faster than one workgroup
        // per tile; FC2's shorter tiles (K = I) are fastest persistent.
        // Up to two rounds of tiles (decode-sized batches): one workgroup per
        // tile, with no persistent part.
        const int64_t fc1_tiles = mt_bound * f1.n_tiles_n;
        const bool hybrid = fc1_tiles > 2 * (int64_t)hybrid_persist();
        f1.persist = hybrid ? hybrid_persist() : 0;
        e = launch_gemm(kGemmSwiGLU, f1, hybrid ? hybrid_grid(fc1_tiles) : (int)fc1_tiles, s, online);
        if (e != hipSuccess || !mark(2)) return NVFP4_E_HIP;
    }

    uint8_t* a2c = ws + L.pub.a2_codes;
    uint8_t* a2s = ws + L.pub.a2_scales;
    float* a2g = (float*)(ws + L.pub.a2_g);
    const int64_t rows_bound =
        capacity > 0 ? L.pub.rows_cap
                     : std::min<int64_t>(L.pub.rows_cap, (P + used * (kMAlign - 1) + kMAlign - 1) / kMAlign * kMAlign);
    e = launch_quant_h(f1.out, rows_bound, I, rb.expert_off, (int32_t)E, capacity, rb.expert_count, rb.row2pair,
                       f1.amax_part, f1.n_part, a2c, a2s, a2g, ru, s);
    if (e != hipSuccess || !mark(3)) return NVFP4_E_HIP;

    GemmParams f2{};
    f2.a_codes = a2c;
    f2.a_scales = a2s;
    f2.a_g = a2g;
    f2.b_codes = W2q->codes;
    f2.b_scales = W2q->scales;
    f2.b_g = W2q->g;
    f2.K = (int32_t)I;
    f2.N = (int32_t)H;
    f2.n_tiles_n = col_tiles(H, kGemmPlain);
    f2.mtiles = rb.mtiles;
    f2.n_mtiles = rb.n_mtiles;
    f2.dense_m = -1;
    f2.out = (uint16_t*)(ws + L.pub.y2);
    f2.ld_out = H;
    e = launch_gemm(kGemmPlain, f2, grid_blocks(mt_bound * f2.n_tiles_n), s);
    if (e != hipSuccess || !mark(4)) return NVFP4_E_HIP;

    e = launch_combine(f2.out, rb.pair2row, T, (int32_t)H, (int32_t)K, out, s);
    if (e != hipSuccess || !mark(5)) return NVFP4_E_HIP;
    return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4moe_moe_expert_forward(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T, const int32_t* ids,
                                const float* probs, const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q,
                                uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
    return forward_impl(cfg, x, T, ids, probs, W1q, W2q, out, workspace, workspace_bytes, stream, nullptr);
}

int nvfp4moe_moe_expert_forward_online(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T, const int32_t* ids,
                                       const float* probs, const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q,
                                       uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
    return forward_impl(cfg, x, T, ids, probs, W1q, W2q, out, workspace, workspace_bytes, stream, nullptr, 0, false,
                        nullptr, true);
}

int nvfp4moe_moe_expert_forward_events(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T, const int32_t* ids,
                                       const float* probs, const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q,
                                       uint16_t* out, void* workspace, size_t workspace_bytes, void* const* events,
                                       void* stream) {
    if (!events) return NVFP4_E_NULL;
    for (int i = 0; i < NVFP4MOE_N_STAGE_EVENTS; i++)
        if (!events[i]) return NVFP4_E_NULL;
    return forward_impl(cfg, x, T, ids, probs, W1q, W2q, out, workspace, workspace_bytes, stream, events);
}

int nvfp4moe_moe_expert_forward_masked(const nvfp4moe_config* cfg, int32_t capacity, const uint16_t* x, int32_t T,
                                       const int32_t* ids, const float* probs, const nvfp4_qtensor* W1q,
                                       const nvfp4_qtensor* W2q, uint16_t* out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    if (cfg && cfg_ok(cfg) && !capacity_ok(cfg, capacity)) return NVFP4_E_SHAPE;
    return forward_impl(cfg, x, T, ids, probs, W1q, W2q, out, workspace, workspace_bytes, stream, nullptr, capacity);
}

int nvfp4moe_moe_expert_forward_noalloc(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T, const int32_t* ids,
                                        const float* probs, const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q,
                                        uint16_t* out, int32_t* err_word, void* stream) {
    if (!cfg) return NVFP4_E_NULL;
    if (!cfg_ok(cfg)) return NVFP4_E_SHAPE;
    if (T < 0) return NVFP4_E_SHAPE;
    if (T > cfg->max_tokens) return NVFP4_E_CAPACITY;
    if (err_word && !aligned(err_word, 4)) return NVFP4_E_ALIGN;
    nvfp4moe_config c = *cfg;
    c.max_tokens = T;  // the intermediates of exactly this call
    const Layout L = make_layout(&c);
    if (L.total > kNoAllocScratchBytes) return NVFP4_E_SCRATCH;
    if (T == 0) return NVFP4_OK;
    void* ws = nullptr;
    const int st = noalloc_scratch(&ws);
    if (st != NVFP4_OK) return st;
    const int r = forward_impl(&c, x, T, ids, probs, W1q, W2q, out, ws, kNoAllocScratchBytes, stream, nullptr);
    if (r != NVFP4_OK || !err_word) return r;
    return hip_status(hipMemcpyAsync(err_word, (const uint8_t*)ws + L.pub.err, 4, hipMemcpyDeviceToDevice,
                                     (hipStream_t)stream));
}

int nvfp4moe_moe_expert_forward_unfused(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T, const int32_t* ids,
                                        const float* probs, const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q,
                                        uint16_t* out, uint16_t* y1, int64_t y1_rows, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    if (!cfg) return NVFP4_E_NULL;
    if (!cfg_ok(cfg)) return NVFP4_E_SHAPE;
    if (y1_rows < make_layout(cfg).pub.rows_cap) return NVFP4_E_SHAPE;
    if (T > 0 && !y1) return NVFP4_E_NULL;
    if (y1 && !aligned(y1, 16)) return NVFP4_E_ALIGN;
    return forward_impl(cfg, x, T, ids, probs, W1q, W2q, out, workspace, workspace_bytes, stream, nullptr, 0, false,
                        T > 0 ? y1 : nullptr);
}

size_t nvfp4moe_backward_workspace_bytes(const nvfp4moe_config* cfg) {
    if (!cfg_ok(cfg)) return 0;
    const size_t rows = (size_t)make_layout(cfg).pub.rows_cap;
    const size_t I = cfg->inter, H = cfg->hidden;
    return up(rows * I * 2, kAlign) + up(rows * 2 * I * 2, kAlign) + up(rows * H * 2, kAlign);
}

int nvfp4moe_moe_expert_backward(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T, const uint16_t* w1,
                                 const uint16_t* w2, const uint16_t* y1, int64_t y1_rows, const void* fwd_workspace,
                                 size_t fwd_workspace_bytes, const uint16_t* dout, uint16_t* dx, float* dprobs,
                                 float* dw1, float* dw2, void* workspace, size_t workspace_bytes, void* stream) {
    if (!cfg) return NVFP4_E_NULL;
    if (!cfg_ok(cfg)) return NVFP4_E_SHAPE;
    if (T < 0) return NVFP4_E_SHAPE;
    if (T > cfg->max_tokens) return NVFP4_E_CAPACITY;
    const Layout L = make_layout(cfg);
    if (y1_rows < L.pub.rows_cap) return NVFP4_E_SHAPE;
    if (!fwd_workspace || !workspace) return NVFP4_E_NULL;
    if (fwd_workspace_bytes < L.total || workspace_bytes < nvfp4moe_backward_workspace_bytes(cfg))
        return NVFP4_E_WORKSPACE;
    if (!aligned(fwd_workspace, kAlign) || !aligned(workspace, kAlign)) return NVFP4_E_ALIGN;
    if (T == 0) return NVFP4_OK;
    if (!x || !w1 || !w2 || !y1 || !dout || !dx || !dprobs || !dw1 || !dw2) return NVFP4_E_NULL;
    if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(y1, 16) || !aligned(dout, 16) ||
        !aligned(dx, 16) || !aligned(dprobs, 4) || !aligned(dw1, 4) || !aligned(dw2, 4))
        return NVFP4_E_ALIGN;
    const int64_t E = cfg->n_experts, K = cfg->top_k, H = cfg->hidden, I = cfg->inter;
    const uint8_t* fw = (const uint8_t*)fwd_workspace;
    uint8_t* ws = (uint8_t*)workspace;
    const size_t rows = (size_t)L.pub.rows_cap;
    BwdArgs A{};
    A.T = T;
    A.top_k = (int32_t)K;
    A.E = E;
    A.H = H;
    A.I = I;
    A.x = x;
    A.w1 = w1;
    A.w2 = w2;
    A.y1 = y1;
    A.h = (const uint16_t*)(fw + L.pub.h);
    A.dout = dout;
    A.row2pair = (const int32_t*)(fw + L.pub.row2pair);
    A.pair2row = (const int32_t*)(fw + L.pub.pair2row);
    A.row_prob = (const float*)(fw + L.row_prob);
    A.mtiles = (const int4*)(fw + L.mtiles);
    A.n_mtiles = (const int32_t*)(fw + L.n_mtiles);
    A.expert_off = (const int32_t*)(fw + L.pub.expert_off);
    A.expert_count = (const int32_t*)(fw + L.pub.expert_count);
    const int64_t P = (int64_t)T * K, used = std::min<int64_t>(E, P);
    A.mt_bound = (P + used * (kMAlign - 1)) / kTileRows + used + 1;
    A.rows_bound = std::min<int64_t>((int64_t)rows, (P + used * (kMAlign - 1) + kMAlign - 1) / kMAlign * kMAlign);
    A.dh = (uint16_t*)ws;
    A.dy1 = (uint16_t*)(ws + up(rows * I * 2, kAlign));
    A.dxp = (uint16_t*)(ws + up(rows * I * 2, kAlign) + up(rows * 2 * I * 2, kAlign));
    A.dx = dx;
    A.dprobs = dprobs;
    A.dw1 = dw1;
    A.dw2 = dw2;
    return hip_status(launch_moe_backward(A, (hipStream_t)stream));
}

int nvfp4moe_moe_expert_forward_w4a16(const nvfp4moe_config* cfg, const uint16_t* x, int32_t T, const int32_t* ids,
                                      const float* probs, const nvfp4_qtensor* W1q, const nvfp4_qtensor* W2q,
                                      uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
    return forward_impl(cfg, x, T, ids, probs, W1q, W2q, out, workspace, workspace_bytes, stream, nullptr, 0, true);
}

int nvfp4moe_device_error(const nvfp4moe_config* cfg, const void* workspace, int32_t* code_host, void* stream) {
    if (!cfg || !workspace || !code_host) return NVFP4_E_NULL;
    if (!cfg_ok(cfg)) return NVFP4_E_SHAPE;
    const Layout L = make_layout(cfg);
    hipStream_t s = (hipStream_t)stream;
    int32_t v = 0;
    if (hipMemcpyAsync(&v, (const uint8_t*)workspace + L.pub.err, 4, hipMemcpyDeviceToHost, s) != hipSuccess)
        return NVFP4_E_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return NVFP4_E_HIP;
    *code_host = v;
    return NVFP4_OK;
}

int nvfp4moe_router_topk(const uint16_t* x, int32_t T, int32_t H, const uint16_t* w_router, int32_t E, int32_t K,
                         int32_t renormalize, float* logits, int32_t* ids, float* probs, void* stream) {
    if (T < 0 || H <= 0 || H % 16 != 0 || E < 1 || E > kMaxExperts || K < 1 || K > E || K > kMaxTopK)
        return NVFP4_E_SHAPE;
    if ((int64_t)T * std::max(H, E) >= ((int64_t)1 << 31)) return NVFP4_E_SHAPE;
    if (renormalize != 0 && renormalize != 1) return NVFP4_E_ARG;
    if (T == 0) return NVFP4_OK;
    if (!x || !w_router || !logits || !ids || !probs) return NVFP4_E_NULL;
    if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(logits, 4) || !aligned(ids, 4) || !aligned(probs, 4))
        return NVFP4_E_ALIGN;
    return hip_status(launch_router(x, T, H, w_router, E, K, renormalize != 0, logits, ids, probs,
                                    (hipStream_t)stream));
}

size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t K) {
    if (M < 0 || K <= 0 || K % 128 != 0) return 0;
    const size_t rows = up((size_t)std::max<int64_t>(M, 1), 32);
    return up(rows * K / 2, kAlign) + up(rows * K / 16, kAlign) + up(rows * 4, kAlign);
}

int nvfp4_linear(const uint16_t* x, int64_t M, int64_t K, const nvfp4_qtensor* Wq, uint16_t* out,
                 int32_t scale_round, void* workspace, size_t workspace_bytes, void* stream) {
    if (scale_round != NVFP4_SCALE_RU && scale_round != NVFP4_SCALE_RNE) return NVFP4_E_ARG;
    if (M < 0 || K <= 0 || K % 128 != 0 || M >= ((int64_t)1 << 30)) return NVFP4_E_SHAPE;
    if (!Wq) return NVFP4_E_NULL;
    if (!Wq->codes || !Wq->scales || !Wq->g) return NVFP4_E_NULL;
    if (Wq->n_mats != 1 || Wq->cols != K || Wq->rows <= 0 || Wq->rows % 128 != 0 || Wq->layout != NVFP4_LAYOUT_GEMM)
        return NVFP4_E_SHAPE;
    if (!workspace) return NVFP4_E_NULL;
    if (workspace_bytes < nvfp4_linear_workspace_bytes(M, K)) return NVFP4_E_WORKSPACE;
    if (!aligned(workspace, kAlign)) return NVFP4_E_ALIGN;
    if (M == 0) return NVFP4_OK;
    if (!x || !out) return NVFP4_E_NULL;
    if (!aligned(x, 16) || !aligned(out, 4)) return NVFP4_E_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const size_t rows = up((size_t)M, 32);
    uint8_t* ws = (uint8_t*)workspace;
    uint8_t* xc = ws;
    uint8_t* xs = ws + up(rows * K / 2, kAlign);
    float* xg = (float*)(ws + up(rows * K / 2, kAlign) + up(rows * K / 16, kAlign));
    hipError_t e = launch_quant_rows(x, M, K, K, xc, xs, xg, true, scale_round == NVFP4_SCALE_RU, s);
    if (e != hipSuccess) return NVFP4_E_HIP;
    GemmParams p{};
    p.a_codes = xc;
    p.a_scales = xs;
    p.a_g = xg;
    p.b_codes = Wq->codes;
    p.b_scales = Wq->scales;
    p.b_g = Wq->g;
    p.K = (int32_t)K;
    p.N = Wq->rows;
    p.n_tiles_n = col_tiles(Wq->rows, kGemmPlain);
    p.dense_m = (int32_t)M;
    p.out = out;
    p.ld_out = Wq->rows;
    const int64_t tiles = (M + kTileRows - 1) / kTileRows * p.n_tiles_n;
    return hip_status(launch_gemm(kGemmPlain, p, grid_blocks(tiles), s));
}

}  // extern "C"
