// route.hip -- expert sort with padding and device offsets, fused with the
// amax and quantization of X (miniTE summary page, "how to use it": sort+amax,
// then pad(X, amax), then quantize into the buffer the GEMM reads; expert
// boundaries are device offsets; the metadata is reused by FC1, FC2 and the
// combine).
//
// Four launches (two up to 1024 pairs, see route_small below), all sized
// from T and the config only (no host read-back of counts, article section
// 4.6):
//   route_count   per block of 16 tokens, one wavefront per token: the row
//                 is read once into registers for its amax and quantization
//                 (token-major buffer Xq; skipped for BF16 activations, the
//                 W4A16 variant, which also skips the gather); the block's
//                 (t, k) pairs get stable
//                 per-expert ranks in pair order (wave ballots) and a
//                 per-expert block count; id checks.
//   route_scan    one block: per-expert exclusive prefix over the blocks,
//                 padded expert offsets off[E+1], the GEMM row-tile table,
//                 padding rows marked, error word.
//   route_place   per pair: sorted row = off[e] + block prefix + rank.
//   route_gather  per (32-row tile, up to 256 columns): builds the padded,
//                 sorted GEMM-layout buffer from Xq, writing whole 1 KiB
//                 chunks; padding rows are written as zeros.
// Small batches (T*K <= 1024 pairs, T <= 128, E <= 256: decode sizes) take
// one launch, route_small, for what route_count, route_scan and route_place
// do: its first workgroup ranks the pairs in groups of 64, adds the groups'
// counts up per expert and places every pair, with the same ranks, offsets,
// tables and error bits, while the other workgroups quantize X.
// Integer atomics only on LDS counters: every count and row index is
// independent of scheduling.
//
// Two row layouts (article section 4.4, "two layouts, same row results"):
// contiguous (capacity 0), where expert e's rows start at the padded prefix
// of the counts before it, and masked, where every expert owns a fixed chunk
// of `capacity` rows starting at e * capacity and the chunk's rows past the
// expert's padded count are never touched.  A row's content does not depend
// on where it sits, so both give the same bits per (token, slot).  Pairs
// ranked past the capacity of their expert get no row and raise bit 4 of the
// error word.
#include <algorithm>

#include "nvfp4_device.h"
#include "nvfp4_kernels.h"
#include "nvfp4_quant_row.h"

namespace nvfp4 {

constexpr int kCountThreads = kTokPerBlk * 64;  // one wavefront per token of the block
constexpr int kRouteWaitLgkm0 = 0xC07F;         // s_waitcnt lgkmcnt(0)

// What route_count does with X besides the sort: nothing (BF16 activations,
// the W4A16 variant), quantize each token row (token-major Xq, g in gx), or
// only its max |x| into gx (the forward that quantizes X inside FC1).
constexpr int kXNone = 0, kXQuant = 1, kXAmax = 2;

template <int XM>
__global__ void __launch_bounds__(kCountThreads) route_count_kernel(const uint16_t* __restrict__ x,
                                                                    const int32_t* __restrict__ ids, int32_t T,
                                                                    int32_t H, int32_t K, int32_t E, int round_up,
                                                                    int quant_x,
                                                                    int32_t* __restrict__ blk_counts,
                                                                    int32_t* __restrict__ blk_err,
                                                                    int32_t* __restrict__ lrank,
                                                                    uint8_t* __restrict__ xq_codes,
                                                                    uint8_t* __restrict__ xq_scales,
                                                                    float* __restrict__ gx) {
    __shared__ int32_t cnt[kMaxExperts];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * kTokPerBlk;
    for (int e = tid; e < E; e += kCountThreads) cnt[e] = 0;
    // Wave 0 ranks the block's pairs.  It loads their expert ids before its
    // own token row, so that the row's loads are in flight while it ranks
    // (a wave's loads return in order).
    constexpr int kGroups = kTokPerBlk * kMaxTopK / kWave;  // groups of 64 pairs a block can hold
    const int64_t p0 = t0 * K, p1 = min((t0 + kTokPerBlk) * K, (int64_t)T * K);
    __syncthreads();
    int32_t eg[kGroups];
    if (wave == 0) {
#pragma unroll
        for (int g = 0; g < kGroups; g++) {
            const int64_t p = p0 + (int64_t)g * kWave + lane;
            eg[g] = p < p1 ? ids[p] : -1;
        }
    }
    auto rank = [&]() {
        if (wave != 0) return;
        // Stable ranks in pair order: pairs are taken 64 at a time; lanes with
        // the same expert find each other with one ballot per id bit.
        int nbits = 0;
        while ((1 << nbits) < E) nbits++;
        int err = 0;
#pragma unroll
        for (int g = 0; g < kGroups; g++) {
            const int64_t c0 = p0 + (int64_t)g * kWave;
            if (c0 >= p1) break;
            const int64_t p = c0 + lane;
            const int32_t e = eg[g];
            const bool valid = e >= 0 && e < E;
            if (p < p1 && !valid) err |= 1;
            // A token may not name an expert twice: compare with the token's
            // earlier slots, taken from the lanes that hold them (in the
            // previous group when the token began there; a block starts at a
            // token, so group 0 never looks back).
            const int kk = (int)((uint32_t)p % (uint32_t)K);  // pair indices are < 2^30
            for (int d = 1; d < K; d++) {
                const int32_t ed = __shfl(e, max(lane - d, 0), kWave);
                const int32_t ep = __shfl(eg[g > 0 ? g - 1 : 0], (lane - d + kWave) & (kWave - 1), kWave);
                if (valid && d <= kk) {
                    const int32_t prev = lane >= d ? ed : ep;
                    if (prev == e) err |= 2;
                }
            }
            uint64_t mask = __ballot(valid);
            for (int b = 0; b < nbits; b++) {
                const bool bit = valid && ((e >> b) & 1);
                const uint64_t m1 = __ballot(bit);
                mask &= bit ? m1 : ~m1;
            }
            const uint64_t below = mask & ((1ull << lane) - 1ull);
            int32_t rank = -1;
            if (valid) rank = cnt[e] + __popcll(below);
            __builtin_amdgcn_s_waitcnt(kRouteWaitLgkm0);  // every lane's read of cnt[] precedes the leaders' updates
            __builtin_amdgcn_wave_barrier();
            if (valid && below == 0ull) cnt[e] += __popcll(mask);
            if (p < p1) lrank[p] = rank;
        }
        // OR the lanes' error bits
        for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, kWave);
        if (lane == 0) blk_err[blockIdx.x] = err;
    };
    // Each wave quantizes its token's row once (amax in the same pass).  The
    // row's loads are issued without a branch (a wave past the last token
    // loads the last row and stores nothing), so the rank's waits for the ids
    // count in order past them instead of waiting for everything.
    const int64_t t = t0 + wave;
    const bool qx = XM != kXNone && t < T;
    int64_t groups_per_lane = (H / 32 + kWave - 1) / kWave;
    const uint16_t* xr = x + (t < T ? t : T - 1) * H;
    const bool ru = round_up != 0;
    if (XM == kXNone) {
        rank();
        groups_per_lane = 0;  // nothing to read
    }
    switch (groups_per_lane) {
        case 0: break;
#define NVFP4_ROUTE_COUNT_CASE(G)                                                 \
    case G: {                                                                     \
        RowRegs<G> rr;                                                            \
        row_load<G>(xr, H, rr);                                                   \
        rank();                                                                   \
        if (XM == kXQuant && qx) row_quant<G>(rr, H, ru, false, t, xq_codes, xq_scales, gx); \
        if (XM == kXAmax) {                                                       \
            const float am = row_amax<G>(rr, H);                                  \
            if (qx && lane == 0) gx[t] = am;                                      \
        }                                                                         \
        break;                                                                    \
    }
        NVFP4_ROUTE_COUNT_CASE(1)
        NVFP4_ROUTE_COUNT_CASE(2)
        NVFP4_ROUTE_COUNT_CASE(3)
        NVFP4_ROUTE_COUNT_CASE(4)
#undef NVFP4_ROUTE_COUNT_CASE
        default:
            rank();
            if (XM == kXQuant && qx) quant_row_wave(xr, H, -1.0f, ru, false, t, xq_codes, xq_scales, gx);
            if (XM == kXAmax) {
                const float am = row_amax_wave(xr, H);
                if (qx && lane == 0) gx[t] = am;
            }
            break;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kCountThreads) blk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Block-wide inclusive scan of two ints per thread (1024 threads = 16 waves):
// shuffles within each wave, then one wave scans the 16 wave totals.
__device__ int2 block_scan_incl2(int2 v, int2* wsum /* [16] */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int nx = __shfl_up(v.x, o, kWave), ny = __shfl_up(v.y, o, kWave);
        if (lane >= o) {
            v.x += nx;
            v.y += ny;
        }
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int2 w = lane < 16 ? wsum[lane] : make_int2(0, 0);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int nx = __shfl_up(w.x, o, kWave), ny = __shfl_up(w.y, o, kWave);
            if (lane >= o) {
                w.x += nx;
                w.y += ny;
            }
        }
        if (lane < 16) wsum[lane] = w;
    }
    __syncthreads();
    if (wave > 0) {
        const int2 b = wsum[wave - 1];
        v.x += b.x;
        v.y += b.y;
    }
    return v;
}

constexpr int kScanRegs = 32;  // block counts a scan thread keeps in registers

__global__ void __launch_bounds__(1024) route_scan_kernel(int32_t nblk, int32_t E, int32_t capacity,
                                                          int32_t* __restrict__ blk_counts,
                                                          const int32_t* __restrict__ blk_err,
                                                          int32_t* __restrict__ expert_count,
                                                          int32_t* __restrict__ expert_off,
                                                          int4* __restrict__ mtiles, int4* __restrict__ mtiles_even,
                                                          int32_t* __restrict__ n_mtiles,
                                                          int32_t* __restrict__ row2pair, int32_t* __restrict__ err_word) {
    __shared__ int32_t part[1024];
    __shared__ int2 wsum[16];
    __shared__ int32_t errs;
    const int tid = threadIdx.x;
    if (tid == 0) errs = 0;
    // (1) per-expert exclusive prefix over blocks: tpe threads per expert, each
    //     owning a contiguous segment of blocks.  Segments of up to kScanRegs
    //     blocks are read once into registers with all loads in flight.
    const int tpe = 1024 / E;  // >= 1 since E <= 1024
    const int e1 = tid % E, sub = tid / E;  // consecutive lanes read consecutive experts (coalesced)
    // (threads with sub >= tpe own no segment)
    const int seg = (nblk + tpe - 1) / tpe;
    const int b0 = min(sub * seg, nblk), b1 = sub < tpe ? min(b0 + seg, nblk) : b0;
    const bool in_regs = seg <= kScanRegs;
    int32_t v[kScanRegs];
    int32_t sum = 0;
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < kScanRegs; j++) v[j] = b0 + j < b1 ? blk_counts[(int64_t)(b0 + j) * E + e1] : 0;
#pragma unroll
        for (int j = 0; j < kScanRegs; j++) sum += v[j];
    } else {
        for (int b = b0; b < b1; b++) sum += blk_counts[(int64_t)b * E + e1];
    }
    if (sub < tpe) part[e1 * tpe + sub] = sum;
    int my_err = 0;
    for (int b = tid; b < nblk; b += 1024) my_err |= blk_err[b];
    if (my_err) atomicOr(&errs, my_err);
    __syncthreads();
    if (sub < tpe) {
        int32_t run = 0;
        for (int s = 0; s < sub; s++) run += part[e1 * tpe + s];
        if (in_regs) {
#pragma unroll
            for (int j = 0; j < kScanRegs; j++) {
                if (b0 + j < b1) blk_counts[(int64_t)(b0 + j) * E + e1] = run;  // the block's first rank within e1
                run += v[j];
            }
        } else {
            for (int b = b0; b < b1; b++) {
                const int32_t c = blk_counts[(int64_t)b * E + e1];
                blk_counts[(int64_t)b * E + e1] = run;
                run += c;
            }
        }
    }
    // (2) totals, padded offsets and row-tile counts per expert (thread e);
    //     in the masked layout an expert keeps at most `capacity` rows.
    int32_t cnt = 0, kept = 0, padded = 0, ntile = 0;
    if (tid < E) {
        for (int s = 0; s < tpe; s++) cnt += part[tid * tpe + s];
        kept = capacity > 0 ? min(cnt, capacity) : cnt;
        padded = (kept + kMAlign - 1) / kMAlign * kMAlign;
        ntile = (padded + kTileRows - 1) / kTileRows;
        if (kept < cnt) atomicOr(&errs, 4);
    }
    const int2 incl = block_scan_incl2(make_int2(padded, ntile), wsum);
    if (tid < E) {
        const int32_t off = capacity > 0 ? tid * capacity : incl.x - padded;
        const int32_t t0 = incl.y - ntile;
        expert_count[tid] = cnt;
        expert_off[tid] = off;
        if (tid == E - 1) {
            expert_off[E] = capacity > 0 ? E * capacity : incl.x;
            *n_mtiles = incl.y;
        }
        // Two tables of the same row tiles: full 4-subtile tiles with the
        // remainder last (9 subtiles: 4 + 4 + 1), and the expert's subtiles
        // spread evenly (3 + 3 + 3).  A tile's weight streaming and decoding
        // cost the same for any number of subtiles, so FC1 (K = H, long
        // tiles) runs faster on the even split and FC2 (K = I) on the first.
        const int32_t nsub_all = padded / kMAlign;
        const int32_t base = ntile > 0 ? nsub_all / ntile : 0, extra = ntile > 0 ? nsub_all % ntile : 0;
        int32_t r0e = off;
        for (int i = 0; i < ntile; i++) {
            const int32_t r0 = off + i * kTileRows;
            const int32_t nsub = min(kTileRows, padded - i * kTileRows) / kMAlign;
            mtiles[t0 + i] = make_int4(r0, tid, nsub, off + kept);
            const int32_t nsub_e = base + (i < extra ? 1 : 0);
            mtiles_even[t0 + i] = make_int4(r0e, tid, nsub_e, off + kept);
            r0e += nsub_e * kMAlign;
        }
        for (int r = off + kept; r < off + padded; r++) row2pair[r] = -1;
    }
    __syncthreads();  // every expert's overflow bit is in
    if (tid == 0) *err_word = errs;
}

constexpr int kSmallPairs = 1024;  // pairs a single-workgroup sort takes (16 groups of 64)
constexpr int kSmallExperts = 256;
constexpr int kSmallTokens = 128;
constexpr int kSmallWaves = 8;     // wavefront w takes the pair groups w and w + 8

// The same per-row outputs as route_count + route_scan + route_place for
// T*K <= kSmallPairs, T <= kSmallTokens and E <= kSmallExperts, in one
// workgroup of 512 threads: group g of 64 pairs, [64 g, 64 g + 64), is ranked
// by wavefront g % 8 (stable, pair order, by one ballot per id bit) and
// counted per expert; thread e adds the 16 groups' counts up in group order
// (a pair's rank = its group's prefix + its rank in the group: the same rank
// as the block-wise path); the padded offsets and row-tile tables follow as
// in route_scan.  Workgroups 1, 2, ... quantize the token rows, one per
// wavefront (row 8 (b - 1) + w), once each.
__global__ void __launch_bounds__(kSmallWaves * 64) route_small_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ ids,
                                                           const float* __restrict__ probs, int32_t T, int32_t H,
                                                           int32_t K, int32_t E, int32_t capacity, int round_up,
                                                           RouteBuffers rb) {
    __shared__ int32_t gcnt[16][kSmallExperts];  // per group, then the group's exclusive prefix
    __shared__ int32_t soff[kSmallExperts];
    __shared__ int32_t pe[kSmallPairs], prank[kSmallPairs];  // each pair's expert and rank in its group
    __shared__ int2 wsum[16];
    __shared__ int32_t errs;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (blockIdx.x > 0) {
        // Each wave quantizes its token row once (amax in the same pass).
        const int64_t t = (int64_t)(blockIdx.x - 1) * kSmallWaves + wave;
        if (t >= T) return;
        const int64_t groups_per_lane = (H / 32 + kWave - 1) / kWave;
        const bool ru = round_up != 0;
        const uint16_t* xr = x + t * H;
        switch (groups_per_lane) {
            case 1: quant_row_regs<1>(xr, H, ru, false, t, rb.xq_codes, rb.xq_scales, rb.gx); break;
            case 2: quant_row_regs<2>(xr, H, ru, false, t, rb.xq_codes, rb.xq_scales, rb.gx); break;
            case 3: quant_row_regs<3>(xr, H, ru, false, t, rb.xq_codes, rb.xq_scales, rb.gx); break;
            case 4: quant_row_regs<4>(xr, H, ru, false, t, rb.xq_codes, rb.xq_scales, rb.gx); break;
            default: quant_row_wave(xr, H, -1.0f, ru, false, t, rb.xq_codes, rb.xq_scales, rb.gx); break;
        }
        return;
    }
    const int64_t P = (int64_t)T * K;
    if (tid == 0) errs = 0;
    if (tid < 16) wsum[tid] = make_int2(0, 0);
    for (int i = tid; i < 16 * kSmallExperts; i += kSmallWaves * 64) (&gcnt[0][0])[i] = 0;
    __syncthreads();
    // (1) ranks within each group of 64 pairs, id checks
    int err = 0;
    int nbits = 0;
    while ((1 << nbits) < E) nbits++;
    for (int g = wave; g < 16; g += kSmallWaves) {
        const int64_t p = (int64_t)g * kWave + lane;
        const int32_t e = p < P ? ids[p] : -1;
        const bool valid = e >= 0 && e < E;
        if (p < P && !valid) err |= 1;
        // A token may not name an expert twice: compare with its earlier slots,
        // from the lanes that hold them (or memory across a group boundary).
        const int kk = (int)((uint32_t)p % (uint32_t)K);
        for (int d = 1; d < K; d++) {
            const int32_t ed = __shfl(e, max(lane - d, 0), kWave);
            if (valid && d <= kk) {
                const int32_t prev = lane >= d ? ed : ids[p - d];
                if (prev == e) err |= 2;
            }
        }
        uint64_t mask = __ballot(valid);
        for (int b = 0; b < nbits; b++) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t m1 = __ballot(bit);
            mask &= bit ? m1 : ~m1;
        }
        const uint64_t below = mask & ((1ull << lane) - 1ull);
        pe[p] = valid ? e : -1;
        prank[p] = (int32_t)__popcll(below);
        if (valid && below == 0ull) gcnt[g][e] = (int32_t)__popcll(mask);
    }
    for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, kWave);
    if (lane == 0 && err) atomicOr(&errs, err);
    __syncthreads();
    // (2) per expert: the groups' exclusive prefix, the total, the padded
    //     offset and row tiles (as route_scan)
    int32_t cnt = 0, kept = 0, padded = 0, ntile = 0;
    if (tid < E) {
        for (int g = 0; g < 16; g++) {
            const int32_t c = gcnt[g][tid];
            gcnt[g][tid] = cnt;
            cnt += c;
        }
        kept = capacity > 0 ? min(cnt, capacity) : cnt;
        padded = (kept + kMAlign - 1) / kMAlign * kMAlign;
        ntile = (padded + kTileRows - 1) / kTileRows;
        if (kept < cnt) atomicOr(&errs, 4);
    }
    const int2 incl = block_scan_incl2(make_int2(padded, ntile), wsum);
    if (tid < E) {
        const int32_t off = capacity > 0 ? tid * capacity : incl.x - padded;
        const int32_t t0 = incl.y - ntile;
        soff[tid] = off;
        rb.expert_count[tid] = cnt;
        rb.expert_off[tid] = off;
        if (tid == E - 1) {
            rb.expert_off[E] = capacity > 0 ? E * capacity : incl.x;
            *rb.n_mtiles = incl.y;
        }
        const int32_t nsub_all = padded / kMAlign;
        const int32_t base = ntile > 0 ? nsub_all / ntile : 0, extra = ntile > 0 ? nsub_all % ntile : 0;
        int32_t r0e = off;
        for (int i = 0; i < ntile; i++) {
            const int32_t r0 = off + i * kTileRows;
            const int32_t nsub = min(kTileRows, padded - i * kTileRows) / kMAlign;
            rb.mtiles[t0 + i] = make_int4(r0, tid, nsub, off + kept);
            const int32_t nsub_e = base + (i < extra ? 1 : 0);
            rb.mtiles_even[t0 + i] = make_int4(r0e, tid, nsub_e, off + kept);
            r0e += nsub_e * kMAlign;
        }
        for (int r = off + kept; r < off + padded; r++) rb.row2pair[r] = -1;
    }
    __syncthreads();
    // (3) placement (as route_place)
    for (int64_t p = tid; p < P; p += kSmallWaves * 64) {
        const int32_t ep = pe[p];
        if (ep < 0) {
            rb.pair2row[p] = -1;
        } else {
            const int32_t local = gcnt[p / kWave][ep] + prank[p];
            if (capacity > 0 && local >= capacity) {
                rb.pair2row[p] = -1;
            } else {
                const int32_t row = soff[ep] + local;
                rb.pair2row[p] = row;
                rb.row2pair[row] = (int32_t)p;
                rb.row_prob[row] = probs[p];
            }
        }
    }
    if (tid == 0) *rb.err_word = errs;
}

// pair2row[p] holds the pair's rank within (its block, its expert) on entry
// and its sorted row on exit.
// tok_amax non-null (the forward that quantizes X inside FC1): each placed
// row also gets its token's outer scale g = max|x| / 2688 in row_g.
__global__ void __launch_bounds__(256) route_place_kernel(const int32_t* __restrict__ ids,
                                                          const float* __restrict__ probs, int64_t P, int32_t K,
                                                          int32_t E, int32_t capacity, const int32_t* __restrict__ blk_base,
                                                          const int32_t* __restrict__ expert_off, int32_t* pair2row,
                                                          int32_t* __restrict__ row2pair, float* __restrict__ row_prob,
                                                          const float* __restrict__ tok_amax, float* __restrict__ row_g) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    const int32_t e = ids[p];
    if (e < 0 || e >= E) {  // reported by the error word; the pair gets no row
        pair2row[p] = -1;
        return;
    }
    const int64_t blk = ((uint32_t)p / (uint32_t)K) / kTokPerBlk;  // pair indices are < 2^30
    const int32_t local = blk_base[blk * E + e] + pair2row[p];  // rank within the expert
    if (capacity > 0 && local >= capacity) {  // past the expert's chunk (error bit 4)
        pair2row[p] = -1;
        return;
    }
    const int32_t row = expert_off[e] + local;
    pair2row[p] = row;
    row2pair[row] = (int32_t)p;
    row_prob[row] = probs[p];
    if (tok_amax) row_g[row] = row_scale(tok_amax[(uint32_t)p / (uint32_t)K]).g;
}

constexpr int kGatherSteps = 2;  // 128-column steps per gather wave (one 128-byte line of a row's codes)

// One wave per (32-row tile, two 128-column steps) of the sorted buffer.
// Codes: the two steps' codes of a row are 128 contiguous bytes of its
// token's quantized row, so eight lanes read one row's line (lane l: row
// 8j + l/8, bytes 16 (l % 8)) and each lane stores its 16 bytes straight into
// its GEMM-layout slot -- for a fixed chunk and half, eight consecutive rows
// are 128 contiguous bytes there, so stores are whole lines too.  Scales:
// lane (h, r) reads row r's 8 scale bytes of each step and keeps its GEMM
// word (bytes 2h, 2h+1, 4+2h, 5+2h).  Padding rows are written as zeros;
// every load is in bounds (padding rows read token 0, a step past the end
// re-reads the last one).
__global__ void __launch_bounds__(256) route_gather_kernel(int32_t H, int32_t K, const int32_t* __restrict__ expert_off,
                                                           int32_t E, int32_t capacity,
                                                           const int32_t* __restrict__ expert_count,
                                                           const int32_t* __restrict__ row2pair,
                                                           const uint8_t* __restrict__ xq_codes,
                                                           const uint8_t* __restrict__ xq_scales,
                                                           const float* __restrict__ gx, int64_t n_row_tiles,
                                                           uint8_t* __restrict__ a_codes,
                                                           uint8_t* __restrict__ a_scales, float* __restrict__ a_g) {
    // Block: four 32-row tiles (one per wave) x one group of kGatherSteps
    // 128-column steps; the groups of a quad run together on one XCD
    // (xcd_quad_group), so its rows' pairs and token rows are fetched once.
    const int lane = threadIdx.x & 63;
    const int64_t cps = H / 128;
    int64_t quad, grp;
    if (!xcd_quad_group((n_row_tiles + 3) / 4, (cps + kGatherSteps - 1) / kGatherSteps, quad, grp)) return;
    const int64_t rt = quad * 4 + (threadIdx.x >> 6);
    if (rt >= n_row_tiles) return;
    const int64_t cp0 = grp * kGatherSteps;
    const int q = lane & 7, step = q >> 2, ch = (q >> 1) & 1, hq = q & 1;  // this lane's 16-byte piece
    const int hs = lane >> 5, rs = lane & 31;                              // this lane's scale word
    int32_t pc[4];
#pragma unroll
    for (int j = 0; j < 4; j++) pc[j] = row2pair[rt * 32 + 8 * j + (lane >> 3)];
    const int32_t ps = row2pair[rt * 32 + rs];
    if (!row_tile_used(rt, E, capacity, expert_off, expert_count)) return;
    const int64_t cpq = min(cp0 + step, cps - 1);
    u32x4 c[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int64_t t = pc[j] >= 0 ? (uint32_t)pc[j] / (uint32_t)K : 0;
        c[j] = *reinterpret_cast<const u32x4*>(xq_codes + t * (H / 2) + cpq * 64 + ch * 32 + hq * 16);
    }
    const int64_t ts = ps >= 0 ? (uint32_t)ps / (uint32_t)K : 0;
    const uint8_t* ss = xq_scales + ts * (H / 16);
    const u32x2 w0 = *reinterpret_cast<const u32x2*>(ss + min(cp0, cps - 1) * 8);
    const u32x2 w1 = *reinterpret_cast<const u32x2*>(ss + min(cp0 + 1, cps - 1) * 8);
    const float gt = gx[ts];
    const uint32_t sel = hs ? 0x07060302u : 0x05040100u;
    if (cp0 + step < cps) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int r = 8 * j + (lane >> 3);
            const u32x4 v = pc[j] >= 0 ? c[j] : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(a_codes + (rt * (H / 64) + 2 * (cp0 + step) + ch) * 1024 + (hq * 32 + r) * 16) = v;
        }
    }
#pragma unroll
    for (int st = 0; st < kGatherSteps; st++) {
        if (cp0 + st < cps) {
            const u32x2 w = st ? w1 : w0;
            const uint32_t word = ps >= 0 ? __builtin_amdgcn_perm(w[1], w[0], sel) : 0u;
            *reinterpret_cast<uint32_t*>(a_scales + (rt * (H / 128) + cp0 + st) * 256 + lane * 4) = word;
        }
    }
    if (cp0 == 0 && hs == 0) a_g[rt * 32 + rs] = ps >= 0 ? gt : 0.0f;
}

hipError_t launch_route(const uint16_t* x, const int32_t* ids, const float* probs, int32_t T, int32_t H, int32_t K,
                        int32_t E, int32_t capacity, bool round_up, const RouteBuffers& rb, int64_t rows_cap,
                        hipStream_t stream, bool quant_x, bool online) {
    const int64_t P = (int64_t)T * K;
    hipError_t st;
    if (online) quant_x = false;  // X is quantized inside FC1; the sort records each token's max |x|
    if (!online && P <= kSmallPairs && T <= kSmallTokens && E <= kSmallExperts) {
        // workgroup 0 sorts; with X to quantize, workgroups 1.. take 8 rows each
        const unsigned qblocks = quant_x ? (unsigned)((T + kSmallWaves - 1) / kSmallWaves) : 0u;
        hipLaunchKernelGGL(route_small_kernel, dim3(1 + qblocks), dim3(kSmallWaves * 64), 0, stream, x, ids, probs, T,
                           H, K, E, capacity, round_up ? 1 : 0, rb);
        st = hipGetLastError();
        if (st != hipSuccess) return st;
    } else {
    const int32_t nblk = (T + kTokPerBlk - 1) / kTokPerBlk;
    hipLaunchKernelGGL(online ? route_count_kernel<kXAmax> : quant_x ? route_count_kernel<kXQuant>
                                                                     : route_count_kernel<kXNone>,
                       dim3(nblk), dim3(kCountThreads), 0, stream, x, ids, T, H, K, E, round_up ? 1 : 0,
                       quant_x ? 1 : 0, rb.blk_counts, rb.blk_err, rb.pair2row /* holds the ranks until route_place */,
                       rb.xq_codes, rb.xq_scales, rb.gx);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, nblk, E, capacity, rb.blk_counts, rb.blk_err,
                       rb.expert_count, rb.expert_off, rb.mtiles, rb.mtiles_even, rb.n_mtiles, rb.row2pair,
                       rb.err_word);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
    hipLaunchKernelGGL(route_place_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, stream, ids, probs, P, K, E,
                       capacity, rb.blk_counts, rb.expert_off, rb.pair2row, rb.row2pair, rb.row_prob,
                       online ? rb.gx : nullptr, rb.a_g);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
    }
    if (!quant_x) return hipGetLastError();  // no quantized, sorted copy of X to build
    // Row tiles that can hold rows for this T (the device offsets decide
    // which are used): at most min(E, P) experts receive pairs, each padded
    // by at most kMAlign - 1 rows.
    const int64_t used = std::min<int64_t>(E, P);
    const int64_t rows_bound =
        capacity > 0 ? rows_cap : std::min<int64_t>(rows_cap, (P + used * (kMAlign - 1) + 31) / 32 * 32);
    const int64_t n_row_tiles = rows_bound / 32, groups = (H / 128 + kGatherSteps - 1) / kGatherSteps;
    hipLaunchKernelGGL(route_gather_kernel, dim3(xcd_quad_group_blocks((n_row_tiles + 3) / 4, groups)), dim3(256), 0,
                       stream, H, K, rb.expert_off, E, capacity, rb.expert_count, rb.row2pair, rb.xq_codes, rb.xq_scales,
                       rb.gx, n_row_tiles, rb.a_codes, rb.a_scales, rb.a_g);
    return hipGetLastError();
}

}  // namespace nvfp4
