// route.hip -- expert sort with padding and device offsets, fused with the
// amax and quantization of X (miniTE summary page, "how to use it": sort+amax,
// then pad(X, amax), then quantize into the buffer the GEMM reads; expert
// boundaries are device offsets; the metadata is reused by FC1, FC2 and the
// combine).
//
// Four launches, all sized from T and the config only (no host read-back of
// counts, article section 4.6):
//   route_count   per block of 16 tokens: one pass over each token row takes
//                 its amax and quantizes it once (token-major buffer Xq);
//                 the block's (t, k) pairs get stable per-expert ranks in pair
//                 order (wave ballots) and a per-expert block count; id checks.
//   route_scan    one block: per-expert exclusive prefix over the blocks,
//                 padded expert offsets off[E+1], the GEMM row-tile table,
//                 padding rows marked, error word.
//   route_place   per pair: sorted row = off[e] + block prefix + rank.
//   route_gather  per (32-row tile, 128 columns): builds the padded, sorted
//                 GEMM-layout buffer from Xq, writing whole 1 KiB chunks;
//                 padding rows are written as zeros.
// Integer atomics only on LDS counters: every count and row index is
// independent of scheduling.
#include <algorithm>

#include "nvfp4_device.h"
#include "nvfp4_kernels.h"
#include "nvfp4_quant_row.h"

namespace nvfp4 {

__global__ void __launch_bounds__(256) route_count_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
                                                          int32_t T, int32_t H, int32_t K, int32_t E, int round_up,
                                                          int32_t* __restrict__ blk_counts,
                                                          int32_t* __restrict__ blk_err, int32_t* __restrict__ lrank,
                                                          uint8_t* __restrict__ xq_codes,
                                                          uint8_t* __restrict__ xq_scales, float* __restrict__ gx) {
    __shared__ int32_t cnt[kMaxExperts];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * kTokPerBlk;
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    if (wave == 0) {
        // Stable ranks in pair order: pairs are taken 64 at a time; lanes with
        // the same expert find each other with one ballot per id bit.
        const int64_t p0 = t0 * K, p1 = min((t0 + kTokPerBlk) * K, (int64_t)T * K);
        int nbits = 0;
        while ((1 << nbits) < E) nbits++;
        int err = 0;
        for (int64_t c0 = p0; c0 < p1; c0 += kWave) {
            const int64_t p = c0 + lane;
            const int32_t e = p < p1 ? ids[p] : -1;
            const bool valid = e >= 0 && e < E;
            if (p < p1 && !valid) err |= 1;
            if (valid) {
                const int64_t t = p / K;
                for (int64_t q = t * K; q < p; q++)
                    if (ids[q] == e) err |= 2;
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
            __builtin_amdgcn_s_waitcnt(0);  // every lane's read of cnt[] precedes the leaders' updates
            __builtin_amdgcn_wave_barrier();
            if (valid && below == 0ull) cnt[e] += __popcll(mask);
            if (p < p1) lrank[p] = rank;
        }
        // OR the lanes' error bits
        for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, kWave);
        if (lane == 0) blk_err[blockIdx.x] = err;
    }
    // Each wave quantizes whole token rows once (amax in the same pass).
    for (int64_t t = t0 + wave; t < min(t0 + kTokPerBlk, (int64_t)T); t += 4)
        quant_row_wave(x + t * H, H, -1.0f, round_up != 0, false, t, xq_codes, xq_scales, gx);
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) blk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Block-wide inclusive scan of one int per thread (1024 threads).
__device__ int32_t block_scan_incl(int32_t v, int32_t* buf) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        int32_t add = tid >= o ? buf[tid - o] : 0;
        __syncthreads();
        buf[tid] += add;
        __syncthreads();
    }
    int32_t r = buf[tid];
    __syncthreads();
    return r;
}

__global__ void __launch_bounds__(1024) route_scan_kernel(int32_t nblk, int32_t E, int32_t* __restrict__ blk_counts,
                                                          const int32_t* __restrict__ blk_err,
                                                          int32_t* __restrict__ expert_count,
                                                          int32_t* __restrict__ expert_off,
                                                          int4* __restrict__ mtiles, int32_t* __restrict__ n_mtiles,
                                                          int32_t* __restrict__ row2pair, int32_t* __restrict__ err_word) {
    __shared__ int32_t part[1024];
    __shared__ int32_t scan_buf[1024];
    __shared__ int32_t errs;
    const int tid = threadIdx.x;
    if (tid == 0) errs = 0;
    // (1) per-expert exclusive prefix over blocks: tpe threads per expert, each
    //     owning a contiguous segment of blocks; loads issued 8 at a time.
    const int tpe = 1024 / E;  // >= 1 since E <= 1024
    const int e1 = tid % E, sub = tid / E;  // consecutive lanes read consecutive experts (coalesced)
    // (threads with sub >= tpe own no segment)
    const int seg = (nblk + tpe - 1) / tpe;
    const int b0 = min(sub * seg, nblk), b1 = sub < tpe ? min(b0 + seg, nblk) : b0;
    int32_t sum = 0;
    if (sub < tpe) {
        int b = b0;
        for (; b + 8 <= b1; b += 8) {
            int32_t v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = blk_counts[(int64_t)(b + j) * E + e1];
#pragma unroll
            for (int j = 0; j < 8; j++) sum += v[j];
        }
        for (; b < b1; b++) sum += blk_counts[(int64_t)b * E + e1];
    }
    if (sub < tpe) part[e1 * tpe + sub] = sum;
    int my_err = 0;
    for (int b = tid; b < nblk; b += 1024) my_err |= blk_err[b];
    if (my_err) atomicOr(&errs, my_err);
    __syncthreads();
    if (sub < tpe) {
        int32_t run = 0;
        for (int s = 0; s < sub; s++) run += part[e1 * tpe + s];
        int b = b0;
        for (; b + 8 <= b1; b += 8) {
            int32_t v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = blk_counts[(int64_t)(b + j) * E + e1];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                blk_counts[(int64_t)(b + j) * E + e1] = run;  // this block's first rank within expert e1
                run += v[j];
            }
        }
        for (; b < b1; b++) {
            const int32_t c = blk_counts[(int64_t)b * E + e1];
            blk_counts[(int64_t)b * E + e1] = run;
            run += c;
        }
    }
    __syncthreads();
    // (2) totals, padded offsets and row-tile counts per expert (thread e).
    int32_t cnt = 0, padded = 0, ntile = 0;
    if (tid < E) {
        for (int s = 0; s < tpe; s++) cnt += part[tid * tpe + s];
        padded = (cnt + kMAlign - 1) / kMAlign * kMAlign;
        ntile = (padded + kTileRows - 1) / kTileRows;
    }
    const int32_t off_incl = block_scan_incl(padded, scan_buf);
    const int32_t tile_incl = block_scan_incl(ntile, scan_buf);
    if (tid < E) {
        const int32_t off = off_incl - padded;
        const int32_t t0 = tile_incl - ntile;
        expert_count[tid] = cnt;
        expert_off[tid] = off;
        if (tid == E - 1) {
            expert_off[E] = off_incl;
            *n_mtiles = tile_incl;
            *err_word = errs;
        }
        for (int i = 0; i < ntile; i++) {
            const int32_t r0 = off + i * kTileRows;
            const int32_t nsub = min(kTileRows, padded - i * kTileRows) / kMAlign;
            mtiles[t0 + i] = make_int4(r0, tid, nsub, off + cnt);
        }
        for (int r = off + cnt; r < off + padded; r++) row2pair[r] = -1;
    }
}

// pair2row[p] holds the pair's rank within (its block, its expert) on entry
// and its sorted row on exit.
__global__ void __launch_bounds__(256) route_place_kernel(const int32_t* __restrict__ ids,
                                                          const float* __restrict__ probs, int64_t P, int32_t K,
                                                          int32_t E, const int32_t* __restrict__ blk_base,
                                                          const int32_t* __restrict__ expert_off, int32_t* pair2row,
                                                          int32_t* __restrict__ row2pair, float* __restrict__ row_prob) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    const int32_t e = ids[p];
    if (e < 0 || e >= E) {  // reported by the error word; the pair gets no row
        pair2row[p] = -1;
        return;
    }
    const int64_t blk = (p / K) / kTokPerBlk;
    const int32_t rank = pair2row[p];
    const int32_t row = expert_off[e] + blk_base[blk * E + e] + rank;
    pair2row[p] = row;
    row2pair[row] = (int32_t)p;
    row_prob[row] = probs[p];
}

// One wave per (32-row tile, 128-column step) of the sorted buffer: lane
// (h*32 + r) copies row r's columns [64c + 32h, +32) for c = 2*cp, 2*cp+1 from
// its token's quantized row, so each chunk is written as one contiguous 1 KiB.
__global__ void __launch_bounds__(256) route_gather_kernel(int32_t H, int32_t K, const int32_t* __restrict__ expert_off,
                                                           int32_t E, const int32_t* __restrict__ row2pair,
                                                           const uint8_t* __restrict__ xq_codes,
                                                           const uint8_t* __restrict__ xq_scales,
                                                           const float* __restrict__ gx, int64_t n_units,
                                                           uint8_t* __restrict__ a_codes,
                                                           uint8_t* __restrict__ a_scales, float* __restrict__ a_g) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= n_units) return;
    const int64_t cps = H / 128;
    const int64_t rt = unit / cps, cp = unit % cps;
    if (rt * 32 >= expert_off[E]) return;  // past the last expert's rows
    const int h = lane >> 5, rl = lane & 31;
    const int64_t row = rt * 32 + rl;
    const int32_t p = row2pair[row];
    u32x4 c0 = {0u, 0u, 0u, 0u}, c1 = {0u, 0u, 0u, 0u};
    uint32_t s0 = 0u, s1 = 0u;
    float g = 0.0f;
    if (p >= 0) {
        const int64_t t = p / K;
        const uint8_t* cs = xq_codes + t * (H / 2) + (2 * cp) * 32 + h * 16;
        const uint8_t* ss = xq_scales + t * (H / 16) + (2 * cp) * 4 + h * 2;
        c0 = *reinterpret_cast<const u32x4*>(cs);
        c1 = *reinterpret_cast<const u32x4*>(cs + 32);
        s0 = *reinterpret_cast<const uint16_t*>(ss);
        s1 = *reinterpret_cast<const uint16_t*>(ss + 4);
        g = gx[t];
    }
    *reinterpret_cast<u32x4*>(a_codes + (rt * (H / 64) + 2 * cp) * 1024 + lane * 16) = c0;
    *reinterpret_cast<u32x4*>(a_codes + (rt * (H / 64) + 2 * cp + 1) * 1024 + lane * 16) = c1;
    *reinterpret_cast<uint32_t*>(a_scales + (rt * (H / 128) + cp) * 256 + lane * 4) = s0 | (s1 << 16);
    if (cp == 0 && h == 0) a_g[row] = g;
}

hipError_t launch_route(const uint16_t* x, const int32_t* ids, const float* probs, int32_t T, int32_t H, int32_t K,
                        int32_t E, bool round_up, const RouteBuffers& rb, int64_t rows_cap, hipStream_t stream) {
    const int32_t nblk = (T + kTokPerBlk - 1) / kTokPerBlk;
    hipLaunchKernelGGL(route_count_kernel, dim3(nblk), dim3(256), 0, stream, x, ids, T, H, K, E, round_up ? 1 : 0,
                       rb.blk_counts, rb.blk_err, rb.pair2row /* holds the ranks until route_place */, rb.xq_codes,
                       rb.xq_scales, rb.gx);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, nblk, E, rb.blk_counts, rb.blk_err,
                       rb.expert_count, rb.expert_off, rb.mtiles, rb.n_mtiles, rb.row2pair, rb.err_word);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
    const int64_t P = (int64_t)T * K;
    hipLaunchKernelGGL(route_place_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, stream, ids, probs, P, K, E,
                       rb.blk_counts, rb.expert_off, rb.pair2row, rb.row2pair, rb.row_prob);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
    // Row tiles that can hold rows for this T (the device offsets decide which are used).
    const int64_t rows_bound = std::min<int64_t>(rows_cap, (P + (int64_t)E * (kMAlign - 1) + 31) / 32 * 32);
    const int64_t n_units = rows_bound / 32 * (H / 128);
    hipLaunchKernelGGL(route_gather_kernel, dim3((unsigned)((n_units + 3) / 4)), dim3(256), 0, stream, H, K,
                       rb.expert_off, E, rb.row2pair, rb.xq_codes, rb.xq_scales, rb.gx, n_units, rb.a_codes,
                       rb.a_scales, rb.a_g);
    return hipGetLastError();
}

}  // namespace nvfp4
