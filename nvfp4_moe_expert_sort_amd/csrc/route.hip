// route.hip -- expert sort with padding and device offsets, fused with the
// amax and quantization of X (miniTE summary page, "how to use it": sort+amax,
// then pad(X, amax), then quantize into the buffer the GEMM reads; expert
// boundaries are device offsets; the metadata is reused by FC1, FC2 and the
// combine).
//
// Three launches, all sized from T and the config only (no host read-back of
// counts, article section 4.6):
//   route_hist     per block of 16 tokens: integer histogram of its (t, k)
//                  pairs per expert in LDS; id checks.
//   route_scan     one block: per-expert exclusive prefix over the blocks,
//                  padded expert offsets off[E+1], the GEMM row-tile table,
//                  padding rows marked, error word.
//   route_scatter  per block of 16 tokens: stable rank of each pair inside its
//                  expert (wave ballots, in pair order p = t*K + k), then each
//                  wave quantizes one token row once (amax in registers) and
//                  writes it to the token's K sorted rows.
// Integer atomics only on LDS histograms: the counts and every row index are
// independent of scheduling.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"
#include "nvfp4_quant_row.h"

namespace nvfp4 {

__global__ void __launch_bounds__(256) route_hist_kernel(const int32_t* __restrict__ ids, int32_t T, int32_t K,
                                                         int32_t E, int32_t* __restrict__ blk_counts,
                                                         int32_t* __restrict__ blk_err) {
    __shared__ int32_t hist[kMaxExperts];
    __shared__ int32_t err;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x) hist[e] = 0;
    if (tid == 0) err = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * kTokPerBlk * K;
    const int64_t p1 = min((int64_t)(blockIdx.x + 1) * kTokPerBlk * K, (int64_t)T * K);
    int my_err = 0;
    for (int64_t p = p0 + tid; p < p1; p += blockDim.x) {
        const int32_t e = ids[p];
        if (e < 0 || e >= E) {
            my_err |= 1;
            continue;
        }
        atomicAdd(&hist[e], 1);
        const int64_t t = p / K;
        for (int64_t q = t * K; q < p; q++)
            if (ids[q] == e) my_err |= 2;
    }
    if (my_err) atomicOr(&err, my_err);
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) blk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
    if (tid == 0) blk_err[blockIdx.x] = err;
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
    //     owning a contiguous segment of blocks.
    const int tpe = 1024 / E;  // >= 1 since E <= 1024
    const int e1 = tid / tpe, sub = tid % tpe;
    const int seg = (nblk + tpe - 1) / tpe;
    const int b0 = min(sub * seg, nblk), b1 = min(b0 + seg, nblk);
    int32_t sum = 0;
    if (e1 < E)
        for (int b = b0; b < b1; b++) sum += blk_counts[(int64_t)b * E + e1];
    part[tid] = sum;
    int my_err = 0;
    for (int b = tid; b < nblk; b += 1024) my_err |= blk_err[b];
    if (my_err) atomicOr(&errs, my_err);
    __syncthreads();
    if (e1 < E) {
        int32_t run = 0;
        for (int s = 0; s < sub; s++) run += part[e1 * tpe + s];
        for (int b = b0; b < b1; b++) {
            const int32_t c = blk_counts[(int64_t)b * E + e1];
            blk_counts[(int64_t)b * E + e1] = run;  // becomes this block's first rank within expert e1
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

__global__ void __launch_bounds__(256) route_scatter_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, const float* __restrict__ probs, int32_t T,
    int32_t H, int32_t K, int32_t E, const int32_t* __restrict__ blk_base, const int32_t* __restrict__ expert_off,
    int32_t* __restrict__ pair2row, int32_t* __restrict__ row2pair, float* __restrict__ row_prob,
    uint8_t* __restrict__ a_codes, uint8_t* __restrict__ a_scales, float* __restrict__ a_g, int round_up) {
    __shared__ int32_t running[kMaxExperts];
    __shared__ int32_t pair_row[kTokPerBlk * kMaxTopK];
    __shared__ int64_t dst[4][kMaxTopK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * kTokPerBlk;
    const int64_t p0 = t0 * K;
    const int64_t p1 = min((int64_t)(t0 + kTokPerBlk) * K, (int64_t)T * K);
    for (int e = tid; e < E; e += blockDim.x) running[e] = expert_off[e] + blk_base[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    if (wave == 0) {
        int nbits = 0;
        while ((1 << nbits) < E) nbits++;
        for (int64_t c0 = p0; c0 < p1; c0 += kWave) {
            const int64_t p = c0 + lane;
            int32_t e = p < p1 ? ids[p] : -1;
            const bool valid = e >= 0 && e < E;
            uint64_t mask = __ballot(valid);
            for (int b = 0; b < nbits; b++) {
                const bool bit = valid && ((e >> b) & 1);
                const uint64_t m1 = __ballot(bit);
                mask &= bit ? m1 : ~m1;
            }
            int32_t row = -1;
            if (valid) {
                const uint64_t below = mask & ((1ull << lane) - 1ull);
                row = running[e] + __popcll(below);
            }
            __builtin_amdgcn_s_waitcnt(0);  // every lane's read of running[] precedes the leaders' updates
            __builtin_amdgcn_wave_barrier();
            if (valid && (mask & ((1ull << lane) - 1ull)) == 0ull) running[e] += __popcll(mask);
            if (p < p1) pair_row[p - p0] = row;
        }
    }
    __syncthreads();
    // Each wave quantizes whole token rows: once per token, written to its K rows.
    for (int64_t t = t0 + wave; t < min(t0 + kTokPerBlk, (int64_t)T); t += 4) {
        int n = 0;
        for (int k = 0; k < K; k++) {
            const int32_t r = pair_row[(t - t0) * K + k];
            if (r >= 0) dst[wave][n++] = r;
        }
        if (lane < K) {
            const int64_t p = t * K + lane;
            const int32_t r = pair_row[p - p0];
            pair2row[p] = r;
            if (r >= 0) {
                row2pair[r] = (int32_t)p;
                row_prob[r] = probs[p];
            }
        }
        quant_row_wave(x + t * H, H, -1.0f, round_up != 0, true, dst[wave], n, a_codes, a_scales, a_g);
    }
}

hipError_t launch_route(const uint16_t* x, const int32_t* ids, const float* probs, int32_t T, int32_t H, int32_t K,
                        int32_t E, bool round_up, const RouteBuffers& rb, hipStream_t stream) {
    const int32_t nblk = (T + kTokPerBlk - 1) / kTokPerBlk;
    hipLaunchKernelGGL(route_hist_kernel, dim3(nblk), dim3(256), 0, stream, ids, T, K, E, rb.blk_counts, rb.blk_err);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, nblk, E, rb.blk_counts, rb.blk_err,
                       rb.expert_count, rb.expert_off, rb.mtiles, rb.n_mtiles, rb.row2pair, rb.err_word);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
    hipLaunchKernelGGL(route_scatter_kernel, dim3(nblk), dim3(256), 0, stream, x, ids, probs, T, H, K, E,
                       rb.blk_counts, rb.expert_off, rb.pair2row, rb.row2pair, rb.row_prob, rb.a_codes, rb.a_scales,
                       rb.a_g, round_up ? 1 : 0);
    return hipGetLastError();
}

}  // namespace nvfp4
