// router.hip -- router scores and deterministic top-k: the step that produces
// the expert ids and probabilities the expert forward takes.
//
// Article "Finish RL training faster: bitwise consistent, high-performance,
// agent-driven": section 4.4 ("R3 unnecessary": the scoring GEMM is one
// FP32-output kernel for every batch size, so routing recomputed on the
// training side matches the rollout) and section 2 (the same discrete choice
// needs the same tie-breaking and output order).
//
// Two launches:
//   scores   one wavefront per (32-token tile, 32-expert tile):
//            logits[t][e] = sum_h x[t][h] w[e][h] by BF16 MFMA 32x32x16 with
//            FP32 accumulation over the full H in one fixed order (increasing
//            k), fragments loaded straight from memory (16 contiguous bytes
//            per lane), the next 16 k-steps' loads in flight while the MFMAs
//            of the current 16 run.  A token's scores come from the same
//            instruction sequence whatever T is and wherever the token sits
//            in its tile.
//   top-k    one wavefront per token: 64-bit keys (order-preserving score
//            bits, then the complement of the expert id, so equal scores go
//            to the lower id); slot k gets the k-th expert of that total
//            order.  Up to 256 experts each key's rank is counted against all
//            keys at once; beyond that, K rounds of a wave-wide maximum.
//            Probabilities are the softmax restricted to the selection
//            (renormalize) or over all experts, in FP32 with one fixed
//            summation order.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRouterTok = 32;                        // tokens per workgroup (one MFMA row tile)
constexpr int kRouterKeys = kMaxExperts / kWave;      // scores per lane in phase 2
constexpr int kRankMaxE = 256;                        // phase 2 ranks by counting up to this many experts

// Unsigned integer whose order is the order of the FP32 value (-0 and +0 equal).
__device__ __forceinline__ uint32_t score_order(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float score_value(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// rank[i] = the number of the E keys in sk (zero-padded to an even count)
// larger than key[i], for this lane's first NK keys.
template <int NK>
__device__ __forceinline__ void count_ranks(const uint64_t* sk, int E2, const uint64_t* key, int* rank) {
    for (int j = 0; j < E2; j += 2) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(sk + j);  // two keys, one broadcast read
        const uint64_t k0 = ((uint64_t)kv[1] << 32) | kv[0], k1 = ((uint64_t)kv[3] << 32) | kv[2];
#pragma unroll
        for (int i = 0; i < NK; i++) rank[i] += (k0 > key[i] ? 1 : 0) + (k1 > key[i] ? 1 : 0);
    }
}

constexpr int kScoreSteps = 16;  // k-steps of 16 per load group; two groups in flight

__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1)))
router_scores_kernel(const uint16_t* __restrict__ x, int32_t T, int32_t H, const uint16_t* __restrict__ w,
                     int32_t E, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int32_t n_et = (E + 31) / 32;
    const int64_t t0 = (int64_t)(blockIdx.x / n_et) * kRouterTok;
    const int32_t nt = blockIdx.x % n_et;
    // MFMA operands: lane (kh*32 + r) supplies row r of the token tile (A)
    // and of the expert tile (B), k = 8 kh .. 8 kh + 7 of the step.
    const int r = lane & 31, kh = lane >> 5;
    const int64_t tok = min(t0 + r, (int64_t)T - 1);  // rows past T read the last token, not stored
    const int64_t e = min(nt * 32 + r, E - 1);         // columns past E read the last expert, not stored
    const uint16_t* xa = x + tok * H + 8 * kh;
    const uint16_t* wb = w + e * H + 8 * kh;
    const int n = H / 16;
    f32x16 acc = {};
    // Group g's fragments are loaded while group g - 1's MFMAs run (steps past
    // the end re-read the last one and run no MFMA); the MFMAs run in
    // increasing k.
    u32x4 a0[kScoreSteps], b0[kScoreSteps], a1[kScoreSteps], b1[kScoreSteps];
    auto load = [&](int s0, u32x4 (&a)[kScoreSteps], u32x4 (&b)[kScoreSteps]) {
#pragma unroll
        for (int q = 0; q < kScoreSteps; q++) {
            const int k = 16 * min(s0 + q, n - 1);
            a[q] = *reinterpret_cast<const u32x4*>(xa + k);
            b[q] = *reinterpret_cast<const u32x4*>(wb + k);
        }
    };
    auto mfma = [&](int s0, const u32x4 (&a)[kScoreSteps], const u32x4 (&b)[kScoreSteps]) {
#pragma unroll
        for (int q = 0; q < kScoreSteps; q++)
            if (s0 + q < n)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[q]),
                                                              __builtin_bit_cast(bf16x8, b[q]), acc, 0, 0, 0);
    };
    load(0, a0, b0);
    for (int s0 = 0; s0 < n; s0 += 2 * kScoreSteps) {
        load(s0 + kScoreSteps, a1, b1);
        mfma(s0, a0, b0);
        load(s0 + 2 * kScoreSteps, a0, b0);
        mfma(s0 + kScoreSteps, a1, b1);
    }
    // register j: row (j/4)*8 + kh*4 + j%4 of the token tile, column r
    const int col = nt * 32 + r;
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int64_t t = t0 + (j >> 2) * 8 + kh * 4 + (j & 3);
        if (t < T && col < E) logits[t * E + col] = acc[j];
    }
}

constexpr int kTopkWaves = 4;  // tokens per workgroup of the top-k kernel (one wavefront each)

__global__ void __launch_bounds__(kTopkWaves * 64) router_topk_kernel(int32_t T, int32_t E, int32_t K, int renorm,
                                                                     const float* __restrict__ logits,
                                                                     int32_t* __restrict__ ids,
                                                                     float* __restrict__ probs) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * kTopkWaves + wave;
    __shared__ __attribute__((aligned(16))) uint64_t skey[kTopkWaves][kRankMaxE];
    __shared__ uint64_t ssel[kTopkWaves][kMaxTopK];
    if (t >= T) return;
    const bool by_rank = E <= kRankMaxE;
    const float* lt = logits + t * E;
    uint64_t key[kRouterKeys];
#pragma unroll
    for (int i = 0; i < kRouterKeys; i++) {
        const int e = i * kWave + lane;
        key[i] = e < E ? ((uint64_t)score_order(lt[e]) << 32) | (uint32_t)~(uint32_t)e : 0ull;
    }
    int my_e = 0;
    float my_l = 0.0f;
    if (by_rank) {
        // The keys are unique, so a key's place in the order is the number of
        // larger keys; slot k takes the key of rank k.  Every lane counts
        // against all E keys (read back through LDS as broadcasts), so no
        // round waits on another.  Only the lane's live keys are ranked
        // (ceil(E / 64) of them), two keys per LDS read (an odd E is padded
        // with a zero key, which never outranks a real one).
        constexpr int kR = kRankMaxE / kWave;
        const int E2 = (E + 1) & ~1;
#pragma unroll
        for (int i = 0; i < kR; i++) {
            const int e = i * kWave + lane;
            if (e < E2) skey[wave][e] = e < E ? key[i] : 0ull;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        int rank[kR];
#pragma unroll
        for (int i = 0; i < kR; i++) rank[i] = 0;
        const int nk = (E + kWave - 1) / kWave;
        if (nk == 1)
            count_ranks<1>(&skey[wave][0], E2, key, rank);
        else if (nk == 2)
            count_ranks<2>(&skey[wave][0], E2, key, rank);
        else
            count_ranks<4>(&skey[wave][0], E2, key, rank);
#pragma unroll
        for (int i = 0; i < kR; i++) {
            const int e = i * kWave + lane;
            if (e < E && rank[i] < K) ssel[wave][rank[i]] = key[i];
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
        if (lane < K) {
            const uint64_t b = ssel[wave][lane];
            my_e = (int)~(uint32_t)b;
            my_l = score_value((uint32_t)(b >> 32));
        }
    }
    for (int k = 0; !by_rank && k < K; k++) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < kRouterKeys; i++) best = key[i] > best ? key[i] : best;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const uint64_t u = __shfl_xor(best, o, kWave);
            best = u > best ? u : best;
        }
#pragma unroll
        for (int i = 0; i < kRouterKeys; i++)
            if (key[i] == best) key[i] = 0ull;  // keys are unique: one owner
        if (lane == k) {
            my_e = (int)~(uint32_t)best;
            my_l = score_value((uint32_t)(best >> 32));
        }
    }
    const float top = __shfl(my_l, 0, kWave);
    const float num = lane < K ? expf(my_l - top) : 0.0f;
    float den = 0.0f;
    if (renorm) {
        for (int k = 0; k < K; k++) den += __shfl(num, k, kWave);  // slot order
    } else {
        // this lane's experts in increasing order, then a fixed butterfly
#pragma unroll
        for (int i = 0; i < kRouterKeys; i++) {
            const int e = i * kWave + lane;
            if (e < E) den += expf(lt[e] - top);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, kWave);
    }
    if (lane < K) {
        ids[t * K + lane] = my_e;
        probs[t * K + lane] = num / den;
    }
}

hipError_t launch_router(const uint16_t* x, int32_t T, int32_t H, const uint16_t* w, int32_t E, int32_t K,
                         bool renorm, float* logits, int32_t* ids, float* probs, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const unsigned score_waves = (unsigned)(((T + kRouterTok - 1) / kRouterTok) * ((E + 31) / 32));
    hipLaunchKernelGGL(router_scores_kernel, dim3(score_waves), dim3(64), 0, stream, x, T, H, w, E, logits);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
    hipLaunchKernelGGL(router_topk_kernel, dim3((unsigned)((T + kTopkWaves - 1) / kTopkWaves)), dim3(kTopkWaves * 64),
                       0, stream, T, E, K, renorm ? 1 : 0, logits, ids, probs);
    return hipGetLastError();
}

}  // namespace nvfp4
