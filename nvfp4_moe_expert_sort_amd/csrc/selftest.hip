// selftest.hip -- bitwise batch-invariance self-test of the expert forward.
//
// Article section 4.4: with per-token quantization and a fixed per-row
// accumulation, a row's result does not depend on its neighbours, and the
// article's bitwise router + MoE test checks exactly that; section 2 of the
// article asks that a request give the same bits alone or batched.  This test
// runs every probe token alone, then inside decode batches of every size
// 1..max_decode_batch (probes at varying positions among filler tokens), then
// inside one prefill batch holding all probes, and compares output bits.
// Section 4.4 ("two layouts, same row results"): the prefill batch also runs
// through the masked fixed-capacity layout, and its probes must keep their
// bits there too.
//
// Inputs come from a counter-based generator (SplitMix64 of seed and a
// counter), so the test needs nothing but the quantized weights.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/nvfp4moe.h"

namespace {

uint64_t splitmix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

struct Gen {
    uint64_t seed, ctr;
    uint64_t next() { return splitmix64(seed * 0x100000001B3ull + ctr++); }
    double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }  // (0, 1)
    double normal() {
        const double u1 = uniform(), u2 = uniform();
        return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
    }
};

uint16_t to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One token: N(0,1) activations, K distinct experts, positive probabilities summing to ~1.
void draw_token(Gen& g, int H, int E, int K, uint16_t* x, int32_t* ids, float* probs, std::vector<int>& perm) {
    for (int j = 0; j < H; j++) x[j] = to_bf16((float)g.normal());
    for (int e = 0; e < E; e++) perm[e] = e;
    double sum = 0.0;
    std::vector<double> w(K);
    for (int k = 0; k < K; k++) {
        const int j = k + (int)(g.next() % (uint64_t)(E - k));
        std::swap(perm[k], perm[j]);
        ids[k] = perm[k];
        w[k] = 0.05 + g.uniform();
        sum += w[k];
    }
    for (int k = 0; k < K; k++) probs[k] = (float)(w[k] / sum);
}

}  // namespace

extern "C" int nvfp4moe_selftest_batch_invariance(const nvfp4moe_config* cfg, const nvfp4_qtensor* W1q,
                                                  const nvfp4_qtensor* W2q, uint64_t seed, int32_t n_probe,
                                                  int32_t max_decode_batch, int32_t prefill_tokens,
                                                  int64_t* report_host, void* stream) {
    if (!cfg || !W1q || !W2q) return NVFP4_E_NULL;
    const size_t ws_bytes = nvfp4moe_workspace_bytes(cfg);
    if (ws_bytes == 0) return NVFP4_E_SHAPE;
    if (n_probe < 1 || max_decode_batch < 0 || prefill_tokens < 0) return NVFP4_E_SHAPE;
    if (max_decode_batch > cfg->max_tokens || prefill_tokens > cfg->max_tokens) return NVFP4_E_CAPACITY;
    if (prefill_tokens > 0 && prefill_tokens < n_probe) return NVFP4_E_SHAPE;
    const int H = cfg->hidden, E = cfg->n_experts, K = cfg->top_k;
    const int Tmax = std::max({1, max_decode_batch, prefill_tokens});
    hipStream_t s = (hipStream_t)stream;

    Gen gp{seed, 0}, gf{seed ^ 0xF111E5ull, 0}, gpos{seed ^ 0x9051710Eull, 0};
    std::vector<int> perm(E);
    std::vector<uint16_t> px((size_t)n_probe * H);
    std::vector<int32_t> pid((size_t)n_probe * K);
    std::vector<float> ppr((size_t)n_probe * K);
    for (int i = 0; i < n_probe; i++)
        draw_token(gp, H, E, K, &px[(size_t)i * H], &pid[(size_t)i * K], &ppr[(size_t)i * K], perm);

    void *dx = nullptr, *dids = nullptr, *dpr = nullptr, *dout = nullptr, *dws = nullptr;
    int status = NVFP4_OK;
    auto fail = [&](int st) {
        status = st;
        return st;
    };
    if (hipMalloc(&dx, (size_t)Tmax * H * 2) != hipSuccess || hipMalloc(&dids, (size_t)Tmax * K * 4) != hipSuccess ||
        hipMalloc(&dpr, (size_t)Tmax * K * 4) != hipSuccess || hipMalloc(&dout, (size_t)Tmax * H * 2) != hipSuccess ||
        hipMalloc(&dws, ws_bytes) != hipSuccess)
        fail(NVFP4_E_HIP);

    std::vector<uint16_t> ref((size_t)n_probe * H), bx((size_t)Tmax * H), bout((size_t)Tmax * H);
    std::vector<int32_t> bid((size_t)Tmax * K);
    std::vector<float> bpr((size_t)Tmax * K);
    int64_t n_cmp = 0, n_bad = 0, first_probe = -1, first_batch = -1;

    auto run = [&](int T) -> int {
        if (hipMemcpyAsync(dx, bx.data(), (size_t)T * H * 2, hipMemcpyHostToDevice, s) != hipSuccess ||
            hipMemcpyAsync(dids, bid.data(), (size_t)T * K * 4, hipMemcpyHostToDevice, s) != hipSuccess ||
            hipMemcpyAsync(dpr, bpr.data(), (size_t)T * K * 4, hipMemcpyHostToDevice, s) != hipSuccess)
            return NVFP4_E_HIP;
        int st = nvfp4moe_moe_expert_forward(cfg, (const uint16_t*)dx, T, (const int32_t*)dids, (const float*)dpr,
                                             W1q, W2q, (uint16_t*)dout, dws, ws_bytes, s);
        if (st != NVFP4_OK) return st;
        if (hipMemcpyAsync(bout.data(), dout, (size_t)T * H * 2, hipMemcpyDeviceToHost, s) != hipSuccess)
            return NVFP4_E_HIP;
        return hipStreamSynchronize(s) == hipSuccess ? NVFP4_OK : NVFP4_E_HIP;
    };
    auto place = [&](int slot, int probe) {
        std::memcpy(&bx[(size_t)slot * H], &px[(size_t)probe * H], (size_t)H * 2);
        std::memcpy(&bid[(size_t)slot * K], &pid[(size_t)probe * K], (size_t)K * 4);
        std::memcpy(&bpr[(size_t)slot * K], &ppr[(size_t)probe * K], (size_t)K * 4);
    };
    auto fill = [&](int T) {
        for (int t = 0; t < T; t++) draw_token(gf, H, E, K, &bx[(size_t)t * H], &bid[(size_t)t * K], &bpr[(size_t)t * K], perm);
    };
    auto check = [&](int slot, int probe, int64_t batch) {
        n_cmp++;
        if (std::memcmp(&bout[(size_t)slot * H], &ref[(size_t)probe * H], (size_t)H * 2) != 0) {
            n_bad++;
            if (first_probe < 0) {
                first_probe = probe;
                first_batch = batch;
            }
        }
    };

    // 1. every probe alone
    for (int i = 0; i < n_probe && status == NVFP4_OK; i++) {
        place(0, i);
        if (run(1) != NVFP4_OK) {
            fail(NVFP4_E_HIP);
            break;
        }
        std::memcpy(&ref[(size_t)i * H], bout.data(), (size_t)H * 2);
    }
    // 2. decode batches of every size, probes at random positions among fillers
    for (int b = 1; b <= max_decode_batch && status == NVFP4_OK; b++) {
        fill(b);
        const int np = std::min({b, 4, n_probe});
        std::vector<int> slots(b), probes(np);
        for (int t = 0; t < b; t++) slots[t] = t;
        for (int k = 0; k < np; k++) {
            std::swap(slots[k], slots[k + (int)(gpos.next() % (uint64_t)(b - k))]);
            probes[k] = (int)(gpos.next() % (uint64_t)n_probe);
            place(slots[k], probes[k]);
        }
        const int st = run(b);
        if (st != NVFP4_OK) {
            fail(st);
            break;
        }
        for (int k = 0; k < np; k++) check(slots[k], probes[k], b);
    }
    // 3. one prefill batch holding every probe
    if (prefill_tokens > 0 && status == NVFP4_OK) {
        fill(prefill_tokens);
        std::vector<int> slots(prefill_tokens);
        for (int t = 0; t < prefill_tokens; t++) slots[t] = t;
        for (int k = 0; k < n_probe; k++) {
            std::swap(slots[k], slots[k + (int)(gpos.next() % (uint64_t)(prefill_tokens - k))]);
            place(slots[k], k);
        }
        const int st = run(prefill_tokens);
        if (st != NVFP4_OK)
            fail(st);
        else
            for (int k = 0; k < n_probe; k++) check(slots[k], k, prefill_tokens);
        // 4. the same batch in the masked layout, capacity = the largest
        //    expert count rounded up to 32 (reported as batch -T)
        if (status == NVFP4_OK) {
            std::vector<int64_t> cnt(E, 0);
            for (int p = 0; p < prefill_tokens * K; p++) cnt[bid[p]]++;
            const int64_t mx = *std::max_element(cnt.begin(), cnt.end());
            const int32_t cap = (int32_t)std::max<int64_t>(32, (mx + 31) / 32 * 32);
            const size_t mws_bytes = nvfp4moe_workspace_bytes_masked(cfg, cap);
            void* mws = nullptr;
            if (mws_bytes == 0)
                fail(NVFP4_E_SHAPE);
            else if (hipMalloc(&mws, mws_bytes) != hipSuccess)
                fail(NVFP4_E_HIP);
            else {
                int st2 = nvfp4moe_moe_expert_forward_masked(cfg, cap, (const uint16_t*)dx, prefill_tokens,
                                                             (const int32_t*)dids, (const float*)dpr, W1q, W2q,
                                                             (uint16_t*)dout, mws, mws_bytes, s);
                if (st2 == NVFP4_OK &&
                    hipMemcpyAsync(bout.data(), dout, (size_t)prefill_tokens * H * 2, hipMemcpyDeviceToHost, s) !=
                        hipSuccess)
                    st2 = NVFP4_E_HIP;
                if (st2 == NVFP4_OK && hipStreamSynchronize(s) != hipSuccess) st2 = NVFP4_E_HIP;
                if (st2 != NVFP4_OK)
                    fail(st2);
                else
                    for (int k = 0; k < n_probe; k++) check(slots[k], k, -(int64_t)prefill_tokens);
                (void)hipFree(mws);
            }
        }
    }
    (void)hipFree(dx);
    (void)hipFree(dids);
    (void)hipFree(dpr);
    (void)hipFree(dout);
    (void)hipFree(dws);
    if (report_host) {
        report_host[0] = n_cmp;
        report_host[1] = n_bad;
        report_host[2] = first_probe;
        report_host[3] = first_batch;
    }
    if (status != NVFP4_OK) return status;
    return n_bad == 0 ? NVFP4_OK : NVFP4_E_MISMATCH;
}
