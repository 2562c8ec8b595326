"""Seeded synthetic inputs for the NVFP4 MoE expert forward.

This module is the only code that both the CPU oracle's users (tests, bench
CPU baseline) and the HIP path's users share.  It holds none of the method's
arithmetic: it draws random tensors, rounds them to BF16 (input plumbing) and
routes tokens with a softmax/top-k router that stands in for the upstream
router the pages place before the expert path.

Recipe:
  * numpy ``default_rng`` streams spawned from ``SeedSequence(seed)``: one
    child each for X, W1, W2, router logits and extras; W1 and W2 spawn one
    grandchild per expert so any expert's weights can be drawn alone.
  * normals drawn in float64, scaled, cast to float32, then to BF16 by
    round-to-nearest-even.
  * activations N(0, 1); weights N(0, 0.02^2).
  * router: logits N(0, 1) (+ a per-expert bias for the skewed workload),
    softmax in float64, top-k by descending probability (ties to the lower
    expert id), renormalised over the k picks, cast to float32.

Workloads (the Qwen3-30B-A3B layer shape stands in for the pages' trained
model; no dataset or checkpoint is used):
  tiny    T=64    H=256  E=8   K=2 I=128   seed 0
  dense   X [4096,2048] with 1% of entries x50, W [1536,2048]   seed 1
  qwen3   T=4096  H=2048 E=128 K=8 I=768   seed 2
  skewed  T=16384, same shape, Zipf(1.1) expert popularity       seed 3
  invariance pool: 512 probe tokens + filler tokens, qwen3 shape seed 4
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ACT_STD = 1.0
WEIGHT_STD = 0.02


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def route_topk(logits: np.ndarray, k: int):
    """softmax (float64) -> top-k descending, ties to the lower id -> renormalised float32."""
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(p, order, axis=1)
    top = top / top.sum(axis=1, keepdims=True)
    return order.astype(np.int32), top.astype(np.float32)


@dataclass
class MoEShape:
    T: int
    H: int
    E: int
    K: int
    I: int


class MoEWorkload:
    """Activations, routing and lazily drawn per-expert weights for one seed."""

    def __init__(self, name: str, seed: int, shape: MoEShape, zipf_s: float | None = None):
        self.name = name
        self.seed = seed
        self.shape = shape
        ss = np.random.SeedSequence(seed)
        ch_x, ch_w1, ch_w2, ch_logits, ch_extra = ss.spawn(5)
        self._w1_seeds = ch_w1.spawn(shape.E)
        self._w2_seeds = ch_w2.spawn(shape.E)
        T, H, E, K = shape.T, shape.H, shape.E, shape.K
        self.x = _normal_bf16(np.random.default_rng(ch_x), (T, H), ACT_STD)
        logits = np.random.default_rng(ch_logits).standard_normal((T, E))
        self.bias = np.zeros(E)
        if zipf_s is not None:
            ranks = np.random.default_rng(ch_extra).permutation(E) + 1
            self.bias = -zipf_s * np.log(ranks.astype(np.float64))
        self.ids, self.probs = route_topk(logits + self.bias[None, :], K)

    def w1(self, e: int) -> np.ndarray:
        """Expert e's W1 [2I, H] (rows 0..I-1 gate, I..2I-1 up), BF16 bits."""
        return _normal_bf16(np.random.default_rng(self._w1_seeds[e]), (2 * self.shape.I, self.shape.H), WEIGHT_STD)

    def w2(self, e: int) -> np.ndarray:
        """Expert e's W2 [H, I], BF16 bits."""
        return _normal_bf16(np.random.default_rng(self._w2_seeds[e]), (self.shape.H, self.shape.I), WEIGHT_STD)

    def weights(self, threads: int = 8):
        """All experts' (W1 [E,2I,H], W2 [E,H,I]) BF16 bits; drawn on a thread pool."""
        from concurrent.futures import ThreadPoolExecutor
        E = self.shape.E
        with ThreadPoolExecutor(max(1, threads)) as ex:
            w1 = np.stack(list(ex.map(self.w1, range(E))))
            w2 = np.stack(list(ex.map(self.w2, range(E))))
        return w1, w2

    def expert_counts(self) -> np.ndarray:
        return np.bincount(self.ids.reshape(-1), minlength=self.shape.E)


def tiny(seed: int = 0) -> MoEWorkload:
    """Tiny MoE layer: 64 tokens, hidden 256, 8 experts, top-2, intermediate 128."""
    return MoEWorkload("tiny_moe_T64_H256_E8_K2_I128", seed, MoEShape(T=64, H=256, E=8, K=2, I=128))


def qwen3(seed: int = 2, T: int = 4096) -> MoEWorkload:
    """Qwen3-30B-A3B-shaped layer: hidden 2048, 128 experts, top-8, intermediate 768."""
    return MoEWorkload(f"qwen3_30b_a3b_moe_T{T}", seed, MoEShape(T=T, H=2048, E=128, K=8, I=768))


def skewed(seed: int = 3, T: int = 16384) -> MoEWorkload:
    """Qwen3-30B-A3B layer shape with Zipf(1.1) expert popularity."""
    return MoEWorkload(f"qwen3_30b_a3b_moe_zipf1.1_T{T}", seed, MoEShape(T=T, H=2048, E=128, K=8, I=768),
                       zipf_s=1.1)


class DenseWorkload:
    """Dense NVFP4 linear: X [M,K] N(0,1) with 1% of entries x50, W [N,K] N(0,0.02^2)."""

    def __init__(self, seed: int = 1, M: int = 4096, K: int = 2048, N: int = 1536, outlier_frac: float = 0.01):
        self.name = f"dense_nvfp4_linear_M{M}_K{K}_N{N}"
        self.seed = seed
        ss = np.random.SeedSequence(seed)
        ch_x, ch_w, _ch_logits, ch_extra = ss.spawn(4)
        x = np.random.default_rng(ch_x).standard_normal((M, K)) * ACT_STD
        n_out = int(M * K * outlier_frac)
        idx = np.random.default_rng(ch_extra).choice(M * K, n_out, replace=False)
        x.reshape(-1)[idx] *= 50.0
        self.n_outliers = n_out
        self.x = f32_to_bf16_bits(x.astype(np.float32))
        self.w = _normal_bf16(np.random.default_rng(ch_w), (N, K), WEIGHT_STD)
        self.M, self.K, self.N = M, K, N


def dense(seed: int = 1) -> DenseWorkload:
    return DenseWorkload(seed)


class InvariancePool:
    """Batch-invariance workload on the Qwen3-30B-A3B layer shape.

    A fixed pool of probe tokens (x, ids, probs fixed per token) and a stream
    of filler tokens drawn from their own generator."""

    def __init__(self, seed: int = 4, n_probe: int = 512):
        self.layer = qwen3(seed=seed, T=n_probe)
        self.shape = self.layer.shape
        self.x = self.layer.x
        self.ids = self.layer.ids
        self.probs = self.layer.probs
        ss = np.random.SeedSequence([seed, 1])
        self._filler_rng = np.random.default_rng(ss)

    def fillers(self, n: int):
        s = self.shape
        x = _normal_bf16(self._filler_rng, (n, s.H), ACT_STD)
        logits = self._filler_rng.standard_normal((n, s.E))
        ids, probs = route_topk(logits, s.K)
        return x, ids, probs

    def batch(self, size: int, probes, rng: np.random.Generator):
        """A batch of `size` tokens holding the given probe indices at random positions."""
        probes = list(probes)
        assert len(probes) <= size
        x, ids, probs = self.fillers(size)
        pos = rng.choice(size, len(probes), replace=False)
        for p, i in zip(pos, probes):
            x[p], ids[p], probs[p] = self.x[i], self.ids[i], self.probs[i]
        return x, ids, probs, pos
