"""Seeded synthetic inputs for the attention forward, shared by the tests and the bench.

This module draws random numbers, rounds them to the storage dtype and describes the
workload shapes. It contains none of the attention arithmetic: neither the CPU oracle
nor the HIP path lives here, and it imports neither.

Recipe (the same for every workload):
  * generator  ``np.random.default_rng(seed)`` (PCG64);
  * dense:  ``standard_normal(shape, dtype=float32)`` drawn in the order Q, K, V, each
    multiplied by ``sigma``;
  * varlen: sequence lengths first (``integers(lo, hi, size=S, endpoint=True)``), then one
    packed ``qkv`` draw of shape ``[T, 3, H, d]``, multiplied by ``sigma``;
  * the fp32 draws are rounded to the storage dtype with round-to-nearest-even, and the
    *rounded* values (held exactly in float32 arrays) are what both the oracle and the GPU
    see.

The shapes follow the workloads the pages describe: the [batch, heads, seq, head_dim]
tensors and GQA head counts of the Aule-Attention API examples (jeff.news article
"AMD GPU에서도 동작하는 FlashAttention 구현체, Aule-Attention", API bullets), the A10
sequence-2048 / 32-head / head_dim-64 measurement (xxqk.cn article
"Attention算子实战：从CUDA优化到昇腾/CANN部署", section 2.1) and the packed-QKV varlen
layout with cu_seqlens (ewbang.com article on a PyTorch FlashAttention for Turing,
the varlen function's docstring).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 ``x`` to ``dtype`` with round-to-nearest-even; return float32 holding
    the exactly representable rounded values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32)
        # RNE on the upper 16 bits: add 0x7FFF plus the lowest kept bit, then truncate.
        bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
        return r.view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def dense_inputs(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, *, seed,
                 sigma=1.0, dtype="bf16"):
    """Q [B,Hq,Nq,d], K and V [B,Hkv,Nk,d], drawn in that order from one generator."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, heads_q, seqlen_q, head_dim), dtype=np.float32)
    k = rng.standard_normal((batch, heads_kv, seqlen_k, head_dim), dtype=np.float32)
    v = rng.standard_normal((batch, heads_kv, seqlen_k, head_dim), dtype=np.float32)
    if sigma != 1.0:
        s = np.float32(sigma)
        q *= s
        k *= s
        v *= s
    return round_to_dtype(q, dtype), round_to_dtype(k, dtype), round_to_dtype(v, dtype)


def output_grad(shape, *, seed, dtype="bf16"):
    """dO for the backward: N(0,1) of the given shape from its own stream of ``seed``."""
    rng = np.random.default_rng([seed, 1])
    return round_to_dtype(rng.standard_normal(shape, dtype=np.float32), dtype)


def varlen_lengths(num_seqs, lo, hi, *, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=num_seqs, endpoint=True), rng


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    return cu.astype(np.int32)


def varlen_inputs(lengths, heads, head_dim, *, seed=None, rng=None, sigma=1.0, dtype="bf16"):
    """Packed ``qkv [T,3,H,d]`` and int32 ``cu_seqlens [S+1]`` for the given lengths.

    Pass ``rng`` to continue a generator that already drew the lengths."""
    if rng is None:
        rng = np.random.default_rng(seed)
    cu = cu_seqlens_from_lengths(lengths)
    total = int(cu[-1])
    qkv = rng.standard_normal((total, 3, heads, head_dim), dtype=np.float32)
    if sigma != 1.0:
        qkv *= np.float32(sigma)
    return round_to_dtype(qkv, dtype), cu


def sampled_rows(seqlen: int, *, seed=1004, n_random=49) -> np.ndarray:
    """Query rows checked at the long-context size: tile edges plus seeded random rows."""
    fixed = [0, 1, 2, 63, 64, 127, 128, 255, 256, 4095, 4096, 16383, 16384,
             seqlen - 2, seqlen - 1]
    fixed = sorted({r for r in fixed if 0 <= r < seqlen})
    rng = np.random.default_rng(seed)
    extra = []
    taken = set(fixed)
    while len(extra) < n_random and len(taken) < seqlen:
        for r in rng.choice(seqlen, n_random, replace=False).tolist():
            if r not in taken and len(extra) < n_random:
                taken.add(r)
                extra.append(r)
    return np.array(sorted(fixed + extra), dtype=np.int64)


@dataclass(frozen=True)
class DenseConfig:
    name: str
    dtype: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    causal: bool
    seed: int
    sigma: float = 1.0
    scale: float | None = None

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    def pairs(self) -> int:
        n = self.seqlen
        per = n * (n + 1) // 2 if self.causal else n * n
        return self.batch * per

    def flops(self) -> int:
        """4*d FLOP per unmasked (query, key) pair per q head: QK^T and PV, 2 FLOP/MAC."""
        return 4 * self.head_dim * self.heads_q * self.pairs()

    def bytes_compulsory(self) -> int:
        e = {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]
        n, d = self.seqlen, self.head_dim
        return e * d * n * self.batch * (2 * self.heads_q + 2 * self.heads_kv)

    def inputs(self):
        return dense_inputs(self.batch, self.heads_q, self.heads_kv, self.seqlen, self.seqlen,
                            self.head_dim, seed=self.seed, sigma=self.sigma, dtype=self.dtype)


@dataclass(frozen=True)
class VarlenConfig:
    name: str
    dtype: str
    num_seqs: int
    len_lo: int
    len_hi: int
    heads: int
    head_dim: int
    causal: bool
    seed: int
    sigma: float = 1.0
    scale: float | None = None

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    def lengths(self):
        return varlen_lengths(self.num_seqs, self.len_lo, self.len_hi, seed=self.seed)[0]

    def pairs(self) -> int:
        L = [int(x) for x in self.lengths()]
        return sum(l * (l + 1) // 2 if self.causal else l * l for l in L)

    def flops(self) -> int:
        return 4 * self.head_dim * self.heads * self.pairs()

    def bytes_compulsory(self) -> int:
        e = {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]
        total = int(sum(int(x) for x in self.lengths()))
        return e * total * self.heads * self.head_dim * 4   # q, k, v read + o written

    def inputs(self):
        lengths, rng = varlen_lengths(self.num_seqs, self.len_lo, self.len_hi, seed=self.seed)
        qkv, cu = varlen_inputs(lengths, self.heads, self.head_dim, rng=rng, sigma=self.sigma,
                                dtype=self.dtype)
        return qkv, cu


def alibi_slopes(heads: int) -> np.ndarray:
    """Geometric ALiBi slopes 2^(-8 (h + 1) / heads), fp32 [heads]."""
    return (2.0 ** (-8.0 * (np.arange(heads) + 1) / heads)).astype(np.float32)


def visible_pairs(L: int, causal: bool, left: int, right: int) -> int:
    """Unmasked (query, key) pairs of one sequence of length L under causal / window."""
    i = np.arange(L, dtype=np.int64)
    hi = i if causal else (np.minimum(L - 1, i + right) if right >= 0 else np.full(L, L - 1))
    lo = np.maximum(0, i - left) if left >= 0 else np.zeros(L, dtype=np.int64)
    return int(np.maximum(hi - lo + 1, 0).sum())


@dataclass(frozen=True)
class ModsConfig(VarlenConfig):
    """A varlen workload with score modifiers (sliding window, soft cap, ALiBi)."""
    window_left: int = -1
    window_right: int = -1
    softcap: float = 0.0
    alibi: bool = False

    def pairs(self) -> int:
        return sum(visible_pairs(int(l), self.causal, self.window_left, self.window_right)
                   for l in self.lengths())

    def slopes(self):
        return alibi_slopes(self.heads) if self.alibi else None


@dataclass(frozen=True)
class DecodeConfig:
    """A few new queries per sequence against a key/value cache (causal: the queries are the
    last seqlen_q positions, so query i sees keys j <= i + seqlen_k - seqlen_q)."""
    name: str
    dtype: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen_q: int
    seqlen_k: int
    head_dim: int
    causal: bool
    seed: int
    sigma: float = 1.0
    scale: float | None = None

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    def pairs(self) -> int:
        nq, nk = self.seqlen_q, self.seqlen_k
        per = nq * (nk - nq) + nq * (nq + 1) // 2 if self.causal else nq * nk
        return self.batch * per

    def flops(self) -> int:
        return 4 * self.head_dim * self.heads_q * self.pairs()

    def bytes_compulsory(self) -> int:
        """Q read and O written once, the K/V cache read once."""
        e = {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]
        d, B = self.head_dim, self.batch
        return e * d * B * (2 * self.heads_q * self.seqlen_q + 2 * self.heads_kv * self.seqlen_k)

    def inputs(self):
        return dense_inputs(self.batch, self.heads_q, self.heads_kv, self.seqlen_q, self.seqlen_k,
                            self.head_dim, seed=self.seed, sigma=self.sigma, dtype=self.dtype)


@dataclass(frozen=True)
class ShortConfig:
    """Short queries against short keys at a large batch (cross-attention of a diffusion
    model): Nq and Nk at most 128, so each (batch, kv head) fits the short-sequence kernel."""
    name: str
    dtype: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen_q: int
    seqlen_k: int
    head_dim: int
    causal: bool
    seed: int
    sigma: float = 1.0
    scale: float | None = None

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    def pairs(self) -> int:
        nq, nk = self.seqlen_q, self.seqlen_k
        per = nq * (nq + 1) // 2 if self.causal else nq * nk
        return self.batch * per

    def flops(self) -> int:
        return 4 * self.head_dim * self.heads_q * self.pairs()

    def bytes_compulsory(self) -> int:
        """Q read and O written once, K and V read once."""
        e = {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]
        d, B = self.head_dim, self.batch
        return e * d * B * (2 * self.heads_q * self.seqlen_q + 2 * self.heads_kv * self.seqlen_k)

    def inputs(self):
        return dense_inputs(self.batch, self.heads_q, self.heads_kv, self.seqlen_q, self.seqlen_k,
                            self.head_dim, seed=self.seed, sigma=self.sigma, dtype=self.dtype)


@dataclass(frozen=True)
class BwdConfig(DenseConfig):
    """The backward of a dense workload: dQ, dK, dV from Q, K, V, O, dO and the row LSE."""

    def flops(self) -> int:
        """10*d FLOP per unmasked pair per q head: the recomputed QK^T, dP = dO V^T, dV += P^T dO,
        dQ += dS K and dK += dS^T Q (five products, 2 FLOP/MAC) — 2.5x the forward."""
        return 10 * self.head_dim * self.heads_q * self.pairs()

    def bytes_compulsory(self) -> int:
        """Q, O, dO read and dQ written ([B,Hq,N,d] each); K, V read and dK, dV written
        ([B,Hkv,N,d] each); the fp32 LSE read."""
        e = {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]
        n, d, B = self.seqlen, self.head_dim, self.batch
        return e * d * n * B * (4 * self.heads_q + 4 * self.heads_kv) + 4 * B * self.heads_q * n

    def grad(self):
        return output_grad((self.batch, self.heads_q, self.seqlen, self.head_dim), seed=self.seed,
                           dtype=self.dtype)


# The five workloads: a small fp32 case, the A10-shaped fp16 causal case, the bf16 causal
# GQA case the throughput is quoted on, packed varlen, and a 32k long-context GQA case.
CONFIGS = {
    "c1_f32_dense": DenseConfig("c1_f32_dense", "f32", 1, 2, 2, 128, 64, False, seed=0,
                                scale=0.125),
    "c2_f16_causal": DenseConfig("c2_f16_causal", "f16", 1, 32, 32, 2048, 64, True, seed=1),
    "c3_bf16_causal_gqa": DenseConfig("c3_bf16_causal_gqa", "bf16", 4, 32, 8, 4096, 128, True,
                                      seed=2),
    "c4_bf16_varlen": VarlenConfig("c4_bf16_varlen", "bf16", 16, 64, 4096, 16, 128, True,
                                   seed=3),
    "c5_bf16_long_gqa": DenseConfig("c5_bf16_long_gqa", "bf16", 1, 32, 8, 32768, 128, True,
                                    seed=4, sigma=0.5),
}

# Lengths the varlen workload must draw (regenerated and asserted in the tests).
C4_LENGTHS = [3336, 409, 787, 1019, 795, 3295, 3569, 2411, 222, 443, 1403, 1810, 2569, 1996,
              1131, 708]

# Decoding against a KV cache (the split-KV path): one new query per sequence, GQA, a
# 16k-token bf16 cache of 512 MiB, so the step is bound by reading the cache from HBM.
DECODE_CONFIGS = {
    "d1_bf16_decode_gqa": DecodeConfig("d1_bf16_decode_gqa", "bf16", 8, 32, 8, 1, 16384, 128,
                                       True, seed=6),
}

# The backward of the headline workload (training): same shape, bf16 causal GQA.
BWD_CONFIGS = {
    "b1_bf16_causal_gqa_bwd": BwdConfig("b1_bf16_causal_gqa_bwd", "bf16", 4, 32, 8, 4096, 128,
                                        True, seed=2),
    # the same training shape in fp32
    "b2_f32_causal_gqa_bwd": BwdConfig("b2_f32_causal_gqa_bwd", "f32", 4, 32, 8, 4096, 128,
                                       True, seed=2),
}

# The varlen workload with all three score modifiers on: a 1024-key sliding window (causal),
# a soft cap of 50 on the scaled scores and geometric ALiBi slopes.
MODS_CONFIGS = {
    "m1_bf16_varlen_mods": ModsConfig("m1_bf16_varlen_mods", "bf16", 16, 64, 4096, 16, 128, True,
                                      seed=3, window_left=1024, window_right=0, softcap=50.0,
                                      alibi=True),
}

# Short-sequence cross-attention (the diffusion-model shape of 64 queries against 77 keys,
# 768 = 12 heads x 64 channels), non-causal, at a batch of 256 so the launch fills the GPU.
SHORT_CONFIGS = {
    "s1_bf16_short_cross": ShortConfig("s1_bf16_short_cross", "bf16", 256, 12, 12, 64, 77, 64,
                                       False, seed=7),
}

# The bf16 causal GQA shape in fp32 (the jeff.news page lists fp32 among the supported
# dtypes): it measures the fp32 matrix-core kernel at a size that fills the GPU.
F32_CONFIGS = {
    "f1_f32_causal_gqa": DenseConfig("f1_f32_causal_gqa", "f32", 4, 32, 8, 4096, 128, True, seed=2),
}

# The packed-varlen benchmark harness of the ewbang.com article (its verification script's
# comparison: batch 128, every sequence at the 4096-token maximum, 8 heads, head_dim 64,
# fp16, non-causal): 524288 tokens, a 1.6 GB qkv pack.
HARNESS_CONFIGS = {
    "e1_f16_varlen_b128": VarlenConfig("e1_f16_varlen_b128", "f16", 128, 4096, 4096, 8, 64, False,
                                       seed=8),
}
