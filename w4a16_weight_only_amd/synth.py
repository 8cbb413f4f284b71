"""Seeded synthetic workloads for the fused AWQ W4A16 linear.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the HIP path (tests, benchmark) and the CPU oracle take their
inputs from here.

Packed tensors are drawn as uniformly random 32-bit words.  In the AWQ GEMM
layout every 32-bit pattern is a valid pack of eight 4-bit codes (the pack is a
bijection between eight codes in 0..15 and one word), so uniform random words
are exactly "codes and zeros uniform in 0..15, packed in AWQ order" without
running a packer here.

Draw order for one workload (one numpy Generator seeded per workload):
  1. qweight words  [K, N/8]
  2. qzeros words   [G, N/8]
  3. scales         uniform [1e-3, 2e-2), rounded to fp16, [G, N]
  4. x              standard normal [M, K] (float64 draws)
  5. outlier input channels (only if outlier_count > 0): rng.choice without
     replacement; those columns of x are multiplied by outlier_gain before the
     fp16 rounding
  6. bias           normal(0, 0.01) rounded to fp16, [N] (only if bias)
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    group_size: int
    bias: bool
    outlier_count: int = 0
    outlier_gain: float = 50.0
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def groups(self) -> int:
        return 1 if self.group_size == -1 else self.K // self.group_size

    def algorithmic_bytes(self) -> int:
        """Bytes the fused linear must move at least once: packed weight, packed
        zeros, fp16 scales, fp16 x, fp16 bias (if any) and fp16 y."""
        G = self.groups
        return (self.K * self.N // 2 + G * self.N // 2 + 2 * G * self.N
                + 2 * self.M * self.K + (2 * self.N if self.bias else 0) + 2 * self.M * self.N)

    def flops(self) -> int:
        return 2 * self.M * self.K * self.N


def _down_proj(M: int, g: int) -> Workload:
    return Workload(f"down_proj_m{M}_k11008_n4096_g{g}", M, 11008, 4096, g, True,
                    note="7B MLP down_proj shape sweep")


# The measured and parity workloads: a tiny correctness layer, the 7B attention
# q_proj decode GEMV, the 7B MLP up_proj small-batch decode, a 2048-token
# prefill with activation-outlier channels, and the down_proj M sweep.
WORKLOADS = {w.name: w for w in [
    Workload("tiny_m4_k512_n512_g128", 4, 512, 512, 128, False, note="tiny correctness layer"),
    Workload("decode_m1_k4096_n4096_g128", 1, 4096, 4096, 128, True, note="7B q_proj decode GEMV"),
    Workload("decode_m16_k4096_n11008_g128", 16, 4096, 11008, 128, True, note="7B MLP up_proj small batch"),
    Workload("prefill_m2048_k4096_n4096_g128", 2048, 4096, 4096, 128, False, outlier_count=41,
             note="prefill, 1% of input channels x50"),
    *[_down_proj(M, g) for g in (64, -1) for M in (1, 8, 64, 512)],
]}


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform random 32-bit patterns as int32."""
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32).view(np.int32)


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """numpy inputs for workload `w` (see the module docstring for the draw order)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    M, K, N, G = w.M, w.K, w.N, w.groups
    qweight = random_words(rng, (K, N // 8))
    qzeros = random_words(rng, (G, N // 8))
    scales = rng.uniform(1e-3, 2e-2, size=(G, N)).astype(np.float16)
    x = rng.standard_normal((M, K))
    if w.outlier_count:
        idx = rng.choice(K, size=w.outlier_count, replace=False)
        x[:, idx] *= w.outlier_gain
    x = x.astype(np.float16)
    bias = rng.normal(0.0, 0.01, size=N).astype(np.float16) if w.bias else None
    return dict(x=x, qweight=qweight, qzeros=qzeros, scales=scales, bias=bias,
                group_size=w.group_size)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float draws, rounded by torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make_inputs_bf16(w: Workload, seed: int | None = None) -> dict:
    """The same draws as make_inputs with bfloat16 activations: x and bias are the
    float64 draws rounded to float32 and then to bfloat16 (bit patterns, uint16)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    M, K, N, G = w.M, w.K, w.N, w.groups
    qweight = random_words(rng, (K, N // 8))
    qzeros = random_words(rng, (G, N // 8))
    scales = rng.uniform(1e-3, 2e-2, size=(G, N)).astype(np.float16)
    x = rng.standard_normal((M, K))
    if w.outlier_count:
        idx = rng.choice(K, size=w.outlier_count, replace=False)
        x[:, idx] *= w.outlier_gain
    bias = rng.normal(0.0, 0.01, size=N) if w.bias else None
    return dict(x=to_bf16_bits(x), qweight=qweight, qzeros=qzeros, scales=scales,
                bias=None if bias is None else to_bf16_bits(bias), group_size=w.group_size)


def make_custom_bf16(M, K, N, group_size, bias=True, seed=0, outlier_count=0) -> dict:
    return make_inputs_bf16(Workload(f"custom_m{M}_k{K}_n{N}_g{group_size}", M, K, N, group_size,
                                     bias, outlier_count=outlier_count, seed=seed))


def make_custom(M, K, N, group_size, bias=True, seed=0, outlier_count=0) -> dict:
    """Same distributions at an arbitrary shape (ragged and edge-case tests)."""
    return make_inputs(Workload(f"custom_m{M}_k{K}_n{N}_g{group_size}", M, K, N, group_size,
                                bias, outlier_count=outlier_count, seed=seed))


def make_weights(K: int, N: int, seed: int = 0, std: float = 0.02, outlier_cols: int = 0,
                 outlier_gain: float = 20.0) -> np.ndarray:
    """fp16 dense weight [K, N] (input by output features) for the RTN writer.

    Draw order: normal(0, std) float64 [K, N]; then, if outlier_cols > 0, that many
    output columns (rng.choice without replacement) scaled by outlier_gain (the
    salient channels that make per-column ranges differ); rounded to fp16 last.
    std 0.02 is the usual initialisation scale of transformer linear layers."""
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, std, size=(K, N))
    if outlier_cols:
        idx = rng.choice(N, size=outlier_cols, replace=False)
        w[:, idx] *= outlier_gain
    return w.astype(np.float16)


@dataclass(frozen=True)
class MoeWorkload:
    """Routed-expert layer: T tokens, each sent to topk distinct experts of E; every
    expert holds one AWQ GEMM-layout weight [K, N] (group size g)."""
    name: str
    T: int
    E: int
    topk: int
    K: int
    N: int
    group_size: int
    seed: int = 0

    @property
    def slots(self) -> int:
        return self.T * self.topk

    @property
    def groups(self) -> int:
        return 1 if self.group_size == -1 else self.K // self.group_size


# An 8-expert top-2 layer with 4096-wide tokens and 14336-wide expert projections
# (the shape class of the pages' 7B-scale models, extended to routed experts).
MOE_WORKLOADS = {w.name: w for w in [
    MoeWorkload("moe_decode_t16_e8_top2_k4096_n14336_g128", 16, 8, 2, 4096, 14336, 128),
    MoeWorkload("moe_prefill_t1024_e8_top2_k4096_n14336_g128", 1024, 8, 2, 4096, 14336, 128),
]}


def make_moe_inputs(w: MoeWorkload, seed: int | None = None) -> dict:
    """Draw order (one Generator): per expert e = 0..E-1 its qweight words, qzeros
    words and scales (as make_inputs); then x standard normal [T, K] -> fp16; then per
    token rng.choice(E, topk, replace=False) as its experts (slot t * topk + j)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    G = w.groups
    qw, qz, sc = [], [], []
    for _ in range(w.E):
        qw.append(random_words(rng, (w.K, w.N // 8)))
        qz.append(random_words(rng, (G, w.N // 8)))
        sc.append(rng.uniform(1e-3, 2e-2, size=(G, w.N)).astype(np.float16))
    x = rng.standard_normal((w.T, w.K)).astype(np.float16)
    ids = np.stack([rng.choice(w.E, size=w.topk, replace=False) for _ in range(w.T)]).astype(np.int32).ravel()
    return dict(x=x, qweight=np.stack(qw), qzeros=np.stack(qz), scales=np.stack(sc), expert_ids=ids,
                topk=w.topk, group_size=w.group_size)


def make_moe_custom(T, E, topk, K, N, group_size, seed=0) -> dict:
    return make_moe_inputs(MoeWorkload(f"moe_custom_t{T}_e{E}_top{topk}", T, E, topk, K, N, group_size, seed))
