"""GPU parity on seeded random shapes: every plan branch of both kernel families
(row counts 1..300, K splits, one-group and multi-group wave runs, 4- and 16-row
skinny plans, every tile variant, partial k-tiles, N tails) and of the routed-expert
product (few-token and grouped paths, idle experts), against the oracle within the
fp16 bar of awq_gemm:
    max |y - y_ref| <= 1e-2 * max(1, max |y_ref|)   and   ||y - y_ref||_F <= 2e-3 ||y_ref||_F
Shapes are drawn from a fixed seed, small enough for the oracle's float64 matmul."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import w4a16_weight_only_amd as awq
from oracle import awq_ref as oracle
from w4a16_weight_only_amd import synth

pytestmark = pytest.mark.gpu

MAX_TOL = 1e-2
FRO_TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    awq.load_library()


def tol_check(y, yref, label):
    err = np.abs(y.astype(np.float64) - yref)
    bound = MAX_TOL * max(1.0, float(np.abs(yref).max()))
    fro = float(np.linalg.norm(err) / max(np.linalg.norm(yref), 1e-300))
    print(f"[{label}] max_err={err.max():.3e} (bound {bound:.3e}) rel_fro={fro:.3e}", flush=True)
    assert np.isfinite(y).all(), label
    assert err.max() <= bound, label
    assert fro <= FRO_TOL, label


def draw_shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 17, 24, 33, 64, 65, 100, 128, 129, 200, 300]))
        g = int(rng.choice([32, 64, 128, 256, -1]))
        kg = 32 if g == -1 else g
        K = int(kg * rng.integers(1, max(2, 6144 // kg)))
        if M > 64:
            K = min(K, 2048 // kg * kg or kg)
        N = int(32 * rng.integers(1, 96 if M <= 16 else 48))
        out.append((M, K, N, g))
    return out


SHAPES = draw_shapes(20261202, 40)


@pytest.mark.parametrize("M,K,N,g", SHAPES)
def test_gemm_random_shape(M, K, N, g):
    print(f"sweep M={M} K={K} N={N} g={g} plan={awq.plan(M, K, N, g)}", flush=True)
    d = synth.make_custom(M, K, N, g, bias=(M + N) % 2 == 0, seed=M * 131 + K + N)
    t = {k: (torch.from_numpy(np.ascontiguousarray(v)).cuda() if isinstance(v, np.ndarray) else v)
         for k, v in d.items()}
    y = awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], g)
    torch.cuda.synchronize()
    yref = oracle.gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
    tol_check(y.cpu().numpy(), yref, f"sweep M{M}K{K}N{N}g{g}")


def draw_moe(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        T = int(rng.choice([1, 2, 3, 7, 12, 16, 17, 40, 150]))
        E = int(rng.choice([2, 4, 8, 16, 64]))
        topk = int(rng.integers(1, min(E, 4) + 1))
        g = int(rng.choice([32, 64, 128]))
        K = int(g * rng.integers(1, max(2, 2048 // g)))
        N = int(32 * rng.integers(1, 24))
        out.append((T, E, topk, K, N, g))
    return out


MOE = draw_moe(7, 16)


@pytest.mark.parametrize("T,E,topk,K,N,g", MOE)
def test_moe_random_shape(T, E, topk, K, N, g):
    print(f"moe sweep T={T} E={E} topk={topk} K={K} N={N} g={g}", flush=True)
    d = synth.make_moe_custom(T, E, topk, K, N, g, seed=T * 17 + E * 3 + K + N)
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).cuda() for k in ("x", "qweight", "qzeros", "scales")}
    ids = torch.from_numpy(d["expert_ids"].reshape(T, topk)).cuda()
    y = awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], ids, g)
    torch.cuda.synchronize()
    yref = oracle.moe_gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["expert_ids"], topk, g)
    tol_check(y.cpu().numpy(), yref, f"moe sweep T{T}E{E}k{topk}")
