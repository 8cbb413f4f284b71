"""GPU parity on non-finite and huge values: awq_gemm against the oracle's IEEE reference.

The product's fp32 accumulation must let NaN and infinities through as IEEE arithmetic
does (inf * 0 = NaN, inf + (-inf) = NaN), and partial sums far beyond fp16's range that
cancel across K splits must still cancel.  Each case runs on a plan chosen to reach a
different reduction: the decode family's fixed-point split-K (its exceptional partials
go through the float side words), the older skinny family's fixed-point plans (one
group per wave and LDS group tables), the tile family's fp32 partials and its partial
last k-tile (K % 64 == 32).

Comparison: NaN where the reference is NaN, the same infinity where the reference
rounds to an infinity in fp16, and the finite entries within the fp16 bar
(max |y - y_ref| <= 1e-2 max(1, max |y_ref|), relative Frobenius <= 2e-3) over the
finite entries.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import w4a16_weight_only_amd as awq
from oracle import awq_ref as oracle
from w4a16_weight_only_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    awq.load_library()


def gemm(d):
    t = {k: (torch.from_numpy(np.ascontiguousarray(v)).cuda() if isinstance(v, np.ndarray) else v)
         for k, v in d.items()}
    y = awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], d["group_size"])
    torch.cuda.synchronize()
    return y.cpu().numpy()


def compare(y, yref, label):
    y64 = y.astype(np.float64)
    with np.errstate(over="ignore"):
        r16 = yref.astype(np.float16)  # fp16 rounding of the exact value: overflow -> inf
    assert np.array_equal(np.isnan(y64), np.isnan(yref)), f"{label}: NaN pattern"
    inf_ref = np.isinf(r16) & ~np.isnan(yref)
    assert np.array_equal(np.isinf(y64), inf_ref), f"{label}: infinity pattern"
    assert np.array_equal(np.sign(y64[inf_ref]), np.sign(yref[inf_ref])), f"{label}: infinity signs"
    fin = np.isfinite(r16)
    if fin.any():
        err = np.abs(y64[fin] - yref[fin])
        bound = 1e-2 * max(1.0, float(np.abs(yref[fin]).max()))
        fro = float(np.linalg.norm(err) / max(np.linalg.norm(yref[fin]), 1e-300))
        print(f"[{label}] nan={int(np.isnan(yref).sum())} inf={int(inf_ref.sum())} "
              f"max_err={err.max():.3e} (bound {bound:.3e}) rel_fro={fro:.3e}", flush=True)
        assert err.max() <= bound, label
        assert fro <= 2e-3, label


SHAPES = [  # (M, K, N, g, family): reaching each reduction path
    (1, 4096, 512, 128, "decode"),
    (2, 4096, 544, 64, "decode"),      # partial last 512-column tile
    (3, 2048, 512, 128, "decode"),     # three rows, four kept per lane: fixed point with side words
    (5, 2048, 512, 128, "skinny"),     # fp32 partials and the reduce kernel
    (16, 4096, 512, -1, "skinny"),
    (1, 131072, 64, -1, "skinny"),     # beyond the decode family's split limit: fixed point, one group per wave
    (2, 98304, 128, 64, "skinny"),     # the same with waves over several groups (LDS tables)
    (64, 1024, 256, 64, "tile"),       # 64 x 128 tiles, fp32 partials over K splits
    (2048, 256, 256, 128, "tile"),     # 256 x 128 tiles
]


def _inject(d, kind, M, K):
    """NaN / +-inf in x at k positions spread over K (different K splits), per row."""
    x = d["x"].astype(np.float32)
    ks = np.linspace(0, K - 1, 5).astype(np.int64)
    for m in range(M):
        if kind == "nan":
            x[m, ks[m % 5]] = np.nan
        elif kind == "inf":
            x[m, ks[m % 5]] = np.inf if m % 2 == 0 else -np.inf
        elif kind == "inf_pair":
            x[m, ks[0]] = np.inf
            x[m, ks[4]] = -np.inf if m % 3 != 2 else np.inf
    d["x"] = x.astype(np.float16)
    return d


@pytest.mark.parametrize("kind", ["nan", "inf", "inf_pair"])
@pytest.mark.parametrize("M,K,N,g,family", SHAPES)
def test_nonfinite_x(M, K, N, g, family, kind):
    assert awq.plan(M, K, N, g)["family"] == family
    print(f"nonfinite {kind} M={M} K={K} N={N} g={g} plan={awq.plan(M, K, N, g)}", flush=True)
    d = _inject(synth.make_custom(M, K, N, g, bias=True, seed=M + K + N + 1), kind, M, K)
    yref = oracle.gemm_ref_ieee(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
    assert np.isnan(yref).any() or np.isinf(yref).any()
    compare(gemm(d), yref, f"{kind} M{M}K{K}N{N}g{g}")


@pytest.mark.parametrize("M,K,N,g,family", SHAPES)
def test_cancelling_huge_partials(M, K, N, g, family):
    """Unit scales and zero zero-points (W = q), 8 rows of x = +30000 against 8 rows of
    x = -30000 with identical weight rows half the layer apart: each of those K splits
    holds a partial of about 30000 * 8 * 7.5 (far beyond 2^18, the fixed-point range),
    and they cancel exactly."""
    d = synth.make_custom(M, K, N, g, bias=True, seed=M + K + N + 2)
    d["scales"] = np.ones_like(d["scales"])
    d["qzeros"] = np.zeros_like(d["qzeros"])
    a, b = 0, K // 2
    qw = d["qweight"].copy()
    qw[b:b + 8] = qw[a:a + 8]
    d["qweight"] = qw
    x = d["x"].copy()
    x[:, a:a + 8] = np.float16(30000.0)
    x[:, b:b + 8] = np.float16(-30000.0)
    d["x"] = x
    yref = oracle.gemm_ref_ieee(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
    assert np.isfinite(yref).all() and np.abs(yref).max() < 60000
    compare(gemm(d), yref, f"cancel M{M}K{K}N{N}g{g}")


@pytest.mark.parametrize("M,K,N,g", [(40, 96, 256, 32), (300, 96, 256, 32), (40, 32, 96, 32)])
def test_partial_last_ktile_inf(M, K, N, g):
    """K % 64 == 32 on the tile family: the last k-tile is loaded 32 rows early and only
    its new half is multiplied; +inf in the rows loaded twice must count once (an
    infinite x against the skipped half's weights must not turn into NaN)."""
    assert awq.plan(M, K, N, g)["family"] == "tile"
    d = synth.make_custom(M, K, N, g, bias=False, seed=M + K)
    x = d["x"].copy()
    k_dup = K - 64 + 8 if K >= 64 else 8  # a row of the half that is loaded again
    x[::3, k_dup] = np.inf
    d["x"] = x
    yref = oracle.gemm_ref_ieee(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
    assert np.isinf(yref).any()
    compare(gemm(d), yref, f"partial k-tile M{M}K{K}")


@pytest.mark.parametrize("M,K,N,g", [(1, 4096, 512, 128), (4, 2048, 512, 64)])
def test_nonfinite_then_finite_leaves_clean_workspace(M, K, N, g):
    """A call with NaN partials uses the float side words; they must be left zero, so a
    following finite call on the same stream is exact again (and deterministic)."""
    bad = _inject(synth.make_custom(M, K, N, g, seed=21), "nan", M, K)
    gemm(bad)
    good = synth.make_custom(M, K, N, g, seed=22)
    y1, y2 = gemm(good), gemm(good)
    assert np.isfinite(y1).all()
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    yref = oracle.gemm_ref(good["x"], good["qweight"], good["qzeros"], good["scales"], good["bias"], g)
    compare(y1, yref, "after nan")
