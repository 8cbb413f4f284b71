"""GPU parity of awq_gemm_bf16 (bfloat16 x, bias and y) against the CPU oracle.

Tolerance.  bfloat16 keeps 8 significant bits against fp16's 11, so its unit
roundoff is 8 times larger (2^-8 vs 2^-11).  Every rounding in the path (the one
of y, and the large-M path's rounding of the weight to bfloat16) scales with it,
so the fp16 bar is scaled by the same factor:
    max |y - y_ref| <= 8e-2 * max(1, max |y_ref|)   and   ||y - y_ref||_F <= 1.6e-2 ||y_ref||_F
against the oracle's float64 result on the exact values of the bfloat16 inputs.
Inputs whose result is one exact product, or an exact integer, must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import w4a16_weight_only_amd as awq
from oracle import awq_ref as oracle
from w4a16_weight_only_amd import synth

pytestmark = pytest.mark.gpu

MAX_TOL = 8e-2
FRO_TOL = 1.6e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    awq.load_library()


def to_dev(d):
    t = {}
    for k in ("qweight", "qzeros", "scales"):
        t[k] = torch.from_numpy(np.ascontiguousarray(d[k])).cuda()
    t["x"] = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).cuda().view(torch.bfloat16)
    t["bias"] = None if d["bias"] is None else \
        torch.from_numpy(np.ascontiguousarray(d["bias"]).view(np.int16)).cuda().view(torch.bfloat16)
    return t


def gemm_bits(d, g):
    t = to_dev(d)
    y = awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], g)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def tol_check(ybits, yref, label=""):
    y = oracle.bf16_to_f64(ybits)
    assert y.shape == yref.shape
    assert np.isfinite(y).all(), label
    err = np.abs(y - yref)
    bound = MAX_TOL * max(1.0, float(np.abs(yref).max()))
    fro = float(np.linalg.norm(err) / max(np.linalg.norm(yref), 1e-300))
    print(f"[{label}] max_err={err.max():.3e} (bound {bound:.3e}) rel_fro={fro:.3e}", flush=True)
    assert err.max() <= bound, label
    assert fro <= FRO_TOL, label


@pytest.mark.parametrize("name", [n for n in synth.WORKLOADS])
def test_gemm_bf16_workload(name):
    w = synth.WORKLOADS[name]
    print(f"bf16 gemm {name} plan={awq.plan(w.M, w.K, w.N, w.group_size)}", flush=True)
    d = synth.make_inputs_bf16(w)
    yref = oracle.gemm_ref_bf16(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], w.group_size)
    tol_check(gemm_bits(d, w.group_size), yref, name)


RAGGED = [  # (M, K, N, g, bias): both families, K splits through partials, tails
    (1, 32, 32, 32, False),
    (3, 4096, 96, 128, True),       # skinny, 4 waves, K split: fp32 partials + reduce
    (2, 11008, 32, -1, True),
    (5, 352, 800, 32, True),        # skinny, several groups per workgroup
    (16, 320, 544, 64, True),
    (1, 131072, 64, -1, True),      # 128 splits
    (40, 4128, 96, 32, True),       # tile split over K
    (130, 256, 416, -1, True),
    (300, 4096, 256, 128, False),
    (300, 96, 256, 32, True),       # partial last k-tile
    (40, 32, 96, 32, True),         # K = 32
    (257, 512, 256, 128, False),
    (24, 4096, 512, 128, True),     # 32 x 128 tiles split over K
    (20, 32, 96, 32, True),         # 32 x 128 tiles, K = 32
    (2100, 128, 4096, 64, True),    # last 52 rows in a second launch
]


@pytest.mark.parametrize("M,K,N,g,bias", RAGGED)
def test_gemm_bf16_ragged(M, K, N, g, bias):
    print(f"bf16 ragged M={M} K={K} N={N} g={g} plan={awq.plan(M, K, N, g)}", flush=True)
    d = synth.make_custom_bf16(M, K, N, g, bias=bias, seed=M + K + N + 1)
    yref = oracle.gemm_ref_bf16(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
    tol_check(gemm_bits(d, g), yref, f"bf16 M{M}K{K}N{N}g{g}")


@pytest.mark.parametrize("M,K,N,g", [(16, 8192, 28672, 128), (3, 4096, 114688, 128)])
def test_bf16_layer_sampled_entries(M, K, N, g):
    """Full-size layers (16-row plan on 4-wave workgroups; 3 rows): every row at 520
    columns, each entry from the oracle's one-column dot product on the exact values
    of the bfloat16 inputs."""
    print(f"bf16 layer M={M} K={K} N={N} g={g} plan={awq.plan(M, K, N, g)}", flush=True)
    d = synth.make_custom_bf16(M, K, N, g, bias=True, seed=M + K)
    ybits = gemm_bits(d, g)
    cols = np.unique(np.concatenate([np.linspace(0, N - 1, 512).astype(np.int64), np.arange(N - 8, N)]))
    rows = np.repeat(np.arange(M), len(cols))
    yref = oracle.gemm_ref_entries(oracle.bf16_to_f64(d["x"]), d["qweight"], d["qzeros"], d["scales"],
                                   oracle.bf16_to_f64(d["bias"]), g, rows, np.tile(cols, M)).reshape(M, len(cols))
    tol_check(ybits[:, cols], yref, f"bf16 layer M{M}K{K}N{N}")


def eye_bits(rows, K, pick):
    x = np.zeros((rows, K), dtype=np.float32)
    x[np.arange(rows), pick] = 1.0
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@pytest.mark.parametrize("K,N,g,rows", [(512, 512, 128, 16), (256, 384, 64, 256), (4096, 256, -1, 3),
                                        (4096, 512, 128, 1)])
def test_bf16_identity_rows_exact(K, N, g, rows):
    """x = rows of I_K: every output is one weight, so y == bf16(W) bit for bit, in
    both families (the small-M path's zero correction is exact for one-hot rows)."""
    d = synth.make_custom_bf16(rows, K, N, g, bias=False, seed=6)
    pick = np.linspace(0, K - 1, rows).astype(np.int64) if rows < K else np.arange(K)
    d["x"] = eye_bits(rows, K, pick)
    W = oracle.dequant_ref(d["qweight"], d["qzeros"], d["scales"], g)
    expect = oracle.f32_to_bf16_rne(W[pick])
    got = gemm_bits(d, g)
    assert np.array_equal(got, expect), f"{(got != expect).sum()} of {got.size} differ"


@pytest.mark.parametrize("M", [1, 6, 16, 40, 200])
def test_bf16_integer_weights_exact(M):
    """s = 1, z = 0, codes 0 or 1, x in {-1, 0, 1}, K = 128: |y| <= 128, an integer
    bfloat16 holds exactly, so y equals the integer product bit for bit."""
    K, N = 128, 256
    rng = np.random.default_rng(40 + M)
    codes = rng.integers(0, 2, (K, N))
    xi = rng.integers(-1, 2, (M, K)).astype(np.float32)
    d = dict(qweight=oracle.pack_awq(codes), qzeros=oracle.pack_awq(np.zeros((1, N), dtype=np.int64)),
             scales=np.ones((1, N), dtype=np.float16), bias=None,
             x=(xi.view(np.uint32) >> np.uint32(16)).astype(np.uint16))
    expect = oracle.f32_to_bf16_rne((xi.astype(np.int64) @ codes).astype(np.float32))
    assert np.array_equal(gemm_bits(d, -1), expect)


@pytest.mark.parametrize("name", ["decode_m1_k4096_n4096_g128", "decode_m16_k4096_n11008_g128",
                                  "down_proj_m64_k11008_n4096_g64", "prefill_m2048_k4096_n4096_g128"])
def test_bf16_deterministic(name):
    w = synth.WORKLOADS[name]
    d = synth.make_inputs_bf16(w)
    t = to_dev(d)
    ys = [awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], w.group_size)
          .view(torch.int16).clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], v) for v in ys[1:])


@pytest.mark.parametrize("M,K,N,g", [(1, 4096, 4096, 128), (16, 4096, 2048, 128), (64, 4096, 1024, 64),
                                     (512, 2048, 1024, -1)])
def test_bf16_graph_replays_match_eager(M, K, N, g):
    d = synth.make_custom_bf16(M, K, N, g, seed=9)
    t = to_dev(d)
    s = torch.cuda.Stream()
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], g, out=y)
        eager = y.clone()
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], g, out=y)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            graph.replay()
        s.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16))


def test_bf16_dtype_rules():
    d = synth.make_custom_bf16(4, 256, 64, 64, seed=2)
    t = to_dev(d)
    with pytest.raises(TypeError):  # fp16 bias with bfloat16 x
        awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"].to(torch.float16), 64)
    with pytest.raises(TypeError):  # bfloat16 scales are not the GEMM pack
        awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"].to(torch.bfloat16), t["bias"], 64)
    y = awq.awq_gemm(t["x"].view(2, 2, 256), t["qweight"], t["qzeros"], t["scales"], t["bias"], 64)
    assert y.shape == (2, 2, 64) and y.dtype == torch.bfloat16
