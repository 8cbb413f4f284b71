"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

awq_dequant must match the oracle bit for bit (the fp32 product is exact).
awq_gemm (fp16 out, fp32 accumulation) must satisfy, over the whole output,
    max |y - y_ref| <= 1e-2 * max(1, max |y_ref|)   and   ||y - y_ref||_F <= 2e-3 ||y_ref||_F
against the oracle's float64 result; special inputs whose exact result is a single
rounding (identity rows, integer weights, zero weights) must match bit for bit.
"""
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


def dev(d):
    out = {}
    for k, v in d.items():
        out[k] = torch.from_numpy(np.ascontiguousarray(v)).cuda() if isinstance(v, np.ndarray) else v
    return out


def gemm(d):
    t = dev(d)
    y = awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], d["group_size"])
    torch.cuda.synchronize()
    return y.cpu().numpy()


def tol_check(y, yref, label=""):
    assert y.shape == yref.shape
    assert np.isfinite(y).all(), label
    err = np.abs(y.astype(np.float64) - yref)
    bound = MAX_TOL * max(1.0, float(np.abs(yref).max()))
    fro = float(np.linalg.norm(err) / max(np.linalg.norm(yref), 1e-300))
    print(f"[{label}] max_err={err.max():.3e} (bound {bound:.3e}) rel_fro={fro:.3e}", flush=True)
    assert err.max() <= bound, label
    assert fro <= FRO_TOL, label


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


ALL = list(synth.WORKLOADS)


@pytest.mark.parametrize("name", ALL)
def test_dequant_bit_exact(name):
    w = synth.WORKLOADS[name]
    print(f"dequant {name}", flush=True)
    d = synth.make_inputs(w)
    t = dev(d)
    W = awq.awq_dequant(t["qweight"], t["qzeros"], t["scales"], w.group_size)
    torch.cuda.synchronize()
    ref = oracle.dequant_ref(d["qweight"], d["qzeros"], d["scales"], w.group_size)
    assert np.array_equal(bits(W.cpu().numpy()), bits(ref))


@pytest.mark.parametrize("name", ALL)
def test_gemm_workload(name):
    w = synth.WORKLOADS[name]
    print(f"gemm {name} plan={awq.plan(w.M, w.K, w.N, w.group_size)}", flush=True)
    d = synth.make_inputs(w)
    y = gemm(d)
    yref = oracle.gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], w.group_size)
    tol_check(y, yref, name)


RAGGED = [  # (M, K, N, g, bias): tails in M, N and in the K split
    (1, 32, 32, 32, False),
    (5, 352, 800, 32, True),
    (16, 320, 544, 64, True),
    (3, 4096, 96, 128, True),
    (2, 11008, 32, -1, True),
    (7, 2048, 288, 256, False),
    (17, 320, 544, 64, True),
    (130, 256, 416, -1, True),
    (257, 512, 256, 128, False),
    (64, 1024, 4128, 128, True),
    (1, 131072, 64, -1, True),   # skinny at the 128-split cap, 64 k-steps per wave
    (3, 65536, 96, 32, True),    # too many groups per workgroup for skinny: tile family
    (40, 4128, 96, 32, True),    # tile split over K, last split ends in a half k-tile
    (100, 2080, 160, -1, True),  # two 64 x 128 row tiles split over K
    (300, 4096, 256, 128, False),  # 256 x 128 tiles split over K
    (40, 32, 96, 32, True),      # tile family, K = 32: one k-tile, only half of it real
    (300, 96, 256, 32, True),    # tile family, last k-tile partial (loaded 32 rows early)
    (20, 32, 96, 32, True),      # 32 x 128 tiles: K = 32
    (30, 96, 256, 32, True),     # 32 x 128 tiles: last k-tile partial
    (160, 1024, 512, 128, True),  # 129-192 rows on a short K: three 64 x 128 row tiles, split over K
    (24, 4128, 96, 32, True),    # 32 x 128 tiles split over K, last split ends in a half k-tile
    (1, 3072, 544, 384, True),   # decode, 256-column tiles (last one partial), each half of a
    (2, 3072, 544, 384, False),  # workgroup's waves scaled apart, the halves in one or two groups
    (1, 3072, 544, 96, True),    # decode, one k-step per wave, each wave's sums scaled apart
    (2, 2048, 800, 32, True),    # the same with g = 32
    (1, 40960, 96, 64, True),    # decode past 127 half-width splits: 512-column tiles, 8 waves
    (3, 3072, 544, 384, True),   # decode, three rows (four kept), two groups per workgroup
    (4, 2048, 800, 32, False),   # decode, four rows, each wave's sums scaled apart
    (4, 40960, 96, 64, True),    # decode, four rows on 512-column tiles
    (4, 2048, 544, -1, True),    # decode, four rows, one group: the workgroup scaled once
    (3, 3072, 800, 64, False),   # decode, three rows, each wave's group scaled apart (4 parts)
    (1, 40960, 96, -1, True),    # decode, 512-column tiles in one group (scaled once)
    (1, 20480, 64, 160, True),   # decode, 512-column tiles of one k-step per wave on 8 waves
    (2, 20480, 64, 160, False),  # the same, two rows
    (4, 20480, 64, 160, True),   # the same, four rows
    (2, 40960, 96, -1, False),   # decode, two rows on 512-column tiles in one group
]


@pytest.mark.parametrize("M,K,N,g,bias", RAGGED)
def test_gemm_ragged(M, K, N, g, bias):
    print(f"ragged M={M} K={K} N={N} g={g} plan={awq.plan(M, K, N, g)}", flush=True)
    d = synth.make_custom(M, K, N, g, bias=bias, seed=M + K + N)
    yref = oracle.gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
    tol_check(gemm(d), yref, f"M{M}K{K}N{N}g{g}")


LARGE = [  # (M, K, N, g): extreme grid shapes (the oracle stays cheap with small K or N)
    (8192, 256, 1024, 128),      # 32 x 8 tiles of 256 x 128, every M tile full
    (8190, 128, 256, -1),        # last M tile with 254 rows
    (1, 64, 131072, 32),         # 512 skinny column tiles
    (40, 96, 131072, 32),        # 2048 column tiles of the 64 x 128 variant
    (300, 32768, 64, 128),       # long K on the tile family, split over K
    (2049, 64, 4096, -1),        # one full round of 256-row tiles, then a 1-row second launch
    (2100, 128, 4096, 64),       # second launch: 52 rows on 64 x 128 tiles
    (2248, 1024, 4096, 128),     # second launch: 200 rows on 256 x 128 tiles split over K
]


@pytest.mark.parametrize("M,K,N,g", LARGE)
def test_gemm_large_grids(M, K, N, g):
    print(f"large M={M} K={K} N={N} g={g} plan={awq.plan(M, K, N, g)}", flush=True)
    d = synth.make_custom(M, K, N, g, bias=True, seed=M + N)
    yref = oracle.gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
    tol_check(gemm(d), yref, f"large M{M}K{K}N{N}")


LAYERS = [  # (M, K, N, g): full-size layers whose grids span several rounds of resident workgroups
    (1, 8192, 28672, 128),       # one or two rows: every wave's run held inside one group
    (2, 4096, 114688, 128),
    (1, 28672, 8192, 128),       # 56 K splits
    (4, 8192, 28672, 128),       # four rows on a large layer: 4-row plan, fp32 partials
    (3, 4096, 114688, 128),      # three rows, the same
    (8, 4096, 114688, 128),      # eight rows on a large layer: 8-row plan, one-group runs
    (6, 28672, 8192, 128),       # 8-row plan, runs over several groups (LDS tables)
    (16, 4096, 114688, 128),     # 16 rows on 4-wave workgroups, fp32 partials
    (16, 28672, 8192, 128),      # the same, wave runs over several groups (LDS tables)
    (12, 4096, 11008, 128),      # 16-row plan on 8-wave workgroups
]


@pytest.mark.parametrize("M,K,N,g", LAYERS)
def test_gemm_layer_sampled_entries(M, K, N, g):
    """Every row at 520 output columns (spread over N, first and last included), each
    entry from the oracle's one-column dot product."""
    print(f"layer M={M} K={K} N={N} g={g} plan={awq.plan(M, K, N, g)}", flush=True)
    d = synth.make_custom(M, K, N, g, bias=True, seed=M + K + N)
    y = gemm(d)
    cols = np.unique(np.concatenate([np.linspace(0, N - 1, 512).astype(np.int64), np.arange(N - 8, N)]))
    rows = np.repeat(np.arange(M), len(cols))
    yref = oracle.gemm_ref_entries(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g,
                                   rows, np.tile(cols, M)).reshape(M, len(cols))
    tol_check(y[:, cols], yref, f"layer M{M}K{K}N{N}")


def is_fused_skinny(p):
    """A skinny plan whose K splits are summed by each tile's last workgroup: its
    workspace is the fp32 partials plus one 4-byte arrival counter per column tile."""
    gx, gy = p["grid"]
    extra = p["workspace_bytes"] - 4 * gx
    return p["family"] == "skinny" and gy > 1 and extra > 0 and extra % (gx * gy * 1024) == 0


FUSED = [  # (M, K, N, g): skinny plans on grids of several rounds, splits summed in-kernel
    (4, 2048, 65536, 64),    # 4-row plan, 256 x 8 workgroups
    (8, 1024, 131072, 64),   # 8-row plan, 512 x 4
    (3, 8192, 16384, 64),    # 4-row plan, 32 splits: a first batch of 16 loads, then two of 8
]


@pytest.mark.parametrize("M,K,N,g", FUSED)
def test_fused_split_sum(M, K, N, g):
    """Sampled entries against the oracle, bit-identical repeats, and the same bits
    again after a decode call (fixed-point words in the same zero-kept region as the
    arrival counters) on the same stream: every call leaves its counters at zero."""
    p = awq.plan(M, K, N, g)
    print(f"fused M={M} K={K} N={N} g={g} plan={p}", flush=True)
    assert is_fused_skinny(p)
    d = synth.make_custom(M, K, N, g, bias=True, seed=M + K + N)
    t = dev(d)
    other = dev(synth.make_custom(1, 4096, 4096, 128, seed=7))
    ys = []
    for _ in range(3):
        ys.append(awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], g).clone())
        awq.awq_gemm(other["x"], other["qweight"], other["qzeros"], other["scales"], other["bias"], 128)
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    y = ys[0].cpu().numpy()
    cols = np.unique(np.concatenate([np.linspace(0, N - 1, 512).astype(np.int64), np.arange(N - 8, N)]))
    rows = np.repeat(np.arange(M), len(cols))
    yref = oracle.gemm_ref_entries(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g,
                                   rows, np.tile(cols, M)).reshape(M, len(cols))
    tol_check(y[:, cols], yref, f"fused M{M}K{K}N{N}")


def test_fused_split_sum_graph_replays():
    """A fused plan captured in a graph and replayed three times, with eager calls of an
    unfused skinny plan and a decode plan in between: every replay equals the eager call."""
    M, K, N, g = FUSED[0]
    t = dev(synth.make_custom(M, K, N, g, seed=21))
    o1 = dev(synth.make_custom(16, 4096, 2048, 128, seed=22))
    o2 = dev(synth.make_custom(1, 4096, 4096, 128, seed=23))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], g).clone()
        y = torch.empty_like(eager)
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], g, out=y)
    for _ in range(3):
        with torch.cuda.stream(s):
            y.zero_()  # on the replay stream, ordered before the replay
            graph.replay()
            awq.awq_gemm(o1["x"], o1["qweight"], o1["qzeros"], o1["scales"], o1["bias"], 128)
            awq.awq_gemm(o2["x"], o2["qweight"], o2["qzeros"], o2["scales"], o2["bias"], 128)
        s.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16))


@pytest.mark.parametrize("M,K,N,g", [(5, 352, 800, 32), (2, 11008, 32, -1)])
def test_dequant_ragged_negative_scales(M, K, N, g):
    """Negative scales make (q - z) == 0 a negative zero: bits must still agree."""
    d = synth.make_custom(M, K, N, g, seed=3)
    d["scales"] = (-d["scales"].astype(np.float32)).astype(np.float16)
    t = dev(d)
    W = awq.awq_dequant(t["qweight"], t["qzeros"], t["scales"], g).cpu().numpy()
    ref = oracle.dequant_ref(d["qweight"], d["qzeros"], d["scales"], g)
    assert (np.signbit(ref) & (ref == 0)).any()
    assert np.array_equal(bits(W), bits(ref))


@pytest.mark.parametrize("M,K,N,g", [(9, 1024, 512, 128), (300, 512, 384, 64)])
def test_gemm_negative_scales(M, K, N, g):
    d = synth.make_custom(M, K, N, g, seed=4)
    d["scales"] = (-d["scales"].astype(np.float32)).astype(np.float16)
    yref = oracle.gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
    tol_check(gemm(d), yref, "negative scales")


@pytest.mark.parametrize("K,N,g,rows", [(512, 512, 128, 16), (256, 384, 64, 256), (4096, 256, -1, 3)])
def test_identity_rows_exact(K, N, g, rows):
    """x = rows of I_K: every output is one exact weight, so y == fp16(W) bit for bit."""
    d = synth.make_custom(rows, K, N, g, bias=False, seed=5)
    pick = np.linspace(0, K - 1, rows).astype(np.int64) if rows < K else np.arange(K)
    x = np.zeros((len(pick), K), dtype=np.float16)
    x[np.arange(len(pick)), pick] = 1.0
    d["x"] = x
    W = oracle.dequant_ref(d["qweight"], d["qzeros"], d["scales"], g)
    expect = oracle.fp16_rne(W[pick])
    y = gemm(d)
    assert np.array_equal(bits(y), bits(expect))


@pytest.mark.parametrize("M", [1, 6, 16, 40, 200])
def test_integer_weights_exact(M):
    """s = 1, z = 0, x in {-1, 0, 1}, K = 128: |y| <= 1920, an exact fp16 integer."""
    K, N = 128, 256
    rng = np.random.default_rng(M)
    d = synth.make_custom(M, K, N, -1, bias=False, seed=6)
    d["qzeros"] = np.zeros_like(d["qzeros"])
    d["scales"] = np.ones_like(d["scales"])
    d["x"] = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
    codes = oracle.unpack_awq(d["qweight"]).astype(np.int64)
    expect = (d["x"].astype(np.int64) @ codes).astype(np.float16)
    assert np.array_equal(bits(gemm(d)), bits(expect))


@pytest.mark.parametrize("M", [1, 12, 33])
def test_zero_weights_give_bias(M):
    """codes == zeros in every group: W == 0 and y == bias exactly."""
    K, N, g = 256, 512, 64
    d = synth.make_custom(M, K, N, g, bias=True, seed=7)
    d["qweight"] = np.repeat(d["qzeros"], g, axis=0)
    y = gemm(d)
    assert np.array_equal(bits(y), bits(np.tile(d["bias"], (M, 1))))


@pytest.mark.parametrize("M", [1, 16, 100])
def test_group_minus_one_equals_group_k(M):
    K, N = 1024, 512
    d = synth.make_custom(M, K, N, -1, seed=8)
    y1 = gemm(d)
    d2 = dict(d, group_size=K)
    y2 = gemm(d2)
    assert np.array_equal(bits(y1), bits(y2))


@pytest.mark.parametrize("name", ["decode_m1_k4096_n4096_g128", "decode_m16_k4096_n11008_g128",
                                  "down_proj_m64_k11008_n4096_g64"])
def test_deterministic(name):
    w = synth.WORKLOADS[name]
    t = dev(synth.make_inputs(w))
    ys = [awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], w.group_size).clone()
          for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))


def test_reduction_modes_share_a_stream():
    """Alternate plans that combine K splits differently (fixed-point atomics for
    M <= 2, fp32 partials + reduce kernel for skinny M > 2 and for split tiles) on
    one stream, twice over: each keeps its own workspace state valid for the others."""
    shapes = [(1, 4096, 4096, 128), (16, 4096, 1024, 128), (2, 2048, 512, 64), (3, 2048, 512, 64),
              (9, 4096, 2048, -1), (64, 2048, 512, 64)]
    for rep in range(2):
        for (M, K, N, g) in shapes:
            d = synth.make_custom(M, K, N, g, seed=rep + M)
            yref = oracle.gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
            tol_check(gemm(d), yref, f"alternating M{M} rep{rep}")


def test_m_zero_is_a_noop():
    d = dev(synth.make_custom(1, 256, 256, 128))
    x = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    y = awq.awq_gemm(x, d["qweight"], d["qzeros"], d["scales"], d["bias"], 128)
    assert tuple(y.shape) == (0, 256)


def test_leading_dims_and_side_stream():
    d = synth.make_custom(6, 512, 256, 64, seed=9)
    t = dev(d)
    x3 = t["x"].view(2, 3, 512)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = awq.awq_gemm(x3, t["qweight"], t["qzeros"], t["scales"], t["bias"], 64)
    s.synchronize()
    assert tuple(y.shape) == (2, 3, 256)
    yref = oracle.gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], 64)
    tol_check(y.reshape(6, 256).cpu().numpy(), yref, "leading dims")


def test_bad_arguments_raise_before_launch():
    t = dev(synth.make_custom(2, 256, 256, 64))
    with pytest.raises(ValueError):
        awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], 128)  # wrong group
    with pytest.raises(ValueError):
        awq.awq_gemm(t["x"][:, :128].contiguous(), t["qweight"], t["qzeros"], t["scales"], t["bias"], 64)
    with pytest.raises(TypeError):
        awq.awq_gemm(t["x"].float(), t["qweight"], t["qzeros"], t["scales"], t["bias"], 64)
    with pytest.raises(ValueError):
        awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"][:100].contiguous(), 64)


@pytest.mark.parametrize("M,K,N,g", [(1, 4096, 4096, 128), (16, 4096, 2048, 128), (64, 4096, 1024, 64),
                                     (300, 2048, 1024, -1)])
def test_graph_replays_match_eager(M, K, N, g):
    """awq_gemm captured in a HIP graph (after an eager call has sized the workspace)
    and replayed several times, with eager calls of other shapes in between: every
    replay equals the eager result bit for bit (the split-K accumulators are left zero
    by each call, partial buffers are fully rewritten)."""
    d = synth.make_custom(M, K, N, g, seed=11)
    t = dev(d)
    other = dev(synth.make_custom(3, 2048, 512, 64, seed=12))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], g).clone()
        y = torch.empty_like(eager)
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        awq.awq_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t["bias"], g, out=y)
    for rep in range(3):
        with torch.cuda.stream(s):
            y.zero_()  # on the replay stream, ordered before the replay
            graph.replay()
            awq.awq_gemm(other["x"], other["qweight"], other["qzeros"], other["scales"], other["bias"], 64)
        s.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


@pytest.mark.parametrize("name", ["decode_m1_k4096_n4096_g128", "prefill_m2048_k4096_n4096_g128",
                                  "down_proj_m64_k11008_n4096_g64", "down_proj_m64_k11008_n4096_g-1"])
def test_dequant_f16_bit_exact(name):
    """awq_dequant_f16 = the exact product rounded once to fp16, bit for bit."""
    w = synth.WORKLOADS[name]
    d = synth.make_inputs(w)
    t = dev(d)
    W = awq.awq_dequant(t["qweight"], t["qzeros"], t["scales"], w.group_size, dtype=torch.float16)
    torch.cuda.synchronize()
    ref = oracle.fp16_rne(oracle.dequant_ref(d["qweight"], d["qzeros"], d["scales"], w.group_size))
    assert np.array_equal(bits(W.cpu().numpy()), bits(ref))


def test_dequant_f16_negative_scales():
    d = synth.make_custom(5, 352, 800, 32, seed=13)
    d["scales"] = (-d["scales"].astype(np.float32)).astype(np.float16)
    t = dev(d)
    W = awq.awq_dequant(t["qweight"], t["qzeros"], t["scales"], 32, dtype=torch.float16).cpu().numpy()
    ref = oracle.fp16_rne(oracle.dequant_ref(d["qweight"], d["qzeros"], d["scales"], 32))
    assert np.array_equal(bits(W), bits(ref))


def test_graph_replay_survives_workspace_growth():
    """A graph captured at a small shape keeps replaying correctly after a larger eager
    call on the same stream has replaced the stream's workspace: the replaced buffer is
    retired, not freed, and stays zero between calls."""
    s = torch.cuda.Stream()
    small = synth.make_custom(1, 1024, 512, 128, seed=31)
    big = synth.make_custom(16, 4096, 8192, 128, seed=32)
    ts, tb = dev(small), dev(big)
    with torch.cuda.stream(s):
        eager = awq.awq_gemm(ts["x"], ts["qweight"], ts["qzeros"], ts["scales"], ts["bias"], 128).clone()
        y = torch.empty_like(eager)
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        awq.awq_gemm(ts["x"], ts["qweight"], ts["qzeros"], ts["scales"], ts["bias"], 128, out=y)
    assert awq.plan(16, 4096, 8192, 128)["workspace_bytes"] > 4 * awq.plan(1, 1024, 512, 128)["workspace_bytes"]
    yb_ref = oracle.gemm_ref(big["x"], big["qweight"], big["qzeros"], big["scales"], big["bias"], 128)
    for rep in range(3):
        with torch.cuda.stream(s):
            y.zero_()  # on the replay stream, ordered before the replay
            graph.replay()
            yb = awq.awq_gemm(tb["x"], tb["qweight"], tb["qzeros"], tb["scales"], tb["bias"], 128)
        s.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        tol_check(yb.cpu().numpy(), yb_ref, f"grown workspace rep {rep}")
