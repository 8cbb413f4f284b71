"""GPU parity of the routed-expert entry points against the oracle.

awq_moe_align: the offsets and the tile table are unique and must match bit for
bit; the order of slots within an expert is not, so each expert's segment must
hold exactly the slots routed to it.  awq_moe_gemm: the fp16 tolerance of awq_gemm,
    max |y - y_ref| <= 1e-2 * max(1, max |y_ref|)   and   ||y - y_ref||_F <= 2e-3 ||y_ref||_F,
on every slot (full size: on a spread subset of output columns, whose reference
comes from the oracle on the matching slice of the packed weights).
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


def tol_check(y, yref, label):
    err = np.abs(y.astype(np.float64) - yref)
    bound = MAX_TOL * max(1.0, float(np.abs(yref).max()))
    fro = float(np.linalg.norm(err) / max(np.linalg.norm(yref), 1e-300))
    print(f"[{label}] max_err={err.max():.3e} (bound {bound:.3e}) rel_fro={fro:.3e}", flush=True)
    assert np.isfinite(y).all(), label
    assert err.max() <= bound, label
    assert fro <= FRO_TOL, label


def expected_table(offsets, block_rows, tiles):
    rows = []
    for e in range(len(offsets) - 1):
        c = int(offsets[e + 1] - offsets[e])
        for j in range((c + block_rows - 1) // block_rows):
            rows.append((e, int(offsets[e]) + j * block_rows, min(block_rows, c - j * block_rows), 0))
    rows += [(-1, 0, 0, 0)] * (tiles - len(rows))
    return np.array(rows, dtype=np.int64).reshape(tiles, 4)


@pytest.mark.parametrize("S,E,block_rows,skew", [(1, 1, 64, False), (32, 8, 64, False), (2048, 8, 256, False),
                                                  (999, 64, 128, False), (4096, 1024, 64, False),
                                                  (300, 8, 64, True), (70000, 16, 256, False)])
def test_moe_align(S, E, block_rows, skew):
    rng = np.random.default_rng(S + E)
    ids = np.full(S, 3 % E, dtype=np.int32) if skew else rng.integers(0, E, S).astype(np.int32)
    print(f"align S={S} E={E} block_rows={block_rows}", flush=True)
    off, srt, table = awq.awq_moe_align(torch.from_numpy(ids).cuda(), E, block_rows)
    torch.cuda.synchronize()
    roff, rsrt = oracle.moe_align_ref(ids, E)
    off, srt, table = off.cpu().numpy(), srt.cpu().numpy(), table.cpu().numpy()
    assert np.array_equal(off, roff)
    for e in range(E):
        seg = srt[off[e]:off[e + 1]]
        assert np.array_equal(np.sort(seg), rsrt[roff[e]:roff[e + 1]]), e
    assert np.array_equal(table, expected_table(roff, block_rows, table.shape[0]))


def test_moe_align_ignores_out_of_range_ids():
    ids = np.array([0, 5, -1, 2, 1, 2, 7], dtype=np.int32)  # E = 3: slots 1, 2, 6 are not routed
    off, srt, table = awq.awq_moe_align(torch.from_numpy(ids).cuda(), 3, 64)
    off, srt = off.cpu().numpy(), srt.cpu().numpy()
    assert off.tolist() == [0, 1, 2, 4]
    assert srt[0] == 0 and srt[1] == 4 and sorted(srt[2:4].tolist()) == [3, 5]


def run(d):
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).cuda() for k in ("x", "qweight", "qzeros", "scales")}
    ids = torch.from_numpy(d["expert_ids"].reshape(-1, d["topk"])).cuda()
    y = awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], ids, d["group_size"])
    torch.cuda.synchronize()
    return y.cpu().numpy()


MOE_CASES = [  # (T, E, topk, K, N, g, routing)
    (5, 4, 2, 256, 96, 64, "random"),
    (64, 8, 2, 512, 256, 128, "random"),       # 16 rows per expert: 32-row tiles
    (300, 4, 1, 1024, 544, 32, "random"),
    (200, 2, 1, 96, 128, 32, "random"),        # 64-row tiles, partial last k-tile
    (600, 4, 2, 256, 256, -1, "random"),       # 256-row tiles
    (1, 16, 4, 4096, 64, 128, "random"),
    (300, 8, 1, 512, 128, 64, "one_expert"),   # every slot on expert 3; the others empty
    (130, 6, 3, 320, 160, 64, "random"),
]


@pytest.mark.parametrize("T,E,topk,K,N,g,routing", MOE_CASES)
def test_moe_gemm(T, E, topk, K, N, g, routing):
    d = synth.make_moe_custom(T, E, topk, K, N, g, seed=T + E + K)
    if routing == "one_expert":
        d["expert_ids"] = np.full(T * topk, 3, dtype=np.int32)
    print(f"moe T={T} E={E} topk={topk} K={K} N={N} g={g} {routing}", flush=True)
    y = run(d)
    yref = oracle.moe_gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["expert_ids"], topk, g)
    tol_check(y, yref, f"moe T{T}E{E}k{topk}")


def test_moe_gemm_last_rows_of_256_row_tiles():
    """Slots per expert 384, 383, 356, 64, 1 (top-1): the table has 256-row tiles,
    the full tiles and a last tile of exactly 128 rows take the 256 x 128 launch, last
    tiles of 127 and 100 rows take the 64 x 128 launch as two 64-row parts, those of
    64 and 1 rows as one part (the second leaves)."""
    counts = [384, 383, 356, 64, 1]
    E, K, N, g = len(counts), 512, 384, 64
    T = sum(counts)
    d = synth.make_moe_custom(T, E, 1, K, N, g, seed=97)
    ids = np.repeat(np.arange(E, dtype=np.int32), counts)
    d["expert_ids"] = np.random.default_rng(98).permutation(ids).astype(np.int32)
    y = run(d)
    yref = oracle.moe_gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["expert_ids"], 1, g)
    tol_check(y, yref, "moe last rows of 256-row tiles")


SKINNY_CASES = [  # (T, E, topk, K, N, g): up to 16 tokens take the expert-batched skinny family
    (1, 8, 2, 4096, 512, 128),
    (3, 16, 4, 1024, 96, 32),      # N below one 256-column tile
    (2, 8, 2, 11008, 256, 64),     # 4-row plan: fixed-point K splits
    (4, 8, 2, 11008, 256, 64),     # 16-row plan: fp32 partials
    (2, 4, 1, 8192, 1024, -1),
    (8, 64, 2, 2048, 768, -1),     # most experts receive no slot
    (16, 8, 2, 4096, 1024, 128),   # 8-wave workgroups, fp32 partials
    (13, 6, 3, 4096, 320, 64),
    (24, 16, 2, 4096, 1024, 128),  # 17-64 tokens, <= 8 slots per expert, >= 2 MB per expert:
    (64, 32, 2, 2048, 2048, 64),   # chunks of 16 routed tokens
    (33, 8, 1, 4096, 1056, 32),
    (4, 32, 2, 2048, 2048, 64),    # 3-4 tokens over many column tiles: 4-row plan, fp32 partials
    (3, 16, 1, 4096, 4096, 128),
    (8, 32, 2, 2048, 2048, 64),    # 5-8 tokens over many column tiles: 8-row plan
    (6, 16, 2, 4096, 4096, 128),
    (12, 16, 4, 2048, 4096, 64),
]


@pytest.mark.parametrize("T,E,topk,K,N,g", SKINNY_CASES)
def test_moe_gemm_few_tokens(T, E, topk, K, N, g):
    d = synth.make_moe_custom(T, E, topk, K, N, g, seed=T * 7 + E + K)
    print(f"moe few tokens T={T} E={E} topk={topk} K={K} N={N} g={g}", flush=True)
    y = run(d)
    yref = oracle.moe_gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["expert_ids"], topk, g)
    tol_check(y, yref, f"moe few T{T}E{E}k{topk}")


def test_moe_gemm_few_tokens_one_expert_many_chunks():
    """40 tokens, every one on expert 2 (top-1 of 8): that expert's 40 routed tokens
    take three 16-row chunks (16, 16, 8 rows); the other experts stream nothing."""
    T, E, K, N, g = 40, 8, 4096, 1024, 64
    d = synth.make_moe_custom(T, E, 1, K, N, g, seed=71)
    d["expert_ids"] = np.full(T, 2, dtype=np.int32)
    y = run(d)
    yref = oracle.moe_gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["expert_ids"], 1, g)
    tol_check(y, yref, "moe one expert, three chunks")


@pytest.mark.parametrize("T,E,topk,K,N", [(3, 5, 3, 1024, 256), (12, 5, 3, 1024, 256), (30, 16, 2, 2048, 2048)])
def test_moe_gemm_few_tokens_odd_routing(T, E, topk, K, N):
    """A token that names one expert twice gets that expert's row in both slots; slots
    whose id lies outside [0, E) route nowhere and keep what out held."""
    g = 64
    d = synth.make_moe_custom(T, E, topk, K, N, g, seed=T + 99)
    ids = d["expert_ids"].reshape(T, topk).copy()
    ids[0, 1] = ids[0, 0]          # repeated expert
    ids[1, topk - 1] = -1          # routes nowhere
    ids[T - 1, 0] = E              # routes nowhere
    d["expert_ids"] = ids.ravel()
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).cuda() for k in ("x", "qweight", "qzeros", "scales")}
    out = torch.full((T * topk, N), 7.0, dtype=torch.float16, device="cuda")
    awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], torch.from_numpy(ids).cuda(), g, out=out)
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    valid = (d["expert_ids"] >= 0) & (d["expert_ids"] < E)
    yref = oracle.moe_gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], np.where(valid, d["expert_ids"], E),
                               topk, g)
    tol_check(y[valid], yref[valid], f"moe odd T{T}")
    assert np.all(y[~valid] == 7.0)
    assert np.array_equal(y[0], y[1])


@pytest.mark.parametrize("T", [2, 16])
def test_moe_gemm_few_tokens_graph_replay(T):
    """The K splits of the few-token path meet in zero-maintained accumulators (2
    tokens) or in partials (16): replays must reproduce the eager bits."""
    d = synth.make_moe_custom(T, 8, 2, 4096, 512, 128, seed=T + 5)
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).cuda() for k in ("x", "qweight", "qzeros", "scales")}
    ids = torch.from_numpy(d["expert_ids"].reshape(-1, 2)).cuda()
    y = torch.empty((2 * T, 512), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], ids, 128, out=y)
        eager = y.clone()
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], ids, 128, out=y)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            graph.replay()
        s.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16))


@pytest.mark.parametrize("name", list(synth.MOE_WORKLOADS))
def test_moe_gemm_workload_sampled_columns(name):
    """Full-size layer; the reference covers 64 word columns (512 outputs) spread over N."""
    w = synth.MOE_WORKLOADS[name]
    d = synth.make_moe_inputs(w)
    print(f"moe workload {name}", flush=True)
    y = run(d)
    wc = np.linspace(0, w.N // 8 - 1, 64).astype(np.int64)
    cols = (8 * wc[:, None] + np.arange(8)[None, :]).ravel()
    yref = oracle.moe_gemm_ref(d["x"], d["qweight"][:, :, wc], d["qzeros"][:, :, wc], d["scales"][:, :, cols],
                               d["expert_ids"], w.topk, w.group_size)
    tol_check(y[:, cols], yref, name)


def test_moe_gemm_deterministic_and_graph_replay():
    d = synth.make_moe_custom(96, 8, 2, 1024, 512, 128, seed=12)
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).cuda() for k in ("x", "qweight", "qzeros", "scales")}
    ids = torch.from_numpy(d["expert_ids"].reshape(-1, 2)).cuda()
    y = torch.empty((192, 512), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], ids, 128, out=y)
        eager = y.clone()
        again = awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], ids, 128)
    s.synchronize()
    assert torch.equal(eager.view(torch.int16), again.view(torch.int16))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], ids, 128, out=y)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            graph.replay()
        s.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16))


def test_moe_gemm_argument_errors():
    d = synth.make_moe_custom(4, 2, 2, 64, 32, 32, seed=1)
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).cuda() for k in ("x", "qweight", "qzeros", "scales")}
    ids = torch.from_numpy(d["expert_ids"]).cuda()
    with pytest.raises(ValueError):
        awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], ids[:7], 32)  # not topk per token
    with pytest.raises(ValueError):
        awq.awq_moe_gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], ids, 16)  # group 16: unsupported
