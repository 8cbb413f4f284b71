"""GPU parity of the RTN writer awq_quantize_rtn against the oracle's quantize_rtn.

Every output (packed codes, packed zeros, fp16 scales) is integer or bit-pattern
work decided by float32 arithmetic that both sides do in the same precision and
order, so the bar is bit-exact equality of all three tensors.
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


def run_both(W: np.ndarray, g: int, sym: bool, label: str):
    print(f"[quantize_rtn {label}] K={W.shape[0]} N={W.shape[1]} g={g} sym={sym}", flush=True)
    qw, qz, sc = awq.awq_quantize_rtn(torch.from_numpy(W).cuda(), g, sym)
    torch.cuda.synchronize()
    rqw, rqz, rsc = oracle.quantize_rtn(W, g, sym)
    got = (qw.cpu().numpy(), qz.cpu().numpy(), sc.cpu().numpy().view(np.uint16))
    ref = (rqw, rqz, rsc.view(np.uint16))
    for name, a, b in zip(("qweight", "qzeros", "scales"), got, ref):
        assert a.shape == b.shape, (label, name)
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{label}: {name} differs at {len(bad)} places, first {bad[:4].tolist()}"
    return got


SHAPES = [
    # (K, N, group_size): groups of up to 256 rows in one fused pass (1..16 rows per
    # thread), longer groups in two passes over 128-row chunks (ragged last chunk
    # for 288, 500, 1000 and 3000 rows); N not a multiple of the 128-column block.
    (128, 512, 128),
    (4096, 4096, 128),
    (4096, 1024, 64),
    (256, 96, 32),
    (96, 8, 3),
    (64, 520, 1),
    (384, 136, 128),
    (1024, 512, 256),
    (2048, 264, 1024),
    (4096, 512, -1),
    (3000, 128, -1),
    (1000, 40, 500),
    (600, 64, 200),
    (864, 24, 288),
]


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("K,N,g", SHAPES)
def test_quantize_rtn_bit_exact(K, N, g, sym):
    W = synth.make_weights(K, N, seed=K * 7 + N + (g % 97), outlier_cols=min(4, N // 8))
    run_both(W, g, sym, f"K{K} N{N} g{g}")


def test_quantize_rtn_special_groups():
    """Constant, one-signed, tiny, subnormal and extreme groups; exact ties."""
    g, N = 32, 64
    rng = np.random.default_rng(5)
    cols = []
    cols.append(np.full(g, 0.0))                       # zero range: the 1e-5 floor
    cols.append(np.full(g, -0.0))
    cols.append(np.full(g, 0.37))                      # constant, positive
    cols.append(np.full(g, -2.5))                      # constant, negative
    cols.append(rng.uniform(0.5, 1.0, g))              # all positive: zero clamps to 0
    cols.append(rng.uniform(-1.0, -0.5, g))            # all negative: zero clamps to 15
    cols.append(rng.uniform(-1e-6, 1e-6, g))           # below the floor, fp16 subnormals
    cols.append(np.where(np.arange(g) % 2 == 0, 65504.0, -65504.0))  # full fp16 range
    s = 2.0 ** -6                                       # exact ties: w / s = j + 1/2
    cols.append(np.concatenate([[0.0, 15 * s], (np.arange(g - 2) % 15 + 0.5) * s]))
    cols.append(np.concatenate([[-8 * s, 7 * s], (np.arange(g - 2) % 15 - 7.5) * s]))
    while len(cols) < N:
        cols.append(rng.normal(0, 10.0 ** rng.uniform(-4, 2), g))
    W = np.stack(cols, axis=1).astype(np.float16)
    W = np.concatenate([W, W[::-1]], axis=0)           # two groups, different row order
    for sym in (False, True):
        run_both(W, g, sym, "special")
    for sym in (False, True):
        run_both(W, -1, sym, "special one group")


def test_quantize_rtn_dequant_round_trip():
    """The written pack read back through awq_dequant reproduces each weight within
    half a step of its group's scale (values inside the quantisation range)."""
    K, N, g = 512, 256, 128
    W = synth.make_weights(K, N, seed=11)
    qw, qz, sc = awq.awq_quantize_rtn(torch.from_numpy(W).cuda(), g)
    Wd = awq.awq_dequant(qw, qz, sc, g).cpu().numpy()
    s = np.repeat(sc.cpu().numpy().astype(np.float64), g, axis=0)
    err = np.abs(Wd.astype(np.float64) - W.astype(np.float64))
    assert (err <= 0.5 * s * (1 + 1e-3)).mean() > 0.99
    assert (err <= 1.0 * s).all()


def test_quantize_rtn_writes_into_given_buffers_and_rejects_bad_args():
    K, N, g = 256, 64, 64
    W = torch.from_numpy(synth.make_weights(K, N, seed=3)).cuda()
    out = (torch.full((K, N // 8), -1, dtype=torch.int32, device="cuda"),
           torch.full((K // g, N // 8), -1, dtype=torch.int32, device="cuda"),
           torch.full((K // g, N), float("nan"), dtype=torch.float16, device="cuda"))
    got = awq.awq_quantize_rtn(W, g, out=out)
    assert all(a is b for a, b in zip(got, out))
    ref = oracle.quantize_rtn(W.cpu().numpy(), g)
    assert np.array_equal(out[0].cpu().numpy(), ref[0])
    assert np.array_equal(out[1].cpu().numpy(), ref[1])
    assert np.array_equal(out[2].cpu().numpy().view(np.uint16), ref[2].view(np.uint16))
    with pytest.raises(ValueError, match="AWQ_ERR_GROUP"):
        awq.awq_quantize_rtn(W, 100)                   # does not divide K
    with pytest.raises(ValueError, match="AWQ_ERR_SHAPE"):
        awq.awq_quantize_rtn(W[:, :60].contiguous(), 64)  # N % 8 != 0
