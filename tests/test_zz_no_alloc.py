"""awq_gemm_noalloc (the entry point for callers that cannot allocate) against awq_gemm.

Both run the same plan and kernels, so their outputs must agree bit for bit; only the
split-K buffers differ (the library's static device array instead of the grown
workspace).  Each case makes two noalloc calls in a row on one stream, the second with
a smaller input, so the second call runs on what the first left in the shared array:
fixed-point words that must be back to zero and partials it overwrites.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import w4a16_weight_only_amd as awq
from w4a16_weight_only_amd import _lib, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    awq.load_library()


def _tensors(M, K, N, g, seed):
    d = synth.make_custom(M, K, N, g, bias=True, seed=seed)
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items() if isinstance(v, np.ndarray)}


def _call(name, t, M, K, N, g):
    lib = _lib.load()
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    st = getattr(lib, name)(t["x"].data_ptr(), t["qweight"].data_ptr(), t["qzeros"].data_ptr(),
                            t["scales"].data_ptr(), t["bias"].data_ptr(), M, K, N, g, y.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    return st, y


# (first, second): the second is smaller and runs the same family on what the first left.
PAIRS = [
    ((1, 4096, 4096, 128), (1, 2048, 1024, 128)),      # decode: fixed-point words
    ((2, 8192, 28672, 128), (2, 4096, 544, 64)),       # decode with a partial last tile
    ((3, 4096, 4096, 128), (3, 2048, 512, 128)),       # skinny: fp32 partials + reduce
    ((16, 4096, 4096, -1), (8, 2048, 1024, 128)),      # skinny at M 16 and 8
    ((64, 4096, 4096, 128), (64, 1024, 1024, 64)),     # tile: fp32 partials over K splits
    ((700, 4096, 4096, 128), (600, 4096, 2048, 128)),  # tile with a second launch over the last rows
    ((300, 1024, 768, 64), (256, 1024, 512, 64)),      # tile, 256-row tiles
    ((512, 4096, 14336, 128), (40, 96, 256, 32)),      # tile without split-K, then a ragged one
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_awq_gemm(first, second):
    for i, (M, K, N, g) in enumerate((first, second)):
        print(f"noalloc call {i}: M={M} K={K} N={N} g={g} plan={awq.plan(M, K, N, g)}", flush=True)
        t = _tensors(M, K, N, g, seed=M + K + N + i)
        st, y = _call("awq_gemm_noalloc", t, M, K, N, g)
        assert st == _lib.AWQ_OK, _lib.status_string(st)
        st_ref, y_ref = _call("awq_gemm", t, M, K, N, g)
        assert st_ref == _lib.AWQ_OK
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"call {i} differs from awq_gemm"


def test_noalloc_repeated_small_calls_are_deterministic():
    M, K, N, g = 1, 4096, 1024, 128
    t = _tensors(M, K, N, g, seed=5)
    outs = [_call("awq_gemm_noalloc", t, M, K, N, g)[1] for _ in range(3)]
    torch.cuda.synchronize()
    for y in outs[1:]:
        assert torch.equal(y.view(torch.int16), outs[0].view(torch.int16))


def test_noalloc_rejects_oversized_plan():
    """(2, 8192, 114688): the decode plan's fixed-point words need 2.75 MB, more than
    the 2 MiB word region; the call must fail cleanly and leave y untouched."""
    M, K, N, g = 2, 8192, 114688, 128
    p = awq.plan(M, K, N, g)
    assert p["family"] == "decode" and p["workspace_bytes"] > (2 << 20)
    t = {"x": torch.zeros(M, K, dtype=torch.float16, device="cuda"),
         "qweight": torch.zeros(K, N // 8, dtype=torch.int32, device="cuda"),
         "qzeros": torch.zeros(K // g, N // 8, dtype=torch.int32, device="cuda"),
         "scales": torch.ones(K // g, N, dtype=torch.float16, device="cuda"),
         "bias": torch.zeros(N, dtype=torch.float16, device="cuda")}
    st, y = _call("awq_gemm_noalloc", t, M, K, N, g)
    torch.cuda.synchronize()
    assert st == _lib.AWQ_ERR_UNSUPPORTED
    assert torch.isnan(y).all()
    # and the array is still usable afterwards
    test_noalloc_repeated_small_calls_are_deterministic()
