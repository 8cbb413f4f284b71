"""CPU tests of the C ABI: the library loads, exports what the header declares,
and its host-only checks return the documented statuses.  No device work."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import w4a16_weight_only_amd as awq
from w4a16_weight_only_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq_w4a16.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(awq_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libawq_w4a16.so is not built; run `python -m w4a16_weight_only_amd.build`")
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("awq_validate_pack", "awq_dequant", "awq_gemm", "awq_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), (names, sorted(_lib.SIGNATURES))
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_the_bench_probes():
    # The benchmark's read ceiling and launch floor come from this separate library (not
    # part of the AWQ ABI); bad arguments are rejected before any launch.
    path = os.path.join(ROOT, "w4a16_weight_only_amd", "libawq_probe.so")
    if not os.path.exists(path):
        pytest.fail("libawq_probe.so is not built; run `python -m w4a16_weight_only_amd.build`")
    probe = ctypes.CDLL(path)
    probe.awq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    probe.awq_probe_stream_read.restype = ctypes.c_int
    probe.awq_probe_empty.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.awq_probe_empty.restype = ctypes.c_int
    assert probe.awq_probe_stream_read(None, 16, None, None) != 0
    assert probe.awq_probe_empty(0, 256, ctypes.c_void_p(16), None) != 0
    assert probe.awq_probe_empty(1, 2048, ctypes.c_void_p(16), None) != 0
    assert probe.awq_probe_empty(1, 256, None, None) != 0


def test_status_strings(lib):
    for st in range(-6, 1):
        s = _lib.status_string(st)
        assert s.startswith("AWQ")
    assert "unknown" in _lib.status_string(-99)


def _validate(lib, K=4096, N=4096, g=128, qw=None, qz=None, sc=None, bias=-1):
    G = 1 if g == -1 else (K // g if g > 0 and K % g == 0 else 1)
    qw = qw or (K, N // 8)
    qz = qz or (G, N // 8)
    sc = sc or (G, N)
    return lib.awq_validate_pack(K, N, g, *qw, *qz, *sc, bias)


def test_validate_pack_rules(lib):
    assert _validate(lib) == _lib.AWQ_OK
    assert _validate(lib, bias=4096) == _lib.AWQ_OK
    assert _validate(lib, g=-1) == _lib.AWQ_OK
    assert _validate(lib, K=11008, N=4096, g=64) == _lib.AWQ_OK
    assert _validate(lib, N=4100) == _lib.AWQ_ERR_SHAPE            # N % 8
    assert _validate(lib, g=100) == _lib.AWQ_ERR_GROUP             # K % g
    assert _validate(lib, g=0) == _lib.AWQ_ERR_GROUP
    assert _validate(lib, g=-2) == _lib.AWQ_ERR_GROUP
    assert _validate(lib, qw=(512, 4096)) == _lib.AWQ_ERR_SHAPE    # transposed qweight
    assert _validate(lib, qz=(32, 4096)) == _lib.AWQ_ERR_SHAPE     # unpacked zeros
    assert _validate(lib, sc=(4096, 32)) == _lib.AWQ_ERR_SHAPE     # transposed scales
    assert _validate(lib, bias=4095) == _lib.AWQ_ERR_SHAPE
    assert _validate(lib, K=0) == _lib.AWQ_ERR_SHAPE


def test_kernel_limits(lib):
    assert lib.awq_check_limits(1, 4096, 4096, 128) == _lib.AWQ_OK
    assert lib.awq_check_limits(1, 4096, 4096, -1) == _lib.AWQ_OK
    assert lib.awq_check_limits(0, 4096, 4096, 128) == _lib.AWQ_OK
    assert lib.awq_check_limits(-1, 4096, 4096, 128) == _lib.AWQ_ERR_SHAPE
    assert lib.awq_check_limits(1, 4096, 4104, 8) == _lib.AWQ_ERR_UNSUPPORTED   # N % 32, g % 32
    assert lib.awq_check_limits(1, 4112, 4096, -1) == _lib.AWQ_ERR_UNSUPPORTED  # K % 32
    assert lib.awq_check_limits(1, 4096, 4096, 16) == _lib.AWQ_ERR_UNSUPPORTED  # group 16
    assert lib.awq_check_limits(1, 1 << 25, 4096, -1) == _lib.AWQ_ERR_UNSUPPORTED
    # 256-row tiles address x rows with 32-bit byte offsets: K below 2^23 above 128 rows
    assert lib.awq_check_limits(200, 1 << 23, 4096, -1) == _lib.AWQ_ERR_UNSUPPORTED
    assert lib.awq_check_limits(100, (1 << 23) + 1024, 4096, -1) == _lib.AWQ_OK
    assert lib.awq_moe_tiles(1 << 40, 8, 64) == -1
    assert lib.awq_moe_tiles(100, 8, 64) == 2 + 8


def test_plan_families():
    p1 = awq.plan(1, 4096, 4096, 128)
    assert p1["family"] == "decode" and p1["splits"] > 1 and p1["workspace_bytes"] > 0
    # 256-column tiles, eight 32-row k-steps per workgroup: 16 x 16 workgroups
    assert p1["grid"] == (16, 16) and p1["block"] == 256
    p16 = awq.plan(16, 4096, 11008, 128)
    assert p16["family"] == "skinny"
    assert awq.plan(2, 4096, 4096, 128)["family"] == "decode"
    assert awq.plan(4, 4096, 4096, 128)["family"] == "decode"
    assert awq.plan(5, 4096, 4096, 128)["family"] == "skinny"
    assert awq.plan(3, 8192, 16384, 128)["family"] == "skinny"   # wide and large: the skinny family
    assert awq.plan(4, 28672, 8192, 128)["family"] == "decode"
    # 256-column tiles: two k-steps per wave for g = 64, one for g = 32; past 127 splits
    # of those, 512-column tiles with two k-steps per wave on eight waves; beyond the
    # split limit (127) the older skinny family takes small M.
    assert awq.plan(1, 11008, 4096, 64)["grid"] == (16, 43) and awq.plan(1, 11008, 4096, 64)["block"] == 256
    assert awq.plan(1, 11008, 4096, 32)["grid"] == (16, 86) and awq.plan(1, 11008, 4096, 32)["block"] == 256
    assert awq.plan(1, 40960, 4096, 64)["grid"] == (8, 80) and awq.plan(1, 40960, 4096, 64)["block"] == 512
    assert awq.plan(1, 16384, 4096, 128)["grid"] == (16, 64)
    assert awq.plan(1, 131072, 64, -1)["family"] == "skinny"
    assert awq.plan(2, 98304, 128, 64)["family"] == "skinny"
    assert awq.plan(17, 4096, 4096, 128)["family"] == "tile"
    p2048 = awq.plan(2048, 4096, 4096, 128)
    assert p2048["family"] == "tile" and p2048["workspace_bytes"] == 0 and p2048["splits"] == 1
    assert p2048["grid"] == (8 * 32, 1)  # 8 x 32 tiles: the XCD runs need no padding


def tile_blocks(M, N, tile_rows, tile_cols):
    """Launched tile grid: the column tiles sharing a 128-byte weight line (256 //
    tile_cols of them) form a run; row tiles x runs, padded to whole groups of 8 runs
    (one per XCD), each of 256 // tile_cols blocks."""
    ct = 256 // tile_cols
    units = -(-M // tile_rows) * -(-(-(-N // tile_cols)) // ct)
    return 8 * ct * -(-units // 8)


@pytest.mark.parametrize("M,K,N,g,tile_rows,tile_cols", [
    (64, 11008, 4096, 64, 64, 128), (512, 11008, 4096, 64, 256, 128), (100, 2080, 160, -1, 64, 128)])
def test_tile_split_k_plans(M, K, N, g, tile_rows, tile_cols):
    """The tile family splits K on few tiles: grid (tile blocks, splits), every split
    keeps >= 8 k-tiles of 64 (or there is one split), the splits cover K exactly, and
    the fp32 partial workspace holds splits x M x N."""
    p = awq.plan(M, K, N, g)
    tiles = -(-M // tile_rows) * -(-N // tile_cols)
    kt = -(-K // 64)
    assert p["family"] == "tile" and p["grid"][0] == tile_blocks(M, N, tile_rows, tile_cols)
    assert p["grid"][1] == p["splits"]
    assert p["splits"] > 1
    kps = -(-kt // p["splits"])
    assert kps >= 8 or p["splits"] == 1
    assert -(-kt // kps) == p["splits"]
    assert tiles * p["splits"] >= 192 or p["splits"] == max(1, kt // 8)
    assert p["workspace_bytes"] >= p["splits"] * M * N * 4
    with pytest.raises(ValueError):
        awq.plan(1, 4096, 4104, 128)


@pytest.mark.parametrize("M,K,N,tail_rows", [(2100, 4096, 4096, 52), (1100, 4096, 4096, 76),
                                              (2300, 4096, 4096, 252), (2049, 64, 4096, 1),
                                              (300, 4096, 4096, 0), (600, 4096, 11008, 0),
                                              (2100, 4096, 14336, 0), (2048, 4096, 4096, 0)])
def test_tile_second_launch(M, K, N, tail_rows):
    """A partly filled last 256-row tile goes to a second launch exactly when the
    256 x 128 workgroups (one per compute unit of 256) of the whole would take one
    more round than those of the full tiles; the first launch then covers the full
    tiles, the second the rest, and the workspace covers the larger of the two."""
    def launch(rows):
        bm, bn = (256, 128) if rows > 128 else ((64, 128) if rows > 32 else (32, 128))
        tiles = -(-rows // bm) * -(-N // bn)
        kt = -(-K // 64)
        if bm == 256:
            s = -(-256 // tiles) if tiles < 192 else 1
        else:
            s = max(1, 512 // tiles)
        s = min(s, max(1, kt // 8))
        s = -(-kt // -(-kt // s))
        return tiles * s, s, tile_blocks(rows, N, bm, bn)
    p = awq.plan(M, K, N, 128 if K >= 128 else -1)
    if tail_rows == 0:
        assert p["tail"] is None
        return
    full = M - tail_rows
    wg_all, _, _ = launch(M)
    wg_main, s_main, gx_main = launch(full)
    wg_tail, s_tail, gx_tail = launch(tail_rows)
    assert -(-wg_main // 256) < -(-wg_all // 256)
    assert p["grid"] == (gx_main, s_main) and p["splits"] == s_main
    assert p["tail"]["rows"] == tail_rows and p["tail"]["grid"] == (gx_tail, s_tail)
    need = max(s_main * full * N * 4 if s_main > 1 else 0, s_tail * tail_rows * N * 4 if s_tail > 1 else 0)
    assert p["workspace_bytes"] >= need


def test_gemm_argument_errors_touch_no_device(lib):
    """Checks run before any HIP call, so these are safe without a GPU."""
    p = ctypes.c_void_p(1 << 20)  # aligned dummy, never dereferenced
    # M == 0: nothing to do, no launch.
    assert lib.awq_gemm(p, p, p, p, None, 0, 4096, 4096, 128, p, None) == _lib.AWQ_OK
    assert lib.awq_gemm(None, p, p, p, None, 1, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_NULL
    assert lib.awq_gemm(p, p, p, p, None, 1, 4096, 4096, 128, None, None) == _lib.AWQ_ERR_NULL
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert lib.awq_gemm(odd, p, p, p, None, 1, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_ALIGN
    assert lib.awq_gemm(p, p, p, p, odd, 1, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_ALIGN
    assert lib.awq_gemm(p, p, p, p, None, 1, 4096, 4100, 128, p, None) == _lib.AWQ_ERR_SHAPE
    assert lib.awq_gemm(p, p, p, p, None, 1, 4096, 4096, 100, p, None) == _lib.AWQ_ERR_GROUP
    assert lib.awq_gemm(p, p, p, p, None, 1, 4096, 4096, 16, p, None) == _lib.AWQ_ERR_UNSUPPORTED
    assert lib.awq_dequant(None, p, p, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_NULL
    assert lib.awq_dequant(p, p, odd, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_ALIGN


def test_quantize_rtn_argument_errors_touch_no_device(lib):
    """The writer checks the format rules, sym, pointers and alignment before any HIP call."""
    p = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 2)
    q = lib.awq_quantize_rtn
    assert q(p, 4096, 4100, 128, 0, p, p, p, None) == _lib.AWQ_ERR_SHAPE
    assert q(p, 4096, 4096, 100, 0, p, p, p, None) == _lib.AWQ_ERR_GROUP
    assert q(p, 4096, 4096, 0, 0, p, p, p, None) == _lib.AWQ_ERR_GROUP
    assert q(p, 0, 4096, -1, 0, p, p, p, None) == _lib.AWQ_ERR_SHAPE
    assert q(p, 4096, 4096, 128, 2, p, p, p, None) == _lib.AWQ_ERR_SHAPE
    assert q(p, (1 << 24) + 128, 4096, 128, 0, p, p, p, None) == _lib.AWQ_ERR_UNSUPPORTED
    assert q(None, 4096, 4096, 128, 0, p, p, p, None) == _lib.AWQ_ERR_NULL
    assert q(p, 4096, 4096, 128, 0, p, p, None, None) == _lib.AWQ_ERR_NULL
    assert q(odd, 4096, 4096, 128, 0, p, p, p, None) == _lib.AWQ_ERR_ALIGN
    assert q(p, 4096, 4096, 128, 1, p, odd, p, None) == _lib.AWQ_ERR_ALIGN


def test_moe_and_bf16_argument_errors_touch_no_device(lib):
    """Routed-expert and bfloat16 entry points check their arguments before any HIP call."""
    p = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert lib.awq_moe_tiles(2048, 8, 256) == 8 + 8
    assert lib.awq_moe_tiles(1, 8, 32) == 1 + 8
    assert lib.awq_moe_tiles(10, 0, 32) == -1
    a = lib.awq_moe_align
    assert a(p, 10, 0, 32, p, p, p, None) == _lib.AWQ_ERR_SHAPE
    assert a(p, 10, 1025, 32, p, p, p, None) == _lib.AWQ_ERR_UNSUPPORTED
    assert a(None, 10, 8, 32, p, p, p, None) == _lib.AWQ_ERR_NULL
    assert a(p, 10, 8, 32, p, p, odd, None) == _lib.AWQ_ERR_ALIGN
    g = lib.awq_moe_gemm
    assert g(p, p, p, p, p, 0, 2, 8, 4096, 4096, 128, p, None) == _lib.AWQ_OK  # no tokens: nothing to do
    assert g(p, p, p, p, p, 4, 0, 8, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_SHAPE
    assert g(p, p, p, p, p, 4, 2, 2000, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_UNSUPPORTED
    assert g(p, p, p, p, p, 4, 2, 8, 4096, 4096, 100, p, None) == _lib.AWQ_ERR_GROUP
    assert g(p, p, p, p, None, 4, 2, 8, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_NULL
    assert g(odd, p, p, p, p, 4, 2, 8, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_ALIGN
    assert g(p, p, p, p, p, 1 << 20, 2, 8, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_UNSUPPORTED  # x >= 4 GiB
    b = lib.awq_gemm_bf16
    assert b(p, p, p, p, None, 0, 4096, 4096, 128, p, None) == _lib.AWQ_OK
    assert b(None, p, p, p, None, 1, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_NULL
    assert b(p, p, p, p, odd, 1, 4096, 4096, 128, p, None) == _lib.AWQ_ERR_ALIGN
    assert b(p, p, p, p, None, 1, 4096, 4096, 16, p, None) == _lib.AWQ_ERR_UNSUPPORTED


def test_quantization_config():
    cfg = {"quant_method": "awq", "bits": 4, "group_size": 64, "zero_point": True, "version": "gemm"}
    assert awq.group_size_from_config(cfg) == 64
    for bad in ({**cfg, "bits": 8}, {**cfg, "version": "gemv"}, {**cfg, "zero_point": False},
                {**cfg, "quant_method": "gptq"}):
        with pytest.raises(ValueError):
            awq.group_size_from_config(bad)
