"""Python boundary of the AWQ W4A16 linear: torch tensors in, C ABI calls out.

torch supplies device memory and the current stream; every arithmetic step runs
in libawq_w4a16.so.  Tensor layouts are the AWQ GEMM checkpoint layout
(tensref.org "AWQ" format page; GPTQModel wiki "AWQ", "Saved formats and packing"):
qweight int32 [K, N/8], qzeros int32 [G, N/8], scales fp16 [G, N], bias fp16 [N].
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_tensor(name, t, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def group_size_from_config(cfg: dict) -> int:
    """Accept a checkpoint's quantization_config for the 4-bit GEMM layout and return
    its group size.  Bit width and group size come from this metadata, not from the
    tensors (tensref.org "AWQ" format page, introduction); AWQ keeps zero points even
    for symmetric quantization (GPTQModel wiki "AWQ", "Group quantization and zero
    points"), so a config without zero points is not this layout."""
    method = str(cfg.get("quant_method", "awq")).lower()
    if method != "awq":
        raise ValueError(f"quant_method {method!r} is not awq")
    if int(cfg.get("bits", cfg.get("w_bit", 4))) != 4:
        raise ValueError("only 4-bit AWQ is supported")
    fmt = str(cfg.get("version", cfg.get("format", "gemm"))).lower()
    if fmt != "gemm":
        raise ValueError(f"checkpoint format {fmt!r} is not the GEMM layout")
    if not cfg.get("zero_point", True):
        raise ValueError("GEMM-layout AWQ checkpoints carry zero points")
    return int(cfg.get("group_size", cfg.get("q_group_size", 128)))


def validate(K: int, N: int, group_size: int, qweight, qzeros, scales, bias=None) -> None:
    """Format rules of the GEMM pack, checked by the library (host-only)."""
    lib = _lib.load()
    st = lib.awq_validate_pack(K, N, group_size, *qweight.shape, *qzeros.shape, *scales.shape,
                               -1 if bias is None else bias.numel())
    _lib.check(st, "awq_validate_pack")


def plan(M: int, K: int, N: int, group_size: int) -> dict:
    """The launch plan awq_gemm uses for a shape (host-only); tail: the second tile
    launch over the last rows, or None."""
    lib = _lib.load()
    vals = [ctypes.c_int() for _ in range(5)]
    ws = ctypes.c_int64()
    st = lib.awq_gemm_plan(M, K, N, group_size, *[ctypes.byref(v) for v in vals], ctypes.byref(ws))
    _lib.check(st, "awq_gemm_plan")
    fam, splits, gx, gy, block = (v.value for v in vals)
    rows = ctypes.c_int64()
    tv = [ctypes.c_int() for _ in range(4)]
    st = lib.awq_gemm_plan_tail(M, K, N, group_size, ctypes.byref(rows), *[ctypes.byref(v) for v in tv])
    _lib.check(st, "awq_gemm_plan_tail")
    tail = None
    if rows.value:
        tail = dict(rows=rows.value, splits=tv[0].value, grid=(tv[1].value, tv[2].value), block=tv[3].value)
    return dict(family={0: "skinny", 1: "tile", 2: "decode"}[fam], splits=splits, grid=(gx, gy), block=block,
                workspace_bytes=ws.value, tail=tail)


def awq_dequant(qweight: torch.Tensor, qzeros: torch.Tensor, scales: torch.Tensor,
                group_size: int = 128, out: torch.Tensor | None = None,
                dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """[K, N] = (q - z) * s: float32 bit-exact, or fp16 rounded once (dtype=torch.float16)."""
    if dtype not in (torch.float32, torch.float16):
        raise TypeError("dtype must be torch.float32 or torch.float16")
    _check_tensor("qweight", qweight, torch.int32)
    dev = qweight.device
    _check_tensor("qzeros", qzeros, torch.int32, dev)
    _check_tensor("scales", scales, torch.float16, dev)
    K, N = qweight.shape[0], qweight.shape[1] * 8
    validate(K, N, group_size, qweight, qzeros, scales)
    if out is None:
        out = torch.empty((K, N), dtype=dtype, device=dev)
    else:
        _check_tensor("out", out, dtype, dev)
        if tuple(out.shape) != (K, N):
            raise ValueError(f"out must be [{K}, {N}]")
    fn = _lib.load().awq_dequant if dtype == torch.float32 else _lib.load().awq_dequant_f16
    with torch.cuda.device(dev):
        st = fn(_ptr(qweight), _ptr(qzeros), _ptr(scales), K, N, group_size, _ptr(out), _stream(dev))
    _lib.check(st, "awq_dequant" if dtype == torch.float32 else "awq_dequant_f16")
    return out


def awq_quantize_rtn(w: torch.Tensor, group_size: int = 128, sym: bool = False,
                     out: tuple | None = None) -> tuple:
    """Round-to-nearest writer: fp16 w [K, N] (input by output features) ->
    (qweight int32 [K, N/8], qzeros int32 [G, N/8], scales fp16 [G, N]) in the GEMM
    layout.  out, if given, is such a triple to write into."""
    _check_tensor("w", w, torch.float16)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [K, N]")
    dev = w.device
    K, N = w.shape
    lib = _lib.load()
    if N % 8 != 0:
        _lib.check(_lib.AWQ_ERR_SHAPE, "awq_quantize_rtn")
    if group_size != -1 and (group_size <= 0 or K % group_size != 0):
        _lib.check(_lib.AWQ_ERR_GROUP, "awq_quantize_rtn")
    G = 1 if group_size == -1 else K // group_size
    if out is None:
        out = (torch.empty((K, N // 8), dtype=torch.int32, device=dev),
               torch.empty((G, N // 8), dtype=torch.int32, device=dev),
               torch.empty((G, N), dtype=torch.float16, device=dev))
    qweight, qzeros, scales = out
    for name, t, dt, shape in (("qweight", qweight, torch.int32, (K, N // 8)),
                               ("qzeros", qzeros, torch.int32, (G, N // 8)),
                               ("scales", scales, torch.float16, (G, N))):
        _check_tensor(name, t, dt, dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}")
    with torch.cuda.device(dev):
        st = lib.awq_quantize_rtn(_ptr(w), K, N, group_size, int(bool(sym)), _ptr(qweight), _ptr(qzeros),
                                  _ptr(scales), _stream(dev))
    _lib.check(st, "awq_quantize_rtn")
    return qweight, qzeros, scales


def awq_gemm(x: torch.Tensor, qweight: torch.Tensor, qzeros: torch.Tensor, scales: torch.Tensor,
             bias: torch.Tensor | None = None, group_size: int = 128,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """y = x . dequant(W) + bias with fp32 accumulation, in x's dtype: fp16, or
    bfloat16 (then bias and y are bfloat16 too; scales stay fp16).

    x may have leading dimensions; they are flattened into rows (as the pages'
    kernels do) and restored on the output."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    act = x.dtype if x.dtype in (torch.float16, torch.bfloat16) else torch.float16
    _check_tensor("x", x, act)
    dev = x.device
    _check_tensor("qweight", qweight, torch.int32, dev)
    _check_tensor("qzeros", qzeros, torch.int32, dev)
    _check_tensor("scales", scales, torch.float16, dev)
    if bias is not None:
        _check_tensor("bias", bias, act, dev)
    K, N = qweight.shape[0], qweight.shape[1] * 8
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} input features, qweight has {K}")
    validate(K, N, group_size, qweight, qzeros, scales, bias)
    lead = tuple(x.shape[:-1])
    M = 1
    for d in lead:
        M *= d
    if out is None:
        out = torch.empty(lead + (N,), dtype=act, device=dev)
    else:
        _check_tensor("out", out, act, dev)
        if tuple(out.shape) != lead + (N,):
            raise ValueError(f"out must be {lead + (N,)}")
    lib = _lib.load()
    fn, name = (lib.awq_gemm_bf16, "awq_gemm_bf16") if act == torch.bfloat16 else (lib.awq_gemm, "awq_gemm")
    with torch.cuda.device(dev):
        st = fn(_ptr(x), _ptr(qweight), _ptr(qzeros), _ptr(scales), _ptr(bias), M, K, N, group_size, _ptr(out),
                _stream(dev))
    _lib.check(st, name)
    return out


def awq_moe_align(expert_ids: torch.Tensor, num_experts: int, block_rows: int) -> tuple:
    """Counting sort of routed slots by expert: (offsets [E + 1], sorted_slots [S],
    tile_table [tiles, 4]) as int32 device tensors."""
    _check_tensor("expert_ids", expert_ids, torch.int32)
    dev = expert_ids.device
    S = expert_ids.numel()
    lib = _lib.load()
    tiles = lib.awq_moe_tiles(S, num_experts, block_rows)
    if tiles < 0:
        _lib.check(_lib.AWQ_ERR_SHAPE, "awq_moe_align")
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    sorted_slots = torch.full((max(S, 1),), -1, dtype=torch.int32, device=dev)[:S]
    table = torch.empty((tiles, 4), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        st = lib.awq_moe_align(_ptr(expert_ids), S, num_experts, block_rows, _ptr(offsets), _ptr(sorted_slots),
                               _ptr(table), _stream(dev))
    _lib.check(st, "awq_moe_align")
    return offsets, sorted_slots, table


def awq_moe_gemm(x: torch.Tensor, qweight: torch.Tensor, qzeros: torch.Tensor, scales: torch.Tensor,
                 expert_ids: torch.Tensor, group_size: int = 128, out: torch.Tensor | None = None) -> torch.Tensor:
    """Routed-expert product: x [T, K] fp16, stacked expert weights qweight [E, K, N/8],
    qzeros [E, G, N/8], scales [E, G, N], expert_ids int32 [T, topk] (or [T * topk]);
    returns y [T * topk, N] (slot s = t * topk + j) with y[s] = x[t] . dequant(W[id])."""
    _check_tensor("x", x, torch.float16)
    dev = x.device
    _check_tensor("qweight", qweight, torch.int32, dev)
    _check_tensor("qzeros", qzeros, torch.int32, dev)
    _check_tensor("scales", scales, torch.float16, dev)
    _check_tensor("expert_ids", expert_ids, torch.int32, dev)
    if x.dim() != 2 or qweight.dim() != 3 or qzeros.dim() != 3 or scales.dim() != 3:
        raise ValueError("x must be [T, K]; qweight, qzeros, scales stacked per expert")
    T, K = x.shape
    E, N = qweight.shape[0], qweight.shape[2] * 8
    if qweight.shape[1] != K or qzeros.shape[0] != E or scales.shape[0] != E:
        raise ValueError("expert weight shapes disagree with x")
    validate(K, N, group_size, qweight[0], qzeros[0], scales[0])
    S = expert_ids.numel()
    if T == 0 or S % T != 0:
        if T == 0 and S == 0:
            return torch.empty((0, N), dtype=torch.float16, device=dev) if out is None else out
        raise ValueError("expert_ids must hold the same number of experts for every token")
    topk = S // T
    if out is None:
        out = torch.empty((S, N), dtype=torch.float16, device=dev)
    else:
        _check_tensor("out", out, torch.float16, dev)
        if tuple(out.shape) != (S, N):
            raise ValueError(f"out must be [{S}, {N}]")
    with torch.cuda.device(dev):
        st = _lib.load().awq_moe_gemm(_ptr(x), _ptr(qweight), _ptr(qzeros), _ptr(scales), _ptr(expert_ids), T, topk,
                                      E, K, N, group_size, _ptr(out), _stream(dev))
    _lib.check(st, "awq_moe_gemm")
    return out


class AwqLinear(torch.nn.Module):
    """Inference-only linear layer holding one AWQ GEMM-layout weight."""

    def __init__(self, qweight, qzeros, scales, bias=None, group_size=128):
        super().__init__()
        self.register_buffer("qweight", qweight)
        self.register_buffer("qzeros", qzeros)
        self.register_buffer("scales", scales)
        self.register_buffer("bias", bias)
        self.group_size = group_size
        self.in_features = qweight.shape[0]
        self.out_features = qweight.shape[1] * 8

    def forward(self, x):
        return awq_gemm(x.contiguous(), self.qweight, self.qzeros, self.scales, self.bias, self.group_size)
