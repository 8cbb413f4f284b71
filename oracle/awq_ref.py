"""Plain CPU oracle for the fused AWQ W4A16 linear  y = x . dequant(W) + bias.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  The HIP library
never imports, links or calls it, and it shares no code, table or helper with
the HIP sources: the two sides meet only through the seeded input generator,
which holds none of the method's arithmetic.

Everything here is deliberately slow and literal: numpy integer ops for the
bit work, float32 for the dequantised weights (where the product is exact, see
`dequant_ref`) and float64 for the matrix product.

Sources (cited by page and section):
  [AWQ-SPEC]  tensref.org "AWQ" format page: the "Reader" pseudo-code
              (unpack with the order map, zero/scale row k // group_size,
              dequant (code - zero) * scale) and the "Reject the file when"
              rules AWQ-004 (order map, not sequential nibbles) and AWQ-005
              (stored zero is subtracted as is, no +1).
  [GPTQM]     GPTQModel wiki "AWQ": section "Saved formats and packing"
              (GEMM shapes qweight [K, N/8], qzeros [K/G, N/8], scales [K/G, N];
              the INT4 order and reverse-order constants; INT4 packing rejects
              N not divisible by 8), section "Group quantization and zero
              points" (group_size -1 is one group across the row; GEMM
              dequant is (code - zero) * scale).
  [VLLM]      rkmt.cn article on vLLM's AWQ loading, sections 5.1 (reverse
              pack order [0,4,1,5,2,6,3,7]) and 5.3 (kernels unpack with
              (w >> shift) & 0xF, then (w - z) * s, before the matmul).

The RTN writer `quantize_rtn` (the step before this path: dense fp16 weights to
the GEMM layout) follows [GPTQM] "Group quantization and zero points", the table of
the asymmetric and symmetric quantizers.

Readings where the pages are silent (each is listed in the design notes):
  * group_size == -1 means G = 1 (one group spanning all K rows).
  * N % 8 != 0 and K % group_size != 0 are rejected, never truncated.
  * A stored int32 word may be negative; the nibbles are its two's-complement
    bits, extracted as if the word were unsigned.
  * Bias is added in float64 to the float64 product (one final rounding if the
    caller rounds to fp16).

Pins: every function here is pinned in tests/test_oracle.py against facts that
do not come from this file (a hand-built word, bijectivity, exact rational
arithmetic, closed-form special cases).  No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# Nibble i of a packed word holds column 8*c + AWQ_ORDER[i]   ([AWQ-SPEC] Reader;
# [GPTQM] "Saved formats and packing").
AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)
# Column j of a word sits at nibble AWQ_REVERSE[j]   ([GPTQM] same section; [VLLM] 5.1).
AWQ_REVERSE = (0, 4, 1, 5, 2, 6, 3, 7)


class AwqFormatError(ValueError):
    """A tensor set that the GEMM-format rules reject."""


def resolve_groups(K: int, group_size: int) -> tuple[int, int]:
    """Return (g, G): the effective group length and the number of groups.

    [GPTQM] "Group quantization and zero points": -1 is one group across the
    whole input row, so g = K and G = 1.  A positive g must divide K (reading:
    incompatible dimensions are rejected rather than padded).
    """
    if group_size == -1:
        return K, 1
    if group_size <= 0:
        raise AwqFormatError(f"group_size must be -1 or positive, got {group_size}")
    if K % group_size != 0:
        raise AwqFormatError(f"K={K} is not a multiple of group_size={group_size}")
    return group_size, K // group_size


def validate_pack(K, N, group_size, qweight_shape, qzeros_shape, scales_shape, bias_len=None):
    """Format rules of the GEMM pack ([GPTQM] "Saved formats and packing"; [AWQ-SPEC]).

    qweight int32 [K, N/8], qzeros int32 [G, N/8], scales [G, N], bias [N] or absent.
    Raises AwqFormatError on any mismatch.
    """
    if K < 1 or N < 1:
        raise AwqFormatError("K and N must be positive")
    if N % 8 != 0:
        raise AwqFormatError(f"N={N} is not a multiple of 8")
    _, G = resolve_groups(K, group_size)
    if tuple(qweight_shape) != (K, N // 8):
        raise AwqFormatError(f"qweight shape {tuple(qweight_shape)} != {(K, N // 8)}")
    if tuple(qzeros_shape) != (G, N // 8):
        raise AwqFormatError(f"qzeros shape {tuple(qzeros_shape)} != {(G, N // 8)}")
    if tuple(scales_shape) != (G, N):
        raise AwqFormatError(f"scales shape {tuple(scales_shape)} != {(G, N)}")
    if bias_len is not None and bias_len != N:
        raise AwqFormatError(f"bias length {bias_len} != N={N}")


def pack_awq(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes [R, N] (values 0..15) into int32 words [R, N/8].

    Writer side of the reader in [AWQ-SPEC]: the code of column 8c + ORDER[i]
    goes to bits 4i..4i+3 of word c.  Built in uint32 so the top nibble can
    set the sign bit, then reinterpreted as int32 (the stored container).
    """
    codes = np.asarray(codes)
    if codes.ndim != 2:
        raise AwqFormatError("codes must be 2-D")
    R, N = codes.shape
    if N % 8 != 0:
        raise AwqFormatError(f"N={N} is not a multiple of 8")
    if codes.size and (codes.min() < 0 or codes.max() > 15):
        raise AwqFormatError("codes must lie in 0..15")
    c = codes.astype(np.uint32)
    words = np.zeros((R, N // 8), dtype=np.uint32)
    for col in range(N // 8):
        for i in range(8):
            words[:, col] |= c[:, col * 8 + AWQ_ORDER[i]] << np.uint32(4 * i)
    return words.view(np.int32)


def unpack_awq(words: np.ndarray) -> np.ndarray:
    """Unpack int32 words [R, C] into codes [R, 8C].

    [AWQ-SPEC] Reader / [GPTQM] "Saved formats and packing": a word holds eight 4-bit
    codes, nibble i in bits 4i..4i+3, and nibble i is the code of column ORDER[i] of
    the word's eight columns.  So split every word into its nibble vector (taken
    from the unsigned bit pattern, so negative words read as their bits say) and
    place that vector's entries at positions ORDER along the column axis.
    """
    w = np.asarray(words)
    u = w.view(np.uint32) if w.dtype == np.int32 else w.astype(np.int64).astype(np.uint32)
    R, C = u.shape
    shifts = np.uint32(4) * np.arange(8, dtype=np.uint32)
    nibbles = (u[:, :, None] >> shifts[None, None, :]) & np.uint32(0xF)  # [R, C, nibble]
    cols = np.empty((R, C, 8), dtype=np.int32)
    cols[:, :, list(AWQ_ORDER)] = nibbles  # column ORDER[i] of each word <- nibble i
    return cols.reshape(R, 8 * C)


def unpack_awq_gather(words: np.ndarray) -> np.ndarray:
    """Second, independent formulation of unpack: gather by output column.

    Column j reads word j // 8 at nibble REVERSE[j % 8]  ([GPTQM] reverse
    order constant; [VLLM] 5.1/5.3).  Uses Python integers per element: no
    shared loop structure with `unpack_awq`.
    """
    w = np.asarray(words)
    R, C = w.shape
    out = np.empty((R, 8 * C), dtype=np.int32)
    for r in range(R):
        for j in range(8 * C):
            word = int(w[r, j // 8]) & 0xFFFFFFFF
            out[r, j] = (word >> (4 * AWQ_REVERSE[j % 8])) & 0xF
    return out


def dequant_ref(qweight, qzeros, scales, group_size) -> np.ndarray:
    """Dequantised weight W [K, N] in float32:  W[k, n] = (q[k,n] - z[k//g, n]) * s[k//g, n].

    [AWQ-SPEC] Reader (dequant along in_features, group row k // group_size)
    and rule AWQ-005 (the stored zero is subtracted unchanged).
    (q - z) is an integer in [-15, 15] (at most 4 significant bits) and s is
    fp16 (11 significant bits), so the float32 product is exact: every
    evaluation order gives these same bits.
    Orientation [K, N] matches y = x . W; `dequant_ref_T` gives the page's [N, K].
    """
    q = unpack_awq(qweight)
    K, N = q.shape
    g, G = resolve_groups(K, group_size)
    z = unpack_awq(qzeros)
    s = np.asarray(scales)
    if z.shape != (G, N) or s.shape != (G, N):
        raise AwqFormatError("qzeros/scales shapes do not match K, N, group_size")
    grp = np.arange(K) // g  # the group row of every input row
    return (q.astype(np.float32) - z[grp].astype(np.float32)) * s[grp].astype(np.float32)


def dequant_ref_T(qweight, qzeros, scales, group_size) -> np.ndarray:
    """The same weight in [AWQ-SPEC]'s orientation [N, K] (out_features first), built one
    quantization group at a time: the g rows of group i share zero row i and scale row i."""
    q = unpack_awq(qweight)
    K, N = q.shape
    g, G = resolve_groups(K, group_size)
    z = unpack_awq(qzeros)
    s = np.asarray(scales)
    out = np.empty((N, K), dtype=np.float32)
    for i in range(G):
        block = (q[i * g:(i + 1) * g].astype(np.float32) - z[i].astype(np.float32)) * s[i].astype(np.float32)
        out[:, i * g:(i + 1) * g] = block.T
    return out


def gemm_ref(x, qweight, qzeros, scales, bias, group_size) -> np.ndarray:
    """y = x . dequant(W) + bias, in float64, shape [M, N].

    The fused linear of the GPU-serving blog (section 1.2: the packed weight
    is unpacked and dequantised, then multiplied with 16-bit activations) with
    the dequant of [AWQ-SPEC].  x (fp16) and W (exact fp32) convert to float64
    exactly; the matmul is a library primitive; bias is optional ([AWQ-SPEC]
    tensor table: fp16 [out_features], optional).
    """
    x = np.asarray(x)
    W = dequant_ref(qweight, qzeros, scales, group_size).astype(np.float64)
    if x.ndim != 2 or x.shape[1] != W.shape[0]:
        raise AwqFormatError(f"x shape {x.shape} does not match K={W.shape[0]}")
    y = x.astype(np.float64) @ W
    if bias is not None:
        y = y + np.asarray(bias).astype(np.float64)[None, :]
    return y


def gemm_ref_ieee(x, qweight, qzeros, scales, bias, group_size) -> np.ndarray:
    """gemm_ref for inputs that may hold NaN or infinities (in x, scales or bias).

    The value is still the exact sum of the products x[m, k] * W[k, n] plus bias; for
    non-finite terms IEEE-754 fixes it: a product with a NaN factor, or an infinity
    times zero, is NaN; an infinite term makes the sum that infinity, and infinities
    of both signs (or a NaN term) make it NaN.  A float64 matmul library does not
    promise these rules, so here only the products of two finite factors go through
    the matmul; every product with a non-finite factor is formed elementwise and added
    afterwards (IEEE addition then applies the rules above).
    """
    x = np.asarray(x).astype(np.float64)
    W = dequant_ref(qweight, qzeros, scales, group_size).astype(np.float64)
    if x.ndim != 2 or x.shape[1] != W.shape[0]:
        raise AwqFormatError(f"x shape {x.shape} does not match K={W.shape[0]}")
    fin_x = np.isfinite(x)
    fin_w = np.isfinite(W)
    y = np.where(fin_x, x, 0.0) @ np.where(fin_w, W, 0.0)
    with np.errstate(invalid="ignore"):
        for m, k in zip(*np.nonzero(~fin_x)):  # non-finite x: its whole weight row
            y[m, :] = y[m, :] + x[m, k] * W[k, :]
        for k, n in zip(*np.nonzero(~fin_w)):  # non-finite weight, finite x rows only
            rows = fin_x[:, k]
            y[rows, n] = y[rows, n] + x[rows, k] * W[k, n]
        if bias is not None:
            y = y + np.asarray(bias).astype(np.float64)[None, :]
    return y


def gemm_ref_entries(x, qweight, qzeros, scales, bias, group_size, rows, cols) -> np.ndarray:
    """y[rows[i], cols[i]] one entry at a time (for sampled checks at large sizes).

    Each entry unpacks only column cols[i]: nibble REVERSE[n % 8] of word n // 8
    in every row ([GPTQM] reverse order), dequantises with the group row
    k // g, and takes a float64 dot product with x[rows[i]].
    """
    x = np.asarray(x)
    qw = np.asarray(qweight).view(np.uint32)
    qz = np.asarray(qzeros).view(np.uint32)
    s = np.asarray(scales)
    K = qw.shape[0]
    g, _ = resolve_groups(K, group_size)
    gi = np.arange(K) // g
    out = np.empty(len(rows), dtype=np.float64)
    for t, (m, n) in enumerate(zip(rows, cols)):
        shift = np.uint32(4 * AWQ_REVERSE[n % 8])
        q = ((qw[:, n // 8] >> shift) & np.uint32(0xF)).astype(np.float64)
        z = ((qz[:, n // 8] >> shift) & np.uint32(0xF)).astype(np.float64)[gi]
        w = (q - z) * s[gi, n].astype(np.float64)
        acc = float(np.dot(x[m].astype(np.float64), w))
        if bias is not None:
            acc += float(np.asarray(bias)[n])
        out[t] = acc
    return out


def fp16_rne(a) -> np.ndarray:
    """Round to IEEE binary16, nearest-even (numpy's cast), for exact-output pins."""
    return np.asarray(a).astype(np.float16)


# bfloat16 activations.  The GEMM kernel's declared contract takes FP16 or BF16
# inputs ([GPTQM] "Selection and compatibility", kernel table).  bfloat16 is the
# upper half of an IEEE binary32: sign, 8 exponent bits, 7 fraction bits.  numpy
# has no bfloat16 type, so values travel as their 16-bit patterns (uint16).

def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: the pattern is the top half of a binary32."""
    b = np.asarray(bits).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_bf16_rne(a) -> np.ndarray:
    """Round binary32 values to bfloat16, nearest with ties to even, as bit patterns.

    The 16 low bits are dropped after adding 0x7FFF plus the lowest kept bit: below
    halfway the carry never reaches the kept bits, above it always does, and at
    exactly halfway it does only when the kept value is odd.  Overflow of the
    largest finite values goes to infinity through the exponent, as in IEEE.  NaN
    inputs keep their sign and become the quiet NaN 0x7FC0."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint32) & np.uint32(0xFFFF)
    nan = np.isnan(f)
    sign = (u >> np.uint64(16)).astype(np.uint32) & np.uint32(0x8000)
    r = np.where(nan, sign | np.uint32(0x7FC0), r)
    return r.astype(np.uint16)


def gemm_ref_bf16(x_bits, qweight, qzeros, scales, bias_bits, group_size) -> np.ndarray:
    """gemm_ref with bfloat16 x and bias (bit patterns): both widen exactly to float64;
    the weights are the same fp16-scaled dequant, and the product is float64."""
    x = bf16_to_f64(x_bits)
    bias = None if bias_bits is None else bf16_to_f64(bias_bits)
    return gemm_ref(x, qweight, qzeros, scales, bias, group_size)


# Routed experts.  vLLM's AWQ support sends a routed-expert (MoE) layer to a 4-bit
# WNA16 MoE kernel over per-expert qweight / qzeros / scales ([VLLM] section 5.4).
# Reading taken: each routed slot s (token t = s // topk, its choice s % topk)
# multiplies that token's activations by its expert's dequantised weight; the
# expert's activation function and the weighted sum over the topk choices come
# after this product and are not part of it.

def moe_align_ref(expert_ids, num_experts: int):
    """Counting sort of routed slots by expert (stable: slot order within an expert).

    Returns (offsets [E + 1], sorted_slots [S]): the slots of expert e are
    sorted_slots[offsets[e] : offsets[e + 1]], in increasing slot order."""
    ids = np.asarray(expert_ids).astype(np.int64).ravel()
    if ids.size and (ids.min() < 0 or ids.max() >= num_experts):
        raise AwqFormatError("expert id out of range")
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in ids:
        counts[e] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    sorted_slots = np.empty(ids.size, dtype=np.int64)
    for s, e in enumerate(ids):
        sorted_slots[cursor[e]] = s
        cursor[e] += 1
    return offsets, sorted_slots


def moe_gemm_ref(x, qweights, qzeros, scales, expert_ids, topk: int, group_size: int) -> np.ndarray:
    """y[s] = x[s // topk] . dequant(W[expert_ids[s]]) in float64, shape [S, N].

    qweights / qzeros / scales are stacked per expert ([E, K, N/8], [E, G, N/8],
    [E, G, N]); each expert's product is gemm_ref on the rows routed to it."""
    x = np.asarray(x)
    ids = np.asarray(expert_ids).astype(np.int64).ravel()
    E = np.asarray(qweights).shape[0]
    N = np.asarray(scales).shape[2]
    if ids.size != x.shape[0] * topk:
        raise AwqFormatError("expert_ids must hold topk entries per token")
    y = np.zeros((ids.size, N), dtype=np.float64)
    for e in range(E):
        rows = np.nonzero(ids == e)[0]
        if rows.size:
            y[rows] = gemm_ref(x[rows // topk], qweights[e], qzeros[e], scales[e], None, group_size)
    return y


def quantize_rtn(W, group_size: int, sym: bool = False):
    """Round-to-nearest writer: fp16 W [K, N] -> (qweight [K, N/8], qzeros [G, N/8],
    scales fp16 [G, N]) in the GEMM layout, so that dequant_ref gives back
    (code - zero) * scale.

    [GPTQM] "Group quantization and zero points", per group of g input rows k and
    per output column n (W is in the orientation of dequant_ref, [K, N]):
      asymmetric: scale = max(max - min, 1e-5) / 15,  zero = clamp(-round(min / scale), 0, 15),
                  code  = clamp(round(w / scale) + zero, 0, 15);
      symmetric:  scale = max(max |w|, 1e-5) / 7, signed code = clamp(round(w / scale), -8, 7),
                  stored as code + 8 with zero = 8.
    Readings (the pages give the formulas, not the arithmetic): the scale is
    computed in float32 and rounded once to the stored fp16 value, and every later
    step (min / scale, w / scale) divides by that stored value in float32; round is
    to nearest, ties to even.  A writer thus picks the codes for the scale a reader
    will actually use.
    """
    W = np.asarray(W)
    if W.dtype != np.float16 or W.ndim != 2:
        raise AwqFormatError("W must be a 2-D fp16 array [K, N]")
    K, N = W.shape
    if N % 8 != 0:
        raise AwqFormatError(f"N={N} is not a multiple of 8")
    g, G = resolve_groups(K, group_size)
    Wg = W.astype(np.float32).reshape(G, g, N)
    if sym:
        amax = np.abs(Wg).max(axis=1)
        s32 = np.maximum(amax, np.float32(1e-5)) / np.float32(7)
        scales = s32.astype(np.float16)
        sf = scales.astype(np.float32)
        codes = np.clip(np.rint(Wg / sf[:, None, :]), -8, 7) + 8
        zeros = np.full((G, N), 8.0, dtype=np.float32)
    else:
        mx = Wg.max(axis=1)
        mn = Wg.min(axis=1)
        s32 = np.maximum(mx - mn, np.float32(1e-5)) / np.float32(15)
        scales = s32.astype(np.float16)
        sf = scales.astype(np.float32)
        zeros = np.clip(-np.rint(mn / sf), 0, 15)
        codes = np.clip(np.rint(Wg / sf[:, None, :]) + zeros[:, None, :], 0, 15)
    qweight = pack_awq(codes.reshape(K, N).astype(np.int64))
    qzeros = pack_awq(zeros.astype(np.int64))
    return qweight, qzeros, scales
