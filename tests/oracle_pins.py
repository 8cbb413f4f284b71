"""Pins for the CPU oracle: checks that fix its behaviour from outside itself.

Each `pin_*` takes the oracle module `o` and raises AssertionError if it is
wrong.  tests/test_oracle.py runs them on the real oracle (all must pass) and
on planted mutants of it (each mutant must fail at least one pin).

What a pin compares against never comes from the oracle under test:
  * hand-derived packed words (tests/golden/hand_words.json),
  * bijectivity of the pack on all 32-bit words,
  * exact rational arithmetic (fractions.Fraction) on tiny inputs,
  * closed-form special cases (identity input, integer weights, zero weights).
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(1000 + seed)


def _words(rng, shape):
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32).view(np.int32)


def pin_hand_words(o):
    """Packed values derived by hand from the order constant (golden fixture)."""
    with open(os.path.join(GOLDEN, "hand_words.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        codes = np.array([c["codes"]], dtype=np.int32)
        word = o.pack_awq(codes)
        assert word.shape == (1, 1) and word.dtype == np.int32
        assert int(word[0, 0]) == c["word_int32"], (c, hex(int(word[0, 0]) & 0xFFFFFFFF))
        assert int(c["word_hex"], 16) == (c["word_int32"] & 0xFFFFFFFF)
        back = o.unpack_awq(np.array([[c["word_int32"]]], dtype=np.int32))
        assert back.tolist() == [c["codes"]], (c, back)
        back2 = o.unpack_awq_gather(np.array([[c["word_int32"]]], dtype=np.int32))
        assert back2.tolist() == [c["codes"]], (c, back2)
        if "sequential_word_hex" in c:
            assert int(c["sequential_word_hex"], 16) != (int(word[0, 0]) & 0xFFFFFFFF)


def pin_permutation_inverse(o):
    """ORDER and REVERSE are inverse permutations of 0..7 (brute force)."""
    assert sorted(o.AWQ_ORDER) == list(range(8))
    assert sorted(o.AWQ_REVERSE) == list(range(8))
    for i in range(8):
        assert o.AWQ_REVERSE[o.AWQ_ORDER[i]] == i
        assert o.AWQ_ORDER[o.AWQ_REVERSE[i]] == i


def pin_roundtrip_codes(o):
    """unpack(pack(c)) == c for random codes of several shapes."""
    for seed in range(10):
        rng = _rng(seed)
        R = int(rng.integers(1, 9))
        N = 8 * int(rng.integers(1, 9))
        c = rng.integers(0, 16, size=(R, N)).astype(np.int32)
        w = o.pack_awq(c)
        assert w.shape == (R, N // 8) and w.dtype == np.int32
        assert np.array_equal(o.unpack_awq(w), c)


def pin_roundtrip_words(o):
    """pack(unpack(w)) == w for arbitrary 32-bit words, negatives included:
    unpack is a bijection, so random words are valid packs."""
    for seed in range(10):
        rng = _rng(seed)
        w = _words(rng, (5, 7))
        w[0, 0] = np.int32(-1)
        w[0, 1] = np.int32(-(2 ** 31))
        c = o.unpack_awq(w)
        assert c.min() >= 0 and c.max() <= 15
        assert np.array_equal(o.pack_awq(c), w)


def pin_two_unpacks_agree(o):
    """The reader's scatter form and the reverse-order gather form agree."""
    rng = _rng(3)
    w = _words(rng, (6, 5))
    assert np.array_equal(o.unpack_awq(w), o.unpack_awq_gather(w))


def pin_no_plus_one(o):
    """Rule AWQ-005: dequant subtracts the stored zero unchanged, so q == z gives
    0 and q == z + 1 gives exactly the scale, for every (q, z) pair."""
    q = np.array([[a for a in range(16) for _ in range(16)]], dtype=np.int32)  # [1, 256]
    z = np.array([[b for _ in range(16) for b in range(16)]], dtype=np.int32)
    s = np.full((1, 256), 0.0078125, dtype=np.float16)  # 2^-7
    qw = o.pack_awq(q)
    qz = o.pack_awq(z)
    W = o.dequant_ref(qw, qz, s, -1)
    assert W.dtype == np.float32 and W.shape == (1, 256)
    for j in range(256):
        a, b = int(q[0, j]), int(z[0, j])
        assert W[0, j] == np.float32((a - b) * 0.0078125), (a, b, W[0, j])
        if a == b:
            assert W[0, j] == 0.0
        if a == b + 1:
            assert W[0, j] == np.float32(0.0078125)


def pin_fp32_product_exact():
    """Closed form behind bit-exact dequant: (q - z) in [-15, 15] times any finite
    fp16 scale is exact in float32 (4 + 11 significant bits <= 24).  Checked
    over all 31 differences and all finite fp16 values; the float64 product is
    exact by the same argument (<= 53 bits), and a sample is re-checked with
    Fractions."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    s16 = bits.view(np.float16)
    s16 = s16[np.isfinite(s16)]
    s32 = s16.astype(np.float32)
    s64 = s16.astype(np.float64)
    for d in range(-15, 16):
        p32 = np.float32(d) * s32
        assert np.array_equal(p32.astype(np.float64), np.float64(d) * s64)
    rng = _rng(7)
    for v in rng.choice(s16, size=200, replace=False):
        for d in (-15, -7, 1, 13):
            assert Fraction(float(np.float32(d) * np.float32(v))) == d * Fraction(float(v))


def _brute_force_y(x, codes, zeros, scales, bias, g):
    """Exact rational y = x . ((codes - zeros[k//g]) * scales[k//g]) + bias."""
    M, K = x.shape
    N = codes.shape[1]
    xs = [[Fraction(float(x[m, k])) for k in range(K)] for m in range(M)]
    y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                gi = k // g
                w = (int(codes[k, n]) - int(zeros[gi, n])) * Fraction(float(scales[gi, n]))
                acc += xs[m][k] * w
            if bias is not None:
                acc += Fraction(float(bias[n]))
            y[m][n] = acc
    return y


def pin_brute_force_gemm(o):
    """gemm_ref against exact rational arithmetic on tiny inputs, for several
    group sizes (one group per row via -1 included) and negative scales.
    x, the codes and the zeros are taken from plain integer/float matrices;
    only the packed words the oracle reads come from its packer, which the
    hand-word pin fixes independently."""
    cases = [(3, 8, 16, 8), (3, 16, 16, 4), (2, 16, 24, -1), (3, 16, 16, 16), (1, 32, 8, 8)]
    for t, (M, K, N, g) in enumerate(cases):
        rng = _rng(20 + t)
        gg = K if g == -1 else g
        G = K // gg
        codes = rng.integers(0, 16, size=(K, N)).astype(np.int32)
        zeros = rng.integers(0, 16, size=(G, N)).astype(np.int32)
        scales = (rng.uniform(1e-3, 2e-2, size=(G, N)) * rng.choice([-1, 1], size=(G, N))).astype(np.float16)
        x = rng.standard_normal((M, K)).astype(np.float16)
        bias = rng.normal(0, 0.5, size=N).astype(np.float16) if t % 2 == 0 else None
        y = o.gemm_ref(x, o.pack_awq(codes), o.pack_awq(zeros), scales, bias, g)
        assert y.shape == (M, N) and y.dtype == np.float64
        exact = _brute_force_y(x, codes, zeros, scales, bias, gg)
        for m in range(M):
            for n in range(N):
                e = float(exact[m][n])
                assert abs(y[m, n] - e) <= 1e-12 * max(1.0, abs(e)), (t, m, n, y[m, n], e)
        # dequant alone, exact: W[k, n] must equal the rational value bit for bit
        W = o.dequant_ref(o.pack_awq(codes), o.pack_awq(zeros), scales, g)
        for k in range(K):
            for n in range(N):
                gi = k // gg
                e = (int(codes[k, n]) - int(zeros[gi, n])) * Fraction(float(scales[gi, n]))
                assert Fraction(float(W[k, n])) == e, (t, k, n)


def _ieee_brute_force(x, codes, zeros, scales, bias, g):
    """y by Python float (IEEE binary64) arithmetic, one product and one add at a time:
    the reference semantics of non-finite values, independent of any array library."""
    M, K = x.shape
    N = codes.shape[1]
    y = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                w = float(int(codes[k, n]) - int(zeros[k // g, n])) * float(scales[k // g, n])
                acc = acc + float(x[m, k]) * w
            if bias is not None:
                acc = acc + float(bias[n])
            y[m, n] = acc
    return y


def pin_gemm_ieee(o):
    """gemm_ref_ieee against an elementwise IEEE-754 triple loop on tiny layers that hold
    NaN, +inf and -inf in x (some of them against zero weights, inf * 0 = NaN), an
    infinite scale and a NaN bias entry; on finite inputs it equals gemm_ref."""
    M, K, N, g = 4, 16, 16, 8
    rng = _rng(31)
    codes = rng.integers(0, 16, size=(K, N)).astype(np.int32)
    zeros = rng.integers(0, 16, size=(K // g, N)).astype(np.int32)
    codes[3, :4] = zeros[0, :4]  # zero weights in row 3, columns 0..3
    scales = rng.uniform(1e-3, 2e-2, size=(K // g, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    bias = rng.normal(0, 0.5, size=N).astype(np.float16)
    qw, qz = o.pack_awq(codes), o.pack_awq(zeros)
    fin = o.gemm_ref_ieee(x, qw, qz, scales, bias, g)
    assert np.allclose(fin, o.gemm_ref(x, qw, qz, scales, bias, g), rtol=1e-12, atol=1e-12)
    x[0, 3] = np.inf          # row 0: +inf against row 3 (zero weights in columns 0..3)
    x[1, 5] = np.nan          # row 1: NaN everywhere
    x[2, 2] = np.inf          # row 2: +inf and -inf
    x[2, 12] = -np.inf
    # column 9 of rows 8..15: +inf weights (scale inf, q - z = 7); row 3 multiplies
    # them by positive x and by +inf at k = 10, so y[3, 9] = +inf exactly
    zeros[1, 9] = 3
    codes[8:16, 9] = 10
    x[3, 8:16] = np.abs(x[3, 8:16]) + np.float16(0.5)
    x[3, 10] = np.inf
    qw, qz = o.pack_awq(codes), o.pack_awq(zeros)
    scales[1, 9] = np.inf
    bias[14] = np.nan         # column 14: NaN bias
    y = o.gemm_ref_ieee(x, qw, qz, scales, bias, g)
    with np.errstate(invalid="ignore", over="ignore"):
        e = _ieee_brute_force(x, codes, zeros, scales, bias, g)
    assert np.array_equal(np.isnan(y), np.isnan(e))
    assert np.array_equal(np.isinf(y), np.isinf(e))
    assert np.array_equal(np.sign(y[np.isinf(y)]), np.sign(e[np.isinf(e)]))
    f = np.isfinite(e)
    assert np.allclose(y[f], e[f], rtol=1e-12, atol=1e-12)
    # the constructed cases really occur
    assert np.isnan(y[1]).all() and np.isnan(y[:, 14]).all()
    assert np.isnan(y[0, :4]).all() and np.isinf(y[0, 4:8]).any()
    assert np.isnan(y[2]).any() and np.isinf(y).sum() > 4 and y[3, 9] == np.inf


def pin_dequant_orientation(o):
    """The page's reader returns [out_features, in_features]; ours is its transpose."""
    rng = _rng(5)
    K, N, g = 16, 24, 4
    qw, qz = _words(rng, (K, N // 8)), _words(rng, (K // g, N // 8))
    s = rng.uniform(-1, 1, size=(K // g, N)).astype(np.float16)
    a = o.dequant_ref(qw, qz, s, g)
    b = o.dequant_ref_T(qw, qz, s, g)
    assert a.shape == (K, N) and b.shape == (N, K)
    assert np.array_equal(a.T, b)


def pin_special_cases(o):
    """Closed forms: x = I gives W itself; integer weights give an integer
    matmul; codes == zeros gives y == bias; g = -1 equals g = K."""
    rng = _rng(9)
    K, N = 32, 16
    qw, qz = _words(rng, (K, N // 8)), _words(rng, (1, N // 8))
    s = rng.uniform(1e-3, 2e-2, size=(1, N)).astype(np.float16)
    W = o.dequant_ref(qw, qz, s, -1).astype(np.float64)
    y = o.gemm_ref(np.eye(K, dtype=np.float16), qw, qz, s, None, -1)
    assert np.array_equal(y, W)
    # integer weights: s = 1, z = 0, x in {-1, 0, 1}
    codes = rng.integers(0, 16, size=(K, N)).astype(np.int32)
    zero_codes = np.zeros((1, N), dtype=np.int32)
    x = rng.integers(-1, 2, size=(5, K))
    y = o.gemm_ref(x.astype(np.float16), o.pack_awq(codes), o.pack_awq(zero_codes),
                   np.ones((1, N), np.float16), None, -1)
    assert np.array_equal(y, (x.astype(np.int64) @ codes.astype(np.int64)).astype(np.float64))
    # codes == zeros in every group -> W == 0 -> y == bias
    g = 8
    zc = rng.integers(0, 16, size=(K // g, N)).astype(np.int32)
    codes = np.repeat(zc, g, axis=0)
    bias = rng.normal(0, 1, size=N).astype(np.float16)
    s = rng.uniform(1e-3, 2e-2, size=(K // g, N)).astype(np.float16)
    xx = rng.standard_normal((3, K)).astype(np.float16)
    y = o.gemm_ref(xx, o.pack_awq(codes), o.pack_awq(zc), s, bias, g)
    assert np.array_equal(y, np.tile(bias.astype(np.float64), (3, 1)))
    # g = -1 and g = K are the same layer
    x2 = rng.standard_normal((2, K)).astype(np.float16)
    s1 = rng.uniform(1e-3, 2e-2, size=(1, N)).astype(np.float16)
    assert np.array_equal(o.gemm_ref(x2, qw, qz, s1, bias, -1), o.gemm_ref(x2, qw, qz, s1, bias, K))


def pin_entries_agree(o):
    """Entry-by-entry evaluation (used at large sizes) agrees with the full product."""
    rng = _rng(11)
    M, K, N, g = 3, 64, 40, 16
    qw, qz = _words(rng, (K, N // 8)), _words(rng, (K // g, N // 8))
    s = rng.uniform(1e-3, 2e-2, size=(K // g, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    b = rng.normal(0, 0.01, size=N).astype(np.float16)
    y = o.gemm_ref(x, qw, qz, s, b, g)
    rows = [m for m in range(M) for _ in range(N)]
    cols = [n for _ in range(M) for n in range(N)]
    e = o.gemm_ref_entries(x, qw, qz, s, b, g, rows, cols).reshape(M, N)
    assert np.allclose(e, y, rtol=1e-12, atol=1e-12)


def pin_format_rules(o):
    """Rejections the pages require: N % 8, K % g, shapes of every tensor."""
    ok = dict(K=64, N=32, group_size=16, qweight_shape=(64, 4), qzeros_shape=(4, 4),
              scales_shape=(4, 32), bias_len=32)
    o.validate_pack(**ok)
    o.validate_pack(**{**ok, "group_size": -1, "qzeros_shape": (1, 4), "scales_shape": (1, 32)})
    o.validate_pack(**{**ok, "bias_len": None})
    bad = [dict(N=36, qweight_shape=(64, 4), qzeros_shape=(4, 4), scales_shape=(4, 36), bias_len=36), dict(group_size=24), dict(group_size=0),
           dict(qweight_shape=(4, 64)), dict(qzeros_shape=(4, 32)), dict(scales_shape=(32, 4)),
           dict(bias_len=31), dict(K=0)]
    for b in bad:
        try:
            o.validate_pack(**{**ok, **b})
        except o.AwqFormatError:
            continue
        raise AssertionError(f"accepted bad layer {b}")
    for badcodes in (np.zeros((2, 12), np.int32), np.full((1, 8), 16, np.int32)):
        try:
            o.pack_awq(badcodes)
        except o.AwqFormatError:
            continue
        raise AssertionError("pack accepted an invalid code matrix")


def pin_fp16_rounding(o):
    """fp16_rne rounds once to the nearest binary16, ties to even, checked against
    values built from their definition: the binary16 neighbours of 1 are 1 and
    1 + 2^-10, so 1 + 2^-11 (a tie) goes to the even 1 and 1 + 3 * 2^-11 (a tie) to the
    even 1 + 2^-9; 0.1 lies in [2^-4, 2^-3) where the step is 2^-14, and 0.1 / 2^-14 =
    1638.4 rounds to 1638; exactly representable values, the signed zero and the largest
    finite value pass unchanged; just above the halfway point to 2^16 overflows."""
    from fractions import Fraction
    cases = [(1 + 2.0 ** -11, 1.0), (1 + 3 * 2.0 ** -11, 1 + 2.0 ** -9), (1 + 2.0 ** -11 + 2.0 ** -20, 1 + 2.0 ** -10),
             (-(1 + 2.0 ** -11), -1.0), (0.1, float(Fraction(1638, 2 ** 14))), (65504.0, 65504.0),
             (2.0 ** -24, 2.0 ** -24), (3 * 2.0 ** -26, 2.0 ** -24), (-0.0, -0.0)]
    got = o.fp16_rne(np.array([c for c, _ in cases], dtype=np.float32))
    for (c, want), g in zip(cases, got):
        assert g.dtype == np.float16
        assert float(g) == want and np.signbit(g) == np.signbit(want), (c, float(g), want)
    with np.errstate(over="ignore"):
        assert np.isinf(o.fp16_rne(np.float32(65520.0)))  # halfway to 2^16 rounds to even: overflow


def pin_bf16_conversion(o):
    """bfloat16 = the top 16 bits of a binary32 (sign, 8 exponent bits, 7 fraction
    bits).  Values below are built from that definition: 1.0 = 0x3F80 and the next
    value up is 1 + 2^-7 = 0x3F81, so 1 + 2^-8 is a tie that goes to the even 0x3F80
    and 1 + 3 * 2^-8 a tie that goes to the even 0x3F82; -2.5 = -1.25 * 2 = 0xC020;
    the smallest subnormal 0x0001 is 2^-133; the largest finite 0x7F7F is
    (2 - 2^-7) 2^127, and (2 - 2^-8) 2^127, halfway to 2^128, rounds to the even
    infinity 0x7F80."""
    wide = {0x3F80: 1.0, 0xC020: -2.5, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,
            0x3F81: 1 + 2.0 ** -7, 0x0000: 0.0}
    for b, v in wide.items():
        assert float(o.bf16_to_f64(np.uint16(b))) == v, hex(b)
    assert np.signbit(o.bf16_to_f64(np.uint16(0x8000))) and float(o.bf16_to_f64(np.uint16(0x8000))) == 0.0
    assert np.isinf(o.bf16_to_f64(np.uint16(0x7F80)))
    cases = [(1.0, 0x3F80), (-2.5, 0xC020), (1 + 2.0 ** -8, 0x3F80), (1 + 3 * 2.0 ** -8, 0x3F82),
             (1 + 2.0 ** -8 + 2.0 ** -20, 0x3F81), (1 + 2.0 ** -9, 0x3F80), (-(1 + 3 * 2.0 ** -8), 0xBF82),
             (2.0 ** -133, 0x0001), (1.5 * 2.0 ** -133, 0x0002), ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),
             ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F), (-0.0, 0x8000), (float("inf"), 0x7F80)]
    got = o.f32_to_bf16_rne(np.array([c for c, _ in cases], dtype=np.float32))
    for (c, want), g in zip(cases, got):
        assert int(g) == want, (c, hex(int(g)), hex(want))
    assert int(o.f32_to_bf16_rne(np.float32("nan"))) & 0x7FFF == 0x7FC0
    # Every non-NaN pattern survives widen -> round unchanged (widening is exact).
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ok = ~np.isnan(o.bf16_to_f64(allb))
    back = o.f32_to_bf16_rne(o.bf16_to_f64(allb).astype(np.float32))
    assert np.array_equal(back[ok], allb[ok])


def pin_gemm_bf16_widening(o):
    """gemm_ref_bf16 = gemm_ref on the exact values of the bit patterns: with x the
    bf16 patterns of small integers (exact in bf16) the two references agree bit for
    bit, and an identity x returns the dequantised weight."""
    rng = _rng(31)
    K, N, g = 64, 16, 32
    codes = rng.integers(0, 16, (K, N))
    zeros = rng.integers(0, 16, (K // g, N))
    scales = rng.uniform(1e-3, 2e-2, (K // g, N)).astype(np.float16)
    qw, qz = o.pack_awq(codes), o.pack_awq(zeros)
    xi = rng.integers(-3, 4, (5, K)).astype(np.float32)
    xb = (xi.view(np.uint32) >> np.uint32(16)).astype(np.uint16)  # small integers: exact top halves
    bias = rng.integers(-2, 3, N).astype(np.float32)
    bb = (bias.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(o.gemm_ref_bf16(xb, qw, qz, scales, bb, g), o.gemm_ref(xi, qw, qz, scales, bias, g))
    eye = (np.eye(K, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(o.gemm_ref_bf16(eye, qw, qz, scales, None, g), o.dequant_ref(qw, qz, scales, g))


def pin_moe_align(o):
    """A hand-worked routing: slots 0..5 to experts [2, 0, 2, 1, 0, 2] of 4 give counts
    [2, 1, 3, 0], offsets [0, 2, 3, 6, 6] and slots (1, 4 | 3 | 0, 2, 5), each expert's
    slots in increasing order; on random routings the result is a permutation whose
    segments hold exactly the slots of their expert, in increasing order."""
    off, srt = o.moe_align_ref([2, 0, 2, 1, 0, 2], 4)
    assert off.tolist() == [0, 2, 3, 6, 6] and srt.tolist() == [1, 4, 3, 0, 2, 5]
    rng = _rng(32)
    for S, E in ((1, 1), (37, 5), (500, 64)):
        ids = rng.integers(0, E, S)
        off, srt = o.moe_align_ref(ids, E)
        assert sorted(srt.tolist()) == list(range(S))
        for e in range(E):
            seg = srt[off[e]:off[e + 1]]
            assert (ids[seg] == e).all() and (np.diff(seg) > 0).all() and seg.size == (ids == e).sum()


def pin_moe_gemm(o):
    """One expert and topk = 1 is gemm_ref; relabelling the experts (with their weights)
    leaves y unchanged; and a tiny case matches an exact rational triple loop."""
    from fractions import Fraction
    rng = _rng(33)
    T, K, N, g, E, topk = 3, 16, 8, 8, 3, 2
    qw = np.stack([o.pack_awq(rng.integers(0, 16, (K, N))) for _ in range(E)])
    qz = np.stack([o.pack_awq(rng.integers(0, 16, (K // g, N))) for _ in range(E)])
    sc = rng.uniform(1e-3, 2e-2, (E, K // g, N)).astype(np.float16)
    x = rng.standard_normal((T, K)).astype(np.float16)
    ids = np.array([[0, 2], [1, 0], [2, 1]]).ravel()
    y = o.moe_gemm_ref(x, qw, qz, sc, ids, topk, g)
    assert np.array_equal(o.moe_gemm_ref(x, qw[:1], qz[:1], sc[:1], np.zeros(T, dtype=np.int64), 1, g),
                          o.gemm_ref(x, qw[0], qz[0], sc[0], None, g))
    perm = np.array([2, 0, 1])  # new label of old expert e is perm[e]
    inv = np.argsort(perm)
    assert np.array_equal(o.moe_gemm_ref(x, qw[inv], qz[inv], sc[inv], perm[ids], topk, g), y)
    for s in range(T * topk):
        e, t = ids[s], s // topk
        codes = o.unpack_awq(qw[e]); zeros = o.unpack_awq(qz[e])
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(x[t, k])) * (int(codes[k, n]) - int(zeros[k // g, n])) * \
                       Fraction(float(sc[e, k // g, n]))
            assert abs(float(acc) - y[s, n]) <= 1e-12 * max(1.0, abs(float(acc))), (s, n)


def pin_rtn_hand_example(o):
    """tests/golden/rtn_example.json: one group of 4 rows, 8 equal columns, worked by hand
    from the quantizer table (asymmetric and symmetric)."""
    import json
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rtn_example.json")))
    W = np.tile(np.array(gold["W_column"], dtype=np.float16)[:, None], (1, 8))
    for mode, sym in (("asymmetric", False), ("symmetric", True)):
        qw, qz, sc = o.quantize_rtn(W, gold["group_size"], sym=sym)
        codes = o.unpack_awq(qw)
        assert (codes == np.array(gold[mode]["codes"])[:, None]).all(), (mode, codes[:, 0])
        assert (o.unpack_awq(qz) == gold[mode]["zero"]).all(), mode
        assert (sc.view(np.uint16) == int(gold[mode]["scale_bits"], 16)).all(), (mode, hex(sc.view(np.uint16)[0, 0]))


def pin_rtn_roundtrip(o):
    """A layer that is already on the quantizer's grid comes back unchanged: if every
    group column holds codes 0 and 15 and a normal fp16 scale s, its max - min is 15 s
    exactly, so the scale, the zero (-round(-z) = z) and every code (round(q - z) + z)
    are recovered: quantize(dequant(q, z, s)) == (q, z, s).  (Scales are chosen so that
    the dequantised weights are fp16 values.)"""
    rng = _rng(21)
    for K, N, g in ((64, 16, 32), (128, 24, -1), (96, 8, 32)):
        _, G = o.resolve_groups(K, g)
        gl = K // G
        codes = rng.integers(0, 16, (K, N))
        codes.reshape(G, gl, N)[:, 0, :] = 0
        codes.reshape(G, gl, N)[:, 1, :] = 15
        zeros = rng.integers(0, 16, (G, N))
        # Scales with 7 significant bits, so every (q - z) s (<= 11 bits) is an fp16 value.
        scales = (rng.integers(64, 128, (G, N)) * 2.0 ** -13).astype(np.float16)
        qw, qz = o.pack_awq(codes), o.pack_awq(zeros)
        with np.errstate(over="ignore"):  # (a planted mistake may overflow)
            W = o.dequant_ref(qw, qz, scales, g).astype(np.float16)
        assert (W.astype(np.float32) == o.dequant_ref(qw, qz, scales, g)).all()  # values fit fp16
        qw2, qz2, sc2 = o.quantize_rtn(W, g)
        assert np.array_equal(sc2.view(np.uint16), scales.view(np.uint16))
        assert np.array_equal(o.unpack_awq(qz2), zeros)
        assert np.array_equal(o.unpack_awq(qw2), codes)


def pin_rtn_error_bound(o):
    """Round to nearest: every code that is not clamped reconstructs its weight to within
    half a step, |w - (q - z) s| <= s / 2 (plus the float32 division's rounding); clamped
    codes sit at 0 or 15.  Symmetric: zero is 8 and codes span the signed range."""
    rng = _rng(22)
    for K, N, g in ((256, 32, 64), (128, 16, -1)):
        W = rng.normal(0, 0.02, (K, N)).astype(np.float16)
        _, G = o.resolve_groups(K, g)
        gl = K // G
        for sym in (False, True):
            qw, qz, sc = o.quantize_rtn(W, g, sym=sym)
            q = o.unpack_awq(qw).astype(np.float64)
            z = np.repeat(o.unpack_awq(qz), gl, axis=0).astype(np.float64)
            s = np.repeat(sc.astype(np.float64), gl, axis=0)
            w = W.astype(np.float64)
            err = np.abs(w - (q - z) * s)
            free = (q > 0) & (q < 15)
            assert (err[free] <= s[free] * (0.5 + 2.0 ** -20) + np.abs(w[free]) * 2.0 ** -23).all(), sym
            if sym:
                assert (z == 8).all()
            else:
                # The group's max and min are reconstructed within one step of the grid.
                assert (sc.astype(np.float64) > 0).all()


ALL_PINS = [pin_moe_align, pin_moe_gemm, pin_bf16_conversion, pin_gemm_bf16_widening, pin_rtn_hand_example, pin_rtn_roundtrip, pin_rtn_error_bound, pin_fp16_rounding, pin_hand_words, pin_permutation_inverse, pin_roundtrip_codes, pin_roundtrip_words,
            pin_two_unpacks_agree, pin_no_plus_one, pin_brute_force_gemm, pin_dequant_orientation,
            pin_special_cases, pin_entries_agree, pin_format_rules, pin_gemm_ieee]
