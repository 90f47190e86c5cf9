"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a library routine (torch's float8_e4m3fn
and bfloat16 decoders/encoders), an independent exact implementation
(``exact_spec``: Fractions, brute-force nearest search), a closed form, an
invariant the contract implies, or a hand-derived example.  Together they are
chosen so that a dropped term, a wrong sign, a wrong index or a transposed
operand in the oracle fails at least one of them.
"""
import json
import os
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import exact_spec as X
from nvfp4_block_scaled_amax_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE_BF16 = ALL_BF16[(ALL_BF16 & 0x7F80) != 0x7F80]
NONNEG_FINITE_BF16 = FINITE_BF16[FINITE_BF16 < 0x8000]


def f64(bits):
    return W.bf16_to_f64(bits)


def e4m3_torch(q32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(q32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------------------
# Format decoders
# ---------------------------------------------------------------------------

def test_e4m3_decode_matches_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([orc.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_e4m3_closed_forms(orc):
    pos = np.array([orc.e4m3_value(c) for c in range(127)])
    assert np.all(np.diff(pos) > 0)
    assert pos[0x7E] == 448.0 and pos[0x01] == 2.0 ** -9 and pos[0x38] == 1.0
    assert orc.e4m3_value(0x80) == 0.0 and np.signbit(orc.e4m3_value(0x80))


def test_e2m1_decode_closed_form(orc):
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for c in range(16):
        v = orc.e2m1_value(c)
        assert abs(v) == mags[c & 7]
        assert np.signbit(v) == bool(c & 8)


def test_bf16_decode_matches_torch(orc):
    ref = torch.from_numpy(FINITE_BF16.view(np.int16).copy()).view(torch.bfloat16).to(
        torch.float64).numpy()
    ours = np.array([orc.bf16_value(int(b)) for b in FINITE_BF16])
    assert np.array_equal(ref, ours)
    assert np.array_equal(np.signbit(ref), np.signbit(ours))


def test_e8m0_decode(orc):
    for b in (0, 1, 126, 127, 128, 254):
        assert orc.e8m0_value(b) == 2.0 ** (b - 127)
    assert np.isnan(orc.e8m0_value(255))


# ---------------------------------------------------------------------------
# MXFP8 scale rule and code map
# ---------------------------------------------------------------------------

def test_e8m0_rule_bruteforce_all_bf16(orc):
    """Smallest e >= -127 with A <= 448 * 2^e, for every non-negative finite BF16
    A: no clipping, minimal, and equal to a closed form on A's fields."""
    A = f64(NONNEG_FINITE_BF16)
    byte = orc.e8m0_byte_many(A)
    e = byte.astype(np.int64) - 127
    assert np.all(A <= 448.0 * np.ldexp(1.0, e))                       # never clips
    assert np.all((e == -127) | (A > 448.0 * np.ldexp(1.0, e - 1)))    # minimal
    E = (NONNEG_FINITE_BF16.astype(np.int64) >> 7) & 0xFF
    m = NONNEG_FINITE_BF16.astype(np.int64) & 0x7F
    closed = np.where(E == 0, 0, np.maximum(0, E - 8 + (m > 96)))
    assert np.array_equal(byte, closed)


def test_mxfp8_code_map_exhaustive_vs_torch(orc):
    """Every finite BF16 x times every scale 2^e, e in [-127, 120], with
    |x| <= 448 * 2^e (the only region MXFP8 produces): the oracle's E4M3 code
    of x / 2^e equals torch's float8_e4m3fn conversion (round-to-nearest-even)."""
    x = f64(FINITE_BF16)
    n = 0
    for e in range(-127, 121):
        D = 2.0 ** e
        keep = np.abs(x) <= 448.0 * D
        xs = x[keep]
        ours = orc.e4m3_nearest_many(xs, D)
        q = xs / D
        ref = e4m3_torch(q.astype(np.float32))
        assert np.array_equal(ours, ref), f"e={e}"
        n += xs.size
    assert n > 8_000_000


def test_e4m3_saturates(orc):
    for q in (448.0, 448.5, 463.9, 464.0, 480.0, 1e6, 3.3e38):
        assert orc.e4m3_nearest(q, 1.0) == 0x7E
        assert orc.e4m3_nearest(-q, 1.0) == 0xFE
    # Near the top the E4M3 step is 32: 0x7C = 384, 0x7D = 416, 0x7E = 448.
    assert orc.e4m3_nearest(432.0, 1.0) == 0x7E      # tie 416|448 -> even 0x7E
    assert orc.e4m3_nearest(400.0, 1.0) == 0x7C      # tie 384|416 -> even 0x7C
    assert orc.e4m3_nearest(424.0, 1.0) == 0x7D


def _rand_fp32_scales(rng, n):
    """Random binary32 scales: normal ones over a wide range, and subnormals."""
    e = rng.integers(-140, 110, size=n)
    m = rng.integers(0, 1 << 23, size=n)
    bits = np.where(e < -126, m, ((e + 127) << 23) | m).astype(np.uint32)
    return bits.view(np.float32).astype(np.float64)


def test_e4m3_nearest_vs_exact_spec(orc):
    """Random (A, 6s) pairs plus constructed exact ties: the oracle's E4M3 code of
    A / (6 s) equals a brute-force nearest search on exact rationals."""
    rng = np.random.default_rng(11)
    s = _rand_fp32_scales(rng, 1500)
    target = np.exp2(rng.uniform(-12, 10, size=s.size))          # q around the E4M3 range
    A = f64(W.bf16_bits(target * 6 * s))
    cases = [(a, 6 * si) for a, si in zip(A, s) if a > 0 and np.isfinite(a)]
    v = [float(t) for t in X.E4M3_POS]
    for k in range(126):                                          # exact ties, D = 2^j
        mid = 0.5 * (v[k] + v[k + 1])
        for j in (-3, 0, 5):
            cases.append((mid * 2.0 ** j, 2.0 ** j))
    for a, D in cases:
        want = X.nearest_code(X.E4M3_POS, F(a) / F(D))
        assert orc.e4m3_nearest(a, D) == want, (a, D)
        assert orc.e4m3_nearest(-a, D) == want | 0x80


# ---------------------------------------------------------------------------
# NVFP4 scale and code map
# ---------------------------------------------------------------------------

def test_nvfp4_scale_is_rn32_of_exact_quotient(orc):
    """s = RN32(A / 2688) for every positive finite BF16 A, checked against an
    exact binary32 rounding on Fractions (covers subnormal s)."""
    A = f64(NONNEG_FINITE_BF16)
    s = orc.nvfp4_scale_many(A)
    sub = np.concatenate([np.arange(0, 300), np.arange(300, A.size, 37)])
    for i in sub:
        want = X.rn_binary32(F(A[i]) / 2688)
        assert F(float(s[i])) == want, (A[i], s[i])
    assert s[0] == 0.0
    assert np.all(s[1:] > 0)                                   # never underflows to 0


def _divisor_set(orc):
    """Divisors D = d * s: every positive E4M3 d times several FP32 scales --
    exact powers of two, inexact quotients like RN32(1/448), subnormals."""
    d = np.array([orc.e4m3_value(c) for c in range(1, 127)])
    svals = [2.0 ** -9, float(np.float32(1) / np.float32(448)),
             float(np.float32(0.30078125) / np.float32(2688)),
             float(np.float32(2.0 ** -130) / np.float32(2688)),      # subnormal s
             float(np.float32(3.3895313892515355e38) / np.float32(2688))]
    return [(di, si) for si in svals for di in d]


def test_e2m1_code_map_exhaustive_vs_longdouble(orc):
    """Every finite BF16 x against every divisor of the set: the oracle's E2M1
    code equals nearest-even rounding of x / D computed by an independent route
    (x87 extended-precision division, then a midpoint search).  The exact
    quotient is either a midpoint or at least ~2^-32 relative away from one,
    far above the 2^-64 division error, so this route is exact too."""
    if np.finfo(np.longdouble).nmant < 63:
        pytest.skip("needs 64-bit-mantissa long double")
    x = f64(FINITE_BF16)
    xl = np.abs(x).astype(np.longdouble)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.longdouble)
    neg = np.signbit(x)
    for d, s in _divisor_set(orc):
        D = d * s
        ours = orc.e2m1_nearest_many(x, D)
        q = xl / (np.longdouble(d) * np.longdouble(s))
        k = np.searchsorted(mids, q, side="left")           # number of mids < q
        tie = (k < 7) & (q == mids[np.minimum(k, 6)])
        k = np.where(tie & (k % 2 == 1), k + 1, k)           # tie -> even code
        ref = (k | np.where(neg, 8, 0)).astype(np.uint8)
        assert np.array_equal(ours, ref), (d, s)


def test_e2m1_nearest_vs_exact_spec(orc):
    rng = np.random.default_rng(12)
    dcodes = rng.integers(1, 127, size=800)
    s = _rand_fp32_scales(rng, 800)
    d = np.array([orc.e4m3_value(int(c)) for c in dcodes])
    q = rng.uniform(0, 7, size=800)
    xb = W.bf16_bits(q * d * s)
    for i in range(800):
        xv = float(f64(xb[i:i + 1])[0])
        if not np.isfinite(xv):
            continue
        want = X.nearest_code(X.E2M1_POS, abs(F(xv)) / (F(d[i]) * F(s[i])))
        got = orc.e2m1_nearest(xv, d[i] * s[i])
        assert got & 7 == want
        assert bool(got & 8) == bool(xb[i] & 0x8000)


# ---------------------------------------------------------------------------
# BF16 rounding for dequant
# ---------------------------------------------------------------------------

def test_bf16_round_sat_vs_exact_spec(orc):
    rng = np.random.default_rng(13)
    cases = []
    for _ in range(400):                                   # NVFP4 products
        c = int(rng.integers(0, 16))
        b = int(rng.integers(0, 127))
        s = float(_rand_fp32_scales(rng, 1)[0])
        cases.append(orc.e2m1_value(c) * orc.e4m3_value(b) * s)
    for _ in range(200):                                   # MXFP8 products
        c = int(rng.integers(0, 255))
        if c & 0x7F == 0x7F:
            continue
        e = int(rng.integers(-127, 128))
        cases.append(orc.e4m3_value(c) * 2.0 ** e)
    for y in cases:
        want = X.bf16_nearest_sat(F(y))
        got = orc.bf16_round_sat(y)
        if y == 0:
            assert got & 0x7FFF == 0
        else:
            assert got == want, (y, hex(got), hex(want))


def test_bf16_round_sat_special_cases(orc):
    assert orc.bf16_round_sat(2.0 ** 128) == 0x7F7F          # saturates, no Inf
    assert orc.bf16_round_sat(-(2.0 ** 128)) == 0xFF7F
    assert orc.bf16_round_sat(448.0 * 2.0 ** 127) == 0x7F7F
    assert orc.bf16_round_sat(0.0) == 0x0000
    assert orc.bf16_round_sat(-0.0) == 0x8000
    assert orc.bf16_round_sat(2.0 ** -134) == 0x0000         # tie 0|2^-133 -> even
    assert orc.bf16_round_sat(3 * 2.0 ** -134) == 0x0002     # tie 1|2 -> even 2
    assert orc.bf16_round_sat(1.0 + 2.0 ** -8) == 0x3F80     # tie -> even
    assert orc.bf16_round_sat(1.0 + 3 * 2.0 ** -8) == 0x3F82


def test_golden_scale_is_decode_multiplier(orc):
    """The pages' example of a scale as the decode multiplier."""
    with open(os.path.join(GOLDEN, "scale_is_decode_multiplier.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        codes = np.array([[case["e2m1_code"]]], np.uint8)         # element 0 = code
        bs = np.array([[case["e4m3_block_scale"]]], np.uint8)
        s = np.array([case["fp32_scale"]], np.float32)
        codes16 = np.zeros((1, 8), np.uint8)
        codes16[0, 0] = codes[0, 0]
        out = orc.dequant_nvfp4(codes16, bs, s, 1)
        assert out[0, 0] == int(case["decoded_bf16_bits"], 16)
        assert abs(float(f64(out[0, :1])[0]) - case["decoded_decimal"]) < 2e-3


# ---------------------------------------------------------------------------
# Hand-derived blocks
# ---------------------------------------------------------------------------

def test_hand_blocks_mxfp8(orc):
    # Block of 32 maxes: A = 255 * 2^120; smallest e with A <= 448 * 2^e is 120
    # (byte 0xF7); each element is 255 * 2^120 / 2^120 = 255, nearest E4M3 256 =
    # code 0x78.  Dequant: 256 * 2^120 = 2^128 > BF16 max -> saturates to 0x7F7F.
    x = np.full((1, 32), 0x7F7F, np.uint16)
    c, s = orc.mxfp8_rowwise(x)
    assert s[0, 0] == 0xF7 and np.all(c == 0x78)
    assert np.all(orc.dequant_mxfp8_rowwise(c, s) == 0x7F7F)
    # Zeros: e clamps to -127 (byte 0), codes 0.
    c, s = orc.mxfp8_rowwise(np.zeros((1, 32), np.uint16))
    assert s[0, 0] == 0 and np.all(c == 0)
    # Amax 448 -> e = 0 (0x7F); 1.0625 is the 1|1.125 midpoint -> even 0x38;
    # 1.1875 is the 1.125|1.25 midpoint -> even 0x3A; 2^-10 is the 0|2^-9
    # midpoint -> 0x00; 3*2^-10 -> even 0x02; -2^-11 -> negative zero 0x80.
    vals = [448, 1.0625, 1.1875, 2 ** -10, 3 * 2 ** -10, -2 ** -11] + [0] * 26
    c, s = orc.mxfp8_rowwise(W.bf16_bits(np.array([vals])))
    assert s[0, 0] == 0x7F
    assert list(c[0, :6]) == [0x7E, 0x38, 0x3A, 0x00, 0x02, 0x80]
    # Amax 450 (next BF16 above 448) -> e = 1 (0x80); 450 / 2 = 225 -> 224 (0x76).
    c, s = orc.mxfp8_rowwise(W.bf16_bits(np.array([[450.0] + [0] * 31])))
    assert s[0, 0] == 0x80 and c[0, 0] == 0x76
    # Amax 2^-120 -> 2^-120 <= 448 * 2^-127: byte 0; 2^-120 / 2^-127 = 128 (0x70).
    c, s = orc.mxfp8_rowwise(W.bf16_bits(np.array([[2.0 ** -120] + [0] * 31])))
    assert s[0, 0] == 0x00 and c[0, 0] == 0x70


def test_hand_token_nvfp4(orc):
    # One token of 32: amax 6, s = RN32(6/2688) = RN32(1/448) = 0x3B124925,
    # slightly above 1/448.  Block 0 amax 6 -> 6/(6s) just below 448 -> 0x7E.
    # Block 1 amax 1 -> 448/6 * (1 - eps) = 74.67 -> nearest E4M3 72 (0x69).
    # Element codes follow from x / (d s) with d s just above 1 (block 0) and
    # 72/448 (block 1); ideal midpoints fall just below and round down.
    blk0 = [6, -6, 3, 0.75, 1.75, 3.5, 0.25, 5, 2.5, 1.25, 0, -0.75, 4, 1, 0.5, -3.5]
    blk1 = [1, 0.5, 0.30078125, -0.25, 0.125, 0, 0.75, -0.5, 0.0625, 0.375, 0.625,
            0.875, -1, 0.03125, 0.1875, 0.5625]
    x = W.bf16_bits(np.array([blk0 + blk1]))
    c, b, s = orc.nvfp4_per_token(x)
    assert s.view(np.uint32)[0] == 0x3B124925
    assert list(b[0]) == [0x7E, 0x69]
    assert bytes(c[0]).hex() == "f7155360249026d1" + "57b402d641760f52"
    # Exact scale: amax 5.25 = 21 * 2^-2 -> s = 2^-9 exactly, b = 0x7E, d s = 7/8;
    # elements scale to 6, .75, 1.75, 3.5, .25, 2.5, 5, -.75: all ties but the
    # first, each resolved to the even code.
    x = W.bf16_bits(np.array([[5.25, 0.65625, 1.53125, 3.0625, 0.21875, 2.1875, 4.375,
                               -0.65625] + [0] * 8]))
    c, b, s = orc.nvfp4_per_token(x)
    assert s[0] == 2.0 ** -9 and b[0, 0] == 0x7E
    nib = [(byte >> (4 * h)) & 0xF for byte in c[0, :4] for h in (0, 1)]
    assert nib == [7, 2, 4, 6, 0, 4, 6, 0xA]


def test_hand_zero_block_scale(orc):
    # Row amax 1 -> s = RN32(1/2688).  Block 1's amax 2^-20 gives
    # 2^-20 / (6 s) ~ 2^-11.4, below half the smallest E4M3 subnormal (2^-10),
    # so b = 0x00 and, by the reading for a zero block scale, every code of the
    # block is 0x0 -- also for negative elements and for -0.
    blk0 = [1.0] + [0.5] * 15
    blk1 = [2.0 ** -20, -(2.0 ** -20), -0.0, 2.0 ** -22] + [0.0] * 12
    x = W.bf16_bits(np.array([blk0 + blk1]))
    c, b, s = orc.nvfp4_per_token(x)
    assert b[0, 1] == 0x00 and not c[0, 8:].any()
    assert b[0, 0] == 0x7E
    # A block of -0 under a non-zero block scale keeps the sign: 0x8.
    x = W.bf16_bits(np.array([[1.0, -0.0] + [0.25] * 14]))
    c, b, s = orc.nvfp4_per_token(x)
    assert c[0, 0] == 0x87


# ---------------------------------------------------------------------------
# Whole tensors: oracle == exact spec on small inputs
# ---------------------------------------------------------------------------

def _small_inputs():
    rng = np.random.default_rng(21)
    yield "normal", W.bf16_bits(rng.standard_normal((4, 64)) * 3)
    yield "boundary", W.mode_boundary(32, 64, 5)[:6]
    yield "student", W.student_t_activations(4, 64, 9)
    yield "nvfp4-boundary", W.nvfp4_boundary(8, 64, 3)


@pytest.mark.parametrize("name,x", list(_small_inputs()))
def test_mxfp8_rowwise_matches_exact_spec(orc, name, x):
    codes, scales = orc.mxfp8_rowwise(x)
    ec, es = X.mxfp8_rowwise([[int(v) for v in row] for row in x])
    assert np.array_equal(scales, np.array(es, np.uint8))
    assert np.array_equal(codes, np.array(ec, np.uint8))


def test_mxfp8_colwise_matches_exact_spec(orc):
    x = W.mode_boundary(32, 64, 6)
    codes, scales = orc.mxfp8_colwise(x)
    ec, es = X.mxfp8_rowwise([[int(v) for v in col] for col in x.T])
    assert np.array_equal(scales, np.array(es, np.uint8).T)
    assert np.array_equal(codes, np.array(ec, np.uint8).T)


@pytest.mark.parametrize("name,x", list(_small_inputs()))
def test_nvfp4_per_token_matches_exact_spec(orc, name, x):
    codes, bs, ts = orc.nvfp4_per_token(x)
    ec, eb, es = X.nvfp4_per_token([[int(v) for v in row] for row in x])
    assert [F(float(t)) for t in ts] == es
    assert np.array_equal(bs, np.array(eb, np.uint8))
    assert np.array_equal(codes, np.array(ec, np.uint8))


def test_dequant_matches_exact_spec(orc):
    x = W.nvfp4_boundary(8, 64, 4)
    codes, bs, ts = orc.nvfp4_per_token(x)
    out = orc.dequant_nvfp4(codes, bs, ts, 1)
    for i in range(8):
        for k in range(0, 64, 3):
            c = (codes[i, k // 2] >> (4 * (k % 2))) & 0xF
            y = X.E2M1_POS[c & 7] * X.E4M3_POS[bs[i, k // 16]] * F(float(ts[i]))
            want = X.bf16_nearest_sat(-y if c & 8 else y)
            if y == 0:
                assert out[i, k] == (0x8000 if c & 8 else 0)
            else:
                assert out[i, k] == want
    xm = W.mode_boundary(32, 64, 7)
    c8, s8 = orc.mxfp8_rowwise(xm)
    out = orc.dequant_mxfp8_rowwise(c8, s8)
    for i in range(0, 32, 5):
        for k in range(0, 64, 7):
            y = X.E4M3_POS[c8[i, k] & 0x7F] * F(2) ** (int(s8[i, k // 32]) - 127)
            want = X.bf16_nearest_sat(-y if c8[i, k] & 0x80 else y)
            if y == 0:
                assert out[i, k] & 0x7FFF == 0
            else:
                assert out[i, k] == want


def test_quantize_dequant_matches_exact_spec(orc):
    """The one-pass quantize + dequant composition, whole tensors, against the
    Fraction spec: codes and scales from its quantizers, BF16 from the exact
    product rounded once."""
    xm = W.mode_boundary(32, 64, 9)
    c8, s8, y8 = orc.quantize_dequant_mxfp8_rowwise(xm)
    rc, rs = X.mxfp8_rowwise(xm.tolist())
    assert c8.tolist() == rc and s8.tolist() == rs
    for i in range(32):
        for k in range(64):
            y = X.E4M3_POS[rc[i][k] & 0x7F] * F(2) ** (rs[i][k // 32] - 127)
            want = X.bf16_nearest_sat(-y if rc[i][k] & 0x80 else y)
            if y == 0:
                want = 0x8000 if rc[i][k] & 0x80 else 0
            assert y8[i, k] == want, (i, k)
    xn = W.nvfp4_boundary(8, 64, 5)
    c4, b4, t4, y4 = orc.quantize_dequant_nvfp4(xn)
    C, Bs, S = X.nvfp4_per_token(xn.tolist())
    assert c4.tolist() == C and b4.tolist() == Bs
    assert [F(float(v)) for v in t4] == S
    for i in range(8):
        for k in range(64):
            c = (C[i][k // 2] >> (4 * (k % 2))) & 0xF
            y = X.E2M1_POS[c & 7] * X.E4M3_POS[Bs[i][k // 16]] * S[i]
            want = X.bf16_nearest_sat(-y if c & 8 else y)
            if y == 0:
                want = 0x8000 if c & 8 else 0
            assert y4[i, k] == want, (i, k)


def test_mxfp8_quantize_dequant_is_a_projection(orc):
    """For values in range, dequant(quant(x)) lies on the grid it was rounded
    to, so quantizing it again returns it unchanged (the block amax can only
    lower the exponent, and an E4M3 value times a power of two up to 448 is
    an E4M3 value); and it stays within half a step of x."""
    for x in (W.config1(), W.student_t_activations(64, 256, 31)):
        _, s, y = orc.quantize_dequant_mxfp8_rowwise(x)
        _, s2, y2 = orc.quantize_dequant_mxfp8_rowwise(y)
        assert np.array_equal(y2, y)
        assert np.all(s2 <= s)
        xv, yv = f64(x), f64(y)
        scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
        # E4M3 spacing at |y| / 2^e: 2^(floor(log2) - 3), and 2^-9 below 2^-6
        e = np.floor(np.log2(np.maximum(np.abs(yv) / scale, 2.0 ** -6))).astype(np.int64)
        assert np.all(np.abs(xv - yv) <= np.ldexp(1.0, e - 3) * scale / 2)


# ---------------------------------------------------------------------------
# Invariants the contract implies
# ---------------------------------------------------------------------------

def test_zeros_in_zeros_out(orc):
    z = np.zeros((64, 128), np.uint16)
    for arr in orc.mxfp8_rowwise(z) + orc.mxfp8_colwise(z):
        assert not arr.any()
    c, b, s = orc.nvfp4_per_token(z)
    assert not c.any() and not b.any() and not s.any()
    assert not orc.dequant_nvfp4(c, b, s, 1).any()
    c, sc = orc.mxfp8_rowwise(z)
    assert not orc.dequant_mxfp8_rowwise(c, sc).any()


def test_sign_symmetry(orc):
    x = W.config1()[:64]
    xn = x ^ np.uint16(0x8000)
    c, s = orc.mxfp8_rowwise(x)
    cn, sn = orc.mxfp8_rowwise(xn)
    assert np.array_equal(s, sn) and np.array_equal(c ^ np.uint8(0x80), cn)
    c, s = orc.mxfp8_colwise(x)
    cn, sn = orc.mxfp8_colwise(xn)
    assert np.array_equal(s, sn) and np.array_equal(c ^ np.uint8(0x80), cn)
    c, b, t = orc.nvfp4_per_token(x)
    cn, bn, tn = orc.nvfp4_per_token(xn)
    assert np.array_equal(b, bn) and np.array_equal(t, tn)
    assert np.array_equal(c ^ np.uint8(0x88), cn)      # every block has d > 0 here


def test_power_of_two_equivariance(orc):
    """X * 2^k: MXFP8 codes unchanged, scale bytes + k; NVFP4 codes and block
    scales unchanged, FP32 scales * 2^k (all values stay normal)."""
    x = W.config1()[:64]
    xv = f64(x)
    for k in (-7, 3, 40):
        xk = W.bf16_bits(xv * 2.0 ** k)
        assert np.array_equal(f64(xk), xv * 2.0 ** k)
        c, s = orc.mxfp8_rowwise(x)
        ck, sk = orc.mxfp8_rowwise(xk)
        assert np.array_equal(c, ck) and np.array_equal(s.astype(int) + k, sk.astype(int))
        c, b, t = orc.nvfp4_per_token(x)
        ck, bk, tk = orc.nvfp4_per_token(xk)
        assert np.array_equal(c, ck) and np.array_equal(b, bk)
        assert np.array_equal(t.astype(np.float64) * 2.0 ** k, tk.astype(np.float64))


def test_batch_invariance(orc):
    """Per-token scales make each row's output independent of the other rows:
    permuting, duplicating or splitting the batch maps the outputs the same way."""
    x = W.config3()[:96]
    rng = np.random.default_rng(5)
    perm = rng.permutation(96)
    dup = np.concatenate([x, x[:17]])
    c, b, t = orc.nvfp4_per_token(x)
    cp, bp, tp = orc.nvfp4_per_token(x[perm])
    assert np.array_equal(cp, c[perm]) and np.array_equal(bp, b[perm]) and np.array_equal(tp, t[perm])
    cd, bd, td = orc.nvfp4_per_token(dup)
    assert np.array_equal(cd[96:], c[:17]) and np.array_equal(td[96:], t[:17])
    c1, b1, t1 = orc.nvfp4_per_token(x[:40])
    assert np.array_equal(c1, c[:40]) and np.array_equal(t1, t[:40])
    r, rs = orc.mxfp8_rowwise(x)
    rp, rsp = orc.mxfp8_rowwise(x[perm])
    assert np.array_equal(rp, r[perm]) and np.array_equal(rsp, rs[perm])


def test_colwise_is_rowwise_of_transpose(orc):
    x = W.mode_random(64, 96, 3)
    c, s = orc.mxfp8_colwise(x)
    rc, rs = orc.mxfp8_rowwise(np.ascontiguousarray(x.T))
    assert np.array_equal(c, rc.T) and np.array_equal(s, rs.T)
    assert not np.array_equal(c, orc.mxfp8_rowwise(x)[0])   # the copies differ


def test_no_clip_and_minimal_scale_config1(orc):
    x = W.config1()
    xv = np.abs(f64(x))
    c, s = orc.mxfp8_rowwise(x)
    A = xv.reshape(256, 16, 32).max(axis=2)
    e = s.astype(np.int64) - 127
    assert np.all(A <= 448 * np.ldexp(1.0, e))
    assert np.all((e == -127) | (A > 448 * np.ldexp(1.0, e - 1)))
    c, s = orc.mxfp8_colwise(x)
    A = xv.reshape(8, 32, 512).max(axis=1)
    e = s.astype(np.int64) - 127
    assert np.all(A <= 448 * np.ldexp(1.0, e))
    assert np.all((e == -127) | (A > 448 * np.ldexp(1.0, e - 1)))


def test_half_ulp_round_trip(orc):
    """dequant(quant(x)) is within half a format step of x after scaling:
    MXFP8 |x / 2^e - dec(c)| <= half the E4M3 spacing at dec(c); NVFP4
    |x / (d s) - dec(c)| <= half the E2M1 spacing unless |x / (d s)| > 6."""
    x = W.config1()[:32]
    xv = f64(x)
    c, s = orc.mxfp8_rowwise(x)
    pos = [float(v) for v in X.E4M3_POS]
    for i in range(32):
        for k in range(0, 512, 5):
            q = F(xv[i, k]) / F(2) ** (int(s[i, k // 32]) - 127)
            v = F(pos[c[i, k] & 0x7F])
            idx = c[i, k] & 0x7F
            lo = v - F(pos[idx - 1]) if idx > 0 else F(pos[1])
            hi = F(pos[idx + 1]) - v if idx < 126 else lo
            assert abs(abs(q) - v) <= max(lo, hi) / 2
    xt = W.config3()[:16]
    c, b, t = orc.nvfp4_per_token(xt)
    xv = f64(xt)
    e2 = [F(v) for v in X.E2M1_POS]
    for i in range(16):
        for k in range(0, 2048, 11):
            d = X.E4M3_POS[b[i, k // 16]]
            if d == 0:
                continue
            q = abs(F(xv[i, k])) / (d * F(float(t[i])))
            code = int((c[i, k // 2] >> (4 * (k % 2))) & 7)
            if q > 6:
                assert code == 7
                continue
            gaps = [e2[j + 1] - e2[j] for j in range(7)]
            g = max(gaps[max(code - 1, 0)], gaps[min(code, 6)])
            assert abs(q - e2[code]) <= g / 2


def test_pair_equals_concatenated_scope(orc):
    rng = np.random.default_rng(8)
    g = W.bf16_bits(rng.normal(0, 0.02, size=(3, 16, 64)))
    u = W.bf16_bits(rng.normal(0, 0.03, size=(3, 16, 64)))
    gc, gb, uc, ub, sc = orc.nvfp4_gateup_pair(g, u)
    for e in range(3):
        cat = np.concatenate([g[e], u[e]])
        A = np.abs(f64(cat)).max()
        s = orc.nvfp4_scale(A)
        assert sc[e] == np.float32(s)
        cc, cb = orc.nvfp4_with_scale(cat, s)
        assert np.array_equal(cc[:16], gc[e]) and np.array_equal(cc[16:], uc[e])
        assert np.array_equal(cb[:16], gb[e]) and np.array_equal(cb[16:], ub[e])
    # An up whose magnitudes stay below gate's leaves gate's bytes as gate alone.
    small = W.bf16_bits(f64(g) * 0.5)
    gc2, gb2, _, _, sc2 = orc.nvfp4_gateup_pair(g, small)
    gc1, gb1, _, _, sc1 = orc.nvfp4_gateup_pair(g, None)
    assert np.array_equal(gc1, gc2) and np.array_equal(gb1, gb2) and np.array_equal(sc1, sc2)


def _bf16_of_exact(y: F, negative: bool) -> int:
    """BF16 bits of the exact product y rounded once (nearest-even, saturating);
    a product that is zero keeps the sign of the code that made it."""
    if y == 0:
        return 0x8000 if negative else 0
    return X.bf16_nearest_sat(-y if negative else y)


@pytest.mark.parametrize("mode", ["boundary", "maxes", "codes"])
def test_dequant_mxfp8_colwise_vs_exact_spec(orc, mode):
    """Columnwise MXFP8 -> BF16, every element: the E4M3 value times the scale of
    the element's own 32-row block of its own column, rounded once.  The 'codes'
    case feeds every non-NaN code byte under random scale bytes that differ from
    column to column (the whole E8M0 range, so BF16 saturation and underflow to
    signed zero both occur)."""
    if mode == "codes":
        rng = np.random.default_rng(21)
        rows, cols = 64, 24
        codes = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] ^= 1                 # NaN codes -> +-448
        scales = rng.integers(0, 255, (rows // 32, cols), dtype=np.uint8)
    else:
        rows, cols = 64, 32
        x = W.mxfp8_mode(mode, rows, cols, 11)
        codes, scales = orc.mxfp8_colwise(x)
    out = orc.dequant_mxfp8_colwise(codes, scales)
    for i in range(rows):
        for k in range(cols):
            c = int(codes[i, k])
            y = X.E4M3_POS[c & 0x7F] * F(2) ** (int(scales[i // 32, k]) - 127)
            assert out[i, k] == _bf16_of_exact(y, bool(c & 0x80)), (mode, i, k)


@pytest.mark.parametrize("per", [2, 3, 12])
def test_dequant_nvfp4_shared_fp32_scales_vs_exact_spec(orc, per):
    """NVFP4 -> BF16 where consecutive rows share one FP32 scale (one scale per
    expert or per tensor, as in the weight export round trip): row i uses
    fp32_scales[i // per].  Every group's scale differs from the others'."""
    rng = np.random.default_rng(30 + per)
    rows, cols = 12, 32
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    bs = rng.integers(0, 127, (rows, cols // 16), dtype=np.uint8)
    n_sc = -(-rows // per)
    fs = (rng.uniform(1.0, 2.0, n_sc) * 2.0 ** rng.integers(-30, 30, n_sc)).astype(np.float32)
    assert len(set(fs.tolist())) == n_sc
    out = orc.dequant_nvfp4(codes, bs, fs, per)
    for i in range(rows):
        s = F(float(fs[i // per]))
        for k in range(cols):
            c = (int(codes[i, k // 2]) >> (4 * (k % 2))) & 0xF
            y = X.E2M1_POS[c & 7] * X.E4M3_POS[int(bs[i, k // 16])] * s
            assert out[i, k] == _bf16_of_exact(y, bool(c & 8)), (per, i, k)


def test_scoped_quantize_vs_exact_spec(orc):
    """The weight-export scopes row by row against the Fraction spec: the scope's
    FP32 scale is the binary32 rounding of (amax over every element of the
    scope) / 2688, and each row of each tensor is quantized under it (gate and
    up of one expert share one scope; down is its own).  Also the bare
    'quantize under a given scale' call, under a scale no row picks itself."""
    rng = np.random.default_rng(40)
    E, rows, cols = 2, 6, 32
    g = W.bf16_bits(rng.normal(0, 0.02, (E, rows, cols)))
    u = W.bf16_bits(rng.standard_t(3, (E, rows, cols)) * 0.01)
    gc, gb, uc, ub, sc = orc.nvfp4_gateup_pair(g, u)
    dc, db, _, _, dsc = orc.nvfp4_gateup_pair(u, None)
    for e in range(E):
        A = max(abs(X.bf16_frac(int(b))) for b in np.concatenate([g[e].ravel(), u[e].ravel()]))
        s = X.nvfp4_scale(A)
        assert F(float(sc[e])) == s
        Ad = max(abs(X.bf16_frac(int(b))) for b in u[e].ravel())
        sd = X.nvfp4_scale(Ad)
        assert F(float(dsc[e])) == sd
        for t in range(rows):
            for (src, codes, bsc, ss) in ((g, gc, gb, s), (u, uc, ub, s), (u, dc, db, sd)):
                ec, eb = X.nvfp4_row([int(v) for v in src[e, t]], ss)
                assert codes[e, t].tolist() == ec, (e, t)
                assert bsc[e, t].tolist() == eb, (e, t)
    x = W.student_t_activations(8, 48, 41)
    A = max(abs(X.bf16_frac(int(b))) for b in x.ravel())
    s = X.nvfp4_scale(A) * 3      # not the RN32 of any amax / 2688 of this tensor
    s = X.rn_binary32(s)
    c, b = orc.nvfp4_with_scale(x, float(s))
    for t in range(8):
        ec, eb = X.nvfp4_row([int(v) for v in x[t]], s)
        assert c[t].tolist() == ec and b[t].tolist() == eb, t


def test_grouped_colwise_equals_standalone_and_zero_pad(orc):
    off = np.array([0, 0, 1, 32, 63, 96, 96, 160, 193], np.int64)
    x = W.mode_random(int(off[-1]), 64, 9)
    codes, scales, P = orc.mxfp8_colwise_grouped(x, off)
    assert list(P) == [0, 0, 1, 2, 3, 5, 5, 7, 9]      # sizes 0,1,31,31,33,0,64,33
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1])
        n = b - a
        if n == 0:
            continue
        pad = np.zeros((((n + 31) // 32) * 32, 64), np.uint16)
        pad[:n] = x[a:b]
        sc, ss = orc.mxfp8_colwise(pad)
        assert np.array_equal(codes[a:b], sc[:n])
        assert np.array_equal(scales[P[e]:P[e + 1]], ss)


# ---------------------------------------------------------------------------
# Block-scaled GEMM (the consumer of the rowwise MXFP8 copies)
# ---------------------------------------------------------------------------

def _e4m3_frac(c: int) -> F:
    v = X.E4M3_POS[c & 0x7F]
    return -v if c & 0x80 else v


def test_mxfp8_gemm_bruteforce(orc):
    """Tiny GEMMs against sums of Fractions over every k (M != N, so a
    transposed operand or a scale taken from the wrong block or row fails).
    Over the whole code range the binary64 sum may round (within K 2^-53 of
    the magnitude sum); with codes and scales in a few binades it is exact."""
    rng = np.random.default_rng(61)
    M, N, K = 3, 5, 96
    every = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    narrow = np.array([c for c in every if 5 <= ((c >> 3) & 15) <= 10], np.uint8)
    for codes, lo, hi, exact_sum in ((every, 118, 137, False), (narrow, 125, 130, True)):
        a = rng.choice(codes, (M, K)).astype(np.uint8)
        b = rng.choice(codes, (N, K)).astype(np.uint8)
        sa = rng.integers(lo, hi, (M, K // 32)).astype(np.uint8)
        sb = rng.integers(lo, hi, (N, K // 32)).astype(np.uint8)
        C, S = orc.mxfp8_gemm(a, sa, b, sb)
        for m in range(M):
            for n in range(N):
                terms = [_e4m3_frac(int(a[m, k])) * _e4m3_frac(int(b[n, k])) *
                         F(2) ** (int(sa[m, k // 32]) + int(sb[n, k // 32]) - 254)
                         for k in range(K)]
                exact, mag = sum(terms), sum(abs(v) for v in terms)
                if exact_sum:
                    assert F(C[m, n]) == exact and F(S[m, n]) == mag
                else:
                    assert abs(F(C[m, n]) - exact) <= K * mag / 2 ** 53
                    assert abs(F(S[m, n]) - mag) <= K * mag / 2 ** 53


def test_mxfp8_gemm_special_cases(orc):
    """B = identity-like codes (1.0 at k = n, unit scales) returns A's decoded
    values; raising one scale byte of A doubles exactly that block's share."""
    rng = np.random.default_rng(62)
    M, K = 4, 128
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    a = rng.choice(codes, (M, K)).astype(np.uint8)
    sa = rng.integers(120, 134, (M, K // 32)).astype(np.uint8)
    b = np.zeros((K, K), np.uint8)
    b[np.arange(K), np.arange(K)] = 0x38                    # E4M3 1.0
    sb = np.full((K, K // 32), 127, np.uint8)
    C, _ = orc.mxfp8_gemm(a, sa, b, sb)
    want = np.array([[float(_e4m3_frac(int(a[m, k]))) * 2.0 ** (int(sa[m, k // 32]) - 127)
                      for k in range(K)] for m in range(M)])
    assert np.array_equal(C, want)
    bn = rng.choice(codes, (6, K)).astype(np.uint8)
    sbn = rng.integers(124, 130, (6, K // 32)).astype(np.uint8)
    C0, _ = orc.mxfp8_gemm(a, sa, bn, sbn)
    sa2 = sa.copy()
    sa2[1, 2] += 1
    C1, _ = orc.mxfp8_gemm(a, sa2, bn, sbn)
    blk = a.copy()
    blk[:, :64] = 0
    blk[:, 96:] = 0                                          # only block 2 (k 64..95)
    Cb, _ = orc.mxfp8_gemm(blk, sa, bn, sbn)
    assert np.array_equal(C1[1], C0[1] + Cb[1])
    assert np.array_equal(np.delete(C1, 1, 0), np.delete(C0, 1, 0))


def test_nvfp4_gemm_bruteforce_and_dequant_route(orc):
    """Tiny NVFP4 GEMMs against sums of Fractions (codes, 16-block scales and
    FP32 scales decoded by the Fraction spec's tables); and, with unit FP32
    scales, the same product through the oracle's own (pinned) BF16 dequant,
    which is exact here because dec(code) dec(block scale) is a BF16 value."""
    rng = np.random.default_rng(63)
    M, N, K = 3, 4, 64
    a = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    ba = rng.integers(0, 0x7F, (M, K // 16)).astype(np.uint8)
    bb = rng.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
    sa = np.ldexp(1.0, rng.integers(-4, 5, M)).astype(np.float32) * np.float32(1.25)
    sb = np.array([0.375, 3.0], np.float32)                 # one scale per 2 rows of B
    C, S = orc.nvfp4_gemm(a, ba, sa, 1, b, bb, sb, 2)

    def val(codes, bs, m, k):
        c = (int(codes[m, k // 2]) >> (4 * (k % 2))) & 15
        v = X.E2M1_POS[c & 7] * X.E4M3_POS[int(bs[m, k // 16])]
        return -v if c & 8 else v
    for m in range(M):
        for n in range(N):
            s = F(float(sa[m])) * F(float(sb[n // 2]))
            terms = [val(a, ba, m, k) * val(b, bb, n, k) for k in range(K)]
            exact, mag = s * sum(terms), abs(s) * sum(abs(t) for t in terms)
            assert abs(F(C[m, n]) - exact) <= K * mag / 2 ** 52
    one_a, one_b = np.ones(M, np.float32), np.ones(N, np.float32)
    C1, _ = orc.nvfp4_gemm(a, ba, one_a, 1, b, bb, one_b, N)
    ya = W.bf16_to_f64(orc.dequant_nvfp4(a, ba, one_a, 1))
    yb = W.bf16_to_f64(orc.dequant_nvfp4(b, bb, one_b, 1))
    assert np.array_equal(C1, ya @ yb.T)


# ---------------------------------------------------------------------------
# Comparison variants: OCP MX scale rule, per-tensor activation scope
# ---------------------------------------------------------------------------

def test_ocp_rule_closed_form_and_relation(orc):
    """Every non-negative finite BF16 amax: the OCP byte is max(0, E - 8) on
    the BF16 exponent field E (0 for zero and subnormals), computed here from
    the bit fields; the contract's byte exceeds it by exactly 1 when the
    mantissa is above 1.75 (and E >= 8), else equals it."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    A = W.bf16_to_f64(bits.astype(np.uint16))
    E, m = bits >> 7, bits & 0x7F
    want = np.where(E == 0, 0, np.maximum(0, E.astype(np.int64) - 8))
    got = np.array([orc.e8m0_byte_ocp(float(a)) for a in A])
    assert np.array_equal(got, want)
    contract = orc.e8m0_byte_many(A).astype(np.int64)
    assert np.array_equal(contract - got, ((m > 96) & (E >= 8)).astype(np.int64))


def test_ocp_variant_codes_and_clipping(orc):
    """OCP-rule codes equal torch's E4M3 conversion of x / 2^e clamped to
    +-448 (exact scaling, nearest-even in range); clipping happens exactly
    where |x| / 2^e > 448, which the contract's rule never allows."""
    x = W.config2_activation("random")[:256]
    rc, rs, cc, cs = orc.mxfp8_ocp_floor(x)
    xv = W.bf16_to_f64(x)
    for codes, scales, axis in ((rc, rs, 1), (cc, cs, 0)):
        e = np.repeat(scales.astype(np.int64) - 127, 32, axis=axis)
        q = xv / np.ldexp(1.0, e)
        want = torch.from_numpy(np.clip(q, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
        assert np.array_equal(codes, want.numpy())
        clipped = np.abs(q) > 448
        assert clipped.sum() > 0 and np.all((codes[clipped] & 0x7F) == 0x7E)
    c2, s2 = orc.mxfp8_rowwise(x)
    e2 = np.repeat(s2.astype(np.int64) - 127, 32, axis=1)
    assert not np.any(np.abs(xv / np.ldexp(1.0, e2)) > 448)


def test_per_tensor_scope_is_batch_dependent(orc):
    """The per-tensor activation scope (one FP32 scale for the whole tensor,
    here the one-tensor weight scope) changes a row's bytes when other rows
    of the batch change; the per-token scope does not (the batch-invariance
    paragraph's reason for per-token scales)."""
    x = W.config3()[:64]
    y = x.copy()
    y[5] = W.bf16_bits(W.bf16_to_f64(y[5]) * 8.0)       # a louder token elsewhere in the batch
    px = orc.nvfp4_gateup_pair(x[None], None)
    py = orc.nvfp4_gateup_pair(y[None], None)
    assert px[4][0] != py[4][0]
    assert not np.array_equal(px[0][0][0], py[0][0][0])  # row 0 quantized differently
    tx, ty = orc.nvfp4_per_token(x), orc.nvfp4_per_token(y)
    assert np.array_equal(tx[0][0], ty[0][0]) and tx[2][0] == ty[2][0]


# ---------------------------------------------------------------------------
# Property sweep: the oracle against the exact spec on arbitrary finite BF16
# bit patterns (hypothesis draws the bits, so scales range over the whole
# exponent range, subnormals, ties and saturation included).
# ---------------------------------------------------------------------------

from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

_finite_bf16 = st.integers(0, 0xFFFF).filter(lambda b: (b & 0x7F80) != 0x7F80)


def _narrowed(bits, shift):
    """Bit patterns pulled toward one magnitude band (2^-shift of the range),
    so that blocks hold values of comparable size and codes are not all 0."""
    return [(b & 0x8000) | (0x3F80 + ((b & 0x7FFF) >> shift)) if shift else b for b in bits]


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.lists(_finite_bf16, min_size=64, max_size=64), st.integers(0, 8))
def test_property_mxfp8_rowwise_vs_exact_spec(orc, bits, shift):
    x = np.array(_narrowed(bits, shift), np.uint16).reshape(2, 32)
    codes, scales = orc.mxfp8_rowwise(x)
    ec, es = X.mxfp8_rowwise([[int(v) for v in row] for row in x])
    assert np.array_equal(scales, np.array(es, np.uint8))
    assert np.array_equal(codes, np.array(ec, np.uint8))


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.lists(_finite_bf16, min_size=64, max_size=64), st.integers(0, 8))
def test_property_nvfp4_per_token_vs_exact_spec(orc, bits, shift):
    x = np.array(_narrowed(bits, shift), np.uint16).reshape(2, 32)
    codes, bs, ts = orc.nvfp4_per_token(x)
    ec, eb, es = X.nvfp4_per_token([[int(v) for v in row] for row in x])
    assert [F(float(t)) for t in ts] == es
    assert np.array_equal(bs, np.array(eb, np.uint8))
    assert np.array_equal(codes, np.array(ec, np.uint8))
