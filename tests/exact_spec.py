"""Exact rational spec of the quantizers, for pinning the oracle on tiny inputs.

Independent of the oracle: pure Python with ``fractions.Fraction``; every
rounding is a brute-force search for the nearest value of the target format
(minimum distance, exact tie -> even code), and the FP32 scale is rounded by an
explicit exact round-to-nearest-even on the binary32 grid.  It follows the
same readings as the oracle (nearest-even, saturation, sign kept, smallest
unclipped E8M0 exponent, FP32 scale = amax / 2688 as a decode multiplier), but
shares none of its code or arithmetic route.  Slow: tiny tensors only.
"""
from __future__ import annotations

from fractions import Fraction as F
from functools import lru_cache

TWO = F(2)


@lru_cache(maxsize=None)
def bf16_frac(bits: int) -> F:
    sign = -1 if bits & 0x8000 else 1
    E = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert E != 0xFF, "Inf/NaN outside the contract"
    if E == 0:
        mag = F(m, 128) * TWO ** -126
    else:
        mag = (1 + F(m, 128)) * TWO ** (E - 127)
    return sign * mag


def bf16_negative(bits: int) -> bool:
    return bool(bits & 0x8000)


# Non-negative values in code order.
E4M3_POS = [(F(c & 7, 8) * TWO ** -6) if (c >> 3) == 0 else
            (1 + F(c & 7, 8)) * TWO ** ((c >> 3) - 7) for c in range(127)]
E2M1_POS = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def nearest_code(table, q: F) -> int:
    """Index of the table value nearest to q >= 0 (minimum |q - v|); on an
    exact tie the even index wins.  q beyond the table's end -> last index."""
    best, bestd = None, None
    for k, v in enumerate(table):
        d = abs(q - v)
        if best is None or d < bestd or (d == bestd and k % 2 == 0):
            best, bestd = k, d
    return best


def floor_log2(a: F) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while TWO ** e > a:
        e -= 1
    while TWO ** (e + 1) <= a:
        e += 1
    return e


def rn_binary32(q: F) -> F:
    """Exact round-to-nearest-even of q onto the binary32 grid (with
    subnormals; no overflow handling needed here)."""
    if q == 0:
        return F(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(floor_log2(a), -126)
    ulp = TWO ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def e8m0_exponent(A: F) -> int:
    for e in range(-127, 128):
        if A <= 448 * TWO ** e:
            return e
    raise AssertionError


def mxfp8_block(bits_list):
    """One MXFP8 block (any length): returns (scale_byte, codes)."""
    vals = [bf16_frac(b) for b in bits_list]
    A = max(abs(v) for v in vals)
    e = e8m0_exponent(A)
    codes = []
    for b, v in zip(bits_list, vals):
        k = nearest_code(E4M3_POS, abs(v) / TWO ** e)
        codes.append(k | (0x80 if bf16_negative(b) else 0))
    return e + 127, codes


def mxfp8_rowwise(X):
    """X: list of rows of BF16 bit patterns.  Returns (codes, scales)."""
    codes, scales = [], []
    for row in X:
        rc, rs = [], []
        for j in range(0, len(row), 32):
            byte, c = mxfp8_block(row[j:j + 32])
            rs.append(byte)
            rc.extend(c)
        codes.append(rc)
        scales.append(rs)
    return codes, scales


def nvfp4_scale(A: F) -> F:
    return rn_binary32(A / 2688)


def nvfp4_row(row, s: F):
    """One row under FP32 scale s: (packed code bytes, block scale bytes)."""
    out_codes, out_scales = [], []
    for j in range(0, len(row), 16):
        blk = row[j:j + 16]
        vals = [bf16_frac(b) for b in blk]
        A = max(abs(v) for v in vals)
        b = 0 if s == 0 else nearest_code(E4M3_POS, A / (6 * s))
        out_scales.append(b)
        d = E4M3_POS[b]
        nib = []
        for bits, v in zip(blk, vals):
            if d == 0:
                nib.append(0)
            else:
                k = nearest_code(E2M1_POS, abs(v) / (d * s))
                nib.append(k | (0x8 if bf16_negative(bits) else 0))
        for k in range(0, 16, 2):
            out_codes.append(nib[k] | (nib[k + 1] << 4))
    return out_codes, out_scales


def nvfp4_per_token(X):
    """Returns (codes rows, block-scale rows, token scales as Fractions)."""
    C, B, S = [], [], []
    for row in X:
        A = max(abs(bf16_frac(b)) for b in row)
        s = nvfp4_scale(A)
        c, b = nvfp4_row(row, s)
        C.append(c)
        B.append(b)
        S.append(s)
    return C, B, S


def bf16_nearest_sat(y: F) -> int:
    """Bits of the BF16 value nearest to y (ties to even mantissa), saturating
    at the largest finite BF16, sign kept (y == 0 -> +0)."""
    neg = y < 0
    a = abs(y)
    best, bestd = None, None
    # Search the neighbourhood of a's binade: every finite magnitude with the
    # same or adjacent exponent field, plus zero and the subnormals.
    if a == 0:
        cand = [0]
    else:
        e = min(max(floor_log2(a), -127), 127)
        lo = max(e + 127 - 1, 0)
        hi = min(e + 127 + 1, 254)
        cand = [(E << 7) | m for E in range(lo, hi + 1) for m in range(128)] + [0]
    for c in cand:
        d = abs(a - bf16_frac(c))
        if best is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | (0x8000 if neg else 0)
