"""CPU oracle for the block-scaled quantizers -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The GPU library never does, and shares no
code with it.  The arithmetic lives in ``mxq_oracle.c`` (plain C, exact
comparisons in binary64; its header states the contract and the readings
taken); this module only marshals numpy arrays to it.

Conventions: BF16 tensors are ``numpy.uint16`` arrays of bit patterns; codes
and scale bytes are ``numpy.uint8``; FP32 scales are ``numpy.float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
_LIB = os.path.join(_HERE, "libmxq_oracle.so")

_lib = None


def build(verbose: bool = False, src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile mxq_oracle.c with gcc into libmxq_oracle.so (no fast-math, no
    FMA contraction, OpenMP over rows).  extra_flags: more gcc flags (the
    sanitizer test builds an instrumented copy)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra", *extra_flags,
           src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def lib():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("MXQ_ORACLE_LIB", _LIB)   # the mutation test points it elsewhere
    if not os.path.exists(path):
        raise RuntimeError(f"oracle library not built: {path} (run oracle.build())")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    sig = {
        "oracle_bf16_value": (ctypes.c_double, [ctypes.c_uint16]),
        "oracle_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
        "oracle_e2m1_value": (ctypes.c_double, [ctypes.c_uint8]),
        "oracle_e8m0_value": (ctypes.c_double, [ctypes.c_uint8]),
        "oracle_e4m3_nearest": (ctypes.c_uint8, [ctypes.c_double, ctypes.c_double]),
        "oracle_e2m1_nearest": (ctypes.c_uint8, [ctypes.c_double, ctypes.c_double]),
        "oracle_e8m0_byte": (ctypes.c_int, [ctypes.c_double]),
        "oracle_e8m0_byte_ocp": (ctypes.c_int, [ctypes.c_double]),
        "oracle_mxfp8_rowwise_rule": (None, [P, I64, I64, P, P, ctypes.c_int]),
        "oracle_mxfp8_colwise_rule": (None, [P, I64, I64, P, P, ctypes.c_int]),
        "oracle_nvfp4_scale": (ctypes.c_float, [ctypes.c_double]),
        "oracle_bf16_round_sat": (ctypes.c_uint16, [ctypes.c_double]),
        "oracle_mxfp8_rowwise": (None, [P, I64, I64, P, P]),
        "oracle_mxfp8_colwise": (None, [P, I64, I64, P, P]),
        "oracle_mxfp8_colwise_grouped": (None, [P, I64, P, I64, P, P, P]),
        "oracle_nvfp4_per_token": (None, [P, I64, I64, P, P, P]),
        "oracle_nvfp4_with_scale": (None, [P, I64, I64, ctypes.c_float, P, P]),
        "oracle_nvfp4_gateup_pair": (None, [P, P, I64, I64, I64, P, P, P, P, P]),
        "oracle_dequant_mxfp8_rowwise": (None, [P, P, I64, I64, P]),
        "oracle_dequant_mxfp8_colwise": (None, [P, P, I64, I64, P]),
        "oracle_dequant_nvfp4": (None, [P, P, P, I64, I64, I64, P]),
        "oracle_e4m3_nearest_many": (None, [P, P, I64, P]),
        "oracle_e2m1_nearest_many": (None, [P, P, I64, P]),
        "oracle_e8m0_byte_many": (None, [P, I64, P]),
        "oracle_nvfp4_scale_many": (None, [P, I64, P]),
        "oracle_bf16_round_sat_many": (None, [P, I64, P]),
        "oracle_max_threads": (ctypes.c_int, []),
        "oracle_set_threads": (None, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("BF16 input must be a uint16 array of bit patterns")
    return x


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for later calls (timing only: results never depend on it)."""
    lib().oracle_set_threads(int(n))


# -- scalar helpers ---------------------------------------------------------

def bf16_value(b: int) -> float:
    return lib().oracle_bf16_value(b)


def e4m3_value(c: int) -> float:
    return lib().oracle_e4m3_value(c)


def e2m1_value(c: int) -> float:
    return lib().oracle_e2m1_value(c)


def e8m0_value(b: int) -> float:
    return lib().oracle_e8m0_value(b)


def e8m0_byte(amax: float) -> int:
    return lib().oracle_e8m0_byte(amax)


def nvfp4_scale(amax: float) -> float:
    return lib().oracle_nvfp4_scale(amax)


def e4m3_nearest(x: float, D: float) -> int:
    return lib().oracle_e4m3_nearest(x, D)


def e2m1_nearest(x: float, D: float) -> int:
    return lib().oracle_e2m1_nearest(x, D)


def bf16_round_sat(y: float) -> int:
    return lib().oracle_bf16_round_sat(y)


# -- array helpers ------------------------------------------------------------

def e4m3_nearest_many(x, D) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    D = np.ascontiguousarray(np.broadcast_to(D, x.shape), dtype=np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_nearest_many(_p(x), _p(D), x.size, _p(out))
    return out


def e2m1_nearest_many(x, D) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    D = np.ascontiguousarray(np.broadcast_to(D, x.shape), dtype=np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e2m1_nearest_many(_p(x), _p(D), x.size, _p(out))
    return out


def e8m0_byte_many(A) -> np.ndarray:
    A = np.ascontiguousarray(A, dtype=np.float64)
    out = np.empty(A.shape, np.int32)
    lib().oracle_e8m0_byte_many(_p(A), A.size, _p(out))
    return out


def nvfp4_scale_many(A) -> np.ndarray:
    A = np.ascontiguousarray(A, dtype=np.float64)
    out = np.empty(A.shape, np.float32)
    lib().oracle_nvfp4_scale_many(_p(A), A.size, _p(out))
    return out


def bf16_round_sat_many(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, np.uint16)
    lib().oracle_bf16_round_sat_many(_p(y), y.size, _p(out))
    return out


# -- tensor-level oracle ----------------------------------------------------------

def mxfp8_rowwise(x):
    """MXFP8 rowwise 1x32 copy of X[rows][cols]: (codes[rows][cols],
    scales[rows][cols/32])."""
    x = _u16(x)
    rows, cols = x.shape
    assert cols % 32 == 0
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    lib().oracle_mxfp8_rowwise(_p(x), rows, cols, _p(codes), _p(scales))
    return codes, scales


def mxfp8_colwise(x):
    """MXFP8 columnwise 32x1 copy: (codes[rows][cols], scales[rows/32][cols])."""
    x = _u16(x)
    rows, cols = x.shape
    assert rows % 32 == 0
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty((rows // 32, cols), np.uint8)
    lib().oracle_mxfp8_colwise(_p(x), rows, cols, _p(codes), _p(scales))
    return codes, scales


def e8m0_byte_ocp(amax: float) -> int:
    return lib().oracle_e8m0_byte_ocp(amax)


def mxfp8_ocp_floor(x):
    """Both MXFP8 copies under the OCP MX scale rule instead of the contract's
    (a comparison variant; it clips): the shared exponent is floor(log2 amax)
    - 8, E4M3's largest exponent, and each element is the nearest E4M3 of
    x / 2^e, saturating at 448 (OCP Microscaling Formats v1.0, the
    conversion of a block to MX; named as the alternative to P2's rounded-up
    scale on the page "Miles: end-to-end MXFP8 and per-token NVFP4 RL on
    Blackwell").  Returns (row codes, row scales, col codes, col scales)."""
    x = _u16(x)
    rows, cols = x.shape
    assert cols % 32 == 0 and rows % 32 == 0
    rc = np.empty((rows, cols), np.uint8)
    rs = np.empty((rows, cols // 32), np.uint8)
    cc = np.empty((rows, cols), np.uint8)
    cs = np.empty((rows // 32, cols), np.uint8)
    lib().oracle_mxfp8_rowwise_rule(_p(x), rows, cols, _p(rc), _p(rs), 1)
    lib().oracle_mxfp8_colwise_rule(_p(x), rows, cols, _p(cc), _p(cs), 1)
    return rc, rs, cc, cs


def mxfp8_colwise_grouped(x, offsets):
    """Columnwise copy over ragged segments [offsets[e], offsets[e+1]):
    (codes[R][cols], scales[P_G][cols], P[G+1])."""
    x = _u16(x)
    rows, cols = x.shape
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    G = off.size - 1
    n_scale_rows = int(sum((int(off[e + 1]) - int(off[e]) + 31) // 32 for e in range(G)))
    codes = np.zeros((rows, cols), np.uint8)
    scales = np.zeros((max(n_scale_rows, 0), cols), np.uint8)
    P = np.empty(G + 1, np.int64)
    lib().oracle_mxfp8_colwise_grouped(_p(x), cols, _p(off), G, _p(codes),
                                       _p(scales), _p(P))
    return codes, scales, P


def nvfp4_per_token(x):
    """Per-token NVFP4: (codes[rows][cols/2], block_scales[rows][cols/16],
    token_scales[rows] float32)."""
    x = _u16(x)
    rows, cols = x.shape
    assert cols % 16 == 0
    codes = np.empty((rows, cols // 2), np.uint8)
    bs = np.empty((rows, cols // 16), np.uint8)
    ts = np.empty(rows, np.float32)
    lib().oracle_nvfp4_per_token(_p(x), rows, cols, _p(codes), _p(bs), _p(ts))
    return codes, bs, ts


def nvfp4_with_scale(x, s: float):
    """NVFP4 of X under a given FP32 scale s: (codes, block_scales)."""
    x = _u16(x)
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    bs = np.empty((rows, cols // 16), np.uint8)
    lib().oracle_nvfp4_with_scale(_p(x), rows, cols, ctypes.c_float(float(s)),
                                  _p(codes), _p(bs))
    return codes, bs


def nvfp4_gateup_pair(gate, up=None):
    """Weight export: one FP32 scale per expert over gate[e] and up[e] (or gate[e]
    alone when up is None).  gate, up: [E][rows][cols].  Returns (gate_codes,
    gate_block_scales, up_codes, up_block_scales, scope_scales[E])."""
    gate = _u16(gate)
    E, rows, cols = gate.shape
    gc = np.empty((E, rows, cols // 2), np.uint8)
    gb = np.empty((E, rows, cols // 16), np.uint8)
    sc = np.empty(E, np.float32)
    if up is not None:
        up = _u16(up)
        assert up.shape == gate.shape
        uc = np.empty_like(gc)
        ub = np.empty_like(gb)
        lib().oracle_nvfp4_gateup_pair(_p(gate), _p(up), E, rows, cols, _p(gc), _p(gb),
                                       _p(uc), _p(ub), _p(sc))
        return gc, gb, uc, ub, sc
    lib().oracle_nvfp4_gateup_pair(_p(gate), None, E, rows, cols, _p(gc), _p(gb),
                                   None, None, _p(sc))
    return gc, gb, None, None, sc


def dequant_mxfp8_rowwise(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, cols = codes.shape
    out = np.empty((rows, cols), np.uint16)
    lib().oracle_dequant_mxfp8_rowwise(_p(codes), _p(scales), rows, cols, _p(out))
    return out


def dequant_mxfp8_colwise(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, cols = codes.shape
    out = np.empty((rows, cols), np.uint16)
    lib().oracle_dequant_mxfp8_colwise(_p(codes), _p(scales), rows, cols, _p(out))
    return out


def dequant_nvfp4(codes, block_scales, fp32_scales, rows_per_scale: int) -> np.ndarray:
    """NVFP4 -> BF16 with s = fp32_scales[row // rows_per_scale]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    bs = np.ascontiguousarray(block_scales, np.uint8)
    fs = np.ascontiguousarray(fp32_scales, np.float32)
    rows, half = codes.shape
    cols = 2 * half
    out = np.empty((rows, cols), np.uint16)
    lib().oracle_dequant_nvfp4(_p(codes), _p(bs), _p(fs), int(rows_per_scale), rows,
                               cols, _p(out))
    return out


def quantize_dequant_mxfp8_rowwise(x):
    """Rowwise MXFP8 of x and the BF16 dequantization of those codes: the
    forward operand and the BF16 copy that a dequantized backward consumes
    (page "Miles: end-to-end MXFP8 and per-token NVFP4 RL on Blackwell",
    dequantized-backward paragraph).  By definition the composition of the
    two steps; returns (codes, scales, bf16 bits)."""
    codes, scales = mxfp8_rowwise(x)
    return codes, scales, dequant_mxfp8_rowwise(codes, scales)


def quantize_dequant_nvfp4(x):
    """Per-token NVFP4 of x and its BF16 dequantization (same paragraph);
    returns (codes, block_scales, token_scales, bf16 bits)."""
    codes, bs, ts = nvfp4_per_token(x)
    return codes, bs, ts, dequant_nvfp4(codes, bs, ts, 1)


def mxfp8_gemm(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    """The exact block-scaled product C = A B^T of two MXFP8 operands stored
    K-contiguous (rowwise copies: a [M][K], b [N][K], E8M0 scales per 32
    along K): C[m][n] = sum_k dec(a[m][k]) 2^(sa - 127) dec(b[n][k]) 2^(sb - 127)
    (page "Miles: end-to-end MXFP8 and per-token NVFP4 RL on Blackwell",
    MXFP8 format and recipe paragraphs: the forward GEMM consumes the rowwise
    copies).  Every decoded value and product is exact in binary64; the sum
    is a binary64 matrix product, whose rounding (at most K 2^-53 sum |a b|)
    is far below the fp32 accumulation being checked.  Returns float64 [M][N]
    and the magnitude sum S[m][n] = sum_k |a b| that error bounds scale with."""
    table = np.array([e4m3_value(c) for c in range(256)], np.float64)
    table[[0x7F, 0xFF]] = np.nan                        # never produced by the quantizer

    def decode(codes, scales):
        codes = np.ascontiguousarray(codes, np.uint8)
        scales = np.ascontiguousarray(scales, np.uint8)
        s = np.ldexp(1.0, scales.astype(np.int64) - 127)
        return table[codes] * np.repeat(s, 32, axis=1)

    A = decode(a_codes, a_scales)
    B = decode(b_codes, b_scales)
    return A @ B.T, np.abs(A) @ np.abs(B).T


def nvfp4_gemm(a_codes, a_block_scales, a_scales, rows_per_a, b_codes, b_block_scales,
               b_scales, rows_per_b) -> np.ndarray:
    """The exact block-scaled product of two NVFP4 operands stored
    K-contiguous: C[m][n] = sa[m // rows_per_a] sb[n // rows_per_b]
    sum_k dec(a) dec(ba) dec(b) dec(bb) (page "Miles: end-to-end MXFP8 and
    per-token NVFP4 RL on Blackwell", NVFP4 format and per-token activation
    scale paragraphs: an element's value is its E2M1 code times its 16-block's
    E4M3 scale times the FP32 scale of its scope).  Every decoded value and
    product is exact in binary64, the sum a binary64 matrix product.  Returns
    float64 [M][N] and the magnitude sum S = sum_k |a b| times |sa sb|."""
    e2 = np.array([e2m1_value(c) for c in range(16)], np.float64)
    e4 = np.array([e4m3_value(c) for c in range(256)], np.float64)

    def decode(codes, bs, fs, per):
        codes = np.ascontiguousarray(codes, np.uint8)
        rows, half = codes.shape
        vals = np.empty((rows, 2 * half), np.float64)
        vals[:, 0::2] = e2[codes & 15]
        vals[:, 1::2] = e2[codes >> 4]
        vals *= np.repeat(e4[np.ascontiguousarray(bs, np.uint8)], 16, axis=1)
        s = np.asarray(fs, np.float32).astype(np.float64)[np.arange(rows) // per]
        return vals, s

    A, sa = decode(a_codes, a_block_scales, a_scales, rows_per_a)
    B, sb = decode(b_codes, b_block_scales, b_scales, rows_per_b)
    scale = sa[:, None] * sb[None, :]
    return (A @ B.T) * scale, (np.abs(A) @ np.abs(B).T) * np.abs(scale)
