"""Seeded synthetic inputs for the quantizers (shared by tests, smoke and bench).

This module draws input tensors only; it holds none of the quantizers'
arithmetic.  Every value is drawn in binary64 with numpy's PCG64
(``default_rng(seed)``), rounded to binary32, then rounded to BF16
(round-to-nearest-even, done by torch's CPU conversion).  BF16 tensors are
returned as ``numpy.uint16`` arrays of bit patterns.

Shapes follow the workloads of the page "Miles: end-to-end MXFP8 and per-token
NVFP4 RL on Blackwell": the (2048, 2048) activation with out_features 8192 of
its backward-mode memory tables, the 8192-token maximum response of its
ablation, and the Qwen3-30B-A3B expert layer of that ablation (hidden 2048,
expert intermediate 768, 128 experts, top-8 routing).  No dataset or model
weight is used: synthetic draws stand in for them.

The four MXFP8 data modes (random, boundary, zeros, maxes) follow the page's
bit-alignment paragraph, which names them without defining them; the
definitions below are ours.
"""
from __future__ import annotations

import numpy as np
import torch

BF16_MAX_BITS = 0x7F7F

# Sizes of the expert layer.
HIDDEN = 2048
EXPERT_INTER = 768
N_EXPERTS = 128
TOP_K = 8
N_TOKENS = 32768


def bf16_bits(values) -> np.ndarray:
    """binary64 -> binary32 (numpy, nearest-even) -> BF16 (torch, nearest-even),
    returned as uint16 bit patterns."""
    f32 = np.ascontiguousarray(np.asarray(values, dtype=np.float64).astype(np.float32))
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f64(bits) -> np.ndarray:
    """BF16 bit patterns -> binary64 values (exact), via binary32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# MXFP8 data modes
# ---------------------------------------------------------------------------

def mode_random(rows: int, cols: int, seed: int) -> np.ndarray:
    """N(0,1), then exactly round(0.001 * rows * cols) positions (drawn without
    replacement) multiplied by 100."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, cols))
    n_out = int(round(0.001 * rows * cols))
    idx = rng.choice(rows * cols, size=n_out, replace=False)
    z.reshape(-1)[idx] *= 100.0
    return bf16_bits(z)


def mode_zeros(rows: int, cols: int) -> np.ndarray:
    return np.zeros((rows, cols), np.uint16)


def mode_maxes(rows: int, cols: int) -> np.ndarray:
    """Every element at the largest finite BF16 value."""
    return np.full((rows, cols), BF16_MAX_BITS, np.uint16)


def _e4m3_positive_values() -> np.ndarray:
    """The 127 non-negative finite E4M3 values (format definition: 4-bit
    exponent with bias 7, 3-bit mantissa, subnormals, 0x7F excluded)."""
    vals = []
    for c in range(127):
        E, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if E == 0 else (8 + m) * 2.0 ** (E - 10))
    return np.array(vals, dtype=np.float64)


# Exponents the boundary tiles cycle through: the clamp region (with BF16
# subnormals), the lowest normal exponents, the middle, and the top.
BOUNDARY_EXPONENTS = [-127] + list(range(-126, -116)) + list(range(-20, 21)) + \
    list(range(100, 121))


def _representable(v: np.ndarray) -> np.ndarray:
    """Mask of values that are finite BF16 values (exact round trip)."""
    with np.errstate(over="ignore"):
        back = bf16_to_f64(bf16_bits(v))
    return (back == v) & np.isfinite(back)


def _boundary_candidates(e: int, amax: float) -> np.ndarray:
    """Off-diagonal magnitudes for a tile with exponent e: E4M3 rounding
    midpoints times 2^e and 2^(e+1), and their +-1 BF16-ulp neighbours, kept
    when BF16-representable and not above the tile's amax."""
    v = _e4m3_positive_values()
    mids = 0.5 * (v[:-1] + v[1:])
    cands = np.concatenate([mids * 2.0 ** e, mids * 2.0 ** (e + 1)])
    cands = cands[_representable(cands)]
    bits = bf16_bits(cands)
    neigh = np.concatenate([bits, bits + 1, bits - 1]).astype(np.uint16)
    neigh = neigh[(neigh & 0x7FFF) < 0x7F80]          # finite only
    mags = np.unique(bf16_to_f64(neigh & 0x7FFF))
    mags = mags[(mags > 0) & (mags <= amax)]
    return mags


def mode_boundary(rows: int, cols: int, seed: int) -> np.ndarray:
    """Quantization-boundary data, tiled in 32x32 tiles (rows, cols multiples
    of 32).  Tile t takes exponent e = BOUNDARY_EXPONENTS[t % n] and an amax
    kind k = (t // n) % 3: 448 * 2^e (largest unclipped value), 450 * 2^e
    (next BF16 above it), 2^(e+9) (a power of two).  The amax sits on the
    tile's diagonal, so each row block and each column block of the tile
    holds it once; the other elements are signed E4M3 midpoints times 2^e or
    2^(e+1) and their BF16 neighbours."""
    assert rows % 32 == 0 and cols % 32 == 0
    rng = np.random.default_rng(seed)
    ne = len(BOUNDARY_EXPONENTS)
    cache = {}
    out = np.empty((rows, cols), np.uint16)
    tr, tc = rows // 32, cols // 32
    diag = np.eye(32, dtype=bool)
    for t in range(tr * tc):
        e = BOUNDARY_EXPONENTS[t % ne]
        kind = (t // ne) % 3
        key = (e, kind)
        if key not in cache:
            amax = [448.0 * 2.0 ** e, 450.0 * 2.0 ** e, 2.0 ** (e + 9)][kind]
            if not _representable(np.array([amax]))[0]:
                amax = float(bf16_to_f64(np.array([BF16_MAX_BITS], np.uint16))[0])
            cache[key] = (amax, bf16_bits(_boundary_candidates(e, amax)))
        amax, cand = cache[key]
        tile = np.empty((32, 32), np.uint16)
        amax_bits = bf16_bits(np.array([amax]))[0]
        if cand.size:
            pick = cand[rng.integers(0, cand.size, size=(32, 32))]
        else:
            pick = np.zeros((32, 32), np.uint16)
        signs = rng.integers(0, 2, size=(32, 32)).astype(np.uint16) << 15
        tile[:] = pick | signs
        dsign = rng.integers(0, 2, size=32).astype(np.uint16) << 15
        tile[diag] = amax_bits | dsign
        i, j = divmod(t, tc)
        out[32 * i:32 * i + 32, 32 * j:32 * j + 32] = tile
    return out


def mxfp8_mode(mode: str, rows: int, cols: int, seed: int) -> np.ndarray:
    if mode == "random":
        return mode_random(rows, cols, seed)
    if mode == "boundary":
        return mode_boundary(rows, cols, seed)
    if mode == "zeros":
        return mode_zeros(rows, cols)
    if mode == "maxes":
        return mode_maxes(rows, cols)
    raise ValueError(mode)


MXFP8_MODES = ("random", "boundary", "zeros", "maxes")


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def config1() -> np.ndarray:
    """MXFP8 correctness case: 256x512, i.i.d. N(0,1), seed 0."""
    rng = np.random.default_rng(0)
    return bf16_bits(rng.standard_normal((256, 512)))


def config2_activation(mode: str) -> np.ndarray:
    """MXFP8 row+col of the (2048, 2048) activation, seed 1."""
    return mxfp8_mode(mode, 2048, 2048, 1)


def config2_weight(mode: str) -> np.ndarray:
    """MXFP8 row+col of the 8192x2048 weight (out_features 8192), seed 2."""
    return mxfp8_mode(mode, 8192, 2048, 2)


def student_t_activations(rows: int, cols: int, seed: int) -> np.ndarray:
    """Heavy-tailed activations: Student-t(df=3) * 0.5."""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_t(3, size=(rows, cols)) * 0.5)


def config3() -> np.ndarray:
    """Per-token NVFP4 activations: 8192 tokens x 2048, Student-t(3)*0.5, seed 3."""
    return student_t_activations(8192, HIDDEN, 3)


def config4(n_experts: int = N_EXPERTS):
    """Expert weights N(0, 0.02), drawn expert by expert in the order gate, up,
    down, seed 4.  Returns gate [E][768][2048], up [E][768][2048],
    down [E][2048][768]."""
    rng = np.random.default_rng(4)
    gate = np.empty((n_experts, EXPERT_INTER, HIDDEN), np.uint16)
    up = np.empty_like(gate)
    down = np.empty((n_experts, HIDDEN, EXPERT_INTER), np.uint16)
    for e in range(n_experts):
        gate[e] = bf16_bits(rng.normal(0.0, 0.02, size=(EXPERT_INTER, HIDDEN)))
        up[e] = bf16_bits(rng.normal(0.0, 0.02, size=(EXPERT_INTER, HIDDEN)))
        down[e] = bf16_bits(rng.normal(0.0, 0.02, size=(HIDDEN, EXPERT_INTER)))
    return gate, up, down


def routing(n_tokens: int = N_TOKENS, n_experts: int = N_EXPERTS, top_k: int = TOP_K,
            seed: int = 6):
    """Uniform top-k routing: each token picks top_k distinct experts from
    rng.random((n_tokens, n_experts)).argsort(1)[:, :top_k].  Returns
    (token_index[R], offsets[E+1]) of the rows sorted stably by (expert, token)."""
    rng = np.random.default_rng(seed)
    choice = rng.random((n_tokens, n_experts)).argsort(1)[:, :top_k]
    tok = np.repeat(np.arange(n_tokens, dtype=np.int64), top_k)
    exp = choice.reshape(-1).astype(np.int64)
    order = np.lexsort((tok, exp))
    counts = np.bincount(exp, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return tok[order], offsets


def dispatch_maps(n_tokens: int = N_TOKENS, n_experts: int = N_EXPERTS, top_k: int = TOP_K,
                  seed: int = 6, drop: float = 0.0):
    """Routing of `routing` (same draws for drop = 0) as the two index maps of
    a fused dispatch: row_tokens[R] (token of each expert-sorted row),
    token_rows[n_tokens][top_k] (row of each copy; -1 for a dropped copy) and
    the segment offsets[E+1].  drop > 0 drops that fraction of the copies
    (seed + 1000 picks them), as a capacity limit would."""
    rng = np.random.default_rng(seed)
    choice = rng.random((n_tokens, n_experts)).argsort(1)[:, :top_k]
    tok = np.repeat(np.arange(n_tokens, dtype=np.int64), top_k)
    exp = choice.reshape(-1).astype(np.int64)
    keep = np.ones(tok.size, bool)
    if drop > 0:
        keep = np.random.default_rng(seed + 1000).random(tok.size) >= drop
    flat = np.nonzero(keep)[0]
    order = flat[np.lexsort((tok[flat], exp[flat]))]      # flat copy index of each row
    counts = np.bincount(exp[flat], minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    token_rows = np.full(tok.size, -1, np.int64)
    token_rows[order] = np.arange(order.size, dtype=np.int64)
    return tok[order], token_rows.reshape(n_tokens, top_k), offsets


def config5_dispatch(n_tokens: int = N_TOKENS, hidden: int = HIDDEN):
    """Config 5's tokens (unpermuted, [n_tokens][hidden]) and routing as
    dispatch maps: (tokens, row_tokens, token_rows, offsets).  Gathering
    tokens[row_tokens] gives exactly config5()'s X."""
    tokens = student_t_activations(n_tokens, hidden, 5)
    row_tokens, token_rows, offsets = dispatch_maps(n_tokens, N_EXPERTS, TOP_K, 6)
    return tokens, row_tokens, token_rows, offsets


def config5(n_tokens: int = N_TOKENS, hidden: int = HIDDEN):
    """Grouped MoE input: tokens Student-t(3)*0.5 (seed 5) routed top-8 of 128
    experts (seed 6), gathered expert-sorted.  Returns (X[R][hidden],
    offsets[129])."""
    tokens = student_t_activations(n_tokens, hidden, 5)
    tok_idx, offsets = routing(n_tokens, N_EXPERTS, TOP_K, 6)
    return np.ascontiguousarray(tokens[tok_idx]), offsets


def ragged_offsets(total_rows: int, n_groups: int, seed: int = 7,
                   forced=(0, 1, 31, 32, 33, 4096)) -> np.ndarray:
    """Segment offsets whose sizes include every value in `forced`; the other
    sizes are drawn from U{0..4096}, then rescaled so that all sizes sum to
    total_rows (the forced ones are kept as they are)."""
    rng = np.random.default_rng(seed)
    forced = [f for f in forced if f <= total_rows]
    n_free = n_groups - len(forced)
    assert n_free >= 1
    free = rng.integers(0, 4097, size=n_free).astype(np.float64)
    rest = total_rows - sum(forced)
    assert rest >= 0
    if free.sum() == 0:
        free[:] = 1.0
    free = np.floor(free * rest / free.sum()).astype(np.int64)
    free[-1] += rest - free.sum()
    sizes = np.array(list(forced) + list(free), dtype=np.int64)
    perm = rng.permutation(n_groups)
    sizes = sizes[perm]
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def nvfp4_boundary(rows: int, cols: int, seed: int) -> np.ndarray:
    """NVFP4 boundary rows.  Row kinds cycle: (0) amax 21 * 2^j, so the FP32
    scale amax/2688 is an exact power of two, with small-mantissa dyadic
    elements (k * 2^m, k < 16) that land on E2M1 and E4M3 rounding ties;
    (1) the same with amax 5.25 * 2^j and elements from a coarser grid;
    (2) tiny rows whose amax is a few BF16 subnormal steps, so the FP32 scale
    is itself subnormal; (3) N(0,1) rows with exact zeros and signed zeros, in
    which one 16-block is scaled by 2^-24 so that its block scale is zero."""
    rng = np.random.default_rng(seed)
    out = np.empty((rows, cols), np.uint16)
    for r in range(rows):
        kind = r % 4
        if kind in (0, 1):
            j = int(rng.integers(-100, 100))
            amax = (21.0 if kind == 0 else 5.25) * 2.0 ** j
            k = rng.integers(0, 16, size=cols).astype(np.float64)
            m = rng.integers(-6, 0, size=cols) if kind == 0 else rng.integers(-3, 0, size=cols)
            v = k * 2.0 ** (m + j) * np.where(rng.random(cols) < 0.5, -1.0, 1.0)
            v = np.clip(v, -amax, amax)
            v[int(rng.integers(0, cols))] = amax
            out[r] = bf16_bits(v)
        elif kind == 2:
            steps = rng.integers(0, 64, size=cols)
            bits = steps.astype(np.uint16) | (rng.integers(0, 2, size=cols).astype(np.uint16) << 15)
            out[r] = bits
        else:
            v = rng.standard_normal(cols)
            v[rng.random(cols) < 0.1] = 0.0
            b = bf16_bits(v)
            neg0 = rng.random(cols) < 0.05
            b[neg0] = 0x8000
            j = int(rng.integers(0, cols // 16))
            tiny = bf16_bits(v[16 * j:16 * j + 16] * 2.0 ** -24)
            tiny[rng.random(16) < 0.2] = 0x8000
            b[16 * j:16 * j + 16] = tiny
            out[r] = b
    return out
