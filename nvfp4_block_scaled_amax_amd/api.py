"""Tensor-level helpers over the C ABI: allocate outputs with torch.empty on
the input's device and call the library.  BF16 inputs may be torch.bfloat16 or
int16/uint16 tensors of bit patterns; they must be contiguous HIP tensors."""
from __future__ import annotations

from typing import NamedTuple, Optional

import torch

from . import _binding as B


def _bf16_bits(x: torch.Tensor) -> torch.Tensor:
    if x.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        if not x.is_contiguous():
            raise ValueError("input must be contiguous")
        return x
    raise TypeError(f"expected a BF16 tensor (or its int16 bits), got {x.dtype}")


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


class MXFP8RowCol(NamedTuple):
    row_codes: Optional[torch.Tensor]
    row_scales: Optional[torch.Tensor]
    col_codes: Optional[torch.Tensor]
    col_scales: Optional[torch.Tensor]


def mxfp8_quantize_rowcol(x, rowwise: bool = True, colwise: bool = True,
                          stream=None) -> MXFP8RowCol:
    x = _bf16_bits(x)
    rows, cols = x.shape
    u8 = torch.uint8
    rc = _empty((rows, cols), u8, x) if rowwise else None
    rs = _empty((rows, cols // 32), u8, x) if rowwise else None
    cc = _empty((rows, cols), u8, x) if colwise else None
    cs = _empty((rows // 32, cols), u8, x) if colwise else None
    B.mxq_mxfp8_quantize_rowcol(x, rows, cols, rc, rs, cc, cs, stream)
    return MXFP8RowCol(rc, rs, cc, cs)


def mxfp8_quantize_rowcol_t(x, rowwise: bool = True, stream=None) -> MXFP8RowCol:
    """Both MXFP8 copies, the columnwise one transposed: col_codes [cols][rows],
    col_scales [cols][rows/32] (K-contiguous for a GEMM contracting over rows)."""
    x = _bf16_bits(x)
    rows, cols = x.shape
    u8 = torch.uint8
    rc = _empty((rows, cols), u8, x) if rowwise else None
    rs = _empty((rows, cols // 32), u8, x) if rowwise else None
    cc = _empty((cols, rows), u8, x)
    cs = _empty((cols, rows // 32), u8, x)
    B.mxq_mxfp8_quantize_rowcol_t(x, rows, cols, rc, rs, cc, cs, stream)
    return MXFP8RowCol(rc, rs, cc, cs)


def mxfp8_quantize_ocp_floor(x, rowwise: bool = True, colwise: bool = True,
                             stream=None) -> MXFP8RowCol:
    """Comparison variant: both MXFP8 copies under the OCP MX scale rule
    (floor(log2 amax) - 8, saturating at 448), which clips."""
    x = _bf16_bits(x)
    rows, cols = x.shape
    u8 = torch.uint8
    rc = _empty((rows, cols), u8, x) if rowwise else None
    rs = _empty((rows, cols // 32), u8, x) if rowwise else None
    cc = _empty((rows, cols), u8, x) if colwise else None
    cs = _empty((rows // 32, cols), u8, x) if colwise else None
    B.mxq_mxfp8_quantize_ocp_floor(x, rows, cols, rc, rs, cc, cs, stream)
    return MXFP8RowCol(rc, rs, cc, cs)


class NVFP4(NamedTuple):
    codes: torch.Tensor
    block_scales: torch.Tensor
    fp32_scales: torch.Tensor


def nvfp4_quantize_per_token(x, stream=None) -> NVFP4:
    x = _bf16_bits(x)
    rows, cols = x.shape
    codes = _empty((rows, cols // 2), torch.uint8, x)
    bs = _empty((rows, cols // 16), torch.uint8, x)
    ts = _empty((rows,), torch.float32, x)
    B.mxq_nvfp4_quantize_per_token(x, rows, cols, codes, bs, ts, stream)
    return NVFP4(codes, bs, ts)


def nvfp4_quantize_per_token_approx(x, stream=None) -> NVFP4:
    """Opt-in approximate per-token NVFP4 (not the contract): one
    reciprocal-multiply and one conversion per block scale and per code."""
    x = _bf16_bits(x)
    rows, cols = x.shape
    codes = _empty((rows, cols // 2), torch.uint8, x)
    bs = _empty((rows, cols // 16), torch.uint8, x)
    ts = _empty((rows,), torch.float32, x)
    B.mxq_nvfp4_quantize_per_token_approx(x, rows, cols, codes, bs, ts, stream)
    return NVFP4(codes, bs, ts)


def nvfp4_quantize_per_tensor(x, stream=None) -> NVFP4:
    """Comparison variant: NVFP4 of an activation tensor with ONE FP32 scale
    for the whole tensor (the batch-dependent scope the per-token recipe
    replaces); the weight-export call with a single one-tensor scope."""
    x = _bf16_bits(x)
    rows, cols = x.shape
    codes = _empty((1, rows, cols // 2), torch.uint8, x)
    bs = _empty((1, rows, cols // 16), torch.uint8, x)
    s = _empty((1,), torch.float32, x)
    B.mxq_nvfp4_quantize_gateup_pair(x, None, 1, rows, cols, codes, bs, None, None, s, stream)
    return NVFP4(codes[0], bs[0], s)


class GateUpNVFP4(NamedTuple):
    gate_codes: torch.Tensor
    gate_block_scales: torch.Tensor
    up_codes: Optional[torch.Tensor]
    up_block_scales: Optional[torch.Tensor]
    scope_scales: torch.Tensor


def nvfp4_quantize_gateup_pair(gate, up=None, stream=None) -> GateUpNVFP4:
    gate = _bf16_bits(gate)
    E, rows, cols = gate.shape
    gc = _empty((E, rows, cols // 2), torch.uint8, gate)
    gb = _empty((E, rows, cols // 16), torch.uint8, gate)
    uc = ub = None
    if up is not None:
        up = _bf16_bits(up)
        if up.shape != gate.shape:
            raise ValueError("gate and up must have the same shape")
        uc = torch.empty_like(gc)
        ub = torch.empty_like(gb)
    sc = _empty((E,), torch.float32, gate)
    B.mxq_nvfp4_quantize_gateup_pair(gate, up, E, rows, cols, gc, gb, uc, ub, sc, stream)
    return GateUpNVFP4(gc, gb, uc, ub, sc)


def nvfp4_quantize_gateup_pair_amax(gate, up, scope_amax, stream=None) -> GateUpNVFP4:
    """The export with each scope's amax supplied: scope_amax is a device
    tensor of n_experts BF16 values (torch.bfloat16 or int16 bits)."""
    gate = _bf16_bits(gate)
    E, rows, cols = gate.shape
    amax = _bf16_bits(scope_amax)
    if amax.numel() != E:
        raise ValueError("scope_amax must hold one value per expert")
    gc = _empty((E, rows, cols // 2), torch.uint8, gate)
    gb = _empty((E, rows, cols // 16), torch.uint8, gate)
    uc = ub = None
    if up is not None:
        up = _bf16_bits(up)
        if up.shape != gate.shape:
            raise ValueError("gate and up must have the same shape")
        uc = torch.empty_like(gc)
        ub = torch.empty_like(gb)
    sc = _empty((E,), torch.float32, gate)
    B.mxq_nvfp4_quantize_gateup_pair_amax(gate, up, amax, E, rows, cols, gc, gb, uc, ub, sc,
                                          stream)
    return GateUpNVFP4(gc, gb, uc, ub, sc)


def dequantize_bf16(fmt: int, codes, scales, fp32_scales=None, rows_per_fp32_scale: int = 1,
                    stream=None) -> torch.Tensor:
    """Returns a torch.bfloat16 tensor [rows][cols]."""
    rows = codes.shape[0] if codes.dim() == 2 else codes.shape[0] * codes.shape[1]
    last = codes.shape[-1]
    cols = 2 * last if fmt == B.MXQ_FMT_NVFP4 else last
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=codes.device)
    B.mxq_dequantize_bf16(fmt, codes, scales, fp32_scales, rows_per_fp32_scale, rows, cols, out,
                          stream)
    return out


class QuantDequant(NamedTuple):
    codes: Optional[torch.Tensor]
    scales: Optional[torch.Tensor]
    fp32_scales: Optional[torch.Tensor]     # NVFP4 only
    dequant: torch.Tensor                    # torch.bfloat16 [rows][cols]


def quantize_dequant_bf16(fmt: int, x, keep_codes: bool = True, stream=None) -> QuantDequant:
    """Rowwise MXFP8 (fmt MXQ_FMT_MXFP8_ROW) or per-token NVFP4 and the BF16
    dequantization of the result, in one pass; keep_codes=False stores only
    the dequantized copy."""
    x = _bf16_bits(x)
    rows, cols = x.shape
    u8 = torch.uint8
    codes = scales = ts = None
    if fmt == B.MXQ_FMT_NVFP4:
        if keep_codes:
            codes, scales = _empty((rows, cols // 2), u8, x), _empty((rows, cols // 16), u8, x)
            ts = _empty((rows,), torch.float32, x)
    elif keep_codes:
        codes, scales = _empty((rows, cols), u8, x), _empty((rows, cols // 32), u8, x)
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=x.device)
    B.mxq_quantize_dequant_bf16(fmt, x, rows, cols, codes, scales, ts, out, stream)
    return QuantDequant(codes, scales, ts, out)


def mxfp8_gemm(a_codes, a_scales, b_codes, b_scales, out_dtype=torch.bfloat16,
               stream=None) -> torch.Tensor:
    """C = A x B^T on MXFP8 operands (rowwise copies: a [M][K], b [N][K] with
    [.][K/32] E8M0 scales); returns C [M][N] as fp32 or BF16."""
    M, K = a_codes.shape
    N = b_codes.shape[0]
    c = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    code = B.MXQ_OUT_BF16 if out_dtype == torch.bfloat16 else B.MXQ_OUT_F32
    B.mxq_mxfp8_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, code, c, stream)
    return c


def mxfp8_grouped_gemm(a_codes, a_scales, b_codes, b_scales, seg_offsets,
                       out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    """Per-expert C[r] = A[r] x B_e^T for the rows r of each segment e of
    seg_offsets (device int64 [G+1]): a [R][K] and a_scales [R][K/32] are the
    expert-sorted rowwise MXFP8 copy, b [G][N][K] and b_scales [G][N][K/32]
    the experts' weights; returns C [R][N] as fp32 or BF16 (rows outside
    every segment left unwritten)."""
    R, K = a_codes.shape
    G, N = b_codes.shape[0], b_codes.shape[1]
    c = torch.empty((R, N), dtype=out_dtype, device=a_codes.device)
    code = B.MXQ_OUT_BF16 if out_dtype == torch.bfloat16 else B.MXQ_OUT_F32
    B.mxq_mxfp8_grouped_gemm(a_codes, a_scales, b_codes, b_scales, seg_offsets, G, R, N, K, code,
                             c, stream)
    return c


class GroupedColT(NamedTuple):
    codes_t: torch.Tensor         # [cols][pitch]
    scales_t: torch.Tensor        # [cols][pitch / 32]
    block_offsets: torch.Tensor   # [G + 1] int64: segment e's first 32-row block


def grouped_colt_pitch(total_rows: int, n_groups: int) -> int:
    """Row pitch of the grouped transposed columnwise copy."""
    return -(-total_rows // 128) * 128 + 128 * n_groups


def mxfp8_grouped_colwise_t(x, seg_offsets, stream=None) -> GroupedColT:
    """The grouped columnwise MXFP8 copy of the expert-sorted rows x [R][cols],
    transposed with every segment padded to 128 rows (the weight-gradient
    operand layout)."""
    x = _bf16_bits(x)
    R, cols = x.shape
    G = seg_offsets.numel() - 1
    pitch = grouped_colt_pitch(R, G)
    out = GroupedColT(_empty((cols, pitch), torch.uint8, x),
                      _empty((cols, pitch // 32), torch.uint8, x),
                      _empty((G + 1,), torch.int64, x))
    B.mxq_mxfp8_grouped_colwise_t(x, R, cols, seg_offsets, G, out.codes_t, out.scales_t,
                                  out.block_offsets, stream)
    return out


def mxfp8_grouped_quantize_rowcol_t(x, seg_offsets, stream=None):
    """From one read of the expert-sorted rows x [R][cols]: the rowwise MXFP8
    copy (codes [R][cols], scales [R][cols/32], as the grouped quantize writes
    it) and the grouped transposed padded columnwise copy.  Returns
    (row_codes, row_scales, GroupedColT)."""
    x = _bf16_bits(x)
    R, cols = x.shape
    G = seg_offsets.numel() - 1
    pitch = grouped_colt_pitch(R, G)
    rc = _empty((R, cols), torch.uint8, x)
    rs = _empty((R, cols // 32), torch.uint8, x)
    out = GroupedColT(_empty((cols, pitch), torch.uint8, x),
                      _empty((cols, pitch // 32), torch.uint8, x),
                      _empty((G + 1,), torch.int64, x))
    B.mxq_mxfp8_grouped_quantize_rowcol_t(x, R, cols, seg_offsets, G, rc, rs, out.codes_t,
                                          out.scales_t, out.block_offsets, stream)
    return rc, rs, out


def mxfp8_grouped_wgrad(a: GroupedColT, b: GroupedColT, out_dtype=torch.float32,
                        stream=None) -> torch.Tensor:
    """Per-expert C_e = A_e x B_e^T contracting over each segment's rows, from
    two grouped transposed copies over the same segments (a from dY, b from
    X: C_e = dW_e); returns C [G][M][N]."""
    M, pitch = a.codes_t.shape
    N = b.codes_t.shape[0]
    G = a.block_offsets.numel() - 1
    c = torch.empty((G, M, N), dtype=out_dtype, device=a.codes_t.device)
    code = B.MXQ_OUT_BF16 if out_dtype == torch.bfloat16 else B.MXQ_OUT_F32
    B.mxq_mxfp8_grouped_wgrad(a.codes_t, a.scales_t, b.codes_t, b.scales_t, a.block_offsets, G,
                              M, N, pitch, code, c, stream)
    return c


def nvfp4_grouped_gemm(a_codes, a_block_scales, a_scales, b_codes, b_block_scales, b_scales,
                       seg_offsets, out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    """Per-expert C[r] = a_scales[r] b_scales[e] A[r] x B_e^T for the rows r of
    each segment e of seg_offsets (device int64 [G+1]): a [R][K/2] codes,
    [R][K/16] block scales and [R] FP32 scales (the grouped per-token NVFP4
    copy); b [G][N][K/2], [G][N][K/16] and [G] FP32 scope scales (the
    experts' exported weights); returns C [R][N] as fp32 or BF16."""
    R, K = a_codes.shape[0], 2 * a_codes.shape[1]
    G, N = b_codes.shape[0], b_codes.shape[1]
    c = torch.empty((R, N), dtype=out_dtype, device=a_codes.device)
    code = B.MXQ_OUT_BF16 if out_dtype == torch.bfloat16 else B.MXQ_OUT_F32
    B.mxq_nvfp4_grouped_gemm(a_codes, a_block_scales, a_scales, b_codes, b_block_scales, b_scales,
                             seg_offsets, G, R, N, K, code, c, stream)
    return c


def nvfp4_gemm(a_codes, a_block_scales, a_scales, b_codes, b_block_scales, b_scales,
               rows_per_a_scale: int = 1, rows_per_b_scale: Optional[int] = None,
               out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    """C = A x B^T on NVFP4 operands (a [M][K/2], b [N][K/2], E4M3 block
    scales per 16, FP32 scales per rows_per_*_scale rows; by default one per
    token of A and one for all of B)."""
    M, half = a_codes.shape
    N, K = b_codes.shape[0], 2 * half
    rpb = N if rows_per_b_scale is None else rows_per_b_scale
    c = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    code = B.MXQ_OUT_BF16 if out_dtype == torch.bfloat16 else B.MXQ_OUT_F32
    B.mxq_nvfp4_gemm(a_codes, a_block_scales, a_scales, rows_per_a_scale, b_codes,
                     b_block_scales, b_scales, rpb, M, N, K, code, c, stream)
    return c


class GroupedMXFP8(NamedTuple):
    row_codes: torch.Tensor
    row_scales: torch.Tensor
    col_codes: torch.Tensor
    col_scales: torch.Tensor          # capacity rows; the first P[G] are written
    col_scale_offsets: torch.Tensor


def grouped_quantize_mxfp8(x, seg_offsets, stream=None) -> GroupedMXFP8:
    x = _bf16_bits(x)
    R, cols = x.shape
    G = seg_offsets.numel() - 1
    u8 = torch.uint8
    out = GroupedMXFP8(_empty((R, cols), u8, x), _empty((R, cols // 32), u8, x),
                       _empty((R, cols), u8, x), _empty((R // 32 + G, cols), u8, x),
                       _empty((G + 1,), torch.int64, x))
    B.mxq_grouped_quantize(B.MXQ_FMT_MXFP8_ROWCOL, x, R, cols, seg_offsets, G,
                           out._asdict(), stream)
    return out


def grouped_quantize_nvfp4(x, seg_offsets, stream=None) -> NVFP4:
    x = _bf16_bits(x)
    R, cols = x.shape
    G = seg_offsets.numel() - 1
    res = NVFP4(_empty((R, cols // 2), torch.uint8, x), _empty((R, cols // 16), torch.uint8, x),
                _empty((R,), torch.float32, x))
    B.mxq_grouped_quantize(B.MXQ_FMT_NVFP4, x, R, cols, seg_offsets, G,
                           {"codes": res.codes, "block_scales": res.block_scales,
                            "token_scales": res.fp32_scales}, stream)
    return res


def dispatch_quantize_mxfp8(tokens, row_tokens, seg_offsets, stream=None) -> GroupedMXFP8:
    """Grouped MXFP8 row+col of the expert-sorted rows tokens[row_tokens[r]],
    read straight from the unpermuted tokens."""
    tokens = _bf16_bits(tokens)
    T, cols = tokens.shape
    R = row_tokens.numel()
    G = seg_offsets.numel() - 1
    u8 = torch.uint8
    out = GroupedMXFP8(_empty((R, cols), u8, tokens), _empty((R, cols // 32), u8, tokens),
                       _empty((R, cols), u8, tokens), _empty((R // 32 + G, cols), u8, tokens),
                       _empty((G + 1,), torch.int64, tokens))
    B.mxq_grouped_quantize_dispatch(B.MXQ_FMT_MXFP8_ROWCOL, tokens, T, cols, 0, None,
                                    row_tokens, R, seg_offsets, G, out._asdict(), stream)
    return out


def dispatch_quantize_nvfp4(tokens, token_rows, total_rows, stream=None) -> NVFP4:
    """Per-token NVFP4 of every token, written to its rows token_rows[t][c]
    of a [total_rows] expert-sorted layout."""
    tokens = _bf16_bits(tokens)
    T, cols = tokens.shape
    top_k = token_rows.shape[1]
    res = NVFP4(_empty((total_rows, cols // 2), torch.uint8, tokens),
                _empty((total_rows, cols // 16), torch.uint8, tokens),
                _empty((total_rows,), torch.float32, tokens))
    B.mxq_grouped_quantize_dispatch(B.MXQ_FMT_NVFP4, tokens, T, cols, top_k, token_rows, None,
                                    total_rows, None, 0,
                                    {"codes": res.codes, "block_scales": res.block_scales,
                                     "token_scales": res.fp32_scales}, stream)
    return res
