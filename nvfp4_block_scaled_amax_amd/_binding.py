"""ctypes binding of libmxq.so: one Python function per C entry point, with the
same name and argument order as include/mxq.h.

Array arguments may be torch tensors (their data_ptr() is passed), plain
integer addresses, or None for NULL.  `stream` may be None (torch's current
stream on the current device), a torch.cuda.Stream, or an integer hipStream_t.
A status other than MXQ_OK raises MXQError.  This module only marshals
arguments; every step runs in the library's kernels, and a missing library
raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# MXQ_LIB_PATH selects another build of the same library (the host-sanitizer
# test loads a build instrumented with AddressSanitizer and UBSan).
LIB_PATH = os.environ.get("MXQ_LIB_PATH") or os.path.join(HERE, "libmxq.so")

MXQ_OK = 0
MXQ_ERR_NULL = 1
MXQ_ERR_SIZE = 2
MXQ_ERR_SHAPE = 3
MXQ_ERR_ALIGN = 4
MXQ_ERR_ALIAS = 5
MXQ_ERR_OFFSETS = 6
MXQ_ERR_DEVICE = 7
MXQ_ERR_LAUNCH = 8
MXQ_ERR_ARG = 9

MXQ_FMT_MXFP8_ROW = 1
MXQ_FMT_MXFP8_COL = 2
MXQ_FMT_MXFP8_ROWCOL = 3
MXQ_FMT_NVFP4 = 4
MXQ_OUT_F32 = 0
MXQ_OUT_BF16 = 1

# Every symbol include/mxq.h declares.
EXPORTS = (
    "mxq_mxfp8_quantize_rowcol",
    "mxq_nvfp4_quantize_per_token",
    "mxq_nvfp4_quantize_gateup_pair",
    "mxq_nvfp4_quantize_gateup_pair_amax",
    "mxq_dequantize_bf16",
    "mxq_quantize_dequant_bf16",
    "mxq_mxfp8_gemm",
    "mxq_mxfp8_grouped_gemm",
    "mxq_mxfp8_grouped_colwise_t",
    "mxq_mxfp8_grouped_quantize_rowcol_t",
    "mxq_mxfp8_grouped_wgrad",
    "mxq_nvfp4_gemm",
    "mxq_nvfp4_grouped_gemm",
    "mxq_mxfp8_quantize_ocp_floor",
    "mxq_mxfp8_quantize_rowcol_t",
    "mxq_nvfp4_quantize_per_token_approx",
    "mxq_grouped_quantize",
    "mxq_grouped_quantize_dispatch",
    "mxq_copy_floor",
    "mxq_status_string",
    "mxq_version",
)


class MXQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {mxq_status_string(status)}")


class mxq_grouped_out(ctypes.Structure):
    _fields_ = [("row_codes", ctypes.c_void_p), ("row_scales", ctypes.c_void_p),
                ("col_codes", ctypes.c_void_p), ("col_scales", ctypes.c_void_p),
                ("col_scale_offsets", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("block_scales", ctypes.c_void_p), ("token_scales", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libmxq.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmxq.so is not built ({LIB_PATH}); run "
                           "`python -m nvfp4_block_scaled_amax_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sigs = {
        "mxq_mxfp8_quantize_rowcol": [P, I64, I64, P, P, P, P, P],
        "mxq_nvfp4_quantize_per_token": [P, I64, I64, P, P, P, P],
        "mxq_nvfp4_quantize_gateup_pair": [P, P, I64, I64, I64, P, P, P, P, P, P],
        "mxq_nvfp4_quantize_gateup_pair_amax": [P, P, P, I64, I64, I64, P, P, P, P, P, P],
        "mxq_dequantize_bf16": [I, P, P, P, I64, I64, I64, P, P],
        "mxq_quantize_dequant_bf16": [I, P, I64, I64, P, P, P, P, P],
        "mxq_mxfp8_gemm": [P, P, P, P, I64, I64, I64, I, P, P],
        "mxq_mxfp8_grouped_gemm": [P, P, P, P, P, I64, I64, I64, I64, I, P, P],
        "mxq_mxfp8_grouped_colwise_t": [P, I64, I64, P, I64, P, P, P, P],
        "mxq_mxfp8_grouped_quantize_rowcol_t": [P, I64, I64, P, I64, P, P, P, P, P, P],
        "mxq_mxfp8_grouped_wgrad": [P, P, P, P, P, I64, I64, I64, I64, I, P, P],
        "mxq_nvfp4_grouped_gemm": [P, P, P, P, P, P, P, I64, I64, I64, I64, I, P, P],
        "mxq_nvfp4_gemm": [P, P, P, I64, P, P, P, I64, I64, I64, I64, I, P, P],
        "mxq_mxfp8_quantize_ocp_floor": [P, I64, I64, P, P, P, P, P],
        "mxq_mxfp8_quantize_rowcol_t": [P, I64, I64, P, P, P, P, P],
        "mxq_nvfp4_quantize_per_token_approx": [P, I64, I64, P, P, P, P],
        "mxq_grouped_quantize": [I, P, I64, I64, P, I64, ctypes.POINTER(mxq_grouped_out), P],
        "mxq_grouped_quantize_dispatch": [I, P, I64, I64, I64, P, P, I64, P, I64,
                                          ctypes.POINTER(mxq_grouped_out), P],
        "mxq_copy_floor": [P, I64, P, I64, P],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = I
    L.mxq_status_string.argtypes = [I]
    L.mxq_status_string.restype = ctypes.c_char_p
    L.mxq_version.argtypes = []
    L.mxq_version.restype = I
    _lib = L
    return L


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _current_stream_handle():
    """The raw handle of torch's current stream on the current device: the
    same value as torch.cuda.current_stream().cuda_stream, without building a
    Stream object (0.1 against 2.8 us per call, which matters for back-to-back
    launches of kernels of a few us).  Falls back to the public call on torch
    builds without the raw accessor."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is None:
        return torch.cuda.current_stream().cuda_stream
    return raw(torch.cuda.current_device())


def _stream(stream):
    if stream is None:
        return _current_stream_handle()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != MXQ_OK:
        raise MXQError(status, where)


def mxq_status_string(status: int) -> str:
    return lib().mxq_status_string(status).decode()


def mxq_version() -> int:
    return lib().mxq_version()


def mxq_mxfp8_quantize_rowcol(x, rows, cols, row_codes, row_scales, col_codes, col_scales,
                              stream=None):
    _check(lib().mxq_mxfp8_quantize_rowcol(_ptr(x), rows, cols, _ptr(row_codes),
                                           _ptr(row_scales), _ptr(col_codes), _ptr(col_scales),
                                           _stream(stream)),
           "mxq_mxfp8_quantize_rowcol")


def mxq_mxfp8_quantize_ocp_floor(x, rows, cols, row_codes, row_scales, col_codes, col_scales,
                                 stream=None):
    _check(lib().mxq_mxfp8_quantize_ocp_floor(_ptr(x), rows, cols, _ptr(row_codes),
                                              _ptr(row_scales), _ptr(col_codes),
                                              _ptr(col_scales), _stream(stream)),
           "mxq_mxfp8_quantize_ocp_floor")


def mxq_mxfp8_quantize_rowcol_t(x, rows, cols, row_codes, row_scales, col_codes_t, col_scales_t,
                                stream=None):
    _check(lib().mxq_mxfp8_quantize_rowcol_t(_ptr(x), rows, cols, _ptr(row_codes),
                                             _ptr(row_scales), _ptr(col_codes_t),
                                             _ptr(col_scales_t), _stream(stream)),
           "mxq_mxfp8_quantize_rowcol_t")


def mxq_nvfp4_quantize_per_token(x, rows, cols, codes, block_scales, token_scales, stream=None):
    _check(lib().mxq_nvfp4_quantize_per_token(_ptr(x), rows, cols, _ptr(codes),
                                              _ptr(block_scales), _ptr(token_scales),
                                              _stream(stream)),
           "mxq_nvfp4_quantize_per_token")


def mxq_nvfp4_quantize_per_token_approx(x, rows, cols, codes, block_scales, token_scales,
                                        stream=None):
    _check(lib().mxq_nvfp4_quantize_per_token_approx(_ptr(x), rows, cols, _ptr(codes),
                                                     _ptr(block_scales), _ptr(token_scales),
                                                     _stream(stream)),
           "mxq_nvfp4_quantize_per_token_approx")


def mxq_nvfp4_quantize_gateup_pair(gate, up, n_experts, rows, cols, gate_codes,
                                   gate_block_scales, up_codes, up_block_scales, scope_scales,
                                   stream=None):
    _check(lib().mxq_nvfp4_quantize_gateup_pair(_ptr(gate), _ptr(up), n_experts, rows, cols,
                                                _ptr(gate_codes), _ptr(gate_block_scales),
                                                _ptr(up_codes), _ptr(up_block_scales),
                                                _ptr(scope_scales), _stream(stream)),
           "mxq_nvfp4_quantize_gateup_pair")


def mxq_nvfp4_quantize_gateup_pair_amax(gate, up, scope_amax, n_experts, rows, cols, gate_codes,
                                        gate_block_scales, up_codes, up_block_scales,
                                        scope_scales, stream=None):
    _check(lib().mxq_nvfp4_quantize_gateup_pair_amax(_ptr(gate), _ptr(up), _ptr(scope_amax),
                                                     n_experts, rows, cols, _ptr(gate_codes),
                                                     _ptr(gate_block_scales), _ptr(up_codes),
                                                     _ptr(up_block_scales), _ptr(scope_scales),
                                                     _stream(stream)),
           "mxq_nvfp4_quantize_gateup_pair_amax")


def mxq_dequantize_bf16(fmt, codes, scales, fp32_scales, rows_per_fp32_scale, rows, cols, out,
                        stream=None):
    _check(lib().mxq_dequantize_bf16(fmt, _ptr(codes), _ptr(scales), _ptr(fp32_scales),
                                     rows_per_fp32_scale, rows, cols, _ptr(out), _stream(stream)),
           "mxq_dequantize_bf16")


def mxq_quantize_dequant_bf16(fmt, x, rows, cols, codes, scales, token_scales, out, stream=None):
    _check(lib().mxq_quantize_dequant_bf16(fmt, _ptr(x), rows, cols, _ptr(codes), _ptr(scales),
                                           _ptr(token_scales), _ptr(out), _stream(stream)),
           "mxq_quantize_dequant_bf16")


def mxq_mxfp8_gemm(a, a_scales, b, b_scales, M, N, K, out_dtype, c, stream=None):
    _check(lib().mxq_mxfp8_gemm(_ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales), M, N, K,
                                out_dtype, _ptr(c), _stream(stream)),
           "mxq_mxfp8_gemm")


def mxq_mxfp8_grouped_gemm(a, a_scales, b, b_scales, seg_offsets, n_groups, total_rows, N, K,
                           out_dtype, c, stream=None):
    _check(lib().mxq_mxfp8_grouped_gemm(_ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales),
                                        _ptr(seg_offsets), n_groups, total_rows, N, K, out_dtype,
                                        _ptr(c), _stream(stream)),
           "mxq_mxfp8_grouped_gemm")


def mxq_mxfp8_grouped_colwise_t(x, total_rows, cols, seg_offsets, n_groups, codes_t, scales_t,
                                block_offsets, stream=None):
    _check(lib().mxq_mxfp8_grouped_colwise_t(_ptr(x), total_rows, cols, _ptr(seg_offsets),
                                             n_groups, _ptr(codes_t), _ptr(scales_t),
                                             _ptr(block_offsets), _stream(stream)),
           "mxq_mxfp8_grouped_colwise_t")


def mxq_mxfp8_grouped_quantize_rowcol_t(x, total_rows, cols, seg_offsets, n_groups, row_codes,
                                        row_scales, codes_t, scales_t, block_offsets,
                                        stream=None):
    _check(lib().mxq_mxfp8_grouped_quantize_rowcol_t(_ptr(x), total_rows, cols,
                                                     _ptr(seg_offsets), n_groups,
                                                     _ptr(row_codes), _ptr(row_scales),
                                                     _ptr(codes_t), _ptr(scales_t),
                                                     _ptr(block_offsets), _stream(stream)),
           "mxq_mxfp8_grouped_quantize_rowcol_t")


def mxq_mxfp8_grouped_wgrad(a, a_scales, b, b_scales, block_offsets, n_groups, M, N, pitch,
                            out_dtype, c, stream=None):
    _check(lib().mxq_mxfp8_grouped_wgrad(_ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales),
                                         _ptr(block_offsets), n_groups, M, N, pitch, out_dtype,
                                         _ptr(c), _stream(stream)),
           "mxq_mxfp8_grouped_wgrad")


def mxq_nvfp4_grouped_gemm(a, a_block_scales, a_scales, b, b_block_scales, b_scales,
                           seg_offsets, n_groups, total_rows, N, K, out_dtype, c, stream=None):
    _check(lib().mxq_nvfp4_grouped_gemm(_ptr(a), _ptr(a_block_scales), _ptr(a_scales), _ptr(b),
                                        _ptr(b_block_scales), _ptr(b_scales), _ptr(seg_offsets),
                                        n_groups, total_rows, N, K, out_dtype, _ptr(c),
                                        _stream(stream)),
           "mxq_nvfp4_grouped_gemm")


def mxq_nvfp4_gemm(a, a_block_scales, a_scales, rows_per_a_scale, b, b_block_scales, b_scales,
                   rows_per_b_scale, M, N, K, out_dtype, c, stream=None):
    _check(lib().mxq_nvfp4_gemm(_ptr(a), _ptr(a_block_scales), _ptr(a_scales), rows_per_a_scale,
                                _ptr(b), _ptr(b_block_scales), _ptr(b_scales), rows_per_b_scale,
                                M, N, K, out_dtype, _ptr(c), _stream(stream)),
           "mxq_nvfp4_gemm")


def mxq_grouped_quantize(fmt, x, total_rows, cols, seg_offsets, n_groups, out, stream=None):
    """`out`: an mxq_grouped_out, or a dict with its field names."""
    if not isinstance(out, mxq_grouped_out):
        out = mxq_grouped_out(**{k: _ptr(v) for k, v in out.items()})
    _check(lib().mxq_grouped_quantize(fmt, _ptr(x), total_rows, cols, _ptr(seg_offsets),
                                      n_groups, ctypes.byref(out), _stream(stream)),
           "mxq_grouped_quantize")


def mxq_grouped_quantize_dispatch(fmt, x, n_tokens, cols, top_k, token_rows, row_tokens,
                                  total_rows, seg_offsets, n_groups, out, stream=None):
    """`out`: an mxq_grouped_out, or a dict with its field names."""
    if not isinstance(out, mxq_grouped_out):
        out = mxq_grouped_out(**{k: _ptr(v) for k, v in out.items()})
    _check(lib().mxq_grouped_quantize_dispatch(fmt, _ptr(x), n_tokens, cols, top_k,
                                               _ptr(token_rows), _ptr(row_tokens), total_rows,
                                               _ptr(seg_offsets), n_groups, ctypes.byref(out),
                                               _stream(stream)),
           "mxq_grouped_quantize_dispatch")


def mxq_copy_floor(src, src_bytes, dst, dst_bytes, stream=None):
    _check(lib().mxq_copy_floor(_ptr(src), src_bytes, _ptr(dst), dst_bytes, _stream(stream)),
           "mxq_copy_floor")
