"""MI355X-native bit-exact block-scaled quantizers: MXFP8 (rowwise 1x32 and
columnwise 32x1 copies, E8M0 scales) and NVFP4 (E2M1 codes, E4M3 block scales,
per-token or per-scope FP32 scales), with BF16 dequant and grouped (ragged MoE
segment) variants.  The compute runs in hand-written HIP kernels for gfx950
behind the C ABI in include/mxq.h (libmxq.so); this package is its ctypes
binding.  Allocation helpers live in `nvfp4_block_scaled_amax_amd.api`
(imports torch)."""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, MXQ_ERR_ALIAS, MXQ_ERR_ALIGN, MXQ_ERR_ARG, MXQ_ERR_DEVICE,
    MXQ_ERR_LAUNCH, MXQ_ERR_NULL, MXQ_ERR_OFFSETS, MXQ_ERR_SHAPE, MXQ_ERR_SIZE,
    MXQ_FMT_MXFP8_COL, MXQ_FMT_MXFP8_ROW, MXQ_FMT_MXFP8_ROWCOL, MXQ_FMT_NVFP4, MXQ_OK,
    MXQ_OUT_BF16, MXQ_OUT_F32, mxq_mxfp8_gemm, mxq_mxfp8_grouped_gemm, mxq_nvfp4_gemm,
    mxq_nvfp4_grouped_gemm, mxq_mxfp8_grouped_colwise_t, mxq_mxfp8_grouped_wgrad,
    mxq_mxfp8_grouped_quantize_rowcol_t,
    mxq_mxfp8_quantize_ocp_floor,
    mxq_mxfp8_quantize_rowcol_t, mxq_nvfp4_quantize_per_token_approx,
    MXQError, lib, mxq_dequantize_bf16, mxq_grouped_out, mxq_grouped_quantize,
    mxq_grouped_quantize_dispatch, mxq_copy_floor,
    mxq_mxfp8_quantize_rowcol, mxq_nvfp4_quantize_gateup_pair, mxq_nvfp4_quantize_per_token,
    mxq_nvfp4_quantize_gateup_pair_amax,
    mxq_quantize_dequant_bf16, mxq_status_string, mxq_version)
