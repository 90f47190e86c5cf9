"""The C-ABI library without a GPU: it loads, exports every symbol that
include/mxq.h declares, and its host-side validation rejects bad arguments
before any device call.  No kernel runs here."""
import os
import re

import pytest

import nvfp4_block_scaled_amax_amd as mxq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "mxq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", text)))


def test_library_builds_and_loads():
    if not os.path.exists(mxq.LIB_PATH):
        pytest.skip("libmxq.so not built")
    L = mxq.lib()
    assert L is not None


def test_exports_every_declared_symbol():
    L = mxq.lib()
    decl = declared_functions()
    assert set(decl) == set(mxq.EXPORTS), decl
    for name in decl:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    text = open(HEADER).read()
    v = int(re.search(r"#define MXQ_VERSION (\d+)", text).group(1))
    assert mxq.mxq_version() == v
    msgs = [mxq.mxq_status_string(s) for s in range(10)]
    assert len(set(msgs)) == 10
    assert mxq.mxq_status_string(12345) == "unknown status"


A = 1 << 20          # a fake 16-byte-aligned address; never dereferenced


def status_of(fn, *args):
    with pytest.raises(mxq.MXQError) as ei:
        fn(*args)
    return ei.value.status


def test_validation_before_any_device_call():
    q = mxq.mxq_mxfp8_quantize_rowcol
    assert status_of(q, None, 32, 32, A, A, A, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(q, A, 32, 32, A, None, A, A, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(q, A, 32, 32, None, None, None, None, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(q, A, 0, 32, A, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(q, A, -32, 32, A, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(q, A, 1 << 40, 1 << 40, A, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(q, A, 32, 48, A, A, A, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(q, A, 48, 32, A, A, A, A, 0) == mxq.MXQ_ERR_SHAPE      # colwise needs rows % 32
    assert status_of(q, A + 2, 32, 32, A, A, A, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(q, A, 32, 32, A + 8, A, A, A, 0) == mxq.MXQ_ERR_ALIGN

    n = mxq.mxq_nvfp4_quantize_per_token
    assert status_of(n, A, 4, 16, A, A, None, 0) == mxq.MXQ_ERR_NULL
    assert status_of(n, A, 4, 24, A, A, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(n, A, 4, 16, A, A, A + 2, 0) == mxq.MXQ_ERR_ALIGN

    p = mxq.mxq_nvfp4_quantize_gateup_pair
    assert status_of(p, A, A, 2, 4, 16, A, A, None, A, A, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(p, A, None, 2, 4, 16, A, A, A, None, A, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(p, A, A, 0, 4, 16, A, A, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(p, A, A, 2, 4, 8, A, A, A, A, A, 0) == mxq.MXQ_ERR_SHAPE

    pa = mxq.mxq_nvfp4_quantize_gateup_pair_amax
    assert status_of(pa, A, A, None, 2, 4, 16, A, A, A, A, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(pa, A, A, A, 2, 4, 16, A, A, None, A, A, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(pa, A, None, A, 2, 4, 16, A, A, A, None, A, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(pa, A, A, A, 0, 4, 16, A, A, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(pa, A, None, A, 1 << 26, 1, 16, A, A, None, None, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(pa, A, A, A, 2, 4, 8, A, A, A, A, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(pa, A, A, A + 1, 2, 4, 16, A, A, A, A, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(pa, A, A, A, 2, 4, 16, A + 8, A, A, A, A, 0) == mxq.MXQ_ERR_ALIGN

    d = mxq.mxq_dequantize_bf16
    assert status_of(d, 0, A, A, None, 0, 32, 32, A, 0) == mxq.MXQ_ERR_ARG
    assert status_of(d, mxq.MXQ_FMT_NVFP4, A, A, None, 1, 32, 32, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(d, mxq.MXQ_FMT_NVFP4, A, A, A, 0, 32, 32, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(d, mxq.MXQ_FMT_MXFP8_COL, A, A, None, 0, 48, 32, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(d, mxq.MXQ_FMT_MXFP8_ROW, A, A, None, 0, 32, 16, A, 0) == mxq.MXQ_ERR_SHAPE

    g = mxq.mxq_grouped_quantize
    out8 = {"row_codes": A, "row_scales": A, "col_codes": A, "col_scales": A,
            "col_scale_offsets": A}
    assert status_of(g, 5, A, 64, 32, A, 2, out8, 0) == mxq.MXQ_ERR_ARG
    assert status_of(g, mxq.MXQ_FMT_MXFP8_ROWCOL, A, 64, 32, A, 0, out8, 0) == mxq.MXQ_ERR_SIZE
    bad = dict(out8, col_scale_offsets=None)
    assert status_of(g, mxq.MXQ_FMT_MXFP8_ROWCOL, A, 64, 32, A, 2, bad, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(g, mxq.MXQ_FMT_NVFP4, A, 64, 32, A, 2, {"codes": A}, 0) == mxq.MXQ_ERR_NULL

    qd = mxq.mxq_quantize_dequant_bf16
    R = mxq.MXQ_FMT_MXFP8_ROW
    assert status_of(qd, mxq.MXQ_FMT_MXFP8_COL, A, 32, 32, A, A, None, A, 0) == mxq.MXQ_ERR_ARG
    assert status_of(qd, R, A, 32, 32, A, A, None, None, 0) == mxq.MXQ_ERR_NULL
    assert status_of(qd, R, A, 32, 32, A, None, None, A, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(qd, R, A, 32, 32, A, A, A, A, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(qd, R, A, 32, 48, A, A, None, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(qd, R, A, 0, 32, A, A, None, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(qd, R, A, 32, 32, A, A, None, A + 8, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(qd, F4 := mxq.MXQ_FMT_NVFP4, A, 4, 24, A, A, A, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(qd, F4, A, 1 << 31, 16, A, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(qd, F4, A, 4, 16, A + 4, A, A, A, 0) == mxq.MXQ_ERR_ALIGN

    gm = mxq.mxq_mxfp8_gemm
    assert status_of(gm, A, A, A, A, 64, 64, 128, 7, A, 0) == mxq.MXQ_ERR_ARG
    assert status_of(gm, A, None, A, A, 64, 64, 128, 0, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(gm, A, A, A, A, 64, 64, 96, 0, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(gm, A, A, A, A, 0, 64, 128, 0, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(gm, A, A, A, A, 64, 64, 1 << 24, 0, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(gm, A + 8, A, A, A, 64, 64, 128, 0, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(gm, A, A + 2, A, A, 64, 64, 128, 0, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(gm, A, A, A, A, 64, 64, 128, 0, A + 2, 0) == mxq.MXQ_ERR_ALIGN

    gg = mxq.mxq_mxfp8_grouped_gemm
    assert status_of(gg, A, A, A, A, A, 2, 64, 64, 128, 7, A, 0) == mxq.MXQ_ERR_ARG
    assert status_of(gg, A, A, A, A, None, 2, 64, 64, 128, 0, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(gg, A, A, A, A, A, 0, 64, 64, 128, 0, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(gg, A, A, A, A, A, 2, 0, 64, 128, 0, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(gg, A, A, A, A, A, 2, 64, 64, 96, 0, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(gg, A, A, A, A, A, 2, 64, 64, 1 << 24, 0, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(gg, A + 8, A, A, A, A, 2, 64, 64, 128, 0, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(gg, A, A, A, A, A + 4, 2, 64, 64, 128, 0, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(gg, A, A, A, A, A, 2, 64, 64, 128, 1, A + 1, 0) == mxq.MXQ_ERR_ALIGN

    gn = mxq.mxq_nvfp4_grouped_gemm
    assert status_of(gn, A, A, A, A, A, A, A, 2, 64, 64, 64, 7, A, 0) == mxq.MXQ_ERR_ARG
    assert status_of(gn, A, A, None, A, A, A, A, 2, 64, 64, 64, 0, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(gn, A, A, A, A, A, A, A, 0, 64, 64, 64, 0, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(gn, A, A, A, A, A, A, A, 2, 64, 64, 96, 0, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(gn, A + 8, A, A, A, A, A, A, 2, 64, 64, 64, 0, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(gn, A, A + 2, A, A, A, A, A, 2, 64, 64, 64, 0, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(gn, A, A, A, A, A, A, A + 4, 2, 64, 64, 64, 0, A, 0) == mxq.MXQ_ERR_ALIGN

    ct = mxq.mxq_mxfp8_grouped_colwise_t
    assert status_of(ct, A, 64, 64, A, 2, A, A, None, 0) == mxq.MXQ_ERR_NULL
    assert status_of(ct, A, 64, 64, A, 0, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(ct, A, 64, 48, A, 2, A, A, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(ct, A, 0, 64, A, 2, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(ct, A, 64, 64, A, (1 << 40) + 1, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(ct, A + 8, 64, 64, A, 2, A, A, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(ct, A, 64, 64, A, 2, A, A + 2, A, 0) == mxq.MXQ_ERR_ALIGN
    rt = mxq.mxq_mxfp8_grouped_quantize_rowcol_t
    assert status_of(rt, A, 64, 64, A, 2, None, A, A, A, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(rt, A, 64, 64, A, 2, A, None, A, A, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(rt, A, 64, 64, A, 0, A, A, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(rt, A, 64, 48, A, 2, A, A, A, A, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(rt, A, 64, 64, A, 2, A + 8, A, A, A, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(rt, A, 64, 64, A, 2, A, A, A, A + 2, A, 0) == mxq.MXQ_ERR_ALIGN
    wg = mxq.mxq_mxfp8_grouped_wgrad
    assert status_of(wg, A, A, A, A, A, 2, 64, 64, 256, 9, A, 0) == mxq.MXQ_ERR_ARG
    assert status_of(wg, A, A, A, A, None, 2, 64, 64, 256, 0, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(wg, A, A, A, A, A, 2, 64, 64, 192, 0, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(wg, A, A, A, A, A, 2, 64, 64, 1 << 24, 0, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(wg, A, A, A, A, A, 0, 64, 64, 256, 0, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(wg, A, A + 2, A, A, A, 2, 64, 64, 256, 0, A, 0) == mxq.MXQ_ERR_ALIGN

    ng = mxq.mxq_nvfp4_gemm
    assert status_of(ng, A, A, A, 1, A, A, A, 64, 64, 64, 64, 5, A, 0) == mxq.MXQ_ERR_ARG
    assert status_of(ng, A, A, None, 1, A, A, A, 64, 64, 64, 64, 0, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(ng, A, A, A, 0, A, A, A, 64, 64, 64, 64, 0, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(ng, A, A, A, 1, A, A, A, 64, 64, 64, 96, 0, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(ng, A + 4, A, A, 1, A, A, A, 64, 64, 64, 64, 0, A, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(ng, A, A + 2, A, 1, A, A, A, 64, 64, 64, 64, 0, A, 0) == mxq.MXQ_ERR_ALIGN

    oq = mxq.mxq_mxfp8_quantize_ocp_floor
    assert status_of(oq, None, 32, 32, A, A, A, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(oq, A, 32, 32, A, None, A, A, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(oq, A, 48, 32, A, A, A, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(oq, A + 2, 32, 32, A, A, A, A, 0) == mxq.MXQ_ERR_ALIGN

    ct = mxq.mxq_mxfp8_quantize_rowcol_t
    assert status_of(ct, A, 32, 32, A, A, None, A, 0) == mxq.MXQ_ERR_NULL
    assert status_of(ct, A, 32, 32, A, None, A, A, 0) == mxq.MXQ_ERR_OFFSETS
    assert status_of(ct, A, 48, 32, None, None, A, A, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(ct, A, 32, 32, None, None, A + 8, A, 0) == mxq.MXQ_ERR_ALIGN

    ap = mxq.mxq_nvfp4_quantize_per_token_approx
    assert status_of(ap, A, 4, 16, A, A, None, 0) == mxq.MXQ_ERR_NULL
    assert status_of(ap, A, 4, 8192, A, A, A, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(ap, A, 4, 24, A, A, A, 0) == mxq.MXQ_ERR_SHAPE

    gd = mxq.mxq_grouped_quantize_dispatch
    nv = {"codes": A, "block_scales": A, "token_scales": A}
    F4, F8 = mxq.MXQ_FMT_NVFP4, mxq.MXQ_FMT_MXFP8_ROWCOL
    assert status_of(gd, mxq.MXQ_FMT_MXFP8_ROW, A, 8, 32, 1, A, A, 8, A, 1, out8, 0) == \
        mxq.MXQ_ERR_ARG
    assert status_of(gd, F4, A, 8, 32, 2, None, None, 16, None, 0, nv, 0) == mxq.MXQ_ERR_NULL
    assert status_of(gd, F4, A, 8, 32, 0, A, None, 16, None, 0, nv, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(gd, F4, A, 8, 24, 2, A, None, 16, None, 0, nv, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(gd, F4, A, -1, 32, 2, A, None, 16, None, 0, nv, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(gd, F4, A, 8, 32, 2, A + 4, None, 16, None, 0, nv, 0) == mxq.MXQ_ERR_ALIGN
    assert status_of(gd, F8, A, 8, 32, 0, None, None, 16, A, 1, out8, 0) == mxq.MXQ_ERR_NULL
    assert status_of(gd, F8, A, 8, 32, 0, None, A, 16, None, 1, out8, 0) == mxq.MXQ_ERR_NULL
    assert status_of(gd, F8, A, 8, 32, 0, None, A, 16, A, 0, out8, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(gd, F8, A, 8, 48, 0, None, A, 16, A, 1, out8, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(gd, F8, A, 8, 32, 0, None, A, 16, A, 1, bad, 0) == mxq.MXQ_ERR_OFFSETS
    row_only = {"row_codes": A, "row_scales": A}
    assert status_of(gd, F8, A, 8, 32, 0, None, A + 4, 16, None, 0, row_only, 0) == \
        mxq.MXQ_ERR_ALIGN


def test_grid_limits_are_size_errors():
    """Sizes whose launch would exceed one grid's 2^32 - 1 work-items are
    MXQ_ERR_SIZE before any device call; one below each limit passes the size
    checks and fails only at the device-memory check (the pointers are fake)."""
    B1, B2, B3, B4, B5 = (A * k for k in (2, 3, 4, 5, 6))
    n = mxq.mxq_nvfp4_quantize_per_token
    assert status_of(n, A, 1 << 26, 16, B1, B2, B3, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(n, A, (1 << 26) - 1, 16, B1, B2, B3, 0) == mxq.MXQ_ERR_DEVICE
    qd = mxq.mxq_quantize_dequant_bf16
    assert status_of(qd, mxq.MXQ_FMT_NVFP4, A, 1 << 26, 16, B1, B2, B3, B4, 0) == \
        mxq.MXQ_ERR_SIZE
    # MXFP8 tiles: ceil(rows/32) * ceil(cols/128) <= 2^26 - 9.
    q = mxq.mxq_mxfp8_quantize_rowcol
    top = (1 << 26) - 9
    assert status_of(q, A, 32 * (top + 1), 128, B1, B2, B3, B4, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(q, A, 32 * top, 128, B1, B2, B3, B4, 0) == mxq.MXQ_ERR_DEVICE
    assert status_of(q, A, 32 * ((top + 1) // 2 + 1), 256, B1, B2, None, None, 0) == \
        mxq.MXQ_ERR_SIZE
    ct = mxq.mxq_mxfp8_quantize_rowcol_t
    assert status_of(ct, A, 32 * (top + 1), 128, None, None, B3, B4, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(qd, mxq.MXQ_FMT_MXFP8_ROW, A, 32 * (top + 1), 128, B1, B2, None, B3, 0) \
        == mxq.MXQ_ERR_SIZE
    g = mxq.mxq_grouped_quantize
    out8 = {"row_codes": B1, "row_scales": B2, "col_codes": B3, "col_scales": B4,
            "col_scale_offsets": B5}
    # row tiles with a columnwise copy: total_rows / 32 + n_groups
    assert status_of(g, mxq.MXQ_FMT_MXFP8_ROWCOL, A, 32 * (top - 9), 128, A * 7, 10, out8, 0) \
        == mxq.MXQ_ERR_SIZE
    assert status_of(g, mxq.MXQ_FMT_MXFP8_ROWCOL, A, 32 * (top - 9), 128, A * 7, 9, out8, 0) \
        == mxq.MXQ_ERR_DEVICE
    assert status_of(g, mxq.MXQ_FMT_NVFP4, A, 1 << 26, 16, A * 7, 2,
                     {"codes": B1, "block_scales": B2, "token_scales": B3}, 0) == \
        mxq.MXQ_ERR_SIZE
    gd = mxq.mxq_grouped_quantize_dispatch
    assert status_of(gd, mxq.MXQ_FMT_NVFP4, A, 1 << 26, 16, 1, A * 7, None, 1 << 26, None, 0,
                     {"codes": B1, "block_scales": B2, "token_scales": B3}, 0) == \
        mxq.MXQ_ERR_SIZE
    # GEMM tiles: ceil(M/256) * ceil(N/256) <= 2^24 - 9.
    gm = mxq.mxq_mxfp8_gemm
    assert status_of(gm, A, B1, B2, B3, 256 * ((1 << 24) - 8), 256, 128, 0, B4, 0) == \
        mxq.MXQ_ERR_SIZE
    assert status_of(gm, A, B1, B2, B3, 256 * ((1 << 24) - 9), 256, 128, 0, B4, 0) == \
        mxq.MXQ_ERR_DEVICE
    ng = mxq.mxq_nvfp4_gemm
    assert status_of(ng, A, B1, B2, 1, B3, B4, B5, 1, 256 * ((1 << 24) - 8), 256, 64, 0,
                     A * 7, 0) == mxq.MXQ_ERR_SIZE
    gn = mxq.mxq_nvfp4_grouped_gemm
    assert status_of(gn, A, B1, B2, B3, B4, B5, A * 7, 1, 256 * ((1 << 24) - 9), 256, 64, 0,
                     A * 11, 0) == mxq.MXQ_ERR_SIZE
    # Grouped GEMM: (ceil(R/256) + n_groups) * ceil(N/256) <= 2^24 - 9.
    gg = mxq.mxq_mxfp8_grouped_gemm
    assert status_of(gg, A, B1, B2, B3, B4, 1, 256 * ((1 << 24) - 9), 256, 128, 0, B5, 0) == \
        mxq.MXQ_ERR_SIZE
    assert status_of(gg, A, B1, B2, B3, B4, 1, 256 * ((1 << 24) - 10), 256, 128, 0, B5, 0) == \
        mxq.MXQ_ERR_DEVICE
    # Export: n_experts < 2^26 (with fewer than 2^36 elements this also keeps
    # the amax pass's ceil(scope / 4096) * n_experts chunks below 2^26).
    p = mxq.mxq_nvfp4_quantize_gateup_pair
    assert status_of(p, A, None, 1 << 26, 1, 16, B1, B2, None, None, B3, 0) == \
        mxq.MXQ_ERR_SIZE
    assert status_of(p, A, None, (1 << 26) - 1, 1, 16, B1, B2, None, None, B3, 0) == \
        mxq.MXQ_ERR_DEVICE


def test_copy_floor_validation():
    cf = mxq.mxq_copy_floor
    assert status_of(cf, None, 16, A, 16, 0) == mxq.MXQ_ERR_NULL
    assert status_of(cf, A, 0, A * 2, 16, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(cf, A, 16, A * 2, (1 << 35) + 16, 0) == mxq.MXQ_ERR_SIZE
    assert status_of(cf, A, 24, A * 2, 16, 0) == mxq.MXQ_ERR_SHAPE
    assert status_of(cf, A + 8, 16, A * 2, 16, 0) == mxq.MXQ_ERR_ALIGN


def test_fake_device_pointers_rejected_without_gpu():
    """Well-formed arguments that are not device memory fail host-side."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("covered by the GPU error-path tests")
    st = status_of(mxq.mxq_mxfp8_quantize_rowcol, A, 32, 32, A * 2, A * 3, A * 4, A * 5, 0)
    assert st == mxq.MXQ_ERR_DEVICE
