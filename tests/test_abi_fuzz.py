"""Host-side validation of every C-ABI entry point under random arguments
(no GPU: nothing may launch).  Sizes range over zero, negatives, small
values, ragged values and values near the documented limits; pointers are
NULL or fake addresses with random alignment.  Every call must return one
of the documented error statuses (never MXQ_OK, since no device exists,
and never crash), and the statuses that the arguments alone decide must
be the documented ones."""
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import nvfp4_block_scaled_amax_amd as mxq

BASE = 1 << 24
ERRORS = {mxq.MXQ_ERR_NULL, mxq.MXQ_ERR_SIZE, mxq.MXQ_ERR_SHAPE, mxq.MXQ_ERR_ALIGN,
          mxq.MXQ_ERR_ALIAS, mxq.MXQ_ERR_OFFSETS, mxq.MXQ_ERR_DEVICE, mxq.MXQ_ERR_ARG}

sizes = st.one_of(st.integers(-3, 3), st.integers(1, 5000),
                  st.sampled_from([16, 32, 64, 96, 128, 2048, (1 << 26) - 1, 1 << 26, 1 << 31,
                                   (1 << 62) // 3, (1 << 63) - 1, -(1 << 63)]))
ptrs = st.one_of(st.none(), st.integers(0, 64).map(lambda k: BASE * (k + 1)),
                 st.integers(1, 15).map(lambda k: BASE + k))
SETTINGS = settings(max_examples=300, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


def status(fn, *args):
    try:
        fn(*args)
    except mxq.MXQError as e:
        return e.status
    return mxq.MXQ_OK


@SETTINGS
@given(x=ptrs, rc=ptrs, rs=ptrs, cc=ptrs, cs=ptrs, rows=sizes, cols=sizes)
def test_mxfp8_rowcol(x, rc, rs, cc, cs, rows, cols):
    s = status(mxq.mxq_mxfp8_quantize_rowcol, x, rows, cols, rc, rs, cc, cs, 0)
    assert s in ERRORS
    if x is None:
        assert s == mxq.MXQ_ERR_NULL
    elif rows <= 0 or cols <= 0:
        assert s in (mxq.MXQ_ERR_SIZE, mxq.MXQ_ERR_OFFSETS)


@SETTINGS
@given(x=ptrs, c=ptrs, b=ptrs, t=ptrs, rows=sizes, cols=sizes)
def test_nvfp4_per_token(x, c, b, t, rows, cols):
    s = status(mxq.mxq_nvfp4_quantize_per_token, x, rows, cols, c, b, t, 0)
    assert s in ERRORS
    if None in (x, c, b, t):
        assert s == mxq.MXQ_ERR_NULL
    elif 0 < rows < (1 << 26) and 0 < cols < (1 << 30) and cols % 16:
        assert s == mxq.MXQ_ERR_SHAPE          # sizes in range: the shape decides


@SETTINGS
@given(g=ptrs, u=ptrs, gc=ptrs, gb=ptrs, uc=ptrs, ub=ptrs, sc=ptrs, e=sizes, rows=sizes,
       cols=sizes)
def test_export_pair(g, u, gc, gb, uc, ub, sc, e, rows, cols):
    s = status(mxq.mxq_nvfp4_quantize_gateup_pair, g, u, e, rows, cols, gc, gb, uc, ub, sc, 0)
    assert s in ERRORS


@SETTINGS
@given(fmt=st.integers(-1, 6), c=ptrs, sc=ptrs, f=ptrs, stride=st.integers(-2, 3), rows=sizes,
       cols=sizes, out=ptrs)
def test_dequant(fmt, c, sc, f, stride, rows, cols, out):
    s = status(mxq.mxq_dequantize_bf16, fmt, c, sc, f, stride, rows, cols, out, 0)
    assert s in ERRORS
    if fmt not in (mxq.MXQ_FMT_MXFP8_ROW, mxq.MXQ_FMT_MXFP8_COL, mxq.MXQ_FMT_NVFP4):
        assert s in (mxq.MXQ_ERR_ARG, mxq.MXQ_ERR_NULL)


@SETTINGS
@given(a=ptrs, sa=ptrs, b=ptrs, sb=ptrs, c=ptrs, M=sizes, N=sizes, K=sizes,
       dt=st.integers(-1, 2))
def test_mxfp8_gemm(a, sa, b, sb, c, M, N, K, dt):
    s = status(mxq.mxq_mxfp8_gemm, a, sa, b, sb, M, N, K, dt, c, 0)
    assert s in ERRORS
    if dt not in (0, 1):
        assert s == mxq.MXQ_ERR_ARG


@SETTINGS
@given(a=ptrs, sa=ptrs, b=ptrs, sb=ptrs, off=ptrs, c=ptrs, G=sizes, R=sizes, N=sizes, K=sizes,
       dt=st.integers(0, 1))
def test_grouped_gemms(a, sa, b, sb, off, c, G, R, N, K, dt):
    s = status(mxq.mxq_mxfp8_grouped_gemm, a, sa, b, sb, off, G, R, N, K, dt, c, 0)
    assert s in ERRORS
    if None in (a, sa, b, sb, off, c):
        assert s == mxq.MXQ_ERR_NULL
    s = status(mxq.mxq_nvfp4_grouped_gemm, a, sa, sb, b, sb, sa, off, G, R, N, K, dt, c, 0)
    assert s in ERRORS


@SETTINGS
@given(fmt=st.integers(-1, 6), x=ptrs, off=ptrs, rows=sizes, cols=sizes, G=sizes,
       o=st.lists(ptrs, min_size=8, max_size=8))
def test_grouped_quantize(fmt, x, off, rows, cols, G, o):
    out = {"row_codes": o[0], "row_scales": o[1], "col_codes": o[2], "col_scales": o[3],
           "col_scale_offsets": o[4], "codes": o[5], "block_scales": o[6], "token_scales": o[7]}
    s = status(mxq.mxq_grouped_quantize, fmt, x, rows, cols, off, G, out, 0)
    assert s in ERRORS


@SETTINGS
@given(x=ptrs, off=ptrs, ct=ptrs, cs=ptrs, P=ptrs, rows=sizes, cols=sizes, G=sizes, M=sizes,
       N=sizes, pitch=sizes, dt=st.integers(-1, 2))
def test_grouped_weight_gradient_pair(x, off, ct, cs, P, rows, cols, G, M, N, pitch, dt):
    s = status(mxq.mxq_mxfp8_grouped_colwise_t, x, rows, cols, off, G, ct, cs, P, 0)
    assert s in ERRORS
    s = status(mxq.mxq_mxfp8_grouped_wgrad, ct, cs, x, cs, P, G, M, N, pitch, dt, off, 0)
    assert s in ERRORS
    s = status(mxq.mxq_mxfp8_grouped_quantize_rowcol_t, x, rows, cols, off, G, ct, cs, ct, cs,
               P, 0)
    assert s in ERRORS


@SETTINGS
@given(src=ptrs, dst=ptrs, nr=sizes, nw=sizes)
def test_copy_floor(src, dst, nr, nw):
    s = status(mxq.mxq_copy_floor, src, nr, dst, nw, 0)
    assert s in ERRORS
