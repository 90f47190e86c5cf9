"""GPU parity: every output byte of the HIP path equals the CPU oracle's.

All inputs are seeded and synthetic (nvfp4_block_scaled_amax_amd.workloads, or
constructed here); expected values come only from the oracle.  The bar is
bit-exact for every code, scale byte, FP32 scale and BF16 output.  Full-size
workloads are those the benchmark times, in the same launch configuration,
and every output byte of them is compared (the GEMMs, whose parity is a bound,
compare sampled rows of C).
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amax_amd as mxq
from nvfp4_block_scaled_amax_amd import api
from nvfp4_block_scaled_amax_amd import workloads as W
from gpu_util import ExactBuffer, announce, assert_same, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# ---------------------------------------------------------------------------
# MXFP8
# ---------------------------------------------------------------------------

def check_mxfp8(orc, x: np.ndarray, name: str, rowwise=True, colwise=True):
    announce(f"mxfp8 rowcol {name} shape={x.shape} row={rowwise} col={colwise}")
    r = api.mxfp8_quantize_rowcol(dev(x), rowwise=rowwise, colwise=colwise)
    torch.cuda.synchronize()
    if rowwise:
        c, s = orc.mxfp8_rowwise(x)
        assert_same(host(r.row_scales), s, f"{name} row_scales")
        assert_same(host(r.row_codes), c, f"{name} row_codes")
    if colwise:
        c, s = orc.mxfp8_colwise(x)
        assert_same(host(r.col_scales), s, f"{name} col_scales")
        assert_same(host(r.col_codes), c, f"{name} col_codes")


def test_mxfp8_config1(orc):
    check_mxfp8(orc, W.config1(), "config1 256x512 N(0,1) seed0")


@pytest.mark.parametrize("mode", W.MXFP8_MODES)
def test_mxfp8_config2_activation(orc, mode):
    check_mxfp8(orc, W.config2_activation(mode), f"config2 act 2048x2048 {mode}")


@pytest.mark.parametrize("mode", W.MXFP8_MODES)
def test_mxfp8_config2_weight(orc, mode):
    check_mxfp8(orc, W.config2_weight(mode), f"config2 weight 8192x2048 {mode}")


@pytest.mark.parametrize("rows,cols", [(32, 32), (32, 64), (64, 96), (96, 288), (32, 2080),
                                       (160, 544), (32, 4128)])
def test_mxfp8_shapes(orc, rows, cols):
    """Column counts that leave partial wavefront and workgroup tiles."""
    x = W.mode_random(rows, cols, rows * 7 + cols)
    check_mxfp8(orc, x, f"random {rows}x{cols}")
    xb = W.mode_boundary(rows, cols, rows + cols)
    check_mxfp8(orc, xb, f"boundary {rows}x{cols}")


def test_mxfp8_large_grid(orc):
    """A dense grid above the large-launch threshold (32768 tiles: eight
    wavefronts per workgroup, rowwise codes stored as each row is converted),
    with a partial last column strip."""
    check_mxfp8(orc, W.mode_random(8192, 16416, 12), "random 8192x16416")


@pytest.mark.parametrize("rows,cols", [(288, 1024), (160, 1024), (1056, 2048), (544, 4096),
                                       (800, 1536)])
def test_mxfp8_band_order_shapes(orc, rows, cols):
    """Small dense launches take their workgroups in band order: each group of
    8 k consecutive workgroups (k per 32-row band) is permuted, a last partial
    group keeps launch order.  Shapes with a partial last group (288x1024: 18
    workgroups in groups of 16; 1056x2048: 132 in groups of 32), with no whole
    group (160x1024), with k = 8 (544x4096) and with k = 3 (800x1536, 12
    strips).  Row+col, rowwise + dequant and the OCP variant."""
    x = W.mode_boundary(rows, cols, rows + 11 * cols)
    check_mxfp8(orc, x, f"boundary {rows}x{cols}")
    check_qdq(orc, x, mxq.MXQ_FMT_MXFP8_ROW, f"{rows}x{cols}", codes_only_check=False)
    check_ocp(orc, x, f"{rows}x{cols}")


def test_mxfp8_rowwise_only_and_ragged_rows(orc):
    x = W.mode_boundary(96, 256, 3)[:77]
    check_mxfp8(orc, x, "rowwise 77x256", rowwise=True, colwise=False)
    check_mxfp8(orc, W.mode_random(64, 128, 4), "colwise-only 64x128", rowwise=False,
                colwise=True)


def _mxfp8_exhaustive_input():
    """Rows of 32: for every scale exponent e in [-127, 120], blocks led by the
    amax 448 * 2^e (BF16 max for e = 120) followed by every finite BF16 x with
    |x| <= that amax, 31 per block."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allb[(allb & 0x7F80) != 0x7F80]
    mag = W.bf16_to_f64(fin & 0x7FFF)
    rows = []
    for e in range(-127, 121):
        amax = 448.0 * 2.0 ** e
        abits = W.bf16_bits(np.array([amax]))[0] if e < 120 else np.uint16(0x7F7F)
        A = W.bf16_to_f64(np.array([abits], np.uint16))[0]
        xs = fin[mag <= A]
        n = -(-xs.size // 31)
        pad = np.zeros(n * 31, np.uint16)
        pad[:xs.size] = xs
        blk = np.empty((n, 32), np.uint16)
        blk[:, 0] = abits
        blk[:, 1:] = pad.reshape(n, 31)
        rows.append(blk)
    X = np.concatenate(rows)
    extra = (-X.shape[0]) % 32
    return np.concatenate([X, np.zeros((extra, 32), np.uint16)])


def test_mxfp8_exhaustive_code_map(orc):
    """Every finite BF16 value under every E8M0 scale its block can have, through
    both the rowwise and (transposed) columnwise kernels."""
    X = _mxfp8_exhaustive_input()
    check_mxfp8(orc, X, "exhaustive rows", rowwise=True, colwise=True)
    XT = np.ascontiguousarray(X.T)
    check_mxfp8(orc, XT, "exhaustive transposed", rowwise=True, colwise=True)


def test_binding_stream_is_torch_current_stream():
    """The binding's default stream is torch's current stream, also inside a
    stream context, and a call there is ordered on that stream."""
    from nvfp4_block_scaled_amax_amd import _binding as B
    assert B._stream(None) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    x = dev(W.config1())
    with torch.cuda.stream(s):
        assert B._stream(None) == s.cuda_stream
        r = api.mxfp8_quantize_rowcol(x)
    s.synchronize()
    ref = api.mxfp8_quantize_rowcol(x)
    torch.cuda.synchronize()
    for u, v in zip(r, ref):
        assert torch.equal(u, v)


def test_graph_capture_replays_match_eager():
    """MXFP8 row+col, per-token NVFP4 and the NVFP4 dequant captured in one
    HIP graph: every replay (with eager work and synchronisations between
    replays, and new inputs copied in) gives the eager bytes.  The calls
    launch kernels only (no memset nodes)."""
    x1 = dev(W.config2_weight("random"))
    x2 = dev(W.config3())
    a1 = torch.empty_like(x1)
    a2 = torch.empty_like(x2)
    a1.copy_(x1)
    a2.copy_(x2)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up outside the capture
        api.mxfp8_quantize_rowcol(a1)
        nv = api.nvfp4_quantize_per_token(a2)
        api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, nv.codes, nv.block_scales, nv.fp32_scales)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        r1 = api.mxfp8_quantize_rowcol(a1)
        r2 = api.nvfp4_quantize_per_token(a2)
        y2 = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, r2.codes, r2.block_scales, r2.fp32_scales)
    inputs = [(x1, x2), (dev(W.config2_weight("boundary")), dev(W.config3()[::-1].copy()))]
    for rep in range(4):
        announce(f"graph replay {rep}")
        src1, src2 = inputs[rep % 2]
        a1.copy_(src1)
        a2.copy_(src2)
        g.replay()
        torch.cuda.synchronize()
        e1 = api.mxfp8_quantize_rowcol(src1)
        e2 = api.nvfp4_quantize_per_token(src2)
        ey = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, e2.codes, e2.block_scales, e2.fp32_scales)
        torch.cuda.synchronize()
        for u, v in zip(r1, e1):
            assert torch.equal(u, v), f"replay {rep}: MXFP8"
        for u, v in zip(r2, e2):
            assert torch.equal(u, v), f"replay {rep}: NVFP4"
        assert torch.equal(y2, ey), f"replay {rep}: dequant"



def test_graph_capture_grouped_backward_pair():
    """The expert layer's backward operands and weight gradient captured in one
    HIP graph: the grouped rowwise + transposed quantize of dY and of X (the
    segment prefix formed inside the kernels) and the grouped weight-gradient
    GEMM.  Every replay, with new inputs copied in and eager calls between
    replays, gives the eager bytes."""
    sizes = [0, 1, 31, 33, 128, 200, 0, 64]
    off = dev(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64))
    R = int(sum(sizes))
    srcs = [(dev(W.student_t_activations(R, 256, 51 + k)), dev(W.mode_random(R, 192, 61 + k)))
            for k in range(2)]
    dy, x = torch.empty_like(srcs[0][0]), torch.empty_like(srcs[0][1])
    dy.copy_(srcs[0][0])
    x.copy_(srcs[0][1])
    torch.cuda.synchronize()

    def run(a, b):
        ra = api.mxfp8_grouped_quantize_rowcol_t(a, off)
        rb = api.mxfp8_grouped_quantize_rowcol_t(b, off)
        c = api.mxfp8_grouped_wgrad(ra[2], rb[2], out_dtype=torch.bfloat16)
        return ra, rb, c

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up outside the capture
        run(dy, x)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        got = run(dy, x)
    for rep in range(4):
        announce(f"graph replay (grouped backward pair) {rep}")
        sa, sb = srcs[rep % 2]
        dy.copy_(sa)
        x.copy_(sb)
        g.replay()
        torch.cuda.synchronize()
        want = run(sa, sb)
        torch.cuda.synchronize()
        for gr, wr in zip(got[:2], want[:2]):
            nb = int(wr[2].block_offsets[-1])          # columns past the padding are not written
            assert torch.equal(gr[2].block_offsets, wr[2].block_offsets), f"replay {rep}: P"
            for u, v in ((gr[0], wr[0]), (gr[1], wr[1]),
                         (gr[2].codes_t[:, :32 * nb], wr[2].codes_t[:, :32 * nb]),
                         (gr[2].scales_t[:, :nb], wr[2].scales_t[:, :nb])):
                assert torch.equal(u, v), f"replay {rep}: quantize"
        assert torch.equal(got[2].view(torch.int16), want[2].view(torch.int16)), f"replay {rep}: wgrad"

def test_mxfp8_deterministic():
    x = dev(W.config2_weight("random"))
    announce("mxfp8 determinism 8192x2048")
    a = api.mxfp8_quantize_rowcol(x)
    b = api.mxfp8_quantize_rowcol(x)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ---------------------------------------------------------------------------
# NVFP4 per token
# ---------------------------------------------------------------------------

def check_nvfp4(orc, x: np.ndarray, name: str):
    announce(f"nvfp4 per-token {name} shape={x.shape}")
    r = api.nvfp4_quantize_per_token(dev(x))
    torch.cuda.synchronize()
    c, b, s = orc.nvfp4_per_token(x)
    assert_same(host(r.fp32_scales).view(np.uint32), s.view(np.uint32), f"{name} token_scales")
    assert_same(host(r.block_scales), b, f"{name} block_scales")
    assert_same(host(r.codes), c, f"{name} codes")
    return r


def test_nvfp4_config3(orc):
    check_nvfp4(orc, W.config3(), "config3 8192x2048 t3")


@pytest.mark.parametrize("rows,cols", [(1, 16), (5, 48), (4, 512), (7, 768), (9, 1040),
                                       (6, 2048), (3, 2064), (4, 4096), (2, 4112), (2, 8192)])
def test_nvfp4_shapes(orc, rows, cols):
    """Row lengths for every register-resident chunk count, partial chunks, and
    the generic (re-reading) path above 4096."""
    check_nvfp4(orc, W.student_t_activations(rows, cols, rows + cols), f"t3 {rows}x{cols}")
    check_nvfp4(orc, W.nvfp4_boundary(rows, cols, cols), f"boundary {rows}x{cols}")


@pytest.mark.parametrize("rows,cols", [(8193, 1040), (8200, 2048), (16385, 2064), (16400, 4096)])
def test_nvfp4_shapes_one_wave_rows(orc, rows, cols):
    """Grids above the row counts that split each row over two wavefronts
    (8192 rows up to 2048 columns, 16384 up to 4096): one wavefront per row,
    full and partial rows."""
    check_nvfp4(orc, W.student_t_activations(rows, cols, rows + cols), f"t3 {rows}x{cols}")


@pytest.mark.parametrize("rows,cols", [(300, 2048), (255, 1040), (4097, 4096), (8191, 2064)])
def test_nvfp4_split_row_order(orc, rows, cols):
    """The split kernel takes rows in runs of 32 per XCD within groups of 256
    workgroups, the last partial group in launch order: row counts with a
    partial group (300, 4097, 8191) and with none whole (255), at one and two
    blocks per lane."""
    check_nvfp4(orc, W.student_t_activations(rows, cols, 5 * rows + cols), f"t3 {rows}x{cols}")
    check_qdq(orc, W.nvfp4_boundary(rows, cols, cols + 1), mxq.MXQ_FMT_NVFP4,
              f"boundary {rows}x{cols}", codes_only_check=False)


def test_nvfp4_boundary_rows(orc):
    check_nvfp4(orc, W.nvfp4_boundary(64, 2048, 17), "boundary 64x2048")
    check_nvfp4(orc, W.nvfp4_boundary(64, 64, 18), "boundary 64x64")


def _tie_sweep():
    """Rows whose FP32 scale is an exact power of two (amax 21 * 2^j), blocks
    whose scale is each E4M3 value d in turn (block amax 6 d s), and elements at
    every E2M1 midpoint and value times d s, with their BF16 neighbours: exact
    and near ties of both rounding steps."""
    e4 = [(c & 7) * 2.0 ** -9 if (c >> 3) == 0 else (8 + (c & 7)) * 2.0 ** ((c >> 3) - 10)
          for c in range(1, 127)]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rows = []
    rng = np.random.default_rng(44)
    for j in (-60, -9, 0, 7, 40, 100):
        s = 2.0 ** (j - 7)
        At = 21.0 * 2.0 ** j
        blocks = []
        for d in e4:
            q = np.array(mids + vals) * d * s
            qb = W.bf16_bits(q)
            cand = np.concatenate([qb, qb + 1, qb - 1]).astype(np.uint16)
            cand = cand[(cand & 0x7FFF) < 0x7F80]
            Ab = W.bf16_bits(np.array([6.0 * d * s]))[0]
            cand = cand[W.bf16_to_f64(cand) <= W.bf16_to_f64(np.array([Ab], np.uint16))[0]]
            signs = (rng.integers(0, 2, cand.size).astype(np.uint16) << 15)
            cand = cand | signs
            for k in range(0, cand.size, 15):
                blk = np.zeros(16, np.uint16)
                blk[0] = Ab
                part = cand[k:k + 15]
                blk[1:1 + part.size] = part
                blocks.append(blk)
        flat = np.concatenate(blocks)
        K = 2048
        n_rows = -(-flat.size // (K - 16))
        pad = np.zeros(n_rows * (K - 16), np.uint16)
        pad[:flat.size] = flat
        body = pad.reshape(n_rows, K - 16)
        head = np.zeros((n_rows, 16), np.uint16)
        head[:, 0] = W.bf16_bits(np.array([At]))[0]
        rows.append(np.concatenate([head, body], axis=1))
    return np.concatenate(rows)


def test_nvfp4_tie_sweep(orc):
    check_nvfp4(orc, _tie_sweep(), "tie sweep")


def _wide_range_rows(n_rows: int, cols: int, seed: int):
    """Rows whose amax spans the whole BF16 range (log-uniform exponent, with a
    band around 2^-90, where the kernel changes arithmetic paths) and whose
    blocks sit 0..40 binades below the row amax; zero blocks included."""
    rng = np.random.default_rng(seed)
    X = np.empty((n_rows, cols), np.uint16)
    for r in range(n_rows):
        if r % 3 == 0:
            ea = rng.uniform(-95, -85)
        else:
            ea = rng.uniform(-132, 127)
        A = 2.0 ** ea
        v = np.empty(cols)
        for b in range(cols // 16):
            depth = rng.uniform(0, 40)
            v[16 * b:16 * b + 16] = rng.uniform(-1, 1, 16) * A * 2.0 ** -depth
        v[int(rng.integers(0, cols))] = A
        if r % 5 == 0:
            v[:16] = 0.0
        bits = W.bf16_bits(np.clip(v, -3.38e38, 3.38e38))
        X[r] = bits
    return X


def test_nvfp4_wide_range(orc):
    check_nvfp4(orc, _wide_range_rows(300, 256, 5), "wide range 300x256")
    check_nvfp4(orc, _wide_range_rows(40, 2048, 6), "wide range 40x2048")


def test_nvfp4_every_token_amax(orc):
    """Every finite BF16 magnitude as a token amax (so every FP32 token scale
    the format can produce, subnormal scales included), one row each, with
    the other elements of the row spread below it."""
    mags = np.arange(1, 0x7F80, dtype=np.uint32)            # all finite nonzero magnitudes
    rows, cols = mags.size, 32
    rng = np.random.default_rng(41)
    frac = rng.integers(0, 0x8000, (rows, cols)).astype(np.uint32)
    x = (frac * mags[:, None]) // 0x8000                    # magnitudes <= the row amax
    x[:, 0] = mags
    x |= (rng.integers(0, 2, (rows, cols)).astype(np.uint32) << 15)
    check_nvfp4(orc, x.astype(np.uint16), f"every token amax {rows}x{cols}")


def test_nvfp4_batch_invariance():
    """Per-token outputs of a row do not depend on the other rows of the batch."""
    x = W.config3()[:512]
    announce("nvfp4 batch invariance")
    full = api.nvfp4_quantize_per_token(dev(x))
    perm = np.random.default_rng(3).permutation(512)
    part = api.nvfp4_quantize_per_token(dev(np.ascontiguousarray(x[perm])))
    torch.cuda.synchronize()
    p = torch.from_numpy(perm).cuda()
    for a, b in zip(full, part):
        assert torch.equal(a[p], b)


# ---------------------------------------------------------------------------
# Scoped NVFP4 (gate/up pairs, down)
# ---------------------------------------------------------------------------

def check_pair(orc, gate, up, name):
    """Every byte of the export: codes, block scales and scope scales of all
    experts, against the oracle over the same tensors."""
    announce(f"nvfp4 gateup {name} gate={gate.shape} up={None if up is None else up.shape}")
    r = api.nvfp4_quantize_gateup_pair(dev(gate), None if up is None else dev(up))
    torch.cuda.synchronize()
    gc, gb, uc, ub, s = orc.nvfp4_gateup_pair(gate, up)
    assert_same(host(r.scope_scales).view(np.uint32), s.view(np.uint32), f"{name} scales")
    assert_same(host(r.gate_block_scales), gb, f"{name} gate bs")
    assert_same(host(r.gate_codes), gc, f"{name} gate codes")
    if up is not None:
        assert_same(host(r.up_block_scales), ub, f"{name} up bs")
        assert_same(host(r.up_codes), uc, f"{name} up codes")
    return r, (gc, gb, uc, ub, s)


def scope_amax_bits(gate, up=None):
    """Each scope's largest magnitude as BF16 bits (positive BF16 values order
    like their bit patterns, so this is an integer max)."""
    E = gate.shape[0]
    m = (gate.reshape(E, -1) & 0x7FFF).max(axis=1)
    if up is not None:
        m = np.maximum(m, (up.reshape(E, -1) & 0x7FFF).max(axis=1))
    return m.astype(np.uint16)


def check_pair_amax(orc, gate, up, amax, name):
    """The export with caller-supplied scope amaxes: every scope quantized under
    s_e = fp32(amax_e / 2688) (the oracle's quantize under a given scale)."""
    announce(f"nvfp4 gateup amax {name} gate={gate.shape}")
    r = api.nvfp4_quantize_gateup_pair_amax(dev(gate), None if up is None else dev(up), dev(amax))
    torch.cuda.synchronize()
    sc = host(r.scope_scales)
    for e in range(gate.shape[0]):
        s = orc.nvfp4_scale(float(orc.bf16_value(int(amax[e]) & 0x7FFF)))
        assert sc[e].view(np.uint32) == np.float32(s).view(np.uint32), (name, e)
        for src, codes, bs in ((gate, r.gate_codes, r.gate_block_scales),
                               (up, r.up_codes, r.up_block_scales)):
            if src is None:
                continue
            c, b = orc.nvfp4_with_scale(src[e], s)
            assert_same(host(codes[e]), c, f"{name} e{e} codes")
            assert_same(host(bs[e]), b, f"{name} e{e} block scales")


def test_gateup_amax_variant_small(orc):
    rng = np.random.default_rng(19)
    g = W.bf16_bits(rng.normal(0, 0.02, (4, 48, 64)))
    u = W.bf16_bits(rng.normal(0, 0.05, (4, 48, 64)))
    true = scope_amax_bits(g, u)
    check_pair_amax(orc, g, u, true, "true amax pair")
    check_pair_amax(orc, g, None, scope_amax_bits(g), "true amax single")
    # Not the scopes' own amax: a quarter (codes and block scales saturate),
    # four times, a negative sign bit, zero, and a BF16 subnormal.
    other = W.bf16_bits(W.bf16_to_f64(true) * np.array([0.25, 4.0, 1.0, 1.0]))
    other[2] |= 0x8000
    check_pair_amax(orc, g, u, other, "other amax")
    check_pair_amax(orc, g, u, np.array([0, 1, 0x0080, 0x7F7F], np.uint16), "edge amax")


def test_gateup_small(orc):
    rng = np.random.default_rng(9)
    g = W.bf16_bits(rng.normal(0, 0.02, (3, 48, 64)))
    u = W.bf16_bits(rng.normal(0, 0.05, (3, 48, 64)))
    check_pair(orc, g, u, "small pair")
    check_pair(orc, g, None, "small single")
    z = np.zeros((2, 16, 32), np.uint16)
    check_pair(orc, z, z.copy(), "zeros pair")
    wide = _wide_range_rows(64, 256, 7).reshape(4, 16, 256)
    check_pair(orc, wide, None, "wide single")


def test_gateup_config4_full(orc):
    """The expert-weight export at full size (128 experts; gate/up 768x2048 with
    a shared scale per pair, down 2048x768 alone): every byte of all 128
    experts, then the BF16 round trip of gate, up and down of every expert with
    one FP32 scale per expert (rows_per_fp32_scale = rows of one expert)."""
    gate, up, down = W.config4()
    E = gate.shape[0]
    rp, (gc, gb, uc, ub, sp) = check_pair(orc, gate, up, "config4 gate/up")
    rd, (dc, db, _, _, sd) = check_pair(orc, down, None, "config4 down")
    # The same export with each scope's amax supplied by the caller.
    for g_, u_, want, label in ((gate, up, (gc, gb, uc, ub, sp), "gate/up"),
                                (down, None, (dc, db, None, None, sd), "down")):
        announce(f"nvfp4 gateup amax config4 {label}")
        ra = api.nvfp4_quantize_gateup_pair_amax(dev(g_), None if u_ is None else dev(u_),
                                                 dev(scope_amax_bits(g_, u_)))
        torch.cuda.synchronize()
        assert_same(host(ra.scope_scales).view(np.uint32), want[4].view(np.uint32),
                    f"config4 amax {label} scales")
        assert_same(host(ra.gate_codes), want[0], f"config4 amax {label} codes")
        assert_same(host(ra.gate_block_scales), want[1], f"config4 amax {label} bs")
        if u_ is not None:
            assert_same(host(ra.up_codes), want[2], f"config4 amax {label} up codes")
            assert_same(host(ra.up_block_scales), want[3], f"config4 amax {label} up bs")
        del ra
    del gate, up, down
    for label, codes, bs, sc, wc, wb, ws, rows in (
            ("gate", rp.gate_codes, rp.gate_block_scales, rp.scope_scales, gc, gb, sp, 768),
            ("up", rp.up_codes, rp.up_block_scales, rp.scope_scales, uc, ub, sp, 768),
            ("down", rd.gate_codes, rd.gate_block_scales, rd.scope_scales, dc, db, sd, 2048)):
        announce(f"dequant config4 round trip {label} ({E} experts)")
        y = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, codes, bs, sc, rows)
        torch.cuda.synchronize()
        want = orc.dequant_nvfp4(wc.reshape(E * rows, -1), wb.reshape(E * rows, -1), ws, rows)
        assert_same(host(y).reshape(want.shape), want, f"config4 {label} round trip")
        del y, want


# ---------------------------------------------------------------------------
# Dequant
# ---------------------------------------------------------------------------

def test_dequant_mxfp8(orc):
    for name, x in [("config1", W.config1()), ("boundary", W.mode_boundary(256, 512, 3)),
                    ("maxes", W.mode_maxes(64, 64)), ("zeros", W.mode_zeros(32, 64))]:
        rc, rs = orc.mxfp8_rowwise(x)
        cc, cs = orc.mxfp8_colwise(x)
        announce(f"dequant mxfp8 {name}")
        yr = api.dequantize_bf16(mxq.MXQ_FMT_MXFP8_ROW, dev(rc), dev(rs))
        yc = api.dequantize_bf16(mxq.MXQ_FMT_MXFP8_COL, dev(cc), dev(cs))
        torch.cuda.synchronize()
        assert_same(host(yr), orc.dequant_mxfp8_rowwise(rc, rs), f"{name} row dequant")
        assert_same(host(yc), orc.dequant_mxfp8_colwise(cc, cs), f"{name} col dequant")


def test_dequant_mxfp8_random_bytes(orc):
    """Arbitrary E4M3 codes (no NaN) under every E8M0 byte: overflow saturates,
    underflow rounds into BF16 subnormals."""
    rng = np.random.default_rng(31)
    codes = rng.integers(0, 256, (512, 256)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    scales = rng.integers(0, 255, (512, 8)).astype(np.uint8)
    announce("dequant mxfp8 random bytes")
    y = api.dequantize_bf16(mxq.MXQ_FMT_MXFP8_ROW, dev(codes), dev(scales))
    torch.cuda.synchronize()
    assert_same(host(y), orc.dequant_mxfp8_rowwise(codes, scales), "random row dequant")
    cs = rng.integers(0, 255, (16, 256)).astype(np.uint8)
    y = api.dequantize_bf16(mxq.MXQ_FMT_MXFP8_COL, dev(codes), dev(cs))
    torch.cuda.synchronize()
    assert_same(host(y), orc.dequant_mxfp8_colwise(codes, cs), "random col dequant")


def test_dequant_nvfp4(orc):
    for name, x in [("config3", W.config3()), ("boundary", W.nvfp4_boundary(64, 2048, 2)),
                    ("wide", _wide_range_rows(200, 256, 8)), ("ties", _tie_sweep()[:64])]:
        c, b, s = orc.nvfp4_per_token(x)
        announce(f"dequant nvfp4 {name} {x.shape}")
        y = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, dev(c), dev(b), dev(s), 1)
        torch.cuda.synchronize()
        assert_same(host(y), orc.dequant_nvfp4(c, b, s, 1), f"{name} nvfp4 dequant")


def test_dequant_nvfp4_random_bytes(orc):
    """Random codes and block scales under FP32 scales across the whole range
    (subnormal, around 2^-100, huge), per token and per group of rows."""
    rng = np.random.default_rng(32)
    rows, cols = 1024, 128
    codes = rng.integers(0, 256, (rows, cols // 2)).astype(np.uint8)
    bs = rng.integers(0, 256, (rows, cols // 16)).astype(np.uint8)
    bs[(bs & 0x7F) == 0x7F] = 0x38
    e = rng.integers(-149, 117, rows)
    m = rng.integers(0, 1 << 23, rows)
    sb = np.where(e < -126, m >> np.minimum(-126 - e, 23), ((e + 127) << 23) | m).astype(np.uint32)
    s = sb.view(np.float32)
    s[::7] = np.float32(2.0 ** -100)
    announce("dequant nvfp4 random bytes")
    y = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, dev(codes), dev(bs), dev(s), 1)
    torch.cuda.synchronize()
    assert_same(host(y), orc.dequant_nvfp4(codes, bs, s, 1), "random nvfp4 dequant")
    s8 = np.ascontiguousarray(s[:rows // 8])
    y = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, dev(codes), dev(bs), dev(s8), 8)
    torch.cuda.synchronize()
    assert_same(host(y), orc.dequant_nvfp4(codes, bs, s8, 8), "random nvfp4 dequant /8")


def test_dequant_config4_round_trip_small(orc):
    """Dequant of the export of 8 experts with one scale per expert, gate, up
    and down (the full 128-expert round trip is part of the config-4 test)."""
    gate, up, down = W.config4(8)
    announce("dequant config4 round trip (8 experts)")
    r = api.nvfp4_quantize_gateup_pair(dev(gate), dev(up))
    rd = api.nvfp4_quantize_gateup_pair(dev(down), None)
    yg = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, r.gate_codes, r.gate_block_scales,
                             r.scope_scales, 768)
    yu = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, r.up_codes, r.up_block_scales,
                             r.scope_scales, 768)
    yd = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, rd.gate_codes, rd.gate_block_scales,
                             rd.scope_scales, 2048)
    torch.cuda.synchronize()
    gc, gb, uc, ub, sc = orc.nvfp4_gateup_pair(gate, up)
    dc, db, _, _, sd = orc.nvfp4_gateup_pair(down, None)
    assert_same(host(yg), orc.dequant_nvfp4(gc.reshape(-1, 1024), gb.reshape(-1, 128), sc, 768),
                "config4 gate round trip")
    assert_same(host(yu), orc.dequant_nvfp4(uc.reshape(-1, 1024), ub.reshape(-1, 128), sc, 768),
                "config4 up round trip")
    assert_same(host(yd), orc.dequant_nvfp4(dc.reshape(-1, 384), db.reshape(-1, 48), sd, 2048),
                "config4 down round trip")


# ---------------------------------------------------------------------------
# Grouped
# ---------------------------------------------------------------------------

def check_grouped(orc, x, off, name):
    """Every segment of both grouped outputs against the oracle's standalone
    quantize of that segment alone (columnwise blocks restart at each
    segment; rowwise and per-token bytes depend only on the row)."""
    announce(f"grouped {name} R={x.shape[0]} G={off.size - 1}")
    xd = dev(x)
    od = dev(off)
    g8 = api.grouped_quantize_mxfp8(xd, od)
    g4 = api.grouped_quantize_nvfp4(xd, od)
    torch.cuda.synchronize()
    del xd
    G = off.size - 1
    P = host(g8.col_scale_offsets)
    counts = [(int(off[e + 1]) - int(off[e]) + 31) // 32 for e in range(G)]
    assert list(P) == list(np.concatenate([[0], np.cumsum(counts)]))
    rc, rs = host(g8.row_codes), host(g8.row_scales)
    cc, cs = host(g8.col_codes), host(g8.col_scales)
    c4, b4, s4 = host(g4.codes), host(g4.block_scales), host(g4.fp32_scales)
    assert cs.shape[0] >= P[-1]
    for e in range(G):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        seg = x[a:b]
        sub_off = np.array([0, b - a], np.int64)
        oc, os_, _ = orc.mxfp8_colwise_grouped(seg, sub_off)
        assert_same(cc[a:b], oc, f"{name} seg{e} col codes")
        assert_same(cs[P[e]:P[e + 1]], os_, f"{name} seg{e} col scales")
        orow, orows = orc.mxfp8_rowwise(seg)
        assert_same(rc[a:b], orow, f"{name} seg{e} row codes")
        assert_same(rs[a:b], orows, f"{name} seg{e} row scales")
        nc, nb, ns = orc.nvfp4_per_token(seg)
        assert_same(c4[a:b], nc, f"{name} seg{e} nvfp4 codes")
        assert_same(b4[a:b], nb, f"{name} seg{e} nvfp4 bs")
        assert_same(s4[a:b].view(np.uint32), ns.view(np.uint32), f"{name} seg{e} nvfp4 s")
    return g8, g4, (rc, rs, c4, b4, s4)


def padded_colt(orc, x, off):
    """The oracle's grouped columnwise copy laid out as mxq_mxfp8_grouped_colwise_t
    stores it: transposed, each segment padded to 128 rows with zero codes
    and zero scale bytes.  Returns (codes_t, scales_t, block offsets)."""
    R, cols = x.shape
    G = off.size - 1
    blocks = []
    for e in range(G):
        c = -(-(int(off[e + 1]) - int(off[e])) // 32)          # ceil(rows / 32)
        blocks.append(-(-c // 4) * 4)                           # up to a multiple of 4
    P = np.concatenate([[0], np.cumsum(blocks)]).astype(np.int64)
    ct = np.zeros((cols, 32 * int(P[-1])), np.uint8)
    st = np.zeros((cols, int(P[-1])), np.uint8)
    for e in range(G):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        oc, os_, _ = orc.mxfp8_colwise_grouped(x[a:b], np.array([0, b - a], np.int64))
        ct[:, 32 * P[e]:32 * P[e] + (b - a)] = oc.T
        st[:, P[e]:P[e] + os_.shape[0]] = os_.T
    return ct, st, P


def check_grouped_colt(orc, x, off, name):
    """mxq_mxfp8_grouped_colwise_t against padded_colt, byte for byte, over
    every segment's padded columns and the block offsets."""
    announce(f"grouped colwise transposed {name} R={x.shape[0]} G={off.size - 1}")
    g = api.mxfp8_grouped_colwise_t(dev(x), dev(off))
    torch.cuda.synchronize()
    ct, st, P = padded_colt(orc, x, off)
    assert list(host(g.block_offsets)) == list(P)
    n = 32 * int(P[-1])
    assert_same(host(g.codes_t)[:, :n], ct, f"{name} codes_t")
    assert_same(host(g.scales_t)[:, :int(P[-1])], st, f"{name} scales_t")
    return g


def test_grouped_colwise_transposed_padded(orc):
    """Segments of 0, 1, 31, 33, 128 and 200 rows (partial tail blocks, exact
    128-row segments, empty ones), boundary-mode values."""
    sizes = [0, 1, 31, 33, 128, 200, 0, 64]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    x = W.mode_boundary(512, 96, 4)[:int(off[-1])]
    check_grouped_colt(orc, x, off, "ragged")
    check_grouped_colt(orc, W.mode_random(40, 64, 5), np.array([0, 40], np.int64), "one segment")


def check_grouped_rowcolt(orc, x, off, name):
    """mxq_mxfp8_grouped_quantize_rowcol_t: the transposed copy against
    padded_colt and the rowwise copy against the oracle's rowwise quantize of
    every row, byte for byte."""
    announce(f"grouped rowwise + colwise transposed {name} R={x.shape[0]} G={off.size - 1}")
    rc, rs, g = api.mxfp8_grouped_quantize_rowcol_t(dev(x), dev(off))
    torch.cuda.synchronize()
    ct, st, P = padded_colt(orc, x, off)
    assert list(host(g.block_offsets)) == list(P)
    n = 32 * int(P[-1])
    assert_same(host(g.codes_t)[:, :n], ct, f"{name} codes_t")
    assert_same(host(g.scales_t)[:, :int(P[-1])], st, f"{name} scales_t")
    del ct, st, g
    orow, orows = orc.mxfp8_rowwise(x)
    assert_same(host(rc), orow, f"{name} row codes")
    assert_same(host(rs), orows, f"{name} row scales")


def test_grouped_rowcol_transposed_ragged(orc):
    """Both backward copies from one read: segments of 0, 1, 31, 33, 128 and
    200 rows (96 columns: a partial strip), boundary-mode values."""
    sizes = [0, 1, 31, 33, 128, 200, 0, 64]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    x = W.mode_boundary(512, 96, 4)[:int(off[-1])]
    check_grouped_rowcolt(orc, x, off, "ragged")
    check_grouped_rowcolt(orc, W.mode_random(40, 64, 5), np.array([0, 40], np.int64),
                          "one segment")


def test_grouped_rowcol_transposed_config5_full(orc):
    """Config 5's 262144 x 2048 expert-sorted rows over 128 segments: every
    byte of both copies."""
    x, off = W.config5()
    check_grouped_rowcolt(orc, x, off, "config5")


def test_grouped_weight_gradient(orc):
    """The expert layer's weight gradient dW_e = dY_e^T X_e over each segment's
    rows from two grouped transposed copies (dY [R][256], X [R][192]), every
    expert (an empty one must give zeros) against the oracle's product of the
    same padded operands."""
    sizes = [0, 1, 31, 33, 128, 200, 0, 64]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    R = int(off[-1])
    dy = W.student_t_activations(R, 256, 41)
    x = W.mode_random(R, 192, 42)
    announce(f"mxfp8 grouped wgrad R={R} G={len(sizes)} 256x192")
    gd = api.mxfp8_grouped_colwise_t(dev(dy), dev(off))
    gx = api.mxfp8_grouped_colwise_t(dev(x), dev(off))
    for dt in (torch.float32, torch.bfloat16):
        c = api.mxfp8_grouped_wgrad(gd, gx, out_dtype=dt)
        torch.cuda.synchronize()
        got = c.float().cpu().numpy().astype(np.float64)
        dct, dst, P = padded_colt(orc, dy, off)
        xct, xst, _ = padded_colt(orc, x, off)
        for e in range(len(sizes)):
            k0, k1 = 32 * int(P[e]), 32 * int(P[e + 1])
            if k0 == k1:
                assert np.all(got[e] == 0), f"empty expert {e}"
                continue
            C, S = orc.mxfp8_gemm(dct[:, k0:k1], dst[:, k0 // 32:k1 // 32],
                                  xct[:, k0:k1], xst[:, k0 // 32:k1 // 32])
            bound = (GEMM_REL + (k1 - k0) * 2.0 ** -24) * S
            lim = bound if dt == torch.float32 else bound + 2.0 ** -8 * np.abs(C)
            assert np.all(np.abs(got[e] - C) <= lim), f"expert {e} {dt}"


def test_grouped_weight_gradient_moe_layer_sampled(orc):
    """Config 5's routing (262144 rows, 128 experts): dW_e [768][2048] =
    dY_e^T X_e for experts 0, 63 and 127 in full, the rest computed too."""
    x, off = W.config5()
    dy = W.student_t_activations(x.shape[0], 768, 43)
    announce("mxfp8 grouped wgrad config5 768x2048")
    gd = api.mxfp8_grouped_colwise_t(dev(dy), dev(off))
    gx = api.mxfp8_grouped_colwise_t(dev(x), dev(off))
    c = api.mxfp8_grouped_wgrad(gd, gx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    P = host(gd.block_offsets)
    assert list(P) == list(host(gx.block_offsets))
    for e in (0, 63, 127):
        a, b = int(off[e]), int(off[e + 1])
        sub = np.array([0, b - a], np.int64)
        dct, dst, Pe = padded_colt(orc, dy[a:b], sub)
        xct, xst, _ = padded_colt(orc, x[a:b], sub)
        assert 32 * (int(P[e + 1]) - int(P[e])) == dct.shape[1]
        C, S = orc.mxfp8_gemm(dct, dst, xct, xst)
        got = host(c[e]).astype(np.float64)
        assert np.all(np.abs(got - C) <= (GEMM_REL + dct.shape[1] * 2.0 ** -24) * S), f"expert {e}"


def test_grouped_ragged_stress(orc):
    """Segments of 0, 1, 31, 32, 33 and 4096 rows among random ones."""
    off = W.ragged_offsets(16384, 24, seed=7)
    x = W.student_t_activations(int(off[-1]), 256, 70)
    check_grouped(orc, x, off, "ragged stress")


@pytest.mark.parametrize("G", [65, 256, 257, 300])
def test_grouped_many_segments(orc, G):
    """Segment counts across the in-kernel prefix limit (256 segments; above
    it a prefix launch precedes the kernels) and across the 64-segment scan
    chunks: every segment of both grouped outputs, and both copies of the
    grouped transposed call."""
    off = W.ragged_offsets(8192, G, seed=G, forced=(0, 1, 31, 32, 33, 700))
    x = W.student_t_activations(int(off[-1]), 128, G + 1)
    check_grouped(orc, x, off, f"{G} segments")
    check_grouped_rowcolt(orc, x, off, f"{G} segments")


def test_grouped_small_edge(orc):
    off = np.array([0, 0, 1, 1, 33, 65, 65, 96, 97], np.int64)
    x = W.mode_boundary(128, 64, 3)[:97]
    check_grouped(orc, x, off, "edge segments")
    off1 = np.array([0, 5], np.int64)
    check_grouped(orc, W.mode_random(32, 32, 1)[:5], off1, "one short segment")


def test_grouped_config5_full(orc):
    """The grouped workload at full size (262,144 expert-sorted rows of 2048,
    128 uniform top-8 segments): every segment, then the BF16 dequant of the
    MXFP8 rowwise and NVFP4 outputs over all rows (the dequant inputs are the
    GPU's codes, already shown equal to the oracle's)."""
    x, off = W.config5()
    g8, g4, (rc, rs, c4, b4, s4) = check_grouped(orc, x, off, "config5")
    del x
    announce("grouped config5 dequant")
    y8 = api.dequantize_bf16(mxq.MXQ_FMT_MXFP8_ROW, g8.row_codes, g8.row_scales)
    torch.cuda.synchronize()
    assert_same(host(y8), orc.dequant_mxfp8_rowwise(rc, rs), "config5 mxfp8 row dequant")
    del y8
    y4 = api.dequantize_bf16(mxq.MXQ_FMT_NVFP4, g4.codes, g4.block_scales, g4.fp32_scales, 1)
    torch.cuda.synchronize()
    assert_same(host(y4), orc.dequant_nvfp4(c4, b4, s4, 1), "config5 nvfp4 dequant")


# ---------------------------------------------------------------------------
# Comparison variants (not the contract): OCP MX scale rule, per-tensor scope
# ---------------------------------------------------------------------------

def check_ocp(orc, x: np.ndarray, name: str):
    announce(f"mxfp8 ocp floor {name} shape={x.shape}")
    r = api.mxfp8_quantize_ocp_floor(dev(x))
    torch.cuda.synchronize()
    rc, rs, cc, cs = orc.mxfp8_ocp_floor(x)
    assert_same(host(r.row_scales), rs, f"{name} row scales")
    assert_same(host(r.row_codes), rc, f"{name} row codes")
    assert_same(host(r.col_scales), cs, f"{name} col scales")
    assert_same(host(r.col_codes), cc, f"{name} col codes")
    return rc


@pytest.mark.parametrize("mode", W.MXFP8_MODES)
def test_ocp_floor_config2(orc, mode):
    """The OCP-rule variant on the 8192 x 2048 weight in every data mode
    (boundary: the 448 / 450 / power-of-two amaxes where the two rules part;
    maxes: saturation at the top scale)."""
    rc = check_ocp(orc, W.config2_weight(mode), f"C2b {mode}")
    if mode == "random":
        assert int(((rc & 0x7F) == 0x7E).sum()) > 0      # it clips


def test_ocp_floor_shapes_and_exhaustive(orc):
    for rows, cols in ((32, 32), (64, 96), (96, 288), (32, 4128)):
        check_ocp(orc, W.mode_boundary(rows, cols, rows + cols), f"boundary {rows}x{cols}")
    check_ocp(orc, _mxfp8_exhaustive_input(), "exhaustive rows")


def check_colt(orc, x: np.ndarray, name: str):
    announce(f"mxfp8 transposed columnwise {name} shape={x.shape}")
    r = api.mxfp8_quantize_rowcol_t(dev(x))
    torch.cuda.synchronize()
    cc, cs = orc.mxfp8_colwise(x)
    rc, rs = orc.mxfp8_rowwise(x)
    assert_same(host(r.col_codes), np.ascontiguousarray(cc.T), f"{name} col codes (transposed)")
    assert_same(host(r.col_scales), np.ascontiguousarray(cs.T), f"{name} col scales (transposed)")
    assert_same(host(r.row_codes), rc, f"{name} row codes")
    assert_same(host(r.row_scales), rs, f"{name} row scales")


def test_colwise_transposed_layout(orc):
    """The transposed columnwise layout holds exactly the columnwise bytes,
    permuted; partial column strips included."""
    for mode in ("random", "boundary"):
        check_colt(orc, W.config2_weight(mode), f"C2b {mode}")
    for rows, cols in ((32, 32), (64, 96), (96, 288), (32, 4128)):
        check_colt(orc, W.mode_boundary(rows, cols, rows + 3 * cols), f"boundary {rows}x{cols}")


def test_colwise_transposed_scale_stores(orc):
    """The transposed scales go out as dwords only where whole and 4-byte
    aligned: scale pitches (rows / 32) of 13, 33 and 12 blocks, groups of
    eight blocks that end mid-dword, and a scale pointer one byte past an
    aligned address (every store then a byte store; the byte before it and
    the codes stay as they are)."""
    for rows, cols in ((416, 160), (1056, 64), (384, 128), (288, 4128)):
        check_colt(orc, W.mode_boundary(rows, cols, rows + 5 * cols), f"pitch {rows // 32} "
                   f"{rows}x{cols}")
    rows, cols = 256, 256
    x = W.mode_boundary(rows, cols, 77)
    announce(f"mxfp8 transposed columnwise, scale pointer off alignment {rows}x{cols}")
    ct = torch.zeros((cols, rows), dtype=torch.uint8, device="cuda")
    st = torch.full((cols * (rows // 32) + 1,), 0xAB, dtype=torch.uint8, device="cuda")
    xd = dev(x)
    mxq.mxq_mxfp8_quantize_rowcol_t(xd, rows, cols, None, None, ct, st.data_ptr() + 1)
    torch.cuda.synchronize()
    cc, cs = orc.mxfp8_colwise(x)
    got = host(st)
    assert got[0] == 0xAB, "byte before the scales written"
    assert_same(got[1:].reshape(cols, rows // 32), np.ascontiguousarray(cs.T),
                "misaligned col scales (transposed)")
    assert_same(host(ct), np.ascontiguousarray(cc.T), "col codes (transposed)")


def test_gemm_weight_gradient_from_transposed_copies(orc):
    """dW[N][K] = dY^T X over the M rows: both operands' columnwise copies,
    transposed, are K-contiguous operands of the same GEMM kernel."""
    M, N, K = 512, 256, 384
    dy = W.student_t_activations(M, N, 91)
    x = W.mode_random(M, K, 92)
    announce(f"mxfp8 wgrad {N}x{K} over M={M}")
    qd = api.mxfp8_quantize_rowcol_t(dev(dy), rowwise=False)
    qx = api.mxfp8_quantize_rowcol_t(dev(x), rowwise=False)
    c = api.mxfp8_gemm(qd.col_codes, qd.col_scales, qx.col_codes, qx.col_scales,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    dc, ds = orc.mxfp8_colwise(dy)
    xc, xs = orc.mxfp8_colwise(x)
    C, S = orc.mxfp8_gemm(np.ascontiguousarray(dc.T), np.ascontiguousarray(ds.T),
                          np.ascontiguousarray(xc.T), np.ascontiguousarray(xs.T))
    err = np.abs(host(c).astype(np.float64) - C)
    assert np.all(err <= (GEMM_REL + M * 2.0 ** -24) * S)


def test_grouped_gemm_data_gradient_from_transposed_weights(orc):
    """The expert layer's data gradient dX[r][k] = sum_n dY[r][n] W_e[n][k]
    for the rows r of segment e: dY's rowwise copy times each expert's
    columnwise copy transposed ([K][N], blocks along n), through the grouped
    entry point, against the oracle per segment."""
    sizes = [130, 0, 257, 40]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    R, N, K, G = int(offsets[-1]), 256, 192, len(sizes)
    dy = W.student_t_activations(R, N, 93)
    w = np.stack([W.mode_random(N, K, 94 + e) for e in range(G)])
    announce(f"mxfp8 grouped dgrad R={R} G={G} N={N} K={K}")
    qw = [api.mxfp8_quantize_rowcol_t(dev(w[e]), rowwise=False) for e in range(G)]
    wt = torch.stack([q.col_codes for q in qw])            # [G][K][N]
    wts = torch.stack([q.col_scales for q in qw])          # [G][K][N/32]
    qd = api.mxfp8_quantize_rowcol(dev(dy), colwise=False)
    c = api.mxfp8_grouped_gemm(qd.row_codes, qd.row_scales, wt, wts, dev(offsets),
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = host(c).astype(np.float64)
    dc, ds = orc.mxfp8_rowwise(dy)
    for e in range(G):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        wc, ws = orc.mxfp8_colwise(w[e])
        C, S = orc.mxfp8_gemm(dc[lo:hi], ds[lo:hi], np.ascontiguousarray(wc.T),
                              np.ascontiguousarray(ws.T))
        err = np.abs(got[lo:hi] - C)
        assert np.all(err <= (GEMM_REL + N * 2.0 ** -24) * S), f"expert {e}"


def test_nvfp4_approx_differs_only_at_midpoints(orc):
    """The opt-in approximate variant: the FP32 token scales are exact; a block
    scale differs from the exact one only where amax / (6 s) lies within
    2^-19 (relative) of the E4M3 midpoint between the two; inside blocks with
    the exact scale, a code differs only where |x| / (dec(b) s) lies within
    2^-19 of the E2M1 midpoint between it and the exact code.  Student-t
    tokens plus rows whose scales span the range."""
    x = np.concatenate([W.config3()[:4096], _wide_range_rows(256, 2048, 9)])
    announce(f"nvfp4 approx {x.shape}")
    r = api.nvfp4_quantize_per_token_approx(dev(x))
    torch.cuda.synchronize()
    c, b, s = orc.nvfp4_per_token(x)
    ac, ab, as_ = host(r.codes), host(r.block_scales), host(r.fp32_scales)
    assert_same(as_.view(np.uint32), s.view(np.uint32), "token scales")
    e4 = np.array([orc.e4m3_value(i) for i in range(256)])
    e2 = np.array([orc.e2m1_value(i) for i in range(16)])
    xv = np.abs(W.bf16_to_f64(x))
    S = s.astype(np.float64)[:, None]
    amax = xv.reshape(x.shape[0], -1, 16).max(axis=2)
    bad_b = np.argwhere(ab != b)
    for i, j in bad_b:
        mid = (e4[b[i, j]] + e4[ab[i, j]]) / 2
        assert abs(amax[i, j] / (6 * S[i, 0]) - mid) <= 2.0 ** -19 * mid, (i, j)
    nib = lambda q: np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], -1)
    ce, ca = nib(c), nib(ac)
    same_b = np.repeat(ab == b, 16, axis=1)
    diff = np.argwhere((ce != ca) & same_b)
    with np.errstate(divide="ignore", invalid="ignore"):     # zero scales: never compared
        q = xv / (np.repeat(e4[b], 16, axis=1) * S)
    for i, k in diff:
        ke, ka = int(ce[i, k]), int(ca[i, k])
        assert (ke & 8) == (ka & 8) and abs((ke & 7) - (ka & 7)) == 1, (i, k)
        mid = (e2[ke & 7] + e2[ka & 7]) / 2
        assert abs(q[i, k] - mid) <= 2.0 ** -19 * mid, (i, k)
    announce(f"  approx: {len(bad_b)} block scales and {len(diff)} codes differ "
             f"of {b.size} and {ce.size}")


def test_per_tensor_nvfp4(orc):
    """Per-tensor activation NVFP4 (one FP32 scale for the tensor) equals the
    oracle's one-tensor scope."""
    x = W.config3()[:1024]
    announce("nvfp4 per-tensor 1024x2048")
    r = api.nvfp4_quantize_per_tensor(dev(x))
    torch.cuda.synchronize()
    c, b, _, _, s = orc.nvfp4_gateup_pair(x[None], None)
    assert_same(host(r.fp32_scales).view(np.uint32), s.view(np.uint32), "per-tensor scale")
    assert_same(host(r.codes), c[0], "per-tensor codes")
    assert_same(host(r.block_scales), b[0], "per-tensor block scales")


# ---------------------------------------------------------------------------
# Block-scaled GEMM on MXFP8 operands
# ---------------------------------------------------------------------------

# The fp8 matrix instruction sums the 64 products of one K slice to about
# 12 bits relative to their magnitude sum (measured on MI355X: at most
# 2^-11.6 sum|a b| on all-positive operands, independent of K; the fp32
# accumulator itself adds at full precision).  Realistic operands are held
# to 2^-10 sum|a b| plus the fp32 accumulation term; operands whose products
# fit a narrow window, where the instruction's sum is exact, to bit equality.
GEMM_REL = 2.0 ** -10


def check_gemm(orc, x: np.ndarray, w: np.ndarray, name: str, row_sample=None):
    """A = rowwise MXFP8 of x [M][K], B = rowwise MXFP8 of w [N][K] (both made
    by the oracle), C = A B^T on the GPU in fp32 and BF16, against the
    oracle's exact product: |C - exact| <= (2^-10 + K 2^-24) sum|a b|, plus
    half a BF16 step of |exact| (at most 2^-8 |exact|) for the BF16 result."""
    M, K = x.shape
    N = w.shape[0]
    ac, as_ = orc.mxfp8_rowwise(x)
    bc, bs_ = orc.mxfp8_rowwise(w)
    rows = np.arange(M) if row_sample is None else np.asarray(row_sample)
    C, S = orc.mxfp8_gemm(ac[rows], as_[rows], bc, bs_)
    bound = (GEMM_REL + K * 2.0 ** -24) * S
    for dt in (torch.float32, torch.bfloat16):
        announce(f"mxfp8 gemm {name} M={M} N={N} K={K} {dt}")
        c = api.mxfp8_gemm(dev(ac), dev(as_), dev(bc), dev(bs_), out_dtype=dt)
        torch.cuda.synchronize()
        got = c.float().cpu().numpy().astype(np.float64)[rows]
        err = np.abs(got - C)
        lim = bound if dt == torch.float32 else bound + 2.0 ** -8 * np.abs(C)
        bad = np.argwhere(err > lim)
        assert bad.size == 0, (f"{name} {dt}: {len(bad)} outside the bound, first {tuple(bad[0])}: "
                               f"got {got[tuple(bad[0])]!r} want {C[tuple(bad[0])]!r}")


def test_gemm_exact_when_products_fit(orc):
    """Codes 1 .. 3.75 and block scales 2^-1 .. 2^1: every slice's sum of
    products is exact inside the instruction and every partial sum is exact
    in fp32, so C must equal the oracle bit for bit (fp32), and the BF16
    result must be the nearest-even rounding of it.  Ragged M and N."""
    rng = np.random.default_rng(73)
    M, N, K = 300, 200, 256
    codes = np.array([c for c in range(256) if ((c >> 3) & 15) in (7, 8)], np.uint8)
    a = rng.choice(codes, (M, K)).astype(np.uint8)
    b = rng.choice(codes, (N, K)).astype(np.uint8)
    sa = rng.integers(126, 129, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(126, 129, (N, K // 32)).astype(np.uint8)
    C, _ = orc.mxfp8_gemm(a, sa, b, sb)
    announce(f"mxfp8 gemm exact {M}x{N}x{K}")
    c32 = api.mxfp8_gemm(dev(a), dev(sa), dev(b), dev(sb), out_dtype=torch.float32)
    c16 = api.mxfp8_gemm(dev(a), dev(sa), dev(b), dev(sb), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(C.astype(np.float32), C)          # exact in fp32 by construction
    assert_same(host(c32).view(np.uint32), C.astype(np.float32).view(np.uint32), "fp32 C")
    assert_same(host(c16), orc.bf16_round_sat_many(C).reshape(M, N), "bf16 C")


def test_gemm_small_shapes(orc):
    """One tile, ragged M and N (partial tiles), several K steps."""
    for (M, N, K, seed) in ((256, 256, 128, 1), (300, 200, 256, 2), (1, 1, 128, 3),
                            (64, 520, 384, 4), (513, 33, 640, 5), (40, 300, 128, 6)):
        x = W.student_t_activations(M, K, seed)
        w = W.mode_random(N, K, seed + 100)
        check_gemm(orc, x, w, f"t3 x random {M}x{N}x{K}")


def test_gemm_scale_range(orc):
    """Operands whose 32-blocks span many binades (every block scale differs),
    with products kept inside the fp32 range."""
    rng = np.random.default_rng(71)
    M, N, K = 96, 160, 512
    x = rng.standard_normal((M, K)) * np.ldexp(1.0, rng.integers(-30, 30, (M, K // 32))).repeat(32, 1)
    w = rng.standard_normal((N, K)) * np.ldexp(1.0, rng.integers(-30, 30, (N, K // 32))).repeat(32, 1)
    check_gemm(orc, W.bf16_bits(x), W.bf16_bits(w), "wide scales")


def test_gemm_dense_forward_full(orc):
    """The dense forward of the pages' layer: activation 2048 x 2048 times a
    weight with out_features 8192 (both random mode), every column of 384
    sampled rows."""
    x = W.config2_activation("random")
    w = W.config2_weight("random")
    rng = np.random.default_rng(72)
    rows = np.concatenate([np.arange(64), rng.integers(0, 2048, 256), np.arange(1984, 2048)])
    check_gemm(orc, x, w, "2048x8192x2048", row_sample=rows)


def check_grouped_gemm(orc, x: np.ndarray, offsets: np.ndarray, w: np.ndarray, name: str,
                       per_segment=None):
    """A = rowwise MXFP8 of the expert-sorted rows x [R][K], B_e = rowwise
    MXFP8 of w[e] [N][K] (both made by the oracle); C [R][N] on the GPU in
    fp32 and BF16 through the grouped entry point, each segment's rows (all,
    or per_segment sampled ones) against the oracle's exact product with
    that segment's expert, to check_gemm's bound.  Rows in no segment must
    keep the bytes the output held before the call."""
    R, K = x.shape
    G, N = w.shape[0], w.shape[1]
    ac, as_ = orc.mxfp8_rowwise(x)
    q = [orc.mxfp8_rowwise(w[e]) for e in range(G)]
    bc = np.stack([p[0] for p in q])
    bs_ = np.stack([p[1] for p in q])
    rng = np.random.default_rng(91)
    covered = np.zeros(R, bool)
    for a, b in zip(offsets[:-1], offsets[1:]):
        covered[a:b] = True
    for dt, code in ((torch.float32, mxq.MXQ_OUT_F32), (torch.bfloat16, mxq.MXQ_OUT_BF16)):
        announce(f"mxfp8 grouped gemm {name} R={R} G={G} N={N} K={K} {dt}")
        c = torch.full((R, N), -7.0, dtype=dt, device="cuda")
        before = host(c).copy()
        mxq.mxq_mxfp8_grouped_gemm(dev(ac), dev(as_), dev(bc), dev(bs_), dev(offsets), G, R, N,
                                   K, code, c)
        torch.cuda.synchronize()
        got_all = host(c)
        assert_same(got_all[~covered], before[~covered], "rows in no segment")
        gotf = c.float().cpu().numpy().astype(np.float64)
        for e in range(G):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            if hi <= lo:
                continue
            rows = np.arange(lo, hi)
            if per_segment is not None and rows.size > per_segment:
                rows = np.unique(np.concatenate([rows[:2], rows[-2:],
                                                 rng.choice(rows, per_segment - 4, replace=False)]))
            C, S = orc.mxfp8_gemm(ac[rows], as_[rows], bc[e], bs_[e])
            bound = (GEMM_REL + K * 2.0 ** -24) * S
            lim = bound if dt == torch.float32 else bound + 2.0 ** -8 * np.abs(C)
            err = np.abs(gotf[rows] - C)
            bad = np.argwhere(err > lim)
            assert bad.size == 0, (f"{name} {dt} expert {e}: {len(bad)} outside the bound, first "
                                   f"row {rows[bad[0][0]]} col {bad[0][1]}: "
                                   f"got {gotf[rows][tuple(bad[0])]!r} want {C[tuple(bad[0])]!r}")


def test_grouped_gemm_ragged_segments(orc):
    """Segments of 0, 1, 33, 256, 257 and 300 rows (empty, single-row, partial
    and exact 256-row tiles), rows before the first and after the last
    segment left alone, ragged N, several K steps."""
    sizes = [0, 1, 300, 0, 257, 33, 256]
    offsets = np.concatenate([[3], 3 + np.cumsum(sizes)]).astype(np.int64)
    R, N, K = int(offsets[-1]) + 5, 200, 384
    x = W.student_t_activations(R, K, 21)
    w = np.stack([W.mode_random(N, K, 30 + e) for e in range(len(sizes))])
    check_grouped_gemm(orc, x, offsets, w, "ragged")


def test_grouped_gemm_moe_layer_sampled(orc):
    """The MoE expert layer at the pages' shape: config 5's 262144 expert-sorted
    rows (32768 tokens, top-8 of 128 experts) times 128 experts' gate
    weights 768 x 2048 (N(0, 0.02)), 12 sampled rows of every segment."""
    x, offsets = W.config5()
    rng = np.random.default_rng(92)
    w = W.bf16_bits(rng.normal(0, 0.02, (128, 768, 2048)))
    check_grouped_gemm(orc, x, offsets, w, "config 5 x 768", per_segment=12)


def check_nvfp4_grouped_gemm(orc, x: np.ndarray, offsets: np.ndarray, w: np.ndarray, name: str,
                             per_segment=None):
    """A = per-token NVFP4 of the expert-sorted rows x [R][K], B_e = the
    export's NVFP4 of w[e] [N][K] with one scope scale per expert (both made
    by the oracle); C [R][N] on the GPU in fp32 and BF16 through the grouped
    entry point, each segment's rows (all, or per_segment sampled ones)
    against the oracle's exact product to check_nvfp4_gemm's bound.  Rows in
    no segment must keep their bytes."""
    R, K = x.shape
    G, N = w.shape[0], w.shape[1]
    ac, ab, as_ = orc.nvfp4_per_token(x)
    bc, bb, _, _, bs_ = orc.nvfp4_gateup_pair(w, None)
    rng = np.random.default_rng(94)
    covered = np.zeros(R, bool)
    for a, b in zip(offsets[:-1], offsets[1:]):
        covered[a:b] = True
    for dt, code in ((torch.float32, mxq.MXQ_OUT_F32), (torch.bfloat16, mxq.MXQ_OUT_BF16)):
        announce(f"nvfp4 grouped gemm {name} R={R} G={G} N={N} K={K} {dt}")
        c = torch.full((R, N), -7.0, dtype=dt, device="cuda")
        before = host(c).copy()
        mxq.mxq_nvfp4_grouped_gemm(dev(ac), dev(ab), dev(as_), dev(bc), dev(bb), dev(bs_),
                                   dev(offsets), G, R, N, K, code, c)
        torch.cuda.synchronize()
        assert_same(host(c)[~covered], before[~covered], "rows in no segment")
        gotf = c.float().cpu().numpy().astype(np.float64)
        for e in range(G):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            if hi <= lo:
                continue
            rows = np.arange(lo, hi)
            if per_segment is not None and rows.size > per_segment:
                rows = np.unique(np.concatenate([rows[:2], rows[-2:],
                                                 rng.choice(rows, per_segment - 4, replace=False)]))
            C, S = orc.nvfp4_gemm(ac[rows], ab[rows], as_[rows], 1, bc[e], bb[e], bs_[e:e + 1], N)
            bound = (K * 2.0 ** -24 + 2.0 ** -23) * S
            lim = bound if dt == torch.float32 else bound + 2.0 ** -8 * np.abs(C)
            err = np.abs(gotf[rows] - C)
            bad = np.argwhere(err > lim)
            assert bad.size == 0, (f"{name} {dt} expert {e}: {len(bad)} outside the bound, first "
                                   f"row {rows[bad[0][0]]} col {bad[0][1]}: "
                                   f"got {gotf[rows][tuple(bad[0])]!r} want {C[tuple(bad[0])]!r}")


def test_nvfp4_grouped_gemm_ragged_segments(orc):
    """Per-token NVFP4 rows in segments of 0, 1, 33, 256, 257 and 300 rows
    (rows outside the segments left alone) times experts' weights with
    their own scope scales (expert amplitudes spread over 2^-4 .. 2^4),
    three K steps."""
    sizes = [0, 1, 300, 0, 257, 33, 256]
    offsets = np.concatenate([[3], 3 + np.cumsum(sizes)]).astype(np.int64)
    R, N, K = int(offsets[-1]) + 5, 200, 192
    x = W.student_t_activations(R, K, 23)
    rng = np.random.default_rng(95)
    amp = np.ldexp(1.0, rng.integers(-4, 5, len(sizes)))[:, None, None]
    w = W.bf16_bits(rng.normal(0, 0.02, (len(sizes), N, K)) * amp)
    check_nvfp4_grouped_gemm(orc, x, offsets, w, "ragged")


def test_nvfp4_grouped_gemm_moe_layer_sampled(orc):
    """Config 5's 262144 expert-sorted rows as per-token NVFP4 times 128
    experts' exported gate weights 768 x 2048 (N(0, 0.02)), 12 sampled rows
    of every segment."""
    x, offsets = W.config5()
    w = W.bf16_bits(np.random.default_rng(96).normal(0, 0.02, (128, 768, 2048)))
    check_nvfp4_grouped_gemm(orc, x, offsets, w, "config 5 x 768", per_segment=12)


def check_nvfp4_gemm(orc, qa, qb, rows_per_b, name, row_sample=None, rel=0.0):
    """qa = (codes, block scales, fp32 scales per row), qb = (codes, block
    scales, fp32 scales per rows_per_b rows), both made by the oracle; C on
    the GPU in fp32 and BF16 against the oracle's exact product, to
    (rel + K 2^-24 + 2^-23) sum|a b| |sa sb| (fp32 accumulation -- the FP16
    matrix instructions accumulate at full fp32 precision, measured at most
    2^-23.8 sum|a b| -- and the two FP32 scale multiplications), plus half a
    BF16 step for the BF16 result."""
    ac, ab, as_ = qa
    bc, bb, bs_ = qb
    M, K = ac.shape[0], 2 * ac.shape[1]
    N = bc.shape[0]
    rows = np.arange(M) if row_sample is None else np.asarray(row_sample)
    C, S = orc.nvfp4_gemm(ac[rows], ab[rows], as_[rows], 1, bc, bb, bs_, rows_per_b)
    bound = (rel + K * 2.0 ** -24 + 2.0 ** -23) * S
    for dt in (torch.float32, torch.bfloat16):
        announce(f"nvfp4 gemm {name} M={M} N={N} K={K} {dt}")
        c = api.nvfp4_gemm(dev(ac), dev(ab), dev(as_), dev(bc), dev(bb), dev(bs_),
                           rows_per_b_scale=rows_per_b, out_dtype=dt)
        torch.cuda.synchronize()
        got = c.float().cpu().numpy().astype(np.float64)[rows]
        err = np.abs(got - C)
        lim = bound if dt == torch.float32 else bound + 2.0 ** -8 * np.abs(C)
        bad = np.argwhere(err > lim)
        worst = float(np.max(err / np.maximum(S, 1e-300)))
        announce(f"  max err / sum|ab| = 2^{np.log2(max(worst, 1e-300)):.1f}")
        assert bad.size == 0, (f"{name} {dt}: {len(bad)} outside the bound, first {tuple(bad[0])}: "
                               f"got {got[tuple(bad[0])]!r} want {C[tuple(bad[0])]!r}")


def test_nvfp4_gemm_exact_when_products_fit(orc):
    """E2M1 magnitudes up to 3, block scales 1 .. 1.875, power-of-two FP32
    scales: every partial sum is exact in fp32, so the fp32 result must equal
    the oracle bit for bit.  Ragged M and N, several FP32 scales in B."""
    rng = np.random.default_rng(74)
    M, N, K = 300, 200, 128
    nib = np.array([0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13], np.uint8)   # |value| <= 3
    a = (rng.choice(nib, (M, K // 2)) | (rng.choice(nib, (M, K // 2)) << 4)).astype(np.uint8)
    b = (rng.choice(nib, (N, K // 2)) | (rng.choice(nib, (N, K // 2)) << 4)).astype(np.uint8)
    ba = rng.integers(0x38, 0x40, (M, K // 16)).astype(np.uint8)           # 1 .. 1.875
    bb = rng.integers(0x38, 0x40, (N, K // 16)).astype(np.uint8)
    sa = np.ldexp(1.0, rng.integers(-3, 4, M)).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-3, 4, (N + 49) // 50)).astype(np.float32)
    C, _ = orc.nvfp4_gemm(a, ba, sa, 1, b, bb, sb, 50)
    announce(f"nvfp4 gemm exact {M}x{N}x{K}")
    c32 = api.nvfp4_gemm(dev(a), dev(ba), dev(sa), dev(b), dev(bb), dev(sb), rows_per_b_scale=50,
                         out_dtype=torch.float32)
    c16 = api.nvfp4_gemm(dev(a), dev(ba), dev(sa), dev(b), dev(bb), dev(sb), rows_per_b_scale=50,
                         out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(C.astype(np.float32), C)
    assert_same(host(c32).view(np.uint32), C.astype(np.float32).view(np.uint32), "fp32 C")
    assert_same(host(c16), orc.bf16_round_sat_many(C).reshape(M, N), "bf16 C")


def test_nvfp4_gemm_shapes(orc):
    """Per-token NVFP4 activations (Student-t) times a weight quantized with
    one FP32 scale for the tensor (the down-projection scope), ragged shapes."""
    for (M, N, K, seed) in ((256, 256, 64, 1), (300, 200, 192, 2), (1, 1, 64, 3),
                            (513, 40, 640, 4)):
        qa = orc.nvfp4_per_token(W.student_t_activations(M, K, seed))
        w = W.bf16_bits(np.random.default_rng(seed + 50).normal(0, 0.02, (1, N, K)))
        wc, wb, _, _, ws = orc.nvfp4_gateup_pair(w, None)
        check_nvfp4_gemm(orc, qa, (wc[0], wb[0], ws), N, f"t3 x N(0,0.02) {M}x{N}x{K}")


def test_nvfp4_gemm_per_row_b_scales(orc):
    """Both operands per-token NVFP4 (one FP32 scale per row of A and of B:
    rows_per_b_scale 1), five K steps (the pipeline's odd tail after a full
    unrolled pair), ragged M and N."""
    M, N, K = 300, 200, 320
    qa = orc.nvfp4_per_token(W.student_t_activations(M, K, 11))
    qb = orc.nvfp4_per_token(W.student_t_activations(N, K, 12))
    check_nvfp4_gemm(orc, qa, qb, 1, f"per-token x per-token {M}x{N}x{K}")


def test_nvfp4_gemm_dense_forward_full(orc):
    """The dense forward at the pages' shape: 2048 tokens x 2048 (per-token
    NVFP4) times an 8192 x 2048 weight with one scope scale; 384 sampled rows."""
    qa = orc.nvfp4_per_token(W.student_t_activations(2048, 2048, 83))
    w = W.bf16_bits(np.random.default_rng(84).normal(0, 0.02, (1, 8192, 2048)))
    wc, wb, _, _, ws = orc.nvfp4_gateup_pair(w, None)
    rng = np.random.default_rng(85)
    rows = np.concatenate([np.arange(64), rng.integers(0, 2048, 256), np.arange(1984, 2048)])
    check_nvfp4_gemm(orc, qa, (wc[0], wb[0], ws), 8192, "2048x8192x2048", row_sample=rows)


# ---------------------------------------------------------------------------
# Quantize + dequant in one pass
# ---------------------------------------------------------------------------

def check_qdq(orc, x: np.ndarray, fmt: int, name: str, codes_only_check=True):
    """Codes, scales and the BF16 dequant of the one-pass call against the
    oracle's quantize followed by its dequant; then the dequant-only call
    (no codes stored) must give the same BF16."""
    tag = "mxfp8" if fmt == mxq.MXQ_FMT_MXFP8_ROW else "nvfp4"
    announce(f"quantize-dequant {tag} {name} shape={x.shape}")
    xd = dev(x)
    r = api.quantize_dequant_bf16(fmt, xd)
    torch.cuda.synchronize()
    if fmt == mxq.MXQ_FMT_MXFP8_ROW:
        c, s_, y = orc.quantize_dequant_mxfp8_rowwise(x)
    else:
        c, s_, t, y = orc.quantize_dequant_nvfp4(x)
        assert_same(host(r.fp32_scales).view(np.uint32), t.view(np.uint32), f"{name} ts")
    assert_same(host(r.codes), c, f"{name} codes")
    assert_same(host(r.scales), s_, f"{name} scales")
    assert_same(host(r.dequant), y, f"{name} dequant")
    if codes_only_check:
        announce(f"quantize-dequant {tag} {name} dequant only")
        r2 = api.quantize_dequant_bf16(fmt, xd, keep_codes=False)
        torch.cuda.synchronize()
        assert r2.codes is None
        assert_same(host(r2.dequant), y, f"{name} dequant only")


@pytest.mark.parametrize("mode", W.MXFP8_MODES)
def test_qdq_mxfp8_config2_weight(orc, mode):
    """8192 x 2048 in every data mode (maxes: scale byte 247, the exact
    saturating path)."""
    check_qdq(orc, W.config2_weight(mode), mxq.MXQ_FMT_MXFP8_ROW, f"C2b {mode}")


@pytest.mark.parametrize("rows,cols", [(1, 32), (77, 96), (33, 2080), (160, 544), (5, 4128)])
def test_qdq_mxfp8_shapes(orc, rows, cols):
    """Ragged row counts and partial column strips."""
    check_qdq(orc, W.mode_boundary(-(-rows // 32) * 32, cols, rows)[:rows], mxq.MXQ_FMT_MXFP8_ROW,
              f"boundary {rows}x{cols}")


def test_qdq_mxfp8_exhaustive(orc):
    """Every finite BF16 value under every scale its block can have: every
    (code, scale) pair the dequant can meet in a rowwise copy."""
    check_qdq(orc, _mxfp8_exhaustive_input(), mxq.MXQ_FMT_MXFP8_ROW, "exhaustive rows")


def test_qdq_nvfp4_config3(orc):
    check_qdq(orc, W.config3(), mxq.MXQ_FMT_NVFP4, "C3 8192x2048")


@pytest.mark.parametrize("rows,cols", [(1, 16), (5, 48), (7, 768), (9, 1040), (6, 2048),
                                       (3, 2064), (4, 4096), (2, 4112)])
def test_qdq_nvfp4_shapes(orc, rows, cols):
    """Every register-resident chunk count, partial chunks and the re-reading
    path above 4096, on heavy-tailed and boundary rows."""
    check_qdq(orc, W.student_t_activations(rows, cols, rows * cols), mxq.MXQ_FMT_NVFP4,
              f"t3 {rows}x{cols}")
    check_qdq(orc, W.nvfp4_boundary(rows, cols, cols + 1), mxq.MXQ_FMT_NVFP4,
              f"boundary {rows}x{cols}", codes_only_check=False)


@pytest.mark.parametrize("rows,cols", [(8193, 1040), (8200, 2048), (16385, 2064)])
def test_qdq_nvfp4_shapes_one_wave_rows(orc, rows, cols):
    """Grids above the row counts that split each row over two wavefronts:
    one wavefront per row, full and partial rows."""
    check_qdq(orc, W.student_t_activations(rows, cols, rows * cols), mxq.MXQ_FMT_NVFP4,
              f"t3 {rows}x{cols}")


def test_qdq_nvfp4_ties_and_range(orc):
    """Exact ties of both rounding steps, scales across the whole range (the
    binary64 paths of quantize and dequant) and every token amax."""
    check_qdq(orc, _tie_sweep(), mxq.MXQ_FMT_NVFP4, "tie sweep")
    check_qdq(orc, _wide_range_rows(300, 256, 7), mxq.MXQ_FMT_NVFP4, "wide range")
    mags = np.arange(1, 0x7F80, dtype=np.uint32)
    rng = np.random.default_rng(45)
    frac = rng.integers(0, 0x8000, (mags.size, 32)).astype(np.uint32)
    x = (frac * mags[:, None]) // 0x8000
    x[:, 0] = mags
    x |= (rng.integers(0, 2, x.shape).astype(np.uint32) << 15)
    check_qdq(orc, x.astype(np.uint16), mxq.MXQ_FMT_NVFP4, "every token amax",
              codes_only_check=False)


# ---------------------------------------------------------------------------
# Grouped quantize fused with dispatch (reads the unpermuted tokens)
# ---------------------------------------------------------------------------

def check_dispatch(orc, tokens, row_tokens, token_rows, off, name):
    """Both dispatch outputs, every segment and every row, against the oracle
    on the gathered rows tokens[row_tokens] (the definition of the fused
    call)."""
    R, K = row_tokens.size, tokens.shape[1]
    announce(f"dispatch {name} T={tokens.shape[0]} R={R} K={K} G={off.size - 1}")
    td = dev(tokens)
    d8 = api.dispatch_quantize_mxfp8(td, torch.from_numpy(row_tokens).cuda(),
                                     torch.from_numpy(off).cuda())
    d4 = api.dispatch_quantize_nvfp4(td, torch.from_numpy(token_rows).cuda(), R)
    torch.cuda.synchronize()
    x = tokens[row_tokens]
    G = off.size - 1
    P = host(d8.col_scale_offsets)
    counts = [(int(off[e + 1]) - int(off[e]) + 31) // 32 for e in range(G)]
    assert list(P) == list(np.concatenate([[0], np.cumsum(counts)]))
    rc, rs, cc, cs = host(d8.row_codes), host(d8.row_scales), host(d8.col_codes), \
        host(d8.col_scales)
    for e in range(G):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        seg = x[a:b]
        oc, os_, _ = orc.mxfp8_colwise_grouped(seg, np.array([0, b - a], np.int64))
        assert_same(cc[a:b], oc, f"{name} seg{e} col codes")
        assert_same(cs[P[e]:P[e + 1]], os_, f"{name} seg{e} col scales")
    orow, orows = orc.mxfp8_rowwise(x)
    assert_same(rc, orow, f"{name} row codes")
    assert_same(rs, orows, f"{name} row scales")
    del orow, orows, rc, rs, cc, cs
    nc, nb, ns = orc.nvfp4_per_token(x)
    assert_same(host(d4.codes), nc, f"{name} nvfp4 codes")
    assert_same(host(d4.block_scales), nb, f"{name} nvfp4 bs")
    assert_same(host(d4.fp32_scales).view(np.uint32), ns.view(np.uint32), f"{name} nvfp4 s")
    return d8, d4


def test_dispatch_small_with_dropped_copies(orc):
    """300 tokens, top-3 of 8 experts, 30% of the copies dropped (a capacity
    limit): token_rows holds -1 for them and rows only for the kept copies."""
    row_tokens, token_rows, off = W.dispatch_maps(300, 8, 3, seed=11, drop=0.3)
    tokens = W.student_t_activations(300, 256, 12)
    check_dispatch(orc, tokens, row_tokens, token_rows, off, "small dropped")


def test_dispatch_shapes(orc):
    """Short rows (K = 96: partial NVFP4 row, one partial MXFP8 strip), long
    rows (K = 4160: the two-pass NVFP4 kernel) and empty experts."""
    row_tokens, token_rows, off = W.dispatch_maps(200, 40, 2, seed=13)
    check_dispatch(orc, W.student_t_activations(200, 96, 14), row_tokens, token_rows, off,
                   "K96 40 experts")
    row_tokens, token_rows, off = W.dispatch_maps(70, 6, 2, seed=15)
    check_dispatch(orc, W.student_t_activations(70, 4160, 16), row_tokens, token_rows, off,
                   "K4160")


def test_dispatch_config5_full(orc):
    """The grouped workload read from its 32,768 unpermuted tokens (top-8 of
    128): every segment and every row of both outputs."""
    tokens, row_tokens, token_rows, off = W.config5_dispatch()
    check_dispatch(orc, tokens, row_tokens, token_rows, off, "config5")


# ---------------------------------------------------------------------------
# Measurement reference (the copy floor the benchmark times beside each
# workload): its output is its stated definition, so no load is optimized away
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n_r,n_w", [(1, 1), (300, 300), (1000, 257), (4096, 1024),
                                     (37, 1000), (5, 4096), (70000, 20000), (1000, 100),
                                     (5000, 300), (9000, 1000)])
def test_copy_floor_definition(n_r, n_w):
    rng = np.random.default_rng(n_r * 7 + n_w)
    src = rng.integers(0, 256, (n_r, 16), dtype=np.uint8)
    announce(f"copy floor n_r={n_r} n_w={n_w}")
    dst = torch.empty((n_w, 16), dtype=torch.uint8, device="cuda")
    mxq.mxq_copy_floor(dev(src), 16 * n_r, dst, 16 * n_w)
    torch.cuda.synchronize()
    if n_r >= n_w:
        want = src[:n_w].copy()
        for i in range(1, -(-n_r // n_w)):
            part = src[i * n_w:(i + 1) * n_w]
            want[:part.shape[0]] ^= part
    else:
        m = (n_r << 32) // n_w
        want = src[[(j * m) >> 32 for j in range(n_w)]]
    assert_same(host(dst), want, "copy floor")


# ---------------------------------------------------------------------------
# Error paths: nothing launched, nothing written
# ---------------------------------------------------------------------------

def test_errors_leave_outputs_untouched():
    x = dev(W.config1())
    rows, cols = 256, 512
    rc = torch.full((rows, cols), 0xA5, dtype=torch.uint8, device="cuda")
    rs = torch.full((rows, cols // 32), 0xA5, dtype=torch.uint8, device="cuda")
    cc = torch.full((rows, cols), 0xA5, dtype=torch.uint8, device="cuda")
    cs = torch.full((rows // 32, cols), 0xA5, dtype=torch.uint8, device="cuda")
    host_buf = np.zeros((rows, cols), np.uint8)
    announce("error paths")
    cases = [
        (mxq.MXQ_ERR_ALIGN, (x.data_ptr() + 2, rows, cols, rc, rs, cc, cs)),
        (mxq.MXQ_ERR_DEVICE, (x, rows, cols, host_buf.ctypes.data, rs, cc, cs)),
        (mxq.MXQ_ERR_ALIAS, (x, rows, cols, rc, rs, rc, cs)),
        (mxq.MXQ_ERR_ALIAS, (x, rows, cols, x.data_ptr(), rs, cc, cs)),
        (mxq.MXQ_ERR_SHAPE, (x, rows, cols - 16, rc, rs, cc, cs)),
        (mxq.MXQ_ERR_OFFSETS, (x, rows, cols, rc, None, cc, cs)),
        (mxq.MXQ_ERR_NULL, (None, rows, cols, rc, rs, cc, cs)),
    ]
    for status, args in cases:
        with pytest.raises(mxq.MXQError) as ei:
            mxq.mxq_mxfp8_quantize_rowcol(*args)
        assert ei.value.status == status, (status, ei.value)
    torch.cuda.synchronize()
    for t in (rc, rs, cc, cs):
        assert bool((t == 0xA5).all())
    # A valid call afterwards works and writes.
    mxq.mxq_mxfp8_quantize_rowcol(x, rows, cols, rc, rs, cc, cs)
    torch.cuda.synchronize()
    assert not bool((rs == 0xA5).all())


def test_errors_weight_gradient_pair_leave_outputs_untouched():
    """Rejected calls of the grouped transposed quantize and of the grouped
    weight-gradient GEMM (aliased outputs, host memory, misalignment, bad
    shape) launch nothing: canary-filled outputs keep every byte."""
    R, cols, G = 96, 64, 2
    x = dev(W.mode_random(R, cols, 33))
    off = torch.tensor([0, 40, R], dtype=torch.int64, device="cuda")
    pitch = api.grouped_colt_pitch(R, G)
    fill = lambda n, dt=torch.uint8: torch.full((n,), 0xA5 if dt == torch.uint8 else -7,
                                                dtype=dt, device="cuda")
    rc, rs, ct, st, P = (fill(R * cols), fill(R * cols // 32), fill(cols * pitch),
                         fill(cols * pitch // 32), fill(G + 1, torch.int64))
    host_buf = np.zeros(cols * pitch // 32, np.uint8)
    f = mxq.mxq_mxfp8_grouped_quantize_rowcol_t
    announce("error paths: weight-gradient pair")
    cases = [
        (mxq.MXQ_ERR_ALIAS, (x, R, cols, off, G, ct, rs, ct, st, P)),
        (mxq.MXQ_ERR_DEVICE, (x, R, cols, off, G, rc, rs, ct, host_buf.ctypes.data, P)),
        (mxq.MXQ_ERR_ALIGN, (x, R, cols, off, G, rc, rs, ct, st.data_ptr() + 2, P)),
        (mxq.MXQ_ERR_SHAPE, (x, R, cols - 16, off, G, rc, rs, ct, st, P)),
    ]
    for status, args in cases:
        with pytest.raises(mxq.MXQError) as ei:
            f(*args)
        assert ei.value.status == status, (status, ei.value)
    c = torch.full((G * cols * cols,), -7.0, dtype=torch.float32, device="cuda")
    a, sa = ct.view(cols, pitch), st.view(cols, pitch // 32)
    wcases = [
        (mxq.MXQ_ERR_ALIAS, (a, sa, c, sa, P, G, cols, cols, pitch, mxq.MXQ_OUT_F32, c)),
        (mxq.MXQ_ERR_SHAPE, (a, sa, a, sa, P, G, cols, cols, pitch - 64, mxq.MXQ_OUT_F32, c)),
        (mxq.MXQ_ERR_ARG, (a, sa, a, sa, P, G, cols, cols, pitch, 7, c)),
    ]
    for status, args in wcases:
        with pytest.raises(mxq.MXQError) as ei:
            mxq.mxq_mxfp8_grouped_wgrad(*args)
        assert ei.value.status == status, (status, ei.value)
    torch.cuda.synchronize()
    for t in (rc, rs, ct, st):
        assert bool((t == 0xA5).all())
    assert bool((P == -7).all()) and bool((c == -7.0).all())


def test_errors_buffer_too_small():
    """An array that ends before the call's extent is rejected when the array is
    its own allocation (hipMalloc).  Inside a caching-allocator segment only the
    segment's end is known, so the check guards the allocation, not the tensor."""
    rows, cols = 8192, 512
    need = rows * cols
    x = ExactBuffer(2 * need)
    small = ExactBuffer(need // 2)                 # row codes need `need` bytes
    full = [ExactBuffer(need), ExactBuffer(need // 32), ExactBuffer(need), ExactBuffer(need // 32)]
    try:
        if not (x.exact and small.exact and all(b.exact for b in full)):
            pytest.skip("runtime does not report exact allocation extents")
        announce("error paths: too-small buffers")
        rc, rs, cc, cs = (b.ptr for b in full)
        for args in [(x.ptr, rows, cols, small.ptr, rs, cc, cs),
                     (x.ptr, rows * 2, cols, rc, rs, cc, cs)]:
            with pytest.raises(mxq.MXQError) as ei:
                mxq.mxq_mxfp8_quantize_rowcol(*args)
            assert ei.value.status == mxq.MXQ_ERR_DEVICE
        torch.cuda.synchronize()
    finally:
        for b in [x, small] + full:
            b.free()


def test_errors_other_entry_points():
    """Rejected before launch: outputs overlapping the input, unknown formats,
    empty group lists.  (Too-small arrays: test_errors_buffer_too_small.)"""
    x = dev(W.config1())
    codes = torch.empty((256, 256), dtype=torch.uint8, device="cuda")
    bs = torch.empty((256, 32), dtype=torch.uint8, device="cuda")
    ts = torch.empty((256,), dtype=torch.float32, device="cuda")
    announce("error paths nvfp4/dequant/grouped")
    with pytest.raises(mxq.MXQError) as ei:
        mxq.mxq_nvfp4_quantize_per_token(x, 256, 512, x.data_ptr() + 4096, bs, ts)
    assert ei.value.status == mxq.MXQ_ERR_ALIAS
    out = torch.empty((256, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mxq.MXQError) as ei:
        mxq.mxq_dequantize_bf16(7, codes, bs, None, 1, 256, 512, out)
    assert ei.value.status == mxq.MXQ_ERR_ARG
    with pytest.raises(mxq.MXQError) as ei:
        mxq.mxq_grouped_quantize(mxq.MXQ_FMT_NVFP4, x, 256, 512,
                                 torch.zeros(3, dtype=torch.int64, device="cuda"), 0,
                                 {"codes": codes, "block_scales": bs, "token_scales": ts})
    assert ei.value.status == mxq.MXQ_ERR_SIZE
    with pytest.raises(mxq.MXQError) as ei:
        mxq.mxq_nvfp4_quantize_gateup_pair(x, x, 2, 128, 512, codes, bs, codes, bs, ts)
    assert ei.value.status == mxq.MXQ_ERR_ALIAS


def test_errors_newer_entry_points_write_nothing():
    """The fused, one-pass, variant and GEMM entry points reject aliasing,
    host memory and bad enums before any launch: their canary-filled outputs
    stay untouched."""
    x = dev(W.config1())                                    # 256 x 512 BF16
    rows, cols = 256, 512
    host_buf = np.zeros(rows * cols * 2, np.uint8)
    canary = lambda *shape, dt=torch.uint8: torch.full(shape, 0x5A if dt == torch.uint8 else 7,
                                                       dtype=dt, device="cuda")
    c8, s8 = canary(rows, cols), canary(rows, cols // 32)
    c4, b4, t4 = canary(rows, cols // 2), canary(rows, cols // 16), canary(rows, dt=torch.float32)
    y = canary(rows, cols, dt=torch.int16)
    g = canary(rows, rows, dt=torch.float32)
    announce("error paths: newer entry points")
    cases = [
        (mxq.MXQ_ERR_ALIAS, lambda: mxq.mxq_quantize_dequant_bf16(
            mxq.MXQ_FMT_NVFP4, x, rows, cols, c4, b4, t4, x)),
        (mxq.MXQ_ERR_DEVICE, lambda: mxq.mxq_quantize_dequant_bf16(
            mxq.MXQ_FMT_MXFP8_ROW, x, rows, cols, c8, s8, None, host_buf.ctypes.data)),
        (mxq.MXQ_ERR_ALIAS, lambda: mxq.mxq_mxfp8_quantize_ocp_floor(
            x, rows, cols, c8, s8, c8, s8)),
        (mxq.MXQ_ERR_ALIAS, lambda: mxq.mxq_mxfp8_quantize_rowcol_t(
            x, rows, cols, c8, s8, c8, s8)),
        (mxq.MXQ_ERR_ALIAS, lambda: mxq.mxq_nvfp4_quantize_per_token_approx(
            x, rows, cols, c4, c4, t4)),
        (mxq.MXQ_ERR_ALIAS, lambda: mxq.mxq_mxfp8_gemm(
            c8, s8, c8, s8, rows, rows, cols, mxq.MXQ_OUT_BF16, c8)),
        (mxq.MXQ_ERR_ARG, lambda: mxq.mxq_nvfp4_gemm(
            c4, b4, t4, 1, c4, b4, t4, rows, rows, rows, cols, 9, g)),
        (mxq.MXQ_ERR_DEVICE, lambda: mxq.mxq_nvfp4_gemm(
            c4, b4, t4, 1, host_buf.ctypes.data, b4, t4, rows, rows, rows, cols,
            mxq.MXQ_OUT_F32, g)),
        (mxq.MXQ_ERR_ALIAS, lambda: mxq.mxq_grouped_quantize_dispatch(
            mxq.MXQ_FMT_NVFP4, x, rows, cols, 1, c4, None, rows, None, 0,
            {"codes": c4, "block_scales": b4, "token_scales": t4})),
    ]
    for status, call in cases:
        with pytest.raises(mxq.MXQError) as ei:
            call()
        assert ei.value.status == status, (status, ei.value)
    torch.cuda.synchronize()
    for t, fill in ((c8, 0x5A), (s8, 0x5A), (c4, 0x5A), (b4, 0x5A), (y, 7)):
        assert bool((t == fill).all())
    assert bool((t4 == 7).all()) and bool((g == 7).all())


def test_grouped_malformed_offsets_stay_in_bounds():
    """Offsets are device data the host cannot validate: non-monotone or
    out-of-range offsets must not move any access out of bounds (the call
    completes; its bytes are meaningless).  Outputs are bracketed by canaries."""
    R, cols, G = 64, 64, 3
    x = dev(W.mode_random(R, cols, 5))
    off = torch.tensor([0, 1000, -5, 64], dtype=torch.int64, device="cuda")
    guard = 4096
    big = torch.full((R * cols + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    cs_big = torch.full(((R // 32 + G) * cols + 2 * guard,), 0x5A, dtype=torch.uint8,
                        device="cuda")
    rc = big[guard:guard + R * cols]
    cc = torch.empty(R * cols, dtype=torch.uint8, device="cuda")
    rs = torch.empty(R * cols // 32, dtype=torch.uint8, device="cuda")
    cs = cs_big[guard:guard + (R // 32 + G) * cols]
    P = torch.empty(G + 1, dtype=torch.int64, device="cuda")
    announce("grouped malformed offsets")
    mxq.mxq_grouped_quantize(mxq.MXQ_FMT_MXFP8_ROWCOL, x, R, cols, off, G,
                             {"row_codes": rc, "row_scales": rs, "col_codes": cc,
                              "col_scales": cs, "col_scale_offsets": P})
    torch.cuda.synchronize()
    assert bool((big[:guard] == 0x5A).all()) and bool((big[-guard:] == 0x5A).all())
    assert bool((cs_big[:guard] == 0x5A).all()) and bool((cs_big[-guard:] == 0x5A).all())


def test_weight_gradient_pair_malformed_offsets_stay_in_bounds():
    """The weight-gradient pair under malformed device offsets: overlapping
    segments whose blocks exceed the padded capacity (P[G] past pitch / 32),
    out-of-range and decreasing offsets, then block offsets past the pitch or
    negative for the GEMM.  Every output is bracketed by canaries; the calls
    complete and nothing outside the outputs changes (the bytes inside are
    meaningless)."""
    R, cols, G, guard = 1024, 64, 4, 4096
    x = dev(W.mode_random(R, cols, 31))
    pitch = api.grouped_colt_pitch(R, G)
    fill = 0x5A

    def guarded(n, dt=torch.uint8, v=fill):
        big = torch.full((n + 2 * guard,), v, dtype=dt, device="cuda")
        return big, big[guard:guard + n]

    for off_list in ([0, R, 0, R, 0], [0, 1000, -5, 64, 10 ** 12]):
        off = torch.tensor(off_list, dtype=torch.int64, device="cuda")
        bufs = [guarded(cols * pitch), guarded(cols * pitch // 32), guarded(R * cols),
                guarded(R * cols // 32), guarded(G + 1, torch.int64, -1)]
        ct, st, rc, rs, P = (b[1] for b in bufs)
        announce(f"weight-gradient pair malformed offsets {off_list}")
        mxq.mxq_mxfp8_grouped_quantize_rowcol_t(x, R, cols, off, G, rc, rs, ct, st, P)
        torch.cuda.synchronize()
        for big, _ in bufs:
            v = -1 if big.dtype == torch.int64 else fill
            assert bool((big[:guard] == v).all()) and bool((big[-guard:] == v).all())
    a = ct.view(cols, pitch)
    sa = st.view(cols, pitch // 32)
    bad = torch.tensor([0, 10 ** 9, -7, 3, pitch // 32], dtype=torch.int64, device="cuda")
    cbig, c = guarded(G * cols * cols * 4, torch.uint8)
    announce("weight gradient malformed block offsets")
    mxq.mxq_mxfp8_grouped_wgrad(a, sa, a, sa, bad, G, cols, cols, pitch, mxq.MXQ_OUT_F32, c)
    torch.cuda.synchronize()
    assert bool((cbig[:guard] == fill).all()) and bool((cbig[-guard:] == fill).all())
    cf = c.view(torch.float32).view(G, cols, cols)
    assert bool((cf[1] == 0).all()) and bool((cf[2] == 0).all())   # empty after clamping


def test_dispatch_malformed_maps_stay_in_bounds():
    """The index maps are device data: token_rows entries outside the output
    rows are skipped and row_tokens entries outside the tokens are clamped,
    so no access leaves the arrays (the bytes are meaningless).  Outputs are
    bracketed by canaries."""
    T, cols, R = 16, 64, 40
    x = dev(W.mode_random(T, cols, 21))
    guard = 4096
    token_rows = torch.tensor([[-1, R, 10 ** 9, 3]] * T, dtype=torch.int64, device="cuda")
    c_big = torch.full((R * cols // 2 + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    b_big = torch.full((R * cols // 16 + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    s_big = torch.full((R + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    announce("dispatch malformed token_rows")
    mxq.mxq_grouped_quantize_dispatch(
        mxq.MXQ_FMT_NVFP4, x, T, cols, 4, token_rows, None, R, None, 0,
        {"codes": c_big[guard:guard + R * cols // 2],
         "block_scales": b_big[guard:guard + R * cols // 16],
         "token_scales": s_big[guard:guard + R]})
    torch.cuda.synchronize()
    for big, fill in ((c_big, 0x5A), (b_big, 0x5A), (s_big, 7.0)):
        assert bool((big[:guard] == fill).all()) and bool((big[-guard:] == fill).all())
    row_tokens = torch.tensor([-3, 10 ** 9] * (R // 2), dtype=torch.int64, device="cuda")
    off = torch.tensor([0, 7, R], dtype=torch.int64, device="cuda")
    G = 2
    rc_big = torch.full((R * cols + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    cs_big = torch.full(((R // 32 + G) * cols + 2 * guard,), 0x5A, dtype=torch.uint8,
                        device="cuda")
    announce("dispatch malformed row_tokens")
    mxq.mxq_grouped_quantize_dispatch(
        mxq.MXQ_FMT_MXFP8_ROWCOL, x, T, cols, 0, None, row_tokens, R, off, G,
        {"row_codes": rc_big[guard:guard + R * cols],
         "row_scales": torch.empty(R * cols // 32, dtype=torch.uint8, device="cuda"),
         "col_codes": torch.empty(R * cols, dtype=torch.uint8, device="cuda"),
         "col_scales": cs_big[guard:guard + (R // 32 + G) * cols],
         "col_scale_offsets": torch.empty(G + 1, dtype=torch.int64, device="cuda")})
    torch.cuda.synchronize()
    for big in (rc_big, cs_big):
        assert bool((big[:guard] == 0x5A).all()) and bool((big[-guard:] == 0x5A).all())


def test_dispatch_many_experts(orc):
    """300 experts (past the in-kernel prefix limit of 256 segments): every
    segment and row of both dispatch outputs."""
    row_tokens, token_rows, off = W.dispatch_maps(600, 300, 3, seed=23)
    tokens = W.student_t_activations(600, 256, 24)
    check_dispatch(orc, tokens, row_tokens, token_rows, off, "300 experts")


def test_dispatch_mxfp8_single_copy(orc):
    """Rowwise-only (the dense kernel with a row gather) and columnwise-only
    dispatch calls give the same bytes as the two-copy call."""
    row_tokens, token_rows, off = W.dispatch_maps(500, 16, 4, seed=19)
    tokens = W.student_t_activations(500, 512, 20)
    d8, _ = check_dispatch(orc, tokens, row_tokens, token_rows, off, "single copy ref")
    R, cols, G = row_tokens.size, 512, off.size - 1
    td, rt, od = dev(tokens), torch.from_numpy(row_tokens).cuda(), torch.from_numpy(off).cuda()
    rc = torch.empty(R * cols, dtype=torch.uint8, device="cuda")
    rs = torch.empty(R * cols // 32, dtype=torch.uint8, device="cuda")
    announce("dispatch rowwise only")
    mxq.mxq_grouped_quantize_dispatch(mxq.MXQ_FMT_MXFP8_ROWCOL, td, 500, cols, 0, None, rt, R,
                                      None, 0, {"row_codes": rc, "row_scales": rs})
    cc = torch.empty(R * cols, dtype=torch.uint8, device="cuda")
    cs = torch.empty((R // 32 + G) * cols, dtype=torch.uint8, device="cuda")
    P = torch.empty(G + 1, dtype=torch.int64, device="cuda")
    announce("dispatch columnwise only")
    mxq.mxq_grouped_quantize_dispatch(mxq.MXQ_FMT_MXFP8_ROWCOL, td, 500, cols, 0, None, rt, R,
                                      od, G, {"col_codes": cc, "col_scales": cs,
                                              "col_scale_offsets": P})
    torch.cuda.synchronize()
    assert_same(host(rc).reshape(R, cols), host(d8.row_codes), "row-only codes")
    assert_same(host(rs).reshape(R, cols // 32), host(d8.row_scales), "row-only scales")
    assert_same(host(cc).reshape(R, cols), host(d8.col_codes), "col-only codes")
    used = int(off.size and host(d8.col_scale_offsets)[-1])      # rows past P[G] are unused
    assert_same(host(cs).reshape(-1, cols)[:used], host(d8.col_scales)[:used],
                "col-only scales")
    assert_same(host(P), host(d8.col_scale_offsets), "col-only offsets")


# ---------------------------------------------------------------------------
# Seeded random shapes and value laws across every kernel path
# ---------------------------------------------------------------------------

def _random_values(rng, rows, cols):
    """One of several value laws: normal at a random scale, heavy tails,
    log-uniform magnitudes over many binades, sparse (zeros), or constant
    rows; BF16 bits."""
    kind = int(rng.integers(0, 5))
    if kind == 0:
        v = rng.standard_normal((rows, cols)) * 2.0 ** float(rng.integers(-40, 40))
    elif kind == 1:
        v = rng.standard_t(2, (rows, cols)) * 0.5
    elif kind == 2:
        v = np.exp2(rng.uniform(-60, 60, (rows, cols))) * rng.choice([-1.0, 1.0], (rows, cols))
    elif kind == 3:
        v = rng.standard_normal((rows, cols))
        v[rng.random((rows, cols)) < 0.7] = 0.0
    else:
        v = np.repeat(rng.standard_normal((rows, 1)), cols, axis=1)
    return W.bf16_bits(np.clip(v, -3.38e38, 3.38e38))


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_all_paths(orc, seed):
    """MXFP8 row+col, per-token NVFP4 and both one-pass quantize + dequant
    calls on seeded random shapes: row counts on both sides of the grid-size
    switches, column counts that leave partial tiles, strips and blocks."""
    rng = np.random.default_rng(1000 + seed)
    for _ in range(3):
        rows = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(7000, 9500))]))
        cols16 = int(rng.integers(1, 260)) * 16
        x = _random_values(rng, rows, cols16)
        check_nvfp4(orc, x, f"random {rows}x{cols16}")
        check_qdq(orc, x, mxq.MXQ_FMT_NVFP4, f"random {rows}x{cols16}", codes_only_check=False)
        rows32 = max(32, rows - rows % 32)
        cols32 = int(rng.integers(1, 130)) * 32
        y = _random_values(rng, rows32, cols32)
        check_mxfp8(orc, y, f"random {rows32}x{cols32}")
        check_qdq(orc, y, mxq.MXQ_FMT_MXFP8_ROW, f"random {rows32}x{cols32}",
                  codes_only_check=False)


@pytest.mark.parametrize("seed", range(4))
def test_random_grouped_segments(orc, seed):
    """Grouped MXFP8 row+col and NVFP4 on seeded random segmentations: empty
    segments, segments of 1..31 rows, exact multiples of 32 and long ones,
    random column counts (partial strips), every segment checked."""
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.integers(1, 40))
    kinds = rng.integers(0, 4, G)
    sizes = np.where(kinds == 0, 0,
                     np.where(kinds == 1, rng.integers(1, 32, G),
                              np.where(kinds == 2, 32 * rng.integers(1, 5, G),
                                       rng.integers(33, 700, G))))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    if off[-1] == 0:
        off[-1] = 1
    cols = int(rng.integers(1, 80)) * 32
    x = _random_values(rng, int(off[-1]), cols)
    check_grouped(orc, x, off, f"random G={G} cols={cols}")
    check_grouped_rowcolt(orc, x, off, f"random G={G} cols={cols}")


@pytest.mark.parametrize("seed", range(3))
def test_random_weight_gradient(orc, seed):
    """The grouped weight gradient on seeded random segmentations (empty,
    short, exact and long segments) and random M, N (partial 256-tiles):
    every expert against the oracle's product of the padded operands, to the
    GEMM bound; empty experts give zeros."""
    rng = np.random.default_rng(3000 + seed)
    G = int(rng.integers(1, 24))
    kinds = rng.integers(0, 4, G)
    sizes = np.where(kinds == 0, 0,
                     np.where(kinds == 1, rng.integers(1, 32, G),
                              np.where(kinds == 2, 32 * rng.integers(1, 5, G),
                                       rng.integers(33, 700, G))))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    if off[-1] == 0:
        off[-1] = 1
    R = int(off[-1])
    M, N = int(rng.integers(1, 12)) * 32, int(rng.integers(1, 12)) * 32
    # Products kept inside the fp32 range (as in the dense GEMM tests): normal
    # and heavy-tailed values at a random scale of 2^-10 .. 2^10.
    def values(rows, cols):
        v = (rng.standard_normal((rows, cols)) if rng.integers(0, 2) else
             rng.standard_t(3, (rows, cols))) * 2.0 ** float(rng.integers(-10, 11))
        return W.bf16_bits(v)
    dy, x = values(R, M), values(R, N)
    announce(f"random wgrad G={G} R={R} M={M} N={N}")
    gd = api.mxfp8_grouped_colwise_t(dev(dy), dev(off))
    gx = api.mxfp8_grouped_colwise_t(dev(x), dev(off))
    c = api.mxfp8_grouped_wgrad(gd, gx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = c.cpu().numpy().astype(np.float64)
    dct, dst, P = padded_colt(orc, dy, off)
    xct, xst, _ = padded_colt(orc, x, off)
    for e in range(G):
        k0, k1 = 32 * int(P[e]), 32 * int(P[e + 1])
        if k0 == k1:
            assert np.all(got[e] == 0), f"empty expert {e}"
            continue
        C, S = orc.mxfp8_gemm(dct[:, k0:k1], dst[:, k0 // 32:k1 // 32],
                              xct[:, k0:k1], xst[:, k0 // 32:k1 // 32])
        assert np.all(np.abs(got[e] - C) <= (GEMM_REL + (k1 - k0) * 2.0 ** -24) * S), \
            f"expert {e}"
