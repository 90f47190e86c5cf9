"""Host checks of arithmetic identities the HIP kernels rely on (no GPU).

The per-token NVFP4 kernels compute the FP32 scale s = fp32(A / 2688) of a
BF16 token amax A (the NVFP4 format paragraph of "Miles: end-to-end MXFP8 and
per-token NVFP4 RL on Blackwell": 2688 = 6 * 448, the largest E2M1 value
times the largest E4M3 value) without a division instruction, as
q0 = fp32(A * R), R = fp32(1 / 2688), then fma(fma(-q0, 2688, A), R, q0).
This checks, in exact rational arithmetic with binary32 round-to-nearest-even
at every step (an FMA rounds once), that the sequence gives the correctly
rounded quotient for every finite non-negative BF16 value.
"""
from fractions import Fraction as F

from exact_spec import bf16_frac, rn_binary32


def test_token_scale_division_sequence_is_exact():
    R = rn_binary32(F(1, 2688))
    assert R == F(0x1861862, 1 << 36), "fp32(1/2688) is 0x1.861862p-12"
    bad = []
    for bits in range(0, 0x7F80):
        A = bf16_frac(bits)
        want = rn_binary32(A / 2688)
        q0 = rn_binary32(A * R)
        rem = rn_binary32(-q0 * 2688 + A)
        got = rn_binary32(rem * R + q0)
        if got != want:
            bad.append(bits)
    assert not bad, f"{len(bad)} BF16 values differ, first {hex(bad[0])}"


def _bf16_around(T):
    """The BF16 values within two units of the last place of T > 0."""
    from exact_spec import floor_log2
    e = max(floor_log2(T), -126)
    ulp = F(2) ** (e - 7)
    n = T // ulp
    return [k * ulp for k in (n - 1, n, n + 1, n + 2) if k > 0]


def test_midpoint_fma_decision_is_exact():
    """The per-token and export kernels settle a bracket that straddles a
    rounding midpoint with one FMA, t = fma(m c, s, -a): the sign of t must be
    the sign of the exact m c s - a, and t == 0 exactly at a tie.  Here m runs
    over every E2M1 midpoint with c over every positive E4M3 value (codes), and
    over 3 (dec(k) + dec(k + 1)) for every adjacent E4M3 pair with c = 1 (block
    scales, 6 times the midpoint); s over FP32 scales of the fast path (at
    least 2^-101): token scales fp32(A / 2688) of assorted BF16 amaxes, the
    path's smallest scale and the largest scale a BF16 amax gives; a over the
    BF16 values around m c s.  The FMA is modelled as one binary32
    round-to-nearest-even of the exact value, denormals kept."""
    import random
    from exact_spec import E4M3_POS, E2M1_POS
    rng = random.Random(5)
    amaxes = [bf16_frac(b) for b in
              [rng.randrange(0x0080, 0x7F80) for _ in range(14)] + [0x3F80, 0x4228, 0x7F7F]]
    scales = {rn_binary32(A / 2688) for A in amaxes} | {F(2) ** -101}
    scales = sorted(s for s in scales if s >= F(2) ** -101)
    mids = [(E2M1_POS[k] + E2M1_POS[k + 1]) / 2 for k in range(7)]
    pairs = [(m, c) for m in mids for c in E4M3_POS[1:]]
    pairs += [(3 * (E4M3_POS[k] + E4M3_POS[k + 1]), F(1)) for k in range(126)]
    checked = 0
    for m, c in pairs:
        mc = m * c
        assert rn_binary32(mc) == mc, (m, c)           # m c is exact in FP32
        for s in scales:
            T = mc * s
            for a in _bf16_around(T):
                diff = T - a
                assert diff == 0 or abs(diff) >= F(2) ** -135, (m, c, s, a)
                t = rn_binary32(diff)
                assert (t > 0) == (diff > 0) and (t < 0) == (diff < 0), (m, c, s, a)
                checked += 1
    assert checked > 50000
