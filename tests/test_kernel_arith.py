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
