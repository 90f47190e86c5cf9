"""Planted mistakes in a copy of the oracle must fail the pin suite.

Each mutation below is a plausible slip (a dropped term or factor, a wrong tie
rule, a wrong index, a swapped nibble order, a dropped sign, a reciprocal
instead of a division).  The test compiles a mutated copy of the oracle's C
source into a temporary library, points the oracle at it through
MXQ_ORACLE_LIB, and runs tests/test_oracle_pins.py against it in a child
process: the child must fail.  CPU only.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

MUTATIONS = {
    "tie_to_odd": ("if (k % 2 == 1)\n                k++;", "if (k % 2 == 0)\n                k++;"),
    "e8m0_strict": ("if (A <= ldexp(448.0, e))", "if (A < ldexp(448.0, e))"),
    "e8m0_ceil_log2": ("if (A <= ldexp(448.0, e))", "if (A <= ldexp(256.0, e))"),
    "scale_reciprocal": ("return a / divisor;", "return a * (1.0f / divisor);"),
    "dropped_six": ("oracle_e4m3_nearest(A, 6.0 * sd)", "oracle_e4m3_nearest(A, sd)"),
    "nibble_swap": ("(uint8_t)(c[0] | (c[1] << 4))", "(uint8_t)(c[1] | (c[0] << 4))"),
    "half_column_block": ("for (int64_t r = r0; r < r1; r++) {\n            double a",
                          "for (int64_t r = r0; r < r0 + (r1 - r0) / 2; r++) {\n            double a"),
    "e2m1_sign_dropped": ("(signbit(x) ? 0x8 : 0)", "0"),
    "dequant_drops_block_scale": (
        "oracle_e4m3_value(block_scales[i * (cols / 16) + k / 16]) * s", "s"),
    "bf16_truncates": ("double n = nearbyint(ldexp(a, 7 - e));", "double n = floor(ldexp(a, 7 - e));"),
    "zero_block_not_zero": ("(d > 0.0) ? oracle_e2m1_nearest(v, d * sd) : 0",
                            "oracle_e2m1_nearest(v, d * sd)"),
    "row_block_offset": ("x[i * cols + j * 32 + k]", "x[i * cols + j * 16 + k]"),
    "colwise_dequant_neighbour_scale": ("oracle_e8m0_value(scales[(i / 32) * cols + k])",
                                        "oracle_e8m0_value(scales[(i / 32) * cols + (k ^ 1)])"),
    "dequant_nvfp4_first_fp32_scale": ("(double)fp32_scales[i / rows_per_scale]",
                                       "(double)fp32_scales[0]"),
    "scoped_row_swap": ("float s, uint8_t *codes, uint8_t *block_scales)\n{\n"
                        "#pragma omp parallel for schedule(static)\n"
                        "    for (int64_t t = 0; t < rows; t++)\n"
                        "        nvfp4_row(x + t * cols,",
                        "float s, uint8_t *codes, uint8_t *block_scales)\n{\n"
                        "#pragma omp parallel for schedule(static)\n"
                        "    for (int64_t t = 0; t < rows; t++)\n"
                        "        nvfp4_row(x + (t ^ 1) * cols,"),
}


def _build(name, tmp):
    src = open(oracle._SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, name
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(mutated)
    return oracle.build(src=path, out=os.path.join(tmp, f"lib{name}.so"))


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(4) as ex:
            libs = dict(zip(MUTATIONS, ex.map(lambda n: _build(n, tmp), MUTATIONS)))

        def run(name):
            env = dict(os.environ, MXQ_ORACLE_LIB=libs[name], OMP_NUM_THREADS="2")
            r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                                os.path.join(HERE, "test_oracle_pins.py")],
                               env=env, capture_output=True, text=True, timeout=600)
            return name, r.returncode

        with ThreadPoolExecutor(4) as ex:
            results = dict(ex.map(run, MUTATIONS))
    survived = [n for n, rc in results.items() if rc == 0]
    assert not survived, f"mutations not caught by any pin: {survived}"
