"""Build libmxq.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m nvfp4_block_scaled_amax_amd.build

One hipcc invocation compiles every source under csrc/ into
``nvfp4_block_scaled_amax_amd/libmxq.so``.  Packed-FP32 instruction selection
is disabled (-packed-fp32-ops); division and square root stay IEEE (no
fast-math); FP32 denormals are kept.  IEEE mode is off (-mno-amdgpu-ieee,
which requires -fno-honor-nans): it only changes how min/max treat NaN
operands, so |x| folds into max as a source modifier; NaN inputs are outside
the quantizers' contract and no kernel produces one from finite inputs.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxq.so")
ARCH = os.environ.get("MXQ_OFFLOAD_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + \
        sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def command(out: str = LIB, extra_flags=(), opt: str = "-O3"):
    """The hipcc command.  extra_flags: more flags (the host-sanitizer test
    passes host-only sanitizer flags, each behind -Xarch_host)."""
    return ["hipcc", f"--offload-arch={ARCH}", opt, "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fno-honor-nans", "-mno-amdgpu-ieee", *extra_flags,
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *sources(), "-o", out]


def build(verbose: bool = False, out: str = LIB, extra_flags=(), opt: str = "-O3") -> str:
    cmd = command(out + ".tmp", extra_flags, opt)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    noise = ("packed-fp32-ops", "is not a recognized feature")
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if ln.strip() and not any(n in ln for n in noise)]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
