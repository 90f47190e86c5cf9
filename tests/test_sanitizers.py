"""Host code under AddressSanitizer and UBSan, on the CPU (no GPU is used).

Two instrumented builds, each exercised in a child process that preloads the
sanitizer runtime (the Python interpreter itself is not instrumented):
  - the oracle (oracle/mxq_oracle.c, gcc -fsanitize=address,undefined), run
    through the whole pin suite via MXQ_ORACLE_LIB;
  - libmxq with host-only instrumentation (each -fsanitize= behind
    -Xarch_host, so no GPU code is built with it), run through the C-ABI
    validation tests via MXQ_LIB_PATH: every argument check, size limit and
    status path of the host side.
Any sanitizer report aborts the child (-fno-sanitize-recover=all), which fails
the test."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

import oracle
from nvfp4_block_scaled_amax_amd import build as mxq_build

HERE = os.path.dirname(os.path.abspath(__file__))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1", "OMP_NUM_THREADS": "2"}


def _run(env, test_file, check_maps):
    probe = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r); " % (os.path.dirname(HERE), HERE)
             + check_maps)
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu and not slow", os.path.join(HERE, test_file)],
                       env=env, capture_output=True, text=True, timeout=1800)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


@pytest.mark.slow
def test_oracle_under_asan_ubsan():
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    assert os.path.exists(libasan), libasan
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.build(out=os.path.join(tmp, "libmxq_oracle_san.so"),
                           extra_flags=("-fsanitize=address,undefined",
                                        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                                        "-g"))
        env = dict(os.environ, LD_PRELOAD=libasan, MXQ_ORACLE_LIB=lib, **SAN_ENV)
        check = ("import oracle; oracle.lib(); m = open('/proc/self/maps').read(); "
                 "assert 'libasan' in m and 'libmxq_oracle_san' in m, 'not instrumented'")
        _run(env, "test_oracle_pins.py", check)


@pytest.mark.slow
def test_host_abi_under_asan_ubsan():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not found")
    flags = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-shared-libsan", "-fno-omit-frame-pointer", "-g"):
        flags += ["-Xarch_host", f]
    with tempfile.TemporaryDirectory() as tmp:
        lib = mxq_build.build(out=os.path.join(tmp, "libmxq_san.so"), extra_flags=flags,
                              opt="-O1")
        env = dict(os.environ, LD_PRELOAD=rt[-1], MXQ_LIB_PATH=lib, **SAN_ENV)
        check = ("import nvfp4_block_scaled_amax_amd as m; m.lib(); "
                 "s = open('/proc/self/maps').read(); "
                 "assert 'libclang_rt.asan' in s and 'libmxq_san' in s, 'not instrumented'")
        _run(env, "test_abi_cpu.py", check)
