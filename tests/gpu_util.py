"""Helpers for the GPU tests: moving uint16/uint8 numpy arrays to and from the
device and announcing each GPU step (written straight to the process's stderr
so that it survives pytest's capture if the run ends abruptly)."""
import sys

import numpy as np
import torch

import nvfp4_block_scaled_amax_amd as mxq


def announce(msg: str):
    sys.__stderr__.write(f"[gpu-step] {msg}\n")
    sys.__stderr__.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> contiguous device tensor (uint16 travels as int16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.int16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def first_mismatch(got: np.ndarray, want: np.ndarray, what: str):
    """An assertion message naming the first differing index."""
    bad = np.argwhere(got != want)
    if bad.size == 0:
        return None
    i = tuple(bad[0])
    return f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]!r} want {want[i]!r}"


def assert_same(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    msg = first_mismatch(got, want, what)
    assert msg is None, msg


def hip_runtime():
    """The HIP runtime already loaded in this process (torch's), via ctypes."""
    import ctypes
    for line in open("/proc/self/maps"):
        if "libamdhip64" in line:
            return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("no HIP runtime mapped")


class ExactBuffer:
    """A device buffer from hipMalloc of exactly `nbytes` (not a sub-range of a
    caching-allocator segment), for tests of the library's extent checks.
    `exact` tells whether the runtime reports the allocation's extent as
    exactly nbytes; tests that rely on the check skip when it does not."""

    def __init__(self, nbytes: int):
        import ctypes
        self.hip = hip_runtime()
        p = ctypes.c_void_p()
        rc = self.hip.hipMalloc(ctypes.byref(p), ctypes.c_size_t(nbytes))
        assert rc == 0, rc
        self.ptr = p.value
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        rc = self.hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size),
                                            ctypes.c_void_p(self.ptr))
        self.exact = rc == 0 and base.value == self.ptr and size.value == nbytes

    def free(self):
        import ctypes
        self.hip.hipFree(ctypes.c_void_p(self.ptr))


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mxq.lib()
