"""Helpers shared by the GPU parity tests: device upload and the tolerance.

Tolerance (decode and prefill layer outputs): max |y_gpu - y_oracle| <=
2e-3 * RMS(y_oracle) over one call's q*d outputs.  The oracle is exact up to
one final fp32 rounding; the GPU path uses exact weights and activations and
fp32 accumulation, so its error is fp32 summation order plus the bf16 hi+lo
split of h (relative residual below 2^-16), far inside the bound.
"""
import numpy as np

TOL = 2e-3


def rel_err(y_gpu, y_ref):
    y_ref = np.asarray(y_ref, np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = float(np.max(np.abs(np.asarray(y_gpu, np.float64) - y_ref)))
    return err / rms if rms > 0 else err


def assert_close(y_gpu, y_ref, tol=TOL, what=""):
    r = rel_err(y_gpu, y_ref)
    assert r <= tol, f"{what}: max|dy|/RMS = {r:.3e} > {tol:.1e}"
    return r


def to_device_x(cols_x):
    """float32 columns, or uint16 bf16 bit patterns, to a cuda tensor."""
    import torch
    a = np.ascontiguousarray(cols_x)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a.astype(np.float32)).to("cuda")


class HipEvents:
    """hipEvent_t handles (timing enabled) through the HIP runtime that torch
    has loaded, for the *_timed entry points."""

    def __init__(self):
        import ctypes as C
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        assert path is not None, "HIP runtime not loaded"
        self.C = C
        self.lib = C.CDLL(path)
        self.lib.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.lib.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self, n):
        C = self.C
        arr = (C.c_void_p * n)()
        for i in range(n):
            h = C.c_void_p()
            assert self.lib.hipEventCreate(C.byref(h)) == 0
            arr[i] = h
        return arr

    def ms(self, a, b) -> float:
        out = self.C.c_float()
        assert self.lib.hipEventElapsedTime(self.C.byref(out), a, b) == 0
        return out.value

    def destroy(self, arr):
        for h in arr:
            self.lib.hipEventDestroy(h)


def check_stamps(he, ev):
    """Six stamps of a *_timed call: three start/end intervals of positive
    length, in launch order, inside the first-start-to-last-end span."""
    d = [he.ms(ev[2 * i], ev[2 * i + 1]) for i in range(3)]
    gaps = [he.ms(ev[1], ev[2]), he.ms(ev[3], ev[4])]
    span = he.ms(ev[0], ev[5])
    assert all(x > 0 for x in d), d
    assert all(g >= -1e-3 for g in gaps), gaps
    assert span >= sum(d) + sum(gaps) - 1e-3, (span, d, gaps)
    return d
