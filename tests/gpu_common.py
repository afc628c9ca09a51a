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
