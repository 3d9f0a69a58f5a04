"""Shared helpers of the GPU parity tests: device transfers and the tolerance
check.  Tolerances (elementwise |gpu - ref| <= atol + rtol * |ref|):
  fp32 inputs: rtol = atol = 1e-5 on outputs and states;
  bf16 inputs: rtol = 2e-2 with atol = 2e-2 * RMS(ref) per tensor.
Positions, sequence numbers, reset boundaries and flush counts compare exactly.
"""
import sys

import numpy as np

F32_TOL = dict(rtol=1e-5, atol=1e-5)


def bf16_tol(ref):
    rms = float(np.sqrt(np.mean(np.square(ref)))) if np.size(ref) else 0.0
    return dict(rtol=2e-2, atol=2e-2 * rms)


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[case]", *a, file=sys.stderr, flush=True)


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda", dtype) if dtype is not None else t.to("cuda")


def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(
        torch.bfloat16)


def host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def assert_close(gpu, ref, rtol, atol, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} elements outside tolerance "
            f"(rtol={rtol}, atol={atol}); worst at {i}: gpu={gpu[i]!r} ref={ref[i]!r}")
    return float(err.max()) if err.size else 0.0


def receipt_checksum(words):
    """A receipt's checksum as the library header defines it: the sum over the
    state's 32-bit words w_i of w_i * (2i + 1), modulo 2^64."""
    w = np.frombuffer(np.ascontiguousarray(words, dtype=np.float32).tobytes(), dtype="<u4")
    i = np.arange(w.size, dtype=np.uint64)
    return int(np.sum(w.astype(np.uint64) * (2 * i + 1), dtype=np.uint64))
