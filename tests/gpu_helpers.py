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


# Margins of every comparison in this process: (test, what, margin, normwise
# relative error, elements).  The margin is max |gpu - ref| / (atol + rtol |ref|)
# over the tensor: 1.0 is the tolerance itself.
MARGINS = []


def _current_test():
    import os
    return os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]


def assert_close(gpu, ref, rtol, atol, what=""):
    """Elementwise |gpu - ref| <= atol + rtol |ref|; returns the margin (the
    worst ratio of error to bound) and records it with the normwise relative
    error ||gpu - ref|| / ||ref||."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    margin = float(ratio.max()) if ratio.size else 0.0
    rn = float(np.linalg.norm(ref.ravel()))
    nrel = float(np.linalg.norm((gpu - ref).ravel()) / rn) if rn > 0 else float(err.max(initial=0))
    MARGINS.append((_current_test(), what, margin, nrel, int(err.size)))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} elements outside tolerance "
            f"(rtol={rtol}, atol={atol}); worst at {i}: gpu={gpu[i]!r} ref={ref[i]!r}")
    return margin


def receipt_checksum(words):
    """A receipt's checksum as the library header defines it: the sum over the
    state's 32-bit words w_i of w_i * (2i + 1), modulo 2^64."""
    w = np.frombuffer(np.ascontiguousarray(words, dtype=np.float32).tobytes(), dtype="<u4")
    i = np.arange(w.size, dtype=np.uint64)
    return int(np.sum(w.astype(np.uint64) * (2 * i + 1), dtype=np.uint64))
