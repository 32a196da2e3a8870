"""Shared test helpers: device transfer of synthetic inputs and the parity check."""
import numpy as np

BF16_ATOL, BF16_RTOL = 2e-3, 2e-2      # |gpu - ref| <= atol + rtol |ref|, elementwise
FP8_ATOL, FP8_RTOL = 2e-3, 6e-2


def to_dev_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev(arr, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def bf16_tensor_to_f64(t):
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32).__lshift__(16) \
        .view(np.float32).astype(np.float64)


def assert_close(got, ref, atol=BF16_ATOL, rtol=BF16_RTOL, what="", extra=0.0):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values in GPU output"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref) + extra
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} / {bad.size} elements out of tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} (max abs err {err.max():.3e})")
    return float(err.max())
