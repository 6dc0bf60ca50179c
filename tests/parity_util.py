"""Shared helpers of the GPU parity tests."""
import sys

import torch

BF16_RTOL, BF16_ATOL = 2e-2, 1e-2
F32_RTOL, F32_ATOL = 1e-5, 1e-5


def tol(dtype):
    return (F32_RTOL, F32_ATOL) if dtype == torch.float32 else (BF16_RTOL, BF16_ATOL)


def assert_within(got, ref, rtol, atol, what=""):
    """|got - ref| <= atol + rtol |ref| elementwise (ref in float64)."""
    got = got.detach().double().cpu()
    ref = ref.detach().double().cpu()
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert torch.isfinite(got).all(), f"{what}: non-finite values"
    err = (got - ref).abs()
    bound = atol + rtol * ref.abs()
    bad = err > bound
    if bad.any():
        i = int(torch.argmax((err - bound).flatten()))
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.numel()} elements out of tolerance "
            f"(rtol={rtol}, atol={atol}); worst at flat index {i}: got {got.flatten()[i]:.6g} "
            f"ref {ref.flatten()[i]:.6g}; max abs err {float(err.max()):.3g}")


def announce(msg):
    """Name the case before any GPU work, so a failure can be placed."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def to_gpu(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
