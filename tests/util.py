"""Shared helpers of the test suite (host <-> device marshalling, error metrics)."""
import numpy as np


def to_dev(a: np.ndarray, kind: str = None):
    """Host array of stored elements -> device torch tensor of the same bytes."""
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.uint8 and kind == "fp8":
        t = torch.from_numpy(a).view(torch.float8_e4m3fn)
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def max_rel_err(got, ref, floor=1e-2):
    """max |g - r| / max(|r|, floor) -- the fp32 parity metric."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor))) if ref.size else 0.0


def max_abs_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref))) if ref.size else 0.0


def normwise_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    return max_abs_err(got, ref) / den if den > 0 else max_abs_err(got, ref)


def lse_err(got, ref):
    """max |g - r| over rows, with -inf required to match exactly."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.array_equal(np.isneginf(got), np.isneginf(ref)):
        return float("inf")
    fin = np.isfinite(ref)
    return float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
