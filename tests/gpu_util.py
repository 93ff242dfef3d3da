"""Helpers for the GPU parity tests: bitwise comparison (NaN by class)."""
import numpy as np
import torch


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    return a.view(np.uint64 if a.dtype == np.float64 else np.uint32)


def mismatches(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Indices where the bit patterns differ; NaNs match any NaN."""
    got = np.asarray(got).reshape(-1)
    want = np.asarray(want, dtype=got.dtype).reshape(-1)
    assert got.shape == want.shape
    diff = bits(got) != bits(want)
    both_nan = np.isnan(got) & np.isnan(want)
    return np.nonzero(diff & ~both_nan)[0]


def assert_bit_exact(got, want, what=""):
    bad = mismatches(got, want)
    if bad.size:
        g = np.asarray(got).reshape(-1)
        w = np.asarray(want, dtype=g.dtype).reshape(-1)
        i = bad[0]
        raise AssertionError(
            f"{what}: {bad.size} of {g.size} values differ; first at {i}: "
            f"got {g[i]!r} ({bits(g[i:i+1])[0]:#x}) want {w[i]!r} ({bits(w[i:i+1])[0]:#x})")
