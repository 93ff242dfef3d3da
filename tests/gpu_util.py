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


def scan_tile(dtype, policy="pairwise", param=0) -> int:
    """Elements per tile of the library's 1-d scans for this element type
    (canon_scan_tile_elems): the edge cases sit on its multiples."""
    import scan_canonical_reduce_amd as c
    t = c.scan_tile_elems(policy, param, np.dtype(dtype).itemsize)
    assert t > 0
    return t


def scan_rows_tile(dtype, policy="pairwise", param=0) -> int:
    """Elements per tile within a row of the library's row scans."""
    import scan_canonical_reduce_amd as c
    t = c.scan_rows_tile_elems(policy, param, np.dtype(dtype).itemsize)
    assert t > 0
    return t
