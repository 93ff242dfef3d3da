"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the reduction or scan arithmetic: it only draws
numbers.  Both the GPU path's callers and the oracle consume the very same
host buffers it returns.

Recipes (numpy ``Generator(PCG64(seed))``; one generator per call, draws in
the order written, in chunks of ``CHUNK`` elements so that large buffers are
produced without a second full-size temporary):

* ``uniform01``       -- ``rng.random(c)`` (53-bit uniform in [0, 1))
* ``uniform_pm1``     -- ``2.0 * rng.random(c) - 1.0`` (exact; [-1, 1))
* ``mixed_magnitude`` -- per chunk ``mag = 10.0 ** rng.uniform(-8, 8, c)``
  then ``sign = 1 - 2 * rng.integers(0, 2, c)``; value ``sign * mag``
  (log-uniform magnitude in [1e-8, 1e8], random sign: rounding-order
  sensitive)
* float32 variants draw the float64 values above and round them to nearest.

The pages' own witness inputs ("N doubles, fixed seed") are unpublished, so
these stand in for them; the workload table ``CONFIGS`` mirrors the shapes the
benchmark and the parity tests use.
"""
from __future__ import annotations

import hashlib

import numpy as np

CHUNK = 1 << 22

DISTRIBUTIONS = ("uniform01", "uniform_pm1", "mixed_magnitude")


def generate(n: int, dist: str, seed: int, dtype=np.float64) -> np.ndarray:
    """n values of a distribution, as a new contiguous array of ``dtype``."""
    if dist not in DISTRIBUTIONS:
        raise ValueError(dist)
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty(n, dtype=dtype)
    for s in range(0, n, CHUNK):
        c = min(CHUNK, n - s)
        if dist == "uniform01":
            v = rng.random(c)
        elif dist == "uniform_pm1":
            v = 2.0 * rng.random(c) - 1.0
        else:
            mag = 10.0 ** rng.uniform(-8.0, 8.0, c)
            sign = 1 - 2 * rng.integers(0, 2, c)
            v = sign * mag
        out[s:s + c] = v  # rounds to nearest when dtype is float32
    return out


def integers(n: int, lo: int, hi: int, seed: int, dtype=np.float64) -> np.ndarray:
    """Integer-valued floats drawn uniformly from [lo, hi)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi, n).astype(dtype)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


# The five workloads.  Each: dtype, shape, distribution, seed.
CONFIGS = {
    "reduce_1m": dict(dtype=np.float64, n=1 << 20, dist="uniform01", seed=1001),
    "scan_1m": dict(dtype=np.float64, n=1 << 20, dist="uniform01", seed=1002),
    "reduce_2e28_f64": dict(dtype=np.float64, n=1 << 28, dist="mixed_magnitude", seed=1003),
    "reduce_2e29_f32": dict(dtype=np.float32, n=1 << 29, dist="mixed_magnitude", seed=1013),
    "rows_16384x4096": dict(dtype=np.float64, rows=16384, cols=4096, dist="uniform_pm1", seed=1004),
    "scan_2e27_f64": dict(dtype=np.float64, n=1 << 27, dist="mixed_magnitude", seed=1005),
    "scan_2e28_f32": dict(dtype=np.float32, n=1 << 28, dist="mixed_magnitude", seed=1015),
}


def config_input(name: str) -> np.ndarray:
    c = CONFIGS[name]
    if "rows" in c:
        return generate(c["rows"] * c["cols"], c["dist"], c["seed"], c["dtype"]).reshape(
            c["rows"], c["cols"])
    return generate(c["n"], c["dist"], c["seed"], c["dtype"])
