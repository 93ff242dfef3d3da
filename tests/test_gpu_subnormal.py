"""GPU parity on subnormal inputs: IEEE binary64 / binary32 arithmetic keeps
subnormals (no flush to zero on either side), so every kernel must match the
oracle bit for bit where values, partial sums and outputs are subnormal or
cross between the subnormal and the normal range.

Inputs: the mixed-magnitude generator (magnitudes 1e-8 .. 1e8, random signs)
scaled by 2^-1000 (double) or 2^-110 (float): the smallest values are
subnormal (below 2^-1022, resp. 2^-126), the largest normal, and sums of
neighbours cross the boundary in both directions.  A second input is
subnormal throughout (uniform in (-1, 1) scaled to below the normal range)."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import assert_bit_exact, to_dev, to_host  # noqa: E402


@pytest.fixture(scope="module")
def canon():
    import scan_canonical_reduce_amd as c
    c.lib()
    assert torch.cuda.is_available()
    return c


TINY = {np.float64: np.finfo(np.float64).tiny, np.float32: np.finfo(np.float32).tiny}


def crossing(n, seed, dtype):
    """Mixed magnitudes around the bottom of the normal range."""
    scale = 2.0 ** -1000 if dtype == np.float64 else 2.0 ** -110
    x = (synth.generate(n, "mixed_magnitude", seed) * scale).astype(dtype)
    sub = np.abs(x) < TINY[dtype]
    assert 0.05 < sub.mean() < 0.95, "the input must mix subnormal and normal values"
    return x


def all_subnormal(n, seed, dtype):
    scale = 2.0 ** -1040 if dtype == np.float64 else 2.0 ** -136
    x = (synth.generate(n, "uniform_pm1", seed) * scale).astype(dtype)
    assert np.all(np.abs(x) < TINY[dtype])
    return x


def has_subnormal(a, dtype):
    a = np.asarray(a).reshape(-1)
    return bool(np.any((a != 0) & (np.abs(a) < TINY[dtype])))


INPUTS = [("crossing", crossing), ("all_subnormal", all_subnormal)]


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("kind,make", INPUTS)
def test_reduce(canon, dtype, kind, make):
    x = make(300_007, 61, dtype)
    xd = to_dev(x)
    init = dtype(3) * TINY[dtype] / dtype(8)  # subnormal init
    for L in (1, 7, 16, 128):
        for n in (1, 1000, 65537, x.size):
            got = to_host(canon.reduce(xd[:n], L, init)).reshape(1)
            assert_bit_exact(got, [oracle.reduce(x[:n], L, init)], f"{kind} L={L} n={n}")
        got = to_host(canon.reduce(xd[1:], L, -0.0)).reshape(1)  # unaligned
        assert_bit_exact(got, [oracle.reduce(x[1:], L, -0.0)], f"{kind} unaligned L={L}")


SCANS = [("pairwise", 0), ("block_dyadic", 16), ("block_dyadic", 256),
         ("iterated_pairwise", 128), ("iterated_pairwise", 16), ("iterated_pairwise", 3)]


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("kind,make", INPUTS)
@pytest.mark.parametrize("policy,param", SCANS)
def test_scan(canon, dtype, kind, make, policy, param):
    x = make(300_007, 62, dtype)
    want = oracle.scan(x, policy, param)
    got = to_host(canon.scan(to_dev(x), policy, param))
    assert_bit_exact(got, want, f"{kind} {policy}<{param}>")
    if kind == "all_subnormal":
        assert has_subnormal(got, dtype), "some prefixes are subnormal"
    init = -TINY[dtype] / dtype(4)
    got = to_host(canon.scan_with_init(to_dev(x), policy, param, "exclusive", init))
    assert_bit_exact(got, oracle.scan_with_init(x, policy, param, init, "exclusive"),
                     f"{kind} exclusive {policy}<{param}>")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("kind,make", INPUTS)
def test_rows(canon, dtype, kind, make):
    rows, ld = 33, 5008
    X = make(rows * ld, 63, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for cols in (17, 4096, 5008):
        for L in (16, 3):
            got = to_host(canon.reduce_rows(Xd[:, :cols], L, -0.0))
            assert_bit_exact(got, oracle.reduce_rows(X, L, -0.0, cols=cols),
                             f"{kind} reduce_rows L={L} cols={cols}")
        for policy, param in (("block_dyadic", 16), ("pairwise", 0), ("iterated_pairwise", 16)):
            got = to_host(canon.scan_rows(Xd[:, :cols], policy, param))
            want = oracle.scan_rows(X, policy, param, cols=cols)[:, :cols]
            assert_bit_exact(got, want, f"{kind} scan_rows {policy} cols={cols}")
