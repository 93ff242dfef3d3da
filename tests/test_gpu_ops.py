"""GPU parity of the operator entry points (multiplication, IEEE minimum,
IEEE maximum; canonical-reduce README, P4016R0 "Summary": the expression is
defined for any operator) through the C ABI, against the oracle evaluated
with the same operator, bit for bit."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import assert_bit_exact, scan_tile, to_dev, to_host  # noqa: E402

OPS = ["mul", "min", "max"]
KINDS = ["inclusive", "exclusive", "include_initial"]
IDENT = {"mul": 1.0, "min": np.inf, "max": -np.inf}


@pytest.fixture(scope="module")
def canon():
    import scan_canonical_reduce_amd as c
    c.lib()
    assert torch.cuda.is_available()
    return c


def data(op, n, seed, dtype):
    """Factors near 1 for products (finite, rounding-sensitive), mixed
    magnitudes otherwise."""
    if op == "mul":
        return (1.0 + synth.generate(n, "uniform_pm1", seed) * 1e-3).astype(dtype)
    return synth.generate(n, "mixed_magnitude", seed, dtype)


def tile(dtype):
    return scan_tile(dtype)  # elements per single-pass tile


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("op", OPS)
def test_reduce(canon, dtype, op):
    x = data(op, 300_001, 81, dtype)
    xd = to_dev(x)
    for L in (1, 3, 16, 128, 1000):
        for n in (1, L - 1, L, 5000, x.size):
            if n <= 0:
                continue
            got = to_host(canon.reduce_op(xd[:n], L, op, 1.25)).reshape(1)
            assert_bit_exact(got, [oracle.reduce(x[:n], L, 1.25, op)], f"L={L} n={n}")
        # unaligned start
        got = to_host(canon.reduce_op(xd[1:], L, op, IDENT[op])).reshape(1)
        assert_bit_exact(got, [oracle.reduce(x[1:], L, IDENT[op], op)], f"unaligned L={L}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 2),
                                          ("block_dyadic", 16), ("block_dyadic", 256),
                                          ("block_dyadic", 8192), ("iterated_pairwise", 3),
                                          ("iterated_pairwise", 16), ("iterated_pairwise", 128)])
def test_scan(canon, dtype, op, policy, param):
    S = tile(dtype)
    x = data(op, 66 * S + 777, 82, dtype)
    xd = to_dev(x)
    for kind in KINDS:
        init = IDENT[op] if kind == "inclusive" else 0.5
        full = oracle.scan_with_init(x, policy, param, init, kind, op)
        for n in (1, 2, S - 1, S + 1, 64 * S + 3, x.size):
            y = to_host(canon.scan_op(xd[:n], policy, param, op, kind, init))
            want = full[:n + 1] if kind == "include_initial" else full[:n]
            assert_bit_exact(y, want, f"{kind} n={n}")
    # unaligned input
    y = to_host(canon.scan_op(xd[1:], policy, param, op))
    assert_bit_exact(y, oracle.scan(x[1:], policy, param, op), "unaligned")


@pytest.mark.parametrize("op", OPS)
def test_scan_in_place_and_many_tiles(canon, op):
    x = data(op, (1 << 21) + 4321, 83, np.float64)
    for policy, param in (("pairwise", 0), ("block_dyadic", 256), ("iterated_pairwise", 128)):
        xd = to_dev(x)
        canon.scan_op(xd, policy, param, op, out=xd)
        assert_bit_exact(to_host(xd), oracle.scan(x, policy, param, op), f"{policy}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("op", OPS)
def test_rows(canon, dtype, op):
    rows, ld = 19, 5000
    X = data(op, rows * ld, 84, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for cols in (1, 700, 4096, 5000):
        got = to_host(canon.reduce_rows_op(Xd[:, :cols], 16, op, 2.0))
        assert_bit_exact(got, oracle.reduce_rows(X, 16, 2.0, cols=cols, op=op), f"reduce {cols}")
        for policy, param in (("pairwise", 0), ("block_dyadic", 16), ("iterated_pairwise", 128)):
            got = to_host(canon.scan_rows_op(Xd[:, :cols], policy, param, op, "exclusive", 0.75))
            want = oracle.scan_rows_with_init(X, policy, param, 0.75, "exclusive", cols=cols,
                                              op=op)
            assert_bit_exact(got, want[:, :cols], f"scan {policy} {cols}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_min_max_special_values(canon, dtype):
    x = np.array([3.0, 0.0, -0.0, 0.0, np.inf, -2.0, np.nan, 1.0] * 1000, dtype)
    xd = to_dev(x)
    for op in ("min", "max"):
        for policy, param in (("pairwise", 0), ("block_dyadic", 4)):
            y = to_host(canon.scan_op(xd, policy, param, op))
            assert_bit_exact(y, oracle.scan(x, policy, param, op), f"{op} {policy}")
        r = to_host(canon.reduce_op(xd[:6], 4, op)).reshape(1)
        assert_bit_exact(r, [oracle.reduce(x[:6], 4, IDENT[op], op)], f"{op} zeros")


def test_add_is_the_plain_library(canon):
    x = synth.generate(100_003, "mixed_magnitude", 85)
    xd = to_dev(x)
    assert_bit_exact(to_host(canon.reduce_op(xd, 128, "add", 1.0)).reshape(1),
                     to_host(canon.reduce(xd, 128, 1.0)).reshape(1), "reduce")
    for policy, param in (("pairwise", 0), ("block_dyadic", 256), ("iterated_pairwise", 128)):
        assert_bit_exact(to_host(canon.scan_op(xd, policy, param, "add")),
                         to_host(canon.scan(xd, policy, param)), policy)
