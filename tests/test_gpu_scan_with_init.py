"""GPU parity of the scans with an initial value (inclusive, exclusive,
include_initial) through the C ABI, against the oracle, bit for bit.

The shifted kinds take the value before each tile from the tile-level nodes,
before each wave from the previous wave and before each row (iterated
pairwise) from the previous row's tree, so the sizes below put tile, wave,
row and block boundaries at every kind of position, with ragged tails."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import assert_bit_exact, scan_tile, to_dev, to_host  # noqa: E402

KINDS = ["inclusive", "exclusive", "include_initial"]


@pytest.fixture(scope="module")
def canon():
    import scan_canonical_reduce_amd as c
    c.lib()
    assert torch.cuda.is_available()
    return c


def tile(dtype):
    return scan_tile(dtype)  # elements per single-pass tile


def expect(x, policy, param, kind, init, n):
    """Oracle outputs for x[:n] (a prefix of the outputs over all of x)."""
    full = oracle.scan_with_init(x, policy, param, init, kind)
    return full[:n + 1] if kind == "include_initial" else full[:n]


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 1), ("block_dyadic", 2),
                                          ("block_dyadic", 16), ("block_dyadic", 256),
                                          ("block_dyadic", 8192), ("block_dyadic", 65536)])
@pytest.mark.parametrize("kind", KINDS)
def test_tails(canon, dtype, policy, param, kind):
    S = tile(dtype)
    x = synth.generate(66 * S + 999, "mixed_magnitude", 31, dtype)
    init = dtype(0.1)
    full = oracle.scan_with_init(x, policy, param, init, kind)
    xd = to_dev(x)
    for n in (1, 2, 3, 17, 255, 256, 257, S - 1, S, S + 1, 3 * S + 5, 64 * S - 1, 64 * S,
              64 * S + 1, x.size):
        y = to_host(canon.scan_with_init(xd[:n], policy, param, kind, init))
        want = full[:n + 1] if kind == "include_initial" else full[:n]
        assert_bit_exact(y, want, f"n={n}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [1, 3, 16, 128, 256, 2048])
@pytest.mark.parametrize("kind", KINDS)
def test_iterated_pairwise(canon, dtype, L, kind):
    x = synth.generate(70_001, "mixed_magnitude", 500 + L, dtype)
    init = dtype(-3.75)
    full = oracle.scan_with_init(x, "iterated_pairwise", L, init, kind)
    xd = to_dev(x)
    for n in (1, 2, L - 1, L, L + 1, 3 * L + 2, 5000, 16384, x.size):
        if n <= 0 or n > x.size:
            continue
        y = to_host(canon.scan_with_init(xd[:n], "iterated_pairwise", L, kind, init))
        want = full[:n + 1] if kind == "include_initial" else full[:n]
        assert_bit_exact(y, want, f"n={n}")
        if kind == "inclusive":
            # the last output is the reduction with init of the same expression
            r = to_host(canon.reduce(xd[:n], L, init)).reshape(1)
            assert_bit_exact(y[-1:], r, f"back n={n}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("kind", ["exclusive", "include_initial"])
def test_every_block_size(canon, dtype, kind):
    S = tile(dtype)
    x = synth.generate(5 * S + 123, "mixed_magnitude", 32, dtype)
    xd = to_dev(x)
    for b in range(0, 17):
        B = 1 << b
        want = oracle.scan_with_init(x, "block_dyadic", B, 2.5, kind)
        assert_bit_exact(to_host(canon.scan_with_init(xd, "block_dyadic", B, kind, 2.5)), want,
                         f"B={B}")
        # unaligned input and output (element loads and stores)
        wu = oracle.scan_with_init(x[1:], "block_dyadic", B, 2.5, kind)
        ob = torch.empty(x.size + 2, dtype=xd.dtype, device="cuda")
        y = canon.scan_with_init(xd[1:], "block_dyadic", B, kind, 2.5, out=ob[1:1 + wu.size])
        assert_bit_exact(to_host(y), wu, f"unaligned B={B}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 16),
                                          ("block_dyadic", 256), ("iterated_pairwise", 128)])
def test_many_tiles(canon, dtype, policy, param):
    """Published nodes up to tile level 9; the value before every tile."""
    x = synth.generate((1 << 22) + 12345, "mixed_magnitude", 33, dtype)
    xd = to_dev(x)
    for kind in ("exclusive", "include_initial"):
        y = to_host(canon.scan_with_init(xd, policy, param, kind, 1e3))
        assert_bit_exact(y, oracle.scan_with_init(x, policy, param, 1e3, kind), kind)


@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 16),
                                          ("block_dyadic", 65536), ("iterated_pairwise", 128),
                                          ("iterated_pairwise", 7)])
@pytest.mark.parametrize("kind", KINDS)
def test_in_place(canon, policy, param, kind):
    n = 300_001
    x = synth.generate(n, "mixed_magnitude", 34)
    buf = torch.zeros(n + 1, dtype=torch.float64, device="cuda")
    buf[:n] = to_dev(x)
    xd = buf[:n]
    out = buf if kind == "include_initial" else xd
    canon.scan_with_init(xd, policy, param, kind, -7.0, out=out)
    want = oracle.scan_with_init(x, policy, param, -7.0, kind)
    assert_bit_exact(to_host(out), want, "in place")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 16),
                                          ("iterated_pairwise", 128)])
def test_minus_zero_inclusive_is_the_plain_scan(canon, dtype, policy, param):
    x = synth.generate(200_003, "mixed_magnitude", 35, dtype)
    xd = to_dev(x)
    y = to_host(canon.scan_with_init(xd, policy, param, "inclusive", -0.0))
    assert_bit_exact(y, to_host(canon.scan(xd, policy, param)), "plain")
    # +0.0 is combined too: an all -0.0 input gives +0.0 everywhere
    z = to_dev(np.full(70_000, -0.0, dtype))
    for kind in KINDS:
        y = to_host(canon.scan_with_init(z, policy, param, kind, 0.0))
        assert not np.any(np.signbit(y)) and np.all(y == 0), kind


def test_empty(canon):
    e = torch.empty(0, dtype=torch.float64, device="cuda")
    y = canon.scan_with_init(e, "pairwise", 0, "include_initial", 4.25)
    assert to_host(y).tolist() == [4.25]
    assert canon.scan_with_init(e, "block_dyadic", 16, "exclusive", 4.25).numel() == 0
    Y = canon.scan_rows_with_init(torch.empty((5, 0), dtype=torch.float32, device="cuda"),
                                  "pairwise", 0, "include_initial", 1.5)
    assert Y.shape == (5, 1) and np.all(to_host(Y) == 1.5)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 2),
                                          ("block_dyadic", 16), ("block_dyadic", 8192),
                                          ("iterated_pairwise", 3), ("iterated_pairwise", 128)])
@pytest.mark.parametrize("kind", KINDS)
def test_rows(canon, dtype, policy, param, kind):
    rows, ld = 37, 9000
    X = synth.generate(rows * ld, "mixed_magnitude", 36, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    extra = 1 if kind == "include_initial" else 0
    for cols in (1, 17, 4096, 4097, 9000 - extra):
        got = to_host(canon.scan_rows_with_init(Xd[:, :cols], policy, param, kind, 0.5))
        want = oracle.scan_rows_with_init(X, policy, param, 0.5, kind, cols=cols)
        assert_bit_exact(got, want[:, :cols + extra], f"cols={cols}")


@pytest.mark.parametrize("policy,param", [("block_dyadic", 16), ("iterated_pairwise", 128)])
@pytest.mark.parametrize("kind", KINDS)
def test_rows_in_place_aligned_pitch(canon, policy, param, kind):
    """In place with a 16-byte aligned pitch (the register paths); the extra
    include_initial output of each row lands in that row's pitch padding."""
    rows, ld, cols = 64, 4224, 4096
    X = synth.generate(rows * ld, "uniform_pm1", 37).reshape(rows, ld)
    Xd = to_dev(X)
    out = Xd[:, :cols + (1 if kind == "include_initial" else 0)]
    canon.scan_rows_with_init(Xd[:, :cols], policy, param, kind, 10.0, out=out)
    want = oracle.scan_rows_with_init(X, policy, param, 10.0, kind, cols=cols)
    assert_bit_exact(to_host(out), want[:, :out.shape[1]], "in place")
