"""Pins for the oracle's scan with an initial value (inclusive, exclusive,
include_initial).

Checked against things other than the oracle itself:
  * hand-worked outputs where rounding separates init-after-the-tree from
    init folded into it (tests/golden/scan_with_init.txt);
  * exact results on integer-valued inputs (Python integer prefix sums);
  * signed zeros: init is really combined, and -0.0 is the exact identity;
  * the duality identities of the gt4py scan-redesign research page, B.2
    "Array API standard / NumPy" (exclusive[k] = inclusive[k-1], first
    exclusive output = init, include_initial = exclusive plus the last
    inclusive output);
  * agreement with the reduction with init of the same expression
    (canonical-reduce README, P4016R0 "Key Design Points", init placement,
    and P4229R0 "Key Design Points", scan/reduce consistency);
  * the independently written symbolic trees, evaluated numerically.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import symbolic as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scan_with_init.txt")
DTYPES = [np.float64, np.float32]
KINDS = ["inclusive", "exclusive", "include_initial"]
POLICIES = [("pairwise", 0), ("block_dyadic", 1), ("block_dyadic", 4), ("block_dyadic", 16),
            ("iterated_pairwise", 1), ("iterated_pairwise", 4), ("iterated_pairwise", 16)]


def bits(a):
    a = np.asarray(a)
    return a.view(np.uint64 if a.dtype == np.float64 else np.uint32)


def same_bits(a, b):
    a = np.asarray(a)
    b = np.asarray(b, dtype=a.dtype)
    return a.shape == b.shape and np.array_equal(bits(a), bits(b))


def golden_cases():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("=")
            dt, kind, init = lhs.split()
            out.append((dt, kind, int(init), [int(v) for v in rhs.split()]))
    return out


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: f"{c[0]}-{c[1]}")
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 2),
                                          ("iterated_pairwise", 2)])
def test_hand_worked_rounding(case, policy, param):
    dt, kind, init, want = case
    dtype = np.float64 if dt == "f64" else np.float32
    x = np.ones(4, dtype)
    got = oracle.scan_with_init(x, policy, param, init, kind)
    assert same_bits(got, np.array(want, dtype=dtype))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("policy,param", POLICIES)
def test_integer_inputs_exact(dtype, kind, policy, param):
    rng = np.random.Generator(np.random.PCG64(7))
    for n in (0, 1, 2, 3, 31, 64, 100):
        xi = rng.integers(-1000, 1000, n)
        init = int(rng.integers(-50, 50))
        pre = [0]
        for v in xi:
            pre.append(pre[-1] + int(v))
        if kind == "inclusive":
            want = [init + pre[k + 1] for k in range(n)]
        elif kind == "exclusive":
            want = [init + pre[k] for k in range(n)]
        else:
            want = [init + pre[k] for k in range(n + 1)]
        got = oracle.scan_with_init(xi.astype(dtype), policy, param, init, kind)
        assert same_bits(got, np.array(want, dtype=dtype)), (n, kind)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("policy,param", POLICIES)
def test_signed_zero(dtype, policy, param):
    x = np.full(9, -0.0, dtype)
    plain = oracle.scan(x, policy, param)
    assert np.all(np.signbit(plain))
    # init +0.0 is combined: +0.0 + -0.0 = +0.0 everywhere, also the first output
    for kind in KINDS:
        y = oracle.scan_with_init(x, policy, param, 0.0, kind)
        assert not np.any(np.signbit(y)) and np.all(y == 0)
        y = oracle.scan_with_init(x, policy, param, -0.0, kind)
        assert np.all(np.signbit(y)) and np.all(y == 0)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("policy,param", POLICIES)
def test_duality_identities(dtype, policy, param):
    x = synth.generate(300, "mixed_magnitude", 11, dtype)
    init = dtype(0.3)
    inc = oracle.scan_with_init(x, policy, param, init, "inclusive")
    exc = oracle.scan_with_init(x, policy, param, init, "exclusive")
    ii = oracle.scan_with_init(x, policy, param, init, "include_initial")
    assert inc.shape == (300,) and exc.shape == (300,) and ii.shape == (301,)
    assert same_bits(exc[0], init)
    assert same_bits(exc[1:], inc[:-1])
    assert same_bits(ii[:-1], exc) and same_bits(ii[-1], inc[-1])
    # -0.0 is the exact identity: the plain scan is the inclusive scan with it
    assert same_bits(oracle.scan_with_init(x, policy, param, -0.0, "inclusive"),
                     oracle.scan(x, policy, param))
    # folding init in as an element in front of x is a different expression
    folded = oracle.scan(np.concatenate([[init], x]).astype(dtype), policy, param)[1:]
    assert not same_bits(inc, folded)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("L", [1, 3, 16, 128])
def test_agrees_with_reduce_with_init(dtype, L):
    """Every output equals the reduction with init of the prefix it observes
    (iterated_pairwise<L> is the reduction's own expression)."""
    x = synth.generate(777, "mixed_magnitude", 5, dtype)
    init = dtype(-1.25e3)
    inc = oracle.scan_with_init(x, "iterated_pairwise", L, init, "inclusive")
    ii = oracle.scan_with_init(x, "iterated_pairwise", L, init, "include_initial")
    for i in list(range(0, 40)) + list(range(700, 777)):
        assert same_bits(inc[i], oracle.reduce(x[:i + 1], L, init))
        assert same_bits(ii[i], oracle.reduce(x[:i], L, init))
    assert same_bits(ii[777], oracle.reduce(x, L, init))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 4),
                                          ("iterated_pairwise", 3)])
def test_equals_symbolic(dtype, kind, policy, param):
    n = 37
    x = synth.generate(n, "mixed_magnitude", 21, dtype)
    init = dtype(7.5e-3)
    got = oracle.scan_with_init(x, policy, param, init, kind)
    m = n + 1 if kind == "include_initial" else n
    want = [S.evaluate(S.scan_with_init_tree(k, policy, param, kind), x, init)
            for k in range(m)]
    assert same_bits(got, np.array(want, dtype=dtype))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 8),
                                          ("iterated_pairwise", 5)])
def test_single_output_from_scratch(dtype, kind, policy, param):
    """The from-scratch single output (literal prefix evaluation) agrees with
    the streaming form at every position."""
    x = synth.generate(130, "mixed_magnitude", 22, dtype)
    y = oracle.scan_with_init(x, policy, param, 0.7, kind)
    for k in range(y.size):
        assert same_bits(oracle.scan_with_init_output(x, k, policy, param, 0.7, kind), y[k])
    with pytest.raises(ValueError):
        oracle.scan_with_init_output(x, y.size, policy, param, 0.7, kind)


def test_symbolic_shapes():
    assert S.to_str(S.scan_with_init_tree(0, "pairwise", 0, "exclusive")) == "I"
    assert S.to_str(S.scan_with_init_tree(0, "pairwise", 0, "inclusive")) == "(Ia)"
    assert S.to_str(S.scan_with_init_tree(3, "pairwise", 0, "include_initial")) == "(I((ab)c))"
    assert S.to_str(S.scan_with_init_tree(2, "pairwise", 0, "inclusive")) == "(I((ab)c))"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind", KINDS)
def test_rows_equal_per_row_calls(dtype, kind):
    X = synth.generate(5 * 40, "uniform_pm1", 3, dtype).reshape(5, 40)
    Y = oracle.scan_rows_with_init(X, "block_dyadic", 8, 2.5, kind, cols=33)
    extra = 1 if kind == "include_initial" else 0
    assert Y.shape == (5, 40 + extra)
    for r in range(5):
        y = oracle.scan_with_init(X[r, :33], "block_dyadic", 8, 2.5, kind)
        assert same_bits(Y[r, :33 + extra], y)
        assert np.all(Y[r, 33 + extra:] == 0)


def test_empty_and_bad_kind():
    e = np.zeros(0)
    assert oracle.scan_with_init(e, "pairwise", 0, 3.0, "inclusive").size == 0
    assert oracle.scan_with_init(e, "pairwise", 0, 3.0, "exclusive").size == 0
    assert same_bits(oracle.scan_with_init(e, "pairwise", 0, 3.0, "include_initial"),
                     np.array([3.0]))
    with pytest.raises(ValueError):
        oracle.scan_with_init(np.ones(3), "pairwise", 0, 0.0, 5)
