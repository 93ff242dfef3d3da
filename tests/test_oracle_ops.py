"""Pins for the oracle with other operators: multiplication, minimum and
maximum (the canonical expression is defined for any binary operator:
canonical-reduce README, P4016R0 "Summary"; min and max are read as IEEE
754-2019 minimum / maximum), and "skew", a (+) b = (a + b) + ((a/4) b) b,
neither commutative nor associative (the caller-defined-operator tests use
it: any change of operand order or of parenthesisation changes its values).

Checked against things other than the oracle itself:
  * the independently written symbolic trees evaluated with the operator;
  * products evaluated in exact rational arithmetic, rounded after every
    step (Fraction -> float rounds to nearest even), on the same trees;
  * exact products of powers of two and small integers (closed forms);
  * numpy's min / max where no NaN or signed-zero tie decides;
  * the special cases of minimum / maximum (signed zeros, NaN);
  * identities: init = the operator's identity gives the plain scan; the
    inclusive/exclusive duality; scan back == reduce.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import symbolic as S

DTYPES = [np.float64, np.float32]
OPS = ["mul", "min", "max", "skew"]
IDENT = {"add": -0.0, "mul": 1.0, "min": np.inf, "max": -np.inf, "skew": -0.0}
POLICIES = [("pairwise", 0), ("block_dyadic", 4), ("iterated_pairwise", 3)]


def bits(a):
    a = np.asarray(a)
    return a.view(np.uint64 if a.dtype == np.float64 else np.uint32)


def same_bits(a, b):
    a = np.asarray(a)
    b = np.asarray(b, dtype=a.dtype)
    return a.shape == b.shape and np.array_equal(bits(a), bits(b))


def near_one(n, seed, dtype):
    """Factors close to 1 (products stay finite and rounding-sensitive)."""
    u = synth.generate(n, "uniform_pm1", seed)
    return (1.0 + u * 1e-3).astype(dtype)


def small(n, seed, dtype):
    """Values in (-1e-3, 1e-3): sums and skew terms stay far from overflow."""
    return (synth.generate(n, "uniform_pm1", seed) * 1e-3).astype(dtype)


def data(op, n, seed, dtype):
    if op == "mul":
        return near_one(n, seed, dtype)
    if op == "skew":
        return small(n, seed, dtype)
    return synth.generate(n, "mixed_magnitude", seed, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("policy,param", POLICIES)
def test_scan_and_reduce_equal_symbolic(dtype, op, policy, param):
    n = 45
    x = data(op, n, 70, dtype)
    y = oracle.scan(x, policy, param, op)
    for i in range(n):
        want = S.evaluate(S.scan_tree(i, policy, param), x, op=op)
        assert same_bits(y[i], want), i
    for L in (1, 3, 8):
        want = S.evaluate(S.reduce_tree(n, L), x, init=0.75, op=op)
        assert same_bits(oracle.reduce(x, L, 0.75, op), want)


def _exact_eval(tree, vals):
    """Product over a tree in rationals, rounded to binary64 after each step."""
    if isinstance(tree, int):
        return Fraction(vals[tree])
    a = _exact_eval(tree[0], vals)
    b = _exact_eval(tree[1], vals)
    return Fraction(float(a * b))


def test_products_rounded_step_by_step():
    x = near_one(60, 71, np.float64)
    y = oracle.scan(x, "pairwise", 0, "mul")
    for i in range(60):
        want = float(_exact_eval(S.pw_tree(list(range(i + 1))), [float(v) for v in x]))
        assert same_bits(y[i], want), i
    # the rounding makes the tree visible: the left fold differs somewhere
    fold = np.cumprod(x)
    assert not same_bits(y, fold)


@pytest.mark.parametrize("dtype", DTYPES)
def test_products_exact_closed_forms(dtype):
    rng = np.random.Generator(np.random.PCG64(72))
    e = rng.integers(-3, 4, 200)
    sgn = 1 - 2 * rng.integers(0, 2, 200)
    x = (sgn * np.ldexp(1.0, e)).astype(dtype)
    for policy, param in POLICIES + [("block_dyadic", 16), ("iterated_pairwise", 7)]:
        y = oracle.scan(x, policy, param, "mul")
        want = np.cumprod(sgn) * np.ldexp(1.0, np.cumsum(e))
        assert same_bits(y, want.astype(dtype)), policy
    z = np.array([3, 1, 2, 2, 3, 1, 2], dtype)
    assert same_bits(oracle.reduce(z, 3, 5.0, "mul"), dtype(5 * 72))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", ["min", "max"])
def test_min_max_against_numpy(dtype, op):
    x = synth.generate(5000, "mixed_magnitude", 73, dtype)
    f = np.minimum.accumulate if op == "min" else np.maximum.accumulate
    for policy, param in POLICIES + [("block_dyadic", 256), ("iterated_pairwise", 128)]:
        assert same_bits(oracle.scan(x, policy, param, op), f(x)), policy
    g = np.min if op == "min" else np.max
    for L in (1, 16, 128):
        assert same_bits(oracle.reduce(x, L, IDENT[op], op), g(x))


@pytest.mark.parametrize("dtype", DTYPES)
def test_min_max_special_values(dtype):
    z = np.array([0.0, -0.0, 0.0], dtype)
    assert np.signbit(oracle.reduce(z, 1, np.inf, "min"))
    assert not np.signbit(oracle.reduce(z[::-1].copy(), 2, -np.inf, "max"))
    x = np.array([1.0, np.nan, -5.0, 2.0], dtype)
    for op in ("min", "max"):
        y = oracle.scan(x, "pairwise", 0, op)
        assert not np.isnan(y[0]) and np.all(np.isnan(y[1:]))
        assert np.isnan(oracle.reduce(x, 2, IDENT[op], op))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("policy,param", POLICIES)
def test_identity_init_duality_and_back(dtype, op, policy, param):
    x = data(op, 300, 74, dtype)
    plain = oracle.scan(x, policy, param, op)
    inc = oracle.scan_with_init(x, policy, param, IDENT[op], "inclusive", op)
    assert same_bits(inc, plain)
    init = dtype(1.5)
    inc = oracle.scan_with_init(x, policy, param, init, "inclusive", op)
    exc = oracle.scan_with_init(x, policy, param, init, "exclusive", op)
    ii = oracle.scan_with_init(x, policy, param, init, "include_initial", op)
    assert same_bits(exc[0], init) and same_bits(exc[1:], inc[:-1])
    assert same_bits(ii[:-1], exc) and same_bits(ii[-1], inc[-1])
    for k in (0, 1, 7, 150, 299):
        assert same_bits(oracle.scan_with_init_output(x, k, policy, param, init, "inclusive", op),
                         inc[k])
    if policy == "iterated_pairwise":
        assert same_bits(plain[-1], oracle.reduce(x, param, IDENT[op], op))
    # rows: each row is its own sequence
    X = x[:280].reshape(7, 40)
    R = oracle.scan_rows(X, policy, param, op=op)
    for r in range(7):
        assert same_bits(R[r], oracle.scan(X[r], policy, param, op))


def test_mul_init_placement():
    """op(init, R) once after the tree is not init folded in as an element."""
    diff = 0
    for seed in range(100):
        x = near_one(37, 900 + seed, np.float64)
        got = oracle.reduce(x, 4, 1.0 + 1e-3, "mul")
        folded = oracle.cr(np.concatenate([[1.0 + 1e-3], x]), 4, "mul")
        diff += not same_bits(got, folded)
    assert diff > 20


@pytest.mark.parametrize("dtype", DTYPES)
def test_skew_operator_definition_and_identity(dtype):
    """One application against the definition written with numpy scalars;
    -0.0 is a two-sided identity, signed zeros included; the operator is not
    commutative and not associative on ordinary values."""
    t = dtype
    rng = np.random.Generator(np.random.PCG64(75))
    for a, b in rng.uniform(-3, 3, (200, 2)):
        a, b = t(a), t(b)
        want = t(t(a + b) + t(t(t(a * t(0.25)) * b) * b))
        assert same_bits(oracle.apply(a, b, "skew"), want)
    vals = [t(0.0), t(-0.0), t(1.5), t(-2.25), t(1e-30), t(3e4)]
    for v in vals:
        assert same_bits(oracle.apply(v, t(-0.0), "skew"), v)
        assert same_bits(oracle.apply(t(-0.0), v, "skew"), v)
    a, b, c = t(0.5), t(0.25), t(-0.75)
    assert not same_bits(oracle.apply(a, b, "skew"), oracle.apply(b, a, "skew"))
    ab_c = oracle.apply(oracle.apply(a, b, "skew"), c, "skew")
    a_bc = oracle.apply(a, oracle.apply(b, c, "skew"), "skew")
    assert not same_bits(ab_c, a_bc)


def _swapped(tree):
    return tree if isinstance(tree, (int, str)) else (_swapped(tree[1]), _swapped(tree[0]))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("policy,param", POLICIES)
def test_skew_sees_operand_order(dtype, policy, param):
    """Evaluating the mirrored trees gives other bits for most prefixes, so a
    kernel that swaps operands anywhere cannot match the oracle with skew."""
    x = small(64, 76, dtype)
    y = oracle.scan(x, policy, param, "skew")
    differ = sum(not same_bits(y[i], S.evaluate(_swapped(S.scan_tree(i, policy, param)), x,
                                                op="skew")) for i in range(1, 64))
    assert differ > 40
