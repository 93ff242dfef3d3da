"""Pins for the CPU oracle: what the pages and plain mathematics fix.

The oracle is checked here against things other than itself:
  * hand-derived parenthesisations (tests/golden/tree_shapes.txt);
  * an independently written symbolic tree builder, evaluated numerically;
  * the worked example of the Futhark blog post (non-associativity of +);
  * exact results on integer-valued inputs, one-hot inputs, -0.0 handling;
  * closed-form identities between the policies and the reduction;
  * the aligned power-of-two chunk closure that parallel schedules rely on;
  * a textbook error bound against an exactly rounded sum;
  * power checks: every rejected alternative reading gives different bits.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import symbolic as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_shapes.txt")
DTYPES = [np.float64, np.float32]


def bits(a):
    a = np.asarray(a)
    return a.view(np.uint64 if a.dtype == np.float64 else np.uint32)


def same_bits(a, b):
    a = np.asarray(a)
    b = np.asarray(b, dtype=a.dtype)
    return np.array_equal(bits(a), bits(b))


def golden_lines():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("=")
            out.append((lhs.split(), rhs.strip()))
    return out


# --------------------------------------------------------------------------
# 1. Hand-derived shapes (P4016R0 / P4229R0 "Key Design Points")
# --------------------------------------------------------------------------
@pytest.mark.parametrize("args,expected", golden_lines(), ids=lambda v: str(v))
def test_symbolic_matches_hand_derived(args, expected):
    kind = args[0]
    if kind == "pw":
        tree = S.pw_tree(list(range(int(args[1]))))
    elif kind == "reduce":
        tree = S.reduce_tree(int(args[1]), int(args[2]))
    elif kind == "scan":
        tree = S.scan_tree(int(args[3]), args[1], int(args[2]))
    elif kind == "halving":
        tree = S.halving_tree(int(args[1]))
    else:
        raise AssertionError(kind)
    assert S.to_str(tree) == expected


def _letters_to_values(expr: str, rng, dtype):
    """Random values for the letters of an expression, and the numeric value
    obtained by parsing the hand-written string directly."""
    vals = synth.generate(26, "mixed_magnitude", int(rng.integers(1 << 30)), dtype)
    init = dtype(0.1)
    t = np.dtype(dtype).type

    def parse(s, i):
        if s[i] == "(":
            a, i = parse(s, i + 1)
            b, i = parse(s, i)
            assert s[i] == ")"
            return t(a + b), i + 1
        if s[i] == "I":
            return init, i + 1
        return vals[ord(s[i]) - ord("a")], i + 1

    v, end = parse(expr, 0)
    assert end == len(expr)
    return vals, init, v


@pytest.mark.parametrize("dtype", DTYPES)
def test_numeric_oracle_matches_hand_derived_values(dtype):
    """Evaluate the hand-written strings themselves (a parser, no tree code)
    and compare with the numeric C oracle."""
    rng = np.random.default_rng(7)
    for args, expected in golden_lines():
        if args[0] == "halving":
            continue
        for _ in range(5):
            vals, init, want = _letters_to_values(expected, rng, dtype)
            if args[0] == "pw":
                got = oracle.pw(vals[: int(args[1])])
            elif args[0] == "reduce":
                got = oracle.reduce(vals[: int(args[1])], int(args[2]), init)
            else:
                i = int(args[3])
                got = oracle.scan_prefix(vals[: i + 1], i, args[1], int(args[2]))
                got2 = oracle.scan(vals[: i + 1], args[1], int(args[2]))[i]
                assert same_bits(got2, want), (args, expected)
            assert same_bits(got, want), (args, expected)


# --------------------------------------------------------------------------
# 2. C oracle == independently built symbolic trees, evaluated numerically
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES)
def test_pw_c_equals_symbolic(dtype):
    x = synth.generate(1100, "mixed_magnitude", 11, dtype)
    for n in list(range(0, 130)) + [255, 256, 257, 511, 512, 513, 1000, 1023, 1024, 1025, 1100]:
        t = S.pw_tree(list(range(n)))
        got = oracle.pw(x[:n])
        if n == 0:
            assert got is None
        else:
            assert same_bits(got, S.evaluate(t, x)), n


@pytest.mark.parametrize("dtype", DTYPES)
def test_reduce_c_equals_symbolic(dtype):
    x = synth.generate(300, "mixed_magnitude", 12, dtype)
    for L in [1, 2, 3, 4, 5, 7, 8, 16, 32, 64, 100, 128, 1024]:
        for n in list(range(0, 40)) + [63, 64, 65, 127, 128, 129, 255, 256, 257, 300]:
            for init in (0.1, -0.0, 1.0):
                t = S.reduce_tree(n, L)
                want = S.evaluate(t, x, init)
                got = oracle.reduce(x[:n], L, init)
                assert same_bits(got, want), (L, n, init)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("policy,params", [
    ("pairwise", [0]),
    ("iterated_pairwise", [1, 2, 3, 4, 5, 8, 16, 37]),
    ("block_dyadic", [1, 2, 4, 8, 16, 64]),
])
def test_scan_c_equals_symbolic(dtype, policy, params):
    n = 140
    x = synth.generate(n, "mixed_magnitude", 13, dtype)
    for p in params:
        ys = oracle.scan(x, policy, p)
        for i in range(n):
            want = S.evaluate(S.scan_tree(i, policy, p), x)
            assert same_bits(ys[i], want), (policy, p, i)
            assert same_bits(oracle.scan_prefix(x, i, policy, p), want), (policy, p, i)


# --------------------------------------------------------------------------
# 3. streaming (shift-reduce) form == literal bottom-up form on every prefix
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES)
def test_streaming_equals_literal_all_prefixes(dtype):
    n = 700
    x = synth.generate(n, "mixed_magnitude", 14, dtype)
    cases = [("pairwise", 0)] + [("iterated_pairwise", L) for L in (1, 3, 16, 128)] + \
            [("block_dyadic", B) for B in (1, 2, 16, 256, 4096)]
    for policy, p in cases:
        ys = oracle.scan(x, policy, p)
        lit = np.array([oracle.scan_prefix(x, i, policy, p) for i in range(n)], dtype)
        assert same_bits(ys, lit), (policy, p)


def test_rows_equal_per_row_calls():
    X = synth.generate(7 * 50, "mixed_magnitude", 15).reshape(7, 50)
    r = oracle.reduce_rows(X, 4, 0.1, cols=45)
    for k in range(7):
        assert same_bits(r[k], oracle.reduce(X[k, :45], 4, 0.1))
    Y = oracle.scan_rows(X, "block_dyadic", 4, cols=45)
    for k in range(7):
        assert same_bits(Y[k, :45], oracle.scan(X[k, :45], "block_dyadic", 4))
        assert np.all(Y[k, 45:] == 0)


# --------------------------------------------------------------------------
# 4. The Futhark blog's worked example: (0.1 + 0.2) + 0.3 != 0.1 + (0.2 + 0.3)
# --------------------------------------------------------------------------
def test_worked_example_three_terms():
    a, b, c = 0.1, 0.2, 0.3
    left, right = (a + b) + c, a + (b + c)
    assert left != right  # what the blog post prints ("false")
    x = np.array([a, b, c])
    # PW groups the first pair: ((ab)c)
    assert same_bits(oracle.pw(x), left)
    assert not same_bits(oracle.pw(x), right)
    assert same_bits(oracle.scan(x, "pairwise")[2], left)


# --------------------------------------------------------------------------
# 5. Exact results
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,hi", [(np.float64, 1 << 20), (np.float32, 1 << 8)])
def test_integer_inputs_sum_exactly(dtype, hi):
    n = 2000
    x = synth.integers(n, -hi, hi, 21, dtype)
    ex = np.cumsum(x.astype(np.int64))
    for L in (1, 3, 16, 128):
        for init in (0.0, 5.0, -7.0):
            assert oracle.reduce(x, L, init) == dtype(init + int(ex[-1]))
    for policy, p in [("pairwise", 0), ("iterated_pairwise", 16), ("iterated_pairwise", 5),
                      ("block_dyadic", 16), ("block_dyadic", 256)]:
        ys = oracle.scan(x, policy, p)
        assert np.array_equal(ys.astype(np.int64), ex), (policy, p)


@pytest.mark.parametrize("dtype", DTYPES)
def test_one_hot(dtype):
    n = 77
    for k in range(n):
        x = np.zeros(n, dtype)
        x[k] = 1.0
        for L in (1, 4, 16):
            assert oracle.reduce(x, L, 0.0) == 1.0
        for policy, p in [("pairwise", 0), ("iterated_pairwise", 4), ("block_dyadic", 8)]:
            ys = oracle.scan(x, policy, p)
            assert np.array_equal(ys, (np.arange(n) >= k).astype(dtype))


@pytest.mark.parametrize("dtype", DTYPES)
def test_negative_zero_is_kept(dtype):
    """An all -0.0 input reduces to -0.0 (absent lanes take no part; an
    init of -0.0 leaves R unchanged); +0.0 padding would give +0.0."""
    for n in (1, 2, 3, 5, 17):
        x = np.full(n, -0.0, dtype)
        for L in (1, 4, 16, 32):
            r = oracle.reduce(x, L, -0.0)
            assert r == 0 and math.copysign(1.0, float(r)) < 0
        for policy, p in [("pairwise", 0), ("iterated_pairwise", 4), ("block_dyadic", 2)]:
            ys = oracle.scan(x, policy, p)
            assert np.all(np.signbit(ys))
    r = oracle.reduce(np.zeros(0, dtype), 4, -0.0)
    assert math.copysign(1.0, float(r)) < 0


def test_empty_inputs():
    for dtype in DTYPES:
        x = np.zeros(0, dtype)
        assert same_bits(oracle.reduce(x, 16, 0.25), dtype(0.25))
        assert oracle.scan(x, "pairwise").size == 0
        assert oracle.cr(x, 3) is None


# --------------------------------------------------------------------------
# 6. Closed-form identities
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES)
def test_policy_identities(dtype):
    n = 600
    x = synth.generate(n, "mixed_magnitude", 31, dtype)
    pw = oracle.scan(x, "pairwise")
    assert same_bits(oracle.scan(x, "iterated_pairwise", 1), pw)
    assert same_bits(oracle.scan(x, "block_dyadic", 1), pw)
    assert same_bits(oracle.scan(x, "block_dyadic", 1024), pw)  # B >= n
    for B in (2, 4, 16, 64):
        bd = oracle.scan(x, "block_dyadic", B)
        ends = np.arange(B - 1, n, B)
        assert same_bits(bd[ends], pw[ends]), B  # B divides the prefix length
        # the first block is a pairwise scan of its own
        assert same_bits(bd[:B], pw[:B])
    # block_dyadic<4> departs from pairwise at n = 13 (whole blocks with two
    # set bits and an open tail), but not at n = 5..12 except where stated
    assert S.to_str(S.scan_tree(12, "block_dyadic", 4)) != S.to_str(S.scan_tree(12, "pairwise"))
    ndiff = 0
    for seed in range(50):
        xs = synth.generate(13, "uniform_pm1", 300 + seed, dtype)
        ndiff += not same_bits(oracle.scan(xs, "block_dyadic", 4)[12], oracle.scan(xs, "pairwise")[12])
        # n = 5..12 with B = 4: whole blocks have one set bit or no tail: equal
        assert same_bits(oracle.scan(xs, "block_dyadic", 4)[4:12], oracle.scan(xs, "pairwise")[4:12])
    assert ndiff > 5
    # reduce with L >= n is the pairwise tree over the elements
    for m in (1, 7, 100, 128):
        assert same_bits(oracle.reduce(x[:m], 128, -0.0), pw[m - 1])
        assert same_bits(oracle.reduce(x[:m], 1, -0.0), pw[m - 1])


@pytest.mark.parametrize("dtype", DTYPES)
def test_scan_back_equals_reduce_of_same_expression(dtype):
    """inclusive_scan<E>(x)[i] == reduce<E>(x[0..i]) (P4229R0 consistency)."""
    x = synth.generate(3000, "mixed_magnitude", 32, dtype)
    for n in (1, 2, 17, 1000, 3000):
        xs = x[:n]
        for L in (1, 3, 16, 128):
            assert same_bits(oracle.scan(xs, "iterated_pairwise", L)[-1],
                             oracle.reduce(xs, L, -0.0))
        assert same_bits(oracle.scan(xs, "pairwise")[-1], oracle.reduce(xs, 1, -0.0))
        for B in (1, 16, 256):
            q, t = divmod(n, B)
            parts = []
            if q:
                parts.append(oracle.pw(np.array([oracle.pw(xs[k * B:(k + 1) * B]) for k in range(q)],
                                                dtype)))
            if t:
                parts.append(oracle.pw(xs[q * B:]))
            want = parts[0] if len(parts) == 1 else dtype(parts[0] + parts[1])
            assert same_bits(oracle.scan(xs, "block_dyadic", B)[-1], want)


# --------------------------------------------------------------------------
# 7. Aligned power-of-two chunk closure (what every parallel schedule and
#    any sharding across devices relies on)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES)
def test_aligned_chunk_closure(dtype):
    x = synth.generate(300, "mixed_magnitude", 41, dtype)
    for n in range(1, 300, 7):
        whole = oracle.pw(x[:n])
        for k in range(0, 6):
            C = 1 << k
            parts = np.array([oracle.pw(x[s:min(s + C, n)]) for s in range(0, n, C)], dtype)
            assert same_bits(oracle.pw(parts), whole), (n, C)


@pytest.mark.parametrize("dtype", DTYPES)
def test_sharded_reduce_matches(dtype):
    """Split the rows at aligned power-of-two boundaries into G shards, reduce
    each shard's lanes, gather the per-shard lane values and finish: the bits
    equal the unsharded reduce for every G."""
    L = 16
    x = synth.generate(16 * 1000 + 5, "mixed_magnitude", 42, dtype)
    n = x.size
    M = -(-n // L)
    want = oracle.reduce(x, L, 1.0)
    for G in (1, 2, 3, 4, 8):
        rows_per = 1
        while rows_per * G < M:
            rows_per *= 2
        shard_lanes = []
        for g in range(G):
            lo, hi = g * rows_per * L, min((g + 1) * rows_per * L, n)
            if lo >= n:
                break
            shard_lanes.append(oracle.lane_values(x[lo:hi], L))
        lanes = []
        for j in range(min(n, L)):
            vals = [s[j] for s in shard_lanes if j < s.size]
            lanes.append(oracle.pw(np.array(vals, dtype)))
        got = dtype(dtype(1.0) + oracle.pw(np.array(lanes, dtype)))
        assert same_bits(got, want), G


# --------------------------------------------------------------------------
# 8. Textbook error bound (sanity only, not from the pages)
# --------------------------------------------------------------------------
def test_pairwise_error_bound():
    for seed in range(5):
        x = synth.generate(5000, "mixed_magnitude", 50 + seed)
        exact = sum(Fraction(float(v)) for v in x)
        u = 2.0 ** -53
        for n in (5000, 4097, 777):
            k = math.ceil(math.log2(n))
            gamma = k * u / (1 - k * u)
            err = abs(Fraction(float(oracle.pw(x[:n]))) - sum(Fraction(float(v)) for v in x[:n]))
            assert err <= Fraction(gamma) * sum(Fraction(abs(float(v))) for v in x[:n])
        assert exact == exact


# --------------------------------------------------------------------------
# 9. Power: each rejected reading changes the bits on some seeded input
# --------------------------------------------------------------------------
def test_lane_count_changes_bits():
    distinct3 = 0
    for seed in range(4):
        x = synth.generate(1 << 16, "uniform_pm1", 61 + seed)
        r = {L: oracle.reduce(x, L, 0.0) for L in (1, 16, 128)}
        distinct3 += len({bits(v).item() for v in r.values()}) == 3
    assert distinct3 >= 1


def test_halving_tree_differs():
    ndiff = 0
    for seed in range(20):
        x = synth.generate(1024, "uniform_pm1", 62 + seed)
        ndiff += not same_bits(S.evaluate(S.halving_tree(1024), x), oracle.pw(x))
    assert ndiff >= 5


def test_floor_half_split_differs():
    """The recursive n/2 split (rejected reading) differs from PW at n = 3."""
    def half(items):
        if len(items) == 1:
            return items[0]
        h = len(items) // 2
        return (half(items[:h]), half(items[h:]))
    assert S.to_str(half(list(range(3)))) == "(a(bc))"
    x = np.array([0.1, 0.2, 0.3])
    assert not same_bits(S.evaluate(half([0, 1, 2]), x), oracle.pw(x))


def test_init_placement_matters():
    """op(init, R) once after the tree differs from folding init in as an
    element or into lane 0, for a non-integer init."""
    diff_elem = diff_lane0 = 0
    for seed in range(200):
        x = synth.generate(37, "uniform_pm1", 1000 + seed)
        init = 0.1
        got = oracle.reduce(x, 4, init)
        as_elem = oracle.cr(np.concatenate([[init], x]), 4)
        x2 = x.copy()
        x2[0] = init + x2[0]
        lane0 = oracle.cr(x2, 4)
        diff_elem += not same_bits(got, as_elem)
        diff_lane0 += not same_bits(got, lane0)
    assert diff_elem > 50 and diff_lane0 > 50


def test_left_to_right_fold_differs():
    x = synth.generate(4096, "mixed_magnitude", 63)
    acc = 0.0
    for v in x:
        acc = acc + float(v)
    assert not same_bits(oracle.pw(x), acc)
    assert same_bits(oracle.left_fold(x, 0.0), acc)


# --------------------------------------------------------------------------
# The left fold kept for the contrast (P4016R0 "Summary": std::accumulate is
# deterministic but sequential)
# --------------------------------------------------------------------------
def test_left_fold_worked_example():
    """The Futhark post's three terms: the fold is the left grouping."""
    x = np.array([0.1, 0.2, 0.3])
    assert same_bits(oracle.left_fold(x), (0.1 + 0.2) + 0.3)
    assert same_bits(oracle.left_fold_scan(x)[2], (0.1 + 0.2) + 0.3)


@pytest.mark.parametrize("dtype", DTYPES)
def test_left_fold_exact_and_prefixes(dtype):
    rng = np.random.Generator(np.random.PCG64(9))
    xi = rng.integers(-1000, 1000, 500)
    x = xi.astype(dtype)
    assert same_bits(oracle.left_fold(x, 7.0), dtype(7 + int(xi.sum())))
    ys = oracle.left_fold_scan(x, 7.0)
    assert same_bits(ys, (7 + np.cumsum(xi)).astype(dtype))
    assert same_bits(oracle.left_fold(np.zeros(0, dtype), 2.5), dtype(2.5))
    # up to three elements the left fold is the pairwise tree ((ab)c)
    y = synth.generate(3, "mixed_magnitude", 4, dtype)
    for n in (1, 2, 3):
        assert same_bits(oracle.left_fold(y[:n]), oracle.pw(y[:n]))
    # from four on they part: (((ab)c)d) against ((ab)(cd))
    z = synth.generate(4096, "mixed_magnitude", 5, dtype)
    diff = sum(not same_bits(oracle.left_fold_scan(z)[i], oracle.scan(z, "pairwise")[i])
               for i in range(3, 200))
    assert diff > 50


def test_published_golden_values_decode():
    """The README's golden values (N=1M doubles, fixed seed; L=16 and L=128)
    cannot be reproduced: seed, generator and distribution are not given.
    What can be checked: they decode to nearby doubles (about 140.48) that
    differ in the last bits, i.e. the lane count changes the result."""
    a = np.array([0x40618f71f6379380], np.uint64).view(np.float64)[0]
    b = np.array([0x40618f71f6379397], np.uint64).view(np.float64)[0]
    assert abs(a - 140.48266135077) < 1e-9 and a != b
    assert int(0x40618f71f6379397 - 0x40618f71f6379380) == 23
