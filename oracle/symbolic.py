"""Symbolic oracle: the canonical expression trees themselves.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

A tree is a leaf (an ``int`` input index, or the string ``"I"`` for init) or a
pair ``(left, right)`` meaning ``left + right``; the left operand always covers
the lower indices.  The trees are built here from a formulation that differs
from the numeric C oracle on purpose, so that the tests can hold one against
the other:

* PW over n >= 2 items splits at the largest power of two p < n:
  ``PW(s) = PW(s[:p]) + PW(s[p:])``.  (The C oracle pairs neighbours level by
  level and carries an odd trailing element; both state the iterative
  pairwise tree of the canonical-reduce README, P4016R0 "Key Design Points".)
* the two-stage reduction, the init placement and the three scan policies
  follow P4016R0 "Key Design Points" and P4229R0 "Summary" / "Key Design
  Points", written out on trees.

``to_str`` prints a tree with letters a, b, c, ... for indices 0, 1, 2, ...;
``evaluate`` computes its value with one IEEE operation per node (addition by
default; multiplication, minimum or maximum on request) in the dtype of the
given values.
"""
from __future__ import annotations

import numpy as np


def _largest_pow2_below(n: int) -> int:
    p = 1
    while p * 2 < n:
        p *= 2
    return p


def pw_tree(items):
    """PW over a list of subtrees; None for an empty list."""
    n = len(items)
    if n == 0:
        return None
    if n == 1:
        return items[0]
    p = _largest_pow2_below(n)
    return (pw_tree(items[:p]), pw_tree(items[p:]))


def lane_trees(n: int, L: int):
    """PW tree of each lane j < min(n, L); lane j holds indices j, j+L, ..."""
    m = min(n, L)
    return [pw_tree(list(range(j, n, L))) for j in range(m)]


def cr_tree(n: int, L: int):
    """The two-stage expression CR_L over indices 0..n-1 (None if n == 0)."""
    return pw_tree(lane_trees(n, L))


def reduce_tree(n: int, L: int):
    """init + CR_L, init applied once on the left; just init when n == 0."""
    r = cr_tree(n, L)
    return "I" if r is None else ("I", r)


def scan_tree(i: int, policy: str, param: int = 0):
    """The expression whose value scan[i] returns under a policy."""
    n = i + 1
    if policy == "pairwise":
        return pw_tree(list(range(n)))
    if policy == "iterated_pairwise":
        return cr_tree(n, param)
    if policy == "block_dyadic":
        B = param
        q, t = divmod(n, B)
        H = pw_tree([pw_tree(list(range(k * B, (k + 1) * B))) for k in range(q)])
        T = pw_tree(list(range(q * B, n)))
        if H is not None and T is not None:
            return (H, T)
        return H if H is not None else T
    raise ValueError(policy)


def scan_with_init_tree(k: int, policy: str, param: int = 0, kind: str = "inclusive"):
    """Output k of a scan with an initial value: init + (the policy's tree over
    the prefix it observes), or init alone for the empty prefix.  Inclusive
    output k observes x[0..k]; exclusive and include_initial output k observe
    x[0..k-1]."""
    m = k + 1 if kind == "inclusive" else k
    if kind not in ("inclusive", "exclusive", "include_initial"):
        raise ValueError(kind)
    return "I" if m == 0 else ("I", scan_tree(m - 1, policy, param))


def halving_tree(n: int):
    """Futhark blog's sum_tree on a power-of-two n: pair element k with k + n/2,
    repeatedly.  A different exact tree, used as a contrast."""
    items = list(range(n))
    while len(items) > 1:
        m = len(items) // 2
        items = [(items[k], items[k + m]) for k in range(m)]
    return items[0]


def to_str(tree) -> str:
    if tree is None:
        return ""
    if isinstance(tree, str):
        return tree
    if isinstance(tree, int):
        return chr(ord("a") + tree) if tree < 26 else f"[{tree}]"
    return "(" + to_str(tree[0]) + to_str(tree[1]) + ")"


def _minimum(a, b):
    """IEEE 754-2019 minimum: NaN if either is NaN, -0.0 below +0.0."""
    if np.isnan(a) or np.isnan(b):
        return a + b
    if a < b or (a == b and np.signbit(a)):
        return a
    return b


def _maximum(a, b):
    """IEEE 754-2019 maximum: NaN if either is NaN, +0.0 above -0.0."""
    if np.isnan(a) or np.isnan(b):
        return a + b
    if a > b or (a == b and not np.signbit(a)):
        return a
    return b


def _skew(a, b):
    """a (+) b = (a + b) + ((a * 0.25) * b) * b, each step rounded in the
    operands' dtype."""
    t = type(a)
    s = t(a + b)
    q = t(t(a * t(0.25)) * b)
    return t(s + t(q * b))


def evaluate(tree, values, init=None, op="add"):
    """Value of a tree: one application of op ("add", "mul", "min", "max",
    "skew") in values' dtype per internal node."""
    t = values.dtype.type
    if isinstance(tree, str):
        return t(init)
    if isinstance(tree, int):
        return t(values[tree])
    a = evaluate(tree[0], values, init, op)
    b = evaluate(tree[1], values, init, op)
    if op == "add":
        return t(a + b)
    if op == "mul":
        return t(a * b)
    if op == "min":
        return t(_minimum(a, b))
    if op == "max":
        return t(_maximum(a, b))
    if op == "skew":
        return _skew(t(a), t(b))
    raise ValueError(op)


def leaves(tree):
    """Leaves in left-to-right order."""
    if isinstance(tree, (int, str)):
        return [tree]
    return leaves(tree[0]) + leaves(tree[1])


def depth(tree) -> int:
    if isinstance(tree, (int, str)):
        return 0
    return 1 + max(depth(tree[0]), depth(tree[1]))
