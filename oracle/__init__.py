"""CPU oracle for canonical reduction and canonical scans (inclusive, and with
an initial value: inclusive, exclusive, include_initial).

TEST INFRASTRUCTURE.  This package is the slow, literal statement of what the
GPU library computes, and is used only to check it: by the tests, by the
package's smoke check and by the benchmark's CPU-baseline leg.  The GPU path
never imports it, and it imports nothing from the GPU path.

Two independent implementations live here:

* ``canon_oracle.c`` (numeric, loaded through ctypes): the pairwise tree PW is
  evaluated literally bottom-up, the two-stage reduction gathers the lanes
  i mod L explicitly, and scans either evaluate one prefix from scratch
  (``scan_prefix``) or every prefix with the shift-reduce stack (``scan``).
* ``symbolic.py`` (pure Python): builds the expression tree itself from a
  different formulation (split at the largest power of two below n), prints it
  and evaluates it in exact IEEE arithmetic of the requested type.

The semantics follow the canonical-reduce README (sections "P4016R0 —
Canonical Parallel Reduction" and "P4229R0 — Canonical Parallel Scan").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = [os.path.join(_HERE, "canon_oracle.c"), os.path.join(_HERE, "canon_oracle_body.h")]

POLICIES = {"pairwise": 0, "iterated_pairwise": 1, "block_dyadic": 2}

# The operators the expression is evaluated with ("add" is +; min and max are
# IEEE 754-2019 minimum / maximum; "skew" is a (+) b = (a + b) + ((a * 0.25)
# * b) * b, neither commutative nor associative, with -0.0 as its identity:
# the operator of the caller-defined-operator tests).
OPS = ("add", "mul", "min", "max", "skew")

# Which prefix each output of a scan with an initial value observes.
SCAN_KINDS = {"inclusive": 0, "exclusive": 1, "include_initial": 2}

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _SO + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, os.path.join(_HERE, "canon_oracle.c")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        S = ctypes.c_size_t
        U = ctypes.c_uint32
        I = ctypes.c_int
        for base, ct in (("f64", ctypes.c_double), ("f32", ctypes.c_float)):
          for sfx in [base] + [f"{base}_{o}" for o in OPS if o != "add"]:
              f = getattr(L, f"oracle_apply_{sfx}"); f.argtypes = [ct, ct]; f.restype = ct
              f = getattr(L, f"oracle_pw_{sfx}"); f.argtypes = [P, S, P]; f.restype = I
              f = getattr(L, f"oracle_lane_values_{sfx}"); f.argtypes = [P, S, U, P]; f.restype = S
              f = getattr(L, f"oracle_cr_{sfx}"); f.argtypes = [P, S, U, P]; f.restype = I
              f = getattr(L, f"oracle_reduce_{sfx}"); f.argtypes = [P, S, U, ct]; f.restype = ct
              f = getattr(L, f"oracle_scan_prefix_{sfx}"); f.argtypes = [P, S, I, U, P]; f.restype = I
              f = getattr(L, f"oracle_scan_{sfx}"); f.argtypes = [P, P, S, I, U]; f.restype = I
              f = getattr(L, f"oracle_reduce_rows_{sfx}"); f.argtypes = [P, S, S, S, U, ct, P]; f.restype = None
              f = getattr(L, f"oracle_scan_rows_{sfx}"); f.argtypes = [P, S, P, S, S, S, I, U]; f.restype = I
              f = getattr(L, f"oracle_scan_with_init_{sfx}"); f.argtypes = [P, P, S, I, U, I, ct]; f.restype = I
              f = getattr(L, f"oracle_left_fold_{sfx}"); f.argtypes = [P, S, ct]; f.restype = ct
              f = getattr(L, f"oracle_left_fold_scan_{sfx}"); f.argtypes = [P, P, S, ct]; f.restype = None
              f = getattr(L, f"oracle_scan_rows_with_init_{sfx}")
              f.argtypes = [P, S, P, S, S, S, I, U, I, ct]; f.restype = I
        _lib = L
    return _lib


def _sfx(a: np.ndarray, op: str = "add") -> str:
    if op not in OPS:
        raise ValueError(f"operator {op!r} not in {OPS}")
    if a.dtype == np.float64:
        base = "f64"
    elif a.dtype == np.float32:
        base = "f32"
    else:
        raise TypeError(f"oracle supports float64/float32, got {a.dtype}")
    return base if op == "add" else f"{base}_{op}"


def _c(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.ndim != 1:
        a = a.reshape(-1)
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def apply(a, b, op: str = "add"):
    """op(a, b) once, in the dtype of a (a numpy float64 or float32 scalar)."""
    a = np.asarray(a)
    t = a.dtype.type
    return t(getattr(lib(), f"oracle_apply_{_sfx(a, op)}")(t(a), t(b)))


def pw(s: np.ndarray, op: str = "add"):
    """PW(s) as a numpy scalar of s's dtype, or None for an empty sequence."""
    s = _c(s)
    out = np.zeros(1, s.dtype)
    ok = getattr(lib(), f"oracle_pw_{_sfx(s, op)}")(_ptr(s), s.size, _ptr(out))
    return out[0] if ok else None


def lane_values(x: np.ndarray, L: int) -> np.ndarray:
    """[PW(lane 0), ..., PW(lane m-1)], m = min(n, L)."""
    x = _c(x)
    out = np.zeros(max(min(x.size, L), 1), x.dtype)
    m = getattr(lib(), f"oracle_lane_values_{_sfx(x)}")(_ptr(x), x.size, L, _ptr(out))
    return out[:m]


def cr(x: np.ndarray, L: int, op: str = "add"):
    """CR_L(x) (the two-stage expression without init), or None if empty."""
    x = _c(x)
    out = np.zeros(1, x.dtype)
    ok = getattr(lib(), f"oracle_cr_{_sfx(x, op)}")(_ptr(x), x.size, L, _ptr(out))
    return out[0] if ok else None


def reduce(x: np.ndarray, L: int, init=0.0, op: str = "add"):
    """init + CR_L(x); init when x is empty.  Returns a numpy scalar."""
    x = _c(x)
    f = getattr(lib(), f"oracle_reduce_{_sfx(x, op)}")
    return x.dtype.type(f(_ptr(x), x.size, L, x.dtype.type(init)))


def _policy(policy) -> int:
    return POLICIES[policy] if isinstance(policy, str) else int(policy)


def _check_param(policy: int, param: int) -> None:
    if policy in (1, 2) and param < 1:
        raise ValueError("iterated_pairwise / block_dyadic need param >= 1")


def scan_prefix(x: np.ndarray, i: int, policy, param: int = 0, op: str = "add"):
    """Value of the policy's expression on x[0..i], evaluated from scratch."""
    x = _c(x)
    p = _policy(policy)
    _check_param(p, param)
    out = np.zeros(1, x.dtype)
    ok = getattr(lib(), f"oracle_scan_prefix_{_sfx(x, op)}")(_ptr(x), i, p, param, _ptr(out))
    if not ok:
        raise ValueError("bad scan arguments")
    return out[0]


def scan(x: np.ndarray, policy, param: int = 0, op: str = "add") -> np.ndarray:
    """Every prefix of x under the policy (streaming shift-reduce form)."""
    x = _c(x)
    p = _policy(policy)
    _check_param(p, param)
    y = np.empty_like(x)
    ok = getattr(lib(), f"oracle_scan_{_sfx(x, op)}")(_ptr(x), _ptr(y), x.size, p, param)
    if not ok:
        raise ValueError("bad scan arguments")
    return y


def reduce_rows(X: np.ndarray, L: int, init=0.0, cols: int | None = None,
                op: str = "add") -> np.ndarray:
    """Per-row reduce of a 2-D array (rows are independent sequences).

    ``cols`` may be smaller than X.shape[1]; X.shape[1] is then the row pitch.
    """
    X = np.ascontiguousarray(X)
    rows, ld = X.shape
    cols = ld if cols is None else cols
    out = np.empty(rows, X.dtype)
    getattr(lib(), f"oracle_reduce_rows_{_sfx(X, op)}")(
        _ptr(X), rows, cols, ld, L, X.dtype.type(init), _ptr(out))
    return out


def scan_rows(X: np.ndarray, policy, param: int = 0, cols: int | None = None,
              op: str = "add") -> np.ndarray:
    """Per-row scan of a 2-D array; entries past ``cols`` in a row are left 0."""
    X = np.ascontiguousarray(X)
    rows, ld = X.shape
    cols = ld if cols is None else cols
    p = _policy(policy)
    _check_param(p, param)
    Y = np.zeros_like(X)
    ok = getattr(lib(), f"oracle_scan_rows_{_sfx(X, op)}")(
        _ptr(X), ld, _ptr(Y), ld, rows, cols, p, param)
    if not ok:
        raise ValueError("bad scan arguments")
    return Y


def _kind(kind) -> int:
    return SCAN_KINDS[kind] if isinstance(kind, str) else int(kind)


def scan_with_init(x: np.ndarray, policy, param: int = 0, init=-0.0,
                   kind="inclusive", op: str = "add") -> np.ndarray:
    """Scan with an initial value: output k is init + E(x[0..m)), init alone
    when m == 0, where m = k + 1 (inclusive) or k (exclusive,
    include_initial); include_initial has len(x) + 1 outputs.  The default
    init, -0.0, is the exact identity of IEEE addition."""
    x = _c(x)
    p = _policy(policy)
    _check_param(p, param)
    k = _kind(kind)
    y = np.empty(x.size + (1 if k == 2 else 0), x.dtype)
    ok = getattr(lib(), f"oracle_scan_with_init_{_sfx(x, op)}")(
        _ptr(x), _ptr(y), x.size, p, param, k, x.dtype.type(init))
    if not ok:
        raise ValueError("bad scan arguments")
    return y


def scan_with_init_output(x: np.ndarray, k: int, policy, param: int = 0, init=-0.0,
                          kind="inclusive", op: str = "add"):
    """Output k of scan_with_init, evaluated from scratch: op(init, the
    policy's expression over the prefix it observes) (scan_prefix), one
    application in x's dtype; init alone for the empty prefix."""
    x = _c(x)
    kd = _kind(kind)
    m = k + 1 if kd == 0 else k
    if kd not in (0, 1, 2) or k < 0 or m > x.size or (kd != 2 and k >= x.size):
        raise ValueError("bad output index or kind")
    t = x.dtype.type
    if m == 0:
        return t(init)
    return apply(t(init), scan_prefix(x, m - 1, policy, param, op), op)


def scan_rows_with_init(X: np.ndarray, policy, param: int = 0, init=-0.0, kind="inclusive",
                        cols: int | None = None, op: str = "add") -> np.ndarray:
    """Per-row scan_with_init of a 2-D array (``cols`` as in scan_rows).  The
    result has X.shape[1] columns, or X.shape[1] + 1 for include_initial;
    entries past a row's outputs are left 0."""
    X = np.ascontiguousarray(X)
    rows, ld = X.shape
    cols = ld if cols is None else cols
    p = _policy(policy)
    _check_param(p, param)
    k = _kind(kind)
    ldy = ld + (1 if k == 2 else 0)
    Y = np.zeros((rows, ldy), X.dtype)
    ok = getattr(lib(), f"oracle_scan_rows_with_init_{_sfx(X, op)}")(
        _ptr(X), ld, _ptr(Y), ldy, rows, cols, p, param, k, X.dtype.type(init))
    if not ok:
        raise ValueError("bad scan arguments")
    return Y


def left_fold(x: np.ndarray, init=-0.0):
    """((init + x0) + x1) + ... in x's dtype: the sequential fold the canonical
    expression replaces.  A contrast, not an expression the library computes."""
    x = _c(x)
    return x.dtype.type(getattr(lib(), f"oracle_left_fold_{_sfx(x)}")(
        _ptr(x), x.size, x.dtype.type(init)))


def left_fold_scan(x: np.ndarray, init=-0.0) -> np.ndarray:
    """Every prefix of the left fold (init in front of each)."""
    x = _c(x)
    y = np.empty_like(x)
    getattr(lib(), f"oracle_left_fold_scan_{_sfx(x)}")(_ptr(x), _ptr(y), x.size,
                                                       x.dtype.type(init))
    return y
