"""GPU parity of a caller-defined operator built through canon_user_op.hpp
(tests/user_op/skew_op.hip, a (+) b = (a + b) + ((a/4) b) b; canonical-reduce
README, P4016R0 "Summary": the expression is defined for any operator).

The operator is neither commutative nor associative, so these tests check
what the built-in operators cannot: that every kernel (register and general
reduces, the row reduces, the pairwise / block_dyadic tiles of every shape,
both iterated_pairwise paths, the row scans, the output stage of the scans
with an initial value) applies the operator in the expression's order, left
operand on the left, with the expression's parenthesisation.  Results are
compared bit for bit with the oracle evaluated with the same operator."""
import ctypes
import os

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import assert_bit_exact, to_dev, to_host  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "user_op", "libcanon_skew.so")
KINDS = {"inclusive": 0, "exclusive": 1, "include_initial": 2}
POL = {"pairwise": 0, "iterated_pairwise": 1, "block_dyadic": 2}


@pytest.fixture(scope="module")
def canon():
    import scan_canonical_reduce_amd as c
    c.lib()
    assert torch.cuda.is_available()
    return c


@pytest.fixture(scope="module")
def skew():
    assert os.path.exists(LIB), "tests/user_op/libcanon_skew.so is built by build()"
    L = ctypes.CDLL(LIB)
    P, S, U, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_int
    for t, F in (("f64", ctypes.c_double), ("f32", ctypes.c_float)):
        getattr(L, f"canon_skew_reduce_{t}").argtypes = [P, S, U, F, P, P, S, P]
        getattr(L, f"canon_skew_reduce_rows_{t}").argtypes = [P, S, S, S, U, F, P, P, S, P]
        getattr(L, f"canon_skew_scan_{t}").argtypes = [P, P, S, I, U, I, F, P, S, P]
        getattr(L, f"canon_skew_scan_rows_{t}").argtypes = [P, S, P, S, S, S, I, U, I, F, P, S, P]
    return L


def sfx(a):
    return "f64" if a.dtype == torch.float64 else "f32"


def stream():
    return torch.cuda.current_stream().cuda_stream


def data(n, seed, dtype):
    """Values in (-1e-3, 1e-3): prefix values and skew terms stay small."""
    return (synth.generate(n, "uniform_pm1", seed) * 1e-3).astype(dtype)


def ws_tensor(nbytes):
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")


def reduce(skew, canon, xd, L, init):
    out = torch.empty(1, dtype=xd.dtype, device="cuda")
    nb = canon.reduce_workspace_bytes(xd.numel(), L, xd.element_size())
    ws = ws_tensor(nb)
    st = getattr(skew, f"canon_skew_reduce_{sfx(xd)}")(xd.data_ptr(), xd.numel(), L, init,
                                                      out.data_ptr(), ws.data_ptr(), nb, stream())
    assert st == 0, st
    return to_host(out)


def scan(skew, canon, xd, policy, param, kind, init):
    n = xd.numel()
    y = torch.empty(n + (kind == "include_initial"), dtype=xd.dtype, device="cuda")
    nb = canon.scan_workspace_bytes(n, policy, param, xd.element_size())
    ws = ws_tensor(nb)
    st = getattr(skew, f"canon_skew_scan_{sfx(xd)}")(xd.data_ptr(), y.data_ptr(), n, POL[policy],
                                                    param, KINDS[kind], init, ws.data_ptr(), nb,
                                                    stream())
    assert st == 0, st
    assert canon.workspace_error(ws) == 0
    return to_host(y)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_reduce(skew, canon, dtype):
    x = data(300_001, 91, dtype)
    xd = to_dev(x)
    for L in (1, 3, 16, 128, 1000):
        for n in (1, L + 1, 5000, x.size):
            got = reduce(skew, canon, xd[:n], L, 1.25)
            assert_bit_exact(got, [oracle.reduce(x[:n], L, 1.25, "skew")], f"L={L} n={n}")
        got = reduce(skew, canon, xd[1:], L, -0.0)  # unaligned: the general kernel
        assert_bit_exact(got, [oracle.reduce(x[1:], L, -0.0, "skew")], f"unaligned L={L}")


SCANS = [("pairwise", 0), ("block_dyadic", 2), ("block_dyadic", 16), ("block_dyadic", 256),
         ("block_dyadic", 8192), ("iterated_pairwise", 3), ("iterated_pairwise", 16),
         ("iterated_pairwise", 128), ("iterated_pairwise", 256)]


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", SCANS)
def test_scan(skew, canon, dtype, policy, param):
    """Several tiles and a ragged tail; every output kind; aligned and not."""
    n = 70_001
    x = data(n, 92, dtype)
    xd = to_dev(x)
    for kind in KINDS:
        got = scan(skew, canon, xd, policy, param, kind, 0.5)
        want = oracle.scan_with_init(x, policy, param, 0.5, kind, "skew")
        assert_bit_exact(got, want, f"{kind}")
    got = scan(skew, canon, xd[1:], policy, param, "inclusive", -0.0)
    assert_bit_exact(got, oracle.scan(x[1:], policy, param, "skew"), "unaligned")


# Every kernel family past 64 tiles (the 64-tile group rebuild, climbs to
# node levels 7 and 8, the right-spine composition, iterated_pairwise node
# levels 3 and up): FullTile (pairwise; block_dyadic<2> in float),
# LaneBlockTile (blocks inside one vector row: block_dyadic<2> in double,
# <4> in double, <16>), SplitTile (block_dyadic<4> in float, <4096> in
# double: blocks larger than a wave's span, and B of four tiles: one block
# over several tiles), WideTile (block_dyadic<256>), the one-pass
# iterated_pairwise kernel (L = 128 double, 256 both: pipelined and one tile
# per workgroup; L = 16: rows narrower than a wave), the three-kernel
# iterated_pairwise path (L = 3, 100).
LARGE_SCANS = [("pairwise", 0), ("block_dyadic", 2), ("block_dyadic", 4), ("block_dyadic", 16),
               ("block_dyadic", 256), ("block_dyadic", 4096), ("block_dyadic", 65536),
               ("iterated_pairwise", 16), ("iterated_pairwise", 128), ("iterated_pairwise", 256),
               ("iterated_pairwise", 3), ("iterated_pairwise", 100)]


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [4096, 6000])
def test_scan_chunked_lanes(skew, canon, dtype, L):
    """iterated_pairwise with the lanes of a row in chunks (L > 2048): the
    walk above the chunks and the chunk-edge shift, every kind."""
    n = 300_007
    x = data(n, 96, dtype)
    xd = to_dev(x)
    for kind in KINDS:
        print(f"[skew chunked] {np.dtype(dtype).name} L={L} {kind}", flush=True)
        got = scan(skew, canon, xd, "iterated_pairwise", L, kind, 0.5)
        want = oracle.scan_with_init(x, "iterated_pairwise", L, 0.5, kind, "skew")
        assert_bit_exact(got, want, kind)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", LARGE_SCANS)
def test_scan_large(skew, canon, dtype, policy, param):
    """2^22 + 4097 elements (512 double or 256 float tiles and a ragged
    tail), every output kind, and an unaligned start."""
    n = (1 << 22) + 4097
    x = data(n + 1, 94, dtype)
    xd = to_dev(x)
    for kind in KINDS:
        print(f"[skew large] {np.dtype(dtype).name} {policy}<{param}> {kind}", flush=True)
        got = scan(skew, canon, xd[:n], policy, param, kind, 0.5)
        want = oracle.scan_with_init(x[:n], policy, param, 0.5, kind, "skew")
        assert_bit_exact(got, want, f"{kind}")
    got = scan(skew, canon, xd[1:], policy, param, "inclusive", -0.0)
    assert_bit_exact(got, oracle.scan(x[1:], policy, param, "skew"), "unaligned")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_rows_many_tiles(skew, canon, dtype):
    """Row scans whose rows span many tiles (the row kernel's stack of tile
    nodes up to level 6; the iterated_pairwise row segments), every kind."""
    rows, cols = 6, (1 << 19) + 4099
    ld = cols + 1
    X = data(rows * ld, 95, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    e = Xd.element_size()
    for policy, param in (("pairwise", 0), ("block_dyadic", 16), ("block_dyadic", 256),
                          ("iterated_pairwise", 128), ("iterated_pairwise", 3)):
        for kind in KINDS:
            print(f"[skew rows] {np.dtype(dtype).name} {policy}<{param}> {kind}", flush=True)
            Y = torch.empty(rows, ld, dtype=Xd.dtype, device="cuda")
            nb = canon.scan_rows_workspace_bytes(rows, cols, policy, param, e)
            ws = ws_tensor(nb)
            st = getattr(skew, f"canon_skew_scan_rows_{sfx(Xd)}")(
                Xd.data_ptr(), ld, Y.data_ptr(), ld, rows, cols, POL[policy], param, KINDS[kind],
                0.75, ws.data_ptr(), nb, stream())
            assert st == 0, st
            want = oracle.scan_rows_with_init(X, policy, param, 0.75, kind, cols=cols, op="skew")
            ycols = cols + (kind == "include_initial")
            assert_bit_exact(to_host(Y)[:, :ycols], want[:, :ycols], f"{policy} {kind}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_rows(skew, canon, dtype):
    rows = 19
    for ld in (5000, 5008):
        X = data(rows * ld, 93 + ld, dtype).reshape(rows, ld)
        Xd = to_dev(X)
        e = Xd.element_size()
        for cols in (1, 700, 4096, 5000):
            out = torch.empty(rows, dtype=Xd.dtype, device="cuda")
            st = getattr(skew, f"canon_skew_reduce_rows_{sfx(Xd)}")(
                Xd.data_ptr(), rows, cols, ld, 16, 2.0, out.data_ptr(), None, 0, stream())
            assert st == 0, st
            assert_bit_exact(to_host(out), oracle.reduce_rows(X, 16, 2.0, cols=cols, op="skew"),
                             f"reduce ld={ld} cols={cols}")
            for policy, param in (("pairwise", 0), ("block_dyadic", 16),
                                  ("iterated_pairwise", 128)):
                Y = torch.empty(rows, cols + 1, dtype=Xd.dtype, device="cuda")
                nb = canon.scan_rows_workspace_bytes(rows, cols, policy, param, e)
                ws = ws_tensor(nb)
                st = getattr(skew, f"canon_skew_scan_rows_{sfx(Xd)}")(
                    Xd.data_ptr(), ld, Y.data_ptr(), cols + 1, rows, cols, POL[policy], param,
                    KINDS["include_initial"], 0.75, ws.data_ptr(), nb, stream())
                assert st == 0, st
                want = oracle.scan_rows_with_init(X, policy, param, 0.75, "include_initial",
                                                  cols=cols, op="skew")
                assert_bit_exact(to_host(Y), want[:, :cols + 1],
                                 f"scan {policy} ld={ld} cols={cols}")


def test_argument_errors(skew):
    """The caller-defined entry points check their arguments as canon.h's do."""
    fake = ctypes.c_void_p(0x1000)
    assert skew.canon_skew_reduce_f64(fake, 10, 0, 0.0, fake, None, 0, None) == 1
    assert skew.canon_skew_scan_f64(fake, fake, 10, 0, 0, 3, 0.0, None, 0, None) == 1
    assert skew.canon_skew_scan_f32(fake, fake, 1 << 20, 0, 0, 0, 0.0, None, 0, None) == 3
    assert skew.canon_skew_last_hip_error() == 0
