"""Schedule invariance on the GPU: the value is fixed by the expression, so the
bits must not change with how the work is spread over workgroups
(canonical-reduce README, P4016R0 "Summary": an implementation may schedule
the work freely as long as it returns the canonical value; P4229R0 "Key
Design Points": the expression is not the execution).

The library's schedule override (canon_set_schedule) sweeps
  * the number of row ranges (partials) of the streaming reduce, from one
    to many thousands;
  * the grid of the persistent and grid-stride kernels, from a single
    workgroup (every tile in turn, every look-back found complete) to the
    resident grid;
and every setting must give the oracle's bits."""
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
    yield c
    c.set_schedule("grid", 0)
    c.set_schedule("reduce_partials", 0)
    c.set_schedule("spin_limit", 0)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_reduce_partials(canon, dtype):
    n = 3 * (1 << 20) + 12345
    x = synth.generate(n + 1, "mixed_magnitude", 71, dtype)
    xd = to_dev(x)
    for L in (1, 16, 128, 7, 1024):
        want = oracle.reduce(x[:n], L, 1.0)
        want_u = oracle.reduce(x[1:], L, 1.0)
        for parts in (1, 2, 3, 17, 64, 256, 1000, 4096, 65536):
            with canon.schedule(reduce_partials=parts):
                got = to_host(canon.reduce(xd[:n], L, 1.0)).reshape(1)
                assert_bit_exact(got, [want], f"L={L} partials={parts}")
                got = to_host(canon.reduce(xd[1:], L, 1.0)).reshape(1)  # general kernel
                assert_bit_exact(got, [want_u], f"unaligned L={L} partials={parts}")


SCANS = [("pairwise", 0), ("block_dyadic", 16), ("block_dyadic", 256), ("block_dyadic", 4),
         ("iterated_pairwise", 128), ("iterated_pairwise", 256), ("iterated_pairwise", 5)]


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", SCANS)
def test_scan_grid(canon, dtype, policy, param):
    """Grids of 1, 2, 3, 7 and 64 workgroups and the resident grid, over
    enough tiles for look-back nodes up to level 8 (and climbs)."""
    n = (1 << 21) + 999
    x = synth.generate(n, "mixed_magnitude", 72, dtype)
    xd = to_dev(x)
    want = oracle.scan(x, policy, param)
    for grid in (1, 2, 3, 7, 64, 0):
        print(f"[schedule] {np.dtype(dtype).name} {policy}<{param}> grid={grid}", flush=True)
        with canon.schedule(grid=grid):
            got = to_host(canon.scan(xd, policy, param, check=True))
        assert_bit_exact(got, want, f"grid={grid}")
    with canon.schedule(grid=5):
        got = to_host(canon.scan_with_init(xd, policy, param, "exclusive", 0.25, check=True))
    assert_bit_exact(got, oracle.scan_with_init(x, policy, param, 0.25, "exclusive"), "exclusive")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_rows_grid(canon, dtype):
    rows, cols = 77, 9000
    X = synth.generate(rows * cols, "mixed_magnitude", 73, dtype).reshape(rows, cols)
    Xd = to_dev(X)
    want_r = {L: oracle.reduce_rows(X, L, 0.5) for L in (16, 3)}
    want_s = {p: oracle.scan_rows(X, *p) for p in (("block_dyadic", 16), ("iterated_pairwise", 128),
                                                   ("iterated_pairwise", 3))}
    for grid in (1, 3, 0):
        with canon.schedule(grid=grid):
            for L, want in want_r.items():
                assert_bit_exact(to_host(canon.reduce_rows(Xd, L, 0.5)), want,
                                 f"reduce_rows L={L} grid={grid}")
            for p, want in want_s.items():
                assert_bit_exact(to_host(canon.scan_rows(Xd, *p, check=True)), want,
                                 f"scan_rows {p} grid={grid}")


def test_bounded_wait_gives_up(canon):
    """The failure path of the bounded waits, forced from the host (a wait
    that cannot end must not hang the kernel, and the failure must reach
    the caller).
    With a bound of one poll, the reduce's finishing workgroup gives up on
    the flags of workgroups still streaming: the kernel still finishes, its
    error word is set and the binding raises.  Whether a given call waits at
    all depends on timing, so five calls must give at least one error.  The
    scans take the same path when a look-back word is late; they must finish
    either way.  With the bound restored every call is exact again."""
    n = (1 << 26) + 3
    x = synth.generate(n, "mixed_magnitude", 74)
    xd = to_dev(x)
    errors = 0
    with canon.schedule(spin_limit=1):
        for _ in range(5):
            try:
                canon.reduce(xd, 128, 1.0, check=True)
            except canon.CanonError:
                errors += 1
        for policy, param in (("pairwise", 0), ("iterated_pairwise", 128)):
            for _ in range(3):
                try:
                    canon.scan(xd, policy, param, check=True)
                except canon.CanonError:
                    pass
    assert errors >= 1, "no reduce call reported its bounded wait giving up"
    assert canon.get_schedule("spin_limit") == 0
    got = to_host(canon.reduce(xd, 128, 1.0, check=True)).reshape(1)
    assert_bit_exact(got, [oracle.reduce(x, 128, 1.0)], "reduce after")
    m = 1 << 22
    got = to_host(canon.scan(xd[:m], "pairwise", 0, check=True))
    assert_bit_exact(got, oracle.scan(x[:m], "pairwise", 0), "scan after")
