"""GPU parity: the HIP library through its C ABI against the CPU oracle, bit
for bit (0 ULP; NaN compared by class), on seeded synthetic inputs.

Sizes span several tiles / workgroups and ragged tails; the full-size
workloads are in test_gpu_fullsize.py."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import assert_bit_exact, scan_rows_tile, scan_tile, to_dev, to_host  # noqa: E402

DT = {np.float64: torch.float64, np.float32: torch.float32}


@pytest.fixture(scope="module")
def canon():
    import scan_canonical_reduce_amd as c
    c.lib()
    assert torch.cuda.is_available()
    return c


def gpu_reduce(canon, x, L, init):
    r = canon.reduce(to_dev(x), L, init)
    return to_host(r).reshape(1)


# ----------------------------------------------------------------- reduce
@pytest.mark.parametrize("L", [16, 128])
@pytest.mark.parametrize("init", [0.0, 0.1, -0.0])
def test_reduce_1m_uniform(canon, L, init):
    x = synth.config_input("reduce_1m")
    assert_bit_exact(gpu_reduce(canon, x, L, init), [oracle.reduce(x, L, init)], f"L={L}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [1, 2, 3, 4, 5, 7, 8, 16, 32, 64, 100, 128, 256, 512, 1024, 3000,
                               4096, 65536])
def test_reduce_tails(canon, dtype, L):
    x = synth.generate(300_000, "mixed_magnitude", 7000 + L, dtype)
    ns = sorted({0, 1, 2, 3, L - 1, L, L + 1, 2 * L + 3, 1000, 4095, 4096, 4097, 65535, 65536,
                 65537, 131072 + 77, 300_000} - {-1})
    for n in ns:
        if n < 0 or n > x.size:
            continue
        xs = x[:n]
        assert_bit_exact(gpu_reduce(canon, xs, L, 0.1), [oracle.reduce(xs, L, 0.1)],
                         f"n={n} L={L}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [1, 16, 128, 7])
def test_reduce_unaligned_input(canon, dtype, L):
    """A view starting one element in is not 16-byte aligned: other path."""
    base = synth.generate(200_001, "mixed_magnitude", 88, dtype)
    xb = to_dev(base)
    xs = xb[1:]
    got = to_host(canon.reduce(xs, L, 1.0)).reshape(1)
    assert_bit_exact(got, [oracle.reduce(base[1:], L, 1.0)], f"L={L}")


def test_reduce_negative_zero_and_special_values(canon):
    for L in (1, 4, 16, 128):
        for n in (1, 3, 17, 300):
            x = np.full(n, -0.0)
            got = gpu_reduce(canon, x, L, -0.0)
            assert_bit_exact(got, [oracle.reduce(x, L, -0.0)], "all -0")
            assert np.signbit(got[0])
    x = synth.generate(5000, "uniform_pm1", 5)
    x[17] = np.inf
    x[999] = -np.inf
    x[2000] = np.nan
    for L in (1, 16, 100):
        assert_bit_exact(gpu_reduce(canon, x, L, 0.0), [oracle.reduce(x, L, 0.0)], "nan")
    x = synth.generate(5000, "uniform_pm1", 6)
    x[3] = np.inf
    for L in (1, 16, 100):
        assert_bit_exact(gpu_reduce(canon, x, L, 0.0), [oracle.reduce(x, L, 0.0)], "inf")


def test_reduce_cancellation(canon):
    x = synth.generate(100_000, "mixed_magnitude", 9)
    x = np.concatenate([x, -x[::-1]])
    for L in (1, 16, 128):
        assert_bit_exact(gpu_reduce(canon, x, L, 0.0), [oracle.reduce(x, L, 0.0)], f"L={L}")


def test_reduce_repeatable(canon):
    x = synth.generate(3_000_001, "mixed_magnitude", 10)
    xd = to_dev(x)
    want = oracle.reduce(x, 128, 1.0)
    for _ in range(20):
        assert_bit_exact(to_host(canon.reduce(xd, 128, 1.0)).reshape(1), [want], "repeat")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_reduce_workspace_reuse(canon, dtype):
    """The finishing workgroup waits for flags tagged with the call's own id:
    whatever a workspace holds on entry (all bits set, random bytes, the
    flags and partials of earlier calls with larger and smaller grids, other
    lane counts, the general kernel), every call gives the oracle's bits and
    leaves its error word 0."""
    n_big = 5_000_003
    x = synth.generate(n_big + 1, "mixed_magnitude", 12, dtype)
    xd = to_dev(x)
    es = xd.element_size()
    nb = max(canon.reduce_workspace_bytes(n, L, es) for n in (n_big, 777, 65_536)
             for L in (1, 16, 128, 1000))
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    cases = [(n_big, 128), (777, 16), (n_big, 16), (65_536, 1000), (n_big, 1), (777, 128)]
    for i, (n, L) in enumerate(cases):
        if i == 3:
            ws.copy_(torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda"))
        for start in (0, 1):  # aligned: register kernel; start 1: general kernel
            got = to_host(canon.reduce(xd[start:start + n], L, 0.5, ws=ws, check=True))
            assert_bit_exact(got.reshape(1), [oracle.reduce(x[start:start + n], L, 0.5)],
                             f"n={n} L={L} start={start}")
            assert canon.workspace_error(ws) == 0


# ------------------------------------------------------------ reduce rows
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [1, 3, 16, 128, 300, 1024])
def test_reduce_rows(canon, dtype, L):
    rows, ld = 37, 5003
    X = synth.generate(rows * ld, "uniform_pm1", 11 + L, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for cols in (0, 1, 15, 16, 17, 4096, 5000, 5003):
        got = to_host(canon.reduce_rows(Xd[:, :cols], L, 0.1))
        want = oracle.reduce_rows(X, L, 0.1, cols=cols)
        assert_bit_exact(got, want, f"cols={cols}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [1, 2, 4, 16, 64, 128, 256])
def test_reduce_rows_aligned(canon, dtype, L):
    """16-byte aligned rows and a power-of-two L: the one-wave-per-row
    register kernel (for L up to one wave-wide load per row of L), ragged
    row ends, a row count that is not a multiple of the rows per workgroup."""
    rows, ld = 37, 5008
    X = synth.generate(rows * ld, "mixed_magnitude", 40 + L, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for cols in (0, 1, L - 1, L, L + 1, 1023, 1024, 1025, 2049, 4096, 5000, 5008):
        if cols < 0:
            continue
        got = to_host(canon.reduce_rows(Xd[:, :cols], L, 0.1))
        want = oracle.reduce_rows(X, L, 0.1, cols=cols)
        assert_bit_exact(got, want, f"cols={cols}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_reduce_rows_long_rows(canon, dtype):
    """Rows around the register kernel's length limit (64 batches of one
    wave each) and past it (the general row kernel)."""
    e = 2 if dtype == np.float64 else 4
    limit = 64 * 8 * e * 64
    rows, ld = 5, limit + 16
    X = synth.generate(rows * ld, "mixed_magnitude", 47, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for cols in (limit - 1, limit, limit + 1, ld):
        got = to_host(canon.reduce_rows(Xd[:, :cols], 16, -2.5))
        assert_bit_exact(got, oracle.reduce_rows(X, 16, -2.5, cols=cols), f"cols={cols}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [1, 3, 16])
def test_reduce_rows_several_rounds(canon, dtype, L):
    """Rows the general row kernel covers in several rounds: each thread's
    segment is capped at 2^13 rows-of-L (its batch stack's depth), so a row
    of more than 2^13 * S rows-of-L (S = 256 / min(Lp, 256) threads per lane)
    is reduced round by round, the rounds merged per lane.  2^21 + 17
    columns: two rounds for L = 1, 3 and 16; 3 * 2^21 + 5: four to six."""
    for cols in ((1 << 21) + 17, 3 * (1 << 21) + 5):
        rows, ld = 2, cols + 3
        X = synth.generate(rows * ld, "mixed_magnitude", 48 + L + cols % 7, dtype).reshape(rows, ld)
        print(f"[rows rounds] L={L} cols={cols} {np.dtype(dtype).name}", flush=True)
        got = to_host(canon.reduce_rows(to_dev(X)[:, :cols], L, 0.1))
        assert_bit_exact(got, oracle.reduce_rows(X, L, 0.1, cols=cols), f"cols={cols}")


def test_reduce_rows_shape_of_workload(canon):
    rows, cols = 2048, 4096
    X = synth.generate(rows * cols, "uniform_pm1", 1004).reshape(rows, cols)
    assert_bit_exact(to_host(canon.reduce_rows(to_dev(X), 16, 0.0)),
                     oracle.reduce_rows(X, 16, 0.0), "rows")


# ------------------------------------------------------------------- scan
def gpu_scan(canon, x, policy, param):
    xd = to_dev(x)
    ws = torch.empty(max(canon.scan_workspace_bytes(x.size, policy, param, x.itemsize), 1),
                     dtype=torch.uint8, device="cuda")
    y = canon.scan(xd, policy, param, ws=ws)
    out = to_host(y)
    if x.size:
        assert canon.workspace_error(ws) == 0
    return out


@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 256)])
def test_scan_1m_uniform(canon, policy, param):
    x = synth.config_input("scan_1m")
    y = gpu_scan(canon, x, policy, param)
    assert_bit_exact(y, oracle.scan(x, policy, param), policy)
    # scan back element == canonical reduce of the same expression (GPU reduce)
    assert_bit_exact(y[-1:], gpu_reduce(canon, x, 1, -0.0), "back == reduce")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 1), ("block_dyadic", 2),
                                          ("block_dyadic", 4), ("block_dyadic", 16),
                                          ("block_dyadic", 256), ("block_dyadic", 4096),
                                          ("block_dyadic", 8192), ("block_dyadic", 65536)])
def test_scan_tails(canon, dtype, policy, param):
    S = scan_tile(dtype, policy, param)  # elements per scan tile
    x = synth.generate(70 * S + 999, "mixed_magnitude", 12, dtype)
    want_all = oracle.scan(x, policy, param)
    for n in (1, 2, 3, 17, S - 1, S, S + 1, 3 * S + 5, 64 * S - 1, 64 * S, 64 * S + 1, 65 * S + 17,
              x.size):
        y = gpu_scan(canon, x[:n], policy, param)
        assert_bit_exact(y, want_all[:n], f"n={n}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_scan_every_block_size(canon, dtype):
    """Every B = 2^b from 1 to beyond one tile: the fork to block values falls
    at every level inside and above the tile; several tiles, a ragged tail."""
    S = scan_tile(dtype)
    x = synth.generate(5 * S + 123, "mixed_magnitude", 18, dtype)
    for b in range(0, 17):
        B = 1 << b
        assert_bit_exact(gpu_scan(canon, x, "block_dyadic", B), oracle.scan(x, "block_dyadic", B),
                         f"B={B}")
        # an unaligned start (element loads and stores)
        xd = to_dev(x)
        y = to_host(canon.scan(xd[1:], "block_dyadic", B))
        assert_bit_exact(y, oracle.scan(x[1:], "block_dyadic", B), f"unaligned B={B}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 16),
                                          ("block_dyadic", 256)])
def test_scan_many_tiles(canon, dtype, policy, param):
    """Enough tiles for published nodes up to tile level 9."""
    x = synth.generate((1 << 22) + 12345, "mixed_magnitude", 13, dtype)
    y = gpu_scan(canon, x, policy, param)
    assert_bit_exact(y, oracle.scan(x, policy, param), policy)


def test_scan_in_place_and_unaligned(canon):
    x = synth.generate(500_001, "mixed_magnitude", 14)
    for policy, param in (("pairwise", 0), ("block_dyadic", 16)):
        xd = to_dev(x)
        canon.scan(xd, policy, param, out=xd)
        assert_bit_exact(to_host(xd), oracle.scan(x, policy, param), "in place")
        base = to_dev(x)
        y = canon.scan(base[1:], policy, param)
        assert_bit_exact(to_host(y), oracle.scan(x[1:], policy, param), "unaligned")


def test_scan_repeatable(canon):
    x = synth.generate(2_000_003, "mixed_magnitude", 15)
    want = oracle.scan(x, "block_dyadic", 256)
    xd = to_dev(x)
    for _ in range(10):
        assert_bit_exact(to_host(canon.scan(xd, "block_dyadic", 256)), want, "repeat")


def test_scan_special_values(canon):
    x = synth.generate(100_000, "uniform_pm1", 16)
    x[:50] = -0.0
    x[5000] = np.inf
    x[70000] = np.nan
    for policy, param in (("pairwise", 0), ("block_dyadic", 16)):
        assert_bit_exact(gpu_scan(canon, x, policy, param), oracle.scan(x, policy, param), policy)


# -------------------------------------------------------------- scan rows
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 2), ("block_dyadic", 16),
                                          ("block_dyadic", 4096)])
def test_scan_rows(canon, dtype, policy, param):
    rows, ld = 19, 3 * 16384 + 40
    X = synth.generate(rows * ld, "mixed_magnitude", 17, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for cols in (1, 16, 4095, 4096, 8193, 16385, 3 * 16384 + 33):
        got = to_host(canon.scan_rows(Xd[:, :cols], policy, param))
        want = oracle.scan_rows(X, policy, param, cols=cols)[:, :cols]
        assert_bit_exact(got, want, f"cols={cols}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_scan_rows_every_block_size(canon, dtype):
    S = scan_rows_tile(dtype)
    rows, cols, ld = 5, 2 * S + 77, 2 * S + 128
    X = synth.generate(rows * ld, "mixed_magnitude", 19, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for b in range(0, 17):
        B = 1 << b
        got = to_host(canon.scan_rows(Xd[:, :cols], "block_dyadic", B))
        want = oracle.scan_rows(X, "block_dyadic", B, cols=cols)[:, :cols]
        assert_bit_exact(got, want, f"B={B}")


def test_scan_rows_shape_of_workload(canon):
    rows, cols = 2048, 4096
    X = synth.generate(rows * cols, "uniform_pm1", 1004).reshape(rows, cols)
    got = to_host(canon.scan_rows(to_dev(X), "block_dyadic", 16))
    assert_bit_exact(got, oracle.scan_rows(X, "block_dyadic", 16), "rows")
    # per row, the last prefix equals the pairwise reduce of the row (16 | 4096)
    assert_bit_exact(got[:, -1], oracle.reduce_rows(X, 1, -0.0), "row back == PW(row)")


# ------------------------------------------------- iterated_pairwise scan
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [1, 2, 3, 5, 7, 16, 100, 128, 256, 1024, 2048])
def test_scan_iterated_pairwise(canon, dtype, L):
    x = synth.generate(200_003, "mixed_magnitude", 300 + L, dtype)
    want_all = oracle.scan(x[:60_000] if L > 128 else x, "iterated_pairwise", L)
    for n in (1, 2, L - 1, L, L + 1, 3 * L + 2, 5000, 60_000, x.size):
        if n <= 0 or n > want_all.size:
            continue
        y = gpu_scan(canon, x[:n], "iterated_pairwise", L)
        assert_bit_exact(y, want_all[:n], f"n={n}")
        # the last prefix is the canonical reduce with the same L (GPU reduce)
        assert_bit_exact(y[-1:], gpu_reduce(canon, x[:n], L, -0.0), f"back n={n}")


def test_scan_iterated_pairwise_many_tiles(canon):
    x = synth.generate((1 << 21) + 777, "mixed_magnitude", 401)
    for L in (16, 128, 256):
        y = gpu_scan(canon, x, "iterated_pairwise", L)
        assert_bit_exact(y, oracle.scan(x, "iterated_pairwise", L), f"L={L}")


def test_scan_iterated_pairwise_in_place_unaligned(canon):
    x = synth.generate(100_001, "mixed_magnitude", 402)
    xd = to_dev(x)
    canon.scan(xd, "iterated_pairwise", 128, out=xd)
    assert_bit_exact(to_host(xd), oracle.scan(x, "iterated_pairwise", 128), "in place")
    base = to_dev(x)
    y = canon.scan(base[1:], "iterated_pairwise", 7)
    assert_bit_exact(to_host(y), oracle.scan(x[1:], "iterated_pairwise", 7), "unaligned")


@pytest.mark.parametrize("dtype,L", [(np.float64, 128), (np.float64, 256), (np.float64, 1024),
                                     (np.float32, 256), (np.float32, 1024)])
def test_scan_iterated_pairwise_unaligned_register_geometry(canon, dtype, L):
    """L = 64 E 2^k with a start off the 16-byte grid: the one-pass kernel with
    element loads and stores; several tiles, a ragged tail, in place, and an
    exclusive scan with an initial value."""
    n = 200_003
    x = synth.generate(n + 1, "mixed_magnitude", 404 + L, dtype)
    base = to_dev(x)
    y = canon.scan(base[1:], "iterated_pairwise", L)
    assert_bit_exact(to_host(y), oracle.scan(x[1:], "iterated_pairwise", L), "unaligned")
    canon.scan(base[1:], "iterated_pairwise", L, out=base[1:])
    assert_bit_exact(to_host(base[1:]), oracle.scan(x[1:], "iterated_pairwise", L), "in place")
    base = to_dev(x)
    y = canon.scan_with_init(base[1:], "iterated_pairwise", L, "exclusive", 0.5)
    assert_bit_exact(to_host(y), oracle.scan_with_init(x[1:], "iterated_pairwise", L, 0.5,
                                                       "exclusive"), "exclusive")


NARROW = ([(np.float64, L) for L in (2, 4, 8, 16, 32, 64)] +
          [(np.float32, L) for L in (4, 8, 16, 32, 64, 128)])


@pytest.mark.parametrize("dtype,L", NARROW)
def test_scan_iterated_pairwise_narrow_rows(canon, dtype, L):
    """Register geometry with rows narrower than a wave (L = E .. 32 E, a
    wave holding 64 E / L row groups): past 64 tiles (node climbs to level
    6 and up) with a ragged last row, a start off the 16-byte grid, in
    place, the exclusive and include_initial kinds, and rows."""
    S = scan_tile(dtype, "iterated_pairwise", L)
    assert S == 4096 * (2 if dtype == np.float64 else 4)
    n = 67 * S + L // 2 + 3
    x = synth.generate(n + 1, "mixed_magnitude", 510 + L, dtype)
    want = oracle.scan(x[:n], "iterated_pairwise", L)
    assert_bit_exact(to_host(canon.scan(to_dev(x[:n]), "iterated_pairwise", L)), want, "aligned")
    base = to_dev(x)
    want1 = oracle.scan(x[1:], "iterated_pairwise", L)
    assert_bit_exact(to_host(canon.scan(base[1:], "iterated_pairwise", L)), want1, "unaligned")
    canon.scan(base[1:], "iterated_pairwise", L, out=base[1:])
    assert_bit_exact(to_host(base[1:]), want1, "in place")
    xd = to_dev(x[:n])
    for kind in ("exclusive", "include_initial"):
        got = to_host(canon.scan_with_init(xd, "iterated_pairwise", L, kind, 0.5))
        assert_bit_exact(got, oracle.scan_with_init(x[:n], "iterated_pairwise", L, 0.5, kind),
                         kind)
    rows, cols, ld = 5, 2 * S + L + 1, 2 * S + 2 * L + 2
    X = synth.generate(rows * ld, "mixed_magnitude", 520 + L, dtype).reshape(rows, ld)
    got = to_host(canon.scan_rows(to_dev(X)[:, :cols], "iterated_pairwise", L))
    for r in range(rows):
        assert_bit_exact(got[r], oracle.scan(X[r, :cols], "iterated_pairwise", L), f"row {r}")


# iterated_pairwise with L > 2048: the lanes of a row are cut into chunks of
# 512 (their trees in LDS), the trees above the chunks come from the
# workspace; tiles of 4 rows (double) or 8 rows (float).
CHUNK = 512


def chunk_edge_probes(n, L, rows, seed, sparse_rows=()):
    """Outputs at chunk edges (first and last lanes of chunks, the lanes
    either side) of every chunk in `rows` and of a few chunks (the first,
    the middle and the last ones) in `sparse_rows`, at row starts and ends,
    and random ones, below n."""
    rng = np.random.default_rng(seed)
    nc = (L + CHUNK - 1) // CHUNK

    def lanes(chunks):
        v = {0, 1, L - 1, L - 2}
        for c in chunks:
            v |= {c * CHUNK - 1, c * CHUNK, c * CHUNK + 1}
        return [u for u in v if 0 <= u < L]

    idx = {r * L + v for r in rows for v in lanes(range(1, nc))}
    few = {1, 2, nc // 2 - 1, nc // 2, nc // 2 + 1, nc - 1}
    idx |= {r * L + v for r in sparse_rows for v in lanes(c for c in few if 0 < c < nc)}
    idx |= set(rng.integers(0, n, 64).tolist()) | {n - 1}
    return np.array(sorted(i for i in idx if 0 <= i < n), dtype=np.int64)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [4096, 5000])
def test_scan_iterated_pairwise_chunked_lanes(canon, dtype, L):
    """Every prefix over 20 to 40 tiles and a ragged tail, ragged shorter
    inputs at tile and row edges, and the back element against the GPU
    reduce with the same L."""
    x = synth.generate(656_137, "mixed_magnitude", 420 + L, dtype)
    want_all = oracle.scan(x, "iterated_pairwise", L)
    S = scan_tile(dtype, "iterated_pairwise", L)
    for n in (1, L - 1, L, L + 1, 3 * L + 5, S - 1, S, S + 1, 5 * S + 3, x.size):
        print(f"[ip chunked] {np.dtype(dtype).name} L={L} n={n}", flush=True)
        y = gpu_scan(canon, x[:n], "iterated_pairwise", L)
        assert_bit_exact(y, want_all[:n], f"n={n}")
    assert_bit_exact(y[-1:], gpu_reduce(canon, x, L, -0.0), "back == reduce")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_scan_iterated_pairwise_largest_L(canon, dtype):
    """L = 65536 (128 chunks per row) over several tiles: outputs at every
    chunk edge of several rows, row starts and ends and random ones,
    evaluated from scratch; the back element against the GPU reduce."""
    L = 65536
    n = 9 * 4 * L + 12345
    x = synth.generate(n, "mixed_magnitude", 430, dtype)
    y = gpu_scan(canon, x, "iterated_pairwise", L)
    idx = chunk_edge_probes(n, L, (0, 1), 431, sparse_rows=(4, 5, 17, 35, 36))
    want = np.array([oracle.scan_prefix(x, int(i), "iterated_pairwise", L) for i in idx])
    assert_bit_exact(y[idx], want, "chunk-edge probes")
    assert_bit_exact(y[-1:], gpu_reduce(canon, x, L, -0.0), "back == reduce")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("kind", ["exclusive", "include_initial", "inclusive"])
def test_scan_iterated_pairwise_chunked_with_init(canon, dtype, kind):
    """The shifted kinds read the value before a chunk's first lane from the
    chunk trees: every output at L = 4096, chunk-edge outputs at 65536."""
    x = synth.generate(200_003, "mixed_magnitude", 432, dtype)
    got = to_host(canon.scan_with_init(to_dev(x), "iterated_pairwise", 4096, kind, 0.375))
    assert_bit_exact(got, oracle.scan_with_init(x, "iterated_pairwise", 4096, 0.375, kind),
                     f"L=4096 {kind}")
    L = 65536
    n = 5 * L + 777
    x = synth.generate(n, "mixed_magnitude", 433, dtype)
    got = to_host(canon.scan_with_init(to_dev(x), "iterated_pairwise", L, kind, 0.375))
    m = n + (kind == "include_initial")
    idx = chunk_edge_probes(m, L, (0, 1), 434, sparse_rows=(4, 5))
    want = np.array([oracle.scan_with_init_output(x, int(k), "iterated_pairwise", L, 0.375, kind)
                     for k in idx])
    assert_bit_exact(got[idx], want, f"L=65536 {kind}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_scan_rows_iterated_pairwise_chunked_lanes(canon, dtype):
    rows, ld = 3, 2 * 16384 + 4200
    X = synth.generate(rows * ld, "mixed_magnitude", 435, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for L, cols in ((4096, 2 * 16384 + 4097), (4097, ld), (8192, 8191)):
        got = to_host(canon.scan_rows(Xd[:, :cols], "iterated_pairwise", L))
        want = oracle.scan_rows(X, "iterated_pairwise", L, cols=cols)[:, :cols]
        assert_bit_exact(got, want, f"L={L} cols={cols}")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("L", [3, 16, 128])
def test_scan_rows_iterated_pairwise(canon, dtype, L):
    rows, ld = 23, 9001
    X = synth.generate(rows * ld, "mixed_magnitude", 403 + L, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for cols in (1, 17, L, 4096, 9001):
        got = to_host(canon.scan_rows(Xd[:, :cols], "iterated_pairwise", L))
        want = oracle.scan_rows(X, "iterated_pairwise", L, cols=cols)[:, :cols]
        assert_bit_exact(got, want, f"cols={cols}")


@pytest.mark.parametrize("dtype,L", [(np.float64, 128), (np.float64, 256), (np.float64, 1024),
                                     (np.float32, 256), (np.float32, 512)])
def test_scan_rows_iterated_pairwise_aligned_pitch(canon, dtype, L):
    """Row pitch a multiple of 16 bytes: the register path of the scan."""
    rows, ld = 9, 40960
    X = synth.generate(rows * ld, "mixed_magnitude", 410 + L, dtype).reshape(rows, ld)
    Xd = to_dev(X)
    for cols in (L, 3 * L + 8, 20000, 40960):
        got = to_host(canon.scan_rows(Xd[:, :cols], "iterated_pairwise", L))
        want = oracle.scan_rows(X, "iterated_pairwise", L, cols=cols)[:, :cols]
        assert_bit_exact(got, want, f"cols={cols}")


# ------------------------------------------------------- use of the ABI
def test_workspace_reused_across_policies_and_sizes(canon):
    """One workspace, sized for the largest call, serves calls of every policy
    and size in turn on one stream (each call re-initialises what it uses)."""
    x = synth.generate(3 * 16384 * 4 + 77, "mixed_magnitude", 501)
    cases = [("pairwise", 0), ("block_dyadic", 16), ("iterated_pairwise", 128),
             ("block_dyadic", 4096), ("pairwise", 0)]
    nb = max(canon.scan_workspace_bytes(x.size, p, q, 8) for p, q in cases)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    xd = to_dev(x)
    for n in (x.size, 1000, x.size // 2 + 3):
        for p, q in cases:
            y = to_host(canon.scan(xd[:n], p, q, ws=ws))
            assert_bit_exact(y, oracle.scan(x[:n], p, q), f"{p}<{q}> n={n}")
            assert canon.workspace_error(ws) == 0


def test_concurrent_streams(canon):
    """Scans on two streams at once, each with its own workspace, from two
    host threads: the results are those of the oracle."""
    import threading
    xs = [synth.generate((1 << 21) + 5, "mixed_magnitude", 502 + i) for i in range(2)]
    pols = [("block_dyadic", 256), ("pairwise", 0)]
    wants = [oracle.scan(xs[i], *pols[i]) for i in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    xd = [to_dev(x) for x in xs]
    ys = [torch.empty_like(d) for d in xd]
    wss = [torch.empty(canon.scan_workspace_bytes(xs[i].size, *pols[i], 8), dtype=torch.uint8,
                       device="cuda") for i in range(2)]
    torch.cuda.synchronize()
    errors = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(5):
                    canon.scan(xd[i], *pols[i], out=ys[i], ws=wss[i])
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        assert_bit_exact(to_host(ys[i]), wants[i], f"stream {i}")
