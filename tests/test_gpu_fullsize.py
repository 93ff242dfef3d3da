"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same entry points, same 16-byte aligned resident inputs).

The reduce and every scan are compared element by element with the oracle
(its streaming form computes every prefix at this size: about 18 s of host
time for iterated_pairwise<128> at 2^27, 36 s at 2^28), on sampled prefixes
evaluated from scratch (the literal form), and through scan/reduce
consistency (the scan's back element against the GPU reduce of the same
expression, a different kernel)."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")

from gpu_util import assert_bit_exact, to_dev, to_host  # noqa: E402


@pytest.fixture(scope="module")
def canon():
    import scan_canonical_reduce_amd as c
    c.lib()
    return c


def _probes(n, k=6, seed=77):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, n // 2, n - 1], rng.integers(0, n, k)]))


@pytest.mark.parametrize("name,L,init", [("reduce_1m", 16, 0.0), ("reduce_1m", 128, 0.0),
                                         ("reduce_2e28_f64", 128, 1.0),
                                         ("reduce_2e29_f32", 128, 1.0)])
def test_reduce_full_size(canon, name, L, init):
    print(f"[fullsize] reduce {name} L={L}", flush=True)
    x = synth.config_input(name)
    got = to_host(canon.reduce(to_dev(x), L, init)).reshape(1)
    assert_bit_exact(got, [oracle.reduce(x, L, init)], name)


def test_rows_full_size(canon):
    print("[fullsize] rows 16384x4096", flush=True)
    X = synth.config_input("rows_16384x4096")
    Xd = to_dev(X)
    assert_bit_exact(to_host(canon.reduce_rows(Xd, 16, 0.0)), oracle.reduce_rows(X, 16, 0.0),
                     "reduce_rows")
    Y = to_host(canon.scan_rows(Xd, "block_dyadic", 16))
    W = oracle.scan_rows(X, "block_dyadic", 16)
    assert_bit_exact(Y, W, "scan_rows")
    # 16 divides 4096: each row's last prefix is the pairwise value of the row
    assert_bit_exact(Y[:, -1], oracle.reduce_rows(X, 1, -0.0), "row back")


@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 256)])
def test_scan_1m_full(canon, policy, param):
    print(f"[fullsize] scan_1m {policy}<{param}>", flush=True)
    x = synth.config_input("scan_1m")
    y = to_host(canon.scan(to_dev(x), policy, param))
    assert_bit_exact(y, oracle.scan(x, policy, param), policy)
    assert_bit_exact(y[-1:], to_host(canon.reduce(to_dev(x), 1, -0.0)).reshape(1), "back")


@pytest.mark.parametrize("name,policy,param", [
    ("scan_2e27_f64", "block_dyadic", 16), ("scan_2e27_f64", "block_dyadic", 256),
    ("scan_2e28_f32", "block_dyadic", 256)])
def test_scan_full_size(canon, name, policy, param):
    print(f"[fullsize] {name} {policy}<{param}>", flush=True)
    x = synth.config_input(name)
    xd = to_dev(x)
    y = canon.scan(xd, policy, param)
    yh = to_host(y)
    assert_bit_exact(yh, oracle.scan(x, policy, param), name)
    # B divides N: the last prefix is the pairwise value of x (GPU reduce, L = 1)
    back = to_host(canon.reduce(xd, 1, -0.0)).reshape(1)
    assert_bit_exact(yh[-1:], back, "scan back == reduce (GPU)")


def _check_ip_every_prefix(x, y, L, seed):
    """Every prefix against the oracle's streaming form, and sampled
    prefixes against its literal form."""
    yh = to_host(y)
    assert_bit_exact(yh, oracle.scan(x, "iterated_pairwise", L), "every prefix")
    # a literal prefix costs O(i) (about 5 s at 2^28): fewer random probes there
    idx = _probes(x.size, k=6 if x.size <= (1 << 27) else 2, seed=seed)
    want = np.array([oracle.scan_prefix(x, int(i), "iterated_pairwise", L) for i in idx])
    assert_bit_exact(yh[idx], want, "probes (literal)")


@pytest.mark.parametrize("L", [128, 16])
def test_scan_iterated_pairwise_full_size(canon, L):
    print(f"[fullsize] scan_2e27_f64 iterated_pairwise<{L}>", flush=True)
    x = synth.config_input("scan_2e27_f64")
    xd = to_dev(x)
    y = canon.scan(xd, "iterated_pairwise", L)
    _check_ip_every_prefix(x, y, L, 77)
    back = to_host(canon.reduce(xd, L, -0.0)).reshape(1)
    assert_bit_exact(to_host(y[-1:]), back, "scan back == reduce (GPU)")


@pytest.mark.parametrize("policy,param", [("block_dyadic", 256), ("block_dyadic", 16),
                                          ("pairwise", 0), ("iterated_pairwise", 128)])
def test_bench_step_scans_full_size(canon, policy, param):
    """The scans of the benchmark step on its own input (f64, N = 2^28, mixed
    magnitudes, output and workspace passed in as the benchmark does), every
    element against the oracle, and the back element against the GPU reduce
    of the same expression (the block sizes divide 2^28)."""
    print(f"[fullsize] reduce_2e28_f64 scan {policy}<{param}>", flush=True)
    x = synth.config_input("reduce_2e28_f64")
    xd = to_dev(x)
    y = torch.empty_like(xd)
    ws = torch.empty(canon.scan_workspace_bytes(x.size, policy, param, 8),
                     dtype=torch.uint8, device="cuda")
    canon.scan(xd, policy, param, out=y, ws=ws)
    assert canon.workspace_error(ws) == 0
    if policy == "iterated_pairwise":
        _check_ip_every_prefix(x, y, param, 78)
    else:
        assert_bit_exact(to_host(y), oracle.scan(x, policy, param), f"{policy}<{param}>")
    L = param if policy == "iterated_pairwise" else 1
    back = to_host(canon.reduce(xd, L, -0.0)).reshape(1)
    assert_bit_exact(to_host(y[-1:]), back, f"{policy} back == reduce")


# Every register geometry of the one-pass iterated_pairwise kernel: narrow
# rows (f64 L = 16, f32 L = 32), wide rows of 1, 2, 4 and 8 wave-wide vectors
# (pipelined, and one tile per workgroup).  Its two forms (16-byte vector
# loads and stores on an aligned copy, element loads and stores off the
# 16-byte grid) are different kernels with different register use; on
# 2^26 + 12345 elements they must agree on every element, and sampled
# prefixes (literal form) and the back element (GPU reduce) pin the result.
GEOMETRIES = ([(np.float64, L) for L in (16, 128, 256, 512, 1024)] +
              [(np.float32, L) for L in (32, 256, 512, 1024, 2048)])


@pytest.mark.parametrize("dtype,L", GEOMETRIES)
def test_ip_register_geometries_aligned_and_unaligned(canon, dtype, L):
    n = (1 << 26) + 12345
    print(f"[fullsize] iterated_pairwise<{L}> {np.dtype(dtype).name} 2^26+12345, "
          "aligned and unaligned", flush=True)
    x = synth.generate(n + 1, "mixed_magnitude", 900 + L, dtype)
    base = to_dev(x)
    un = to_host(canon.scan(base[1:], "iterated_pairwise", L))
    al = to_host(canon.scan(base[1:].clone(), "iterated_pairwise", L))
    assert_bit_exact(un, al, "unaligned == aligned")
    idx = _probes(n, k=0)
    want = np.array([oracle.scan_prefix(x[1:], int(i), "iterated_pairwise", L) for i in idx])
    assert_bit_exact(al[idx], want, "probes (literal)")
    back = to_host(canon.reduce(base[1:], L, -0.0)).reshape(1)
    assert_bit_exact(al[-1:], back, "scan back == reduce (GPU)")
