"""Inputs of more than 2^32 elements (64-bit element offsets in every kernel
and in the tile bookkeeping), for reduce and the single-pass scans.

The input is x[i] = (i mod 7) - 3: every partial sum is a small integer,
exact in float and double, so every parenthesisation gives the exact sum
and each output has a closed form: with r = i mod 7, the inclusive prefix
through i is r(r+1)/2 - 3(r+1) (each full period of 7 sums to 0).  This
checks addressing and bookkeeping at this size; the trees themselves are
checked bit for bit against the oracle by the other GPU tests.  Data and
expected values are made on the GPU in chunks (about 2.2 N bytes of device
memory per case)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N = (1 << 32) + 12345
CHUNK = 1 << 28


@pytest.fixture(scope="module")
def canon():
    import scan_canonical_reduce_amd as c
    c.lib()
    assert torch.cuda.is_available()
    return c


def make_input(dtype):
    x = torch.empty(N, dtype=dtype, device="cuda")
    for c0 in range(0, N, CHUNK):
        c1 = min(N, c0 + CHUNK)
        i = torch.arange(c0, c1, dtype=torch.int64, device="cuda")
        x[c0:c1] = (i % 7 - 3).to(dtype)
    return x


def prefix(i):
    """Inclusive prefix sum through index i (int64 tensor), exact."""
    r = i % 7
    return r * (r + 1) // 2 - 3 * (r + 1)


def check(y, init, shift, what):
    """y[k] == init + prefix(k - shift) (prefix(-1) = 0), bit for bit."""
    iv = torch.int64 if y.dtype == torch.float64 else torch.int32
    for c0 in range(0, y.numel(), CHUNK):
        c1 = min(y.numel(), c0 + CHUNK)
        k = torch.arange(c0, c1, dtype=torch.int64, device="cuda") - shift
        want = torch.where(k >= 0, prefix(k.clamp(min=0)), torch.zeros_like(k))
        want = (want.to(y.dtype) + init) if init != 0 else want.to(y.dtype)
        ok = torch.equal(y[c0:c1].view(iv), want.view(iv))
        assert ok, f"{what}: mismatch in [{c0}, {c1})"


@pytest.mark.parametrize("dtype", [torch.float32, torch.float64])
def test_reduce_and_scans_past_2_32_elements(canon, dtype):
    x = make_input(dtype)
    total = float(prefix(torch.tensor(N - 1)).item())
    for L in (16, 128):
        got = canon.reduce(x, L, 0.5).item()
        assert got == total + 0.5, f"reduce L={L}: {got} != {total + 0.5}"
    ip = 128 if dtype == torch.float64 else 256
    y = torch.empty_like(x)
    for policy, param in (("pairwise", 0), ("block_dyadic", 16), ("block_dyadic", 256),
                          ("iterated_pairwise", ip)):
        ws = torch.empty(canon.scan_workspace_bytes(N, policy, param, x.element_size()),
                         dtype=torch.uint8, device="cuda")
        canon.scan(x, policy, param, out=y, ws=ws)
        assert canon.workspace_error(ws) == 0
        check(y, 0, 0, f"{policy}<{param}>")
    del ws
    canon.scan_with_init(x, "block_dyadic", 256, "exclusive", 0.5, out=y)
    check(y, 0.5, 1, "exclusive init 0.5")


def test_rows_past_2_32_elements(canon):
    """Row reduce and row scan over more than 2^32 elements in all (rows of
    7 * 586 doubles, so every row holds the same exact pattern)."""
    cols = 7 * 586
    rows = (1 << 32) // cols + 2
    X = torch.empty(rows, cols, dtype=torch.float64, device="cuda")
    row = (torch.arange(cols, dtype=torch.int64, device="cuda") % 7 - 3).to(torch.float64)
    X[:] = row
    assert X.numel() > (1 << 32)
    total = float(prefix(torch.tensor(cols - 1)).item())
    r = canon.reduce_rows(X, 16, 0.5)
    assert bool((r == total + 0.5).all()), "row reduce"
    Y = canon.scan_rows(X, "block_dyadic", 16)
    want = prefix(torch.arange(cols, dtype=torch.int64, device="cuda")).to(torch.float64)
    for r0 in range(0, rows, 1 << 16):
        assert torch.equal(Y[r0:r0 + (1 << 16)].view(torch.int64),
                           want.expand(min(1 << 16, rows - r0), cols).view(torch.int64)), r0
