"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before it
enqueues anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "canon.h")


@pytest.fixture(scope="module")
def canon():
    import scan_canonical_reduce_amd as c
    if not os.path.exists(c.LIB_PATH):
        from scan_canonical_reduce_amd import build
        build.build()
    return c


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(canon_[a-z0-9_]+)\s*\(", text)))


def test_header_lists_the_binding_exports(canon):
    assert header_functions() == sorted(canon.EXPORTS)


def test_library_exports_every_declared_symbol(canon):
    L = canon.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {canon.LIB_PATH}").read()
    for name in header_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_version_and_status_strings(canon):
    L = canon.lib()
    assert L.canon_abi_version() == 4
    for s in range(5):
        assert L.canon_status_str(s).decode().startswith("CANON_")
    assert L.canon_last_hip_error() == 0


def test_workspace_sizes(canon):
    L = canon.lib()
    assert L.canon_reduce_workspace_bytes(0, 16, 8) == 0
    assert L.canon_reduce_workspace_bytes(1 << 20, 0, 8) == 0
    assert L.canon_reduce_workspace_bytes(1 << 20, 16, 3) == 0
    w = L.canon_reduce_workspace_bytes(1 << 28, 128, 8)
    assert w > 0 and w % 256 == 0 and w <= (1 << 16) * 8 + 256
    # enough room for one partial value per lane and range
    assert L.canon_reduce_workspace_bytes(1000, 7, 8) >= 7 * 8
    s = L.canon_scan_workspace_bytes(1 << 27, 2, 256, 8)
    assert s > 0 and s % 256 == 0
    assert L.canon_scan_workspace_bytes(1 << 20, 2, 3, 8) == 0  # B not a power of two
    assert L.canon_scan_workspace_bytes(0, 0, 0, 8) == 0
    assert L.canon_scan_workspace_bytes(1 << 20, 1, 128, 8) > 0       # iterated_pairwise nodes
    # iterated_pairwise with power-of-two L from E to 512 E runs in one pass at
    # any alignment: its workspace is that pass's (L node words per tile and
    # level, f64 2^28: 32768 tiles), not the three-kernel plan's
    assert 64 << 20 < L.canon_scan_workspace_bytes(1 << 28, 1, 128, 8) < 65 << 20
    assert 8 << 20 < L.canon_scan_workspace_bytes(1 << 28, 1, 16, 8) < (8 << 20) + (1 << 18)
    assert L.canon_scan_rows_workspace_bytes(16, 4096, 2, 16, 8) == 0  # block_dyadic rows: none
    assert L.canon_scan_rows_workspace_bytes(16, 4096, 1, 16, 8) > 0


def _call_reduce(L, x, n, lanes, out, ws, wsb):
    return L.canon_reduce_f64(x, n, lanes, 0.0, out, ws, wsb, None)


def test_reduce_argument_errors(canon):
    L = canon.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call fails validation
    assert _call_reduce(L, fake, 10, 0, fake, None, 0) == 1       # L = 0
    assert _call_reduce(L, None, 10, 4, fake, None, 0) == 1       # x NULL with n > 0
    assert _call_reduce(L, fake, 10, 4, None, None, 0) == 1       # out NULL
    assert _call_reduce(L, fake, 10, (1 << 16) + 1, fake, None, 0) == 2  # L too large
    assert _call_reduce(L, fake, 1 << 20, 16, fake, None, 0) == 3  # no workspace
    need = L.canon_reduce_workspace_bytes(1 << 20, 16, 8)
    assert _call_reduce(L, fake, 1 << 20, 16, fake, ctypes.c_void_p(0x1000 + 8), need) == 3
    assert _call_reduce(L, fake, 1 << 20, 16, fake, fake, need - 1) == 3
    assert L.canon_reduce_rows_f64(fake, 4, 10, 9, 4, 0.0, fake, None, 0, None) == 1  # ld < cols
    assert L.canon_reduce_rows_f64(fake, 4, 10, 10, 0, 0.0, fake, None, 0, None) == 1
    # rows longer than the general row kernel's round stack covers (2^25
    # rounds of 2^21 rows-of-1): rejected before launch
    big = 1 << 47
    assert L.canon_reduce_rows_f64(fake, 2, big, big, 1, 0.0, fake, None, 0, None) == 2


def test_scan_argument_errors(canon):
    L = canon.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.canon_scan_f64(fake, fake, 10, 7, 0, None, 0, None) == 1      # bad policy
    assert L.canon_scan_f64(fake, fake, 10, 0, 2, None, 0, None) == 1      # pairwise param
    assert L.canon_scan_f64(fake, fake, 10, 2, 0, None, 0, None) == 1      # B = 0
    assert L.canon_scan_f64(fake, fake, 10, 2, 12, None, 0, None) == 1     # B not pow2
    assert L.canon_scan_f64(fake, fake, 10, 2, 1 << 17, None, 0, None) == 2  # B too large
    assert L.canon_scan_f64(fake, fake, 10, 1, 0, None, 0, None) == 1      # L = 0
    assert L.canon_scan_f64(fake, fake, 10, 1, (1 << 16) + 1, None, 0, None) == 2
    assert L.canon_scan_f64(fake, fake, 10, 1, 65537, None, 0, None) == 2   # L > CANON_MAX_IP_L
    assert L.canon_scan_f64(fake, fake, 10, 1, 65536, None, 0, None) == 3   # no workspace
    assert L.canon_scan_f64(fake, fake, 1 << 20, 1, 128, None, 0, None) == 3  # no workspace
    assert L.canon_scan_rows_f64(fake, 4096, fake, 4096, 8, 4096, 1, 16, None, 0, None) == 3
    assert L.canon_scan_f64(None, fake, 10, 0, 0, None, 0, None) == 1
    assert L.canon_scan_f64(fake, fake, 1 << 20, 0, 0, None, 0, None) == 3  # no workspace
    assert L.canon_scan_f64(fake, fake, 0, 0, 0, None, 0, None) == 0       # nothing to do
    assert L.canon_scan_rows_f64(fake, 5, fake, 10, 3, 10, 0, 0, None, 0, None) == 1
    assert L.canon_scan_rows_f64(fake, 10, fake, 5, 3, 10, 0, 0, None, 0, None) == 1
    assert L.canon_workspace_error(None, None, None) == 1


def test_scan_with_init_argument_errors(canon):
    L = canon.lib()
    fake = ctypes.c_void_p(0x1000)
    f = L.canon_scan_with_init_f64
    assert f(fake, fake, 10, 0, 0, 3, 1.0, None, 0, None) == 1       # bad kind
    assert f(fake, fake, 10, 0, 0, -1, 1.0, None, 0, None) == 1      # bad kind
    assert f(fake, fake, 10, 7, 0, 0, 1.0, None, 0, None) == 1       # bad policy
    assert f(None, fake, 10, 0, 0, 1, 1.0, None, 0, None) == 1       # no input
    assert f(fake, fake, 1 << 20, 0, 0, 1, 1.0, None, 0, None) == 3  # no workspace
    assert f(fake, fake, 1 << 20, 1, 128, 2, 1.0, None, 0, None) == 3
    assert f(None, None, 0, 0, 0, 0, 1.0, None, 0, None) == 0        # nothing to do
    assert f(None, None, 0, 0, 0, 1, 1.0, None, 0, None) == 0
    assert f(None, None, 0, 0, 0, 2, 1.0, None, 0, None) == 1        # include_initial needs y
    assert L.canon_scan_with_init_f32(fake, fake, 10, 2, 12, 0, 1.0, None, 0, None) == 1
    g = L.canon_scan_rows_with_init_f64
    # include_initial needs ldy >= cols + 1
    assert g(fake, 10, fake, 10, 3, 10, 0, 0, 2, 0.0, None, 0, None) == 1
    assert g(fake, 10, fake, 10, 3, 10, 0, 0, 5, 0.0, None, 0, None) == 1
    assert g(fake, 10, fake, 11, 3, 10, 1, 16, 2, 0.0, None, 0, None) == 3  # no workspace
    assert g(None, 10, None, 11, 0, 10, 0, 0, 2, 0.0, None, 0, None) == 0   # no rows
    assert g(None, 1, None, 1, 3, 0, 0, 0, 2, 0.0, None, 0, None) == 1      # cols 0: y needed
    assert g(None, 1, None, 1, 3, 0, 0, 0, 1, 0.0, None, 0, None) == 0      # nothing to write


def test_operator_argument_errors(canon):
    L = canon.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.canon_reduce_op_f64(fake, 10, 4, 9, 1.0, fake, None, 0, None) == 1   # bad operator
    assert L.canon_reduce_op_f64(fake, 10, 0, 1, 1.0, fake, None, 0, None) == 1   # L = 0
    assert L.canon_scan_op_f64(fake, fake, 10, 0, 0, -1, 0, 1.0, None, 0, None) == 1
    assert L.canon_scan_op_f64(fake, fake, 10, 0, 0, 1, 7, 1.0, None, 0, None) == 1  # bad kind
    assert L.canon_scan_op_f32(fake, fake, 1 << 20, 0, 0, 2, 0, 1.0, None, 0, None) == 3
    assert L.canon_scan_op_f32(fake, fake, 1 << 20, 1, 128, 1, 0, 1.0, None, 0, None) == 3
    assert L.canon_scan_rows_op_f64(fake, 10, fake, 10, 3, 10, 0, 0, 3, 2, 0.0, None, 0,
                                    None) == 1                                   # ldy < cols+1
    assert L.canon_reduce_rows_op_f32(fake, 4, 10, 9, 4, 1, 0.0, fake, None, 0, None) == 1


def test_tile_geometry(canon):
    """Tile sizes the tests place their edge cases on: 4 waves x 64 lanes x
    16 vectors of 16 bytes for the 1-d scans, 8 vectors for double rows;
    iterated_pairwise tiles of the same 4096 E elements in the register
    geometry (power-of-two L from E to 512 E: 64 / RV rows of wide rows,
    4096 E / L rows of narrow ones) or of the rows whose lane trees fit the
    LDS budget."""
    L = canon.lib()
    for pol, par in ((0, 0), (2, 1), (2, 16), (2, 256), (2, 65536), (1, 1)):
        assert L.canon_scan_tile_elems(pol, par, 8) == 8192
        assert L.canon_scan_tile_elems(pol, par, 4) == 16384
    assert L.canon_scan_rows_tile_elems(2, 16, 8) == 4096
    assert L.canon_scan_rows_tile_elems(0, 0, 4) == 16384
    assert L.canon_scan_tile_elems(1, 128, 8) == 64 * 128     # RV = 1
    assert L.canon_scan_tile_elems(1, 512, 8) == 16 * 512     # RV = 4
    assert L.canon_scan_tile_elems(1, 256, 4) == 64 * 256
    assert L.canon_scan_tile_elems(1, 3, 8) == 64 * 3         # LDS path, 64 rows
    assert L.canon_scan_tile_elems(1, 2048, 8) == 1 * 2048    # LDS path, 1 row
    assert L.canon_scan_tile_elems(1, 2, 4) == 64 * 2         # L < E: LDS path
    for lanes in (2, 4, 8, 16, 32, 64):                        # narrow rows
        assert L.canon_scan_tile_elems(1, lanes, 8) == 8192
        assert L.canon_scan_tile_elems(1, 2 * lanes, 4) == 16384
    assert L.canon_scan_rows_tile_elems(1, 16, 8) == 512 * 16
    assert L.canon_scan_tile_elems(7, 0, 8) == 0
    assert L.canon_scan_tile_elems(2, 12, 8) == 0
    assert L.canon_scan_tile_elems(0, 0, 2) == 0


def test_schedule_override(canon):
    L = canon.lib()
    assert L.canon_get_schedule(0) == 0 and L.canon_get_schedule(1) == 0
    with canon.schedule(grid=3, reduce_partials=7):
        assert L.canon_get_schedule(0) == 3
        assert L.canon_get_schedule(1) == 7
    assert L.canon_get_schedule(0) == 0 and L.canon_get_schedule(1) == 0
    default = L.canon_reduce_workspace_bytes(1 << 24, 16, 8)
    with canon.schedule(reduce_partials=4096):
        assert L.canon_reduce_workspace_bytes(1 << 24, 16, 8) > default
    with canon.schedule(spin_limit=5):
        assert L.canon_get_schedule(2) == 5
    assert L.canon_get_schedule(2) == 0
    assert L.canon_set_schedule(3, 1) == 1  # unknown knob: CANON_EINVAL
    assert L.canon_get_schedule(9) == 0


def _gpu_count():
    import torch
    return torch.cuda.device_count()  # counts devices without initialising HIP


@pytest.mark.skipif(_gpu_count() > 0, reason="needs a host without a GPU: the launch must fail")
def test_launch_failure_maps_to_ehip(canon):
    """Valid arguments on a host with no GPU: the enqueue fails, the call
    returns CANON_EHIP and the HIP code is kept for this thread only."""
    import threading
    L = canon.lib()
    fake = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x100000)
    n = 1 << 20
    need = L.canon_reduce_workspace_bytes(n, 16, 8)
    assert L.canon_reduce_f64(fake, n, 16, 0.0, fake, ws, need, None) == 4
    code = L.canon_last_hip_error()
    assert code != 0
    assert "HIP" in L.canon_status_str(4).decode()
    need = L.canon_scan_workspace_bytes(n, 2, 256, 8)
    assert L.canon_scan_f64(fake, fake, n, 2, 256, ws, need, None) == 4
    assert L.canon_scan_rows_f64(fake, 4096, fake, 4096, 16, 4096, 0, 0, None, 0, None) == 4
    other = []
    t = threading.Thread(target=lambda: other.append(L.canon_last_hip_error()))
    t.start()
    t.join()
    assert other == [0]
    # the binding turns it into an exception naming the HIP code
    with pytest.raises(canon.CanonError, match="hip error"):
        canon._check(4, "reduce")


def test_noalloc_scan_limits(canon):
    """The allocation-free scan checks its arguments as canon_scan_f64 does
    and rejects scans whose workspace exceeds its static array, before
    anything is enqueued."""
    L = canon.lib()
    fake = ctypes.c_void_p(0x1000)
    cap = 8 << 20
    f = L.canon_scan_noalloc_f64
    assert f(fake, fake, 10, 7, 0, None) == 1            # bad policy
    assert f(fake, fake, 10, 2, 12, None) == 1           # B not a power of two
    assert f(None, fake, 10, 0, 0, None) == 1            # no input
    assert f(None, None, 0, 0, 0, None) == 0             # nothing to do
    for pol, par in ((0, 0), (2, 256), (1, 128)):
        n = 1 << 20
        while L.canon_scan_workspace_bytes(n, pol, par, 8) <= cap:
            n *= 2
        assert f(fake, fake, n, pol, par, None) == 2     # beyond the static array
    assert L.canon_scan_workspace_bytes(1 << 32, 0, 0, 8) <= cap
    assert L.canon_scan_workspace_bytes(1 << 23, 1, 128, 8) <= cap


def test_binding_refuses_cpu_tensors(canon):
    import torch
    x = torch.zeros(8, dtype=torch.float64)
    with pytest.raises(ValueError):
        canon.reduce(x, 4)
    with pytest.raises(ValueError):
        canon.scan(x, "pairwise")
    with pytest.raises(TypeError):
        canon._sfx(torch.zeros(2, dtype=torch.int32))


USER_OP_LIB = os.path.join(ROOT, "tests", "user_op", "libcanon_skew.so")


@pytest.mark.skipif(not os.path.exists(USER_OP_LIB),
                    reason="the caller-defined-operator library is built by build()")
def test_user_op_library_exports():
    """CANON_USER_OP defines the entry points its header documents."""
    text = open(os.path.join(ROOT, "include", "canon_user_op.hpp")).read()
    documented = set(re.findall(r"\bprefix_([A-Za-z_0-9]+)\(", text))
    assert {"reduce_T", "reduce_rows_T", "scan_T", "scan_rows_T", "last_hip_error"} <= documented
    out = os.popen(f"nm -D --defined-only {USER_OP_LIB}").read()
    names = ["canon_skew_last_hip_error"] + [
        f"canon_skew_{f}_{t}" for f in ("reduce", "reduce_rows", "scan", "scan_rows")
        for t in ("f64", "f32")]
    for name in names:
        assert re.search(rf"\bT {name}\b", out), name
