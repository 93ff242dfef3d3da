"""The allocation-free scan (canon_scan_noalloc_f64, workspace in the
library's static device array) against canon_scan_f64 with a caller's
workspace, through the C ABI, bit for bit: two calls in a row per policy,
the second on a smaller input (the array keeps the first call's contents),
and both against the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import assert_bit_exact, to_dev, to_host  # noqa: E402

POL = {"pairwise": 0, "iterated_pairwise": 1, "block_dyadic": 2}


@pytest.fixture(scope="module")
def lib():
    import scan_canonical_reduce_amd as c
    return c.lib()


def scan_with_ws(lib, xd, n, policy, param):
    y = torch.empty(n, dtype=torch.float64, device="cuda")
    nb = lib.canon_scan_workspace_bytes(n, POL[policy], param, 8)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    st = lib.canon_scan_f64(xd.data_ptr(), y.data_ptr(), n, POL[policy], param, ws.data_ptr(), nb,
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    return to_host(y)


def scan_noalloc(lib, xd, n, policy, param):
    y = torch.empty(n, dtype=torch.float64, device="cuda")
    st = lib.canon_scan_noalloc_f64(xd.data_ptr(), y.data_ptr(), n, POL[policy], param,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    return to_host(y)


@pytest.mark.parametrize("policy,param", [("pairwise", 0), ("block_dyadic", 256),
                                          ("block_dyadic", 16), ("iterated_pairwise", 128),
                                          ("iterated_pairwise", 3)])
def test_noalloc_scan_matches(lib, policy, param):
    big = (1 << 22) + 777 if policy != "iterated_pairwise" else (1 << 21) + 777
    x = synth.generate(big, "mixed_magnitude", 601, np.float64)
    xd = to_dev(x)
    for n in (big, big // 3 + 5):
        print(f"[noalloc] {policy}<{param}> n={n}", flush=True)
        want = scan_with_ws(lib, xd, n, policy, param)
        got = scan_noalloc(lib, xd, n, policy, param)
        assert_bit_exact(got, want, f"noalloc vs canon_scan_f64 n={n}")
        assert_bit_exact(got, oracle.scan(x[:n], policy, param), f"noalloc vs oracle n={n}")
