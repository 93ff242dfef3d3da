"""Calls on two streams at once: the single-pass scans' persistent grids
compete for the same compute units, and the reduces run their arrival flags
side by side.  Tile numbers come from a ticket counter per call, so a tile
waits only on tiles held by running workgroups of its own call, and each
reduce call tags its flags with an id of its own: every call must finish
with the oracle's bits and a clear error word (canonical-reduce README,
P4016R0 "Summary": the value does not depend on how the work is run)."""
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
    return c


def _ws(nbytes):
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_two_streams(canon, dtype):
    n = (1 << 23) + 17
    x = synth.generate(n, "mixed_magnitude", 81, dtype)
    xd = to_dev(x)
    es = xd.element_size()
    jobs = [("pairwise", 0), ("block_dyadic", 256), ("iterated_pairwise", 128),
            ("block_dyadic", 16)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for i, (policy, param) in enumerate(jobs):
        st = streams[i % 2]
        with torch.cuda.stream(st):
            ws = _ws(canon.scan_workspace_bytes(n, policy, param, es))
            y = torch.empty_like(xd)
            canon.scan(xd, policy, param, out=y, ws=ws, check=False)
            wr = _ws(canon.reduce_workspace_bytes(n, 16 * (i + 1), es))
            r = torch.empty((), dtype=xd.dtype, device="cuda")
            canon.reduce(xd, 16 * (i + 1), 0.5, out=r, ws=wr, check=False)
            outs.append((policy, param, y, ws, 16 * (i + 1), r, wr))
    torch.cuda.synchronize()
    for policy, param, y, ws, L, r, wr in outs:
        assert canon.workspace_error(ws) == 0, f"{policy}<{param}>"
        assert canon.workspace_error(wr) == 0, f"reduce L={L}"
        assert_bit_exact(to_host(y), oracle.scan(x, policy, param), f"{policy}<{param}>")
        assert_bit_exact(to_host(r).reshape(1), [oracle.reduce(x, L, 0.5)], f"reduce L={L}")
