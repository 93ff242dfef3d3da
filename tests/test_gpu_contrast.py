"""The contrast the canonical-reduce README draws with CUB (P4229R0 "Key
results"), for ROCm: torch.sum and torch.cumsum next to the canonical
library on the same inputs.  Only the canonical side is asserted (its scan
back element equals its reduce, and its bits never change between calls);
torch's figures are printed, since nothing fixes them."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import to_dev, to_host  # noqa: E402


@pytest.fixture(scope="module")
def canon():
    import scan_canonical_reduce_amd as c
    c.lib()
    return c


def test_contrast_with_torch(canon):
    xn = synth.config_input("scan_1m")
    x = to_dev(xn)
    cs = to_host(canon.scan(x, "pairwise"))
    cr = to_host(canon.reduce(x, 1, -0.0)).reshape(1)
    assert cs[-1:].view(np.uint64)[0] == cr.view(np.uint64)[0]
    for _ in range(5):
        assert np.array_equal(to_host(canon.scan(x, "pairwise")).view(np.uint64),
                              cs.view(np.uint64))
    ts = to_host(torch.cumsum(x, 0))
    tr = to_host(torch.sum(x)).reshape(1)
    lf = oracle.left_fold_scan(xn)
    differ = int(np.count_nonzero(ts.view(np.uint64) != cs.view(np.uint64)))
    differ_lf = int(np.count_nonzero(lf.view(np.uint64) != cs.view(np.uint64)))
    print(f"[contrast] torch.cumsum differs from the canonical pairwise scan in {differ} of "
          f"{xn.size} elements; the left fold in {differ_lf}; torch cumsum[-1] == sum: "
          f"{bool(ts[-1] == tr[0])}", flush=True)
    # the canonical scan is not the left fold (mixed rounding order)
    assert differ_lf > 0
