"""na_bwd_noalloc (the backward whose delta rows live in the library's static
device array) against na_bwd with a caller workspace, through the C ABI: two
calls in a row on the same device, the second with a smaller problem, so the
second reads the array after the first left it holding other values."""
import sys

import numpy as np
import pytest
import torch

from fwd_bwd_amd import na
from fwd_bwd_amd.inputs import make_random

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    na.load()


def _rel(a, b):
    a, b = a.double().cpu().numpy(), b.double().cpu().numpy()
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


CASES = [
    # (shape, kernel, dilation, dtype): the larger first, then a smaller one
    ((1, 40, 37, 2, 32), (9, 9), 1, torch.float32),
    ((1, 5, 11, 13, 2, 32), (3, 5, 5), 1, torch.float32),
    ((2, 26, 27, 2, 64), (5, 5), 2, torch.bfloat16),
]


def test_noalloc_matches_workspace_backward_on_consecutive_calls():
    dev = torch.device("cuda:0")
    for i, (shape, kernel, dil, dtype) in enumerate(CASES):
        say("noalloc case", i, shape, kernel, dil, dtype)
        q, k, v, dout = (t.to(dev) for t in make_random(shape, dtype, seed=40 + i))
        out, lse = na.na_fwd(q, k, v, kernel, dil)
        ref = na.na_bwd(q, k, v, out, dout, lse, kernel, dil)
        grads = tuple(torch.full_like(q, float("nan")) for _ in range(3))
        got = na.na_bwd_noalloc(q, k, v, out, dout, lse, kernel, dil, grads=grads)
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            err = _rel(g, r)
            say(f"  {name}: rel err {err:.2e}, bitwise equal {torch.equal(g, r)}")
            assert torch.isfinite(g).all(), name
            assert err <= TOL[dtype], (name, err)


def test_noalloc_rejects_more_rows_than_its_array():
    # 1 x 1024 x 1024 x 9 heads: 9 * 2^20 rows > 2^23; rejected before any launch
    shape = (1, 1024, 1024, 9, 16)
    q = torch.zeros(shape, device="cuda:0")
    lse = torch.zeros(shape[:-1], device="cuda:0")
    with pytest.raises(na.NaError) as e:
        na.na_bwd_noalloc(q, q, q, q, q, lse, (3, 3))
    assert e.value.status == na.NA_ERR_WORKSPACE
