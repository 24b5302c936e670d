"""GPU parity on the seeded random option cases (tests/random_cases.py), each
checked bit-exact against the oracle.  Before a case is launched, the host
replay of its kernel tables must have passed (every access in range, every
unit moved once), so no launch reaches memory the tables do not name."""
import numpy as np
import pytest

import oracle
from emulate import run_plan_on_host
from random_cases import cases, plan_or_none
from test_gpu_parity import SENTINEL, _note, _torch

pytestmark = pytest.mark.gpu

BATCHES = 6


@pytest.mark.parametrize("batch", range(BATCHES))
def test_random_cases_on_gpu(batch):
    torch = _torch()
    mine = cases()[batch::BATCHES]
    ran = 0
    for case in mine:
        P = plan_or_none(case)
        if P is None:
            continue
        A, c = case.matrix()
        x = case.data()
        want = oracle.apply(A, c, x)
        assert np.array_equal(run_plan_on_host(P, x), want), case.ident()
        _note(case.ident())
        raw = np.ascontiguousarray(x).view(np.uint8).reshape(-1)
        d_in = torch.from_numpy(raw.copy()).to("cuda:0")
        d_out = torch.full_like(d_in, SENTINEL)
        P(d_in, d_out)
        torch.cuda.synchronize()
        got = d_out.cpu().numpy().view(x.dtype).reshape(x.shape)
        assert np.array_equal(got, want), (case.ident(), P.describe())
        ran += 1
    assert ran >= 0.9 * len(mine)
