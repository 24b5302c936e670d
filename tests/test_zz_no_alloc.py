"""GPU: bmmc_execute_noalloc, the entry point that allocates nothing, against
bmmc_execute on the same plans and inputs, through the C ABI, bit for bit.

Two-pass plans stage their middle array in the library's fixed device buffer;
calls follow one another on one GPU, the later ones smaller, so a stale buffer
from the previous call would show.  One-pass plans need no buffer.
"""
import sys

import numpy as np
import pytest

import oracle
import bmmc_affine_index_amd as bm
from bmmc_affine_index_amd import workloads as wl

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(n, A, c, elem, seed, **kw):
    """(bmmc_execute result, bmmc_execute_noalloc result, host input, plan)."""
    torch = _torch()
    x = wl.fill_random_bytes(n, elem, seed)
    raw = np.ascontiguousarray(x).view(np.uint8).reshape(-1)
    P = bm.Plan(n, A, c, elem, **kw)
    d_in = torch.from_numpy(raw.copy()).to("cuda:0")
    ref = torch.full_like(d_in, SENTINEL)
    got = torch.full_like(d_in, SENTINEL ^ 0xFF)
    h = int(torch.cuda.current_stream().cuda_stream)
    assert bm.bmmc_execute(P.handle, d_in, ref, h) == bm.OK
    st = bm.bmmc_execute_noalloc(P.handle, d_in, got, h)
    assert st == bm.OK, bm.bmmc_status_string(st)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy(), x, P


def _random(n, seed):
    return wl.random_bmmc(n, seed, lambda r: oracle.rank(r) == n)


@pytest.mark.parametrize("sizes", [(22, 18), (24, 20, 13)])
def test_noalloc_two_pass_matches_execute(sizes):
    """Calls in a row on one GPU, each smaller than the one before; the first
    of the second case fills the whole fixed buffer (2^24 int32 = 64 MiB)."""
    for k, n in enumerate(sizes):
        A, c = _random(n, 900 + n)
        _note("noalloc two-pass n=%d int32 (call %d of %d)" % (n, k + 1, len(sizes)))
        ref, got, x, P = _both(n, A, c, 4, 910 + n, route=bm.ROUTE_TWO_PASS)
        assert P.info.passes == 2 and P.info.scratch_bytes == 4 << n
        assert np.array_equal(ref, got), "n=%d: noalloc differs from bmmc_execute" % n
        if n <= 20:
            want = oracle.apply(A, c, x, threads=16).view(np.uint8).reshape(-1)
            assert np.array_equal(got, want), "n=%d: differs from the oracle" % n


def test_noalloc_one_pass_and_small_elements():
    """One-pass plans (no buffer) and a two-pass plan of 16-byte elements."""
    cases = [(20, wl.bit_reverse_matrix(20), 0, 4, {}),
             (18, *_random(18, 918), 16, {"route": bm.ROUTE_TWO_PASS}),
             (16, *_random(16, 916), 2, {})]
    for n, A, c, elem, kw in cases:
        _note("noalloc n=%d elem=%d %s" % (n, elem, kw))
        ref, got, _, P = _both(n, A, c, elem, 920 + n, **kw)
        assert np.array_equal(ref, got), (n, elem, kw)


def test_noalloc_rejects_plans_beyond_the_buffer():
    """A two-pass plan whose array exceeds the fixed buffer is refused before
    any GPU call; the buffer is then still usable."""
    torch = _torch()
    n = 25  # 2^25 int32 = 128 MiB > 64 MiB
    A, c = _random(n, 925)
    P = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS)
    d = torch.empty(2 << n, dtype=torch.int32, device="cuda:0")
    st = bm.bmmc_execute_noalloc(P.handle, d[: 1 << n], d[1 << n:],
                                 int(torch.cuda.current_stream().cuda_stream))
    assert st == bm.ERR_SCRATCH_LIMIT
    del d
    ref, got, _, _ = _both(14, *_random(14, 914), 4, 914, route=bm.ROUTE_TWO_PASS)
    assert np.array_equal(ref, got)
