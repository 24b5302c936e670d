"""GPU tests of the permutation's users: tensor-dimension permutes and flips
against PyTorch's CPU reference, and parm against its definition."""
import numpy as np
import pytest

import bmmc_affine_index_amd as bm

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


DTYPES = ["uint8", "float16", "float32", "int64", "complex128"]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("seed", range(4))
def test_permute_dims_matches_torch(dtype, seed):
    torch = _torch()
    rng = np.random.Generator(np.random.PCG64(seed))
    k = int(rng.integers(2, 6))
    shape = [1 << int(v) for v in rng.integers(0, 6, size=k)]
    perm = [int(v) for v in rng.permutation(k)]
    flips = [d for d in range(k) if rng.random() < 0.4]
    dt = getattr(torch, dtype)
    x = torch.from_numpy(rng.integers(0, 100, size=shape).astype(np.float64)).to(dt)
    want = (x.flip(flips) if flips else x).permute(perm).contiguous()
    got = bm.permute_dims(x.to("cuda:0"), perm, flip=flips)
    torch.cuda.synchronize()
    assert got.shape == want.shape
    assert torch.equal(got.cpu(), want)


def test_flip_and_transpose():
    torch = _torch()
    x = torch.arange(1 << 20, dtype=torch.int32).reshape(256, 64, 64)
    d = x.to("cuda:0")
    assert torch.equal(bm.flip(d, [0, 2]).cpu(), x.flip([0, 2]))
    m = torch.arange(1 << 18, dtype=torch.float32).reshape(512, 512)
    assert torch.equal(bm.transpose2d(m.to("cuda:0")).cpu(), m.T.contiguous())
    r = torch.arange(1 << 16, dtype=torch.float32).reshape(64, 1024)
    assert torch.equal(bm.transpose2d(r.to("cuda:0")).cpu(), r.T.contiguous())


def _parm_reference(x, mask, f):
    n = x.shape[0].bit_length() - 1
    cls = np.array([bin(i & mask).count("1") & 1 for i in range(1 << n)])
    out = np.empty_like(x)
    for b in (0, 1):
        idx = np.nonzero(cls == b)[0]
        out[idx] = f(x[idx])
    return out


@pytest.mark.parametrize("n,mask", [(4, 0b0011), (10, 0b1000000001), (16, 0xF0F1), (18, 0x20000)])
def test_parm_matches_definition(n, mask):
    torch = _torch()
    rng = np.random.Generator(np.random.PCG64(n))
    x = rng.integers(0, 1000, size=1 << n).astype(np.int64)
    got = bm.parm(torch.from_numpy(x).to("cuda:0"), mask, lambda t: torch.cumsum(t, 0))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), _parm_reference(x, mask, np.cumsum))
    # a 2-D payload: rows move whole
    y = rng.random((1 << n, 4)).astype(np.float32)
    got = bm.parm(torch.from_numpy(y).to("cuda:0"), mask, lambda t: t.flip(0))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), _parm_reference(y, mask, lambda a: a[::-1]))


@pytest.mark.parametrize("as_handle", [False, True])
def test_side_stream_is_ordered_with_current_stream(as_handle):
    """parm and permute_dims on a side stream (a torch stream, or its raw
    handle): the inputs are produced on the current stream right before the
    call and the results consumed there right after, with no synchronisation
    in between; they must match the same calls on the current stream."""
    torch = _torch()
    side = torch.cuda.Stream()
    stream = int(side.cuda_stream) if as_handle else side
    n, mask = 20, 0x8421
    rng = np.random.Generator(np.random.PCG64(77))
    host = torch.from_numpy(rng.integers(0, 1000, size=1 << n).astype(np.int64))
    for rep in range(3):
        d = host.to("cuda:0")
        d.mul_(3).add_(rep)  # producer on the current stream
        want = bm.parm(d, mask, lambda t: torch.cumsum(t, 0))
        got = bm.parm(d, mask, lambda t: torch.cumsum(t, 0), stream=stream)
        got2 = got * 1  # consumer on the current stream
        x = torch.arange(1 << 18, dtype=torch.float32, device="cuda:0").reshape(8, 64, 512)
        x.add_(rep)
        pw = bm.permute_dims(x, [2, 0, 1], flip=[1])
        pg = bm.permute_dims(x, [2, 0, 1], flip=[1], stream=stream)
        pg2 = pg + 0
        torch.cuda.synchronize()
        assert torch.equal(got2, want), rep
        assert torch.equal(pg2, pw), rep
        assert torch.equal(pw.cpu(), x.cpu().flip([1]).permute(2, 0, 1).contiguous())


def test_tuned_front_end_calls_keep_one_tuned_plan():
    """tune=True tunes a new plan on the call's tensors and keeps it: the
    result equals torch's on the first and on a later call, the later call
    reuses the kept (tuned) plan, and an untuned call keeps its own."""
    torch = _torch()
    bm.clear_plan_cache()
    x = torch.rand(16, 32, 64, 64, device="cuda:0")
    want = x.permute(0, 3, 2, 1).contiguous()
    a = bm.permute_dims(x, (0, 3, 2, 1), tune=True)
    torch.cuda.synchronize()
    assert torch.equal(a, want)
    n_kept = len(bm._PLAN_CACHE)
    b = bm.permute_dims(x, (0, 3, 2, 1), tune=True)
    torch.cuda.synchronize()
    assert torch.equal(b, want) and len(bm._PLAN_CACHE) == n_kept
    c = bm.permute_dims(x, (0, 3, 2, 1))
    torch.cuda.synchronize()
    assert torch.equal(c, want) and len(bm._PLAN_CACHE) == n_kept + 1
    y = torch.arange(1 << 18, dtype=torch.int32, device="cuda:0")
    z = bm.parm(y, 0b1011, lambda t: t.flip(0), tune=True)
    torch.cuda.synchronize()
    ref = _parm_reference(y.cpu().numpy(), 0b1011, lambda t: t[::-1])
    assert np.array_equal(z.cpu().numpy(), ref)
    bm.clear_plan_cache()
