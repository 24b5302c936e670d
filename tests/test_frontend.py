"""CPU tests of the permutation's users: the parm matrix, the tensor-dimension
matrix and the F2 inverse, checked against their definitions with the oracle
and numpy (no GPU call)."""
import numpy as np
import pytest

import oracle
import bmmc_affine_index_amd as bm
from bmmc_affine_index_amd import workloads as wl


def _dot(i, mask):
    return bin(i & mask).count("1") & 1


def parm_reference(x, mask, f):
    """parm mask f x from its definition: the rows i with i.mask = 0 (in
    increasing order) form the first part, the others the second; f is
    applied to each part and the results go back to the same rows."""
    n = x.shape[0].bit_length() - 1
    cls = np.array([_dot(i, mask) for i in range(1 << n)])
    out = np.empty_like(x)
    for b in (0, 1):
        idx = np.nonzero(cls == b)[0]
        out[idx] = f(x[idx])
    return out


@pytest.mark.parametrize("n,mask", [(1, 1), (2, 3), (4, 0b0011), (4, 0b1010), (6, 0b100001),
                                    (9, 0x1FF), (10, 0b1000000000), (11, 0x2A5)])
def test_parm_matrix_definition(n, mask):
    A = bm.bmmc_parm_matrix(n, mask)
    assert oracle.rank(A) == n
    assert A[n - 1] == mask
    N = 1 << n
    y = np.array([oracle.map_index(A, 0, i) for i in range(N)])
    # the top output bit is the dot product, so the parts are the halves
    assert all((y[i] >> (n - 1)) == _dot(i, mask) for i in range(N))
    # each part keeps increasing index order
    for b in (0, 1):
        part = [i for i in range(N) if _dot(i, mask) == b]
        assert [y[i] - (b << (n - 1)) for i in part] == list(range(N // 2))


@pytest.mark.parametrize("seed", range(6))
def test_parm_by_permutations_equals_definition(seed):
    """parm = (inverse BMMC) . (f on both halves) . (BMMC), with the
    permutations done by the oracle."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(rng.integers(2, 11))
    mask = int(rng.integers(1, 1 << n))
    x = rng.integers(0, 1000, size=1 << n).astype(np.int64)
    f = np.cumsum  # order-dependent, so the order inside each part matters
    A = bm.bmmc_parm_matrix(n, mask)
    Ainv = bm.bmmc_matrix_inverse(A)
    y = oracle.apply(A, 0, x)
    half = 1 << (n - 1)
    z = np.concatenate([f(y[:half]), f(y[half:])])
    assert np.array_equal(oracle.apply(Ainv, 0, z), parm_reference(x, mask, f))


def test_parm_matrix_errors():
    for n, mask in [(4, 0), (4, 16), (0, 1), (33, 1)]:
        with pytest.raises(bm.BmmcError):
            bm.bmmc_parm_matrix(n, mask)


@pytest.mark.parametrize("n,seed", [(3, 1), (12, 2), (20, 3), (32, 4)])
def test_matrix_inverse(n, seed):
    A, c = wl.random_bmmc(n, seed, lambda r: oracle.rank(r) == n)
    Ainv = bm.bmmc_matrix_inverse(A)
    assert np.array_equal(np.asarray(Ainv, dtype=np.uint64), oracle.inverse(A))
    with pytest.raises(bm.BmmcError) as e:
        bm.bmmc_matrix_inverse([1, 2, 3])
    assert e.value.status == bm.ERR_SINGULAR


def _random_case(rng):
    k = int(rng.integers(1, 6))
    dl = [int(v) for v in rng.integers(0, 5, size=k)]
    perm = [int(v) for v in rng.permutation(k)]
    flips = [d for d in range(k) if rng.random() < 0.4]
    return dl, perm, flips


@pytest.mark.parametrize("seed", range(20))
def test_tensor_permute_matrix_matches_numpy(seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    dl, perm, flips = _random_case(rng)
    fm = sum(1 << d for d in flips)
    A, c, n = bm.bmmc_tensor_permute_matrix(dl, perm, fm)
    assert n == sum(dl)
    shape = [1 << b for b in dl]
    x = rng.integers(0, 1 << 30, size=int(np.prod(shape))).astype(np.int32).reshape(shape)
    want = np.ascontiguousarray(np.transpose(np.flip(x, axis=tuple(flips)) if flips else x,
                                             perm)).reshape(-1)
    if n == 0:
        assert want.size == 1
        return
    got = oracle.apply(A, c, x.reshape(-1))
    assert np.array_equal(got, want)


def test_tensor_permute_matrix_errors():
    for dl, perm, fm in [([2, 3], [0, 0], 0), ([2, 3], [0, 2], 0), ([20, 20], [1, 0], 0),
                         ([2, 3], [1, 0], 4), ([-1, 2], [1, 0], 0)]:
        with pytest.raises(bm.BmmcError):
            bm.bmmc_tensor_permute_matrix(dl, perm, fm)


def test_plan_cache_keeps_single_pass_plans_only():
    """The front-end keeps one plan per (map, element size, options) and
    hands the same one back; two-pass plans (which own a scratch array) are
    not kept; the cache is bounded and can be cleared."""
    import bmmc_affine_index_amd as bmi
    bmi.clear_plan_cache()
    A = wl.bit_reverse_matrix(12)
    p1 = bmi._cached_plan(12, A, 0, 4, {})
    assert bmi._cached_plan(12, list(A), 0, 4, {}) is p1
    assert bmi._cached_plan(12, A, 1, 4, {}) is not p1
    assert bmi._cached_plan(12, A, 0, 8, {}) is not p1
    assert bmi._cached_plan(12, A, 0, 4, {"block_map": 1}) is not p1
    # tuned plans are kept apart from untuned ones; a new one is tuned once
    calls = []
    t1 = bmi._cached_plan(12, A, 0, 4, {}, tuned=True, tune_fn=calls.append)
    assert t1 is not p1 and calls == [t1]
    assert bmi._cached_plan(12, A, 0, 4, {}, tuned=True, tune_fn=calls.append) is t1
    assert calls == [t1]
    R, c = wl.random_bmmc(14, 3, lambda r: oracle.rank(r) == 14)
    two = bmi._cached_plan(14, R, c, 4, {"route": bm.ROUTE_TWO_PASS})
    assert two.info.passes == 2 and two.info.scratch_bytes > 0
    assert bmi._cached_plan(14, R, c, 4, {"route": bm.ROUTE_TWO_PASS}) is not two
    for k in range(bmi._PLAN_CACHE_SIZE + 5):
        bmi._cached_plan(12, A, k, 2, {})
    assert len(bmi._PLAN_CACHE) == bmi._PLAN_CACHE_SIZE
    bmi.clear_plan_cache()
    assert len(bmi._PLAN_CACHE) == 0
