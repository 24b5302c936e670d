"""Pins for the CPU oracle: facts the pages and the mathematics fix.

Each test checks the oracle against something other than its own formula:
printed worked examples (tests/golden/worked_examples.txt), library routines
that realise special cases independently (numpy axis permutations and flips,
numpy's transpose), closed-form group orders, and algebraic laws (composition,
inverse, affinity).  A transposed matrix, a gather instead of a scatter, a
dropped complement or a flipped bit order each fails at least one of them.
"""
import os

import numpy as np
import pytest

import oracle
from bmmc_affine_index_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.txt")


def _golden():
    facts = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            kind, *kv = line.split()
            facts.append((kind, {k: int(v) if v.lstrip("-").isdigit() else v
                                 for k, v in (p.split("=") for p in kv)}))
    return facts


def _matrix_for(case, d):
    if case == "bitrev":
        return wl.bit_reverse_matrix(d["n"])
    if case == "transpose":
        return wl.transpose_matrix(d["row_bits"], d["col_bits"])
    raise KeyError(case)


def _bits(n):
    """2^n x n array of index bits, bit 0 in column 0."""
    i = np.arange(1 << n, dtype=np.int64)
    return ((i[:, None] >> np.arange(n)) & 1).astype(np.int64)


def _rows_to_dense(A, n):
    return ((np.asarray(A, dtype=np.uint64)[:, None] >> np.arange(n, dtype=np.uint64)) & 1
            ).astype(np.int64)


def _dense_to_rows(M):
    n = M.shape[1]
    return np.array([int(sum(int(M[r, j]) << j for j in range(n))) for r in range(M.shape[0])],
                    dtype=np.uint64)


def _gf2_mat_mul(A, B, n):
    """Product over F2 via numpy's integer matmul (a library primitive)."""
    return _dense_to_rows((_rows_to_dense(A, n) @ _rows_to_dense(B, n)) % 2)


def _gf2_mat_vec(A, v, n):
    vb = (np.uint64(v) >> np.arange(n, dtype=np.uint64)) & np.uint64(1)
    y = (_rows_to_dense(A, n) @ vb.astype(np.int64)) % 2
    return int(sum(int(y[r]) << r for r in range(n)))


# --------------------------------------------------------------------------
# Printed worked examples
# --------------------------------------------------------------------------

def test_golden_maps():
    seen = 0
    for kind, d in _golden():
        if kind == "map":
            A = _matrix_for(d["case"], d)
            assert oracle.map_index(A, 0, d["in"]) == d["out"], d
            # and the array form scatters that element there
            n = len(A)
            x = np.arange(1 << n, dtype=np.int32)
            out = oracle.apply(A, 0, x)
            assert out[d["out"]] == d["in"]
            seen += 1
    assert seen == 2


def test_map_indices_is_map_index_per_index():
    """The batched map used for sampled checks at large n gives the printed
    examples and agrees with the one-index map everywhere it is sampled,
    including indices with bit 31 set."""
    for kind, d in _golden():
        if kind == "map":
            A = _matrix_for(d["case"], d)
            assert int(oracle.map_indices(A, 0, [d["in"]])[0]) == d["out"]
    A = wl.bit_reverse_matrix(15)
    ys = oracle.map_indices(A, 0, [1 << k for k in range(15)])
    assert [int(y) for y in ys] == [1 << (14 - k) for k in range(15)]
    rng = np.random.Generator(np.random.PCG64(77))
    for n in (5, 20, 32):
        A, c = wl.random_bmmc(n, n, lambda r: oracle.rank(r) == len(r))
        idx = rng.integers(0, 1 << n, size=500, dtype=np.uint64)
        idx[:2] = [0, (1 << n) - 1]
        ys = oracle.map_indices(A, c, idx)
        assert [int(y) for y in ys] == [oracle.map_index(A, c, int(i)) for i in idx]
    assert oracle.map_indices(A, c, np.zeros(0, dtype=np.uint64)).size == 0


def test_golden_reverse16():
    facts = [d for k, d in _golden() if k == "reverse"]
    assert facts
    for d in facts:
        n = d["n"]
        x = np.arange(1 << n, dtype=np.int32) * 7 + 3
        out = oracle.apply(wl.identity_matrix(n), d["c"], x)
        assert np.array_equal(out, x[::-1])


def test_golden_appendix_bitmoves():
    facts = [d for k, d in _golden() if k == "bitmove"]
    assert len(facts) == 3
    for d in facts:
        A = _matrix_for(d["case"], d)
        assert oracle.map_index(A, 0, 1 << d["in_bit"]) == 1 << d["out_bit"]
    # every input bit of the 15-bit reversal goes to 14 - k
    A = wl.bit_reverse_matrix(15)
    for k in range(15):
        assert oracle.map_index(A, 0, 1 << k) == 1 << (14 - k)


def test_golden_transpose_16x8():
    d = [d for k, d in _golden() if k == "transpose_shape"][0]
    rb, cb = d["rows"].bit_length() - 1, d["cols"].bit_length() - 1
    assert (1 << rb) == d["rows"] and (1 << cb) == d["cols"]
    x = np.arange(d["rows"] * d["cols"], dtype=np.int32)
    out = oracle.apply(wl.transpose_matrix(rb, cb), 0, x)
    assert np.array_equal(out, x.reshape(d["rows"], d["cols"]).T.reshape(-1))
    assert oracle.is_bijective(wl.transpose_matrix(rb, cb), 0)


def _two_loop_transpose(inp, n):
    """The two-loop CPU reference of "A kernel that is correct" (the check):
    ref[x*n + y] = in[y*n + x]."""
    ref = np.empty_like(inp)
    for y in range(n):
        ref[np.arange(n) * n + y] = inp[y * n:(y + 1) * n]
    return ref


@pytest.mark.parametrize("log_n", [3, 6, 9])
def test_transpose_equals_two_loop_reference(log_n):
    n = 1 << log_n
    inp = np.arange(n * n, dtype=np.float32)
    out = oracle.apply(wl.transpose_matrix(log_n, log_n), 0, inp)
    assert np.array_equal(out.view(np.uint32), _two_loop_transpose(inp, n).view(np.uint32))


def test_transpose_4096_workload():
    d = [d for k, d in _golden() if k == "transpose_bytes"][0]
    n = d["n"]
    inp = wl.workload_data("c2")
    assert inp.dtype == np.float32 and inp.size == n * n
    assert 2 * inp.nbytes == d["bytes"]
    # the fill is exact: every value is its own index
    assert np.array_equal(inp.astype(np.int64), np.arange(n * n))
    A, c = wl.workload_matrix("c2")
    out = oracle.apply(A, c, inp, threads=os.cpu_count() or 1)
    assert np.array_equal(out.view(np.uint32), inp.reshape(n, n).T.reshape(-1).view(np.uint32))


# --------------------------------------------------------------------------
# Special cases that reduce to library routines
# --------------------------------------------------------------------------

def _bpc_by_axes(x, perm, c):
    """A BPC realised with numpy only: view the 2^n array as shape [2]*n (axis a
    holds index bit n-1-a), move axes so that output bit perm[j] takes input
    bit j, then flip the axes whose complement bit is set."""
    n = len(perm)
    pinv = np.argsort(perm)
    t = x.reshape([2] * n + list(x.shape[1:]))
    axes = [n - 1 - int(pinv[n - 1 - a]) for a in range(n)] + list(range(n, t.ndim))
    t = np.transpose(t, axes)
    flips = tuple(n - 1 - b for b in range(n) if (c >> b) & 1)
    if flips:
        t = np.flip(t, axis=flips)
    return np.ascontiguousarray(t).reshape(x.shape)


@pytest.mark.parametrize("n,seed", [(1, 0), (2, 1), (5, 2), (8, 3), (11, 4), (14, 5)])
def test_random_bpc_matches_axis_permutation(n, seed):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    perm = rng.permutation(n)
    c = int(rng.integers(0, 1 << n))
    A = wl.bit_permutation_matrix(perm)
    x = rng.integers(0, 1 << 31, size=1 << n, dtype=np.int64).astype(np.int32)
    assert np.array_equal(oracle.apply(A, c, x), _bpc_by_axes(x, perm, c))


def test_bit_reverse_matches_axis_reversal():
    n = 16
    x = wl.fill_uniform_uint32(n, 28).view(np.int32)
    expect = np.ascontiguousarray(np.transpose(x.reshape([2] * n))).reshape(-1)
    assert np.array_equal(oracle.apply(wl.bit_reverse_matrix(n), 0, x), expect)


def test_complement_only_is_flip():
    n = 10
    x = np.arange(1 << n, dtype=np.int32)
    for c in [1, 2, 0x155, (1 << n) - 1]:
        out = oracle.apply(wl.identity_matrix(n), c, x)
        assert np.array_equal(out, x[np.arange(1 << n) ^ c])


@pytest.mark.parametrize("elem_bytes", [1, 2, 3, 4, 8, 12, 16, 32])
def test_elements_move_whole(elem_bytes):
    """Multi-byte elements move as opaque units: the result equals the int32
    index permutation applied to rows of bytes."""
    n = 9
    A, c = wl.random_bpc(n, 77)
    x = wl.fill_random_bytes(n, elem_bytes, seed=elem_bytes)
    out = oracle.apply(A, c, x)
    perm_idx = oracle.apply(A, c, np.arange(1 << n, dtype=np.int32))
    assert np.array_equal(out, x[perm_idx])


# --------------------------------------------------------------------------
# Closed forms and algebraic laws
# --------------------------------------------------------------------------

def test_rank_counts_match_group_orders():
    """|GL(n, 2)| = prod_{k<n} (2^n - 2^k): 168 for n = 3, 20160 for n = 4."""
    for n, order in [(2, 6), (3, 168), (4, 20160)]:
        count = 0
        for code in range(1 << (n * n)):
            rows = [(code >> (r * n)) & ((1 << n) - 1) for r in range(n)]
            if oracle.rank(rows) == n:
                count += 1
        assert count == order


def test_rank_matches_bijectivity_bruteforce():
    """Invertible over F2 <=> the index map is a bijection (all 3x3 matrices,
    with a few complements)."""
    n = 3
    for code in range(1 << 9):
        rows = np.array([(code >> (3 * r)) & 7 for r in range(3)], dtype=np.uint64)
        for c in (0, 5):
            assert oracle.is_bijective(rows, c) == (oracle.rank(rows) == n)


def test_all_gl3_by_dense_bruteforce():
    """Every invertible 3x3 matrix and every complement: the scatter equals the
    permutation given by numpy's dense bit products."""
    n = 3
    B = _bits(n)
    x = np.arange(8, dtype=np.int32) * 11 + 5
    for code in range(1 << 9):
        rows = np.array([(code >> (3 * r)) & 7 for r in range(3)], dtype=np.uint64)
        if oracle.rank(rows) != 3:
            continue
        Y = (B @ _rows_to_dense(rows, n).T) % 2
        for c in range(8):
            dest = (Y @ (1 << np.arange(n))) ^ c
            expect = np.empty_like(x)
            expect[dest] = x
            assert np.array_equal(oracle.apply(rows, c, x), expect)


def _random_invertible(n, seed):
    return wl.random_bmmc(n, seed, lambda r: oracle.rank(r) == n)


@pytest.mark.parametrize("n,seed", [(4, 1), (7, 2), (10, 3), (13, 4)])
def test_composition_is_product(n, seed):
    """Applying (A2, c2) then (A1, c1) equals (A1 A2, A1 c2 XOR c1)."""
    A1, c1 = _random_invertible(n, seed)
    A2, c2 = _random_invertible(n, seed + 100)
    x = np.arange(1 << n, dtype=np.int32)
    two = oracle.apply(A1, c1, oracle.apply(A2, c2, x))
    A = _gf2_mat_mul(A1, A2, n)
    c = _gf2_mat_vec(A1, c2, n) ^ c1
    assert np.array_equal(two, oracle.apply(A, c, x))
    # order matters for these matrices, so a swapped product would fail
    A_sw = _gf2_mat_mul(A2, A1, n)
    if not np.array_equal(A_sw, A):
        assert not np.array_equal(two, oracle.apply(A_sw, _gf2_mat_vec(A2, c1, n) ^ c2, x))


@pytest.mark.parametrize("n,seed", [(5, 11), (9, 12), (12, 13)])
def test_inverse_undoes(n, seed):
    A, c = _random_invertible(n, seed)
    Ainv = oracle.inverse(A)
    assert np.array_equal(_gf2_mat_mul(A, Ainv, n), wl.identity_matrix(n))
    x = wl.fill_uniform_uint32(n, seed)
    back = oracle.apply(Ainv, _gf2_mat_vec(Ainv, c, n), oracle.apply(A, c, x))
    assert np.array_equal(back, x)


@pytest.mark.parametrize("n,seed", [(6, 21), (16, 22), (30, 23)])
def test_affine_laws(n, seed):
    """map(0) = c, map(e_j) = column j of A XOR c, and
    map(i XOR k) = map(i) XOR map(k) XOR c."""
    A, c = _random_invertible(n, seed)
    assert oracle.map_index(A, c, 0) == c
    for j in range(n):
        col = sum(((int(A[r]) >> j) & 1) << r for r in range(n))
        assert oracle.map_index(A, c, 1 << j) == col ^ c
    rng = np.random.Generator(np.random.PCG64(seed))
    for _ in range(200):
        i, k = (int(v) for v in rng.integers(0, 1 << n, size=2))
        assert oracle.map_index(A, c, i ^ k) == (
            oracle.map_index(A, c, i) ^ oracle.map_index(A, c, k) ^ c)


@pytest.mark.parametrize("n,seed", [(8, 31), (14, 32), (18, 33)])
def test_bijective_for_invertible(n, seed):
    A, c = _random_invertible(n, seed)
    assert oracle.is_bijective(A, c)
    x = np.arange(1 << n, dtype=np.int32)
    out = oracle.apply(A, c, x, threads=4)
    assert np.array_equal(np.sort(out), x)


def test_singular_rejected():
    A = np.array([1, 2, 3], dtype=np.uint64)  # row 2 = row 0 XOR row 1
    assert oracle.rank(A) == 2
    assert not oracle.is_bijective(A, 0)
    with pytest.raises(ValueError):
        oracle.apply(A, 0, np.zeros(8, dtype=np.int32))
    with pytest.raises(ValueError):
        oracle.inverse(A)


def test_threads_do_not_change_result():
    n = 15
    A, c = _random_invertible(n, 41)
    x = wl.fill_uniform_uint32(n, 41)
    assert np.array_equal(oracle.apply(A, c, x, threads=1), oracle.apply(A, c, x, threads=7))


def test_apply_range_covers_pieces():
    n = 12
    A, c = _random_invertible(n, 42)
    x = wl.fill_uniform_uint32(n, 42)
    out = np.zeros_like(x)
    oracle.apply_range(A, c, x, out, 0, 1000, threads=3)
    oracle.apply_range(A, c, x, out, 1000, 1 << n, threads=2)
    assert np.array_equal(out, oracle.apply(A, c, x))


def test_sampled_check_detects_planted_error():
    n = 12
    A, c = _random_invertible(n, 43)
    x = wl.fill_uniform_uint32(n, 43)
    out = oracle.apply(A, c, x)
    idx = np.arange(1 << n, dtype=np.uint64)
    assert oracle.check_sampled(A, c, x, out, idx) == (0, None)
    bad = out.copy()
    j = oracle.map_index(A, c, 1234)
    bad[j] ^= 1
    assert oracle.check_sampled(A, c, x, bad, idx) == (1, 1234)


def test_random_bmmc_candidates_are_deterministic():
    rows_a, c_a = _random_invertible(20, 20)
    rows_b, c_b = _random_invertible(20, 20)
    assert np.array_equal(rows_a, rows_b) and c_a == c_b
    assert oracle.rank(rows_a) == 20
    # it is the first invertible candidate of the seeded stream
    for cand in wl.candidate_rows(20, 20):
        if oracle.rank(cand) == 20:
            assert np.array_equal(cand, rows_a)
            break
