"""Seeded synthetic inputs for BMMC permutations.

This module is shared by the GPU tests, the benchmark and the oracle tests,
so it holds no part of the permutation's arithmetic: it only draws matrices,
complement vectors and array contents from seeded generators, and builds the
matrices of the named special cases from their definitions.

Matrix convention (row masks): ``A[r]`` is the mask of input index bits that
feed output bit r, so bit j of ``A[r]`` is the entry A_rj.  Index bit 0 is the
least significant bit (the appendix kernels of "Efficient GPU Implementation
of Affine Index Permutations on Arrays" send input bit 0 to output bit 14 for
the 15-bit reversal).

Workloads follow the pages' descriptions: "random BPC / bit-reverse / random
BMMC" on 32-bit elements at 2^20 and up (that paper, evaluation), and the
4096 x 4096 fp32 transpose with in[i] = (float)i ("A kernel that is correct",
the check).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Iterator, Optional, Tuple

import numpy as np


# --------------------------------------------------------------------------
# Matrices of the special cases
# --------------------------------------------------------------------------

def identity_matrix(n: int) -> np.ndarray:
    return np.array([1 << r for r in range(n)], dtype=np.uint64)


def bit_reverse_matrix(n: int) -> np.ndarray:
    """Anti-identity: output bit r is input bit n-1-r (bit-rev(4, 7) = 14)."""
    return np.array([1 << (n - 1 - r) for r in range(n)], dtype=np.uint64)


def transpose_matrix(row_bits: int, col_bits: int) -> np.ndarray:
    """Transpose of a 2^row_bits x 2^col_bits row-major matrix.

    Element (row, col) sits at index row * 2^col_bits + col and moves to
    col * 2^row_bits + row, so the output's low row_bits bits are the input's
    high bits and the output's high bits are the input's low bits: a rotation
    of the index bits.  For the 4 x 4 case this sends bits [x0,x1,x2,x3] to
    [x2,x3,x0,x1] (index 6 -> 9).
    """
    n = row_bits + col_bits
    rows = []
    for r in range(n):
        src = col_bits + r if r < row_bits else r - row_bits
        rows.append(1 << src)
    return np.array(rows, dtype=np.uint64)


def bit_permutation_matrix(perm) -> np.ndarray:
    """BP matrix that sends input bit j to output bit perm[j]."""
    n = len(perm)
    rows = [0] * n
    for j, p in enumerate(perm):
        rows[int(p)] = 1 << j
    return np.array(rows, dtype=np.uint64)


def random_bpc(n: int, seed: int) -> Tuple[np.ndarray, int]:
    """Random bit permutation plus random complement.

    p = permutation(n) from PCG64(seed); output bit p[j] = input bit j;
    c uniform in [0, 2^n) from the same stream.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.permutation(n)
    A = bit_permutation_matrix(p)
    c = int(rng.integers(0, 1 << n, dtype=np.uint64))
    return A, c


def random_rows(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(0, 1 << n, size=n, dtype=np.uint64)


def random_bmmc(n: int, seed: int,
                accept: Callable[[np.ndarray], bool]) -> Tuple[np.ndarray, int]:
    """Rejection-sampled random matrix plus a random complement.

    Draws n rows uniform in [0, 2^n) from PCG64(seed) until ``accept(rows)``
    holds, then draws c uniform in [0, 2^n) from the same stream.  The caller
    supplies the acceptance test (invertibility over F2, and any further
    condition), so this module holds no F2 arithmetic: the test suite passes
    the oracle's rank test, the benchmark passes the library's own.  Both must
    accept the same first candidate, which the tests check.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    for _ in range(100000):
        rows = random_rows(rng, n)
        if accept(rows):
            c = int(rng.integers(0, 1 << n, dtype=np.uint64))
            return rows, c
    raise RuntimeError("no candidate accepted")


def candidate_rows(n: int, seed: int) -> Iterator[np.ndarray]:
    """The raw candidate sequence that random_bmmc draws from."""
    rng = np.random.Generator(np.random.PCG64(seed))
    while True:
        yield random_rows(rng, n)


# --------------------------------------------------------------------------
# Array contents
# --------------------------------------------------------------------------

def fill_index_int32(n: int) -> np.ndarray:
    """in[i] = i as int32 (every element distinct up to 2^31)."""
    return np.arange(1 << n, dtype=np.int64).astype(np.int32)


def fill_index_float32(n: int) -> np.ndarray:
    """in[i] = (float)i, exact while i <= 2^24."""
    return np.arange(1 << n, dtype=np.float32)


def fill_uniform_uint32(n: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 1 << 32, size=1 << n, dtype=np.uint32)


def fill_uniform_f32_records(n: int, seed: int, width: int = 4) -> np.ndarray:
    """2^n records of `width` fp32 values, uniform in [0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.random((1 << n) * width, dtype=np.float32).reshape(1 << n, width)


def fill_random_bytes(n: int, elem_bytes: int, seed: int) -> np.ndarray:
    """2^n elements of `elem_bytes` random bytes each, shape (2^n, elem_bytes)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 256, size=((1 << n), elem_bytes), dtype=np.uint8)


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    n: int
    elem_bytes: int
    description: str


WORKLOADS = {
    "c1a": Workload("c1a", 20, 4, "n=20 int32 in[i]=i, random invertible A and c (seed 20)"),
    "c1b": Workload("c1b", 20, 4, "n=20 int32 in[i]=i, bit reversal"),
    "c2": Workload("c2", 24, 4, "4096x4096 fp32 transpose (rotation by 12 on n=24), "
                                "in[i]=(float)i"),
    "c3": Workload("c3", 28, 4, "n=28 int32 bit reversal, uniform uint32 data (seed 28)"),
    "c4": Workload("c4", 30, 4, "n=30 int32 in[i]=i, random invertible A (not tiled) "
                                "and c (seed 30)"),
    "c5": Workload("c5", 27, 16, "n=27 16-byte records (4 x fp32 U[0,1), seed 27), "
                                 "random BPC (seeds 2700..2731)"),
}


def workload_matrix(name: str, accept: Optional[Callable[[np.ndarray], bool]] = None,
                    perm_index: int = 0) -> Tuple[np.ndarray, int]:
    """(A, c) of a workload.  Random-BMMC workloads need the acceptance test."""
    w = WORKLOADS[name]
    if name == "c1b" or name == "c3":
        return bit_reverse_matrix(w.n), 0
    if name == "c2":
        return transpose_matrix(12, 12), 0
    if name == "c5":
        return random_bpc(w.n, 2700 + perm_index)
    if name in ("c1a", "c4"):
        if accept is None:
            raise ValueError("random BMMC workloads need an acceptance test")
        return random_bmmc(w.n, w.n, accept)
    raise KeyError(name)


def workload_data(name: str) -> np.ndarray:
    """Input array of a workload, shape (2^n,) or (2^n, 4) for 16-byte records."""
    w = WORKLOADS[name]
    if name in ("c1a", "c1b", "c4"):
        return fill_index_int32(w.n)
    if name == "c2":
        return fill_index_float32(w.n)
    if name == "c3":
        return fill_uniform_uint32(w.n, 28).view(np.int32)
    if name == "c5":
        return fill_uniform_f32_records(w.n, 27)
    raise KeyError(name)
