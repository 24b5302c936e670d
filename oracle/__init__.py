"""The plain CPU oracle for BMMC index permutations -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.

The arithmetic lives in ``bmmc_oracle.c`` (plain C, built with gcc into
``liboracle.so`` next to this file).  This module only marshals numpy arrays
into those C functions.  The definition it follows is the BMMC transformation
of "Efficient GPU Implementation of Affine Index Permutations on Arrays"
(introduction): y = A.x XOR c over F2, with x the bit vector of the index
(bit 0 = least significant bit), and the scatter out[A.i XOR c] = in[i] used
by that page's appendix kernels.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bmmc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, BAD_ARG, SINGULAR, NOT_BIJECTIVE = 0, 1, 2, 3

_lib = None


def build() -> str:
    """Compile bmmc_oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp]
    )
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.oracle_gf2_rank.argtypes = [ctypes.c_int, u64p]
    lib.oracle_gf2_rank.restype = ctypes.c_int
    lib.oracle_gf2_inverse.argtypes = [ctypes.c_int, u64p, u64p]
    lib.oracle_gf2_inverse.restype = ctypes.c_int
    lib.oracle_map_index.argtypes = [ctypes.c_int, u64p, ctypes.c_uint64, ctypes.c_uint64]
    lib.oracle_map_index.restype = ctypes.c_uint64
    lib.oracle_map_indices.argtypes = [ctypes.c_int, u64p, ctypes.c_uint64, u64p, u64p,
                                       ctypes.c_size_t]
    lib.oracle_map_indices.restype = None
    lib.oracle_bmmc_apply.argtypes = [ctypes.c_int, u64p, ctypes.c_uint64, ctypes.c_size_t,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_bmmc_apply.restype = ctypes.c_int
    lib.oracle_bmmc_apply_range.argtypes = [ctypes.c_int, u64p, ctypes.c_uint64,
                                            ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_uint64,
                                            ctypes.c_uint64, ctypes.c_int]
    lib.oracle_bmmc_apply_range.restype = ctypes.c_int
    lib.oracle_check_bijective.argtypes = [ctypes.c_int, u64p, ctypes.c_uint64,
                                           ctypes.c_void_p]
    lib.oracle_check_bijective.restype = ctypes.c_int
    lib.oracle_check_sampled.argtypes = [ctypes.c_int, u64p, ctypes.c_uint64,
                                         ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                         u64p, ctypes.c_uint64, u64p]
    lib.oracle_check_sampled.restype = ctypes.c_int64
    _lib = lib
    return lib


def _rows(A) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(A, dtype=np.uint64))
    return a


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))


def rank(A) -> int:
    """Rank over F2 of the matrix given as row masks."""
    a = _rows(A)
    return int(_load().oracle_gf2_rank(len(a), _p(a)))


def inverse(A) -> np.ndarray:
    """Inverse over F2 (row masks); raises ValueError if A is singular."""
    a = _rows(A)
    out = np.zeros_like(a)
    st = _load().oracle_gf2_inverse(len(a), _p(a), _p(out))
    if st != OK:
        raise ValueError("singular matrix" if st == SINGULAR else "bad argument")
    return out


def map_index(A, c: int, i: int) -> int:
    """y = A.i XOR c for one index."""
    a = _rows(A)
    return int(_load().oracle_map_index(len(a), _p(a), int(c), int(i)))


def map_indices(A, c: int, idx) -> np.ndarray:
    """y[k] = A.idx[k] XOR c for an array of indices (uint64)."""
    a = _rows(A)
    x = np.ascontiguousarray(np.asarray(idx, dtype=np.uint64))
    y = np.empty_like(x)
    _load().oracle_map_indices(len(a), _p(a), ctypes.c_uint64(int(c)),
                               x.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                               y.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                               ctypes.c_size_t(x.size))
    return y


def apply(A, c: int, x: np.ndarray, threads: int = 1) -> np.ndarray:
    """Return out with out[A.i XOR c] = x[i] over the whole array.

    ``x`` is any contiguous numpy array whose first axis has 2^n entries (the
    element is one row of the remaining axes, copied as raw bytes).
    """
    a = _rows(A)
    n = len(a)
    x = np.ascontiguousarray(x)
    if x.shape[0] != (1 << n):
        raise ValueError("array length is not 2^n")
    out = np.empty_like(x)
    elem = x.nbytes >> n
    st = _load().oracle_bmmc_apply(n, _p(a), int(c), elem, x.ctypes.data, out.ctypes.data,
                                   int(threads))
    if st != OK:
        raise ValueError({BAD_ARG: "bad argument", SINGULAR: "singular matrix"}.get(st, st))
    return out


def apply_range(A, c: int, x: np.ndarray, out: np.ndarray, i0: int, i1: int,
                threads: int = 1) -> None:
    """Scatter only the input indices in [i0, i1) into ``out``."""
    a = _rows(A)
    n = len(a)
    elem = x.nbytes >> n
    st = _load().oracle_bmmc_apply_range(n, _p(a), int(c), elem, x.ctypes.data,
                                         out.ctypes.data, int(i0), int(i1), int(threads))
    if st != OK:
        raise ValueError("oracle_bmmc_apply_range failed with status %d" % st)


def is_bijective(A, c: int) -> bool:
    """Mark every image A.i XOR c; True iff each index is hit exactly once."""
    a = _rows(A)
    n = len(a)
    seen = np.zeros(1 << n, dtype=np.uint8)
    st = _load().oracle_check_bijective(n, _p(a), int(c), seen.ctypes.data)
    if st == BAD_ARG:
        raise ValueError("bad argument")
    return st == OK


def check_sampled(A, c: int, x: np.ndarray, out: np.ndarray, idx: np.ndarray):
    """Count listed input indices i whose element is not at out[A.i XOR c].

    Returns (mismatches, first_bad_index or None).
    """
    a = _rows(A)
    n = len(a)
    elem = x.nbytes >> n
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    first = np.zeros(1, dtype=np.uint64)
    bad = _load().oracle_check_sampled(n, _p(a), int(c), elem, x.ctypes.data,
                                       out.ctypes.data, _p(idx), len(idx), _p(first))
    if bad < 0:
        raise ValueError("bad argument to oracle_check_sampled")
    return int(bad), (int(first[0]) if bad else None)
