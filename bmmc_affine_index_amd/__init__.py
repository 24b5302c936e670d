"""MI355X-native BMMC index permutations: out[A.i XOR c] = in[i].

A thin ctypes binding over ``libbmmc.so`` (built from ``csrc/`` by
``bmmc_affine_index_amd.build``).  The functions named like the C ABI
(``bmmc_plan_create``, ``bmmc_execute``, ``bmmc_copy``, ...) only marshal
arguments; every step of the permutation runs in the library's HIP kernels.
There is no CPU fallback: if the library is missing, every call raises.

Matrices are n row masks (``A[r]`` = mask of input bits feeding output bit r;
bit 0 = least significant index bit), as in include/bmmc.h.
"""
from __future__ import annotations

import collections
import ctypes
import os
import threading
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# BMMC_LIB names another build of the same library (the host-sanitized one
# the CPU tests load); by default the in-tree libbmmc.so.
LIB_PATH = os.environ.get("BMMC_LIB") or os.path.join(_HERE, "libbmmc.so")

# status codes (include/bmmc.h)
OK = 0
ERR_INVALID_ARG = 1
ERR_SINGULAR = 2
ERR_UNSUPPORTED = 3
ERR_ALIAS = 4
ERR_OUT_OF_MEMORY = 5
ERR_HIP = 6
ERR_SCRATCH_LIMIT = 7
NOALLOC_SCRATCH_BYTES = 1 << 26

KIND_IDENTITY, KIND_BPC, KIND_TILED, KIND_GENERAL = 0, 1, 2, 3
KIND_NAMES = {0: "identity", 1: "bpc", 2: "tiled", 3: "general"}
ROUTE_AUTO, ROUTE_NAIVE, ROUTE_TWO_PASS, ROUTE_FUSED = 0, 1, 2, 3
ROUTE_NAMES = {0: "auto", 1: "naive", 2: "two_pass", 3: "fused"}
KERNEL_COPY, KERNEL_CHUNK, KERNEL_TILED, KERNEL_NAIVE, KERNEL_CHUNK_SCATTER = 0, 1, 2, 3, 4
LAUNCH_AUTO, LAUNCH_ONE_TILE, LAUNCH_PERSISTENT, LAUNCH_STREAMED = 0, 1, 2, 3
WALK_AUTO, WALK_RANGES, WALK_INTERLEAVED = 0, 1, 2

MAX_N = 32
MAX_BITS = 36
MAX_TILE = 8
MAX_CHUNK_BITS = 16
MAX_PASSES = 2

EXPORTED = (
    "bmmc_plan_create", "bmmc_plan_create_ex", "bmmc_execute", "bmmc_execute_noalloc",
    "bmmc_plan_tune", "bmmc_plan_tune_pairs", "bmmc_plan_tune_candidates",
    "bmmc_copy",
    "bmmc_plan_destroy", "bmmc_last_error", "bmmc_status_string", "bmmc_plan_get_info",
    "bmmc_plan_get_factor", "bmmc_plan_get_pass", "bmmc_plan_get_options", "bmmc_parm_matrix",
    "bmmc_matrix_inverse", "bmmc_tensor_permute_matrix",
    "bmmc_testing_fail_scratch_allocs",
)


class bmmc_plan_options(ctypes.Structure):
    _fields_ = [("route", ctypes.c_int), ("tile_log2", ctypes.c_int),
                ("no_swizzle", ctypes.c_int), ("iters_log2", ctypes.c_int),
                ("launch", ctypes.c_int), ("grid_log2", ctypes.c_int),
                ("walk", ctypes.c_int), ("depth", ctypes.c_int), ("cache_hint", ctypes.c_int),
                ("block_map", ctypes.c_int), ("tile_skew", ctypes.c_int),
                ("tile_threads_log2", ctypes.c_int), ("split_stage", ctypes.c_int),
                ("buffer_loads", ctypes.c_int)]


class bmmc_plan_info(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("elem_bytes", ctypes.c_int), ("kind", ctypes.c_int),
                ("route", ctypes.c_int), ("passes", ctypes.c_int),
                ("unit_bytes", ctypes.c_int), ("unit_bits", ctypes.c_int),
                ("tile_log2", ctypes.c_int), ("n_over", ctypes.c_int),
                ("scratch_bytes", ctypes.c_size_t)]


class bmmc_pass_desc(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("unit_log2", ctypes.c_int32),
                ("nbits", ctypes.c_int32), ("t", ctypes.c_int32),
                ("chunk_log2", ctypes.c_int32), ("blk_bits", ctypes.c_int32),
                ("iters_log2", ctypes.c_int32), ("unit_xor", ctypes.c_int32),
                ("launch", ctypes.c_int32), ("grid_log2", ctypes.c_int32),
                ("walk", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("cache_hint", ctypes.c_int32), ("block_map", ctypes.c_int32),
                ("out_c", ctypes.c_uint64), ("lds_c", ctypes.c_uint32),
                ("lds_bytes", ctypes.c_uint32),
                ("in_blk", ctypes.c_uint64 * MAX_BITS), ("out_blk", ctypes.c_uint64 * MAX_BITS),
                ("lds_blk", ctypes.c_uint32 * MAX_BITS),
                ("ld_in", ctypes.c_uint64 * MAX_CHUNK_BITS),
                ("ld_lds", ctypes.c_uint32 * MAX_CHUNK_BITS),
                ("st_out", ctypes.c_uint64 * MAX_CHUNK_BITS),
                ("st_lds", ctypes.c_uint32 * MAX_CHUNK_BITS),
                ("st_unit", ctypes.c_uint32 * 4), ("in_c", ctypes.c_uint64),
                ("in_row_log2", ctypes.c_int32), ("out_row_log2", ctypes.c_int32),
                ("threads_log2", ctypes.c_int32), ("split_stage", ctypes.c_int32),
                ("buffer_loads", ctypes.c_int32)]


class BmmcError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = _status_text(status)
        super().__init__("%s%s (status %d)" % (what + ": " if what else "", msg, status))


_lib = None


def library_loaded() -> bool:
    return _lib is not None


def lib():
    """The loaded libbmmc.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libbmmc.so is missing at %s: build it with "
            "`python -m bmmc_affine_index_amd.build` (there is no fallback path)" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    L.bmmc_plan_create.argtypes = [ctypes.c_int, u64p, ctypes.c_uint64, ctypes.c_size_t]
    L.bmmc_plan_create.restype = ctypes.c_void_p
    L.bmmc_plan_create_ex.argtypes = [ctypes.c_int, u64p, ctypes.c_uint64, ctypes.c_size_t,
                                      ctypes.POINTER(bmmc_plan_options)]
    L.bmmc_plan_create_ex.restype = ctypes.c_void_p
    L.bmmc_execute.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p]
    L.bmmc_execute.restype = ctypes.c_int
    L.bmmc_execute_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
    L.bmmc_execute_noalloc.restype = ctypes.c_int
    L.bmmc_plan_tune.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int]
    L.bmmc_plan_tune.restype = ctypes.c_int
    L.bmmc_plan_tune_pairs.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                       ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int]
    L.bmmc_plan_tune_pairs.restype = ctypes.c_int
    L.bmmc_plan_tune_candidates.argtypes = [ctypes.c_void_p, ctypes.POINTER(bmmc_plan_options),
                                            ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.bmmc_plan_tune_candidates.restype = ctypes.c_int
    L.bmmc_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.bmmc_copy.restype = ctypes.c_int
    L.bmmc_plan_destroy.argtypes = [ctypes.c_void_p]
    L.bmmc_plan_destroy.restype = None
    L.bmmc_last_error.argtypes = []
    L.bmmc_last_error.restype = ctypes.c_int
    L.bmmc_status_string.argtypes = [ctypes.c_int]
    L.bmmc_status_string.restype = ctypes.c_char_p
    L.bmmc_plan_get_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(bmmc_plan_info)]
    L.bmmc_plan_get_info.restype = ctypes.c_int
    L.bmmc_plan_get_factor.argtypes = [ctypes.c_void_p, ctypes.c_int, u64p, u64p]
    L.bmmc_plan_get_factor.restype = ctypes.c_int
    L.bmmc_plan_get_pass.argtypes = [ctypes.c_void_p, ctypes.c_int,
                                     ctypes.POINTER(bmmc_pass_desc)]
    L.bmmc_plan_get_pass.restype = ctypes.c_int
    L.bmmc_plan_get_options.argtypes = [ctypes.c_void_p, ctypes.POINTER(bmmc_plan_options)]
    L.bmmc_plan_get_options.restype = ctypes.c_int
    L.bmmc_parm_matrix.argtypes = [ctypes.c_int, ctypes.c_uint64, u64p]
    L.bmmc_parm_matrix.restype = ctypes.c_int
    L.bmmc_matrix_inverse.argtypes = [ctypes.c_int, u64p, u64p]
    L.bmmc_matrix_inverse.restype = ctypes.c_int
    intp = ctypes.POINTER(ctypes.c_int)
    L.bmmc_tensor_permute_matrix.argtypes = [ctypes.c_int, intp, intp, ctypes.c_uint64, u64p,
                                             u64p, intp]
    L.bmmc_tensor_permute_matrix.restype = ctypes.c_int
    L.bmmc_testing_fail_scratch_allocs.argtypes = [ctypes.c_int]
    L.bmmc_testing_fail_scratch_allocs.restype = ctypes.c_int
    _lib = L
    return L


def _status_text(status: int) -> str:
    try:
        return lib().bmmc_status_string(int(status)).decode()
    except Exception:  # library missing: still report the code
        return "status"


def _rows(A: Sequence[int]):
    n = len(A)
    arr = (ctypes.c_uint64 * max(n, 1))(*[int(a) for a in A])
    return n, arr


def _ptr(x) -> int:
    """Device address of a torch tensor, or an int address as given."""
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError("expected a device tensor or an address")


def _stream(stream) -> Optional[int]:
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except ImportError:
            pass
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


# ---------------------------------------------------------------------------
# C-ABI names, marshalling only
# ---------------------------------------------------------------------------

def bmmc_plan_create(n: int, A: Sequence[int], c: int, elem_bytes: int) -> int:
    """Plan handle (an address) or 0; the reason of a 0 is bmmc_last_error()."""
    _, arr = _rows(A)
    return lib().bmmc_plan_create(int(n), arr, int(c), int(elem_bytes)) or 0


def bmmc_plan_create_ex(n: int, A: Sequence[int], c: int, elem_bytes: int,
                        route: int = ROUTE_AUTO, tile_log2: int = 0, no_swizzle: int = 0,
                        iters_log2: int = 0, launch: int = LAUNCH_AUTO,
                        grid_log2: int = 0, walk: int = WALK_AUTO, block_map: int = 0,
                        depth: int = 0, cache_hint: int = 0, tile_skew: int = 0,
                        tile_threads_log2: int = 0, split_stage: int = 0,
                        buffer_loads: int = 0) -> int:
    _, arr = _rows(A)
    opt = bmmc_plan_options(route, tile_log2, no_swizzle, iters_log2, launch, grid_log2, walk,
                            depth, cache_hint, block_map, tile_skew, tile_threads_log2,
                            split_stage, buffer_loads)
    return lib().bmmc_plan_create_ex(int(n), arr, int(c), int(elem_bytes),
                                     ctypes.byref(opt)) or 0


def bmmc_execute(plan: int, inp, out, stream=None) -> int:
    return lib().bmmc_execute(plan, _ptr(inp), _ptr(out), _stream(stream))


def bmmc_execute_noalloc(plan: int, inp, out, stream=None) -> int:
    return lib().bmmc_execute_noalloc(plan, _ptr(inp), _ptr(out), _stream(stream))


def bmmc_plan_tune(plan: int, inp, out, stream=None, reps: int = 0) -> int:
    return lib().bmmc_plan_tune(plan, _ptr(inp), _ptr(out), _stream(stream), int(reps))


def bmmc_plan_tune_pairs(plan: int, pairs, stream=None, reps: int = 0) -> int:
    """pairs: a sequence of (input, output) device buffers (tensors or
    addresses)."""
    k = len(pairs)
    ins = (ctypes.c_void_p * max(k, 1))(*[_ptr(i) for i, _ in pairs])
    outs = (ctypes.c_void_p * max(k, 1))(*[_ptr(o) for _, o in pairs])
    return lib().bmmc_plan_tune_pairs(plan, ins if k else None, outs if k else None, k,
                                      _stream(stream), int(reps))


def bmmc_plan_tune_candidates(plan: int):
    """Options of every candidate bmmc_plan_tune_pairs would time, in order."""
    count = ctypes.c_int()
    st = lib().bmmc_plan_tune_candidates(plan, None, 0, ctypes.byref(count))
    if st != OK:
        raise BmmcError(st, "bmmc_plan_tune_candidates")
    opts = (bmmc_plan_options * max(count.value, 1))()
    st = lib().bmmc_plan_tune_candidates(plan, opts, count.value, ctypes.byref(count))
    if st != OK:
        raise BmmcError(st, "bmmc_plan_tune_candidates")
    return [{name: int(getattr(o, name)) for name, _ in bmmc_plan_options._fields_}
            for o in opts[:count.value]]


def bmmc_copy(inp, out, nbytes: int, stream=None) -> int:
    return lib().bmmc_copy(_ptr(inp), _ptr(out), int(nbytes), _stream(stream))


def bmmc_testing_fail_scratch_allocs(count: int) -> int:
    """Fault injection (include/bmmc_testing.h): the next `count` scratch
    allocations of two-pass plans fail with ERR_OUT_OF_MEMORY."""
    return lib().bmmc_testing_fail_scratch_allocs(int(count))


def bmmc_plan_destroy(plan: int) -> None:
    if plan:
        lib().bmmc_plan_destroy(plan)


def bmmc_last_error() -> int:
    return lib().bmmc_last_error()


def bmmc_status_string(status: int) -> str:
    return lib().bmmc_status_string(int(status)).decode()


def bmmc_plan_get_info(plan: int) -> bmmc_plan_info:
    info = bmmc_plan_info()
    st = lib().bmmc_plan_get_info(plan, ctypes.byref(info))
    if st != OK:
        raise BmmcError(st, "bmmc_plan_get_info")
    return info


def bmmc_plan_get_factor(plan: int, pass_index: int, n: int):
    A = (ctypes.c_uint64 * n)()
    c = ctypes.c_uint64()
    st = lib().bmmc_plan_get_factor(plan, int(pass_index), A, ctypes.byref(c))
    if st != OK:
        raise BmmcError(st, "bmmc_plan_get_factor")
    return [int(a) for a in A], int(c.value)


def bmmc_plan_get_options(plan: int) -> dict:
    o = bmmc_plan_options()
    st = lib().bmmc_plan_get_options(plan, ctypes.byref(o))
    if st != OK:
        raise BmmcError(st, "bmmc_plan_get_options")
    return {name: int(getattr(o, name)) for name, _ in bmmc_plan_options._fields_}


def bmmc_plan_get_pass(plan: int, pass_index: int) -> bmmc_pass_desc:
    d = bmmc_pass_desc()
    st = lib().bmmc_plan_get_pass(plan, int(pass_index), ctypes.byref(d))
    if st != OK:
        raise BmmcError(st, "bmmc_plan_get_pass")
    return d


def bmmc_parm_matrix(n: int, mask: int):
    """Row masks of the BMMC that parm conjugates with (see include/bmmc.h)."""
    A = (ctypes.c_uint64 * max(n, 1))()
    st = lib().bmmc_parm_matrix(int(n), int(mask), A)
    if st != OK:
        raise BmmcError(st, "bmmc_parm_matrix")
    return [int(a) for a in A[:n]]


def bmmc_matrix_inverse(A: Sequence[int]):
    """Row masks of A^{-1} over F2."""
    n, arr = _rows(A)
    out = (ctypes.c_uint64 * max(n, 1))()
    st = lib().bmmc_matrix_inverse(n, arr, out)
    if st != OK:
        raise BmmcError(st, "bmmc_matrix_inverse")
    return [int(a) for a in out[:n]]


def bmmc_tensor_permute_matrix(dim_log2: Sequence[int], perm: Sequence[int],
                               flip_mask: int = 0):
    """(A, c, n) of the BPC that permutes and flips tensor dimensions."""
    k = len(dim_log2)
    dl = (ctypes.c_int * k)(*[int(v) for v in dim_log2])
    pm = (ctypes.c_int * k)(*[int(v) for v in perm])
    A = (ctypes.c_uint64 * MAX_N)()
    c = ctypes.c_uint64()
    n = ctypes.c_int()
    st = lib().bmmc_tensor_permute_matrix(k, dl, pm, int(flip_mask), A, ctypes.byref(c),
                                          ctypes.byref(n))
    if st != OK:
        raise BmmcError(st, "bmmc_tensor_permute_matrix")
    return [int(a) for a in A[:n.value]], int(c.value), n.value


# ---------------------------------------------------------------------------
# Convenience wrapper
# ---------------------------------------------------------------------------

class Plan:
    """Owns a bmmc_plan; ``plan(inp, out)`` runs it on device tensors."""

    def __init__(self, n: int, A: Sequence[int], c: int, elem_bytes: int,
                 route: int = ROUTE_AUTO, tile_log2: int = 0, no_swizzle: bool = False,
                 iters_log2: int = 0, launch: int = LAUNCH_AUTO, grid_log2: int = 0,
                 walk: int = WALK_AUTO, block_map: int = 0, depth: int = 0,
                 cache_hint: int = 0, tile_skew: int = 0, tile_threads_log2: int = 0,
                 split_stage: int = 0, buffer_loads: int = 0):
        self.n, self.elem_bytes = int(n), int(elem_bytes)
        self.A, self.c = [int(a) for a in A], int(c)
        self.handle = bmmc_plan_create_ex(n, A, c, elem_bytes, route, tile_log2,
                                          int(bool(no_swizzle)), iters_log2, launch, grid_log2,
                                          walk, block_map, depth, cache_hint, tile_skew,
                                          tile_threads_log2, split_stage, buffer_loads)
        if not self.handle:
            raise BmmcError(bmmc_last_error(), "bmmc_plan_create")
        self.info = bmmc_plan_get_info(self.handle)

    @property
    def nbytes(self) -> int:
        return self.elem_bytes << self.n

    def options(self) -> dict:
        """Keyword arguments that rebuild this plan's current tables
        (bmmc_plan_get_options): ``Plan(n, A, c, elem_bytes, **p.options())``."""
        return bmmc_plan_get_options(self.handle)

    def tune_candidates(self) -> list:
        """Options of every plan ``tune`` would time, in order
        (bmmc_plan_tune_candidates); each rebuilds with
        ``Plan(n, A, c, elem_bytes, **opts)``."""
        return bmmc_plan_tune_candidates(self.handle)

    def passes(self):
        return [bmmc_plan_get_pass(self.handle, k) for k in range(self.info.passes)]

    def factors(self):
        return [bmmc_plan_get_factor(self.handle, k, self.n) for k in range(self.info.passes)]

    def __call__(self, inp, out, stream=None) -> None:
        self._check(inp, out)
        st = bmmc_execute(self.handle, inp, out, stream)
        if st != OK:
            raise BmmcError(st, "bmmc_execute")

    def _check(self, inp, out) -> None:
        for t in (inp, out):
            if hasattr(t, "is_cuda"):
                if not t.is_cuda or not t.is_contiguous():
                    raise ValueError("tensors must be contiguous device tensors")
                if t.numel() * t.element_size() != self.nbytes:
                    raise ValueError("tensor holds %d bytes, the plan moves %d"
                                     % (t.numel() * t.element_size(), self.nbytes))

    def tune(self, inp=None, out=None, stream=None, reps: int = 0, pairs=None) -> None:
        """Time the candidate tile orders and keep the fastest
        (bmmc_plan_tune_pairs), rotating over ``pairs`` [(in, out), ...] or
        the one pair (inp, out); the first output then holds the permutation
        of the first input."""
        pairs = list(pairs) if pairs is not None else [(inp, out)]
        for i, o in pairs:
            self._check(i, o)
        st = bmmc_plan_tune_pairs(self.handle, pairs, stream, reps)
        if st != OK:
            raise BmmcError(st, "bmmc_plan_tune_pairs")
        self.info = bmmc_plan_get_info(self.handle)

    def close(self) -> None:
        if getattr(self, "handle", 0):
            bmmc_plan_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def describe(self) -> dict:
        i = self.info
        launch = [{1: "one_tile", 2: "persistent", 3: "streamed"}.get(d.launch, "-")
                  if d.kernel == KERNEL_TILED
                  else {0: "copy", 1: "chunk", 3: "naive", 4: "chunk_scatter"}.get(d.kernel, "?")
                  for d in self.passes()]
        grid = [d.grid_log2 for d in self.passes() if d.kernel == KERNEL_TILED]
        walk = [{1: "ranges", 2: "interleaved"}.get(d.walk) for d in self.passes()
                if d.kernel == KERNEL_TILED and d.launch in (LAUNCH_PERSISTENT, LAUNCH_STREAMED)]
        depth = [d.depth for d in self.passes()
                 if d.kernel == KERNEL_TILED and d.launch == LAUNCH_STREAMED]
        bmap = [d.block_map for d in self.passes() if d.kernel == KERNEL_TILED]
        skew = [d.out_row_log2 - d.t for d in self.passes() if d.kernel == KERNEL_TILED]
        thr = [d.threads_log2 for d in self.passes() if d.kernel == KERNEL_TILED]
        split = [d.split_stage for d in self.passes() if d.kernel == KERNEL_TILED]
        bufld = [d.buffer_loads for d in self.passes() if d.kernel == KERNEL_TILED]
        return {"n": i.n, "elem_bytes": i.elem_bytes, "kind": KIND_NAMES[i.kind],
                "route": ROUTE_NAMES[i.route], "passes": i.passes, "unit_bytes": i.unit_bytes,
                "unit_bits": i.unit_bits, "tile_log2": i.tile_log2, "n_over": i.n_over,
                "scratch_bytes": i.scratch_bytes, "kernels": launch,
                "grid_log2": grid[0] if grid else None, "walk": walk[0] if walk else None,
                "depth": depth[0] if depth else None,
                "block_map": bmap[0] if bmap else None,
                "tile_skew": skew[-1] if skew else None,
                "tile_threads": (1 << thr[-1]) if thr else None,
                "split_stage": split[-1] if split else None,
                "buffer_loads": bufld[-1] if bufld else None}


def copy(inp, out, nbytes: Optional[int] = None, stream=None) -> None:
    if nbytes is None:
        nbytes = inp.numel() * inp.element_size()
    st = bmmc_copy(inp, out, nbytes, stream)
    if st != OK:
        raise BmmcError(st, "bmmc_copy")


def _ordered(run, tensors, stream) -> None:
    """Call run(stream_handle) on `stream` (None = torch's current stream)
    in order with torch's current stream: the launch waits for work already
    queued on the current stream (the producers of the inputs), the current
    stream then waits for the launch (so its later work sees the outputs),
    and the tensors are recorded as used on `stream` for the caching
    allocator."""
    import torch
    cur = torch.cuda.current_stream()
    if stream is None:
        run(int(cur.cuda_stream))
        return
    side = (torch.cuda.ExternalStream(int(stream)) if isinstance(stream, int) else stream)
    if int(side.cuda_stream) == int(cur.cuda_stream):
        run(int(cur.cuda_stream))
        return
    side.wait_stream(cur)
    run(int(side.cuda_stream))
    for t in tensors:
        t.record_stream(side)
    cur.wait_stream(side)


# Plans the front-end made, most recently used last: planning costs tens of
# microseconds to a millisecond on the host, a single-pass plan holds no
# device memory and its tables do not change while it runs, so one plan
# serves every later call with the same map, element size and options, on
# any stream.  Plans with a scratch array (the two-pass route) are not kept.
_PLAN_CACHE = collections.OrderedDict()
_PLAN_CACHE_SIZE = 32
_PLAN_CACHE_LOCK = threading.Lock()


def _cached_plan(n: int, A: Sequence[int], c: int, elem: int, plan_kw: dict,
                 tuned: bool = False, tune_fn=None) -> "Plan":
    """The kept plan for this map, element size and options (tuned ones are
    kept apart from untuned ones), or a new one; a new plan for a tuned call
    is tuned by tune_fn(plan) before it is kept."""
    key = (n, tuple(int(a) for a in A), int(c), int(elem), tuple(sorted(plan_kw.items())),
           bool(tuned))
    with _PLAN_CACHE_LOCK:
        plan = _PLAN_CACHE.get(key)
        if plan is not None:
            _PLAN_CACHE.move_to_end(key)
            return plan
    plan = Plan(n, A, c, elem, **plan_kw)
    if tuned and tune_fn is not None:
        tune_fn(plan)
    if plan.info.scratch_bytes == 0:
        with _PLAN_CACHE_LOCK:
            _PLAN_CACHE[key] = plan
            while len(_PLAN_CACHE) > _PLAN_CACHE_SIZE:
                _PLAN_CACHE.popitem(last=False)
    return plan


def clear_plan_cache() -> None:
    """Drop the plans kept by permute, parm, permute_dims, flip and transpose2d."""
    with _PLAN_CACHE_LOCK:
        _PLAN_CACHE.clear()


def permute(inp, A: Sequence[int], c: int = 0, out=None, stream=None, tune: bool = False,
            **plan_kw):
    """out[A.i XOR c] = inp[i] over the first axis of a contiguous device
    tensor with 2^n rows (a row is one element).  With a `stream` other than
    torch's current one, the permutation runs there, ordered after the work
    already queued on the current stream and before the work queued on it
    afterwards.  Single-pass plans are kept for later calls with the same
    map (clear_plan_cache drops them).  tune=True tunes a new plan on this
    call's tensors (bmmc_plan_tune) before it is kept, so later tuned calls
    with the same map run the tuned plan without timing."""
    import torch
    n = len(A)
    if inp.shape[0] != (1 << n):
        raise ValueError("first axis must have 2^n entries")
    elem = inp.numel() * inp.element_size() >> n
    if out is None:
        out = torch.empty_like(inp)

    def tune_fn(plan):
        _ordered(lambda h: plan.tune(inp, out, stream=h), [inp, out], stream)
    plan = _cached_plan(n, A, c, elem, plan_kw, tuned=tune, tune_fn=tune_fn)
    _ordered(lambda h: plan(inp, out, h), [inp, out], stream)
    return out


# ---------------------------------------------------------------------------
# Users of the permutation: parm and tensor dimensions
# ---------------------------------------------------------------------------

def parm(x, mask: int, f, stream=None, tune: bool = False):
    """parm mask f x: split the 2^n rows of x by the F2 dot product i.mask,
    apply f to the part with i.mask = 0 and to the other part (each in
    increasing index order, as a tensor of 2^(n-1) rows), and stitch the
    results back in place of the parts.  f takes and returns a device tensor
    of the same shape.  The two permutations run in this library's kernels."""
    import torch
    rows = x.shape[0]
    n = rows.bit_length() - 1
    if rows != (1 << n) or n < 1:
        raise ValueError("the first axis must have 2^n entries, n >= 1")
    A = bmmc_parm_matrix(n, mask)
    y = permute(x, A, 0, stream=stream, tune=tune)
    half = rows // 2
    z = torch.empty_like(y)
    z[:half] = f(y[:half])
    z[half:] = f(y[half:])
    return permute(z, bmmc_matrix_inverse(A), 0, stream=stream, tune=tune)


def permute_dims(t, perm: Sequence[int], flip: Sequence[int] = (), stream=None,
                 tune: bool = False):
    """t.flip(flip).permute(perm).contiguous() for a contiguous device tensor
    whose dimensions are powers of two, as one BPC permutation (tune as in
    permute)."""
    shape = list(t.shape)
    dl = []
    for s in shape:
        if s < 1 or s & (s - 1):
            raise ValueError("every dimension must be a power of two")
        dl.append(s.bit_length() - 1)
    fm = 0
    for d in flip:
        fm |= 1 << (d % len(shape))
    A, c, n = bmmc_tensor_permute_matrix(dl, [p % len(shape) for p in perm], fm)
    out_shape = [shape[p % len(shape)] for p in perm]
    if n == 0:
        return t.clone().reshape(out_shape)
    flat = t.reshape(1 << n, -1) if t.numel() else t
    return permute(flat, A, c, stream=stream, tune=tune).reshape(out_shape)


def flip(t, dims: Sequence[int], stream=None, tune: bool = False):
    """t.flip(dims) for power-of-two dimensions, as one BPC permutation."""
    return permute_dims(t, list(range(t.dim())), flip=dims, stream=stream, tune=tune)


def transpose2d(t, stream=None, tune: bool = False):
    """The transpose of a 2^a x 2^b matrix (a rotation of the index bits)."""
    return permute_dims(t, [1, 0], stream=stream, tune=tune)
