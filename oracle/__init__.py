"""CPU oracle for the N-way tensor-parallel AllReduce sum and its protocol models.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``message_allreduce_amd``) and never imports it.

Contents
--------
* ``oracle.c`` / this module: the reduction result (plain definition):
  decode each element to binary64, add in rank order starting from rank 0's
  value, round once to the output type (round-to-nearest-even).  Source: "Every
  Microsecond Matters: Achieving Near Speed-of-Light Latency in GPU
  Collectives" (agihunt.info summary) -- the per-token AllReduce merges the
  tensor-parallel shard outputs; paragraph "Two-shot LL128": add-only, FP32 /
  FP16 / BF16.
* ``pyref.py``: a second, pure-Python implementation of the same definition
  that rounds by exact rational comparison (small cases only), used to pin the
  C code.
* ``reduce_scatter``: segment j of the same sum for rank j (definition from
  the yololab.net article's collective table).
* ``models.py``: bit-level models of the LL line, the Sentinel buffer, the
  LL128 atomic line, the double-buffer/credit schedule, and what a receiver
  gets over a wire (point-to-point and AllGather).

dtype codes: ``F32 = 0``, ``F16 = 1``, ``BF16 = 2``.  Element arrays are
passed as their bit patterns (``uint32`` for binary32, ``uint16`` otherwise).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "fp32", F16: "fp16", BF16: "bf16"}
BITS_DTYPE = {F32: np.uint32, F16: np.uint16, BF16: np.uint16}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain C, no GPU code)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        vp, sz, i32, dp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double)
        lib.oracle_allreduce.argtypes = [ctypes.POINTER(vp), i32, sz, i32, vp]
        lib.oracle_allreduce.restype = i32
        lib.oracle_sum_f64.argtypes = [ctypes.POINTER(vp), i32, sz, i32, vp]
        lib.oracle_sum_f64.restype = i32
        lib.oracle_decode_array.argtypes = [i32, vp, sz, vp]
        lib.oracle_decode_array.restype = None
        lib.oracle_round_array.argtypes = [i32, vp, sz, vp]
        lib.oracle_round_array.restype = None
        lib.oracle_decode_bits.argtypes = [i32, ctypes.c_uint32]
        lib.oracle_decode_bits.restype = ctypes.c_double
        lib.oracle_round_bits.argtypes = [i32, ctypes.c_double]
        lib.oracle_round_bits.restype = ctypes.c_uint32
        del dp
        _lib = lib
    return _lib


def as_bits(a: np.ndarray, dtype: int) -> np.ndarray:
    """View an array of the element type (float32/float16/raw uint16) as bits."""
    a = np.ascontiguousarray(a)
    want = BITS_DTYPE[dtype]
    if a.dtype == want:
        return a
    if a.dtype.itemsize != np.dtype(want).itemsize:
        raise TypeError("element size %d does not match %s" % (a.dtype.itemsize, DTYPE_NAMES[dtype]))
    return a.view(want)


def _rank_ptrs(parts: np.ndarray):
    n_ranks = parts.shape[0]
    arr = (ctypes.c_void_p * n_ranks)()
    for r in range(n_ranks):
        arr[r] = parts[r].ctypes.data
    return arr


def allreduce(partials: np.ndarray, dtype: int) -> np.ndarray:
    """out[i] = RNE_T(sum_r partials[r, i]) with binary64 rank-order sums.

    ``partials``: shape (N, n) array of the element bits (or float32/float16).
    Returns an (n,) array of output bits.
    """
    parts = np.ascontiguousarray(as_bits(np.asarray(partials), dtype))
    if parts.ndim != 2:
        raise ValueError("partials must be (N, n)")
    n_ranks, n = parts.shape
    out = np.empty(n, dtype=BITS_DTYPE[dtype])
    rc = _load().oracle_allreduce(_rank_ptrs(parts), n_ranks, n, dtype, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_allreduce rejected its arguments")
    return out


def allreduce_threads(partials: np.ndarray, dtype: int, threads: int) -> np.ndarray:
    """``allreduce`` with the elements split into ``threads`` contiguous
    ranges, each reduced by the same C routine on its own host thread (the
    call releases the interpreter lock).  Every element is an independent
    sum, so the result is identical; only the wall time changes."""
    import concurrent.futures as cf
    parts = np.ascontiguousarray(as_bits(np.asarray(partials), dtype))
    n_ranks, n = parts.shape
    out = np.empty(n, dtype=BITS_DTYPE[dtype])
    threads = max(1, min(int(threads), n))
    bounds = [n * t // threads for t in range(threads + 1)]
    lib = _load()
    esz = parts.dtype.itemsize

    def run(t):
        lo, hi = bounds[t], bounds[t + 1]
        if hi <= lo:
            return 0
        arr = (ctypes.c_void_p * n_ranks)(*[parts[r].ctypes.data + lo * esz for r in range(n_ranks)])
        return lib.oracle_allreduce(arr, n_ranks, hi - lo, dtype, out.ctypes.data + lo * esz)

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        rcs = list(ex.map(run, range(threads)))
    if any(rcs):
        raise ValueError("oracle_allreduce rejected its arguments")
    return out


def reduce_scatter(partials: np.ndarray, dtype: int) -> list:
    """Rank j keeps segment j of the element-wise sum: the yololab.net article
    on network architecture for LLM inference, table of its All-Reduce /
    All-Gather / Reduce-Scatter section.  ``partials``: (N, N * c) bits;
    returns N arrays of c output bits, segment j = elements [j c, (j+1) c)
    summed like ``allreduce`` (binary64 in rank order, one rounding)."""
    parts = np.ascontiguousarray(as_bits(np.asarray(partials), dtype))
    n_ranks, n = parts.shape
    if n % n_ranks:
        raise ValueError("each partial must hold N equal segments")
    c = n // n_ranks
    return [allreduce(parts[:, j * c:(j + 1) * c], dtype) for j in range(n_ranks)]


def sum_f64(partials: np.ndarray, dtype: int) -> np.ndarray:
    """The binary64 rank-order sum before the final rounding."""
    parts = np.ascontiguousarray(as_bits(np.asarray(partials), dtype))
    n_ranks, n = parts.shape
    out = np.empty(n, dtype=np.float64)
    rc = _load().oracle_sum_f64(_rank_ptrs(parts), n_ranks, n, dtype, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_sum_f64 rejected its arguments")
    return out


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact binary64 value of each element bit pattern."""
    b = np.ascontiguousarray(as_bits(np.asarray(bits), dtype))
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode_array(dtype, b.ctypes.data, b.size, out.ctypes.data)
    return out


def round_to(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round binary64 values to the nearest element (ties to even); returns bits."""
    xx = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(xx.shape, dtype=BITS_DTYPE[dtype])
    _load().oracle_round_array(dtype, xx.ctypes.data, xx.size, out.ctypes.data)
    return out


def is_nan_bits(bits: np.ndarray, dtype: int) -> np.ndarray:
    """NaN test on bit patterns (exponent all ones, fraction non-zero)."""
    b = np.asarray(bits).astype(np.uint64)
    if dtype == F32:
        return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)
    if dtype == F16:
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def same_result(got_bits: np.ndarray, want_bits: np.ndarray, dtype: int) -> np.ndarray:
    """Element-wise bit equality, with any NaN equal to any NaN."""
    g = np.asarray(got_bits)
    w = np.asarray(want_bits)
    gn = is_nan_bits(g, dtype)
    wn = is_nan_bits(w, dtype)
    return np.where(gn | wn, gn & wn, g == w)
