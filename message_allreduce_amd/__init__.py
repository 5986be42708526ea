"""message_allreduce_amd -- barrier-free small-message AllReduce protocols
(LL, Sentinel, two-shot LL128 atomic, double-buffered pipelines) with N
tensor-parallel ranks emulated on one MI355X.

The work is done by the C-ABI library ``libllar.so`` (hand-written HIP for
gfx950, see ``include/llar.h``); this package only marshals arguments to it
through ctypes.  PyTorch supplies device memory and streams.  There is no
fallback path: if the library or a GPU is missing, the calls raise.

Python names mirror the C ABI::

    h = llar_create(n_ranks, dtype, max_bytes)
    llar_allreduce(h, partials, out, n_elems, dtype, protocol, stream)
    llar_send_recv(h, send, recv, n_elems, dtype, protocol, stream)
    llar_reduce_scatter(h, partials, outs, recv_count, dtype, protocol, stream)
    llar_all_gather(h, inputs, outs, n_outs, send_count, dtype, protocol, stream)
    llar_destroy(h)

and ``Communicator`` wraps them for torch tensors.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "FP32", "FP16", "BF16", "AUTO", "LL", "SENTINEL", "LL128", "LL128_PIPELINED", "SENTINEL_PIPELINED",
    "PROTOCOLS", "LlarError", "lib", "library_path", "llar_create", "llar_allreduce", "llar_destroy",
    "llar_send_recv", "llar_reduce_scatter", "llar_all_gather", "llar_allreduce_noalloc", "llar_set_option", "llar_get_option", "llar_get_device_status", "llar_clear_device_status",
    "llar_select_protocol", "llar_debug_copy_staging", "llar_staging_bytes", "llar_get_epoch",
    "llar_get_timing", "llar_wallclock_hz", "llar_launch_geometry", "llar_floor_measure",
    "llar_status_string", "llar_last_error", "llar_get_trace", "llar_get_pipeline_trace", "Communicator", "EXPORTED_SYMBOLS",
]

FP32, FP16, BF16 = 0, 1, 2
AUTO, LL, SENTINEL, LL128, LL128_PIPELINED, SENTINEL_PIPELINED = 0, 1, 2, 3, 4, 5
PROTOCOLS = {"auto": AUTO, "ll": LL, "sentinel": SENTINEL, "ll128": LL128,
             "ll128_pipelined": LL128_PIPELINED, "sentinel_pipelined": SENTINEL_PIPELINED}
STATUS = {0: "LLAR_OK", -1: "LLAR_ERR_ARG", -2: "LLAR_ERR_UNSUPPORTED", -3: "LLAR_ERR_NOMEM",
          -4: "LLAR_ERR_HIP", -5: "LLAR_ERR_TIMEOUT", -6: "LLAR_ERR_DEVICE"}

# every symbol include/llar.h declares
EXPORTED_SYMBOLS = (
    "llar_create", "llar_allreduce", "llar_destroy", "llar_last_error", "llar_status_string",
    "llar_get_device_status", "llar_clear_device_status", "llar_set_option", "llar_get_option",
    "llar_select_protocol", "llar_debug_copy_staging", "llar_staging_bytes", "llar_get_epoch",
    "llar_get_timing", "llar_wallclock_hz", "llar_launch_geometry", "llar_floor_measure",
    "llar_get_trace", "llar_get_pipeline_trace", "llar_send_recv", "llar_reduce_scatter", "llar_all_gather",
    "llar_allreduce_noalloc",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libllar.so")
_lib = None


class LlarError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s%s" % (what + ": " if what else "", STATUS.get(status, "status %d" % status)))


def lib() -> ctypes.CDLL:
    """Load libllar.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise LlarError(-4, "libllar.so is not built (run __graft_entry__.build()) at %s" % library_path)
    L = ctypes.CDLL(library_path)
    vp, sz, i32, ll = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_longlong
    u32p, u64p = ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint64)
    ip = ctypes.POINTER(ctypes.c_int)
    sig = {
        "llar_create": (vp, [i32, i32, sz]),
        "llar_allreduce": (i32, [vp, ctypes.POINTER(vp), vp, sz, i32, i32, vp]),
        "llar_allreduce_noalloc": (i32, [i32, ctypes.POINTER(vp), vp, sz, i32, vp]),
        "llar_send_recv": (i32, [vp, vp, vp, sz, i32, i32, vp]),
        "llar_reduce_scatter": (i32, [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), sz, i32, i32, vp]),
        "llar_all_gather": (i32, [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, sz, i32, i32, vp]),
        "llar_destroy": (i32, [vp]),
        "llar_last_error": (i32, []),
        "llar_status_string": (ctypes.c_char_p, [i32]),
        "llar_get_device_status": (i32, [vp, u32p]),
        "llar_clear_device_status": (i32, [vp]),
        "llar_set_option": (i32, [vp, ctypes.c_char_p, ll]),
        "llar_get_option": (i32, [vp, ctypes.c_char_p, ctypes.POINTER(ll)]),
        "llar_select_protocol": (i32, [vp, sz]),
        "llar_debug_copy_staging": (i32, [vp, i32, vp, sz]),
        "llar_staging_bytes": (sz, [vp, i32]),
        "llar_get_epoch": (i32, [vp, u32p]),
        "llar_get_timing": (i32, [vp, u64p, i32]),
        "llar_wallclock_hz": (ctypes.c_double, []),
        "llar_launch_geometry": (i32, [vp, sz, i32, ip, ip, ip, ip]),
        "llar_floor_measure": (i32, [i32, i32, ctypes.POINTER(ctypes.c_double)]),
        "llar_get_trace": (i32, [vp, u64p, i32]),
        "llar_get_pipeline_trace": (i32, [vp, u64p, i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int, what: str) -> int:
    if status < 0:
        raise LlarError(status, what)
    return status


# ---- thin wrappers with the C names --------------------------------------------
def llar_create(n_ranks: int, dtype: int, max_bytes: int) -> int:
    h = lib().llar_create(int(n_ranks), int(dtype), int(max_bytes))
    if not h:
        raise LlarError(lib().llar_last_error(), "llar_create")
    return h


def llar_allreduce(h: int, partials, out: int, n_elems: int, dtype: int, protocol: int, stream: int) -> int:
    """partials: sequence of device pointers (ints); out: device pointer."""
    arr = (ctypes.c_void_p * len(partials))(*[int(p) for p in partials])
    return lib().llar_allreduce(h, arr, ctypes.c_void_p(int(out)), int(n_elems), int(dtype), int(protocol),
                                ctypes.c_void_p(int(stream)))


def llar_allreduce_noalloc(n_ranks: int, partials, out: int, n_elems: int, dtype: int, stream: int) -> int:
    """The LL AllReduce over the library's static per-GPU array (no
    communicator, no allocation); partials: device pointers (ints)."""
    arr = (ctypes.c_void_p * len(partials))(*[int(p) for p in partials])
    return lib().llar_allreduce_noalloc(int(n_ranks), arr, ctypes.c_void_p(int(out)), int(n_elems), int(dtype),
                                        ctypes.c_void_p(int(stream)))


def llar_send_recv(h: int, send: int, recv: int, n_elems: int, dtype: int, protocol: int, stream: int) -> int:
    """send, recv: device pointers (ints)."""
    return lib().llar_send_recv(h, ctypes.c_void_p(int(send)), ctypes.c_void_p(int(recv)), int(n_elems), int(dtype),
                                int(protocol), ctypes.c_void_p(int(stream)))


def _ptrs(seq):
    return (ctypes.c_void_p * len(seq))(*[int(p) for p in seq])


def llar_reduce_scatter(h: int, partials, outs, recv_count: int, dtype: int, protocol: int, stream: int) -> int:
    """partials, outs: sequences of device pointers (ints)."""
    return lib().llar_reduce_scatter(h, _ptrs(partials), _ptrs(outs), int(recv_count), int(dtype), int(protocol),
                                     ctypes.c_void_p(int(stream)))


def llar_all_gather(h: int, inputs, outs, send_count: int, dtype: int, protocol: int, stream: int) -> int:
    """inputs, outs: sequences of device pointers (ints); len(outs) is n_outs."""
    return lib().llar_all_gather(h, _ptrs(inputs), _ptrs(outs), len(outs), int(send_count), int(dtype),
                                 int(protocol), ctypes.c_void_p(int(stream)))


def llar_destroy(h: int) -> int:
    return lib().llar_destroy(h)


def llar_last_error() -> int:
    return lib().llar_last_error()


def llar_status_string(status: int) -> str:
    return lib().llar_status_string(int(status)).decode()


def llar_set_option(h: int, key: str, value: int) -> int:
    return lib().llar_set_option(h, key.encode(), int(value))


def llar_get_option(h: int, key: str) -> int:
    v = ctypes.c_longlong(0)
    _check(lib().llar_get_option(h, key.encode(), ctypes.byref(v)), "llar_get_option(%s)" % key)
    return v.value


def llar_get_device_status(h: int):
    bits = ctypes.c_uint32(0)
    st = lib().llar_get_device_status(h, ctypes.byref(bits))
    return st, bits.value


def llar_clear_device_status(h: int) -> int:
    return lib().llar_clear_device_status(h)


def llar_select_protocol(h: int, nbytes: int) -> int:
    return lib().llar_select_protocol(h, int(nbytes))


def llar_staging_bytes(h: int, protocol: int) -> int:
    return lib().llar_staging_bytes(h, int(protocol))


def llar_debug_copy_staging(h: int, protocol: int, nbytes: int):
    import numpy as np
    buf = np.empty(int(nbytes), dtype=np.uint8)
    _check(lib().llar_debug_copy_staging(h, int(protocol), buf.ctypes.data, int(nbytes)), "llar_debug_copy_staging")
    return buf


def llar_get_epoch(h: int) -> int:
    e = ctypes.c_uint32(0)
    _check(lib().llar_get_epoch(h, ctypes.byref(e)), "llar_get_epoch")
    return e.value


def llar_get_timing(h: int, count: int):
    """List of (first_start, last_end) wall-clock ticks of the last `count` calls."""
    arr = (ctypes.c_uint64 * (2 * int(count)))()
    n = _check(lib().llar_get_timing(h, arr, int(count)), "llar_get_timing")
    return [(arr[2 * i], arr[2 * i + 1]) for i in range(n)]


def llar_get_trace(h: int, max_records: int = 4096):
    """(n_workgroups, 8) uint64 phase stamps of the last traced one-shot call."""
    import numpy as np
    buf = np.zeros((int(max_records), 8), dtype=np.uint64)
    n = _check(lib().llar_get_trace(h, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), int(max_records)),
               "llar_get_trace")
    return buf[:n]


def llar_get_pipeline_trace(h: int, max_records: int = 1024):
    """(n_workgroups, 512) uint64 per-chunk stamps of the last traced pipelined call."""
    import numpy as np
    buf = np.zeros((int(max_records), 512), dtype=np.uint64)
    n = _check(lib().llar_get_pipeline_trace(h, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), int(max_records)),
               "llar_get_pipeline_trace")
    return buf[:n]


def llar_wallclock_hz() -> float:
    return lib().llar_wallclock_hz()


def llar_launch_geometry(h: int, n_elems: int, protocol: int):
    g, t, s, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().llar_launch_geometry(h, int(n_elems), int(protocol), ctypes.byref(g), ctypes.byref(t),
                                      ctypes.byref(s), ctypes.byref(c)), "llar_launch_geometry")
    return {"grid": g.value, "threads": t.value, "slices": s.value, "chunks": c.value}


def llar_floor_measure(kind: int, param: int = 0) -> float:
    v = ctypes.c_double(0.0)
    _check(lib().llar_floor_measure(int(kind), int(param), ctypes.byref(v)), "llar_floor_measure(%d)" % kind)
    return v.value


# ---- torch convenience -------------------------------------------------------------
_TORCH_DTYPE = None


def _dtype_code(t) -> int:
    import torch
    m = {torch.float32: FP32, torch.float16: FP16, torch.bfloat16: BF16}
    if t.dtype not in m:
        raise TypeError("unsupported dtype %s (fp32, fp16, bf16 only)" % t.dtype)
    return m[t.dtype]


class Communicator:
    """N emulated ranks on the current CUDA/HIP device (torch tensors in/out)."""

    def __init__(self, n_ranks: int, dtype, max_bytes: int):
        import torch
        code = {torch.float32: FP32, torch.float16: FP16, torch.bfloat16: BF16}.get(dtype, dtype)
        if not torch.cuda.is_available():
            raise LlarError(-4, "no GPU: the llar protocols run only on the HIP device")
        self.n_ranks, self.dtype, self.max_bytes = int(n_ranks), int(code), int(max_bytes)
        self.h = llar_create(self.n_ranks, self.dtype, self.max_bytes)

    def allreduce(self, partials, out, protocol=AUTO, stream=None):
        import torch
        if isinstance(protocol, str):
            protocol = PROTOCOLS[protocol]
        self._validate(partials, out)
        n = out.numel()
        s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
        st = llar_allreduce(self.h, [p.data_ptr() for p in partials], out.data_ptr(), n, self.dtype, protocol, s)
        return _check(st, "llar_allreduce")

    def send_recv(self, send, recv, protocol=AUTO, stream=None):
        """Copy ``send`` into ``recv`` (``recv.numel()`` elements) from one
        sending rank to one receiving rank over the LL or Sentinel wire."""
        import torch
        if isinstance(protocol, str):
            protocol = PROTOCOLS[protocol]
        n = recv.numel()
        for t, what in ((send, "send"), (recv, "recv")):
            if not (t.is_cuda and t.is_contiguous() and _dtype_code(t) == self.dtype):
                raise ValueError("%s must be a contiguous device tensor of the communicator's dtype" % what)
        if send.numel() < n:
            raise ValueError("send holds fewer elements than recv")
        s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
        st = llar_send_recv(self.h, send.data_ptr(), recv.data_ptr(), n, self.dtype, protocol, s)
        return _check(st, "llar_send_recv")

    def reduce_scatter(self, partials, outs, protocol=AUTO, stream=None):
        """outs[j] (``outs[j].numel()`` elements, the same for every j) gets
        segment j of the sum of ``partials``."""
        import torch
        if isinstance(protocol, str):
            protocol = PROTOCOLS[protocol]
        if len(partials) != self.n_ranks or len(outs) != self.n_ranks:
            raise ValueError("expected %d partials and %d outputs" % (self.n_ranks, self.n_ranks))
        count = outs[0].numel()
        self._check_tensors(partials, self.n_ranks * count, "partials")
        self._check_tensors(outs, count, "outs")
        s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
        st = llar_reduce_scatter(self.h, [p.data_ptr() for p in partials], [o.data_ptr() for o in outs], count,
                                 self.dtype, protocol, s)
        return _check(st, "llar_reduce_scatter")

    def all_gather(self, inputs, outs, protocol=AUTO, stream=None):
        """Every tensor of ``outs`` (N of them, or one: rank 0's copy) gets
        the N fragments ``inputs`` (``inputs[0].numel()`` elements each)
        back to back."""
        import torch
        if isinstance(protocol, str):
            protocol = PROTOCOLS[protocol]
        if len(inputs) != self.n_ranks or len(outs) not in (1, self.n_ranks):
            raise ValueError("expected %d inputs and 1 or %d outputs" % (self.n_ranks, self.n_ranks))
        count = inputs[0].numel()
        self._check_tensors(inputs, count, "inputs")
        self._check_tensors(outs, self.n_ranks * count, "outs")
        s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
        st = llar_all_gather(self.h, [p.data_ptr() for p in inputs], [o.data_ptr() for o in outs], count,
                             self.dtype, protocol, s)
        return _check(st, "llar_all_gather")

    def _check_tensors(self, ts, min_numel, what):
        for t in ts:
            if not (t.is_cuda and t.is_contiguous() and t.numel() >= min_numel and _dtype_code(t) == self.dtype):
                raise ValueError("%s must be contiguous device tensors of the communicator's dtype with at least "
                                 "%d elements" % (what, min_numel))

    def prepare(self, partials, out, protocol=AUTO, stream=None):
        """Validate and marshal the arguments once; return a no-argument
        callable that issues exactly this llar_allreduce call (for tight
        loops where per-call Python checks would dominate)."""
        import torch
        if isinstance(protocol, str):
            protocol = PROTOCOLS[protocol]
        self._validate(partials, out)
        s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
        fn = lib().llar_allreduce
        arr = (ctypes.c_void_p * len(partials))(*[p.data_ptr() for p in partials])
        args = (ctypes.c_void_p(self.h), arr, ctypes.c_void_p(out.data_ptr()), ctypes.c_size_t(out.numel()),
                ctypes.c_int(self.dtype), ctypes.c_int(protocol), ctypes.c_void_p(s))
        keep = (partials, out)  # the tensors stay alive as long as the callable

        def call():
            st = fn(*args)
            if st < 0:
                raise LlarError(st, "llar_allreduce")
            return keep is not None

        return call

    def _validate(self, partials, out):
        if len(partials) != self.n_ranks:
            raise ValueError("expected %d partials" % self.n_ranks)
        n = out.numel()
        for p in partials:
            if not (p.is_cuda and p.is_contiguous() and p.numel() >= n and _dtype_code(p) == self.dtype):
                raise ValueError("partials must be contiguous device tensors of the communicator's dtype")
        if not (out.is_cuda and out.is_contiguous() and _dtype_code(out) == self.dtype):
            raise ValueError("out must be a contiguous device tensor of the communicator's dtype")

    def set_option(self, key: str, value: int):
        return _check(llar_set_option(self.h, key, value), "llar_set_option(%s)" % key)

    def get_option(self, key: str) -> int:
        return llar_get_option(self.h, key)

    def device_status(self):
        return llar_get_device_status(self.h)

    def clear_device_status(self):
        return _check(llar_clear_device_status(self.h), "llar_clear_device_status")

    def select_protocol(self, nbytes: int) -> int:
        return llar_select_protocol(self.h, nbytes)

    def staging(self, protocol: int, nbytes: int = None):
        if nbytes is None:
            nbytes = llar_staging_bytes(self.h, protocol)
        return llar_debug_copy_staging(self.h, protocol, nbytes)

    def staging_bytes(self, protocol: int) -> int:
        return llar_staging_bytes(self.h, protocol)

    def epoch(self) -> int:
        return llar_get_epoch(self.h)

    def timing(self, count: int):
        return llar_get_timing(self.h, count)

    def geometry(self, n_elems: int, protocol: int = AUTO):
        return llar_launch_geometry(self.h, n_elems, protocol)

    def close(self):
        if getattr(self, "h", None):
            llar_destroy(self.h)
            self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
