"""The device-side primitive API (include/llar_wire.h), exercised by custom
kernels written only against it (tests/device_api/wire_demo.hip), checked
against the oracle.

* LL: a scaling epilogue fused with an AllReduce -- every rank's partial is
  scaled (binary32 product), put on the LL wire and summed by rank 0 in
  binary64, rank order, one rounding: bit-exact against the oracle's sum of
  the rounded products.  The staging is reused across calls with new epochs,
  so stale lines must be rejected.
* Sentinel: a relay, each rank adding its value to the running binary32 sum
  it waits for: bit-exact against sequential binary32 additions; the staging
  is all-ones again afterwards.
* LL128: atomic adds into lines with a contribution count: within the
  tolerance of the atomic protocol; the lines are zero again afterwards.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import F32

from gpu_util import assert_exact, assert_tol, to_host

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "device_api", "libwire_demo.so")
SPIN = 10_000_000  # 0.1 s of the 100 MHz wall clock
SIZES = [1, 2, 3, 31, 32, 1000, 65537]


@pytest.fixture(scope="module")
def demo():
    if not os.path.exists(LIB):
        raise RuntimeError("libwire_demo.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    vp, u32, u64, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
    L.demo_scaled_allreduce_ll.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_float), vp, u32, i32, vp,
                                           u32, u32, u64, vp, vp]
    L.demo_sentinel_chain.argtypes = [ctypes.POINTER(vp), vp, u32, i32, vp, u32, u64, vp, vp]
    L.demo_ll128_reduce.argtypes = [ctypes.POINTER(vp), vp, u32, i32, vp, u32, u64, vp, vp, i32]
    for f in (L.demo_scaled_allreduce_ll, L.demo_sentinel_chain, L.demo_ll128_reduce):
        f.restype = i32
    return L


def partials(seed, n_ranks, n):
    g = np.random.default_rng([seed, n_ranks, n])
    return g.standard_normal((n_ranks, n), dtype=np.float32)


def ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("n_ranks", [2, 4, 8])
def test_ll_scaled_allreduce_epilogue(demo, n_ranks):
    n_max = max(SIZES)
    units = (n_max + 1) // 2
    stage = torch.zeros((n_ranks - 1) * units * 16, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    epoch = 0
    for i, n in enumerate(SIZES):
        for rep in range(2):
            p = partials(100 + i, n_ranks, n) * np.float32(1 + rep)
            scales = np.random.default_rng([7, i, rep]).uniform(0.5, 2.0, n_ranks).astype(np.float32)
            dev = [torch.from_numpy(p[r].copy()).cuda() for r in range(n_ranks)]
            out = torch.empty(n, dtype=torch.float32, device="cuda")
            epoch += 1
            rc = demo.demo_scaled_allreduce_ll(ptrs(dev), (ctypes.c_float * n_ranks)(*scales), out.data_ptr(), n,
                                               n_ranks, stage.data_ptr(), stage.numel(), epoch, SPIN,
                                               status.data_ptr(), stream())
            assert rc == 0
            torch.cuda.synchronize()
            assert int(status.item()) == 0, "a wait expired"
            prod = (p * scales[:, None]).astype(np.float32)      # IEEE binary32 products
            want = oracle.allreduce(prod.view(np.uint32), F32)
            assert_exact(to_host(out, F32), want, F32, "N=%d n=%d rep %d" % (n_ranks, n, rep))


@pytest.mark.parametrize("n_ranks", [2, 3, 8])
def test_sentinel_relay(demo, n_ranks):
    n_max = max(SIZES)
    vecs = (n_max + 3) // 4
    stage = torch.full(((n_ranks - 1) * vecs * 16,), 0xFF, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i, n in enumerate(SIZES):
        p = partials(200 + i, n_ranks, n)
        dev = [torch.from_numpy(p[r].copy()).cuda() for r in range(n_ranks)]
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        rc = demo.demo_sentinel_chain(ptrs(dev), out.data_ptr(), n, n_ranks, stage.data_ptr(), stage.numel(), SPIN,
                                      status.data_ptr(), stream())
        assert rc == 0
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a wait expired"
        want = p[0].copy()
        for r in range(1, n_ranks):
            want = (want + p[r]).astype(np.float32)               # binary32 additions in rank order
        assert_exact(to_host(out, F32), want.view(np.uint32), F32, "N=%d n=%d" % (n_ranks, n))
        assert (stage.cpu().numpy() == 0xFF).all(), "every slot is reset by its reader"


@pytest.mark.parametrize("take", [0, 1], ids=["read_reset", "take"])
@pytest.mark.parametrize("n_ranks", [2, 4, 8])
def test_ll128_atomic_reduce(demo, n_ranks, take):
    n_max = max(SIZES)
    lines = (n_max + 30) // 31
    stage = torch.zeros(lines * 128, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i, n in enumerate(SIZES):
        p = partials(300 + i, n_ranks, n)
        dev = [torch.from_numpy(p[r].copy()).cuda() for r in range(n_ranks)]
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        rc = demo.demo_ll128_reduce(ptrs(dev), out.data_ptr(), n, n_ranks, stage.data_ptr(), stage.numel(), SPIN,
                                    status.data_ptr(), stream(), take)
        assert rc == 0
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a wait expired"
        assert_tol(to_host(out, F32), oracle.allreduce(p.view(np.uint32), F32), F32, "N=%d n=%d" % (n_ranks, n))
        assert not stage.cpu().numpy().any(), "every line is zeroed by its owner"
