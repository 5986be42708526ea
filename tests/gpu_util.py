"""Helpers of the GPU parity tests: move element bit patterns between numpy
and device tensors, run one AllReduce through the C ABI, compare with the
oracle (bit-exact, or within the tolerance of the atomic protocol)."""
from __future__ import annotations

import numpy as np
import torch

import message_allreduce_amd as llar
import oracle

TORCH_DT = {oracle.F32: torch.float32, oracle.F16: torch.float16, oracle.BF16: torch.bfloat16}
INT_DT = {oracle.F32: torch.int32, oracle.F16: torch.int16, oracle.BF16: torch.int16}
NP_INT = {oracle.F32: np.int32, oracle.F16: np.int16, oracle.BF16: np.int16}
CODE = {"fp32": oracle.F32, "fp16": oracle.F16, "bf16": oracle.BF16}
# relative tolerance of the non-deterministic atomic protocol, with an
# absolute floor of 1e-3: |got - oracle| <= 1e-3 + rtol * |oracle|
RTOL = {oracle.F32: 1e-5, oracle.F16: 2e-3, oracle.BF16: 1.6e-2}
ATOL = 1e-3


def to_device(bits: np.ndarray, dt: int, dev="cuda") -> torch.Tensor:
    b = np.ascontiguousarray(bits).view(NP_INT[dt])
    return torch.from_numpy(b.copy()).to(dev).view(TORCH_DT[dt])


def to_host(t: torch.Tensor, dt: int) -> np.ndarray:
    return t.view(INT_DT[dt]).cpu().numpy().view(oracle.BITS_DTYPE[dt])


def run(comm: llar.Communicator, parts_bits: np.ndarray, protocol, dt: int, out: torch.Tensor = None,
        parts_dev=None) -> np.ndarray:
    n = parts_bits.shape[1]
    if parts_dev is None:
        parts_dev = [to_device(parts_bits[r], dt) for r in range(parts_bits.shape[0])]
    if out is None:
        out = torch.empty(n, dtype=TORCH_DT[dt], device="cuda")
    comm.allreduce(parts_dev, out, protocol)
    torch.cuda.synchronize()
    st, bits = comm.device_status()
    assert st == 0, "device status %d bits %#x" % (st, bits)
    return to_host(out, dt)


def assert_exact(got: np.ndarray, want: np.ndarray, dt: int, what: str = ""):
    ok = oracle.same_result(got, want, dt)
    if not ok.all():
        idx = np.nonzero(~ok)[0]
        i = idx[0]
        raise AssertionError("%s: %d of %d differ; first at %d: got %#x want %#x"
                             % (what, idx.size, ok.size, i, int(got[i]), int(want[i])))


def assert_tol(got: np.ndarray, want: np.ndarray, dt: int, what: str = ""):
    g = oracle.decode(got, dt)
    o = oracle.decode(want, dt)
    both_nan = np.isnan(g) & np.isnan(o)
    with np.errstate(invalid="ignore"):
        ok = both_nan | (g == o) | (np.abs(g - o) <= ATOL + RTOL[dt] * np.abs(o))
    if not ok.all():
        idx = np.nonzero(~ok)[0]
        i = idx[0]
        raise AssertionError("%s: %d of %d outside tolerance; first at %d: got %r want %r"
                             % (what, idx.size, ok.size, i, g[i], o[i]))
