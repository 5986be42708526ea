"""Seeded synthetic inputs for the N-way AllReduce: the workload table and the
generators shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the reduction or its protocols: it only
draws random partial outputs of the stated shapes and distributions and hands
out their bit patterns.  Both the CPU oracle and the GPU library consume what
it returns; neither is imported here.

Shapes follow the tensor-parallel decode setting of "Every Microsecond
Matters: Achieving Near Speed-of-Light Latency in GPU Collectives"
(agihunt.info summary): every decode step of every layer reduces the N shard
outputs of width hidden x batch, a few KB to a few hundred KB.  hidden = 8192
is the output width used for the TP cases.  No dataset or trained weights are
involved; the values stand in for partial outputs of a layer (N(0,1) * 0.02)
or for generic data (U[-1, 1], N(0,1)).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")
ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}
BITS_NP = {"fp32": np.uint32, "fp16": np.uint16, "bf16": np.uint16}
CODE = {"fp32": 0, "fp16": 1, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    n_ranks: int
    dtype: str
    n_elems: int               # elements per rank (for the sweep: the default size)
    dist: str                  # "uniform" (U[-1,1]*scale) or "normal" (N(0,1)*scale)
    scale: float
    protocol: str              # "ll", "sentinel", "ll128", "ll128_pipelined", "auto"
    reps: int
    chunk_bytes: int = 0       # pipelined protocol: bytes per rank per chunk
    sweep_bytes: Optional[List[int]] = field(default=None, hash=False)

    @property
    def bytes_per_rank(self) -> int:
        return self.n_elems * ELEM_BYTES[self.dtype]


WORKLOADS = {
    1: Workload(1, "ll_n2_fp32_128B", 2, "fp32", 32, "uniform", 1.0, "ll", 1000),
    2: Workload(2, "ll128_n4_bf16_16KiB", 4, "bf16", 8192, "normal", 0.02, "ll128", 1000),
    3: Workload(3, "sentinel_n8_fp16_128KiB", 8, "fp16", 65536, "normal", 0.02, "sentinel", 1000),
    4: Workload(4, "ll128pipe_n8_fp32_4MiB", 8, "fp32", 1 << 20, "uniform", 1.0, "ll128_pipelined", 200,
                chunk_bytes=65536),
    5: Workload(5, "sweep_n8_bf16", 8, "bf16", 8192, "normal", 1.0, "auto", 1000,
                sweep_bytes=[1 << k for k in range(7, 27)]),
}


def draw_values(cfg_id: int, rep: int, n_ranks: int, n_elems: int, dist: str, scale: float) -> np.ndarray:
    """(n_ranks, n_elems) binary64 draws from numpy's PCG64 seeded by [cfg_id, rep]."""
    rng = np.random.default_rng([int(cfg_id), int(rep)])
    shape = (n_ranks, n_elems)
    if dist == "uniform":
        v = rng.random(shape) * 2.0 - 1.0
    elif dist == "normal":
        v = rng.standard_normal(shape)
    elif dist == "integer":
        # small integers: every partial sum is exact in all three formats
        v = rng.integers(-64, 65, size=shape).astype(np.float64)
    else:
        raise ValueError(dist)
    if scale != 1.0:
        v *= scale
    return v


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of finite binary64 values, rounded once to
    nearest, ties to even (numpy has no bfloat16).  The values must be zero or
    within bfloat16's normal range, which every draw above is."""
    b = np.ascontiguousarray(v, dtype=np.float64).view(np.uint64)
    sign = (b >> np.uint64(63)).astype(np.uint16) << np.uint16(15)
    mag = b & np.uint64(0x7FFFFFFFFFFFFFFF)
    # keep the exponent and the top 7 of the 52 fraction bits: add just under
    # half of the dropped 45 bits, plus the lowest kept bit (ties to even); a
    # carry out of the fraction moves into the exponent, as it must
    lsb = (mag >> np.uint64(45)) & np.uint64(1)
    r = (mag + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)
    exp = (r >> np.uint64(7)).astype(np.int64)
    zero = mag == 0
    e16 = exp - 1023 + 127
    if np.any(~zero & ((e16 < 1) | (e16 > 254))):
        raise ValueError("a value outside bfloat16's normal range")
    out = ((np.where(zero, 0, e16).astype(np.uint16) << np.uint16(7))
           | (r & np.uint64(0x7F)).astype(np.uint16))
    return out | sign


def to_bits(values: np.ndarray, dtype: str) -> np.ndarray:
    """Element bit patterns of the binary64 draws in the I/O type, each rounded
    once to nearest, ties to even (numpy's float32 and float16 conversions of
    a double round that way; bfloat16 is rounded from the binary64 bits)."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=BITS_NP[dtype])
    for r in range(v.shape[0]):  # row by row: bounded temporaries for 64 MiB ranks
        if dtype == "fp32":
            out[r] = v[r].astype(np.float32).view(np.uint32)
        elif dtype == "fp16":
            out[r] = v[r].astype(np.float16).view(np.uint16)
        elif dtype == "bf16":
            out[r] = _bf16_bits(v[r])
        else:
            raise ValueError(dtype)
    return out


def make_partials(cfg_id: int, rep: int, n_ranks: int, dtype: str, n_elems: int,
                  dist: str = "normal", scale: float = 1.0) -> np.ndarray:
    """(n_ranks, n_elems) array of element bits, seeded by [cfg_id, rep]."""
    return to_bits(draw_values(cfg_id, rep, n_ranks, n_elems, dist, scale), dtype)


def workload_partials(w: Workload, rep: int, n_elems: Optional[int] = None) -> np.ndarray:
    n = w.n_elems if n_elems is None else n_elems
    return make_partials(w.cfg_id, rep, w.n_ranks, w.dtype, n, w.dist, w.scale)


def random_bits(cfg_id: int, rep: int, n_elems: int, dtype: str) -> np.ndarray:
    """n_elems element bit patterns drawn uniformly over every pattern of the
    I/O type (NaNs, infinities, subnormals and the all-ones pattern
    included), seeded by [cfg_id, rep]: the payload of a pure data move."""
    rng = np.random.default_rng([int(cfg_id), int(rep)])
    width = 32 if dtype == "fp32" else 16
    b = rng.integers(0, 1 << width, size=n_elems, dtype=np.uint64)
    return b.astype(np.uint32 if width == 32 else np.uint16)
