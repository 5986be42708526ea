"""One-shot LL consumer lane granularity on the GPU, against the CPU oracle.

A consumer workgroup of the one-shot LL AllReduce gives each lane one 4-byte
half line {data, epoch} when every half of its units has a lane of its own,
and one 8-byte unit (a whole line) per lane otherwise, looping when the units
outnumber the lanes.  With two ranks the half-line consumer keeps two poll
passes in flight.  These tests pin the switch: one 256-thread slice, so the
switch sits at a known message size, and sizes on both sides of it and ragged
ones at it, bit-exact against oracle.allreduce (or the transfer model for
send/recv, the copy form of the same kernel).  Fresh inputs every repetition,
so a lane reading the previous call's line would fail.
"""
import numpy as np
import pytest
import torch

import message_allreduce_amd as llar
import oracle
from oracle import models
from workloads import make_partials, random_bits

from gpu_util import CODE, TORCH_DT, assert_exact, run, to_device, to_host

pytestmark = pytest.mark.gpu

ESIZE = {"fp32": 4, "fp16": 2, "bf16": 2}


def comm_for(n_ranks, dt, max_bytes, **opts):
    c = llar.Communicator(n_ranks, TORCH_DT[dt], max_bytes)
    c.set_option("spin_timeout_us", 100_000)
    for k, v in opts.items():
        c.set_option(k, v)
    return c


def switch_bytes(split):
    """Largest message (bytes per rank) whose consumer workgroups still give
    every half line a lane: one slice of 256 threads holds ceil(S/16) vectors,
    2 units each, split over `split` consumer workgroups, and a workgroup takes
    half lines while 2 x its units <= 256."""
    return 2048 if split == 2 else 1024


def sizes_around(split, esize):
    b = switch_bytes(split)
    return sorted({b - 16, b - esize, b, b + esize, b + 16, b + 18 if esize == 2 else b + 20, 2 * b + esize})


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("n_ranks,split", [(8, 2), (8, 1), (4, 2), (2, 1)])
def test_ll_consumer_switch_bit_exact(n_ranks, split, dtype):
    dt = CODE[dtype]
    esize = ESIZE[dtype]
    with comm_for(n_ranks, dt, 64 << 10, threads=256, slices=1, consumer_split=split) as c:
        for nbytes in sizes_around(split, esize):
            n = nbytes // esize
            geo = c.geometry(n, llar.LL)
            assert geo["threads"] == 256 and geo["slices"] == 1, geo
            for rep in range(3):
                bits = make_partials(70 + n_ranks, rep * 1000 + nbytes, n_ranks, dtype, n, "normal", 1.0)
                got = run(c, bits, "ll", dt)
                assert_exact(got, oracle.allreduce(bits, dt), dt,
                             "N=%d split=%d %s %d B rep %d" % (n_ranks, split, dtype, nbytes, rep))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ll_send_recv_switch_bit_exact(dtype):
    """send/recv is the copy form of the kernel at two ranks (split 1): every
    bit pattern arrives unchanged on either side of the switch."""
    dt = CODE[dtype]
    esize = ESIZE[dtype]
    with comm_for(2, dt, 64 << 10, threads=256, slices=1) as c:
        for nbytes in sizes_around(1, esize):
            n = nbytes // esize
            for rep in range(3):
                bits = random_bits(80, rep * 1000 + nbytes, n, dtype)
                send = to_device(bits, dt)
                recv = torch.empty(n, dtype=TORCH_DT[dt], device="cuda")
                c.send_recv(send, recv, "ll")
                torch.cuda.synchronize()
                st, sbits = c.device_status()
                assert st == 0, "device status %d bits %#x" % (st, sbits)
                assert_exact(to_host(recv, dt), models.p2p_transfer(bits, dt, "ll"), dt,
                             "send/recv %s %d B rep %d" % (dtype, nbytes, rep))


@pytest.mark.parametrize("copy", [False, True], ids=["allreduce", "send_recv"])
def test_two_rank_two_pass_poll_times_out_and_recovers(copy):
    """Two ranks: the half-line consumer keeps two poll passes in flight.  With
    the sending rank silenced from the host its bounded wait still expires
    (status TIMEOUT, the kernel ends), and after a reset the same call is
    exact again."""
    dt = CODE["fp32"]
    n = 32
    bits = make_partials(910, 0, 2, "fp32", n, "uniform", 1.0)
    with comm_for(2, dt, 64 << 10) as c:
        c.set_option("spin_timeout_us", 2000)
        c.set_option("debug_drop_rank", 1)
        out = torch.empty(n, dtype=TORCH_DT[dt], device="cuda")
        parts = [to_device(bits[r], dt) for r in range(2)]
        if copy:
            c.send_recv(parts[1], out, "ll")
        else:
            c.allreduce(parts, out, "ll")
        torch.cuda.synchronize()
        st, status_bits = c.device_status()
        assert st == -5 and (status_bits & 1), (st, status_bits)
        c.clear_device_status()
        c.set_option("debug_drop_rank", -1)
        c.set_option("spin_timeout_us", 100_000)
        if copy:
            c.send_recv(parts[1], out, "ll")
            torch.cuda.synchronize()
            st, status_bits = c.device_status()
            assert st == 0, (st, status_bits)
            assert_exact(to_host(out, dt), models.p2p_transfer(bits[1], dt, "ll"), dt, "send/recv after recovery")
        else:
            got = run(c, bits, "ll", dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "allreduce after recovery")
