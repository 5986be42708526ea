"""GPU tests of the epoch wrap, through the C ABI.

The LL flag is the only arrival signal ("Every Microsecond Matters",
agihunt.info summary, LL paragraph): a consumer accepts a line as soon as it
carries the call's epoch.  Epochs run 1 .. 2^31-1 (host-numbered calls) and
2^31 + (1 .. 2^31-1) (device-numbered calls) and then come round again, so
an LL line -- or an owner-credit progress word, tagged with its call's epoch
-- that no call has written for a whole cycle would pass for a fresh one.
The library clears that state at every wrap.  The tests place the epoch just
before the wrap (options "debug_host_epoch" / "debug_device_epoch", which
leave staging as earlier calls wrote it, as a real cycle would) and:

* cross it with a large message, smaller ones, then the large one again,
  bit-exact against oracle.allreduce (LL, the owner credit, graph replays);
* show that the clear happened: after the wrap, a call whose rank 3 writes
  nothing (forced from the host) must end in the bounded time-out.  Without
  the clear that rank's lines would still carry the same epoch from the
  call made one cycle earlier, and the consumer would finish from them.
"""
import pytest
import torch

import message_allreduce_amd as llar
import oracle
from oracle import BF16
from workloads import make_partials

from gpu_util import assert_exact, assert_tol, run, to_device, to_host

pytestmark = pytest.mark.gpu

HOST_LAST = 0x7FFFFFFF
DEVICE_LAST = 0xFFFFFFFF
N_RANKS = 8
N_BIG = 32768   # 64 KiB of bf16 per rank
N_SMALL = 1000


def comm(**opts):
    c = llar.Communicator(N_RANKS, torch.bfloat16, N_BIG * 2)
    c.set_option("spin_timeout_us", 100_000)
    for k, v in opts.items():
        c.set_option(k, v)
    return c


def exact_call(c, seed, rep, n, proto="ll"):
    bits = make_partials(seed, rep, N_RANKS, "bf16", n, "normal", 1.0)
    got = run(c, bits, proto, BF16)
    assert_exact(got, oracle.allreduce(bits, BF16), BF16, "seed %d rep %d n %d %s" % (seed, rep, n, proto))


def expect_timeout_with_rank_dropped(c, seed, n):
    bits = make_partials(seed, 0, N_RANKS, "bf16", n, "normal", 1.0)
    parts = [to_device(bits[r], BF16) for r in range(N_RANKS)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    c.set_option("spin_timeout_us", 2000)
    c.set_option("debug_drop_rank", 3)
    c.allreduce(parts, out, "ll")
    torch.cuda.synchronize()
    st, sbits = c.device_status()
    assert st == -5 and (sbits & 1), "a stale line passed for a fresh one: status %d bits %#x" % (st, sbits)
    c.clear_device_status()
    c.set_option("debug_drop_rank", -1)
    c.set_option("spin_timeout_us", 100_000)


def test_host_epoch_wrap_large_small_large_bit_exact():
    with comm() as c:
        exact_call(c, 3100, 0, N_BIG)          # epoch 1
        exact_call(c, 3100, 1, N_BIG)          # epoch 2
        c.set_option("debug_host_epoch", HOST_LAST - 3)
        exact_call(c, 3100, 2, N_BIG)          # 3 calls before the wrap: the large message
        exact_call(c, 3100, 3, N_SMALL)
        exact_call(c, 3100, 4, N_SMALL)
        exact_call(c, 3100, 5, N_SMALL)        # the last epoch of the range
        assert c.get_option("debug_host_epoch") == 1
        for rep in range(6, 12):               # across the wrap: 1, 2, ... again
            exact_call(c, 3100, rep, N_BIG if rep % 3 else N_SMALL)
        assert c.get_option("debug_host_epoch") == 7


def test_host_epoch_wrap_clears_lines_of_the_previous_cycle():
    with comm() as c:
        exact_call(c, 3200, 0, N_BIG)          # epoch 1: every line of the odd parity
        c.set_option("debug_host_epoch", HOST_LAST)
        exact_call(c, 3200, 1, N_BIG, "sentinel")  # the last epoch (the LL region is untouched)
        assert c.get_option("debug_host_epoch") == 1
        expect_timeout_with_rank_dropped(c, 3200, N_BIG)
        exact_call(c, 3200, 2, N_BIG)          # recovery


def test_device_epoch_wrap_clears_lines_of_the_previous_cycle():
    with comm(device_epoch=1) as c:
        assert c.get_option("debug_device_epoch") == 0x80000001
        exact_call(c, 3300, 0, N_BIG)          # device epoch 2^31 + 1
        c.set_option("debug_device_epoch", DEVICE_LAST)
        exact_call(c, 3300, 1, N_BIG, "sentinel")  # the wrapping call clears on the device
        assert c.get_option("debug_device_epoch") == 0x80000001
        assert c.device_status()[0] == 0
        expect_timeout_with_rank_dropped(c, 3300, N_BIG)
        exact_call(c, 3300, 2, N_BIG)


@pytest.mark.parametrize("wrap_proto", ["ll", "sentinel", "ll128", "sentinel_pipelined"])
def test_device_epoch_wrap_in_every_kernel_family(wrap_proto):
    """Whichever kernel makes the wrapping call performs the clear; the
    calls around it stay exact (LL128 within its tolerance)."""
    with comm(device_epoch=1, chunk_bytes=8192) as c:
        exact_call(c, 3400, 0, N_BIG)
        c.set_option("debug_device_epoch", DEVICE_LAST - 1)
        exact_call(c, 3400, 1, N_SMALL)
        bits = make_partials(3400, 2, N_RANKS, "bf16", N_BIG, "normal", 1.0)
        got = run(c, bits, wrap_proto, BF16)  # the wrapping call
        want = oracle.allreduce(bits, BF16)
        if wrap_proto == "ll128":
            assert_tol(got, want, BF16, "wrapping call")
        else:
            assert_exact(got, want, BF16, "wrapping call")
        assert c.get_option("debug_device_epoch") == 0x80000001
        for rep in range(3, 7):
            exact_call(c, 3400, rep, N_BIG if rep % 2 else N_SMALL)


def test_owner_credit_words_across_the_host_wrap():
    """The owner credit's progress words carry their call's epoch; one cycle
    later the same epoch must not find the old words' counts."""
    n = N_BIG
    with comm(sentinel_credit=2, chunk_bytes=2048, pipeline_buffers=3) as c:
        exact_call(c, 3500, 0, n, "sentinel_pipelined")      # epoch 1: 64 chunks of progress
        c.set_option("debug_host_epoch", HOST_LAST)
        exact_call(c, 3500, 1, N_SMALL, "ll")
        for rep in range(2, 6):
            exact_call(c, 3500, rep, n, "sentinel_pipelined")  # epochs 1, 2, ... again


def test_owner_credit_words_across_the_device_wrap():
    n = N_BIG
    with comm(sentinel_credit=2, chunk_bytes=2048, pipeline_buffers=3, device_epoch=1) as c:
        exact_call(c, 3600, 0, n, "sentinel_pipelined")
        c.set_option("debug_device_epoch", DEVICE_LAST)
        exact_call(c, 3600, 1, N_SMALL, "ll")
        for rep in range(2, 6):
            exact_call(c, 3600, rep, n, "sentinel_pipelined")


def test_graph_replays_cross_the_device_wrap():
    """A captured graph of a large LL call, a small LL call and an
    owner-credit pipelined call, replayed across the device wrap with fresh
    inputs and eager work between replays; every replay bit-exact."""
    dt = BF16
    c = comm(sentinel_credit=2, chunk_bytes=4096, pipeline_buffers=3)
    try:
        big = [torch.empty(N_BIG, dtype=torch.bfloat16, device="cuda") for _ in range(N_RANKS)]
        small = [torch.empty(N_SMALL, dtype=torch.bfloat16, device="cuda") for _ in range(N_RANKS)]
        outs = [torch.empty(N_BIG, dtype=torch.bfloat16, device="cuda"),
                torch.empty(N_SMALL, dtype=torch.bfloat16, device="cuda"),
                torch.empty(N_BIG, dtype=torch.bfloat16, device="cuda")]

        def calls():
            c.allreduce(big, outs[0], "ll")
            c.allreduce(small, outs[1], "ll")
            c.allreduce(big, outs[2], "sentinel_pipelined")

        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        torch.cuda.synchronize()
        # three calls per replay: the wrap falls inside the second replay
        c.set_option("debug_device_epoch", DEVICE_LAST - 4)
        for rep in range(6):
            bb = make_partials(3700, 2 * rep, N_RANKS, "bf16", N_BIG, "normal", 1.0)
            bs = make_partials(3700, 2 * rep + 1, N_RANKS, "bf16", N_SMALL, "normal", 1.0)
            for r in range(N_RANKS):
                big[r].copy_(to_device(bb[r], dt))
                small[r].copy_(to_device(bs[r], dt))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            st, sbits = c.device_status()
            assert st == 0, (rep, st, sbits)
            want_b = oracle.allreduce(bb, dt)
            assert_exact(to_host(outs[0], dt), want_b, dt, "replay %d large LL" % rep)
            assert_exact(to_host(outs[1], dt), oracle.allreduce(bs, dt), dt, "replay %d small LL" % rep)
            assert_exact(to_host(outs[2], dt), want_b, dt, "replay %d owner credit" % rep)
            exact_call(c, 3701, rep, N_SMALL)   # eager, host-numbered
        assert c.get_option("debug_device_epoch") == 0x80000000 | 14
    finally:
        c.close()


def test_debug_epoch_options_reject_out_of_range_values():
    with comm() as c:
        for key, bad in (("debug_host_epoch", 0), ("debug_host_epoch", 0x80000000),
                         ("debug_device_epoch", 0x80000000), ("debug_device_epoch", 0x7FFFFFFF),
                         ("debug_device_epoch", 1 << 32)):
            assert llar.llar_set_option(c.h, key, bad) == -1
