"""Point-to-point LL / Sentinel send/recv on the GPU against the oracle's
transfer model, through the C ABI.

The receiver's output must equal models.p2p_transfer bit for bit: LL moves
every pattern unchanged; the Sentinel wire moves every pattern but its own
all-ones one, which arrives as the pattern one below.  Payloads are drawn
over every bit pattern of the type.  Sizes cover one element, ragged tails,
the 8 KB hidden state of a 4096-wide fp16 model and several slices.
"""
import numpy as np
import pytest
import torch

import message_allreduce_amd as llar
import oracle
from oracle import F32, F16, BF16, models
from workloads import make_partials, random_bits

from gpu_util import CODE, TORCH_DT, assert_exact, run, to_device, to_host

pytestmark = pytest.mark.gpu

WIRES = ["ll", "sentinel"]
DTYPE_NAME = {F32: "fp32", F16: "fp16", BF16: "bf16"}


def comm_for(n_ranks, dt, max_bytes, **opts):
    c = llar.Communicator(n_ranks, TORCH_DT[dt], max_bytes)
    c.set_option("spin_timeout_us", 100_000)
    for k, v in opts.items():
        c.set_option(k, v)
    return c


def send_recv(c, bits, dt, wire, recv=None):
    send = to_device(bits, dt)
    if recv is None:
        recv = torch.empty(bits.size, dtype=TORCH_DT[dt], device="cuda")
    c.send_recv(send, recv, wire)
    torch.cuda.synchronize()
    st, sbits = c.device_status()
    assert st == 0, "device status %d bits %#x" % (st, sbits)
    return to_host(recv, dt)


def assert_bits_equal(got, want, what):
    if not np.array_equal(got, want):
        i = int(np.nonzero(got != want)[0][0])
        raise AssertionError("%s: %d of %d differ; first at %d: got %#x want %#x"
                             % (what, int((got != want).sum()), got.size, i, int(got[i]), int(want[i])))


@pytest.mark.parametrize("placement", [1, 2], ids=["spread", "local"])
@pytest.mark.parametrize("wire", WIRES)
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_send_recv_bit_exact_ragged_sizes(dtype, wire, placement):
    dt = CODE[dtype]
    sizes = [1, 3, 7, 129, 4096, 12345, 262149]
    with comm_for(4, dt, max(sizes) * 4, placement=placement) as c:
        for i, n in enumerate(sizes):
            bits = random_bits(2000 + dt, i, n, dtype)
            bits[:: 97] = models.SENTINEL_BITS[dt]
            got = send_recv(c, bits, dt, wire)
            assert_bits_equal(got, models.p2p_transfer(bits, dt, wire), "%s %s n=%d" % (dtype, wire, n))
        if wire == "sentinel":
            stage = c.staging(llar.SENTINEL).view(np.uint8)
            assert (stage == 0xFF).all(), "sentinel staging must be reset after use"


@pytest.mark.parametrize("wire", WIRES)
def test_send_recv_pipeline_hidden_state_8KB_fp16_1000_reps(wire):
    """4096 x fp16 = 8 KB per token from one pipeline stage to the next,
    fresh activations every call."""
    dt = F16
    n = 4096
    with comm_for(2, dt, n * 2) as c:
        send = torch.empty(n, dtype=torch.float16, device="cuda")
        recv = torch.empty(n, dtype=torch.float16, device="cuda")
        for rep in range(1000):
            bits = make_partials(2100, rep, 1, "fp16", n, "normal", 1.0)[0]
            send.copy_(to_device(bits, dt))
            c.send_recv(send, recv, wire)
            if rep % 100 == 99 or rep < 3:
                torch.cuda.synchronize()
                got = to_host(recv, dt)
                assert_bits_equal(got, models.p2p_transfer(bits, dt, wire), "rep %d" % rep)
        torch.cuda.synchronize()
        st, sbits = c.device_status()
        assert st == 0, (st, sbits)


@pytest.mark.parametrize("n_ranks", [1, 2, 8])
def test_send_recv_on_any_communicator(n_ranks):
    """The transfer uses one sending and one receiving rank whatever the
    communicator's rank count."""
    dt = BF16
    n = 5003
    with comm_for(n_ranks, dt, n * 2) as c:
        for k, wire in enumerate(WIRES):
            bits = random_bits(2200 + n_ranks, k, n, "bf16")
            got = send_recv(c, bits, dt, wire)
            assert_bits_equal(got, models.p2p_transfer(bits, dt, wire), "N=%d %s" % (n_ranks, wire))


def test_send_recv_interleaved_with_allreduce():
    """send/recv and AllReduce share the staging and the epoch sequence."""
    dt = BF16
    n, n_ranks = 3001, 8
    with comm_for(n_ranks, dt, n * 2) as c:
        for rep in range(40):
            wire = WIRES[rep % 2]
            bits = make_partials(2300, rep, n_ranks, "bf16", n, "normal", 1.0)
            got = run(c, bits, wire, dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "allreduce rep %d" % rep)
            got = send_recv(c, bits[rep % n_ranks], dt, wire)
            assert_bits_equal(got, models.p2p_transfer(bits[rep % n_ranks], dt, wire), "p2p rep %d" % rep)
        assert (c.staging(llar.SENTINEL).view(np.uint8) == 0xFF).all()


def test_send_recv_graph_capture_replays():
    """Captured send/recv calls read the device-resident epoch: every replay
    is a new transfer, and eager calls between replays still work."""
    dt = F16
    n = 4096
    c = comm_for(2, dt, n * 2)
    try:
        send = torch.empty(n, dtype=torch.float16, device="cuda")
        recvs = {w: torch.empty(n, dtype=torch.float16, device="cuda") for w in WIRES}
        send.copy_(to_device(make_partials(2400, 0, 1, "fp16", n)[0], dt))
        for w in WIRES:
            c.send_recv(send, recvs[w], w)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for w in WIRES:
                c.send_recv(send, recvs[w], w)
        torch.cuda.synchronize()
        for rep in range(1, 6):
            bits = make_partials(2400, rep, 1, "fp16", n)[0]
            send.copy_(to_device(bits, dt))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            st, sbits = c.device_status()
            assert st == 0, (st, sbits)
            for w in WIRES:
                assert_bits_equal(to_host(recvs[w], dt), models.p2p_transfer(bits, dt, w), "replay %d %s" % (rep, w))
            got = send_recv(c, bits, dt, "ll")
            assert_bits_equal(got, bits, "eager after replay %d" % rep)
    finally:
        c.close()


@pytest.mark.parametrize("wire", WIRES)
def test_send_recv_lost_sender_times_out_and_recovers(wire):
    """A sender that writes nothing (forced from the host) makes the
    receiver's bounded polls expire; after a reset the next transfer works."""
    dt = BF16
    n = 4096
    bits = random_bits(2500, 0, n, "bf16")
    with comm_for(2, dt, n * 2) as c:
        c.set_option("spin_timeout_us", 2000)
        c.set_option("debug_drop_rank", 1)
        recv = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        c.send_recv(to_device(bits, dt), recv, wire)
        torch.cuda.synchronize()
        st, sbits = c.device_status()
        assert st == -5 and (sbits & 1), (st, sbits)
        c.clear_device_status()
        c.set_option("debug_drop_rank", -1)
        c.set_option("spin_timeout_us", 100_000)
        got = send_recv(c, bits, dt, wire)
        assert_bits_equal(got, models.p2p_transfer(bits, dt, wire), "after recovery")


def test_send_recv_argument_errors():
    dt = BF16
    n = 1024
    with comm_for(2, dt, n * 2) as c:
        a = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        b = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        for proto in ("ll128", "ll128_pipelined", "sentinel_pipelined"):
            with pytest.raises(llar.LlarError) as e:
                c.send_recv(a, b, proto)
            assert e.value.status == -1
        with pytest.raises(llar.LlarError) as e:        # beyond max_bytes
            c.send_recv(torch.zeros(2 * n, dtype=torch.bfloat16, device="cuda"),
                        torch.zeros(2 * n, dtype=torch.bfloat16, device="cuda"), "ll")
        assert e.value.status == -1
        assert llar.llar_send_recv(c.h, a.data_ptr() + 2, b.data_ptr(), 8, BF16, llar.LL, 0) == -1  # misaligned
        assert llar.llar_send_recv(c.h, a.data_ptr(), b.data_ptr(), 8, F32, llar.LL, 0) == -1      # wrong dtype
        assert llar.llar_send_recv(c.h, a.data_ptr(), b.data_ptr(), 0, BF16, llar.LL, 0) == 0      # no-op
        with pytest.raises(ValueError):
            c.send_recv(a[: n // 2], b, "ll")
    big = 9 << 20                                       # LL caps at 8 MiB per message
    with comm_for(2, F32, big) as c:
        a = torch.zeros(big // 4, dtype=torch.float32, device="cuda")
        b = torch.zeros(big // 4, dtype=torch.float32, device="cuda")
        with pytest.raises(llar.LlarError) as e:
            c.send_recv(a, b, "ll")
        assert e.value.status == -2
        c.send_recv(a, b, "auto")                        # AUTO picks the Sentinel wire
        torch.cuda.synchronize()
        assert c.device_status()[0] == 0


def test_send_recv_maximum_sizes():
    """The byte limits of both wires: 8 MiB over LL, 16 MiB over the Sentinel."""
    dt = F32
    for wire, nbytes in (("ll", 8 << 20), ("sentinel", 16 << 20)):
        n = nbytes // 4
        with comm_for(2, dt, nbytes) as c:
            bits = random_bits(2600, nbytes, n, "fp32")
            got = send_recv(c, bits, dt, wire)
            assert_bits_equal(got, models.p2p_transfer(bits, dt, wire), "%s %d bytes" % (wire, nbytes))
