"""The no-allocation entry point, through the C ABI.

llar_allreduce_noalloc runs the LL one-shot AllReduce over a static device
array instead of a communicator's staging.  Its output must equal
llar_allreduce's with LLAR_LL bit for bit (and the oracle's), on calls in a
row with shrinking inputs -- the array keeps the previous call's lines --
for every element type and several rank counts.
"""
import pytest
import torch

import message_allreduce_amd as llar
import oracle
from oracle import BF16, F16, F32
from workloads import make_partials

from gpu_util import TORCH_DT, assert_exact, to_device, to_host

pytestmark = pytest.mark.gpu

MAX_BYTES = 64 << 10


def noalloc(parts, out, dt, stream=None):
    s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
    return llar.llar_allreduce_noalloc(len(parts), [p.data_ptr() for p in parts], out.data_ptr(), out.numel(), dt, s)


@pytest.mark.parametrize("dt", [F32, F16, BF16])
@pytest.mark.parametrize("n_ranks", [2, 5, 8])
def test_noalloc_equals_the_communicator_call_on_calls_in_a_row(dt, n_ranks):
    elem = 4 if dt == F32 else 2
    sizes = [MAX_BYTES // elem, 3001, 8192 // elem, 17]   # each call smaller than the one before
    with llar.Communicator(n_ranks, TORCH_DT[dt], MAX_BYTES) as c:
        c.set_option("spin_timeout_us", 100_000)
        for i, n in enumerate(sizes):
            bits = make_partials(4100 + dt, i, n_ranks, {F32: "fp32", F16: "fp16", BF16: "bf16"}[dt], n, "normal", 1.0)
            parts = [to_device(bits[r], dt) for r in range(n_ranks)]
            out_c = torch.empty(n, dtype=TORCH_DT[dt], device="cuda")
            out_n = torch.full((n,), 7.0, dtype=TORCH_DT[dt], device="cuda")
            c.allreduce(parts, out_c, "ll")
            assert noalloc(parts, out_n, dt) == 0
            torch.cuda.synchronize()
            assert c.device_status()[0] == 0
            got_c, got_n = to_host(out_c, dt), to_host(out_n, dt)
            assert_exact(got_n, got_c, dt, "call %d (n=%d): no-alloc vs communicator" % (i, n))
            assert_exact(got_n, oracle.allreduce(bits, dt), dt, "call %d (n=%d): no-alloc vs oracle" % (i, n))


def test_noalloc_rejects_sizes_beyond_its_maximum_and_bad_arguments():
    n = MAX_BYTES // 2 + 1
    parts = [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    assert noalloc(parts, out, BF16) == -2                       # beyond 64 KiB per rank
    assert noalloc(parts[:1] * 9, out[:16], BF16) == -2          # more than 8 ranks
    assert llar.llar_allreduce_noalloc(0, [], out.data_ptr(), 16, BF16, 0) == -1
    assert noalloc(parts, out[1:17], BF16) == -1                 # misaligned output
    assert noalloc(parts, out[:0], BF16) == 0                    # nothing to do


def test_noalloc_on_a_side_stream_and_under_graph_capture():
    """Stream-ordered calls on a side stream, then the same call captured
    (its first use was eager) and replayed with fresh inputs."""
    dt, n_ranks, n = BF16, 8, 8192
    s = torch.cuda.Stream()
    parts = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    for rep in range(3):
        bits = make_partials(4200, rep, n_ranks, "bf16", n, "normal", 1.0)
        for r in range(n_ranks):
            parts[r].copy_(to_device(bits[r], dt))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            assert noalloc(parts, out, dt, s) == 0
        s.synchronize()
        assert_exact(to_host(out, dt), oracle.allreduce(bits, dt), dt, "side stream rep %d" % rep)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert noalloc(parts, out, dt) == 0
    torch.cuda.synchronize()
    for rep in range(3, 7):
        bits = make_partials(4200, rep, n_ranks, "bf16", n, "normal", 1.0)
        for r in range(n_ranks):
            parts[r].copy_(to_device(bits[r], dt))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_exact(to_host(out, dt), oracle.allreduce(bits, dt), dt, "replay %d" % rep)
