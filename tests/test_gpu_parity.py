"""GPU parity of the HIP protocols against the CPU oracle, through the C ABI.

LL and Sentinel (one-shot and pipelined) must match the oracle bit for bit
(binary64 rank-order sums, one rounding).  The atomic LL128 protocol is
non-deterministic: it must stay within |got - oracle| <= 1e-3 + rtol*|oracle|
(rtol 1e-5 fp32, 2e-3 fp16, 1.6e-2 bf16), and be bit-exact on integer data.
Every repetition draws fresh inputs (seed [workload, rep]) so that a consumer
reading the previous call's staging would fail.
"""
import numpy as np
import pytest
import torch

import message_allreduce_amd as llar
import oracle
from oracle import F32, F16, BF16, models
from workloads import WORKLOADS, make_partials, workload_partials

from gpu_util import CODE, TORCH_DT, assert_exact, assert_tol, run, to_device, to_host

pytestmark = pytest.mark.gpu

ALL_PROTOCOLS = ["ll", "sentinel", "ll128", "ll128_pipelined", "sentinel_pipelined"]
EXACT = {"ll", "sentinel", "sentinel_pipelined"}


def comm_for(n_ranks, dt, max_bytes, **opts):
    c = llar.Communicator(n_ranks, TORCH_DT[dt], max_bytes)
    c.set_option("spin_timeout_us", 100_000)
    for k, v in opts.items():
        c.set_option(k, v)
    return c


def check(got, want, dt, proto, what):
    if proto in EXACT:
        assert_exact(got, want, dt, what)
    else:
        assert_tol(got, want, dt, what)


# --------------------------------------------------------------------------- the five workloads
def test_workload1_ll_n2_fp32_1000_reps():
    w = WORKLOADS[1]
    dt = CODE[w.dtype]
    with comm_for(w.n_ranks, dt, w.bytes_per_rank) as c:
        out = torch.empty(w.n_elems, dtype=TORCH_DT[dt], device="cuda")
        for rep in range(w.reps):
            bits = workload_partials(w, rep)
            got = run(c, bits, "ll", dt, out=out)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "rep %d" % rep)
        # LL staging of the last call: both 8-byte halves carry the epoch
        e_last = c.epoch() - 1
        stage = c.staging(llar.LL).view(np.uint32)
        n_lines = 2 * ((w.bytes_per_rank + 15) // 16)
        par = (e_last & 1) * (stage.size // 2)
        lines = stage[par: par + n_lines * 4].reshape(n_lines, 4)
        want_lines = models.ll_pack(models.ll_payload_words(bits[1]), e_last)
        assert np.array_equal(lines, want_lines[:n_lines])


@pytest.mark.parametrize("acc", [0, 1], ids=["fp32_staging", "bf16_staging"])
def test_workload2_ll128_n4_bf16(acc):
    w = WORKLOADS[2]
    dt = CODE[w.dtype]
    with comm_for(w.n_ranks, dt, w.bytes_per_rank, ll128_acc=acc) as c:
        out = torch.empty(w.n_elems, dtype=TORCH_DT[dt], device="cuda")
        for rep in range(300):
            bits = workload_partials(w, rep)
            got = run(c, bits, "ll128", dt, out=out)
            assert_tol(got, oracle.allreduce(bits, dt), dt, "rep %d" % rep)
        stage = c.staging(llar.LL128)
        assert not stage.any(), "LL128 staging must be zero after every call"


def test_workload3_sentinel_n8_fp16():
    w = WORKLOADS[3]
    dt = CODE[w.dtype]
    with comm_for(w.n_ranks, dt, w.bytes_per_rank) as c:
        out = torch.empty(w.n_elems, dtype=TORCH_DT[dt], device="cuda")
        for rep in range(200):
            bits = workload_partials(w, rep)
            got = run(c, bits, "sentinel", dt, out=out)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "rep %d" % rep)
            if rep % 50 == 0:
                stage = c.staging(llar.SENTINEL).view(np.uint16)
                assert (stage == 0xFFFF).all(), "sentinel staging must be reset after use"


def test_workload4_ll128_pipelined_n8_fp32():
    w = WORKLOADS[4]
    dt = CODE[w.dtype]
    with comm_for(w.n_ranks, dt, w.bytes_per_rank, chunk_bytes=w.chunk_bytes) as c:
        assert c.geometry(w.n_elems, llar.LL128_PIPELINED)["chunks"] == 64
        out = torch.empty(w.n_elems, dtype=TORCH_DT[dt], device="cuda")
        for rep in range(12):
            bits = workload_partials(w, rep)
            got = run(c, bits, "ll128_pipelined", dt, out=out)
            assert_tol(got, oracle.allreduce(bits, dt), dt, "rep %d" % rep)
        assert not c.staging(llar.LL128_PIPELINED).any()


def test_workload5_sweep_auto_n8_bf16():
    w = WORKLOADS[5]
    dt = CODE[w.dtype]
    top = max(w.sweep_bytes)
    with comm_for(w.n_ranks, dt, top) as c:
        for nbytes in w.sweep_bytes:
            n = nbytes // 2
            bits = make_partials(w.cfg_id, nbytes, w.n_ranks, w.dtype, n, w.dist, w.scale)
            proto = c.select_protocol(nbytes)
            got = run(c, bits, "auto", dt)
            want = oracle.allreduce(bits, dt)
            name = [k for k, v in llar.PROTOCOLS.items() if v == proto][0]
            print("sweep %9d B -> %s" % (nbytes, name), flush=True)
            check(got, want, dt, name, "%d bytes (%s)" % (nbytes, name))


# --------------------------------------------------------------------------- every protocol, ragged sizes
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("proto", ALL_PROTOCOLS)
def test_protocols_ragged_sizes(proto, dtype):
    dt = CODE[dtype]
    sizes = [1, 2, 3, 7, 8, 9, 31, 33, 63, 65, 127, 1000, 4097, 8191, 20001]
    n_ranks = 8 if dtype != "fp32" else 5
    with comm_for(n_ranks, dt, 65536 * 4, chunk_bytes=4096) as c:
        for i, n in enumerate(sizes):
            bits = make_partials(100 + dt, i, n_ranks, dtype, n, "normal", 1.0)
            got = run(c, bits, proto, dt)
            check(got, oracle.allreduce(bits, dt), dt, proto, "n=%d" % n)


@pytest.mark.parametrize("n_ranks", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("proto", ALL_PROTOCOLS)
def test_protocols_every_rank_count(proto, n_ranks):
    dt = BF16
    n = 5000
    with comm_for(n_ranks, dt, n * 2, chunk_bytes=2048) as c:
        for rep in range(3):
            bits = make_partials(200 + n_ranks, rep, n_ranks, "bf16", n, "normal", 0.5)
            got = run(c, bits, proto, dt)
            check(got, oracle.allreduce(bits, dt), dt, proto, "N=%d rep %d" % (n_ranks, rep))


@pytest.mark.parametrize("proto", ALL_PROTOCOLS)
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_integer_data_is_exact_for_every_protocol(proto, dtype):
    dt = CODE[dtype]
    n = 9000
    with comm_for(8, dt, n * 4, chunk_bytes=4096) as c:
        bits = make_partials(300 + dt, 0, 8, dtype, n, "integer", 1.0)
        got = run(c, bits, proto, dt)
        assert_exact(got, oracle.allreduce(bits, dt), dt, proto)


@pytest.mark.parametrize("proto", ["ll", "sentinel", "sentinel_pipelined"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_special_values_bit_exact(proto, dtype):
    dt = CODE[dtype]
    n_ranks, n = 4, 4096
    g = np.random.default_rng(7 + dt)
    bits = make_partials(400 + dt, 0, n_ranks, dtype, n, "normal", 1.0)
    specials = {
        F32: [0x7F800000, 0xFF800000, 0x7FC00000, 0xFFFFFFFF, 0x80000000, 0x00000001, 0x80000001, 0x7F7FFFFF, 0x00800000],
        F16: [0x7C00, 0xFC00, 0x7E00, 0xFFFF, 0x8000, 0x0001, 0x8001, 0x7BFF, 0x0400],
        BF16: [0x7F80, 0xFF80, 0x7FC0, 0xFFFF, 0x8000, 0x0001, 0x8001, 0x7F7F, 0x0080],
    }[dt]
    for r in range(n_ranks):
        idx = g.choice(n, size=400, replace=False)
        bits[r, idx] = g.choice(specials, size=400)
    # every element where all ranks hold -0, and overflow to +-Inf
    bits[:, :8] = specials[4]
    bits[:, 8:16] = specials[7]
    with comm_for(n_ranks, dt, n * 4, chunk_bytes=2048) as c:
        got = run(c, bits, proto, dt)
        want = oracle.allreduce(bits, dt)
        assert_exact(got, want, dt, proto)
        if proto == "sentinel":
            stage = c.staging(llar.SENTINEL)
            assert (stage == 0xFF).all()


@pytest.mark.parametrize("proto", ["ll", "sentinel", "sentinel_pipelined"])
def test_subnormal_sums_bit_exact(proto):
    for dtype in ("fp32", "fp16", "bf16"):
        dt = CODE[dtype]
        n = 2048
        g = np.random.default_rng(11)
        mant = g.integers(0, 1 << (23 if dt == F32 else 10 if dt == F16 else 7), size=(3, n))
        sign = g.integers(0, 2, size=(3, n)) << (31 if dt == F32 else 15)
        bits = (mant | sign).astype(oracle.BITS_DTYPE[dt])
        with comm_for(3, dt, n * 4, chunk_bytes=1024) as c:
            got = run(c, bits, proto, dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "%s %s" % (proto, dtype))


# --------------------------------------------------------------------------- edge cases
@pytest.mark.parametrize("proto", ALL_PROTOCOLS)
def test_in_place_output_aliases_a_partial(proto):
    dt = BF16
    n = 6000
    bits = make_partials(500, 0, 4, "bf16", n, "normal", 1.0)
    want = oracle.allreduce(bits, dt)
    for alias in (0, 3):
        with comm_for(4, dt, n * 2, chunk_bytes=2048) as c:
            parts = [to_device(bits[r], dt) for r in range(4)]
            c.allreduce(parts, parts[alias], proto)
            torch.cuda.synchronize()
            assert c.device_status()[0] == 0
            check(to_host(parts[alias], dt), want, dt, proto, "alias %d" % alias)


def test_zero_elements_is_a_noop():
    with comm_for(2, F32, 1024) as c:
        parts = [torch.zeros(4, device="cuda") for _ in range(2)]
        out = torch.full((4,), 7.0, device="cuda")
        e0 = c.epoch()
        c.allreduce(parts, out[:0], "ll")
        torch.cuda.synchronize()
        assert c.epoch() == e0 and (out == 7.0).all()


def test_argument_errors():
    with comm_for(2, F32, 1024) as c:
        parts = [torch.zeros(256, device="cuda") for _ in range(2)]
        out = torch.zeros(256, device="cuda")
        h = c.h
        ptrs = [p.data_ptr() for p in parts]
        assert llar.llar_allreduce(h, ptrs, out.data_ptr(), 257, F32, 0, 0) == -1          # over max_bytes
        assert llar.llar_allreduce(h, ptrs, out.data_ptr(), 16, F16, 0, 0) == -1           # wrong dtype
        assert llar.llar_allreduce(h, [ptrs[0] + 4, ptrs[1]], out.data_ptr(), 16, F32, 0, 0) == -1  # misaligned
        assert llar.llar_allreduce(h, ptrs, out.data_ptr() + 8, 16, F32, 0, 0) == -1       # misaligned out
        assert llar.llar_allreduce(h, ptrs, out.data_ptr(), 16, F32, 9, 0) == -1           # bad protocol
        assert llar.llar_set_option(h, "no_such_option", 1) == -1
        assert llar.llar_set_option(h, "threads", 96) == -1


@pytest.mark.parametrize("proto", ALL_PROTOCOLS)
def test_maximum_size(proto):
    dt = F16
    n = (1 << 20) // 2  # 1 MiB per rank, the communicator's maximum
    bits = make_partials(600, 0, 8, "fp16", n, "normal", 0.02)
    with comm_for(8, dt, n * 2) as c:
        got = run(c, bits, proto, dt)
        check(got, oracle.allreduce(bits, dt), dt, proto, "max size")


def test_non_default_stream_and_back_to_back_calls():
    dt = BF16
    n = 8192
    with comm_for(8, dt, n * 2) as c:
        s = torch.cuda.Stream()
        outs, wants = [], []
        with torch.cuda.stream(s):
            for rep in range(20):
                bits = make_partials(700, rep, 8, "bf16", n, "normal", 1.0)
                parts = [to_device(bits[r], dt) for r in range(8)]
                out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
                c.allreduce(parts, out, ["ll", "sentinel", "sentinel_pipelined", "auto"][rep % 4], stream=s)
                outs.append((out, parts))
                wants.append(oracle.allreduce(bits, dt))
        s.synchronize()
        assert c.device_status()[0] == 0
        for i, ((out, _), want) in enumerate(zip(outs, wants)):
            assert_exact(to_host(out, dt), want, dt, "call %d" % i)


def test_epoch_advances_once_per_call_and_timing_records():
    with comm_for(4, BF16, 16384, timing=1) as c:
        bits = make_partials(800, 0, 4, "bf16", 8192, "normal", 1.0)
        parts = [to_device(bits[r], BF16) for r in range(4)]
        out = torch.empty(8192, dtype=torch.bfloat16, device="cuda")
        e0 = c.epoch()
        for proto in ALL_PROTOCOLS:
            c.allreduce(parts, out, proto)
        torch.cuda.synchronize()
        assert c.epoch() == e0 + len(ALL_PROTOCOLS)
        recs = c.timing(len(ALL_PROTOCOLS))
        assert len(recs) == len(ALL_PROTOCOLS)
        hz = llar.llar_wallclock_hz()
        for t0, t1 in recs:
            assert t0 != 2**64 - 1 and t1 > t0
            assert (t1 - t0) / hz < 0.05


@pytest.mark.parametrize("proto", ALL_PROTOCOLS)
def test_lost_contribution_times_out_and_recovers(proto):
    """A rank whose producers write nothing (forced from the host) makes the
    consumers' bounded polls expire: the kernel ends, the status word says
    TIMEOUT, and after a reset the communicator works again."""
    dt = BF16
    n = 4096
    bits = make_partials(900, 0, 4, "bf16", n, "normal", 1.0)
    with comm_for(4, dt, n * 2, chunk_bytes=2048) as c:
        c.set_option("spin_timeout_us", 2000)
        c.set_option("debug_drop_rank", 2)
        parts = [to_device(bits[r], dt) for r in range(4)]
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        c.allreduce(parts, out, proto)
        torch.cuda.synchronize()
        st, status_bits = c.device_status()
        assert st == -5 and (status_bits & 1), (st, status_bits)
        c.clear_device_status()
        c.set_option("debug_drop_rank", -1)
        c.set_option("spin_timeout_us", 100_000)
        got = run(c, bits, proto, dt)
        check(got, oracle.allreduce(bits, dt), dt, proto, "after recovery")


@pytest.mark.parametrize("placement", [1, 2])
@pytest.mark.parametrize("chunk", [1024, 65536, 1 << 20])
def test_sentinel_pipelined_chunks_and_placements(placement, chunk):
    dt = BF16
    n = (3 << 20) // 2 + 37  # 3 MiB + a ragged tail
    bits = make_partials(1000, chunk, 8, "bf16", n, "normal", 1.0)
    with comm_for(8, dt, n * 2, chunk_bytes=chunk, placement=placement) as c:
        got = run(c, bits, "sentinel_pipelined", dt)
        assert_exact(got, oracle.allreduce(bits, dt), dt, "chunk %d placement %d" % (chunk, placement))
        assert (c.staging(llar.SENTINEL_PIPELINED) == 0xFF).all()


@pytest.mark.parametrize("buffers", [2, 4, 6, 8, 16, 32])
def test_sentinel_pipelined_buffers_and_credit_order(buffers):
    """Every staging-buffer count gives the exact sum, and the per-chunk
    stamps of each workgroup follow the credit rule: with B buffers the
    producers enter chunk c only after this workgroup's consumers finished
    chunk c - B/2 (lag B/2 - 1), and one consumer group takes the chunks in
    order (several groups: test_sentinel_pipelined_consumer_groups)."""
    dt = BF16
    n = (3 << 20) // 2 + 11  # 3 MiB + a ragged tail: 49 chunks of 64 KiB
    chunk = 65536
    bits = make_partials(1050, buffers, 8, "bf16", n, "normal", 1.0)
    with comm_for(8, dt, n * 2, chunk_bytes=chunk, pipeline_buffers=buffers, consumer_groups=1, trace=1) as c:
        got = run(c, bits, "sentinel_pipelined", dt)
        assert_exact(got, oracle.allreduce(bits, dt), dt, "buffers %d" % buffers)
        assert (c.staging(llar.SENTINEL_PIPELINED) == 0xFF).all()
        geo = c.geometry(n, llar.SENTINEL_PIPELINED)
        chunks = geo["chunks"]
        assert chunks == -(-(n * 2) // chunk) and chunks <= 128
        tr = llar.llar_get_pipeline_trace(c.h).astype(np.int64)
        assert tr.shape[0] == geo["grid"]
        lag = buffers // 2 - 1
        working = tr[:, 0] != 0  # padding workgroups of the local placement record nothing
        assert working.sum() == 8 * geo["slices"]
        credit, stored = tr[working, 0:chunks], tr[working, 128:128 + chunks]
        ready, done = tr[working, 256:256 + chunks], tr[working, 384:384 + chunks]
        for a_ in (credit, stored, ready, done):
            assert (a_ > 0).all()
        assert (stored >= credit).all()
        assert (done >= ready).all()
        assert (ready[:, 1:] >= done[:, :-1]).all()
        assert (credit[:, lag + 1:] >= done[:, :chunks - lag - 1]).all()


@pytest.mark.parametrize("groups,pgroups,buffers", [(2, 1, 2), (2, 1, 4), (2, 1, 8), (4, 1, 4), (4, 1, 8), (2, 1, 16),
                                                     (1, 2, 4), (2, 2, 4), (2, 4, 8), (4, 2, 8)])
def test_sentinel_pipelined_consumer_groups(groups, pgroups, buffers):
    """Chunks dealt to G consumer groups (group g takes chunks g, g + G, ...)
    and to PG producer groups under the workgroup credit: exact, the staging
    left all-ones, and the per-chunk stamps follow the rules -- a consumer
    group takes its chunks in order, and chunk c is stored only after every
    chunk up to c - 1 - lag is done, whichever groups had them."""
    dt = BF16
    n = (3 << 20) // 2 + 11  # 3 MiB + a ragged tail: 49 chunks of 64 KiB
    chunk = 65536
    bits = make_partials(1060, 100 * pgroups + 10 * groups + buffers, 8, "bf16", n, "normal", 1.0)
    with comm_for(8, dt, n * 2, chunk_bytes=chunk, pipeline_buffers=buffers, consumer_groups=groups,
                  producer_groups=pgroups, trace=1) as c:
        got = run(c, bits, "sentinel_pipelined", dt)
        assert_exact(got, oracle.allreduce(bits, dt), dt, "groups %d buffers %d" % (groups, buffers))
        assert (c.staging(llar.SENTINEL_PIPELINED) == 0xFF).all()
        geo = c.geometry(n, llar.SENTINEL_PIPELINED)
        chunks = geo["chunks"]
        tr = llar.llar_get_pipeline_trace(c.h).astype(np.int64)
        lag = buffers // 2 - 1
        working = tr[:, 0] != 0
        credit, stored = tr[working, 0:chunks], tr[working, 128:128 + chunks]
        ready, done = tr[working, 256:256 + chunks], tr[working, 384:384 + chunks]
        for a_ in (credit, stored, ready, done):
            assert (a_ > 0).all()
        assert (stored >= credit).all() and (done >= ready).all()
        assert (ready[:, groups:] >= done[:, :-groups]).all()
        for ch in range(lag + 1, chunks):
            assert (credit[:, ch] >= done[:, :ch - lag].max(axis=1)).all(), ch
        # a second call through the same buffers stays exact
        bits = make_partials(1061, 100 * pgroups + 10 * groups + buffers, 8, "bf16", n, "normal", 1.0)
        assert_exact(run(c, bits, "sentinel_pipelined", dt), oracle.allreduce(bits, dt), dt, "second call")


def test_sentinel_pipelined_consumer_groups_refusals():
    """Consumer groups that do not divide the consumer waves or the buffer
    count, and producer groups that do not divide the producer waves, are
    refused with nothing launched; the default afterwards is exact."""
    dt = BF16
    n = 200000
    bits = make_partials(1062, 0, 8, "bf16", n, "normal", 1.0)
    with comm_for(8, dt, n * 2, chunk_bytes=65536, pipeline_buffers=4, threads=512) as c:
        for g in (3, 8):  # 3 divides neither 4 consumer waves nor 4 buffers; 8 exceeds the waves
            c.set_option("consumer_groups", g)
            with pytest.raises(llar.LlarError):
                run(c, bits, "sentinel_pipelined", dt)
        c.set_option("pipeline_buffers", 6)
        c.set_option("consumer_groups", 4)  # divides the waves, not the 6 buffers
        with pytest.raises(llar.LlarError):
            run(c, bits, "sentinel_pipelined", dt)
        c.set_option("consumer_groups", 0)
        c.set_option("producer_groups", 3)  # does not divide the 4 producer waves
        with pytest.raises(llar.LlarError):
            run(c, bits, "sentinel_pipelined", dt)
        c.set_option("producer_groups", 0)
        assert_exact(run(c, bits, "sentinel_pipelined", dt), oracle.allreduce(bits, dt), dt, "after the refusals")


@pytest.mark.parametrize("threads", [256, 512])
def test_ll128_pipelined_multiwave_credit_regression(threads):
    """Workload-4 shape (N = 8, fp32, 4 MiB in 64 KiB chunks) with several
    waves per workgroup and 8 slices: owner slices then differ by one line,
    so a wave can produce into another owner's line while having no line of
    its own to consume.  The credit must still hold (it is the workgroup's)."""
    dt = F32
    n = 1 << 20
    bits = make_partials(1700, threads, 8, "fp32", n, "uniform", 1.0)
    with comm_for(8, dt, n * 4, chunk_bytes=65536, threads=threads, slices=8) as c:
        c.set_option("spin_timeout_us", 20_000)
        for rep in range(3):
            got = run(c, bits, "ll128_pipelined", dt)
            assert_tol(got, oracle.allreduce(bits, dt), dt, "threads %d rep %d" % (threads, rep))


@pytest.mark.parametrize("proto", ["ll128_pipelined", "sentinel_pipelined"])
def test_pipelined_slices_are_clamped_to_non_empty_owner_slices(proto):
    """Asking for more slices than the smallest owner shard of a chunk has
    lines / vectors gives the largest safe count, and stays exact.  The
    message is cut into equal chunks of at most chunk_bytes (whole 16-byte
    vectors for the Sentinel): 41 chunks of 1001 elements (33 LL128 lines,
    4 per owner) or of 2016 bytes (126 vectors, 15 per owner)."""
    dt = BF16
    n_ranks, chunk = 8, 2048
    n = 40 * 1024 + 77
    n_chunks = -(-(n * 2) // chunk)
    bits = make_partials(1710, 0, n_ranks, "bf16", n, "normal", 1.0)
    with comm_for(n_ranks, dt, n * 2, chunk_bytes=chunk, slices=64) as c:
        geo = c.geometry(n, llar.PROTOCOLS[proto])
        assert geo["chunks"] == n_chunks == 41
        if proto == "ll128_pipelined":
            chunk_elems = -(-n // n_chunks)
            per_owner = (chunk_elems + 30) // 31 // n_ranks
        else:
            chunk_vecs = -(-(-(-(n * 2) // n_chunks)) // 16)
            per_owner = chunk_vecs // n_ranks
        assert geo["slices"] == per_owner
        for rep in range(3):
            got = run(c, bits, proto, dt)
            check(got, oracle.allreduce(bits, dt), dt, proto, "rep %d" % rep)


# --------------------------------------------------------------------------- slot handshake (sentinel_credit = 1)
@pytest.mark.parametrize("placement", [1, 2])
@pytest.mark.parametrize("chunk,threads,cons", [(1024, 0, 0), (4096, 512, 2), (65536, 0, 0), (1 << 20, 256, 1),
                                                (262144, 1024, 8)])
def test_sentinel_handshake_exact(placement, chunk, threads, cons):
    """The pipelined Sentinel whose credit is the slot reset itself: exact
    for every chunk size, wave split and placement, a ragged tail vector,
    fresh inputs on every call, and every slot empty again afterwards."""
    dt = BF16
    n = (3 << 20) // 2 + 37  # 3 MiB + 74 bytes: the last vector is partial
    with comm_for(8, dt, n * 2, sentinel_credit=1, chunk_bytes=chunk, threads=threads, consumer_waves=cons,
                  placement=placement) as c:
        for rep in range(2):
            bits = make_partials(1800 + placement, chunk + rep, 8, "bf16", n, "normal", 1.0)
            got = run(c, bits, "sentinel_pipelined", dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "chunk %d rep %d" % (chunk, rep))
        assert (c.staging(llar.SENTINEL_PIPELINED) == 0xFF).all()


@pytest.mark.parametrize("n_ranks", [1, 2, 3, 4, 5, 6, 7, 8])
def test_sentinel_handshake_every_rank_count(n_ranks):
    dt = BF16
    n = 5001
    with comm_for(n_ranks, dt, n * 2, sentinel_credit=1, chunk_bytes=2048) as c:
        for rep in range(3):
            bits = make_partials(1900 + n_ranks, rep, n_ranks, "bf16", n, "normal", 0.5)
            got = run(c, bits, "sentinel_pipelined", dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "N=%d rep %d" % (n_ranks, rep))


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_sentinel_handshake_ragged_sizes_and_slices(dtype):
    """Sizes around every vector and chunk boundary, and slice counts that
    give one, several or a fraction of a 64-vector batch per chunk (the
    buffer count then changes with the wave period)."""
    dt = CODE[dtype]
    n_ranks = 8 if dtype != "fp32" else 5
    sizes = [1, 7, 9, 63, 65, 1000, 4097, 20001, 70001]
    with comm_for(n_ranks, dt, 70001 * 4, sentinel_credit=1, chunk_bytes=8192) as c:
        for slices in (1, 3, 7, 32):
            c.set_option("slices", slices)
            for i, n in enumerate(sizes):
                bits = make_partials(2000 + dt, slices * 100 + i, n_ranks, dtype, n, "normal", 1.0)
                got = run(c, bits, "sentinel_pipelined", dt)
                assert_exact(got, oracle.allreduce(bits, dt), dt, "slices %d n=%d" % (slices, n))


def test_sentinel_handshake_lost_contribution_times_out_and_recovers():
    dt = BF16
    n = 40000
    bits = make_partials(2100, 0, 4, "bf16", n, "normal", 1.0)
    with comm_for(4, dt, n * 2, sentinel_credit=1, chunk_bytes=4096) as c:
        c.set_option("spin_timeout_us", 2000)
        c.set_option("debug_drop_rank", 1)
        parts = [to_device(bits[r], dt) for r in range(4)]
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        c.allreduce(parts, out, "sentinel_pipelined")
        torch.cuda.synchronize()
        st, status_bits = c.device_status()
        assert st == -5 and (status_bits & 1), (st, status_bits)
        c.clear_device_status()
        c.set_option("debug_drop_rank", -1)
        c.set_option("spin_timeout_us", 100_000)
        got = run(c, bits, "sentinel_pipelined", dt)
        assert_exact(got, oracle.allreduce(bits, dt), dt, "after recovery")


# --------------------------------------------------------------------------- owner credit (sentinel_credit = 2)
@pytest.mark.parametrize("placement", [1, 2])
@pytest.mark.parametrize("chunk,threads,cons,buffers", [(1024, 0, 0, 2), (4096, 512, 2, 3), (65536, 0, 0, 5),
                                                        (1 << 20, 256, 1, 2), (262144, 1024, 8, 4),
                                                        (16384, 1024, 3, 7)])
def test_sentinel_owner_credit_exact(placement, chunk, threads, cons, buffers):
    """The pipelined Sentinel whose credit is every owner's published
    progress: exact for every chunk size, wave split, buffer count (odd ones
    too) and placement, with a ragged tail vector, fresh inputs on every
    call, and every slot empty again afterwards."""
    dt = BF16
    n = (3 << 20) // 2 + 37  # 3 MiB + 74 bytes: the last vector is partial
    with comm_for(8, dt, n * 2, sentinel_credit=2, chunk_bytes=chunk, threads=threads, consumer_waves=cons,
                  pipeline_buffers=buffers, placement=placement) as c:
        for rep in range(2):
            bits = make_partials(2200 + placement, chunk + rep, 8, "bf16", n, "normal", 1.0)
            got = run(c, bits, "sentinel_pipelined", dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "chunk %d rep %d" % (chunk, rep))
        assert (c.staging(llar.SENTINEL_PIPELINED) == 0xFF).all()


@pytest.mark.parametrize("n_ranks", [1, 2, 3, 4, 5, 6, 7, 8])
def test_sentinel_owner_credit_every_rank_count(n_ranks):
    dt = BF16
    n = 5001
    with comm_for(n_ranks, dt, n * 2, sentinel_credit=2, chunk_bytes=2048, pipeline_buffers=3) as c:
        for rep in range(3):
            bits = make_partials(2300 + n_ranks, rep, n_ranks, "bf16", n, "normal", 0.5)
            got = run(c, bits, "sentinel_pipelined", dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "N=%d rep %d" % (n_ranks, rep))


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_sentinel_owner_credit_ragged_sizes_and_slices(dtype):
    """Sizes around every vector and chunk boundary, and slice counts that
    leave some slices of an owner's shard empty in a chunk (their consumer
    waves still publish progress)."""
    dt = CODE[dtype]
    n_ranks = 8 if dtype != "fp32" else 5
    sizes = [1, 7, 9, 63, 65, 1000, 4097, 20001, 70001]
    with comm_for(n_ranks, dt, 70001 * 4, sentinel_credit=2, chunk_bytes=8192, pipeline_buffers=2) as c:
        for slices in (1, 3, 7, 24, 32):
            c.set_option("slices", slices)
            for i, n in enumerate(sizes):
                bits = make_partials(2400 + dt, slices * 100 + i, n_ranks, dtype, n, "normal", 1.0)
                got = run(c, bits, "sentinel_pipelined", dt)
                assert_exact(got, oracle.allreduce(bits, dt), dt, "slices %d n=%d" % (slices, n))


def test_sentinel_owner_credit_many_chunks_device_epoch_and_other_credits():
    """16 MiB per rank in 512 chunks through two buffers, with the device-
    resident epoch (the progress words are tagged with it) and calls of the
    other two credit schemes on the same staging in between."""
    dt = BF16
    n = 8 << 20
    with comm_for(8, dt, n * 2, chunk_bytes=32768) as c:
        for rep, (credit, dev) in enumerate([(2, 1), (0, 0), (2, 0), (1, 1), (2, 1)]):
            c.set_option("sentinel_credit", credit)
            c.set_option("device_epoch", dev)
            c.set_option("pipeline_buffers", 2 if credit == 2 else 4)
            bits = make_partials(2500, rep, 8, "bf16", n, "normal", 1.0)
            got = run(c, bits, "sentinel_pipelined", dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "rep %d credit %d" % (rep, credit))
        assert (c.staging(llar.SENTINEL_PIPELINED) == 0xFF).all()


def test_sentinel_owner_credit_limits():
    dt = BF16
    n = 40000
    bits = make_partials(2600, 0, 4, "bf16", n, "normal", 1.0)
    with comm_for(4, dt, n * 2, sentinel_credit=2, chunk_bytes=4096) as c:
        # more consumer waves than progress words per slice, or than the
        # workgroup has room for next to a producer and the credit wave
        for threads, cons in ((1024, 9), (256, 3)):
            c.set_option("threads", threads)
            c.set_option("consumer_waves", cons)
            with pytest.raises(llar.LlarError) as ei:
                run(c, bits, "sentinel_pipelined", dt)
            assert ei.value.status == -1
        c.set_option("threads", 0)
        c.set_option("consumer_waves", 0)
        # kept staging is never reset: a buffer used twice is refused
        c.set_option("keep_staging", 1)
        with pytest.raises(llar.LlarError) as ei:
            run(c, bits, "sentinel_pipelined", dt)
        assert ei.value.status == -2
        c.set_option("keep_staging", 0)
        got = run(c, bits, "sentinel_pipelined", dt)
        assert_exact(got, oracle.allreduce(bits, dt), dt, "after refusals")


def test_sentinel_owner_credit_lost_contribution_times_out_and_recovers():
    dt = BF16
    n = 40000
    bits = make_partials(2700, 0, 4, "bf16", n, "normal", 1.0)
    with comm_for(4, dt, n * 2, sentinel_credit=2, chunk_bytes=4096, pipeline_buffers=3) as c:
        c.set_option("spin_timeout_us", 2000)
        c.set_option("debug_drop_rank", 1)
        parts = [to_device(bits[r], dt) for r in range(4)]
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        c.allreduce(parts, out, "sentinel_pipelined")
        torch.cuda.synchronize()
        st, status_bits = c.device_status()
        assert st == -5 and (status_bits & 1), (st, status_bits)
        c.clear_device_status()
        c.set_option("debug_drop_rank", -1)
        c.set_option("spin_timeout_us", 100_000)
        got = run(c, bits, "sentinel_pipelined", dt)
        assert_exact(got, oracle.allreduce(bits, dt), dt, "after recovery")


@pytest.mark.parametrize("threads", [64, 128, 256, 512])
@pytest.mark.parametrize("proto", ALL_PROTOCOLS)
def test_workgroup_sizes(proto, threads):
    dt = F32
    n = 30000
    bits = make_partials(1100, threads, 6, "fp32", n, "uniform", 1.0)
    with comm_for(6, dt, n * 4, threads=threads, chunk_bytes=8192) as c:
        if proto == "sentinel_pipelined" and threads < 128:
            # producer and consumer waves need at least two waves
            with pytest.raises(llar.LlarError) as ei:
                run(c, bits, proto, dt)
            assert ei.value.status == -1
            return
        got = run(c, bits, proto, dt)
        check(got, oracle.allreduce(bits, dt), dt, proto, "threads %d" % threads)


def test_ll128_keep_staging_matches_line_model():
    """With integer data every atomic order gives the same staged sums: the
    kept staging must equal the line model bit for bit (flag slot == N)."""
    dt = BF16
    n_ranks, n = 4, 3000
    bits = make_partials(1200, 0, n_ranks, "bf16", n, "integer", 1.0)
    with comm_for(n_ranks, dt, n * 2, keep_staging=1) as c:
        run(c, bits, "ll128", dt)
        g = models.LL128Geometry(n, n_ranks, 4)
        stage = c.staging(llar.LL128)[: g.staging_bytes].view(np.float32).reshape(g.lines, g.slots)
        model = models.ll128_staging_image(bits, dt, F32)
        assert np.array_equal(stage.astype(np.float64), model)
        assert (stage[:, 0] == n_ranks).all()


@pytest.mark.parametrize("placement", [1, 2])
@pytest.mark.parametrize("proto", ["ll", "sentinel"])
def test_one_shot_placements(proto, placement):
    dt = F16
    with comm_for(8, dt, 1 << 20, placement=placement) as c:
        for i, n in enumerate([5, 64, 8192, 65536 + 3, 300000]):
            bits = make_partials(1300 + placement, i, 8, "fp16", n, "normal", 1.0)
            got = run(c, bits, proto, dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "%s placement %d n=%d" % (proto, placement, n))
        if proto == "sentinel":
            assert (c.staging(llar.SENTINEL) == 0xFF).all()


@pytest.mark.parametrize("proto", ALL_PROTOCOLS)
def test_device_epoch_option(proto):
    dt = BF16
    n = 7000
    with comm_for(4, dt, n * 2, device_epoch=1, chunk_bytes=4096) as c:
        for rep in range(4):
            bits = make_partials(1400, rep, 4, "bf16", n, "normal", 1.0)
            got = run(c, bits, proto, dt)
            check(got, oracle.allreduce(bits, dt), dt, proto, "rep %d" % rep)
        e = c.epoch()
        assert e & 0x80000000


def test_graph_capture_replays_use_fresh_epochs():
    """Calls captured into a graph read the device-resident epoch, so every
    replay is a new call: stale LL lines from the previous replay are
    rejected.  Eager work (new inputs, synchronisation) sits between replays,
    and every replay is checked against the oracle."""
    dt = BF16
    n, n_ranks = 4096, 8
    c = comm_for(n_ranks, dt, n * 2, chunk_bytes=2048)
    try:
        parts = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
        outs = {p: torch.empty(n, dtype=torch.bfloat16, device="cuda") for p in ALL_PROTOCOLS}
        bits0 = make_partials(1500, 0, n_ranks, "bf16", n, "normal", 1.0)
        for r in range(n_ranks):
            parts[r].copy_(to_device(bits0[r], dt))
        # warm up eagerly, then capture one call of every protocol
        for p in ALL_PROTOCOLS:
            c.allreduce(parts, outs[p], p)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for p in ALL_PROTOCOLS:
                c.allreduce(parts, outs[p], p)
        torch.cuda.synchronize()
        for rep in range(1, 6):
            bits = make_partials(1500, rep, n_ranks, "bf16", n, "normal", 1.0)
            for r in range(n_ranks):
                parts[r].copy_(to_device(bits[r], dt))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            st, sbits = c.device_status()
            assert st == 0, (st, sbits)
            want = oracle.allreduce(bits, dt)
            for p in ALL_PROTOCOLS:
                check(to_host(outs[p], dt), want, dt, p, "replay %d %s" % (rep, p))
            # an eager call between replays (host-numbered epoch)
            got = run(c, bits, "ll", dt)
            assert_exact(got, want, dt, "eager after replay %d" % rep)
    finally:
        c.close()


@pytest.mark.parametrize("proto", ["ll128_pipelined", "sentinel_pipelined"])
def test_pipelined_short_last_chunk_regression(proto):
    """A chunk that is shorter than the others reuses a parity: the lines /
    slots must keep their (owner, slice) so the implicit credit still covers
    them.  Sizes leave every kind of ragged last chunk; many repetitions."""
    dt = BF16
    chunk = 2048
    for n_ranks in (4, 8):
        with comm_for(n_ranks, dt, 64 * chunk, chunk_bytes=chunk) as c:
            for i, n in enumerate([5000, 1024 * 5 + 1, 1024 * 3 + 700, 1024 * 9 + 31, 1024 * 2 + 1]):
                for rep in range(8):
                    bits = make_partials(1600 + i, rep, n_ranks, "bf16", n, "normal", 1.0)
                    got = run(c, bits, proto, dt)
                    check(got, oracle.allreduce(bits, dt), dt, proto, "N=%d n=%d rep %d" % (n_ranks, n, rep))


def test_default_geometry_rules():
    """The host's default geometry: one-shot workgroups of 256 threads below
    64 slices' worth of 8-byte units, 512 from there; under the local
    placement a call of 5 to 8 slices keeps to XCDs 0-2 (the grid covers
    three slices per round of eight XCDs), others use all eight, and from
    four ranks on rank 0's part of a slice runs on two workgroups (N + 1 per
    slice); pipelined messages cut into the fewest chunks of at most the
    configured size, and a message shorter than the chunk as one chunk."""
    with comm_for(8, BF16, 8 << 20) as c:
        local = c.get_option("local_placement_ok") == 1
        for nbytes, threads, span in ((8192, 256, 8), (8192 + 16, 256, 3), (16384, 256, 3), (16384 + 16, 256, 8),
                                      (131072 - 16, 256, 8), (131072, 512, 8), (524288, 512, 8)):
            for proto in (llar.LL, llar.SENTINEL):
                geo = c.geometry(nbytes // 2, proto)
                assert geo["threads"] == threads, (nbytes, geo)
                units = 2 * (-(-nbytes // 16))
                slices = min(64, -(-units // threads))
                assert geo["slices"] == slices, (nbytes, geo)
                if local:
                    assert geo["grid"] == 9 * 8 * (-(-slices // span)), (nbytes, geo)
        # a given thread count or slice count keeps all eight XCDs
        c.set_option("threads", 256)
        assert c.geometry(8192, llar.LL)["grid"] == (72 if local else 64)
        c.set_option("consumer_split", 1)
        assert c.geometry(8192, llar.LL)["grid"] == 64
        c.set_option("consumer_split", 0)
        c.set_option("threads", 0)
        for nbytes in (128, 65536, (1 << 20) - 16, 1 << 20, (1 << 20) + 16, (3 << 19), 8 << 20):
            geo = c.geometry(nbytes // 2, llar.SENTINEL_PIPELINED)
            assert geo["chunks"] == max(1, -(-nbytes // (1 << 20))), (nbytes, geo)
        c.set_option("chunk_bytes", 65536)
        geo = c.geometry((1 << 20) // 2 + 8, llar.LL128_PIPELINED)
        assert geo["chunks"] == 17
    # equal chunks of a ragged message stay exact
    dt = BF16
    n = (3 << 19) // 2 + 77
    bits = make_partials(2800, 0, 8, "bf16", n, "normal", 1.0)
    with comm_for(8, dt, n * 2) as c:
        got = run(c, bits, "sentinel_pipelined", dt)
        assert_exact(got, oracle.allreduce(bits, dt), dt, "1.5 MiB + 154 B")


def test_ll128_default_geometry():
    """LL128 defaults: one round keeps 256-thread workgroups while a slice
    holds fewer than 32 lines of each owner and takes 512 from there; the
    pipeline splits 1024-thread workgroups into producer and consumer waves,
    with at most 32 slices and 256 KiB chunks (the alternating pipeline,
    option ll128_kernel = 1, keeps 512 threads and 1 MiB chunks)."""
    with comm_for(8, BF16, 2 << 20) as c:
        geo = c.geometry(8192, llar.LL128)  # 265 lines, 34 per owner, one per slice
        assert (geo["threads"], geo["slices"]) == (256, 34), geo
        geo = c.geometry(1 << 20, llar.LL128)  # 33 826 lines, 4229 per owner, 67 per slice
        assert (geo["threads"], geo["slices"]) == (512, 64), geo
    with comm_for(8, F32, 4 << 20, chunk_bytes=65536) as c:
        geo = c.geometry(1 << 20, llar.LL128_PIPELINED)  # 529 lines a chunk, 66-67 per owner
        assert (geo["threads"], geo["slices"], geo["chunks"]) == (1024, 32, 64), geo
        c.set_option("ll128_kernel", 1)
        geo = c.geometry(1 << 20, llar.LL128_PIPELINED)
        assert (geo["threads"], geo["slices"], geo["chunks"]) == (512, 32, 64), geo
    with comm_for(8, F32, 4 << 20) as c:
        assert c.geometry(1 << 20, llar.LL128_PIPELINED)["chunks"] == 16   # 256 KiB chunks
        c.set_option("ll128_kernel", 1)
        assert c.geometry(1 << 20, llar.LL128_PIPELINED)["chunks"] == 4    # 1 MiB chunks


@pytest.mark.parametrize("threads,cons,buffers", [(1024, 0, 0), (1024, 8, 16), (1024, 2, 2), (512, 0, 4), (512, 3, 6),
                                                  (256, 1, 2), (128, 1, 64), (1024, 15, 30)])
@pytest.mark.parametrize("acc", [0, 1])
def test_ll128_wave_split_pipeline_configurations(threads, cons, buffers, acc):
    """The wave-split LL128 pipeline over wave splits and buffer counts
    (B = 2 lag + 2, the consumer of chunk c - B is the consumer of chunk c):
    integer data is exact in every order (bfloat16 with binary32 staging;
    binary16 with 16-bit staging, whose 11 bits hold every partial sum of
    eight integers up to 64), normal data within tolerance; the alternating
    pipeline on the same staging in between stays right."""
    dt, name = (BF16, "bf16") if acc == 0 else (F16, "fp16")
    n = 3 * 8192 + 333   # ragged: 13 chunks of 4 KiB, the last one short
    with comm_for(8, dt, n * 2, chunk_bytes=4096, threads=threads, consumer_waves=cons, ll128_buffers=buffers,
                  ll128_acc=acc) as c:
        for rep in range(3):
            bits = make_partials(2900 + acc, rep, 8, name, n, "integer", 1.0)
            got = run(c, bits, "ll128_pipelined", dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "integer rep %d" % rep)
            bits = make_partials(2910 + acc, rep, 8, name, n, "normal", 0.02)
            got = run(c, bits, "ll128_pipelined", dt)
            assert_tol(got, oracle.allreduce(bits, dt), dt, "normal rep %d" % rep)
        c.set_option("ll128_kernel", 1)
        c.set_option("threads", 512 if threads == 1024 else threads)
        bits = make_partials(2920, acc, 8, name, n, "integer", 1.0)
        assert_exact(run(c, bits, "ll128_pipelined", dt), oracle.allreduce(bits, dt), dt, "alternating kernel")
        c.set_option("ll128_kernel", 0)
        c.set_option("threads", threads)
        assert_exact(run(c, bits, "ll128_pipelined", dt), oracle.allreduce(bits, dt), dt, "wave split again")


def test_ll128_wave_split_refuses_what_cannot_work():
    """Too many consumer waves for the workgroup, or kept staging that a
    later chunk would have to reuse, are refused with nothing launched."""
    dt = BF16
    n = 8192
    bits = make_partials(2930, 0, 4, "bf16", n, "normal", 1.0)
    parts = [to_device(bits[r], dt) for r in range(4)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    with comm_for(4, dt, n * 2, chunk_bytes=1024, threads=256, consumer_waves=4) as c:
        with pytest.raises(llar.LlarError):
            c.allreduce(parts, out, "ll128_pipelined")   # 4 waves, 4 consumers, no producer
        c.set_option("consumer_waves", 0)
        c.set_option("keep_staging", 1)
        c.set_option("ll128_buffers", 2)
        with pytest.raises(llar.LlarError):
            c.allreduce(parts, out, "ll128_pipelined")   # 16 chunks through 2 kept buffers
        c.set_option("keep_staging", 0)
        got = run(c, bits, "ll128_pipelined", dt)
        assert_tol(got, oracle.allreduce(bits, dt), dt, "after the refusals")


# --------------------------------------------------------------------------- the barrier ablation
@pytest.mark.parametrize("placement", [1, 2], ids=["spread", "local"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_barrier_ablation_is_exact_and_leaves_the_protocols_working(dtype, placement):
    """The one-shot reduce behind a grid-wide barrier (measurement option)
    computes the same bit-exact sum; LL and Sentinel calls before and after
    it stay exact, so the staging it borrows is left valid."""
    dt = CODE[dtype]
    n_ranks = 8
    sizes = [1, 7, 8192, 65537]
    with comm_for(n_ranks, dt, max(sizes) * 4, placement=placement) as c:
        for i, n in enumerate(sizes):
            bits = make_partials(5000 + dt, i, n_ranks, dtype, n, "normal", 1.0)
            want = oracle.allreduce(bits, dt)
            c.set_option("barrier_ablation", 1)
            for proto in ("ll", "sentinel", "auto"):
                assert_exact(run(c, bits, proto, dt), want, dt, "ablation %s n=%d" % (proto, n))
            c.set_option("barrier_ablation", 0)
            for proto in ALL_PROTOCOLS:
                check(run(c, bits, proto, dt), want, dt, proto, "after ablation %s n=%d" % (proto, n))


@pytest.mark.parametrize("n_ranks", [1, 2, 3, 5, 8])
def test_barrier_ablation_every_rank_count_and_graph_replays(n_ranks):
    dt = BF16
    n = 3000
    c = comm_for(n_ranks, dt, n * 2, barrier_ablation=1)
    try:
        parts = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        bits = make_partials(5100 + n_ranks, 0, n_ranks, "bf16", n)
        for r in range(n_ranks):
            parts[r].copy_(to_device(bits[r], dt))
        c.allreduce(parts, out, "ll")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            c.allreduce(parts, out, "ll")
            c.allreduce(parts, out, "ll")
        torch.cuda.synchronize()
        for rep in range(1, 4):
            bits = make_partials(5100 + n_ranks, rep, n_ranks, "bf16", n)
            for r in range(n_ranks):
                parts[r].copy_(to_device(bits[r], dt))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            st, sbits = c.device_status()
            assert st == 0, (st, sbits)
            assert_exact(to_host(out, dt), oracle.allreduce(bits, dt), dt, "N=%d replay %d" % (n_ranks, rep))
    finally:
        c.close()


# --------------------------------------------------------------------------- process defaults and logging
def test_process_defaults_reach_new_communicators_and_log_prints_geometry(capfd):
    """Defaults set with a NULL handle (as the LLAR_* environment knobs do)
    are what a new communicator starts from: a forced AUTO protocol runs and
    stays exact, and "log" prints each call's protocol and geometry."""
    dt = BF16
    n = 4096
    bits = make_partials(3000, 0, 8, "bf16", n, "normal", 1.0)
    assert llar.llar_set_option(None, "auto_protocol", llar.SENTINEL_PIPELINED) == 0
    assert llar.llar_set_option(None, "log", 1) == 0
    try:
        with comm_for(8, dt, n * 2) as c:
            assert c.get_option("auto_protocol") == llar.SENTINEL_PIPELINED and c.get_option("log") == 1
            assert c.select_protocol(n * 2) == llar.SENTINEL_PIPELINED
            capfd.readouterr()
            got = run(c, bits, "auto", dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "forced sentinel_pipelined")
            err = capfd.readouterr().err
            assert "llar: allreduce n_ranks=8 dtype=bf16 elems=4096" in err and "protocol=sentinel_pipelined" in err, err
            c.set_option("log", 0)
            run(c, bits, "ll", dt)
            assert "llar:" not in capfd.readouterr().err
    finally:
        assert llar.llar_set_option(None, "auto_protocol", 0) == 0
        assert llar.llar_set_option(None, "log", 0) == 0
    with comm_for(8, dt, n * 2) as c:
        assert c.get_option("auto_protocol") == 0 and c.select_protocol(n * 2) == llar.LL


@pytest.mark.parametrize("split", [1, 2])
@pytest.mark.parametrize("n_ranks", [2, 5, 8])
@pytest.mark.parametrize("proto", ["ll", "sentinel"])
def test_one_shot_consumer_split(proto, n_ranks, split):
    """Rank 0's part of each slice on one or two consumer workgroups (option
    consumer_split): bit-exact over ragged sizes, slice counts and thread
    counts (a part may be empty), under the local placement and, where the
    split does not apply, the spread one."""
    dt = BF16
    with comm_for(n_ranks, dt, 256 << 10, consumer_split=split) as c:
        for i, n in enumerate((1, 3, 999, 8192, 8192 + 5, 65536 + 77, 131072)):
            bits = make_partials(3400 + 10 * n_ranks + split, i, n_ranks, "bf16", n, "normal", 1.0)
            assert_exact(run(c, bits, proto, dt), oracle.allreduce(bits, dt), dt, "%s N=%d n=%d split %d" % (proto, n_ranks, n, split))
        bits = make_partials(3450 + split, n_ranks, n_ranks, "bf16", 20000, "normal", 1.0)
        for threads, slices in ((64, 3), (128, 7), (512, 1)):
            c.set_option("threads", threads)
            c.set_option("slices", slices)
            assert_exact(run(c, bits, proto, dt), oracle.allreduce(bits, dt), dt, "threads %d slices %d" % (threads, slices))
        c.set_option("threads", 0)
        c.set_option("slices", 0)
        c.set_option("placement", 1)
        assert_exact(run(c, bits, proto, dt), oracle.allreduce(bits, dt), dt, "spread placement")


@pytest.mark.parametrize("xcds", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("proto", ["ll", "sentinel"])
def test_one_shot_on_the_first_xcds(proto, xcds):
    """Option local_xcds keeps a one-shot call's slices on XCDs 0 .. k-1
    (slice w on XCD w mod k, the other workgroups idle): bit-exact over
    ragged sizes and slice counts, send/recv too, and the barrier ablation
    (which keeps all eight XCDs) still right beside it."""
    dt = BF16
    with comm_for(8, dt, 64 << 10, local_xcds=xcds, threads=256) as c:
        for i, n in enumerate((1, 999, 8192, 8192 + 5, 32768)):
            bits = make_partials(3100 + xcds, i, 8, "bf16", n, "normal", 1.0)
            got = run(c, bits, proto, dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "%s n=%d xcds=%d" % (proto, n, xcds))
        c.set_option("slices", 7)
        bits = make_partials(3110 + xcds, 0, 8, "bf16", 20000, "normal", 1.0)
        assert_exact(run(c, bits, proto, dt), oracle.allreduce(bits, dt), dt, "7 slices")
        c.set_option("slices", 0)
        send = to_device(bits[3], dt)
        recv = torch.empty(20000, dtype=torch.bfloat16, device="cuda")
        c.send_recv(send, recv, proto)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(recv, dt), models.p2p_transfer(bits[3], dt, proto))
        c.set_option("barrier_ablation", 1)
        assert_exact(run(c, bits, proto, dt), oracle.allreduce(bits, dt), dt, "barrier ablation")


@pytest.mark.parametrize("xcds", [1, 2])
@pytest.mark.parametrize("proto", ["ll", "sentinel"])
def test_first_xcds_default_slices_fit_the_span(proto, xcds):
    """With local_xcds = k and no slice count given, a message that would
    take more slices than k XCDs hold at once gets fewer slices (every
    workgroup must be resident together) and is still bit-exact; an explicit
    slice count beyond that stays a refusal with nothing launched."""
    dt, n = BF16, 1 << 19  # 1 MiB per rank: 64 slices by default on all eight XCDs
    # 512-thread workgroups: a CU holds at most four, fewer than 8 x 64 / k / 32
    with comm_for(8, dt, n * 2, local_xcds=xcds, threads=512) as c:
        geo = c.geometry(n, llar.PROTOCOLS[proto])
        assert geo["slices"] < 64, geo
        bits = make_partials(3300 + xcds, 0, 8, "bf16", n, "normal", 1.0)
        assert_exact(run(c, bits, proto, dt), oracle.allreduce(bits, dt), dt, "%s xcds=%d %s" % (proto, xcds, geo))
        c.set_option("slices", 64 * xcds)  # 8 x 64 workgroups on each XCD: more than its CUs hold
        with pytest.raises(llar.LlarError):
            run(c, bits, proto, dt)


@pytest.mark.parametrize("slices", [1, 2, 3, 5, 7, 31, 33, 63, 64])
@pytest.mark.parametrize("n_ranks,n,acc", [(4, 8192, 0), (8, 8192, 0), (4, 8191, 1), (8, 3001, 0)])
def test_ll128_line_partition_every_slice_count(slices, n_ranks, n, acc):
    """The one-round LL128 kernel splits every owner's lines into slices (the
    host's reciprocal multiply where it is exact, a division otherwise).  A
    line left to no slice would never be consumed (time-out); a line in two
    slices would be counted twice.  Integer data sums exactly in any order,
    so the result must equal the oracle bit for bit, and the staging must be
    zero again afterwards."""
    dt = BF16
    with comm_for(n_ranks, dt, n * 2, slices=slices, ll128_acc=acc) as c:
        for rep in range(2):
            bits = make_partials(950 + n_ranks, rep * 100 + slices, n_ranks, "bf16", n, "integer", 1.0)
            got = run(c, bits, "ll128", dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "slices %d rep %d" % (slices, rep))
        assert not c.staging(llar.LL128).any(), "LL128 staging must be zero after every call"
