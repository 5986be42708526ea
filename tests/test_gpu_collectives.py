"""ReduceScatter and AllGather on the GPU against the oracle, through the C ABI.

ReduceScatter: outs[j] must equal oracle.reduce_scatter(...)[j] bit for bit
(binary64 rank-order sums, one rounding; NaN compared as a class).
AllGather: every output copy must equal models.all_gather(...) bit for bit
(LL: every pattern unchanged; Sentinel: the all-ones pattern arrives as the
one below).  Counts are ragged (blocks that are not whole 16-byte vectors),
rank counts 1..8, both wires, both placements, every dtype.
"""
import numpy as np
import pytest
import torch

import message_allreduce_amd as llar
import oracle
from oracle import F32, F16, BF16, models
from workloads import make_partials, random_bits

from gpu_util import CODE, TORCH_DT, assert_exact, assert_tol, run, to_device, to_host

pytestmark = pytest.mark.gpu

WIRES = ["ll", "sentinel"]
NAME = {F32: "fp32", F16: "fp16", BF16: "bf16"}


def comm_for(n_ranks, dt, max_bytes, **opts):
    c = llar.Communicator(n_ranks, TORCH_DT[dt], max_bytes)
    c.set_option("spin_timeout_us", 100_000)
    for k, v in opts.items():
        c.set_option(k, v)
    return c


def ok_status(c):
    torch.cuda.synchronize()
    st, sbits = c.device_status()
    assert st == 0, "device status %d bits %#x" % (st, sbits)


def rs_run(c, bits, dt, wire, outs=None):
    n_ranks, n = bits.shape
    cnt = n // n_ranks
    parts = [to_device(bits[r], dt) for r in range(n_ranks)]
    if outs is None:
        outs = [torch.empty(cnt, dtype=TORCH_DT[dt], device="cuda") for _ in range(n_ranks)]
    c.reduce_scatter(parts, outs, wire)
    ok_status(c)
    return [to_host(o, dt) for o in outs]


def ag_run(c, frags, dt, wire, n_outs):
    n_ranks, cnt = frags.shape
    ins = [to_device(frags[r], dt) for r in range(n_ranks)]
    outs = [torch.empty(n_ranks * cnt, dtype=TORCH_DT[dt], device="cuda") for _ in range(n_outs)]
    c.all_gather(ins, outs, wire)
    ok_status(c)
    return [to_host(o, dt) for o in outs]


def rs_inputs(seed, rep, n_ranks, cnt, dtype):
    bits = make_partials(seed, rep, n_ranks, dtype, n_ranks * cnt, "normal", 1.0)
    dt = CODE[dtype]
    bits[n_ranks - 1, ::37] = models.SENTINEL_BITS[dt]       # NaN class, and the Sentinel's own pattern
    return bits


def assert_bits_equal(got, want, what):
    if not np.array_equal(got, want):
        i = int(np.nonzero(got != want)[0][0])
        raise AssertionError("%s: %d of %d differ; first at %d: got %#x want %#x"
                             % (what, int((got != want).sum()), got.size, i, int(got[i]), int(want[i])))


COUNTS = [1, 3, 7, 8, 64, 1000, 4097]


# --------------------------------------------------------------------------- ReduceScatter
@pytest.mark.parametrize("placement", [1, 2], ids=["spread", "local"])
@pytest.mark.parametrize("wire", WIRES)
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_reduce_scatter_exact_ragged_counts(dtype, wire, placement):
    dt = CODE[dtype]
    n_ranks = 8
    with comm_for(n_ranks, dt, n_ranks * max(COUNTS) * 4, placement=placement) as c:
        for i, cnt in enumerate(COUNTS):
            bits = rs_inputs(3000 + dt, i, n_ranks, cnt, dtype)
            got = rs_run(c, bits, dt, wire)
            want = oracle.reduce_scatter(bits, dt)
            for j in range(n_ranks):
                assert_exact(got[j], want[j], dt, "%s %s count=%d rank %d" % (dtype, wire, cnt, j))
        if wire == "sentinel":
            assert (c.staging(llar.SENTINEL).view(np.uint8) == 0xFF).all()


@pytest.mark.parametrize("wire", WIRES + ["auto"])
@pytest.mark.parametrize("n_ranks", [1, 2, 3, 4, 5, 6, 7, 8])
def test_reduce_scatter_every_rank_count(n_ranks, wire):
    dt = BF16
    cnt = 333
    with comm_for(n_ranks, dt, n_ranks * cnt * 2) as c:
        for rep in range(3):
            bits = rs_inputs(3100 + n_ranks, rep, n_ranks, cnt, "bf16")
            got = rs_run(c, bits, dt, wire)
            want = oracle.reduce_scatter(bits, dt)
            for j in range(n_ranks):
                assert_exact(got[j], want[j], dt, "N=%d rep %d rank %d" % (n_ranks, rep, j))


def test_reduce_scatter_in_place():
    """outs[j] is segment j of partials[j] itself."""
    dt = F32
    n_ranks, cnt = 4, 1032           # segments start on 16-byte boundaries
    with comm_for(n_ranks, dt, n_ranks * cnt * 4) as c:
        for k, wire in enumerate(WIRES):
            bits = rs_inputs(3200, k, n_ranks, cnt, "fp32")
            parts = [to_device(bits[r], dt) for r in range(n_ranks)]
            outs = [parts[j][j * cnt:(j + 1) * cnt] for j in range(n_ranks)]
            c.reduce_scatter(parts, outs, wire)
            ok_status(c)
            want = oracle.reduce_scatter(bits, dt)
            for j in range(n_ranks):
                assert_exact(to_host(outs[j], dt), want[j], dt, "%s rank %d" % (wire, j))


def test_reduce_scatter_maximum_size():
    """N * count at the byte limits of both wires (8 MiB LL, 16 MiB Sentinel)."""
    dt = BF16
    n_ranks = 8
    for wire, total in (("ll", 8 << 20), ("sentinel", 16 << 20)):
        cnt = total // 2 // n_ranks
        with comm_for(n_ranks, dt, total) as c:
            bits = make_partials(3300, 0, n_ranks, "bf16", n_ranks * cnt, "normal", 1.0)
            got = rs_run(c, bits, dt, wire)
            want = oracle.reduce_scatter(bits, dt)
            for j in range(n_ranks):
                assert_exact(got[j], want[j], dt, "%s rank %d" % (wire, j))


@pytest.mark.parametrize("acc", [0, 1], ids=["fp32_staging", "16bit_staging"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_reduce_scatter_ll128_atomic_within_tolerance(dtype, acc):
    """The reduce-scatter half of the two-shot LL128 AllReduce: within the
    atomic protocol's tolerance, exact on small integers with binary32
    staging, lines zero after."""
    dt = CODE[dtype]
    if acc == 1 and dt == F32:
        pytest.skip("16-bit staging applies to 16-bit types only")
    n_ranks = 8
    with comm_for(n_ranks, dt, n_ranks * max(COUNTS) * 4, ll128_acc=acc) as c:
        for i, cnt in enumerate(COUNTS):
            bits = make_partials(4000 + dt, i, n_ranks, dtype, n_ranks * cnt, "normal", 0.02)
            got = rs_run(c, bits, dt, "ll128")
            want = oracle.reduce_scatter(bits, dt)
            for j in range(n_ranks):
                assert_tol(got[j], want[j], dt, "%s acc%d count=%d rank %d" % (dtype, acc, cnt, j))
            if acc == 1:
                continue  # 16-bit staging rounds partial sums of integers above 256 (bf16)
            ints = make_partials(4100 + dt, i, n_ranks, dtype, n_ranks * cnt, "integer", 1.0)
            got = rs_run(c, ints, dt, "ll128")
            want = oracle.reduce_scatter(ints, dt)
            for j in range(n_ranks):
                assert_exact(got[j], want[j], dt, "integers %s acc%d count=%d rank %d" % (dtype, acc, cnt, j))
        assert not c.staging(llar.LL128).any(), "every line is zeroed by its owner"


@pytest.mark.parametrize("n_ranks", [1, 2, 3, 5, 8])
def test_reduce_scatter_ll128_every_rank_count(n_ranks):
    dt = BF16
    cnt = 1000
    with comm_for(n_ranks, dt, n_ranks * cnt * 2) as c:
        for rep in range(3):
            bits = make_partials(4200 + n_ranks, rep, n_ranks, "bf16", n_ranks * cnt, "normal", 1.0)
            got = rs_run(c, bits, dt, "ll128")
            want = oracle.reduce_scatter(bits, dt)
            for j in range(n_ranks):
                assert_tol(got[j], want[j], dt, "N=%d rep %d rank %d" % (n_ranks, rep, j))
        assert not c.staging(llar.LL128).any()


def test_reduce_scatter_ll128_maximum_size_and_allreduce_interleaving():
    """16 MiB in total (the LL128 limit), then AllReduce and ReduceScatter
    calls sharing the LL128 staging."""
    dt = BF16
    n_ranks = 8
    total = 16 << 20
    cnt = total // 2 // n_ranks
    with comm_for(n_ranks, dt, total) as c:
        bits = make_partials(4300, 0, n_ranks, "bf16", n_ranks * cnt, "normal", 0.02)
        got = rs_run(c, bits, dt, "ll128")
        want = oracle.reduce_scatter(bits, dt)
        for j in range(n_ranks):
            assert_tol(got[j], want[j], dt, "max size rank %d" % j)
        for rep in range(6):
            small = make_partials(4301, rep, n_ranks, "bf16", n_ranks * 1024, "normal", 0.02)
            got = run(c, small, "ll128", dt)
            assert_tol(got, oracle.allreduce(small, dt), dt, "allreduce rep %d" % rep)
            got = rs_run(c, small, dt, "ll128")
            want = oracle.reduce_scatter(small, dt)
            for j in range(n_ranks):
                assert_tol(got[j], want[j], dt, "rs rep %d rank %d" % (rep, j))
        assert not c.staging(llar.LL128).any()


def test_reduce_scatter_ll128_keep_staging_matches_segment_line_model():
    """Owner o's lines hold exactly segment o: with integer data every atomic
    order stages the same sums, so the kept staging must equal, bit for bit,
    the page's line model applied to each segment, owners back to back, with
    every count at N."""
    dt = BF16
    n_ranks, cnt = 4, 100  # 100 = 3 full lines of 31 and a ragged fourth
    bits = make_partials(4400, 0, n_ranks, "bf16", n_ranks * cnt, "integer", 1.0)
    with comm_for(n_ranks, dt, n_ranks * cnt * 2, keep_staging=1) as c:
        rs_run(c, bits, dt, "ll128")
        model = np.concatenate([models.ll128_staging_image(bits[:, o * cnt:(o + 1) * cnt], dt, F32)
                                for o in range(n_ranks)])
        lines = model.shape[0]
        stage = c.staging(llar.LL128)[: lines * 128].view(np.float32).reshape(lines, 32)
        assert np.array_equal(stage.astype(np.float64), model)
        assert (stage[:, 0] == n_ranks).all()
        c.set_option("keep_staging", 0)


# --------------------------------------------------------------------------- AllGather
@pytest.mark.parametrize("replicated", [False, True], ids=["rank0", "every_rank"])
@pytest.mark.parametrize("placement", [1, 2], ids=["spread", "local"])
@pytest.mark.parametrize("wire", WIRES)
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_all_gather_exact_ragged_counts(dtype, wire, placement, replicated):
    dt = CODE[dtype]
    n_ranks = 8
    n_outs = n_ranks if replicated else 1
    with comm_for(n_ranks, dt, n_ranks * max(COUNTS) * 4, placement=placement) as c:
        for i, cnt in enumerate(COUNTS):
            frags = np.stack([random_bits(3400 + dt, 8 * i + r, cnt, dtype) for r in range(n_ranks)])
            frags[3, ::5] = models.SENTINEL_BITS[dt]
            got = ag_run(c, frags, dt, wire, n_outs)
            want = models.all_gather(list(frags), dt, wire)
            for j in range(n_outs):
                assert_bits_equal(got[j], want, "%s %s count=%d copy %d" % (dtype, wire, cnt, j))
        if wire == "sentinel":
            assert (c.staging(llar.SENTINEL).view(np.uint8) == 0xFF).all()


@pytest.mark.parametrize("wire", WIRES)
@pytest.mark.parametrize("n_ranks", [1, 2, 3, 4, 5, 6, 7, 8])
def test_all_gather_every_rank_count(n_ranks, wire):
    dt = F16
    cnt = 517
    with comm_for(n_ranks, dt, n_ranks * cnt * 2) as c:
        for rep in range(3):
            frags = np.stack([random_bits(3500 + n_ranks, 8 * rep + r, cnt, "fp16") for r in range(n_ranks)])
            got = ag_run(c, frags, dt, wire, n_ranks)
            want = models.all_gather(list(frags), dt, wire)
            for j in range(n_ranks):
                assert_bits_equal(got[j], want, "N=%d rep %d copy %d" % (n_ranks, rep, j))


def test_all_gather_maximum_size_every_copy():
    """N * count at the Sentinel's 16 MiB limit, every rank's copy."""
    dt = BF16
    n_ranks = 8
    total = 16 << 20
    cnt = total // 2 // n_ranks
    with comm_for(n_ranks, dt, total) as c:
        frags = np.stack([random_bits(3450, r, cnt, "bf16") for r in range(n_ranks)])
        got = ag_run(c, frags, dt, "sentinel", n_ranks)
        want = models.all_gather(list(frags), dt, "sentinel")
        for j in range(n_ranks):
            assert_bits_equal(got[j], want, "copy %d" % j)


# --------------------------------------------------------------------------- composition, epochs, failures
@pytest.mark.parametrize("wire", WIRES)
def test_reduce_scatter_then_all_gather_is_the_allreduce(wire):
    """The two halves of the two-shot AllReduce, run one after the other,
    leave every rank with the AllReduce result."""
    dt = BF16
    n_ranks, cnt = 8, 1024            # 8192 bf16 = 16 KiB, the TP hidden state
    with comm_for(n_ranks, dt, n_ranks * cnt * 2) as c:
        for rep in range(20):
            bits = make_partials(3600, rep, n_ranks, "bf16", n_ranks * cnt, "normal", 1.0)
            parts = [to_device(bits[r], dt) for r in range(n_ranks)]
            segs = [torch.empty(cnt, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
            full = [torch.empty(n_ranks * cnt, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
            c.reduce_scatter(parts, segs, wire)
            c.all_gather(segs, full, wire)
            ok_status(c)
            want = oracle.allreduce(bits, dt)
            for j in range(n_ranks):
                assert_exact(to_host(full[j], dt), want, dt, "rep %d copy %d" % (rep, j))


def test_collectives_interleaved_with_allreduce_and_send_recv():
    """All calls share the staging and the epoch sequence."""
    dt = F32
    n_ranks, cnt = 4, 777
    with comm_for(n_ranks, dt, n_ranks * cnt * 4) as c:
        for rep in range(24):
            wire = WIRES[rep % 2]
            bits = make_partials(3700, rep, n_ranks, "fp32", n_ranks * cnt, "normal", 1.0)
            got = run(c, bits, wire, dt)
            assert_exact(got, oracle.allreduce(bits, dt), dt, "allreduce rep %d" % rep)
            got = rs_run(c, bits, dt, wire)
            want = oracle.reduce_scatter(bits, dt)
            for j in range(n_ranks):
                assert_exact(got[j], want[j], dt, "rs rep %d rank %d" % (rep, j))
            frags = bits[:, :cnt].copy()
            got = ag_run(c, frags, dt, wire, n_ranks if rep % 3 else 1)
            for g in got:
                assert_bits_equal(g, models.all_gather(list(frags), dt, wire), "ag rep %d" % rep)
            recv = torch.empty(cnt, dtype=torch.float32, device="cuda")
            c.send_recv(to_device(frags[1], dt), recv, wire)
            ok_status(c)
            assert_bits_equal(to_host(recv, dt), models.p2p_transfer(frags[1], dt, wire), "p2p rep %d" % rep)
        assert (c.staging(llar.SENTINEL).view(np.uint8) == 0xFF).all()


def test_collectives_graph_capture_replays():
    """Captured calls read the device-resident epoch: every replay is a new
    call.  Eager work between replays; every replay checked."""
    dt = BF16
    n_ranks, cnt = 8, 1024
    c = comm_for(n_ranks, dt, n_ranks * cnt * 2)
    try:
        parts = [torch.empty(n_ranks * cnt, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
        segs = {w: [torch.empty(cnt, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)] for w in WIRES}
        full = {w: [torch.empty(n_ranks * cnt, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
                for w in WIRES}
        bits0 = make_partials(3800, 0, n_ranks, "bf16", n_ranks * cnt)
        for r in range(n_ranks):
            parts[r].copy_(to_device(bits0[r], dt))

        def calls():
            for w in WIRES:
                c.reduce_scatter(parts, segs[w], w)
                c.all_gather(segs[w], full[w], w)

        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        torch.cuda.synchronize()
        for rep in range(1, 6):
            bits = make_partials(3800, rep, n_ranks, "bf16", n_ranks * cnt)
            for r in range(n_ranks):
                parts[r].copy_(to_device(bits[r], dt))
            torch.cuda.synchronize()
            g.replay()
            ok_status(c)
            want = oracle.allreduce(bits, dt)
            for w in WIRES:
                for j in range(n_ranks):
                    assert_exact(to_host(full[w][j], dt), want, dt, "replay %d %s copy %d" % (rep, w, j))
            got = rs_run(c, bits, dt, "ll")
            want_rs = oracle.reduce_scatter(bits, dt)
            for j in range(n_ranks):
                assert_exact(got[j], want_rs[j], dt, "eager after replay %d" % rep)
    finally:
        c.close()


@pytest.mark.parametrize("op,wire", [("reduce_scatter", "ll"), ("reduce_scatter", "sentinel"),
                                     ("reduce_scatter", "ll128"), ("all_gather", "ll"), ("all_gather", "sentinel")])
def test_collectives_lost_contribution_times_out_and_recovers(op, wire):
    """A rank whose sends are dropped (forced from the host) makes the other
    receivers' bounded polls expire; after a reset the next call works."""
    dt = BF16
    n_ranks, cnt = 4, 2048
    bits = make_partials(3900, 0, n_ranks, "bf16", n_ranks * cnt)
    with comm_for(n_ranks, dt, n_ranks * cnt * 2) as c:
        c.set_option("spin_timeout_us", 2000)
        c.set_option("debug_drop_rank", 2)
        if op == "reduce_scatter":
            parts = [to_device(bits[r], dt) for r in range(n_ranks)]
            outs = [torch.empty(cnt, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
            c.reduce_scatter(parts, outs, wire)
        else:
            frags = [to_device(bits[r, :cnt], dt) for r in range(n_ranks)]
            outs = [torch.empty(n_ranks * cnt, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
            c.all_gather(frags, outs, wire)
        torch.cuda.synchronize()
        st, sbits = c.device_status()
        assert st == -5 and (sbits & 1), (st, sbits)
        c.clear_device_status()
        c.set_option("debug_drop_rank", -1)
        c.set_option("spin_timeout_us", 100_000)
        got = rs_run(c, bits, dt, wire)
        want = oracle.reduce_scatter(bits, dt)
        for j in range(n_ranks):
            (assert_tol if wire == "ll128" else assert_exact)(got[j], want[j], dt, "after recovery rank %d" % j)


def test_collectives_argument_errors():
    dt = BF16
    n_ranks, cnt = 4, 256
    with comm_for(n_ranks, dt, n_ranks * cnt * 2) as c:
        parts = [torch.zeros(n_ranks * cnt, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
        outs = [torch.zeros(cnt, dtype=torch.bfloat16, device="cuda") for _ in range(n_ranks)]
        p = [t.data_ptr() for t in parts]
        o = [t.data_ptr() for t in outs]
        for proto in (llar.LL128_PIPELINED, llar.SENTINEL_PIPELINED, 9):
            assert llar.llar_reduce_scatter(c.h, p, o, cnt, BF16, proto, 0) == -1
        for proto in (llar.LL128, llar.LL128_PIPELINED, llar.SENTINEL_PIPELINED, 9):
            assert llar.llar_all_gather(c.h, o, p, cnt, BF16, proto, 0) == -1
        assert llar.llar_reduce_scatter(c.h, p, o, cnt + 1, BF16, llar.LL, 0) == -1      # beyond max_bytes
        assert llar.llar_reduce_scatter(c.h, p, o, cnt, F32, llar.LL, 0) == -1          # wrong dtype
        assert llar.llar_reduce_scatter(c.h, p, o[:1] + [o[1] + 2] + o[2:], cnt, BF16, llar.LL, 0) == -1
        assert llar.llar_all_gather(c.h, o, p[:2], cnt, BF16, llar.LL, 0) == -1         # n_outs not 1 or N
        assert llar.llar_reduce_scatter(c.h, p, o, 0, BF16, llar.LL, 0) == 0            # no-op
        assert llar.llar_all_gather(c.h, o, p, 0, BF16, llar.LL, 0) == 0
        ok_status(c)


# --------------------------------------------------------------------------- LL receiver lanes
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("n_ranks", [8, 3, 2])
def test_reduce_scatter_ll_half_line_switch_bit_exact(n_ranks, dtype):
    """The LL ReduceScatter's receiver gives each lane one 4-byte half line
    while every half of its slice has a lane (one 256-thread slice: blocks up
    to 64 vectors, 1 KiB), and whole 8-byte units per lane beyond.  Blocks on
    both sides of that switch, ragged ones included (partial last vector, a
    last half holding one 16-bit element), bit-exact against the oracle with
    fresh inputs each repetition."""
    dt = CODE[dtype]
    esize = 4 if dtype == "fp32" else 2
    blocks = sorted({1024 - 16, 1024 - esize, 1024, 1024 + esize, 1024 + 16, 2 * 1024 + esize, 8, esize})
    with comm_for(n_ranks, dt, n_ranks * 16384, threads=256, slices=1) as c:
        for blk in blocks:
            cnt = blk // esize
            for rep in range(2):
                bits = rs_inputs(5100 + n_ranks, rep * 10000 + blk, n_ranks, cnt, dtype)
                got = rs_run(c, bits, dt, "ll")
                want = oracle.reduce_scatter(bits, dt)
                for j in range(n_ranks):
                    assert_exact(got[j], want[j], dt, "N=%d %s block %d B rep %d rank %d" % (n_ranks, dtype, blk, rep, j))
