"""Pins for the protocol models (LL line, Sentinel buffer, LL128 atomic line,
double buffering with implicit credits) against the figures the page prints,
closed forms, exhaustive enumeration and model checking."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import F32, F16, BF16, models

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def pages():
    with open(os.path.join(GOLDEN, "pages_figures.json")) as f:
        return json.load(f)


# --------------------------------------------------------------------------- SoL
def test_sol_floor_reproduces_page_figure(pages):
    s = pages["sol"]
    assert models.sol_floor(s["l2_round_trip_us"], s["remote_write_us"]) == pytest.approx(s["bound_us"], abs=1e-12)


def test_alpha_beta_fit_recovers_synthetic_line():
    sizes = [2**k for k in range(7, 27)]
    alpha, beta = 3.2, 1.7e-4
    t = [alpha + beta * s for s in sizes]
    a, b = models.fit_alpha_beta(sizes, t)
    assert a == pytest.approx(alpha, rel=1e-9) and b == pytest.approx(beta, rel=1e-9)


# --------------------------------------------------------------------------- LL
def test_ll_line_is_one_16_byte_store_of_8_flag_and_8_data_bytes(pages):
    ll = pages["ll"]
    assert models.LL_LINE_BYTES == ll["store_bytes"] == ll["flag_bytes"] + ll["data_bytes"]
    assert models.LL_PAYLOAD_BYTES == ll["data_bytes"]


@pytest.mark.parametrize("nbytes", [8, 128, 16384, 1 << 20])
def test_ll_staging_is_exactly_double(pages, nbytes):
    assert models.ll_staging_bytes(nbytes) == pages["ll"]["staging_factor"] * nbytes


def test_ll_pack_unpack_roundtrip_and_stale_detection():
    g = np.random.default_rng(0)
    payload = g.integers(0, 2**32, size=(1000, 2), dtype=np.uint64).astype(np.uint32)
    for e in [1, 2, 7, 0xFFFFFFFF]:
        lines = models.ll_pack(payload, e)
        valid, back = models.ll_unpack(lines, e)
        assert valid.all() and np.array_equal(back, payload)
        # last call's epoch is stale
        prev = e - 1 if e > 1 else 0xFFFFFFFF
        valid_prev, _ = models.ll_unpack(models.ll_pack(payload, prev), e)
        assert not valid_prev.any()
        # a half-updated line (one 8-byte half from the old epoch) is rejected
        torn = lines.copy()
        torn[:, 3] = prev
        assert not models.ll_unpack(torn, e)[0].any()
        torn = lines.copy()
        torn[:, 1] = prev
        assert not models.ll_unpack(torn, e)[0].any()
    # a zeroed buffer is never valid
    assert not models.ll_unpack(np.zeros((4, 4), np.uint32), 1)[0].any()


def test_epoch_sequence_skips_zero():
    """Host epochs: 1 .. 2^31-1, then 1 again; device epochs: the same with
    bit 31 set; the two ranges never meet and neither holds 0 (the state of a
    zeroed line)."""
    assert models.next_epoch(1) == 2
    assert models.next_epoch(0x7FFFFFFF) == 1
    assert models.next_device_epoch(0xFFFFFFFF) == 0x80000001
    assert models.next_device_epoch(0x80000001) == 0x80000002
    assert models.epoch_wraps(0x7FFFFFFF) and models.epoch_wraps(0xFFFFFFFF)
    assert not models.epoch_wraps(0x7FFFFFFE) and not models.epoch_wraps(0x80000001)
    for start, step in ((0x7FFFFFF0, models.next_epoch), (0xFFFFFFF0, models.next_device_epoch)):
        e, seen = start, []
        for _ in range(40):
            e = step(e)
            assert e != 0
            seen.append(e)
        # one wrap inside the window: 15 values before it, then 1.., all distinct within a cycle
        assert len(set(seen)) == 40
        host = step is models.next_epoch
        assert all(((x & 0x80000000) == 0) == host for x in seen)


def test_ll_region_reuse_across_the_epoch_wrap():
    """The LL flag is the only arrival signal (LL paragraph), so a line that
    carries the current epoch must have been written by the current call.
    On a short cycle (last epoch 7) a large message, then small ones for the
    rest of the cycle, then the large one again: without clearing at the
    wrap the large message's tail lines still carry their old epoch when it
    comes round, and would be accepted before the producer writes them;
    clearing at the wrap leaves none, over many cycles and random sizes."""
    r = models.LLRegion(64, last=7, clear_at_wrap=False)
    r.call(64)                   # epoch 1 writes every line
    for _ in range(6):           # epochs 2..7 write only the first 4 lines
        r.call(4)
    assert r.call(64) == 60      # epoch 1 again: 60 stale lines look fresh
    rng = np.random.default_rng(7)
    for clear in (True, False):
        r = models.LLRegion(64, last=7, clear_at_wrap=clear)
        r.call(64)
        for _ in range(6):
            r.call(4)
        r.call(64)
        for _ in range(2000):
            r.call(int(rng.integers(1, 65)))
        assert (r.stale_hits == 0) == clear


def test_ll_payload_padding_is_zero_and_bytes_are_preserved():
    parts = np.arange(13, dtype=np.uint16)  # 26 bytes -> 4 payloads
    w = models.ll_payload_words(parts)
    assert w.shape == (4, 2)
    raw = w.reshape(-1).view(np.uint8)
    assert np.array_equal(raw[:26], parts.view(np.uint8)) and not raw[26:].any()


# --------------------------------------------------------------------------- Sentinel
@pytest.mark.parametrize("dt", [F16, BF16])
def test_sentinel_canonicalization_exhaustive_16bit(dt):
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    c = models.sentinel_canon(allb, dt)
    s = models.SENTINEL_BITS[dt]
    assert not (c == s).any()                          # never equals the sentinel
    changed = c != allb
    assert changed.sum() == 1 and allb[changed][0] == s  # only the sentinel moves
    assert oracle.is_nan_bits(c[changed], dt).all()      # and stays a NaN
    assert (c[changed] & 0x8000).all()                   # a negative one
    # the sentinel itself is a negative NaN ("e.g. -NaN")
    assert oracle.is_nan_bits(np.array([s], np.uint16), dt)[0] and (s & 0x8000)


def test_sentinel_fp32_specials_and_random():
    s = models.SENTINEL_BITS[F32]
    assert oracle.is_nan_bits(np.array([s], np.uint32), F32)[0] and (s >> 31)
    # the x86 default NaN, the canonical quiet NaN, Inf and zeros are not it
    for b in [0x7FC00000, 0xFFC00000, 0x7F800000, 0x80000000, 0]:
        assert b != s
    g = np.random.default_rng(1)
    b = g.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    b[::100_000] = s
    c = models.sentinel_canon(b, F32)
    assert not (c == s).any()
    assert np.array_equal(c[b != s], b[b != s])
    assert oracle.is_nan_bits(c[b == s], F32).all()


@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_sentinel_canonicalization_does_not_change_the_sum(dt):
    g = np.random.default_rng(2 + dt)
    bits = oracle.round_to(g.standard_normal((4, 5000)), dt)
    bits[1, ::97] = models.SENTINEL_BITS[dt]
    want = oracle.allreduce(bits, dt)
    canon = np.stack([models.sentinel_canon(bits[r], dt) for r in range(4)])
    got = oracle.allreduce(canon, dt)
    assert oracle.same_result(got, want, dt).all()


def test_sentinel_reset_and_readiness():
    for dt in (F32, F16, BF16):
        buf = models.sentinel_reset(64, dt)
        assert not models.sentinel_ready(buf, dt).any()
        buf[3] = 0
        assert models.sentinel_ready(buf, dt)[3] and models.sentinel_ready(buf, dt).sum() == 1


def test_workload_3_is_sentinel_free():
    from workloads import WORKLOADS, workload_partials
    w = WORKLOADS[3]
    for rep in range(3):
        p = workload_partials(w, rep)
        assert not (p == models.SENTINEL_BITS[F16]).any()


# --------------------------------------------------------------------------- point-to-point
@pytest.mark.parametrize("dt", [F16, BF16])
def test_p2p_ll_delivers_every_16bit_pattern_unchanged(dt):
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for n in (65536, 65535, 1, 3):       # ragged: a last line only partly filled
        got = models.p2p_transfer(allb[:n], dt, "ll", epoch=7)
        assert got.dtype == allb.dtype and np.array_equal(got, allb[:n])


def test_p2p_ll_delivers_fp32_bits_unchanged():
    g = np.random.default_rng(11)
    b = g.integers(0, 2**32, size=100_003, dtype=np.uint64).astype(np.uint32)
    b[:4] = [models.SENTINEL_BITS[F32], 0x7FC00000, 0x80000000, 0x7F800000]
    assert np.array_equal(models.p2p_transfer(b, F32, "ll", epoch=0xFFFFFFFF), b)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_p2p_sentinel_moves_only_the_sentinel_exhaustive_16bit(dt):
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = models.p2p_transfer(allb, dt, "sentinel")
    s = models.SENTINEL_BITS[dt]
    moved = got != allb
    assert moved.sum() == 1 and allb[moved][0] == s
    assert oracle.is_nan_bits(got[moved], dt).all() and (got[moved] & 0x8000).all()


@pytest.mark.parametrize("dt", [F32, F16, BF16])
@pytest.mark.parametrize("wire", ["ll", "sentinel"])
def test_p2p_equals_a_two_rank_sum_with_negative_zero(dt, wire):
    # x + (-0) == x for every x (IEEE 754 section 6.3), so a copy is the
    # two-rank AllReduce of the message and a negative-zero partial; the C
    # oracle's binary64 sum checks the model independently (NaN as a class)
    g = np.random.default_rng(40 + dt)
    nb = {F32: 32, F16: 16, BF16: 16}[dt]
    b = g.integers(0, 2**nb, size=20_001, dtype=np.uint64).astype(oracle.BITS_DTYPE[dt])
    b[::101] = models.SENTINEL_BITS[dt]
    neg0 = np.full_like(b, 1 << (nb - 1))
    want = oracle.allreduce(np.stack([neg0, b]), dt)
    got = models.p2p_transfer(b, dt, wire)
    assert oracle.same_result(got, want, dt).all()


# --------------------------------------------------------------------------- ReduceScatter / AllGather
@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_reduce_scatter_segments_tile_the_allreduce(dt):
    # the N segments, back to back, are the AllReduce of the whole message
    g = np.random.default_rng(60 + dt)
    for n_ranks, c in [(1, 5), (3, 7), (8, 129)]:
        bits = oracle.round_to(g.standard_normal((n_ranks, n_ranks * c)) * 8.0, dt)
        segs = oracle.reduce_scatter(bits, dt)
        assert len(segs) == n_ranks and all(s.size == c for s in segs)
        assert oracle.same_result(np.concatenate(segs), oracle.allreduce(bits, dt), dt).all()


def test_reduce_scatter_brute_force_against_pure_python():
    # tiny case, element by element with the pure-Python rational rounding
    from oracle import pyref
    g = np.random.default_rng(61)
    for dt in (F32, F16, BF16):
        bits = oracle.round_to(g.standard_normal((3, 6)) * 1e3, dt)
        segs = oracle.reduce_scatter(bits, dt)
        for j in range(3):
            cols = [[int(bits[r, 2 * j + i]) for i in range(2)] for r in range(3)]
            assert [int(x) for x in segs[j]] == pyref.allreduce(cols, dt)


def test_reduce_scatter_keeps_the_right_segment():
    # rank r holds r+1 in segment j = r only: segment j sums to j+1
    n_ranks, c = 4, 3
    parts = np.zeros((n_ranks, n_ranks * c), np.float32)
    for r in range(n_ranks):
        parts[r, r * c:(r + 1) * c] = r + 1
    segs = oracle.reduce_scatter(oracle.as_bits(parts, F32), F32)
    for j in range(n_ranks):
        assert (oracle.decode(segs[j], F32) == j + 1).all()
    with pytest.raises(ValueError):
        oracle.reduce_scatter(np.zeros((3, 7), np.uint32), F32)


@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_all_gather_rebuilds_the_sharded_tensor(dt):
    g = np.random.default_rng(62 + dt)
    nb = 32 if dt == F32 else 16
    full = g.integers(0, 2**nb, size=8 * 37, dtype=np.uint64).astype(oracle.BITS_DTYPE[dt])
    frags = np.split(full, 8)
    assert np.array_equal(models.all_gather(frags, dt, "ll"), full)
    got = models.all_gather(frags, dt, "sentinel")
    s = models.SENTINEL_BITS[dt]
    assert np.array_equal(got[full != s], full[full != s]) and not (got == s).any()
    assert oracle.is_nan_bits(got[full == s], dt).all()


# --------------------------------------------------------------------------- LL128
def test_ll128_lane_grouping_matches_page(pages):
    p = pages["ll128"]
    assert models.LL128_LINE_BYTES == p["line_bytes"]
    assert models.LL128_LINE_BYTES // models.LL128_LANE_BYTES == p["threads_per_line"] == models.LL128_LANES


def test_ll128_waste_recomputed_from_layout(pages):
    p = pages["ll128"]
    w16 = models.LL128Geometry(8192, 4, 2).waste
    w32 = models.LL128Geometry(8192, 4, 4).waste
    assert w16 == 1 / 64 and w32 == 1 / 32
    assert abs(w16 - p["waste_fp16_approx"]) <= p["waste_tolerance_of_approx"]
    assert abs(w32 - p["waste_fp32_approx"]) <= p["waste_tolerance_of_approx"]


def test_ll128_geometry_closed_forms_for_the_workloads():
    g2 = models.LL128Geometry(8192, 4, 2)          # 16 KiB bf16, 16-bit staging
    assert g2.k == 63 and g2.lines == 131 and g2.staging_bytes == 16768
    g2f = models.LL128Geometry(8192, 4, 4)         # same, fp32 staging
    assert g2f.k == 31 and g2f.lines == 265 and g2f.staging_bytes == 33920
    g4 = models.LL128Geometry(16384, 8, 4)         # one 64 KiB fp32 chunk
    assert g4.lines == 529 and g4.staging_bytes == 67712
    # owner ranges tile the lines exactly, balanced within one line
    for g in (g2, g2f, g4):
        spans = [g.owner_range(s) for s in range(g.n_ranks)]
        assert spans[0][0] == 0 and spans[-1][1] == g.lines
        assert all(a[1] == b[0] for a, b in zip(spans, spans[1:]))
        sizes = [b - a for a, b in spans]
        assert max(sizes) - min(sizes) <= 1


@pytest.mark.parametrize("n_ranks", [2, 4, 8])
def test_ll128_staging_per_owner_is_about_d_over_n(n_ranks):
    n = 8192
    g = models.LL128Geometry(n, n_ranks, 2)
    d = n * 2
    per_owner = g.max_owner_staging_bytes()
    assert per_owner <= (d / n_ranks) * (g.slots / g.k) + models.LL128_LINE_BYTES


def test_ll128_element_mapping_is_a_bijection_onto_data_slots():
    g = models.LL128Geometry(1000, 4, 4)
    seen = set()
    for e in range(1000):
        line, slot = g.line_slot(e)
        assert 1 <= slot < g.slots and 0 <= line < g.lines
        seen.add((line, slot))
    assert len(seen) == 1000


def ints_bits(seed, n_ranks, n, dt):
    g = np.random.default_rng(seed)
    return oracle.round_to(g.integers(-50, 51, size=(n_ranks, n)).astype(np.float64), dt)


@pytest.mark.parametrize("dt,acc", [(BF16, BF16), (F16, F16), (BF16, F32), (F32, F32)])
def test_ll128_flag_counts_contributions_exactly(dt, acc):
    parts = ints_bits(3, 4, 300, dt)
    for k in range(1, 5):
        img = models.ll128_staging_image(parts[:k], dt, acc)
        assert (img[:, 0] == k).all()
    # a missing contribution leaves N-1, a duplicate gives N+1
    full = models.ll128_staging_image(parts, dt, acc)
    assert (full[:, 0] == 4).all()
    dup = models.ll128_staging_image(parts, dt, acc, order=[0, 1, 2, 3, 2])
    assert (dup[:, 0] == 5).all()


@pytest.mark.parametrize("dt,acc", [(BF16, BF16), (F16, F16), (BF16, F32), (F16, F32), (F32, F32)])
def test_ll128_integer_data_is_exact_in_every_order(dt, acc):
    parts = ints_bits(4, 4, 200, dt)
    want = oracle.allreduce(parts, dt)
    for order in itertools.permutations(range(4)):
        img = models.ll128_staging_image(parts, dt, acc, order)
        got = models.ll128_result(img, 200, dt)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("dt,acc", [(BF16, BF16), (F16, F16), (BF16, F32), (F16, F32), (F32, F32)])
def test_ll128_any_order_within_error_bound(dt, acc):
    g = np.random.default_rng(5 + dt + 3 * acc)
    parts = oracle.round_to(g.standard_normal((4, 2000)) * 0.02, dt)
    exact = oracle.sum_f64(parts, dt)  # binary64 sum of <=4 such values is exact here
    bound = models.ll128_error_bound(parts, dt, acc)
    for order in itertools.permutations(range(4)):
        img = models.ll128_staging_image(parts, dt, acc, order)
        got = oracle.decode(models.ll128_result(img, 2000, dt), dt)
        assert (np.abs(got - exact) <= bound).all()


def test_ll128_error_bound_is_not_vacuous():
    # the bound must be tight enough that a dropped rank breaks it
    g = np.random.default_rng(9)
    parts = oracle.round_to(g.standard_normal((4, 2000)) * 0.02, BF16)
    exact = oracle.sum_f64(parts, BF16)
    bound = models.ll128_error_bound(parts, BF16, F32)
    img = models.ll128_staging_image(parts[:3], BF16, F32)
    got = oracle.decode(models.ll128_result(img, 2000, BF16), BF16)
    assert (np.abs(got - exact) > bound).mean() > 0.5


# --------------------------------------------------------------------------- credits
def test_pipeline_double_buffer_is_safe_exhaustively_n2():
    r = models.check_pipeline(n_ranks=2, slices=1, chunks=3)
    assert not r.violations and r.deadlocks == 0 and r.terminal_ok == 1 and r.states > 20


def test_pipeline_double_buffer_is_safe_exhaustively_n3():
    r = models.check_pipeline(n_ranks=3, slices=1, chunks=3)
    assert not r.violations and r.deadlocks == 0 and r.terminal_ok == 1


def test_pipeline_two_slices_is_safe():
    r = models.check_pipeline(n_ranks=2, slices=2, chunks=3)
    assert not r.violations and r.deadlocks == 0


def test_pipeline_single_buffer_overwrites():
    r = models.check_pipeline(n_ranks=2, slices=1, chunks=3, parities=1)
    assert any(v[0] == "overwrite" for v in r.violations)


def test_pipeline_without_credit_overwrites():
    r = models.check_pipeline(n_ranks=2, slices=1, chunks=4, run_ahead=True)
    assert any(v[0] == "overwrite" for v in r.violations)


def test_pipeline_split_producer_consumer_is_safe_exhaustively():
    for n_ranks, slices, chunks in [(2, 1, 4), (3, 1, 3), (2, 2, 3)]:
        r = models.check_pipeline(n_ranks, slices, chunks, split=True)
        assert not r.violations and r.deadlocks == 0 and r.terminal_ok == 1, (n_ranks, slices, chunks, r)


def test_pipeline_split_with_one_buffer_overwrites():
    r = models.check_pipeline(2, 1, 3, parities=1, split=True)
    assert any(v[0] == "overwrite" for v in r.violations)


def test_pipeline_split_with_a_weaker_credit_overwrites():
    # emitting chunk c after the own consumer finished only chunk c-2
    r = models.check_pipeline(3, 1, 3, split=True, credit_lag=1)
    assert any(v[0] == "overwrite" for v in r.violations)


def test_pipeline_credit_lag_needs_two_lag_plus_two_buffers():
    # producing chunk c once the own consumer finished chunk c-1-lag is safe
    # exactly when the buffer count is at least 2*lag + 2
    for shape in [(2, 1, 6), (3, 1, 5), (2, 2, 5)]:
        ok = models.check_pipeline(*shape, split=True, parities=4, credit_lag=1)
        assert not ok.violations and ok.deadlocks == 0 and ok.terminal_ok == 1
        bad = models.check_pipeline(*shape, split=True, parities=3, credit_lag=1)
        assert any(v[0] == "overwrite" for v in bad.violations)


def test_owner_credit_is_safe_exhaustively():
    # every owner publishes its progress; a producer stores chunk c once every
    # owner consumed every chunk <= c - B: safe for any B >= 1 and any number
    # of consumer waves taking whole chunks round-robin
    for shape in [dict(n_ranks=2, slices=1, chunks=4, buffers=1), dict(n_ranks=2, slices=1, chunks=4, buffers=2, cons_waves=2),
                  dict(n_ranks=2, slices=1, chunks=5, buffers=3, cons_waves=2), dict(n_ranks=3, slices=1, chunks=3, buffers=2, cons_waves=2),
                  dict(n_ranks=2, slices=2, chunks=3, buffers=2, cons_waves=2), dict(n_ranks=2, slices=1, chunks=4, buffers=2, cons_waves=3)]:
        r = models.check_owner_credit(**shape)
        assert not r.violations and r.deadlocks == 0 and r.terminal_ok == 1 and r.states > 10, (shape, r)


def test_owner_credit_needs_the_wave_order_check():
    # a consumer wave that polls chunk c before another wave consumed chunk
    # c - B finds the old chunk's full line and takes it for its own
    for shape in [dict(n_ranks=2, slices=1, chunks=3, buffers=1, cons_waves=2),
                  dict(n_ranks=2, slices=1, chunks=3, buffers=2, cons_waves=3)]:
        r = models.check_owner_credit(**shape, wave_order=False)
        assert any(v[0] == "stale read" for v in r.violations), shape


def test_owner_credit_from_the_own_consumer_alone_overwrites():
    # the same buffer count with only the producer's own consumer as credit
    # lets a fast rank overwrite a slower owner's unconsumed chunk
    for n_ranks in (2, 3):
        r = models.check_owner_credit(n_ranks=n_ranks, slices=1, chunks=4, buffers=2, credit="own")
        assert any(v[0] == "overwrite" for v in r.violations), n_ranks


def test_workgroup_credit_with_consumer_groups_is_safe():
    # the workgroup pipeline with its chunks dealt to G consumer groups
    # (group g takes chunks g, g + G, ...): with B >= 2 lag + 2 buffers and G
    # dividing B, no overwrite, no stale read and no deadlock, with no
    # explicit wave-order wait (the group that polls chunk c consumed c - B)
    for shape in [dict(n_ranks=2, slices=1, chunks=6, buffers=4, cons_waves=2, lag=1),
                  dict(n_ranks=3, slices=1, chunks=5, buffers=4, cons_waves=2, lag=1),
                  dict(n_ranks=2, slices=1, chunks=7, buffers=6, cons_waves=3, lag=2),
                  dict(n_ranks=2, slices=1, chunks=6, buffers=4, cons_waves=4, lag=1),
                  dict(n_ranks=2, slices=1, chunks=5, buffers=4, cons_waves=1, lag=1),
                  dict(n_ranks=3, slices=1, chunks=4, buffers=2, cons_waves=2, lag=0)]:
        r = models.check_owner_credit(**shape, credit="workgroup", wave_order=False)
        assert not r.violations and r.deadlocks == 0 and r.terminal_ok == 1, (shape, r)


def test_workgroup_credit_with_producer_groups_is_safe():
    # producers in PG groups (group p stores chunks p, p + PG, ..., so chunks
    # land out of order) under the same credit: still no overwrite, no stale
    # read, no deadlock; one buffer too few or a lag too large still overwrites
    for shape in [dict(n_ranks=2, slices=1, chunks=6, buffers=4, cons_waves=2, lag=1, prod_groups=2),
                  dict(n_ranks=3, slices=1, chunks=5, buffers=4, cons_waves=2, lag=1, prod_groups=2),
                  dict(n_ranks=2, slices=1, chunks=7, buffers=6, cons_waves=2, lag=2, prod_groups=3),
                  dict(n_ranks=2, slices=1, chunks=6, buffers=4, cons_waves=1, lag=1, prod_groups=2)]:
        r = models.check_owner_credit(**shape, credit="workgroup", wave_order=False)
        assert not r.violations and r.deadlocks == 0 and r.terminal_ok == 1, (shape, r)
    for shape in [dict(n_ranks=2, slices=1, chunks=6, buffers=3, cons_waves=1, lag=1, prod_groups=2),
                  dict(n_ranks=3, slices=1, chunks=6, buffers=4, cons_waves=2, lag=2, prod_groups=2)]:
        r = models.check_owner_credit(**shape, credit="workgroup", wave_order=False)
        assert any(v[0] == "overwrite" for v in r.violations), shape


def test_workgroup_credit_with_consumer_groups_failure_modes():
    # one buffer too few overwrites; groups that do not divide B read a
    # previous chunk's full line as their own; a lag too large for B overwrites
    cases = [(dict(n_ranks=2, slices=1, chunks=6, buffers=3, cons_waves=1, lag=1), "overwrite"),
             (dict(n_ranks=2, slices=1, chunks=6, buffers=4, cons_waves=3, lag=1), "stale read"),
             (dict(n_ranks=3, slices=1, chunks=6, buffers=4, cons_waves=2, lag=2), "overwrite")]
    for shape, kind in cases:
        r = models.check_owner_credit(**shape, credit="workgroup", wave_order=False)
        assert any(v[0] == kind for v in r.violations), (shape, r.violations[:2])
