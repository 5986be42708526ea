"""Pins for the CPU oracle (reduction result): it is checked against things
other than itself -- numpy/struct conversions, exact rational rounding,
hand-derived worked examples, closed forms and invariants."""
import itertools
import json
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle import F32, F16, BF16, pyref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def random_doubles(seed, n):
    """Doubles spanning every binade of interest, plus exact ties of the
    target grids (multiples of fine powers of two)."""
    g = rng(seed)
    mant = g.random(n) + 1.0
    expo = g.integers(-160, 140, size=n)
    sign = np.where(g.random(n) < 0.5, -1.0, 1.0)
    x = sign * np.ldexp(mant, expo)
    # short significands create exact halfway cases for every target format
    k = n // 4
    short = np.ldexp(g.integers(1, 1 << 14, size=k).astype(np.float64), g.integers(-150, 120, size=k))
    x[:k] = short * sign[:k]
    return x


# --------------------------------------------------------------------------- decode
def test_decode_fp32_matches_numpy():
    b = rng(1).integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    got = oracle.decode(b, F32)
    want = b.view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m].view(np.uint64), want[m].view(np.uint64))


def test_decode_fp16_matches_numpy_all_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(b, F16)
    want = b.view(np.float16).astype(np.float64)
    m = ~np.isnan(want)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[m].view(np.uint64), want[m].view(np.uint64))


def test_decode_bf16_is_upper_half_of_binary32_all_patterns():
    b = np.arange(65536, dtype=np.uint32)
    got = oracle.decode(b.astype(np.uint16), BF16)
    want = (b << 16).view(np.float32).astype(np.float64)
    m = ~np.isnan(want)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[m].view(np.uint64), want[m].view(np.uint64))


# --------------------------------------------------------------------------- round
def test_round_fp32_matches_numpy_cast():
    x = random_doubles(2, 300_000)
    got = oracle.round_to(x, F32)
    want = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


def test_round_fp16_matches_numpy_cast():
    # numpy converts binary64 -> binary16 with one correct rounding
    assert np.float64(1 + 2**-11 + 2**-40).astype(np.float16) == np.float16(1 + 2**-10)
    x = random_doubles(3, 300_000) * 2.0**-100  # pull the range onto binary16's
    x = np.concatenate([x, random_doubles(4, 100_000) * 2.0**-120])
    got = oracle.round_to(x, F16)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def _bf16_finite_values():
    b = np.arange(0, 0x7F80, dtype=np.uint32)
    return b, (b << 16).view(np.float32).astype(np.float64)


def test_round_bf16_exhaustive_roundtrip_and_midpoints():
    b, v = _bf16_finite_values()
    # every pattern maps back to itself (both signs)
    assert np.array_equal(oracle.round_to(v, BF16), b.astype(np.uint16))
    assert np.array_equal(oracle.round_to(-v, BF16), (b | 0x8000).astype(np.uint16))
    # midpoints between neighbours: exactly halfway -> even pattern; one binary64
    # ulp either side -> the nearer neighbour
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2.0  # exact in binary64
    even = np.where((b[:-1] & 1) == 0, b[:-1], b[1:]).astype(np.uint16)
    assert np.array_equal(oracle.round_to(mid, BF16), even)
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    assert np.array_equal(oracle.round_to(below, BF16), b[:-1].astype(np.uint16))
    assert np.array_equal(oracle.round_to(above, BF16), b[1:].astype(np.uint16))


def test_round_bf16_overflow_threshold():
    top = float(np.array([0x7F7F << 16], dtype=np.uint32).view(np.float32)[0])
    ulp = 2.0 ** (127 - 7)
    assert oracle.round_to(np.array([top + ulp / 2]), BF16)[0] == 0x7F80
    assert oracle.round_to(np.array([np.nextafter(top + ulp / 2, 0)]), BF16)[0] == 0x7F7F
    assert oracle.round_to(np.array([-(top + ulp)]), BF16)[0] == 0xFF80


def test_round_bf16_against_fp32_path_via_torch():
    # binary64 -> binary32 (RNE, numpy) -> bfloat16 (RNE, torch) is a double
    # rounding; it equals the direct rounding unless the first step lands
    # exactly on a bf16 midpoint it created.  Compare where binary32 was exact.
    x = random_doubles(5, 200_000)
    f = x.astype(np.float32)
    exact = f.astype(np.float64) == x
    tb = torch.from_numpy(f[exact]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_to(x[exact], BF16)
    assert exact.sum() > 10_000
    assert np.array_equal(got, tb)


@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_round_matches_exact_rational_pyref(dt):
    scale = {F32: 1.0, F16: 2.0**-100, BF16: 1.0}[dt]
    x = random_doubles(10 + dt, 3000) * scale
    specials = [0.0, -0.0, math.inf, -math.inf, 5e-324, -5e-324, 2.0**-1022]
    x = np.concatenate([x, np.array(specials)])
    got = oracle.round_to(x, dt)
    want = np.array([pyref.round_to_bits(float(v), dt) for v in x], dtype=got.dtype)
    assert np.array_equal(got, want)


def test_round_nan_stays_nan():
    for dt in (F32, F16, BF16):
        r = oracle.round_to(np.array([np.nan, -np.nan]), dt)
        assert oracle.is_nan_bits(r, dt).all()


# --------------------------------------------------------------------------- allreduce
def load_cases():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["dtype"] + ":" + c["why"][:30])
def test_allreduce_worked_examples(case):
    dt = {"fp32": F32, "fp16": F16, "bf16": BF16}[case["dtype"]]
    parts = np.array([[int(h, 16) for h in row] for row in case["partials"]], dtype=oracle.BITS_DTYPE[dt])
    got = oracle.allreduce(parts, dt)
    for g, w in zip(got, case["out"]):
        if w == "NaN":
            assert oracle.is_nan_bits(np.array([g]), dt)[0]
        else:
            assert int(g) == int(w, 16), (hex(int(g)), w)
    # the pure-Python statement agrees
    py = pyref.allreduce([list(map(int, row)) for row in parts], dt)
    assert oracle.same_result(np.array(py, dtype=got.dtype), got, dt).all()


def rand_bits(seed, dt, shape, nan_free=True):
    g = rng(seed)
    if dt == F32:
        b = g.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32)
    else:
        b = g.integers(0, 2**16, size=shape, dtype=np.uint32).astype(np.uint16)
    if nan_free:
        b = np.where(oracle.is_nan_bits(b, dt), b & ~np.array(1 << (30 if dt == F32 else 14), dtype=b.dtype), b)
    return b


@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_allreduce_n1_is_identity(dt):
    b = rand_bits(20 + dt, dt, (1, 50_000), nan_free=False)
    out = oracle.allreduce(b, dt)
    assert oracle.same_result(out, b[0], dt).all()


def test_allreduce_n2_fp32_is_numpy_float32_add():
    # one binary32 add is correctly rounded; the binary64 sum then rounded to
    # binary32 is the same since 53 >= 2*24 + 2
    b = rand_bits(30, F32, (2, 200_000))
    out = oracle.allreduce(b, F32)
    f = b.view(np.float32)
    with np.errstate(all="ignore"):
        want = (f[0] + f[1]).view(np.uint32)
    assert oracle.same_result(out, want, F32).all()


def test_allreduce_n2_fp16_is_numpy_float16_add():
    b = rand_bits(31, F16, (2, 200_000))
    out = oracle.allreduce(b, F16)
    f = b.view(np.float16)
    with np.errstate(all="ignore"):
        want = (f[0] + f[1]).view(np.uint16)
    assert oracle.same_result(out, want, F16).all()


def test_allreduce_n2_bf16_via_binary32_add_and_torch_rounding():
    b = rand_bits(32, BF16, (2, 200_000))
    out = oracle.allreduce(b, BF16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(all="ignore"):
        s = f[0] + f[1]  # binary32 add: correctly rounded, 24 >= 2*8 + 2
    want = torch.from_numpy(s).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert oracle.same_result(out, want, BF16).all()


@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_allreduce_integer_values_any_rank_order(dt):
    # small integers: every partial sum is exact, so any order gives one answer
    g = rng(40 + dt)
    vals = g.integers(-64, 65, size=(8, 4096)).astype(np.float64)
    parts = oracle.round_to(vals, dt).reshape(8, 4096)
    want = oracle.round_to(vals.sum(axis=0), dt)
    for perm in [range(8), [7, 6, 5, 4, 3, 2, 1, 0], [3, 1, 4, 0, 5, 2, 7, 6]]:
        out = oracle.allreduce(parts[list(perm)], dt)
        assert np.array_equal(out, want)


@pytest.mark.parametrize("dt", [F32, F16, BF16])
@pytest.mark.parametrize("n_ranks", [2, 3, 4, 8])
def test_allreduce_constant_inputs_give_n_times_c(dt, n_ranks):
    c = oracle.round_to(np.array([0.75, -1.5, 3.0, 0.125]), dt)
    parts = np.tile(c, (n_ranks, 1))
    out = oracle.allreduce(parts, dt)
    want = oracle.round_to(np.array([0.75, -1.5, 3.0, 0.125]) * n_ranks, dt)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_allreduce_matches_pure_python_random(dt):
    parts = rand_bits(50 + dt, dt, (5, 400), nan_free=False)
    out = oracle.allreduce(parts, dt)
    py = pyref.allreduce([list(map(int, row)) for row in parts], dt)
    assert oracle.same_result(np.array(py, dtype=out.dtype), out, dt).all()


def test_allreduce_small_fp16_bruteforce_exact_sums():
    # N=2 over a grid of fp16 values: the binary64 sum is exact, so the result
    # must be the representable value nearest to the exact sum
    vals = np.arange(0, 65536, 97, dtype=np.uint32).astype(np.uint16)
    vals = vals[~oracle.is_nan_bits(vals, F16)]
    a, b = np.meshgrid(vals, vals[::7])
    parts = np.stack([a.ravel(), b.ravel()])
    out = oracle.allreduce(parts, F16)
    with np.errstate(all="ignore"):
        exact = oracle.decode(parts[0], F16) + oracle.decode(parts[1], F16)
    want = exact.astype(np.float16).view(np.uint16)
    assert oracle.same_result(out, want, F16).all()


def test_allreduce_rank_order_matters_only_by_rounding_of_binary64():
    # the oracle adds left to right: a result that depends on association
    # order in binary64 pins the order (2^60 + 1 - 2^60)
    big = np.array([2.0**60, 1.0, -2.0**60])
    parts = oracle.round_to(big, F32).reshape(3, 1)
    assert oracle.decode(oracle.allreduce(parts, F32), F32)[0] == 0.0
    parts2 = parts[[0, 2, 1]]
    assert oracle.decode(oracle.allreduce(parts2, F32), F32)[0] == 1.0


def test_sum_f64_matches_plain_python_sum():
    parts = rand_bits(60, BF16, (4, 1000))
    s = oracle.sum_f64(parts, BF16)
    for i in range(0, 1000, 37):
        acc = pyref.decode(int(parts[0, i]), BF16)
        for r in range(1, 4):
            acc += pyref.decode(int(parts[r, i]), BF16)
        assert (math.isnan(acc) and math.isnan(s[i])) or acc == s[i]


def test_threaded_oracle_equals_the_single_call():
    """Splitting the elements over host threads changes nothing: every
    element is its own sum (ragged ranges, more threads than useful)."""
    rng = np.random.default_rng(11)
    for dt, n in ((oracle.F32, 1001), (oracle.F16, 4099), (oracle.BF16, 7)):
        bits = rng.integers(0, 2 ** (8 * oracle.ELEM_BYTES[dt]), size=(5, n), dtype=np.uint64).astype(oracle.BITS_DTYPE[dt])
        want = oracle.allreduce(bits, dt)
        for t in (1, 3, 16):
            got = oracle.allreduce_threads(bits, dt, t)
            assert np.array_equal(oracle.same_result(got, want, dt), np.ones(n, bool))
