"""The seeded input generators: binary64 draws rounded once to the I/O type,
to nearest with ties to even, pinned against the exact-rational rounding of
oracle/pyref.py; shapes, seeding and the distributions' own guarantees."""
import numpy as np
import pytest

import oracle
from oracle import F32, F16, BF16, pyref
from workloads import WORKLOADS, draw_values, make_partials, to_bits

CODE = {"fp32": F32, "fp16": F16, "bf16": BF16}


def spread_doubles(seed, n=2000):
    """Doubles over many binades, both signs, with zeros and exact ties of the
    16-bit types (1 + 2^-8: the bfloat16 midpoint of 1 and 1 + 2^-7; 1 + 2^-11:
    the binary16 midpoint of 1 and 1 + 2^-10), and their neighbours."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * 10.0 ** rng.integers(-4, 5, n)
    ties = [1 + 2.0**-8, 1 + 3 * 2.0**-8, 1 + 2.0**-11, 1 + 3 * 2.0**-11, 0.5 + 2.0**-9]
    x = np.concatenate([x, ties, np.negative(ties), np.nextafter(ties, 2), np.nextafter(ties, 0), [0.0, -0.0]])
    return x


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_rounding_is_nearest_even_from_binary64(dtype):
    x = spread_doubles(11)
    got = to_bits(x[None, :], dtype)[0]
    want = np.array([pyref.round_to_bits(float(v), CODE[dtype]) for v in x], dtype=got.dtype)
    assert np.array_equal(got, want)


def test_bf16_ties_go_to_even():
    x = np.array([[1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8), 2.0**-8 * (1 + 2.0**-8)]])
    # 1 + 2^-8 lies halfway between 0x3f80 and 0x3f81: the even one, 0x3f80;
    # 1 + 3 * 2^-8 halfway between 0x3f81 and 0x3f82: 0x3f82
    assert [hex(int(b)) for b in to_bits(x, "bf16")[0]] == ["0x3f80", "0x3f82", "0xbf80", "0x3b80"]


def test_bf16_refuses_values_outside_the_normal_range():
    with pytest.raises(ValueError):
        to_bits(np.array([[1e-40]]), "bf16")
    with pytest.raises(ValueError):
        to_bits(np.array([[1e39]]), "bf16")


def test_seeded_shapes_and_repeatability():
    a = make_partials(5, 3, 8, "bf16", 1000, "normal", 1.0)
    b = make_partials(5, 3, 8, "bf16", 1000, "normal", 1.0)
    c = make_partials(5, 4, 8, "bf16", 1000, "normal", 1.0)
    assert a.shape == (8, 1000) and a.dtype == np.uint16
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # the ranks draw different values
    assert not np.array_equal(a[0], a[1])


def test_draws_are_binary64_and_follow_their_distribution():
    v = draw_values(9, 0, 4, 20000, "uniform", 1.0)
    assert v.dtype == np.float64 and v.min() >= -1.0 and v.max() < 1.0
    n = draw_values(9, 0, 4, 20000, "normal", 0.02)
    assert abs(n.mean()) < 1e-3 and abs(n.std() - 0.02) < 1e-3
    k = draw_values(9, 0, 8, 20000, "integer", 1.0)
    assert np.array_equal(k, np.round(k)) and k.min() >= -64 and k.max() <= 64


def test_workload_inputs_never_hold_the_sentinel_or_a_nan():
    """Every workload draw is finite: in particular no element is the
    Sentinel protocol's all-ones pattern (a NaN in every type)."""
    for w in WORKLOADS.values():
        bits = make_partials(w.cfg_id, 0, w.n_ranks, w.dtype, min(w.n_elems, 1 << 16), w.dist, w.scale)
        vals = oracle.decode(bits.reshape(-1), CODE[w.dtype])
        assert np.isfinite(vals).all()
        assert not (bits == np.iinfo(bits.dtype).max).any()
