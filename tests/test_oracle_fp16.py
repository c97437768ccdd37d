"""Pins of the oracle's binary16 conversions against numpy's independent
implementation (numpy rounds float32 -> float16 to nearest, ties to even)."""
import numpy as np


def _conv_many(O, xs):
    return np.array([O.f32_to_f16(float(x)) for x in xs], np.uint16)


def test_f16_to_f32_all_patterns(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([O.f16_to_f32(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_roundtrip_every_finite_value(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    fin = np.isfinite(vals)
    got = _conv_many(O, vals[fin].astype(np.float32))
    assert np.array_equal(got, bits[fin])


def test_f32_to_f16_ties_and_neighbours(O):
    # midpoints between consecutive positive fp16 values (exact in fp32) and
    # their fp32 neighbours: ties must go to the even mantissa
    h = np.arange(0, 0x7bff, 7, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float32)
    hi = (h + 1).view(np.float16).astype(np.float32)
    mid = ((lo.astype(np.float64) + hi.astype(np.float64)) / 2).astype(np.float32)
    xs = np.concatenate([mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9)),
                         -mid])
    ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(_conv_many(O, xs), ref)


def test_f32_to_f16_random_and_overflow(O):
    rng = np.random.default_rng(0)
    e = rng.uniform(-30, 17, 20000)
    xs = (rng.choice([-1, 1], e.size) * 2.0 ** e).astype(np.float32)
    xs = np.concatenate([xs, np.float32([65504, 65519.99, 65520, 65536, 1e30, -1e30, 0.0, -0.0,
                                          2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26, 2.0 ** -14])])
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(_conv_many(O, xs), ref)
