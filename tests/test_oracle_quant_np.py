"""Two quantizer oracles, one answer: the C oracle's asymmetric 2-/4-bit group
quantizer and its subtractive-dither INT8 quantizer against the NumPy
quantizers of ``oracle/quant_np.py``, written apart from it from the same
passages (KIVI explainer 3.1; Kitty summary, Observation 1 and the
quantization step; WitCert, the write-kernel paragraph).  Scales, zero
points and codes must agree bit for bit on over 10^5 seeded groups per
quantizer, drawn to include rounding ties, constant groups, fp16-subnormal
ranges, +0 and -0 minima and full-range values.

The NumPy side is itself checked against what the pages fix (the Kitty
[0, 10] example, the half-step bound, no clipping), so that agreement is
not agreement on a shared mistake.
"""
import ctypes as C
import json
import os

import numpy as np
import pytest

from oracle import quant_np as Q

GOLD = os.path.join(os.path.dirname(__file__), "golden")
N_GROUPS = 100_000


def _finite_f16(rng, shape):
    """Uniform over the finite fp16 bit patterns (both zeros, subnormals, normals)."""
    b = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    bad = (b & 0x7C00) == 0x7C00
    while bad.any():
        b[bad] = rng.integers(0, 1 << 16, size=int(bad.sum()), dtype=np.uint32).astype(np.uint16)
        bad = (b & 0x7C00) == 0x7C00
    return b


def _asym_groups(rng, n_groups, n, bits):
    """Rows of fp16 bits, a fixed mix of kinds; each kind keeps its name."""
    top = (1 << bits) - 1
    kinds = ["normal", "any_bits", "subnormal", "tiny_span", "constant", "zero_min", "ties", "wide"]
    per = n_groups // len(kinds) + 1
    rows = {}
    # N(0, 1) at scales from 1e-4 to 1e3
    scale = 10.0 ** rng.uniform(-4, 3, size=(per, 1))
    rows["normal"] = (rng.standard_normal((per, n)) * scale).astype(np.float16).view(np.uint16)
    rows["any_bits"] = _finite_f16(rng, (per, n))
    # every value an fp16 subnormal or zero, either sign
    sub = rng.integers(0, 1 << 10, size=(per, n), dtype=np.uint32).astype(np.uint16)
    rows["subnormal"] = sub | (rng.integers(0, 2, size=(per, n), dtype=np.uint16) << 15)
    # spans of 1 .. 8 subnormal ulps (2^-24): the steps the guard raises
    base = rng.integers(-1000, 1000, size=(per, 1))
    span = rng.integers(1, 9, size=(per, 1))
    off = rng.integers(0, 2 ** 20, size=(per, n)) % (span + 1)
    off[:, 0] = 0
    off[:, 1] = span[:, 0]
    rows["tiny_span"] = ((base + off) * 2.0 ** -24).astype(np.float16).view(np.uint16)
    # one value repeated: random finite, with +0 and -0 among them
    c = _finite_f16(rng, (per, 1))
    c[: per // 8] = 0x0000
    c[per // 8: per // 4] = 0x8000
    rows["constant"] = np.repeat(c, n, axis=1)
    # non-negative values whose minimum is a zero of either sign
    zm = np.abs(rng.standard_normal((per, n)) * 10.0 ** rng.uniform(-6, 2, size=(per, 1)))
    zm = zm.astype(np.float16).view(np.uint16)
    k = rng.integers(1, 4, size=per)
    for i in range(per):
        at = rng.choice(n, size=k[i], replace=False)
        zm[i, at] = rng.choice(np.array([0x0000, 0x8000], np.uint16), size=k[i])
    rows["zero_min"] = zm
    # exact half-step ties: z = m 2^e, top step z + top 2^e, the rest at
    # z + (j + 1/2) 2^e (all exact in fp16); s comes out as 2^e
    e = rng.integers(-14, 5, size=(per, 1)).astype(np.float64)
    m = rng.integers(-600, 600, size=(per, 1)).astype(np.float64)
    j = rng.integers(0, top, size=(per, n)).astype(np.float64)
    t = (m + j + 0.5) * 2.0 ** e
    t[:, 0] = (m[:, 0]) * 2.0 ** e[:, 0]
    t[:, 1] = (m[:, 0] + top) * 2.0 ** e[:, 0]
    rows["ties"] = t.astype(np.float16).view(np.uint16)
    assert np.array_equal(rows["ties"].view(np.float16).astype(np.float64), t)
    # extremes of the fp16 range in one group
    w = _finite_f16(rng, (per, n))
    w[:, 0] = 0x7BFF        # 65504
    w[:, 1] = 0xFBFF        # -65504
    w[per // 2:, 1] = 0x0001  # or the smallest subnormal
    rows["wide"] = w
    x = np.concatenate([rows[k_] for k_ in kinds])[:n_groups]
    where = {k_: slice(i * per, min((i + 1) * per, n_groups)) for i, k_ in enumerate(kinds)}
    return np.ascontiguousarray(x), where


def _c_quant_asym(O, x, bits):
    """The C oracle over every row, through its group entry point."""
    L = O.lib()
    N, n = x.shape
    s = np.zeros(N, np.uint16)
    z = np.zeros(N, np.uint16)
    codes = np.zeros((N, n), np.uint8)
    px, ps, pz, pc = (a.ctypes.data for a in (x, s, z, codes))
    f = L.ko_quant_asym
    for i in range(N):
        f(C.c_void_p(px + 2 * n * i), n, 1, bits, C.c_void_p(ps + 2 * i), C.c_void_p(pz + 2 * i),
          C.c_void_p(pc + n * i), 1)
    return s, z, codes


def _c_quant_dither(O, x, xi):
    L = O.lib()
    N, n = x.shape
    s = np.zeros(N, np.uint16)
    codes = np.zeros((N, n), np.int8)
    px, pxi, ps, pc = (a.ctypes.data for a in (x, xi, s, codes))
    f = L.ko_witcert_quant
    for i in range(N):
        f(C.c_void_p(px + 2 * n * i), n, 1, C.c_void_p(pxi + 4 * n * i), C.c_void_p(ps + 2 * i),
          C.c_void_p(pc + n * i), 1)
    return s, codes


def _diff_report(name, a, b):
    bad = np.flatnonzero(a.reshape(a.shape[0], -1) != b.reshape(b.shape[0], -1))
    return f"{name}: {bad.size} mismatches, first rows {np.unique(bad // max(1, a[0].size))[:5]}"


@pytest.mark.parametrize("bits", [2, 4])
def test_asym_numpy_equals_c_bit_for_bit(O, bits):
    rng = np.random.default_rng(1000 + bits)
    x, where = _asym_groups(rng, N_GROUPS, 32, bits)
    assert x.shape[0] >= 100_000
    s_np, z_np, c_np = Q.quant_asym(x, bits)
    s_c, z_c, c_c = _c_quant_asym(O, x, bits)
    assert np.array_equal(s_np, s_c), _diff_report("scale", s_np, s_c)
    assert np.array_equal(z_np, z_c), _diff_report("zero point", z_np, z_c)
    assert np.array_equal(c_np, c_c), _diff_report("codes", c_np, c_c)
    # the cases the mix was built for did occur
    xv = x.view(np.float16).astype(np.float64)
    assert (s_np == 0).sum() >= N_GROUPS // 9                       # constant groups
    assert ((s_np.view(np.float16) < np.float16(2.0 ** -14)) & (s_np != 0)).sum() > 1000  # subnormal steps
    assert (z_np == 0x0000).sum() > 1000 and not (z_np == 0x8000).any()  # minima stored +0
    # the built ties: exact in binary32 too, each on a half step below the top
    tw = where["ties"]
    sf = s_np[tw].view(np.float16).astype(np.float64)[:, None]
    zf = z_np[tw].view(np.float16).astype(np.float64)[:, None]
    r = (xv[tw] - zf) / sf
    ties = r - np.floor(r) == 0.5
    assert ties.sum() > 10 * (N_GROUPS // 8)                         # exact half-step ties
    assert (r[ties] < (1 << bits) - 1).all() and (c_np[tw][ties] % 2 == 0).all()  # ... to even


@pytest.mark.parametrize("n", [32, 256])
def test_dither_int8_numpy_equals_c_bit_for_bit(O, n):
    rng = np.random.default_rng(2000 + n)
    n_groups = N_GROUPS if n == 32 else 12_000
    x, _ = _asym_groups(rng, n_groups, n, 2)
    xi = Q.dither_from_word(rng.integers(0, 1 << 32, size=x.shape, dtype=np.uint64).astype(np.uint32))
    # ties of x / s + xi: groups with amax = 126.5 2^e (s = 2^e), values
    # j 2^(e-1) and xi = 0 (odd j) or -1/2 (even j)
    nt = n_groups // 8
    e = rng.integers(-13, 7, size=(nt, 1)).astype(np.float64)
    j = rng.integers(-253, 254, size=(nt, n)).astype(np.float64)
    j[:, 0] = 253 * rng.choice([-1.0, 1.0], size=nt)
    x[:nt] = (j * 2.0 ** (e - 1)).astype(np.float16).view(np.uint16)
    xi[:nt] = np.where(j % 2 == 1, np.float32(0.0), np.float32(-0.5))
    x = np.ascontiguousarray(x)
    xi = np.ascontiguousarray(xi, dtype=np.float32)
    s_np, c_np = Q.quant_dither_int8(x, xi)
    s_c, c_c = _c_quant_dither(O, x, xi)
    assert np.array_equal(s_np, s_c), _diff_report("scale", s_np, s_c)
    assert np.array_equal(c_np, c_c), _diff_report("codes", c_np, c_c)
    sf = s_np.view(np.float16).astype(np.float64)
    assert (sf[:nt] == 2.0 ** e[:, 0]).all()
    t = x[:nt].view(np.float16).astype(np.float64) / sf[:nt, None] + xi[:nt]
    assert (t - np.floor(t) == 0.5).all() and (c_np[:nt] % 2 == 0).all()
    assert (s_np == 0).sum() >= n_groups // 40                      # all-zero blocks


# ---- the NumPy quantizers against what the pages and arithmetic fix ----

def test_numpy_asym_kitty_example_and_half_step():
    """Kitty summary, Observation 1: a channel over [0, 10] at 2 bits has
    steps of 10/3, one over [0, 1] steps of 1/3; every value lies within
    half a step of its reconstruction and its code is a nearest level, up to
    the binary32 roundings of x - z, of the quotient and of x_hat (at most
    2^-24 |x - z| each for the first two, 2^-24 |x_hat| for the last: a value
    a hair above a half step, far from z, can round onto it and then to the
    even level)."""
    with open(os.path.join(GOLD, "kitty_obs1_steps.json")) as fh:
        gold = json.load(fh)
    for case in gold["cases"]:
        lo, hi = case["span"]
        x = np.linspace(lo, hi, 32).astype(np.float16).view(np.uint16)[None]
        s, z, codes = Q.quant_asym(x, 2)
        assert abs(float(s.view(np.float16)[0]) - case["step"]) <= case["step"] * 2.0 ** -11
        assert codes[0, 0] == 0 and codes[0, -1] == 3
    rng = np.random.default_rng(7)
    for bits in (2, 4):
        x, _ = _asym_groups(rng, 20_000, 32, bits)
        s, z, codes = Q.quant_asym(x, bits)
        xh = Q.dequant_asym(codes, s, z).astype(np.float64)
        xv = x.view(np.float16).astype(np.float64)
        sf = s.view(np.float16).astype(np.float64)[:, None]
        zf = z.view(np.float16).astype(np.float64)[:, None]
        slack = (np.abs(xv - zf) * 2.0 ** -23 + np.abs(xh) * 2.0 ** -24 + 2.0 ** -149)
        assert (np.abs(xv - xh) <= sf / 2 + slack).all()
        # brute force: the code is a nearest of the 2^b levels (in fp64)
        lv = np.arange(1 << bits)[None, None, :] * sf[:, :, None] + \
            z.view(np.float16).astype(np.float64)[:, None, None]
        dist = np.abs(xv[:, :, None] - lv)
        best = dist.min(axis=2)
        got = np.take_along_axis(dist, codes[:, :, None].astype(np.int64), axis=2)[:, :, 0]
        assert (got <= best + 2 * slack).all()


def test_numpy_dither_no_clipping_and_half_step():
    """WitCert write kernel: with the stored fp16 scale of amax / 126.5 no
    code clips and |x - x_hat| <= s/2 with x_hat = s (code - xi)."""
    rng = np.random.default_rng(8)
    x, _ = _asym_groups(rng, 20_000, 256, 2)
    xi = Q.dither_from_word(rng.integers(0, 1 << 32, size=x.shape, dtype=np.uint64).astype(np.uint32))
    s, codes = Q.quant_dither_int8(x, xi)
    xv = x.view(np.float16).astype(np.float64)
    sf = s.view(np.float16).astype(np.float64)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        raw = np.where(sf > 0, xv / sf + xi, 0.0)
    assert (np.abs(raw) < 127.5).all()                              # never clipped
    # up to the binary32 roundings of x / s and of the sum (|x / s| < 127.5)
    err = np.abs(xv - sf * (codes.astype(np.float64) - xi))
    assert (err <= sf / 2 + sf * 2.0 ** -16).all()
    assert (xi >= -0.5).all() and (xi < 0.5).all()
