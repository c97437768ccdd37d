"""Pins of the oracle's Philox4x32-10 dither and WitCert INT8 quantizer.

* Philox4x32-10 agrees with an independent open-source implementation
  (PyTorch's ATen philox_engine, compiled here as a host program and used as
  a black box) on random counters and keys.
* WitCert write-kernel paragraph: scale s = amax/126.5 (Q - 1/2) stored fp16
  and reused; no clipping; |x - x_hat| <= s/2 for every element
  (subtractive dither); quantizing with the unrounded fp32 scale while
  storing fp16 breaks that bound (the page measured 1639 violations).
* Five-tuple stream uniqueness: distinct (request, layer, KV head, token,
  channel) tuples map to distinct (counter, output word) pairs.
* Dither statistics: xi uniform on [-1/2, 1/2): mean 0, variance 1/12,
  Kolmogorov-Smirnov against U(-1/2, 1/2); the error x - x_hat is uniform on
  [-s/2, s/2] and uncorrelated with x.
"""
import json
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

HERE = os.path.dirname(__file__)
GOLD = os.path.join(HERE, "golden")


def f16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f32(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float32)


@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ missing")
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    exe = str(tmp_path_factory.mktemp("philox") / "ref")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-I" + inc,
                           os.path.join(HERE, "philox_torch_ref.cpp"), "-o", exe])

    def run(rows):
        inp = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return np.array([[int(v) for v in line.split()] for line in out.strip().splitlines()],
                        np.uint64)
    return run


def test_philox_matches_independent_implementation(O, torch_philox):
    rng = np.random.default_rng(11)
    rows = rng.integers(0, 2 ** 32, size=(400, 6), dtype=np.uint64)
    rows[:4] = [[0] * 6, [2 ** 32 - 1] * 6, [1, 0, 0, 0, 0, 0], [0, 0, 0, 0, 0, 1]]
    ref = torch_philox(rows)
    got = np.array([O.philox(r[:4], r[4:]) for r in rows], np.uint64)
    assert np.array_equal(got, ref)


def test_dither_uses_counter_word_and_side_key(O, torch_philox):
    seed = 0x1234_5678_9ABC_DEF0
    cases = [(0, 3, 0, 5, 100, 77), (1, 3, 0, 5, 100, 77), (0, 31, 2, 7, 16383, 127)]
    for side, req, layer, kvh, tok, ch in cases:
        ctr = [tok, ch >> 2, (layer << 16) | kvh, req]
        key = [seed & 0xFFFFFFFF, (seed >> 32) ^ side]
        u = int(torch_philox([ctr + key])[0][ch & 3])
        xi = O.dither(seed, side, req, layer, kvh, tok, ch)
        assert xi == np.float32((u >> 8) * 2.0 ** -24) - np.float32(0.5)


def test_five_tuple_stream_uniqueness():
    # the (counter, word) map of the dither is injective on the tuple ranges
    # the library accepts (layer, kv head < 2^16; token, request < 2^32)
    seen = set()
    for req in (0, 1, 2 ** 31):
        for layer in (0, 1, 65535):
            for kvh in (0, 1, 7, 65535):
                for tok in (0, 1, 255, 256, 2 ** 31 + 5):
                    for ch in (0, 1, 3, 4, 127):
                        key = (tok, ch >> 2, (layer << 16) | kvh, req, ch & 3)
                        assert key not in seen
                        seen.add(key)
    assert len(seen) == 3 * 3 * 4 * 5 * 5


def test_dither_statistics(O):
    xi = np.array([O.dither(99, side, 1, 0, 2, t, c)
                   for side in (0, 1) for t in range(200) for c in range(0, 128, 3)], np.float64)
    assert xi.min() >= -0.5 and xi.max() < 0.5
    assert abs(xi.mean()) < 0.01
    assert abs(xi.var() - 1 / 12) < 0.004
    assert stats.kstest(xi + 0.5, "uniform").pvalue > 1e-3
    # sides differ (keys carry the side)
    assert O.dither(99, 0, 1, 0, 2, 5, 9) != O.dither(99, 1, 1, 0, 2, 5, 9)


def _block(seed, n=256, scale=1.0, outlier=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n).astype(np.float32) * np.float32(scale)
    if outlier is not None:
        x[outlier] *= np.float32(40)
    return f16(x)


def test_witcert_scale_no_clip_half_step(O):
    with open(os.path.join(GOLD, "witcert_scale.json")) as f:
        gold = json.load(f)
    Q = gold["Q"]
    rng = np.random.default_rng(3)
    for trial in range(300):
        x = _block(trial, scale=2.0 ** rng.uniform(-12, 7), outlier=trial % 256 if trial % 3 else None)
        assert np.all(np.isfinite(f32(x)))
        xi = rng.uniform(-0.5, 0.5, x.size).astype(np.float32)
        s16, codes = O.witcert_quant(x, xi)
        xv = f32(x).astype(np.float64)
        amax = np.abs(xv).max()
        assert s16 == f16(np.float32(amax) / np.float32(Q - 0.5))   # s = amax / 126.5, fp16
        s = float(f32(s16))
        assert np.abs(codes).max() <= Q                        # no clipping
        t = xv / s + xi
        assert np.all(np.abs(t) < Q + 0.5)                     # clamp never active
        xhat = np.array([O.witcert_dequant(c, s16, d) for c, d in zip(codes, xi)], np.float64)
        assert np.all(np.abs(xv - xhat) <= s / 2 * (1 + 2.0 ** -20) + 2.0 ** -30)


def test_witcert_stored_fp16_scale_rule_negative_control(O):
    # quantizing with the unrounded fp32 scale but dequantizing with the
    # stored fp16 one breaks |err| <= s/2 on some elements; the oracle's rule
    # (quantize with the stored fp16 scale) has none
    bad = 0
    good = 0
    rng = np.random.default_rng(5)
    for trial in range(200):
        x = _block(1000 + trial, scale=3.0)
        xi = rng.uniform(-0.5, 0.5, x.size).astype(np.float32)
        xv = f32(x)
        s32 = np.float32(np.abs(xv).max()) / np.float32(126.5)
        s16 = f16(s32)
        s = f32(s16)
        c32 = np.clip(np.rint(xv / s32 + xi), -127, 127)
        xh32 = s * (c32.astype(np.float32) - xi)
        bad += int(np.sum(np.abs(xv.astype(np.float64) - xh32) > s / 2 * (1 + 2.0 ** -20)))
        so, codes = O.witcert_quant(x, xi)
        xho = np.array([O.witcert_dequant(c, so, d) for c, d in zip(codes, xi)], np.float64)
        good += int(np.sum(np.abs(xv.astype(np.float64) - xho) > float(f32(so)) / 2 * (1 + 2.0 ** -20)))
    assert good == 0
    assert bad > 0


def test_witcert_error_uniform_and_independent(O):
    x = _block(77, n=4096, scale=1.0)
    xi = np.array([O.dither(5, 0, 0, 0, 0, t, 0) for t in range(x.size)], np.float32)
    s16, codes = O.witcert_quant(x, xi)
    s = float(f32(s16))
    xv = f32(x).astype(np.float64)
    xhat = np.array([O.witcert_dequant(c, s16, d) for c, d in zip(codes, xi)], np.float64)
    e = (xv - xhat) / s
    assert stats.kstest(e + 0.5, "uniform").pvalue > 1e-3
    assert abs(np.corrcoef(e, xv)[0, 1]) < 0.06


def test_witcert_zero_block(O):
    x = f16(np.zeros(256))
    s16, codes = O.witcert_quant(x, np.full(256, 0.3, np.float32))
    assert s16 == 0 and np.all(codes == 0)
    assert O.witcert_dequant(0, 0, 0.3) == 0.0
