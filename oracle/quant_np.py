"""A second, vectorised quantizer oracle in NumPy.

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the library.
It is written from the pages' quantizer passages and their readings, apart
from the C oracle, with which it shares no code; a test holds the two equal
bit for bit.  Arrays: fp16 values as ``uint16`` bit patterns, one group per
row.  Every float step is one IEEE binary32 operation (NumPy's float32
arithmetic, round to nearest even); binary32 -> binary16 is NumPy's
correctly rounded conversion; comparisons that only decide a guard are made
exactly (binary64 holds the operands and products exactly).

Asymmetric group quantizer (KIVI explainer, 3.1; Kitty summary, Observation 1
and the quantization step):
    z = min of the group (a zero minimum is kept as +0),
    s = fp16(fl32(fl32(max - min) / (2^b - 1))),
    raised once to the next fp16 value if (2^b - 1/2) s < max - min (a
    subnormal step rounded down too far),
    code = clamp(rint(fl32(fl32(x - z) / s)), 0, 2^b - 1), ties to even;
    a constant group has s = 0 and all codes 0.

Subtractive-dither INT8 quantizer (WitCert, the write-kernel paragraph: a
stored fp16 scale of amax / 126.5, codes round(x / s + xi)):
    s = fp16(fl32(amax / 126.5)), raised once to the next fp16 value if
    127 s <= amax; amax = 0 gives s = 0 and codes 0;
    code = clamp(rint(fl32(fl32(x / s) + xi)), -127, 127), ties to even,
    with the stored s.  The dither xi is an input here.
"""
from __future__ import annotations

import numpy as np

_F16_INF = np.float16(np.inf)


def _values(x16: np.ndarray) -> np.ndarray:
    x16 = np.asarray(x16, np.uint16)
    if x16.ndim != 2:
        raise ValueError("groups are rows of a 2-D array")
    return x16.view(np.float16).astype(np.float32)


def quant_asym(x16: np.ndarray, bits: int):
    """Groups [N, n] of fp16 bits -> (s16 [N], z16 [N], codes [N, n] uint8)."""
    if bits not in (2, 4):
        raise ValueError("bits is 2 or 4")
    x = _values(x16)
    top = (1 << bits) - 1
    mn = x.min(axis=1)
    mx = x.max(axis=1)
    span = mx - mn                                        # binary32
    s = (span / np.float32(top)).astype(np.float16)       # one binary32 division, then RNE to fp16
    short = (top + 0.5) * s.astype(np.float64) < (mx.astype(np.float64) - mn.astype(np.float64))
    s = np.where(short, np.nextafter(s, _F16_INF), s)
    z = mn.astype(np.float16)                             # exact: mn is an fp16 value
    z = np.where(z == 0, np.float16(0.0), z)              # +0, whatever the sign of the minimum
    sf = s.astype(np.float32)[:, None]
    zf = z.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (x - zf) / sf                                 # two binary32 operations
    codes = np.clip(np.rint(r), 0, top)
    codes = np.where(sf == 0, 0, codes)
    return s.view(np.uint16), z.view(np.uint16), codes.astype(np.uint8)


def dequant_asym(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """x_hat = fl32(fl32(code * s) + z), per group row."""
    s = np.asarray(s16, np.uint16).view(np.float16).astype(np.float32)[:, None]
    z = np.asarray(z16, np.uint16).view(np.float16).astype(np.float32)[:, None]
    return np.asarray(codes, np.float32) * s + z


def quant_dither_int8(x16: np.ndarray, xi: np.ndarray):
    """Groups [N, n] of fp16 bits and dither xi [N, n] (fp32) ->
    (s16 [N], codes [N, n] int8)."""
    x = _values(x16)
    xi = np.asarray(xi, np.float32)
    if xi.shape != x.shape:
        raise ValueError("one dither value per element")
    amax = np.abs(x).max(axis=1)
    s = (amax / np.float32(126.5)).astype(np.float16)
    clips = 127.0 * s.astype(np.float64) <= amax.astype(np.float64)
    s = np.where(clips, np.nextafter(s, _F16_INF), s)
    s = np.where(amax == 0, np.float16(0.0), s)
    sf = s.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = x / sf + xi                                   # two binary32 operations
    codes = np.clip(np.rint(t), -127, 127)
    codes = np.where(sf == 0, 0, codes)
    return s.view(np.uint16), codes.astype(np.int8)


def dither_from_word(u: np.ndarray) -> np.ndarray:
    """A dither value from a 32-bit generator word: its top 24 bits as a
    fraction of 2^24, minus one half (exact in binary32)."""
    u = np.asarray(u, np.uint32)
    return ((u >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)) - np.float32(0.5)
