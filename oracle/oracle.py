"""ctypes binding of the CPU oracle (``kvq_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke entry
point and by the benchmark's cpu_baseline leg; never by the library.  It
shares no code with the HIP path.  Arrays cross as numpy buffers: fp16
values as ``uint16`` bit patterns, codes as ``uint8`` (WitCert codes are
int8 bit patterns).  See ``kvq_oracle.c`` for the sources each function
follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "_build", "libkvq_oracle.so")

KIVI, KITTY, WITCERT, KITTY_DYN, KIVI4, WITCERT_TOK = 0, 1, 2, 3, 4, 5

GCC_FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-fno-finite-math-only"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        L = C.CDLL(LIB)
        P = C.c_void_p
        L.ko_f16_to_f32.argtypes = [C.c_uint16]
        L.ko_f16_to_f32.restype = C.c_float
        L.ko_f32_to_f16.argtypes = [C.c_float]
        L.ko_f32_to_f16.restype = C.c_uint16
        L.ko_quant_asym.argtypes = [P, C.c_long, C.c_long, C.c_int, P, P, P, C.c_long]
        L.ko_dequant_asym.argtypes = [C.c_int, C.c_uint16, C.c_uint16]
        L.ko_dequant_asym.restype = C.c_float
        L.ko_philox4x32_10.argtypes = [P, P, P]
        L.ko_dither.argtypes = [C.c_uint64, C.c_int, C.c_uint32, C.c_uint32,
                                C.c_uint32, C.c_uint32, C.c_uint32]
        L.ko_dither.restype = C.c_float
        L.ko_dither_slot.argtypes = [C.c_uint64, C.c_int, C.c_uint32, C.c_uint32,
                                     C.c_uint64, C.c_uint32]
        L.ko_dither_slot.restype = C.c_float
        L.ko_witcert_select_pairs.argtypes = [P, C.c_long, C.c_int, C.c_int, P]
        L.ko_stream_set_slots.argtypes = [P, P]
        L.ko_witcert_quant.argtypes = [P, C.c_long, C.c_long, P, P, P, C.c_long]
        L.ko_witcert_dequant.argtypes = [C.c_int, C.c_uint16, C.c_float]
        L.ko_witcert_dequant.restype = C.c_float
        L.ko_kitty_select.argtypes = [P, C.c_long, C.c_int, C.c_int, P]
        L.ko_kitty_select_dyn.argtypes = [P, C.c_long, C.c_long, C.c_int, C.c_int, P]
        L.ko_stream_new.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                    C.c_int, C.c_int, P, C.c_long, C.c_uint64,
                                    C.c_uint32, C.c_uint32, C.c_uint32, C.c_long, C.c_long]
        L.ko_stream_new.restype = P
        L.ko_stream_free.argtypes = [P]
        L.ko_stream_flush.argtypes = [P]
        L.ko_stream_append.argtypes = [P, P, P]
        L.ko_stream_prefill.argtypes = [P, P, P, C.c_long]
        L.ko_stream_state.argtypes = [P, P]
        for name in ("ko_stream_kcodes", "ko_stream_vcodes", "ko_stream_uidx"):
            getattr(L, name).argtypes = [P]
            getattr(L, name).restype = C.POINTER(C.c_uint8)
        for name in ("ko_stream_kscale", "ko_stream_kzero", "ko_stream_vscale",
                     "ko_stream_vzero"):
            getattr(L, name).argtypes = [P]
            getattr(L, name).restype = C.POINTER(C.c_uint16)
        L.ko_stream_dequant.argtypes = [P, C.c_long, C.c_long, P, P]
        L.ko_stream_attend_range.argtypes = [P, P, C.c_int, C.c_float, C.c_float,
                                             C.c_long, C.c_long, P, P, P]
        L.ko_merge.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, P]
        L.ko_stream_decode.argtypes = [P, P, C.c_int, C.c_float, C.c_float, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(C.c_void_p)


# --------------------------------------------------------------------------
# scalar / group primitives
# --------------------------------------------------------------------------

def f16_to_f32(h: int) -> float:
    return lib().ko_f16_to_f32(int(h))


def f32_to_f16(x: float) -> int:
    return lib().ko_f32_to_f16(float(np.float32(x)))


def quant_asym(x: np.ndarray, bits: int):
    """Quantize one group (fp16 bits, 1-D).  Returns (s16, z16, codes)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    codes = np.zeros(x.size, np.uint8)
    lib().ko_quant_asym(_p(x), x.size, 1, bits, _p(s), _p(z), _p(codes), 1)
    return int(s[0]), int(z[0]), codes


def dequant_asym(code: int, s16: int, z16: int) -> float:
    return lib().ko_dequant_asym(int(code), int(s16), int(z16))


def philox(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().ko_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def dither(seed: int, side: int, req: int, layer: int, kvh: int, token: int, ch: int) -> float:
    return lib().ko_dither(seed, side, req, layer, kvh, token, ch)


def dither_slot(seed: int, side: int, layer: int, kvh: int, slot: int, ch: int) -> float:
    return lib().ko_dither_slot(seed, side, layer, kvh, slot, ch)


def witcert_select_pairs(k: np.ndarray, m: int) -> np.ndarray:
    """Bypass mask [D] (1 for both channels of the m chosen RoPE pairs) from a
    calibration slice k [T][D] (fp16 bits)."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    T, D = k.shape
    mask = np.zeros(D, np.uint8)
    lib().ko_witcert_select_pairs(_p(k), T, D, m, _p(mask))
    return mask


def witcert_quant(x: np.ndarray, xi: np.ndarray):
    """Quantize one channel-block (fp16 bits) with dither xi.  Returns (s16, int8 codes)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    xi = np.ascontiguousarray(xi, dtype=np.float32)
    s = np.zeros(1, np.uint16)
    codes = np.zeros(x.size, np.int8)
    lib().ko_witcert_quant(_p(x), x.size, 1, _p(xi), _p(s), _p(codes), 1)
    return int(s[0]), codes


def witcert_dequant(code: int, s16: int, xi: float) -> float:
    return lib().ko_witcert_dequant(int(code), int(s16), float(xi))


def kitty_select(k: np.ndarray, nb: int) -> np.ndarray:
    """Static boost index from a calibration slice k [T][D] (fp16 bits)."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    T, D = k.shape
    idx = np.zeros(D, np.uint8)
    lib().ko_kitty_select(_p(k), T, D, nb, _p(idx))
    return idx


def kitty_select_dyn(k: np.ndarray, nb: int) -> np.ndarray:
    """Dynamic boost index of one selection unit k [T][D] (fp16 bits):
    top nb channels by mean |x| over the unit, ties to the lower channel."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    T, D = k.shape
    idx = np.zeros(D, np.uint8)
    lib().ko_kitty_select_dyn(_p(k), T, D, D, nb, _p(idx))
    return idx


# --------------------------------------------------------------------------
# one (request, KV head) stream
# --------------------------------------------------------------------------

class Stream:
    """Raw history + quantized record of one (request, KV head)."""

    def __init__(self, scheme: int, cap: int, D: int = 128, G: int = 32, R: int = 128,
                 VG: int = 32, BLK: int = 256, nb: int = 0, idx=None,
                 seed: int = 0, req: int = 0, layer: int = 0, kvh: int = 0, sel: int = 64,
                 sink: int = 0, slots=None):
        """WITCERT_TOK: idx = bypass mask [D] (or None), VG = scale group,
        slots = cache slot of every token [cap] (default: slot t for token t)."""
        self.scheme, self.cap, self.D, self.G, self.R = scheme, cap, D, G, R
        self.VG, self.BLK, self.nb, self.sel, self.sink = VG, BLK, nb, sel, sink
        self._idx = None if idx is None else np.ascontiguousarray(idx, np.uint8)
        h = lib().ko_stream_new(scheme, D, G, R, VG, BLK, nb,
                                None if self._idx is None else _p(self._idx),
                                cap, seed, req, layer, kvh, sel, sink)
        if not h:
            raise ValueError("invalid stream parameters")
        self.h = h
        if slots is not None:
            self._slots = np.ascontiguousarray(slots, np.uint64)
            assert self._slots.shape == (cap,)
            if lib().ko_stream_set_slots(h, _p(self._slots)) != 0:
                raise ValueError("slots rejected")

    def __del__(self):
        h = getattr(self, "h", None)
        if h:
            lib().ko_stream_free(h)
            self.h = None

    # state machine -------------------------------------------------------
    def prefill(self, K: np.ndarray, V: np.ndarray):
        K = np.ascontiguousarray(K, np.uint16)
        V = np.ascontiguousarray(V, np.uint16)
        if lib().ko_stream_prefill(self.h, _p(K), _p(V), K.shape[0]) != 0:
            raise ValueError("prefill rejected")

    def flush(self) -> bool:
        return bool(lib().ko_stream_flush(self.h))

    def append(self, k: np.ndarray, v: np.ndarray) -> int:
        k = np.ascontiguousarray(k, np.uint16)
        v = np.ascontiguousarray(v, np.uint16)
        return lib().ko_stream_append(self.h, _p(k), _p(v))

    @property
    def state(self):
        out = np.zeros(3, np.int64)
        lib().ko_stream_state(self.h, _p(out))
        return tuple(int(v) for v in out)   # (l, n_kq, n_vq)

    # read-back -----------------------------------------------------------
    def _arr(self, fn, n, dtype):
        ptr = getattr(lib(), fn)(self.h)
        return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dtype).copy()

    def key_codes(self):
        return self._arr("ko_stream_kcodes", self.cap * self.D, np.uint8).reshape(self.cap, self.D)

    def value_codes(self):
        return self._arr("ko_stream_vcodes", self.cap * self.D, np.uint8).reshape(self.cap, self.D)

    def unit_index(self):
        """Kitty dynamic: boost index per selection unit [cap/sel + 1][D]."""
        n = self.cap // self.sel + 1
        return self._arr("ko_stream_uidx", n * self.D, np.uint8).reshape(n, self.D)

    def key_stats(self):
        """(scale, zero) fp16 bits: [groups][D] (WitCert: [blocks][D], zero unused;
        WITCERT_TOK: scales [cap][D/VG]); groups count from the first token after
        the sink."""
        if self.scheme == WITCERT_TOK:
            ng = self.D // self.VG
            s = self._arr("ko_stream_kscale", self.cap * ng, np.uint16).reshape(self.cap, ng)
            return s, np.zeros_like(s)
        n = (self.cap // (self.BLK if self.scheme == WITCERT else self.G)) + 1
        s = self._arr("ko_stream_kscale", n * self.D, np.uint16).reshape(n, self.D)
        z = self._arr("ko_stream_kzero", n * self.D, np.uint16).reshape(n, self.D)
        return s, z

    def value_stats(self):
        """(scale, zero): KIVI/Kitty [cap][D/VG]; WitCert [blocks][D] scales."""
        if self.scheme == WITCERT:
            n = (self.cap // self.BLK) + 1
            s = self._arr("ko_stream_vscale", n * self.D, np.uint16).reshape(n, self.D)
            z = self._arr("ko_stream_vzero", n * self.D, np.uint16).reshape(n, self.D)
            return s, z
        ng = self.D // self.VG
        s = self._arr("ko_stream_vscale", self.cap * ng, np.uint16).reshape(self.cap, ng)
        if self.scheme == WITCERT_TOK:
            return s, np.zeros_like(s)
        z = self._arr("ko_stream_vzero", self.cap * ng, np.uint16).reshape(self.cap, ng)
        return s, z

    def dequant(self, t0: int = 0, t1: int | None = None):
        """(K~, V~) float32 [t1-t0][D] as seen by attention."""
        if t1 is None:
            t1 = self.state[0]
        n = t1 - t0
        K = np.zeros((max(n, 1), self.D), np.float32)
        V = np.zeros((max(n, 1), self.D), np.float32)
        if n > 0:
            lib().ko_stream_dequant(self.h, t0, t1, _p(K), _p(V))
        return K[:n], V[:n]

    # attention -----------------------------------------------------------
    def attend_range(self, q: np.ndarray, sm_scale: float, kappa: float, t0: int, t1: int):
        q = np.ascontiguousarray(q, np.uint16).reshape(-1, self.D)
        nq = q.shape[0]
        o = np.zeros((nq, self.D), np.float64)
        lse = np.zeros(nq, np.float64)
        a = np.zeros(nq, np.float64)
        lib().ko_stream_attend_range(self.h, _p(q), nq, float(sm_scale), float(kappa),
                                     t0, t1, _p(o), _p(lse), _p(a))
        return o, lse, a

    def decode(self, q: np.ndarray, sm_scale: float, kappa: float = 0.0):
        """fp64 attention over the current state.  Returns (out [nq][D], cert [nq])."""
        q = np.ascontiguousarray(q, np.uint16).reshape(-1, self.D)
        nq = q.shape[0]
        out = np.zeros((nq, self.D), np.float64)
        cert = np.zeros(nq, np.float64)
        lib().ko_stream_decode(self.h, _p(q), nq, float(sm_scale), float(kappa),
                               _p(out), _p(cert))
        return out, cert


def merge(o_parts: np.ndarray, lses: np.ndarray, a_parts: np.ndarray):
    """LSE merge of per-split partials: o_parts [S][nq][D], lses/a_parts [S][nq]."""
    o_parts = np.ascontiguousarray(o_parts, np.float64)
    lses = np.ascontiguousarray(lses, np.float64)
    a_parts = np.ascontiguousarray(a_parts, np.float64)
    S, nq, D = o_parts.shape
    o = np.zeros((nq, D), np.float64)
    a = np.zeros(nq, np.float64)
    lib().ko_merge(S, nq, D, _p(o_parts), _p(lses), _p(a_parts), _p(o), _p(a))
    return o, a
