"""Test-side reader of the library's page layout (as documented in
bit_kv_cache_kivi_amd/csrc/kvq_common.hpp): maps the packed bytes of a
(page, KV head) block back to logical codes and statistics so they can be
compared with the oracle's.  Written independently of the HIP code."""
from __future__ import annotations

import numpy as np

D = 128
PT = 64
WPT = 256

GEOM = {  # kc, kh, ks, vc, vs, (ki,) bytes
    0: dict(kc=0, kh=0, ks=2048, vc=3072, vs=5120, bytes=6144, tokens=PT),
    1: dict(kc=0, kh=2048, ks=2304, vc=3328, vs=5376, bytes=6400, tokens=PT),
    2: dict(kc=0, kh=0, ks=32768, vc=33024, vs=65792, bytes=66048, tokens=WPT),
    3: dict(kc=0, kh=2048, ks=2304, vc=3328, vs=5376, ki=6400, bytes=6416, tokens=PT),
}
KITTY_SCHEMES = (1, 3)


def _key_index():
    t = np.arange(PT)[:, None]
    c = np.arange(D)[None, :]
    n, r, kc, g, j = t >> 4, t & 15, c >> 5, (c >> 3) & 3, c & 7
    lane = 16 * g + r
    d = 2 * n + (kc >> 1)
    h = kc & 1
    dword = (d >> 2) * 256 + lane * 4 + (d & 3)
    shift = 4 * j + 2 * h
    return dword, shift


def _value_index():
    t = np.arange(PT)[:, None]
    c = np.arange(D)[None, :]
    nt, r, ks, g, j = c >> 4, c & 15, t >> 5, (t >> 3) & 3, t & 7
    lane = 16 * g + r
    dword = (nt >> 2) * 256 + lane * 4 + (nt & 3)
    shift = 4 * j + 2 * ks
    return dword, shift


def _high_index():
    t = np.arange(PT)[:, None]
    o = np.arange(16)[None, :]
    n, r, g, i = t >> 4, t & 15, o >> 2, o & 3
    dword = 16 * g + r
    shift = 4 * (4 * (n & 1) + i) + 2 * (n >> 1)
    return dword, shift


KEY_DW, KEY_SH = _key_index()
VAL_DW, VAL_SH = _value_index()
HI_DW, HI_SH = _high_index()
KEY_SLOT = np.arange(D)            # key statistics in channel order


def _u32(block: np.ndarray, off: int, n: int) -> np.ndarray:
    return block[off:off + 4 * n].view(np.uint32)


def key_codes(block: np.ndarray, scheme: int) -> np.ndarray:
    """Low 2-bit key codes [64][128]."""
    g = GEOM[scheme]
    kc = _u32(block, g["kc"], 512)
    return ((kc[KEY_DW] >> KEY_SH) & 3).astype(np.uint8)


def key_high(block: np.ndarray) -> np.ndarray:
    """Kitty high plane [64][16] by boosted offset (same place in both Kitty schemes)."""
    g = GEOM[1]
    kh = _u32(block, g["kh"], 64)
    return ((kh[HI_DW] >> HI_SH) & 3).astype(np.uint8)


def key_stats(block: np.ndarray, scheme: int):
    """(scale, zero) fp16 bits [2 groups][128 channels]."""
    g = GEOM[scheme]
    ks = _u32(block, g["ks"], 256).reshape(2, 128)[:, KEY_SLOT]
    return (ks & 0xFFFF).astype(np.uint16), (ks >> 16).astype(np.uint16)


def page_boost_index(block: np.ndarray, nb: int = 16) -> np.ndarray:
    """Kitty dynamic: the page's boost index per channel (offset, or nb + 1)
    from its stored channel ids."""
    ids = block[GEOM[3]["ki"]:GEOM[3]["ki"] + nb]
    idx = np.full(D, nb + 1, np.uint8)
    idx[ids.astype(np.int64)] = np.arange(nb, dtype=np.uint8)
    return idx


def value_codes(block: np.ndarray, scheme: int) -> np.ndarray:
    g = GEOM[scheme]
    vc = _u32(block, g["vc"], 512)
    return ((vc[VAL_DW] >> VAL_SH) & 3).astype(np.uint8)


def value_stats(block: np.ndarray, scheme: int):
    """(scale, zero) fp16 bits [64 tokens][4 groups]."""
    g = GEOM[scheme]
    vs = _u32(block, g["vs"], 256).reshape(64, 4)
    return (vs & 0xFFFF).astype(np.uint16), (vs >> 16).astype(np.uint16)


def witcert_block(block: np.ndarray):
    """(key codes int8 [256][128], key scales [128], value codes, value scales)."""
    g = GEOM[2]
    kc = block[g["kc"]:g["kc"] + WPT * D].view(np.int8).reshape(WPT, D)
    ks = block[g["ks"]:g["ks"] + 2 * D].view(np.uint16)
    vc = block[g["vc"]:g["vc"] + WPT * D].view(np.int8).reshape(WPT, D)
    vs = block[g["vs"]:g["vs"] + 2 * D].view(np.uint16)
    return kc, ks, vc, vs


def page_block(pool: np.ndarray, pid: int, h: int, Hkv: int, scheme: int) -> np.ndarray:
    nb = GEOM[scheme]["bytes"]
    off = (pid * Hkv + h) * nb
    return pool[off:off + nb]


def gather_kivi(pool, table_row, h, Hkv, scheme, n_kq, n_vq, idx=None, page_idx=None):
    """Logical record of one (request, KV head) for tokens below n_kq / n_vq:
    key codes (4-bit for Kitty boosted channels) [n_kq][128], key stats
    [n_kq/32][128] x2, value codes [n_vq][128], value stats [n_vq][4] x2.
    Kitty dynamic: each page's own index; pass a list as page_idx to receive
    the indices of the key pages."""
    kcodes = np.zeros((n_kq, D), np.uint8)
    ks = np.zeros((n_kq // 32, D), np.uint16)
    kz = np.zeros((n_kq // 32, D), np.uint16)
    vcodes = np.zeros((n_vq, D), np.uint8)
    vs = np.zeros((n_vq, 4), np.uint16)
    vz = np.zeros((n_vq, 4), np.uint16)
    for p in range((max(n_kq, n_vq) + PT - 1) // PT):
        blk = page_block(pool, int(table_row[p]), h, Hkv, scheme)
        t0 = p * PT
        if t0 < n_kq:
            codes = key_codes(blk, scheme).astype(np.uint8)
            if scheme in KITTY_SCHEMES:
                pidx = idx if scheme == 1 else page_boost_index(blk)
                if page_idx is not None:
                    page_idx.append(pidx)
                hi = key_high(blk)
                for c in range(D):
                    if pidx[c] < 16:
                        codes[:, c] |= hi[:, pidx[c]] << 2
            kcodes[t0:t0 + PT] = codes
            s, z = key_stats(blk, scheme)
            ks[t0 // 32:t0 // 32 + 2] = s
            kz[t0 // 32:t0 // 32 + 2] = z
        if t0 < n_vq:
            n = min(PT, n_vq - t0)
            vcodes[t0:t0 + n] = value_codes(blk, scheme)[:n]
            s, z = value_stats(blk, scheme)
            vs[t0:t0 + n] = s[:n]
            vz[t0:t0 + n] = z[:n]
    return kcodes, ks, kz, vcodes, vs, vz
